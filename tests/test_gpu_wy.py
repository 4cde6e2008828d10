"""GPU parity of the WY-representation forward (gla_wy_fwd through the C ABI)
with the fp64 oracle (oracle.wy_reference), element by element: max|err| <=
tol * rms(ref) per output, tol = 1e-4 for fp32 inputs and 2e-2 for bf16 (the
forward's rule), plus half a bf16 ulp per element for bf16 outputs."""
import numpy as np
import pytest

import gla_inputs as gi
import oracle
from gpu_helpers import TOL, check_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import chunkwise_gated_linear_amd as gla
    gla.load_library()


def run_wy(d, dtype):
    import torch
    import chunkwise_gated_linear_amd as gla
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(d[n]).to(tdt).to(dev).contiguous() for n in ("k", "v", "A")}
    beta = torch.from_numpy(d["beta"]).to(dev)
    g = None if d["g"] is None else torch.from_numpy(d["g"]).to(dev)
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    w, u = gla.wy_fwd(t["k"], t["v"], beta, t["A"], g=g, cu_seqlens=cu)
    torch.cuda.synchronize()
    return w.float().cpu().numpy().astype(np.float64), u.float().cpu().numpy().astype(np.float64)


def check_wy(d, dtype, label):
    say(f"wy {label}: k{tuple(d['k'].shape)} v{tuple(d['v'].shape)} {dtype} g={d['g'] is not None} "
        f"packed={d['cu_seqlens'] is not None}")
    w, u = run_wy(d, dtype)
    rw, ru = oracle.wy_reference(d["k"], d["v"], d["beta"], d["A"], d["g"], cu_seqlens=d["cu_seqlens"])
    ew = check_close("w", w, rw, TOL[dtype], out_dtype=dtype)
    eu = check_close("u", u, ru, TOL[dtype], out_dtype=dtype)
    say(f"   max|err|/rms: w={ew:.2e} u={eu:.2e}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("H,HV,K,V", [(2, 2, 64, 64), (2, 4, 128, 128), (1, 3, 128, 64), (4, 4, 64, 128)])
@pytest.mark.parametrize("use_g", [True, False])
def test_shapes(dtype, H, HV, K, V, use_g):
    d = gi.draw_wy(100 + HV + K, 2, 200, H, K, V, dtype=dtype, HV=HV, use_g=use_g)
    check_wy(d, dtype, "shapes")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("K,V", [(16, 16), (48, 96), (256, 16), (112, 256)])
def test_widths(dtype, K, V):
    d = gi.draw_wy(200 + K + V, 1, 150, 2, K, V, dtype=dtype, HV=2)
    check_wy(d, dtype, "widths")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_ragged_lengths(dtype, T):
    d = gi.draw_wy(300 + T, 2, T, 2, 64, 64, dtype=dtype, dense_A=True)
    check_wy(d, dtype, f"T={T}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_packed(dtype):
    d = gi.draw_wy(400, 1, 0, 2, 64, 128, dtype=dtype, HV=4, lengths=[0, 1, 64, 65, 200, 3], dense_A=True)
    check_wy(d, dtype, "packed")


def test_workload_shape():
    # the c2048 shape of the GLA workloads: B=8, H=16, T=2048, K=V=128, bf16
    d = gi.draw_wy(1006, 8, 2048, 16, 128, 128, dtype="bf16")
    check_wy(d, "bf16", "B=8 H=16 T=2048 K=V=128")


def test_deterministic():
    d = gi.draw_wy(500, 2, 300, 2, 128, 128, dtype="bf16", HV=4)
    a = run_wy(d, "bf16")
    b = run_wy(d, "bf16")
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
