"""The no-allocation entry point gla_fwd_noalloc, called through the C ABI:
its output must equal gla_fwd's on the same inputs (same kernels, same plan,
so bit-identical) and meet the oracle's tolerance, on consecutive calls that
reuse the library's device scratch, the second with a smaller input."""
import ctypes

import numpy as np
import pytest

import gla_inputs as gi
from gpu_helpers import TOL, TOL_HT, check_close, run_oracle, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_gated_linear_amd as gla
    import oracle
    oracle.build(force=False)
    return gla.load_library()


def _problem(d, dtype):
    import chunkwise_gated_linear_amd as gla
    B, T, H, K = d["q"].shape
    V = d["v"].shape[-1]
    packed = d["cu_seqlens"] is not None
    N = len(d["cu_seqlens"]) - 1 if packed else B
    code = gla.GLA_BF16 if dtype == "bf16" else gla.GLA_F32
    return gla.make_problem(B, T, H, K, V, code, N, scale=K ** -0.5, packed=packed), N


def _noalloc(lib, d, dtype):
    """One call of gla_fwd_noalloc through ctypes; returns o, ht (device) and the status word."""
    import torch
    t = to_device(d, dtype)
    prob, N = _problem(d, dtype)
    B, T, H, K = d["q"].shape
    V = d["v"].shape[-1]
    o = torch.full_like(t["v"], float("nan"))
    ht = torch.full((N, H, K, V), float("nan"), dtype=torch.float32, device=o.device)
    status = torch.zeros(1, dtype=torch.int32, device=o.device)
    ptr = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    rc = lib.gla_fwd_noalloc(ctypes.byref(prob), ptr(t["q"]), ptr(t["k"]), ptr(t["v"]), ptr(t["g"]),
                             ptr(t["h0"]), ptr(t["cu_seqlens"]), ptr(o), ptr(ht), ptr(status),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, f"gla_fwd_noalloc returned {rc}"
    torch.cuda.synchronize()
    return t, o, ht, int(status.item())


def _check(lib, d, dtype, tag):
    import torch
    import chunkwise_gated_linear_amd as gla
    say(f"[case] no-alloc {tag} dtype={dtype} shape={d['q'].shape} V={d['v'].shape[-1]}")
    t, o, ht, st = _noalloc(lib, d, dtype)
    assert st == 0
    ro_dev, rht_dev = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
                                  output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o, ro_dev), "no-alloc o differs from gla_fwd's"
    assert torch.equal(ht, rht_dev), "no-alloc ht differs from gla_fwd's"
    ro, rht = run_oracle(d)
    eo = check_close(f"{tag} o", o.float().cpu().numpy().astype(np.float64), ro, TOL[dtype], out_dtype=dtype)
    eh = check_close(f"{tag} ht", ht.cpu().numpy().astype(np.float64), rht, TOL_HT)
    say(f"[ok]   no-alloc {tag}: identical to gla_fwd; o {eo:.3e}, ht {eh:.3e} x rms")


def test_no_alloc_matches_gla_fwd_on_consecutive_calls(lib):
    # 1) long sequences cut into many segments: summaries and start states in
    #    the scratch (about 10 MB)
    d1 = gi.draw(1201, 1, 5000, 4, 128, 128, dtype="bf16", h0=True)
    _check(lib, d1, "bf16", "segmented B=1 H=4 T=5000 K=V=128")
    # 2) a smaller input right after: split keys (the fp32 partial output of the
    #    first key block in the scratch) and segments, over the previous contents
    d2 = gi.draw(1202, 1, 700, 2, 144, 96, dtype="fp32", h0=True)
    _check(lib, d2, "fp32", "split keys B=1 H=2 T=700 K=144 V=96")
    # 3) smaller still, packed: segment table and dispatch order in the scratch
    d3 = gi.draw(1203, 1, 0, 2, 64, 64, dtype="bf16", h0=True, lengths=[300, 0, 1, 65, 129])
    _check(lib, d3, "bf16", "packed H=2 K=V=64")


def test_no_alloc_rejects_a_workspace_beyond_its_scratch(lib):
    import torch
    import chunkwise_gated_linear_amd as gla
    # split keys: the fp32 partial output alone is 1*40000*8*256*4 B = 328 MB > 64 MiB
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 40000, 8, 256, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(1, 40000, 8, 256, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(1, 40000, 8, 256, dtype=torch.float32, device=dev)
    o = torch.empty_like(v)
    with pytest.raises(gla.GlaError) as e:
        gla.gla_fwd_noalloc(q, q, v, g, o)
    assert e.value.code == 6  # GLA_ERR_WORKSPACE
