"""GPU parity of the backward (gla_bwd through the C ABI) with the fp64 oracle.

Every output (dq, dk, dv, dg, dh0) is compared element by element with
oracle.gla_reference_bwd on the same seeded inputs.  Rules, per output:
max|err| <= tol * rms(ref), tol = 1e-4 for fp32 inputs and 2e-2 for bf16
inputs (the forward's rule), plus half a bf16 ulp per element for outputs
stored in bf16.  dg and dh0 are fp32 for either input dtype and are formed from
fp32 products of exact inputs, so they are held to 1e-4 as the final state is.
"""
import numpy as np
import pytest

import gla_inputs as gi
import oracle
from gpu_helpers import TOL, TOL_HT, check_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import chunkwise_gated_linear_amd as gla
    gla.load_library()
    oracle.build(force=False)


def grads_in(d, dtype, seed):
    """do (v's shape, rounded like v) and dht (fp32) for input set d."""
    rng = np.random.default_rng(seed)
    do = rng.standard_normal(d["v"].shape).astype(np.float32)
    if dtype == "bf16":
        do = gi.to_bf16_f32(do)
    N = len(d["cu_seqlens"]) - 1 if d["cu_seqlens"] is not None else d["q"].shape[0]
    HV, K, V = d["v"].shape[2], d["q"].shape[3], d["v"].shape[3]
    dht = rng.standard_normal((N, HV, K, V)).astype(np.float32)
    return do, dht


def run_bwd_gpu(d, do, dht, dtype, scale=None, need_dh0=True, schedule=0, wait_limit=0, status=None):
    import torch
    import chunkwise_gated_linear_amd as gla
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(d[n]).to(tdt).to(dev).contiguous() for n in ("q", "k", "v")}
    g = torch.from_numpy(d["g"]).to(dev).contiguous()
    h0 = None if d["h0"] is None else torch.from_numpy(d["h0"]).to(dev).contiguous()
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    tdo = torch.from_numpy(do).to(tdt).to(dev).contiguous()
    tdht = None if dht is None else torch.from_numpy(dht).to(dev).contiguous()
    ws = None
    if status is not None:  # a zeroed workspace whose status word is returned in status[0]
        prob, _, _ = gla._problem_for(t["q"], t["k"], t["v"], g, h0, cu, None, scale, 64, 0, 0, wait_limit,
                                      schedule)
        ws = torch.zeros(gla.bwd_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    dq, dk, dv, dg, dh0 = gla.gla_bwd(t["q"], t["k"], t["v"], g, tdo, h0=h0, dht=tdht, cu_seqlens=cu,
                                      scale=scale, need_dh0=need_dh0, workspace=ws, schedule=schedule,
                                      wait_limit=wait_limit)
    torch.cuda.synchronize()
    if status is not None:
        status.append(gla.read_status(ws))
    f = lambda x: None if x is None else x.float().cpu().numpy().astype(np.float64)
    return f(dq), f(dk), f(dv), f(dg), f(dh0)


def check_bwd(d, dtype, seed, scale=None, use_dht=True, need_dh0=True, label="", schedule=0):
    do, dht = grads_in(d, dtype, seed)
    if not use_dht:
        dht = None
    say(f"bwd {label}: q{tuple(d['q'].shape)} v{tuple(d['v'].shape)} g{tuple(d['g'].shape)} {dtype} "
        f"h0={d['h0'] is not None} dht={dht is not None} packed={d['cu_seqlens'] is not None} "
        f"schedule={schedule}")
    got = run_bwd_gpu(d, do, dht, dtype, scale=scale, need_dh0=need_dh0, schedule=schedule)
    ref = oracle.gla_reference_bwd(d["q"], d["k"], d["v"], d["g"], do, h0=d["h0"], dht=dht,
                                   cu_seqlens=d["cu_seqlens"], scale=scale)
    tol = TOL[dtype]
    errs = {}
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dh0"), got, ref):
        if name == "dh0" and not need_dh0:
            assert a is None
            continue
        if name in ("dg", "dh0"):
            errs[name] = check_close(name, a, b, TOL_HT)
        else:
            errs[name] = check_close(name, a, b, tol, out_dtype=dtype)
    say("   max|err|/rms: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return errs


# schedule 1: summaries, a separate scan launch, chunk kernel; 2: the scan
# chained into the summary kernel; 3: the summary kernel walks whole chains
SCHEDULES = [1, 2, 3]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,T,H,K,V", [
    (2, 200, 2, 64, 64),
    (1, 256, 2, 128, 128),
    (2, 130, 3, 128, 64),
    (1, 150, 2, 64, 128),
])
def test_shapes(dtype, B, T, H, K, V, schedule):
    d = gi.draw(100 + T + K, B, T, H, K, V, dtype=dtype, h0=True)
    check_bwd(d, dtype, seed=7, label="shapes", schedule=schedule)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("K,V", [(16, 16), (48, 96), (16, 128), (112, 32)])
def test_narrow_and_odd_widths(dtype, K, V, schedule):
    # keys and columns past K and V inside the kernels' 64- or 128-wide tiles:
    # every schedule's state steps leave them out
    d = gi.draw(200 + K + V, 2, 100, 2, K, V, dtype=dtype, h0=True)
    check_bwd(d, dtype, seed=8, label="widths", schedule=schedule)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 129])
def test_ragged_lengths(dtype, T, schedule):
    d = gi.draw(300 + T, 2, T, 2, 64, 64, dtype=dtype, h0=True)
    check_bwd(d, dtype, seed=9, label=f"T={T}", schedule=schedule)


# V past 128 runs as value slices of 128 columns; dq, dk and dg are summed
# over the slices' fp32 shares, dv and dh0 are written per slice
@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("K,V", [(64, 144), (128, 256), (32, 192)])
def test_value_slices(dtype, K, V, schedule):
    d = gi.draw(350 + K + V, 2, 150, 2, K, V, dtype=dtype, h0=True)
    check_bwd(d, dtype, seed=24, label=f"K={K} V={V}", schedule=schedule)


# K past 128 runs as two key blocks; dv (and a per-head gate's dg) are summed
# over the blocks' fp32 shares
@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("K,V", [(144, 64), (256, 128), (192, 256)])
def test_key_blocks(dtype, K, V, schedule):
    d = gi.draw(370 + K + V, 2, 150, 2, K, V, dtype=dtype, h0=True)
    check_bwd(d, dtype, seed=28, label=f"K={K} V={V}", schedule=schedule)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_key_blocks_variants(dtype):
    d = gi.draw(380, 2, 140, 2, 256, 64, dtype=dtype, h0=True, HV=4, gate="head")
    check_bwd(d, dtype, seed=29, label="K=256 HV=4 gate=head")
    d = gi.draw(381, 1, 0, 2, 160, 160, dtype=dtype, h0=True, lengths=[70, 0, 190, 5])
    check_bwd(d, dtype, seed=30, label="K=V=160 packed")
    check_bwd(d, dtype, seed=30, label="K=V=160 packed, chained scan", schedule=2)
    d = gi.draw(382, 2, 200, 2, 256, 128, dtype=dtype, h0=True, gate_scale=40.0)
    check_bwd(d, dtype, seed=31, label="K=256 gates x40")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_value_slices_variants(dtype):
    # value-head groups and a per-head gate; packed sequences; strong gates
    # (chunks in the token-by-token kernel), each with two value slices
    d = gi.draw(360, 2, 140, 2, 64, 256, dtype=dtype, h0=True, HV=4, gate="head")
    check_bwd(d, dtype, seed=25, label="V=256 HV=4 gate=head")
    d = gi.draw(361, 1, 0, 2, 64, 160, dtype=dtype, h0=True, lengths=[70, 0, 190, 5])
    check_bwd(d, dtype, seed=26, label="V=160 packed")
    check_bwd(d, dtype, seed=26, label="V=160 packed, chained scan", schedule=2)
    d = gi.draw(362, 2, 200, 2, 64, 256, dtype=dtype, h0=True, gate_scale=40.0)
    check_bwd(d, dtype, seed=27, label="V=256 gates x40")


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_packed(dtype, schedule):
    d = gi.draw(401, 1, 0, 2, 64, 128, dtype=dtype, h0=True, lengths=[0, 1, 64, 65, 200, 3, 128])
    check_bwd(d, dtype, seed=10, label="packed", schedule=schedule)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("h0,use_dht,need_dh0", [(False, True, True), (True, False, True), (False, False, False),
                                                 (True, True, False)])
def test_optional_states(dtype, h0, use_dht, need_dh0, schedule):
    d = gi.draw(500, 2, 150, 2, 64, 64, dtype=dtype, h0=h0)
    check_bwd(d, dtype, seed=11, use_dht=use_dht, need_dh0=need_dh0, label="optional", schedule=schedule)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("HV,gate", [(2, "key"), (1, "head"), (3, "head")])
def test_head_and_gate_variants(dtype, HV, gate, schedule):
    H = 2
    d = gi.draw(600 + HV, 2, 140, H, 64, 64, dtype=dtype, h0=True, HV=H * HV, gate=gate)
    check_bwd(d, dtype, seed=12, label=f"HV={H * HV} gate={gate}", schedule=schedule)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_head_variants_packed(dtype, schedule):
    d = gi.draw(650, 1, 0, 2, 64, 128, dtype=dtype, h0=True, lengths=[70, 0, 190, 5], HV=4, gate="head")
    check_bwd(d, dtype, seed=13, label="packed heads", schedule=schedule)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("gate_scale", [4.0, 40.0])
def test_strong_gates(dtype, gate_scale, schedule):
    # logsigmoid(N(0,1)) * gate_scale: with 4, some chunks decay by more than
    # e^-80 over 64 tokens on some key; with 40 nearly every chunk does.  Those
    # chunks take the token-by-token kernel; the results must not change.
    d = gi.draw(700, 2, 200, 2, 64, 64, dtype=dtype, h0=True, gate_scale=gate_scale)
    check_bwd(d, dtype, seed=14, label=f"gate x{gate_scale}", schedule=schedule)


def test_strong_gates_packed_heads():
    d = gi.draw(710, 1, 0, 2, 64, 64, dtype="bf16", h0=True, lengths=[100, 64, 7], gate_scale=8.0, HV=4)
    check_bwd(d, "bf16", seed=15, label="strong packed heads")


def test_scale():
    d = gi.draw(800, 1, 100, 2, 64, 64, dtype="fp32", h0=True)
    check_bwd(d, "fp32", seed=16, scale=0.37, label="scale")


def test_zero_gate_is_linear_attention():
    # g == 0: dq = scale (tril(dO V^T) K + dO h0^T), etc.; also the GPU result
    d = gi.draw(810, 1, 130, 1, 64, 64, dtype="fp32", h0=True)
    d["g"] = np.zeros_like(d["g"])
    check_bwd(d, "fp32", seed=17, label="g=0")


@pytest.mark.parametrize("gate,strong", [("key", False), ("head", False), ("head", True)])
def test_deterministic(gate, strong):
    # every sum has a fixed order, the per-head gate's sums over keys included
    # (strong gates: in the token-by-token kernel)
    d = gi.draw(900, 2, 300, 2, 128, 128, dtype="bf16", h0=True, gate=gate, gate_scale=40.0 if strong else 1.0 / 16.0)
    do, dht = grads_in(d, "bf16", 18)
    say(f"bwd determinism: B=2 T=300 H=2 K=V=128 bf16 gate={gate} strong={strong}")
    a = run_bwd_gpu(d, do, dht, "bf16")
    b = run_bwd_gpu(d, do, dht, "bf16")
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dh0"), a, b):
        assert np.array_equal(x, y), name


def head_slice(d, heads):
    """The same inputs restricted to some heads (heads are independent)."""
    out = dict(d)
    for n in ("q", "k", "v", "g"):
        out[n] = np.ascontiguousarray(d[n][:, :, heads])
    if d["h0"] is not None:
        out["h0"] = np.ascontiguousarray(d["h0"][:, heads])
    return out


@pytest.mark.parametrize("name", ["c2048", "varlen", "c4096"])
def test_workload_sampled_heads(name):
    """A full-size workload on the GPU; the oracle on two of its heads."""
    w = gi.WORKLOADS[name]
    d = gi.make_inputs(w)
    do, dht = grads_in(d, w.dtype, 19)
    say(f"bwd workload {name}: {w.describe() if hasattr(w, 'describe') else name}")
    got = run_bwd_gpu(d, do, dht, w.dtype)
    heads = [0, w.H - 1]
    ds = head_slice(d, heads)
    ref = oracle.gla_reference_bwd(ds["q"], ds["k"], ds["v"], ds["g"], np.ascontiguousarray(do[:, :, heads]),
                                   h0=ds["h0"], dht=np.ascontiguousarray(dht[:, heads]),
                                   cu_seqlens=d["cu_seqlens"])
    errs = {}
    for name_, a, b in zip(("dq", "dk", "dv", "dg", "dh0"), got, ref):
        a = a[:, heads] if name_ == "dh0" else a[:, :, heads]
        tol = TOL_HT if name_ in ("dg", "dh0") else TOL[w.dtype]
        errs[name_] = check_close(name_, a, b, tol, out_dtype="fp32" if name_ in ("dg", "dh0") else w.dtype)
    say("   max|err|/rms: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("schedule", [2, 3])
@pytest.mark.parametrize("dtype,gate,K,V", [("bf16", "key", 128, 128), ("fp32", "key", 128, 128),
                                             ("bf16", "head", 128, 128), ("bf16", "key", 128, 256),
                                             ("bf16", "head", 256, 128)])
def test_chained_scan_matches_separate_scan(dtype, gate, K, V, schedule):
    """The chained scan (schedule 2) and the walk (3) apply the separate scan's
    recurrences in the same order and precision to the same summaries: every
    output agrees bit for bit.  Many chains of many chunks (B=4, H=16, T=1000:
    64 chains of 16 chunks per direction; chained, they cross workgroups on
    different dies); the oracle checks two heads.  With V = 256 or K = 256 each
    value slice's or key block's h0, dht and dh0 rows and columns are staged."""
    d = gi.draw(920, 4, 1000, 16, K, V, dtype=dtype, h0=True, gate=gate)
    do, dht = grads_in(d, dtype, 21)
    say(f"bwd schedule {schedule} vs separate scan: B=4 T=1000 H=16 K={K} V={V} {dtype} gate={gate}")
    a = run_bwd_gpu(d, do, dht, dtype, schedule=1)
    b = run_bwd_gpu(d, do, dht, dtype, schedule=schedule)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dh0"), a, b):
        assert np.array_equal(x, y), f"{name}: max|diff| {np.max(np.abs(x - y)):.3e}"
    heads = [3, 14]
    ds = head_slice(d, heads)
    ref = oracle.gla_reference_bwd(ds["q"], ds["k"], ds["v"], ds["g"], np.ascontiguousarray(do[:, :, heads]),
                                   h0=ds["h0"], dht=np.ascontiguousarray(dht[:, heads]))
    for name, x, r in zip(("dq", "dk", "dv", "dg", "dh0"), b, ref):
        x = x[:, heads] if name == "dh0" else x[:, :, heads]
        check_close(name, x, r, TOL_HT if name in ("dg", "dh0") else TOL[dtype],
                    out_dtype="fp32" if name in ("dg", "dh0") else dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_walk_more_chains_than_workgroups(dtype):
    """The walk with 1024 chains (B=64, H=8, three chunks each) on at most two
    workgroups per compute unit: each workgroup walks several chains in turn,
    carrying each from its own first chunk.  Bit for bit against the separate
    scan; the oracle checks two heads."""
    d = gi.draw(960, 64, 130, 8, 64, 64, dtype=dtype, h0=True)
    do, dht = grads_in(d, dtype, 34)
    say(f"bwd walk, 1024 chains: B=64 T=130 H=8 K=V=64 {dtype}")
    a = run_bwd_gpu(d, do, dht, dtype, schedule=1)
    b = run_bwd_gpu(d, do, dht, dtype, schedule=3)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dh0"), a, b):
        assert np.array_equal(x, y), f"{name}: max|diff| {np.max(np.abs(x - y)):.3e}"
    heads = [0, 5]
    ds = head_slice(d, heads)
    ref = oracle.gla_reference_bwd(ds["q"], ds["k"], ds["v"], ds["g"], np.ascontiguousarray(do[:, :, heads]),
                                   h0=ds["h0"], dht=np.ascontiguousarray(dht[:, heads]))
    for name, x, r in zip(("dq", "dk", "dv", "dg", "dh0"), b, ref):
        x = x[:, heads] if name == "dh0" else x[:, :, heads]
        check_close(name, x, r, TOL_HT if name in ("dg", "dh0") else TOL[dtype],
                    out_dtype="fp32" if name in ("dg", "dh0") else dtype)


@pytest.mark.parametrize("schedule", [2, 3])
@pytest.mark.parametrize("dtype,K,V", [("bf16", 64, 64), ("fp32", 64, 64), ("bf16", 160, 192)])
def test_chained_scan_packed_matches_separate_scan(dtype, K, V, schedule):
    """Packed sequences: the chain plan orders each step's chains by sequence
    length (chained), each workgroup walks the chains of its sequences (walk);
    sequences without chunks keep dh0 = dht.  Every output agrees bit for bit
    with the separate scan; the oracle checks two heads."""
    rng = np.random.default_rng(945)
    lengths = [int(x) for x in rng.integers(0, 700, size=40)]
    lengths[3] = lengths[17] = 0
    lengths[5], lengths[8], lengths[9], lengths[30] = 1, 64, 65, 1500
    d = gi.draw(946, 1, 0, 8, K, V, dtype=dtype, h0=True, lengths=lengths)
    do, dht = grads_in(d, dtype, 32)
    say(f"bwd packed schedule {schedule} vs separate scan: 40 sequences H=8 K={K} V={V} {dtype}")
    a = run_bwd_gpu(d, do, dht, dtype, schedule=1)
    b = run_bwd_gpu(d, do, dht, dtype, schedule=schedule)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dh0"), a, b):
        assert np.array_equal(x, y), f"{name}: max|diff| {np.max(np.abs(x - y)):.3e}"
    heads = [2, 7]
    ds = head_slice(d, heads)
    ref = oracle.gla_reference_bwd(ds["q"], ds["k"], ds["v"], ds["g"], np.ascontiguousarray(do[:, :, heads]),
                                   h0=ds["h0"], dht=np.ascontiguousarray(dht[:, heads]), cu_seqlens=d["cu_seqlens"])
    for name, x, r in zip(("dq", "dk", "dv", "dg", "dh0"), b, ref):
        x = x[:, heads] if name == "dh0" else x[:, :, heads]
        check_close(name, x, r, TOL_HT if name in ("dg", "dh0") else TOL[dtype],
                    out_dtype="fp32" if name in ("dg", "dh0") else dtype)


@pytest.mark.parametrize("schedule", [2, 3])
def test_chained_scan_many_packed_sequences(schedule):
    """1500 short packed sequences (empty, one token, up to three chunks):
    the chain plan's loops over sequences and steps run several rounds of its
    1024 threads (chained), each workgroup walks several chains (walk: 6000
    chains); bit for bit against the separate scan, the oracle on one head."""
    rng = np.random.default_rng(950)
    lengths = [int(x) for x in rng.integers(0, 190, size=1500)]
    lengths[0] = lengths[700] = lengths[1499] = 0
    lengths[1] = 1
    d = gi.draw(951, 1, 0, 2, 64, 64, dtype="bf16", h0=True, lengths=lengths)
    do, dht = grads_in(d, "bf16", 33)
    say(f"bwd packed schedule {schedule} vs separate scan: 1500 sequences H=2 K=V=64 bf16")
    a = run_bwd_gpu(d, do, dht, "bf16", schedule=1)
    b = run_bwd_gpu(d, do, dht, "bf16", schedule=schedule)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dh0"), a, b):
        assert np.array_equal(x, y), f"{name}: max|diff| {np.max(np.abs(x - y)):.3e}"
    ds = head_slice(d, [1])
    ref = oracle.gla_reference_bwd(ds["q"], ds["k"], ds["v"], ds["g"], np.ascontiguousarray(do[:, :, [1]]),
                                   h0=ds["h0"], dht=np.ascontiguousarray(dht[:, [1]]), cu_seqlens=d["cu_seqlens"])
    for name, x, r in zip(("dq", "dk", "dv", "dg", "dh0"), b, ref):
        x = x[:, [1]] if name == "dh0" else x[:, :, [1]]
        check_close(name, x, r, TOL_HT if name in ("dg", "dh0") else TOL["bf16"],
                    out_dtype="fp32" if name in ("dg", "dh0") else "bf16")


def test_chained_scan_repeated_calls():
    """Back-to-back chained backward calls on one workspace: each call clears
    the chains' flags before its summary kernel, so no call sees another's."""
    import torch
    import chunkwise_gated_linear_amd as gla
    d = gi.draw(930, 8, 300, 8, 64, 64, dtype="bf16", h0=True)
    do, dht = grads_in(d, "bf16", 22)
    ref = run_bwd_gpu(d, do, dht, "bf16", schedule=1)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(d[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v")}
    g, h0 = torch.from_numpy(d["g"]).to(dev), torch.from_numpy(d["h0"]).to(dev)
    tdo, tdht = torch.from_numpy(do).to(torch.bfloat16).to(dev), torch.from_numpy(dht).to(dev)
    prob, _, _ = gla._problem_for(t["q"], t["k"], t["v"], g, h0, None, None, None, 64, 0, 0, 0, 2)
    ws = torch.zeros(gla.bwd_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    say("bwd chained: 5 calls on one workspace, B=8 T=300 H=8 K=V=64 bf16")
    outs = [gla.gla_bwd(t["q"], t["k"], t["v"], g, tdo, h0=h0, dht=tdht, workspace=ws, schedule=2)
            for _ in range(5)]
    torch.cuda.synchronize()
    assert gla.read_status(ws) == 0
    for out in outs:
        for name, x, y in zip(("dq", "dk", "dv", "dg", "dh0"), out, ref):
            assert np.array_equal(x.float().cpu().numpy().astype(np.float64), y), name


def test_chained_scan_wait_bound_reports():
    """wait_limit = -1 turns every wait of the chained scan into an immediate
    report: the kernels still end, and the status word says the results are
    not to be trusted.  The separate scan has no waits and reports nothing."""
    d = gi.draw(940, 2, 300, 2, 64, 64, dtype="bf16", h0=True)
    do, dht = grads_in(d, "bf16", 23)
    say("bwd chained with wait_limit=-1 (status report), B=2 T=300 H=2 K=V=64 bf16")
    st = []
    run_bwd_gpu(d, do, dht, "bf16", schedule=2, wait_limit=-1, status=st)
    run_bwd_gpu(d, do, dht, "bf16", schedule=1, wait_limit=-1, status=st)
    assert st[0] & 1 == 1
    assert st[1] == 0
