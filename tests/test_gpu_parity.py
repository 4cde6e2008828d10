"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance (stated for the method): max|err| <= 1e-4 * rms(o_oracle) for fp32
inputs and <= 2e-2 * rms(o_oracle) for bf16 inputs.  The final state is fp32
for either input dtype and is held to max|err| <= 1e-4 * rms(ht_oracle).  A bf16 output also carries its own
storage rounding (half a bf16 ulp per element), which by itself exceeds
2e-2 * rms on some small inputs (e.g. the T=63 case below: 2.0145e-2), so every
case is checked against tol * rms plus that half ulp, and the five full-size
workloads are additionally checked against the rule as stated.
"""
import numpy as np
import pytest

import gla_inputs as gi
from gpu_helpers import TOL, TOL_HT, check_close, rounding_floor, run_gpu, run_oracle, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_gated_linear_amd as gla
    gla.load_library()
    import oracle
    oracle.build(force=False)


def _compare(d, dtype, tag, scale=None, segment_chunks=0, literal=False, value_tile=0):
    say(f"[case] {tag} dtype={dtype} seg={segment_chunks} vtile={value_tile} shape={d['q'].shape} "
        f"V={d['v'].shape[-1]}")
    o, ht = run_gpu(d, dtype, scale=scale, segment_chunks=segment_chunks, value_tile=value_tile)
    ro, rht = run_oracle(d, scale=scale)
    floor = rounding_floor(ro) if dtype == "bf16" else 0.0
    eo = check_close(f"{tag} o", o, ro, TOL[dtype], out_dtype=dtype, literal=literal)
    eh = check_close(f"{tag} ht", ht, rht, TOL_HT)
    say(f"[ok]   {tag}: o max|err| {eo:.4e} rms (bf16 rounding of the exact o: {floor:.4e}), "
        f"ht {eh:.3e} rms")
    return o, ht


# ------------------------------------------------------------------ the five workloads, full size
@pytest.mark.parametrize("name", ["small", "c2048", "c4096", "varlen", "long"])
def test_workload_full_size(name):
    w = gi.WORKLOADS[name]
    d = gi.make_inputs(w)
    # on these workloads the stated rule holds without the rounding allowance
    _compare(d, w.dtype, f"workload {name}", literal=True)


# ------------------------------------------------------------------ ragged lengths, several tiles
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 200])
def test_ragged_lengths(dtype, T):
    d = gi.draw(100 + T, 2, T, 3, 64, 64, dtype=dtype, h0=True)
    _compare(d, dtype, f"ragged T={T}")


@pytest.mark.parametrize("dtype,K,V", [("bf16", 32, 64), ("bf16", 64, 64), ("bf16", 64, 128), ("bf16", 128, 256),
                                        ("bf16", 128, 64), ("fp32", 16, 64), ("fp32", 32, 128),
                                        ("fp32", 64, 256), ("fp32", 128, 128)])
def test_head_dims(dtype, K, V):
    d = gi.draw(7 * K + V, 2, 300, 2, K, V, dtype=dtype, h0=True)
    _compare(d, dtype, f"K={K} V={V}")


# every K and V that is a multiple of 16 in [16, 256]: keys are padded to the
# kernel's width (64 or 128 for bf16, 16..128 for fp32) and K > 128 runs as two
# key blocks whose outputs add; value columns past V are masked
@pytest.mark.parametrize("dtype,K,V", [("bf16", 16, 16), ("bf16", 48, 96), ("bf16", 80, 48), ("bf16", 96, 144),
                                        ("bf16", 112, 256), ("bf16", 144, 64), ("bf16", 176, 80),
                                        ("bf16", 256, 128), ("bf16", 256, 256), ("bf16", 128, 16),
                                        ("fp32", 48, 16), ("fp32", 80, 112), ("fp32", 144, 96),
                                        ("fp32", 256, 32), ("fp32", 208, 256)])
@pytest.mark.parametrize("seg", [0, 2])
def test_key_and_value_widths(dtype, K, V, seg):
    d = gi.draw(11 * K + V + seg, 2, 200, 2, K, V, dtype=dtype, h0=True)
    _compare(d, dtype, f"K={K} V={V}", segment_chunks=seg)


@pytest.mark.parametrize("dtype,K,V", [("bf16", 256, 96), ("bf16", 48, 80), ("fp32", 160, 48)])
def test_odd_widths_packed(dtype, K, V):
    lengths = [130, 0, 1, 64, 257]
    d = gi.draw(13 * K + V, 1, 0, 2, K, V, dtype=dtype, h0=True, lengths=lengths)
    _compare(d, dtype, f"packed K={K} V={V}", segment_chunks=2)


@pytest.mark.parametrize("dtype,vtile", [("bf16", 64), ("bf16", 128), ("fp32", 0)])
@pytest.mark.parametrize("seg,packed", [(0, False), (3, False), (0, True), (2, True)])
def test_without_final_state(dtype, vtile, seg, packed):
    # o alone (ht not requested): the walkers skip the state store, segment
    # summaries are still formed when the sequence is cut
    lengths = [300, 1, 0, 129, 64] if packed else None
    d = gi.draw(700 + seg + (50 if packed else 0), 1 if packed else 2, 0 if packed else 400, 2, 128, 128,
                dtype=dtype, h0=True, lengths=lengths)
    say(f"[case] no ht, dtype={dtype} vtile={vtile or 'auto'} seg={seg} packed={packed}")
    o, ht = run_gpu(d, dtype, output_final_state=False, segment_chunks=seg, value_tile=vtile)
    assert ht is None
    ro, _ = run_oracle(d)
    eo = check_close("o without ht", o, ro, TOL[dtype], out_dtype=dtype)
    say(f"[ok]   no ht: o max|err| {eo:.4e} rms")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("gate", ["zero", "strong", "mixed"])
def test_gate_extremes(dtype, gate):
    # g = 0 is plain causal linear attention; g = -1 per step puts a chunk's
    # summed log decay at -64, where the in-chunk factors exp(G_i - G_last) and
    # exp(G_last - G_j) reach e^64 and e^-64 (the kernels require |sum| < ~80
    # per chunk); "mixed" gives half the keys each
    d = gi.draw(640, 2, 200, 2, 128, 128, dtype=dtype, h0=True)
    g = np.zeros_like(d["g"])
    if gate == "strong":
        g[:] = -1.0
    elif gate == "mixed":
        g[..., ::2] = -1.0
    d["g"] = g
    _compare(d, dtype, f"gate {gate}", segment_chunks=2)


# Gates whose summed log decay over one 64-token chunk goes below -80 on some
# key: beyond the fp32 range of the factorised in-chunk form, such segments are
# re-evaluated token by token.  g = -2 per step gives -128 per chunk, -6 gives
# -384 (exp(-6) per step), -40 makes every step forget the state almost
# entirely, -1.3 stays in range for most chunks (-83 per chunk); "one" puts a
# single strong chunk among ordinary ones, "keys" only some keys.
@pytest.mark.parametrize("dtype,vtile", [("bf16", 64), ("bf16", 128), ("fp32", 0)])
@pytest.mark.parametrize("gate", ["m2", "m6", "m40", "m1.3", "one", "keys"])
@pytest.mark.parametrize("seg", [0, 2, 6])  # 6: one segment per sequence
def test_gates_beyond_the_chunk_range(dtype, vtile, gate, seg):
    d = gi.draw(660 + seg, 2, 333, 2, 128, 128, dtype=dtype, h0=True)
    g = d["g"].copy()
    if gate.startswith("m"):
        g[:] = -float(gate[1:])
    elif gate == "one":
        g[:, 130:190] = -3.0  # chunk 2 (tokens 128..191) mostly
    else:
        g[..., 5:40] = -2.5
    d["g"] = g.astype(np.float32)
    _compare(d, dtype, f"gate {gate}", segment_chunks=seg, value_tile=vtile)


@pytest.mark.parametrize("dtype,K,V", [("bf16", 48, 80), ("bf16", 256, 64), ("fp32", 160, 48)])
def test_strong_gates_packed_and_split_keys(dtype, K, V):
    lengths = [200, 0, 65, 131]
    d = gi.draw(670 + K, 1, 0, 2, K, V, dtype=dtype, h0=True, lengths=lengths)
    g = d["g"].copy()
    g[:, 60:140] = -2.0
    d["g"] = g
    _compare(d, dtype, f"strong gates packed K={K} V={V}", segment_chunks=1)


# value heads grouped on key heads (HV = G H: value head hv reads key head
# hv // G) and a gate per value head and token instead of per key
@pytest.mark.parametrize("dtype,K,V,vtile", [("bf16", 128, 128, 128), ("bf16", 128, 128, 64), ("bf16", 64, 96, 0),
                                             ("fp32", 64, 64, 0), ("bf16", 192, 64, 0)])
@pytest.mark.parametrize("H,HV,gate", [(2, 2, "head"), (1, 4, "key"), (2, 6, "head"), (2, 4, "key")])
@pytest.mark.parametrize("seg", [0, 3])
def test_head_and_gate_variants(dtype, K, V, vtile, H, HV, gate, seg):
    d = gi.draw(1300 + HV + K + seg, 2, 200, H, K, V, dtype=dtype, h0=True, HV=HV, gate=gate)
    _compare(d, dtype, f"H={H} HV={HV} gate={gate} K={K} V={V}", segment_chunks=seg, value_tile=vtile)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_head_variants_packed_and_strong(dtype):
    # packed sequences with a per-head gate strong enough for the token-by-token path
    lengths = [150, 0, 64, 97]
    d = gi.draw(1310, 1, 0, 2, 128, 64, dtype=dtype, h0=True, lengths=lengths, HV=4, gate="head")
    g = d["g"].copy()
    g[:, 40:120, 1] = -3.0
    d["g"] = g
    _compare(d, dtype, "packed H=2 HV=4 per-head gate", segment_chunks=1)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seg", [1, 2, 3, 5])
def test_forced_segments(dtype, seg):
    # long sequences cut into segments: summary kernel + state scan + output walk
    d = gi.draw(300 + seg, 2, 700, 2, 64, 128, dtype=dtype, h0=(seg % 2 == 1))
    _compare(d, dtype, f"segments of {seg} chunks", segment_chunks=seg)


@pytest.mark.parametrize("vtile", [64, 128])
@pytest.mark.parametrize("K,V,seg", [(128, 256, 0), (128, 128, 3), (64, 256, 0), (64, 128, 2), (128, 192, 0),
                                     (96, 80, 2)])
def test_value_tile_widths(vtile, K, V, seg):
    # the bf16 walker runs 64- or 128-column workgroups; pin each width on the
    # same inputs (ragged tail, initial state, with and without segments, a
    # last value slice that is partly past V)
    d = gi.draw(800 + K + V + seg, 2, 333, 3, K, V, dtype="bf16", h0=True)
    _compare(d, "bf16", f"vtile={vtile} K={K} V={V}", segment_chunks=seg, value_tile=vtile)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seg", [0, 1, 2])
def test_packed_sequences(dtype, seg):
    lengths = [0, 1, 64, 65, 130, 7, 256, 0, 191]
    d = gi.draw(500 + seg, 1, 0, 3, 64, 64, dtype=dtype, h0=True, lengths=lengths)
    o, ht = _compare(d, dtype, f"packed lengths={lengths}", segment_chunks=seg)
    # empty sequences return their initial state unchanged
    np.testing.assert_array_equal(ht[0], d["h0"][0].astype(np.float64))
    np.testing.assert_array_equal(ht[7], d["h0"][7].astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_many_packed_sequences(dtype):
    # more sequences than one pass of the segment-plan workgroup (1024), with a
    # spread of lengths (empty to several segments) so the segment table, the
    # longest-first order and the state scan all see multi-block inputs
    rng = np.random.default_rng(900)
    lengths = rng.integers(0, 140, size=1500).tolist()
    lengths[7] = 1300   # one sequence much longer than the others
    lengths[1200] = 900
    d = gi.draw(901, 1, 0, 1, 64, 64, dtype=dtype, h0=True, lengths=lengths)
    _compare(d, dtype, f"{len(lengths)} packed sequences", segment_chunks=3)


@pytest.mark.parametrize("vtile", [64, 128])
def test_uneven_packed_lengths(vtile):
    # a few long sequences among many short ones: several segments each, short
    # ones in the tail of the longest-first dispatch
    lengths = [1800, 3, 64, 129, 0, 700, 1, 65, 2500, 17, 300, 63]
    d = gi.draw(902, 1, 0, 2, 128, 128, dtype="bf16", h0=True, lengths=lengths)
    _compare(d, "bf16", f"uneven packed lengths vtile={vtile}", segment_chunks=5, value_tile=vtile)


def test_empty_sequence_batch_returns_h0():
    d = gi.draw(601, 2, 0, 2, 64, 64, dtype="bf16", h0=True)
    o, ht = run_gpu(d, "bf16")
    assert o.shape == (2, 0, 2, 64)
    np.testing.assert_array_equal(ht, d["h0"].astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_packed_batch_of_empty_sequences_returns_h0(dtype):
    # packed input with no tokens at all: every sequence keeps its initial state
    d = gi.draw(605, 1, 0, 2, 64, 64, dtype=dtype, h0=True, lengths=[0, 0, 0])
    say(f"[case] packed, all sequences empty, dtype={dtype}")
    o, ht = run_gpu(d, dtype)
    assert o.shape == (1, 0, 2, 64)
    np.testing.assert_array_equal(ht, d["h0"].astype(np.float64))


def test_no_initial_state_and_explicit_scale():
    d = gi.draw(602, 3, 150, 2, 128, 128, dtype="bf16", h0=False)
    _compare(d, "bf16", "scale=0.3", scale=0.3)


def test_split_sequence_resume_on_gpu():
    import torch
    import chunkwise_gated_linear_amd as gla
    from gpu_helpers import to_device
    d = gi.draw(603, 1, 1000, 4, 128, 128, dtype="bf16", h0=True)
    t = to_device(d, "bf16")
    o, ht = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], output_final_state=True)
    T1 = 333
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o1, h1 = gla.gla_fwd(*(sl(t[x], 0, T1) for x in "qkvg"), h0=t["h0"], output_final_state=True)
    o2, h2 = gla.gla_fwd(*(sl(t[x], T1, 1000) for x in "qkvg"), h0=h1, output_final_state=True)
    torch.cuda.synchronize()
    both = torch.cat([o1, o2], dim=1).float()
    ref = o.float()
    r = ref.pow(2).mean().sqrt().item()
    assert (both - ref).abs().max().item() <= 2e-2 * r
    assert (h2 - ht).abs().max().item() <= 1e-4 * ht.pow(2).mean().sqrt().item()


def test_bitwise_deterministic():
    import torch
    import chunkwise_gated_linear_amd as gla
    from gpu_helpers import to_device
    d = gi.draw(604, 2, 777, 4, 128, 128, dtype="bf16", h0=True)
    t = to_device(d, "bf16")
    a = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], output_final_state=True, segment_chunks=3)
    b = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], output_final_state=True, segment_chunks=3)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_invalid_arguments_raise():
    import torch
    import chunkwise_gated_linear_amd as gla
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(1, 8, 1, 64, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        gla.gla_fwd(q, q, v, g, scale=-1.0)
    with pytest.raises(ValueError):
        gla.gla_fwd(q, q.float(), v, g)
    with pytest.raises(gla.GlaError):  # K must be a multiple of 16
        gla.gla_fwd(q[..., :40].contiguous(), q[..., :40].contiguous(), v, g[..., :40].contiguous())
    q2 = torch.zeros(2, 8, 1, 64, dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 4, 8], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        gla.gla_fwd(q2, q2, q2, g.expand(2, 8, 1, 64).contiguous(), cu_seqlens=cu)


# ------------------------------------------------------------------ bounded waits
@pytest.mark.parametrize("name,segment_chunks,vtile", [("c2048", 0, 0), ("c2048", 8, 64), ("c4096", 0, 0),
                                                       ("varlen", 0, 0), ("long", 0, 0)])
def test_bounded_waits_are_never_exhausted(name, segment_chunks, vtile):
    """The walkers' counter waits between waves are bounded so that a wave always
    leaves them; a wait that runs to its bound sets a bit in the workspace status
    word.  On the full-size workloads no wait may run out (status word clear),
    and every launch finishes in well under one exhausted wait (tens of
    milliseconds of polling)."""
    import torch
    import chunkwise_gated_linear_amd as gla
    w = gi.WORKLOADS[name]
    d = gi.make_inputs(w)
    t = to_device(d, w.dtype)
    call = gla.GlaCall(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
                       output_final_state=w.ht, segment_chunks=segment_chunks, value_tile=vtile)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        call(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        call(stream)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    say(f"[ok]   {name} seg={segment_chunks} vtile={vtile or 'auto'}: {ms:.3f} ms per launch, "
        f"status {call.status():#x}")
    assert call.status() == 0, "a bounded wait between waves ran out"
    assert ms < 20.0, f"{name}: {ms:.1f} ms per launch; a bounded wait probably ran out"


def test_exhausted_wait_is_reported():
    """A wait that runs out is visible: with the bound forced to zero polls (a
    test hook of the ABI) every score hand-off of the 64-column output walker
    reports at once, the kernels still finish, and the status word holds
    GLA_STATUS_WAIT_EXHAUSTED.  A fresh call with the default bound on another
    workspace leaves its word clear."""
    import torch
    import chunkwise_gated_linear_amd as gla
    d = gi.draw(905, 2, 300, 2, 128, 128, dtype="bf16", h0=True)
    t = to_device(d, "bf16")
    say("[case] forced wait run-out, 64-column output walker")
    forced = gla.GlaCall(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], output_final_state=True,
                         value_tile=64, wait_limit=-1)
    torch.cuda.synchronize()
    assert forced.status() & gla.STATUS_WAIT_EXHAUSTED
    normal = gla.GlaCall(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], output_final_state=True,
                         value_tile=64)
    torch.cuda.synchronize()
    assert normal.status() == 0
    # the word is sticky: a later call with the default bound on the same
    # workspace (whose waits all finish) leaves the bit set
    o, _ = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], value_tile=64, workspace=forced.workspace)
    torch.cuda.synchronize()
    assert gla.read_status(forced.workspace) & gla.STATUS_WAIT_EXHAUSTED
