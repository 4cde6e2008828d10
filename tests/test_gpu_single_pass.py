"""GPU parity of the single-pass forward (schedule = 2) with the fp64 oracle.

The single pass runs a sequence's segments in one launch: each workgroup forms
its segment's summary, waits for the previous segment's end state, publishes
its own, and then walks its chunks (page "fla/ops/gla/fused_chunk.py",
fused_chunk_gla_fwd_kernel, carries the state through a serial chunk loop; the
segments are joined by the same state recurrence).  It must agree with the
oracle under the forward's rule (max|err| <= 2e-2 rms(o) for bf16 plus half a
bf16 ulp per element; ht to 1e-4 rms(ht)) wherever segments are cut: several
segments per sequence, ragged tails, packed sequences of every length class,
gates beyond the chunk form's range (token-by-token segments inside the
chain), value-head groups and per-head gates, both value-tile widths."""
import numpy as np
import pytest

import gla_inputs as gi
from gpu_helpers import TOL, TOL_HT, check_close, rounding_floor, run_gpu, run_oracle, say, to_device

pytestmark = pytest.mark.gpu

SINGLE = 2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_gated_linear_amd as gla
    gla.load_library()
    import oracle
    oracle.build(force=False)


def _compare(d, tag, segment_chunks=0, value_tile=0, literal=False, output_final_state=True):
    say(f"[case] single pass: {tag} seg={segment_chunks} vtile={value_tile} shape={d['q'].shape} "
        f"V={d['v'].shape[-1]}")
    o, ht = run_gpu(d, "bf16", segment_chunks=segment_chunks, value_tile=value_tile, schedule=SINGLE,
                    output_final_state=output_final_state)
    ro, rht = run_oracle(d)
    floor = rounding_floor(ro)
    eo = check_close(f"{tag} o", o, ro, TOL["bf16"], out_dtype="bf16", literal=literal)
    msg = f"[ok]   {tag}: o max|err| {eo:.4e} rms (bf16 rounding of the exact o: {floor:.4e})"
    if output_final_state:
        eh = check_close(f"{tag} ht", ht, rht, TOL_HT)
        msg += f", ht {eh:.3e} rms"
    say(msg)
    return o, ht


@pytest.mark.parametrize("seg", [1, 2, 3, 5])
@pytest.mark.parametrize("K,V,vtile", [(64, 128, 0), (128, 128, 128), (128, 128, 64), (64, 96, 0)])
def test_segments(seg, K, V, vtile):
    d = gi.draw(2100 + seg + K + V, 2, 700, 2, K, V, dtype="bf16", h0=(seg % 2 == 1))
    _compare(d, f"segments of {seg} chunks K={K} V={V}", segment_chunks=seg, value_tile=vtile)


@pytest.mark.parametrize("T", [65, 127, 128, 129, 200])
def test_ragged_tails(T):
    d = gi.draw(2200 + T, 3, T, 2, 128, 128, dtype="bf16", h0=True)
    _compare(d, f"T={T}", segment_chunks=1)


@pytest.mark.parametrize("seg", [1, 2, 3])
def test_packed_sequences(seg):
    lengths = [0, 1, 64, 65, 130, 7, 256, 0, 191]
    d = gi.draw(2300 + seg, 1, 0, 3, 64, 64, dtype="bf16", h0=True, lengths=lengths)
    o, ht = _compare(d, f"packed lengths={lengths}", segment_chunks=seg)
    np.testing.assert_array_equal(ht[0], d["h0"][0].astype(np.float64))
    np.testing.assert_array_equal(ht[7], d["h0"][7].astype(np.float64))


@pytest.mark.parametrize("vtile", [64, 128])
def test_uneven_packed_lengths(vtile):
    lengths = [1800, 3, 64, 129, 0, 700, 1, 65, 2500, 17, 300, 63]
    d = gi.draw(2400, 1, 0, 2, 128, 128, dtype="bf16", h0=True, lengths=lengths)
    _compare(d, f"uneven packed lengths vtile={vtile}", segment_chunks=5, value_tile=vtile)


def test_many_packed_sequences():
    rng = np.random.default_rng(2500)
    lengths = rng.integers(0, 140, size=1500).tolist()
    lengths[7] = 1300
    lengths[1200] = 900
    d = gi.draw(2501, 1, 0, 1, 64, 64, dtype="bf16", h0=True, lengths=lengths)
    _compare(d, f"{len(lengths)} packed sequences", segment_chunks=3)


@pytest.mark.parametrize("vtile", [64, 128])
@pytest.mark.parametrize("gate", ["m2", "one", "keys"])
def test_gates_beyond_the_chunk_range(vtile, gate):
    d = gi.draw(2600, 2, 333, 2, 128, 128, dtype="bf16", h0=True)
    g = d["g"].copy()
    if gate == "m2":
        g[:] = -2.0
    elif gate == "one":
        g[:, 130:190] = -3.0
    else:
        g[..., 5:40] = -2.5
    d["g"] = g.astype(np.float32)
    _compare(d, f"gate {gate}", segment_chunks=2, value_tile=vtile)


@pytest.mark.parametrize("H,HV,gate,K,V", [(1, 4, "key", 128, 128), (2, 6, "head", 64, 96),
                                           (2, 4, "head", 128, 128)])
def test_head_and_gate_variants(H, HV, gate, K, V):
    d = gi.draw(2700 + HV, 2, 300, H, K, V, dtype="bf16", h0=True, HV=HV, gate=gate)
    _compare(d, f"H={H} HV={HV} gate={gate} K={K} V={V}", segment_chunks=2)


def test_without_final_state():
    d = gi.draw(2800, 2, 500, 2, 128, 128, dtype="bf16", h0=True)
    _compare(d, "no ht", segment_chunks=2, output_final_state=False)


@pytest.mark.parametrize("name", ["long", "varlen"])
def test_workload_full_size(name):
    w = gi.WORKLOADS[name]
    d = gi.make_inputs(w)
    _compare(d, f"workload {name}", literal=True)


def test_agrees_with_three_passes():
    # the two schedules evaluate the same chunk form; only the order of a few
    # fp32 state additions differs
    d = gi.draw(2900, 2, 900, 3, 128, 128, dtype="bf16", h0=True)
    o1, h1 = run_gpu(d, "bf16", segment_chunks=3, schedule=1)
    o2, h2 = run_gpu(d, "bf16", segment_chunks=3, schedule=SINGLE)
    r = float(np.sqrt(np.mean(h1 ** 2)))
    assert np.max(np.abs(h1 - h2)) <= 1e-5 * r
    ro = float(np.sqrt(np.mean(o1 ** 2)))
    assert np.max(np.abs(o1 - o2)) <= 2e-2 * ro


def test_bitwise_deterministic():
    import torch
    import chunkwise_gated_linear_amd as gla
    d = gi.draw(2950, 2, 777, 4, 128, 128, dtype="bf16", h0=True)
    t = to_device(d, "bf16")
    kw = dict(h0=t["h0"], output_final_state=True, segment_chunks=2, schedule=SINGLE)
    a = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], **kw)
    b = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", ["long", "varlen"])
def test_bounded_waits_are_never_exhausted(name):
    """Every wait for a previous segment's state ends before its bound on the
    full-size workloads, and a launch takes far less than one exhausted wait."""
    import torch
    import chunkwise_gated_linear_amd as gla
    w = gi.WORKLOADS[name]
    d = gi.make_inputs(w)
    t = to_device(d, w.dtype)
    call = gla.GlaCall(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
                       output_final_state=w.ht, schedule=SINGLE)
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
    say(f"[ok]   single pass {name}: {ms:.3f} ms per launch, status {call.status():#x}")
    assert call.status() == 0
    assert ms < 20.0


def test_exhausted_wait_is_reported():
    """With the wait bound forced to zero polls, a segment that finds its
    predecessor's state not yet published reports GLA_STATUS_WAIT_EXHAUSTED and
    goes on; every workgroup still finishes."""
    import torch
    import chunkwise_gated_linear_amd as gla
    d = gi.draw(2990, 1, 4096, 4, 128, 128, dtype="bf16", h0=True)
    t = to_device(d, "bf16")
    say("[case] single pass, forced wait run-out")
    forced = gla.GlaCall(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], output_final_state=True,
                         segment_chunks=1, schedule=SINGLE, wait_limit=-1)
    torch.cuda.synchronize()
    assert forced.status() & gla.STATUS_WAIT_EXHAUSTED
    normal = gla.GlaCall(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], output_final_state=True,
                         segment_chunks=1, schedule=SINGLE)
    torch.cuda.synchronize()
    assert normal.status() == 0


# ------------------------------------------------------------------ the three-pass schedule
# Segmented bf16 inputs run the single pass unless schedule = 1 asks for the
# three passes (summaries, a scan of them, outputs); that path stays pinned too.
@pytest.mark.parametrize("seg,vtile", [(1, 0), (3, 128), (5, 64)])
def test_three_passes_segments(seg, vtile):
    d = gi.draw(3000 + seg, 2, 700, 2, 128, 128, dtype="bf16", h0=True)
    say(f"[case] three passes: segments of {seg} chunks vtile={vtile}")
    o, ht = run_gpu(d, "bf16", segment_chunks=seg, value_tile=vtile, schedule=1)
    ro, rht = run_oracle(d)
    check_close("o", o, ro, TOL["bf16"], out_dtype="bf16")
    check_close("ht", ht, rht, TOL_HT)


def test_three_passes_packed():
    lengths = [1800, 3, 64, 129, 0, 700, 1, 65, 2500, 17, 300, 63]
    d = gi.draw(3100, 1, 0, 2, 128, 128, dtype="bf16", h0=True, lengths=lengths)
    say("[case] three passes: uneven packed lengths")
    o, ht = run_gpu(d, "bf16", segment_chunks=5, schedule=1)
    ro, rht = run_oracle(d)
    check_close("o", o, ro, TOL["bf16"], out_dtype="bf16")
    check_close("ht", ht, rht, TOL_HT)


def test_repeated_calls_on_many_short_chains():
    """States passed between workgroups of one launch are read and written
    device-coherently (agent-scope atomics): a reader on another die never sees
    a stale copy.  Small states (K = V = 64) and few chains leave lines in the
    caches longest, so the 1500-sequence input is run several times in a row,
    every result checked against the oracle."""
    import torch
    import chunkwise_gated_linear_amd as gla
    rng = np.random.default_rng(900)
    lengths = rng.integers(0, 140, size=1500).tolist()
    lengths[7] = 1300
    lengths[1200] = 900
    d = gi.draw(901, 1, 0, 1, 64, 64, dtype="bf16", h0=True, lengths=lengths)
    ro, rht = run_oracle(d)
    t = to_device(d, "bf16")
    for i in range(6):
        say(f"[case] single pass, 1500 packed sequences, call {i}")
        o, ht = gla.gla_fwd(t["q"], t["k"], t["v"], t["g"], h0=t["h0"], cu_seqlens=t["cu_seqlens"],
                            output_final_state=True, segment_chunks=3, schedule=SINGLE)
        torch.cuda.synchronize()
        check_close(f"call {i} o", o.float().cpu().numpy().astype(np.float64), ro, TOL["bf16"], out_dtype="bf16")
        check_close(f"call {i} ht", ht.cpu().numpy().astype(np.float64), rht, TOL_HT)
