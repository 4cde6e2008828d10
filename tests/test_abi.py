"""The C ABI library without a GPU: it loads, exports every function that
include/gla.h declares, and rejects invalid arguments on the host with the
documented status codes before anything is enqueued (no compute calls)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import chunkwise_gated_linear_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")
OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_SCALE, UNSUPPORTED, WORKSPACE, HIP = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gla.library_path()):
        from chunkwise_gated_linear_amd import build
        build.build()
    return gla.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["gla_bwd", "gla_bwd_workspace_bytes", "gla_fwd", "gla_fwd_noalloc",
                                    "gla_fwd_workspace_bytes", "gla_status_str", "gla_wy_fwd",
                                    "gla_wy_fwd_workspace_bytes"]


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gla.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert getattr(lib, name) is not None


def prob(**kw):
    base = dict(B=2, T=100, H=3, K=64, V=128, dtype=gla.GLA_BF16, n_seqs=2, chunk=64, scale=0.125,
                segment_chunks=1, packed=0, value_tile=0, wait_limit=0, HV=0, gate=0)
    base.update(kw)
    return gla.Problem(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def call(lib, p, q=FAKE, k=FAKE, v=FAKE, g=FAKE, cu=None, o=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.gla_fwd(ctypes.byref(p) if p is not None else None, q, k, v, g, None, cu, o, None,
                       ws, ws_bytes, None)


def call_noalloc(lib, p, q=FAKE, k=FAKE, v=FAKE, g=FAKE, cu=None, o=FAKE):
    return lib.gla_fwd_noalloc(ctypes.byref(p) if p is not None else None, q, k, v, g, None, cu, o, None,
                               None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), BAD_DTYPE),
    (dict(scale=0.0), BAD_SCALE),
    (dict(scale=-1.0), BAD_SCALE),
    (dict(scale=math.nan), BAD_SCALE),
    (dict(scale=math.inf), BAD_SCALE),
    (dict(chunk=32), UNSUPPORTED),
    (dict(K=8), UNSUPPORTED),           # K and V: multiples of 16 in [16, 256]
    (dict(K=24), UNSUPPORTED),
    (dict(K=272), UNSUPPORTED),
    (dict(V=8), UNSUPPORTED),
    (dict(V=40), UNSUPPORTED),
    (dict(V=272), UNSUPPORTED),
    (dict(value_tile=32), UNSUPPORTED),
    (dict(T=-1), BAD_SHAPE),
    (dict(H=0), BAD_SHAPE),
    (dict(H=20000, K=256), BAD_SHAPE),  # one chunk of one tensor would span 2^30 bytes or more
    (dict(n_seqs=3), BAD_SHAPE),        # without packing N must equal B
    (dict(packed=1), BAD_SHAPE),        # packing needs B == 1
    (dict(segment_chunks=-2), BAD_SHAPE),
    (dict(wait_limit=-2), BAD_SHAPE),
    (dict(HV=4), BAD_SHAPE),            # value heads must be a multiple of the key heads
    (dict(HV=-3), BAD_SHAPE),
    (dict(gate=2), UNSUPPORTED),
    (dict(schedule=3), UNSUPPORTED),    # the backward's walk
    (dict(schedule=4), UNSUPPORTED),
    (dict(schedule=-1), UNSUPPORTED),
])
def test_invalid_problems_are_rejected(lib, kw, code):
    p = prob(**kw)
    assert call(lib, p) == code
    assert call_noalloc(lib, p) == code
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("dtype", [gla.GLA_BF16, gla.GLA_F32])
@pytest.mark.parametrize("K", [16, 48, 64, 96, 128, 144, 256])
@pytest.mark.parametrize("V", [16, 96, 128, 256])
def test_every_multiple_of_16_up_to_256_is_accepted(lib, dtype, K, V):
    p = prob(dtype=dtype, K=K, V=V)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) != ctypes.c_size_t(-1).value


def up(x):
    return (x + 255) // 256 * 256


WS_HEADER = 256  # status word + padding at the start of every workspace


def test_workspace_size_and_check(lib):
    # B=2, T=1000 -> 16 chunks per sequence; 2 chunks per segment -> 8 segments each.
    # Three passes: segment states and decay products
    p = prob(T=1000, K=64, V=128, H=3, segment_chunks=2, schedule=1)
    slots = 2 * 8
    expect = WS_HEADER + up(slots * 3 * 64 * 128 * 4) + up(slots * 3 * 64 * 4)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) == expect
    # fixed-length sequences default to three passes
    p0 = prob(T=1000, K=64, V=128, H=3, segment_chunks=2, schedule=0)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p0)) == expect
    # one pass: also an item counter and one flag per (segment, head, value slice)
    link = up((1 + slots * 3) * 4)
    p1 = prob(T=1000, K=64, V=128, H=3, segment_chunks=2, schedule=2)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p1)) == expect + link
    # fp32 runs three passes whatever the schedule
    p2 = prob(T=1000, K=64, V=128, H=3, segment_chunks=2, schedule=2, dtype=gla.GLA_F32)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p2)) == expect
    assert call(lib, p, ws=None, ws_bytes=0) == WORKSPACE
    assert call(lib, p, ws=FAKE, ws_bytes=expect - 1) == WORKSPACE
    assert call(lib, p1, ws=FAKE, ws_bytes=expect + link - 1) == WORKSPACE
    # one segment per sequence: the status header only
    p1 = prob(T=1000, segment_chunks=16)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p1)) == WS_HEADER
    assert call(lib, p1, ws=None, ws_bytes=0) == WORKSPACE
    # packed: slots bounded by N + ceil((ceil(T/64) + N) / R), plus N+1 offsets and the order
    pv = prob(B=1, T=1000, n_seqs=5, packed=1, segment_chunks=3)
    slots_v = 5 + -(-(16 + 5) // 3)
    expect_v = WS_HEADER + up(slots_v * 3 * 64 * 128 * 4) + up(slots_v * 3 * 64 * 4) + up((6 + slots_v) * 4)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(pv)) == expect_v + up((1 + slots_v * 3) * 4)
    pv.schedule = 1
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(pv)) == expect_v


def test_workspace_of_split_keys(lib):
    # K > 128 runs as two key blocks (here 80 + 64); the first block's fp32
    # partial output [B, T, H, V] lives in the workspace, segment summaries are
    # sized for the wider block
    p = prob(T=1000, K=144, V=96, H=3, segment_chunks=16)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) == WS_HEADER + up(2 * 1000 * 3 * 96 * 4)
    p2 = prob(T=1000, K=144, V=96, H=3, segment_chunks=2)
    slots = 2 * 8
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p2)) == (WS_HEADER + up(slots * 3 * 80 * 96 * 4)
                                                            + up(slots * 3 * 80 * 4) + up(2 * 1000 * 3 * 96 * 4))


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    # the no-allocation entry point holds 64 MiB of device scratch; a larger
    # workspace (here the fp32 partial output of split keys, 328 MB) is refused
    # on the host before anything touches the device
    big = prob(B=1, T=40000, H=8, K=256, V=256, n_seqs=1, segment_chunks=0)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(big)) > (64 << 20)
    assert call_noalloc(lib, big) == WORKSPACE
    assert call_noalloc(lib, None) == NULL_ARG
    assert call_noalloc(lib, prob(), q=None) == NULL_ARG


def test_value_heads_size_the_workspace(lib):
    # states and segment summaries exist per value head
    p = prob(T=1000, K=64, V=128, H=3, HV=6, segment_chunks=2, gate=1)
    slots = 2 * 8
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) == (WS_HEADER + up(slots * 6 * 64 * 128 * 4)
                                                           + up(slots * 6 * 64 * 4))
    p.schedule = 2
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) == (WS_HEADER + up(slots * 6 * 64 * 128 * 4)
                                                           + up(slots * 6 * 64 * 4) + up((1 + slots * 6) * 4))


def test_status_strings(lib):
    seen = set()
    for code in range(8):
        s = lib.gla_status_str(code).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.gla_status_str(99).decode() == "unknown status"


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        gla.gla_fwd(x, x, x, x)


# ---------------------------------------------------------------- backward entry point

def call_bwd(lib, p, ws=FAKE, ws_bytes=1 << 40, cu=None, dq=FAKE, do=FAKE):
    return lib.gla_bwd(ctypes.byref(p) if p is not None else None, FAKE, FAKE, FAKE, FAKE, None, cu,
                       do, None, dq, FAKE, FAKE, FAKE, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), BAD_DTYPE),
    (dict(scale=0.0), BAD_SCALE),
    (dict(chunk=32), UNSUPPORTED),
    (dict(K=24), UNSUPPORTED),
    (dict(K=272), UNSUPPORTED),         # the backward takes what the forward takes
    (dict(V=272), UNSUPPORTED),
    (dict(n_seqs=3), BAD_SHAPE),
    (dict(HV=4), BAD_SHAPE),
    (dict(gate=2), UNSUPPORTED),
    (dict(schedule=4), UNSUPPORTED),    # 3, the walk, is the backward's own
    (dict(schedule=-1), UNSUPPORTED),
])
def test_backward_rejects_invalid_problems(lib, kw, code):
    p = prob(**kw)
    assert call_bwd(lib, p) == code
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(p)) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("schedule", [0, 1, 2, 3])
def test_backward_schedules_share_one_workspace(lib, schedule):
    # every schedule runs in the workspace the size query gives for schedule 0
    p0, p = prob(B=2, T=1000, H=3), prob(B=2, T=1000, H=3, schedule=schedule)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(p)) == lib.gla_bwd_workspace_bytes(ctypes.byref(p0))


def test_backward_null_arguments(lib):
    assert call_bwd(lib, None) == NULL_ARG
    assert call_bwd(lib, prob(), dq=None) == NULL_ARG
    assert call_bwd(lib, prob(), do=None) == NULL_ARG
    assert call_bwd(lib, prob(B=1, n_seqs=1, packed=1)) == NULL_ARG   # packed without cu_seqlens


@pytest.mark.parametrize("dtype", [gla.GLA_BF16, gla.GLA_F32])
@pytest.mark.parametrize("K", [16, 48, 64, 128, 144, 256])
@pytest.mark.parametrize("V", [16, 96, 128, 144, 256])
def test_backward_accepts_its_widths(lib, dtype, K, V):
    p = prob(dtype=dtype, K=K, V=V)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(p)) != ctypes.c_size_t(-1).value


def test_backward_workspace_size_and_check(lib):
    # B=2, T=1000: 16 chunks per sequence, one chunk per slot; the state and
    # the state gradient of every chunk, the chunk decays, the flags
    B, T, H, K, V = 2, 1000, 3, 64, 128
    p = prob(B=B, T=T, H=H, K=K, V=V)
    slots = 2 * 16
    states = up(slots * H * K * V * 4)
    decays = up(slots * H * K * 4)
    expect = WS_HEADER + states + states + decays + up(slots * H * 4)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(p)) == expect
    assert call_bwd(lib, p, ws=None, ws_bytes=0) == WORKSPACE
    assert call_bwd(lib, p, ws_bytes=expect - 1) == WORKSPACE
    # value-head groups add the fp32 shares of dq and dk per value head
    pg = prob(B=B, T=T, H=H, K=K, V=V, HV=6)
    states6, decays6 = up(slots * 6 * K * V * 4), up(slots * 6 * K * 4)
    expect_g = WS_HEADER + 2 * states6 + decays6 + up(slots * 6 * 4) + 2 * up(B * T * 6 * K * 4)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(pg)) == expect_g
    # packed: the slot table (N + 1 offsets and the order) comes first
    pv = prob(B=1, T=1000, n_seqs=5, packed=1, H=H, K=K, V=V)
    slots_v = 5 + 16 + 5
    sv, dv_ = up(slots_v * H * K * V * 4), up(slots_v * H * K * 4)
    # ... and the chained scan's task table (a count and an int pair per slot)
    # with its plan's scratch (3 cmax + 4 + N words, cmax = ceil(T / 64))
    plan_v = up((2 + 2 * slots_v) * 4) + up((3 * 16 + 4 + 5) * 4)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(pv)) == (WS_HEADER + up((6 + slots_v) * 4) + 2 * sv + dv_
                                                             + up(slots_v * H * 4) + plan_v)
    # V = 256: two value slices of 128 columns run one after the other over
    # state tables of 128 columns, with fp32 shares of dq, dk and dg per slice,
    # and one slice's columns of h0, dht and dh0 staged for the chained scan
    pw = prob(B=B, T=T, H=H, K=K, V=256)
    sw = up(slots * H * K * 128 * 4)
    shares = up(2 * B * T * H * K * 4)
    staged = 3 * up(B * H * K * 128 * 4)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(pw)) == (WS_HEADER + 2 * sw + decays + up(slots * H * 4)
                                                             + 3 * shares + staged)
    pwh = prob(B=B, T=T, H=H, K=K, V=256, gate=gla.GATE_PER_HEAD)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(pwh)) == (WS_HEADER + 2 * sw + decays + up(slots * H * 4)
                                                              + 2 * shares + up(2 * B * T * H * 4) + staged)
    # K = 192: two key blocks of 96 keys over state tables of 96 keys, dv as
    # fp32 shares per block, and the staged boundary rows of one block
    pk = prob(B=B, T=T, H=H, K=192, V=V)
    sk = up(slots * H * 96 * V * 4)
    assert lib.gla_bwd_workspace_bytes(ctypes.byref(pk)) == (WS_HEADER + 2 * sk + up(slots * H * 96 * 4)
                                                             + up(slots * H * 4) + up(2 * B * T * H * V * 4)
                                                             + 3 * up(B * H * 96 * V * 4))


# ---------------------------------------------------------------- WY-representation forward

def wy_prob(**kw):
    base = dict(B=2, T=100, H=2, HV=4, K=64, V=128, dtype=gla.GLA_BF16, n_seqs=2, chunk=64, packed=0)
    base.update(kw)
    return gla.WyProblem(**base)


def call_wy(lib, p, ws=FAKE, ws_bytes=1 << 40, cu=None, k=FAKE):
    return lib.gla_wy_fwd(ctypes.byref(p) if p is not None else None, k, FAKE, FAKE, FAKE, None, cu,
                          FAKE, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), BAD_DTYPE),
    (dict(chunk=32), UNSUPPORTED),
    (dict(K=24), UNSUPPORTED),
    (dict(V=272), UNSUPPORTED),
    (dict(HV=3), BAD_SHAPE),
    (dict(n_seqs=3), BAD_SHAPE),
    (dict(packed=1), BAD_SHAPE),
    (dict(T=-1), BAD_SHAPE),
])
def test_wy_rejects_invalid_problems(lib, kw, code):
    p = wy_prob(**kw)
    assert call_wy(lib, p) == code
    assert lib.gla_wy_fwd_workspace_bytes(ctypes.byref(p)) == ctypes.c_size_t(-1).value


def test_wy_null_arguments_and_workspace(lib):
    assert call_wy(lib, None) == NULL_ARG
    assert call_wy(lib, wy_prob(), k=None) == NULL_ARG
    assert call_wy(lib, wy_prob(B=1, n_seqs=1, packed=1)) == NULL_ARG  # packed without cu_seqlens
    assert lib.gla_wy_fwd_workspace_bytes(ctypes.byref(wy_prob())) == WS_HEADER
    pv = wy_prob(B=1, T=1000, n_seqs=5, packed=1)
    slots = 5 + 16 + 5
    assert lib.gla_wy_fwd_workspace_bytes(ctypes.byref(pv)) == WS_HEADER + up((6 + slots) * 4)
    assert call_wy(lib, wy_prob(), ws=None, ws_bytes=0) == WORKSPACE
