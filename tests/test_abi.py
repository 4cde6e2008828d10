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
    assert declared_functions() == ["gla_fwd", "gla_fwd_workspace_bytes", "gla_status_str"]


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gla.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert getattr(lib, name) is not None


def prob(**kw):
    base = dict(B=2, T=100, H=3, K=64, V=128, dtype=gla.GLA_BF16, n_seqs=2, chunk=64, scale=0.125,
                segment_chunks=1, packed=0)
    base.update(kw)
    return gla.Problem(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def call(lib, p, q=FAKE, k=FAKE, v=FAKE, g=FAKE, cu=None, o=FAKE, ws=None, ws_bytes=0):
    return lib.gla_fwd(ctypes.byref(p) if p is not None else None, q, k, v, g, None, cu, o, None,
                       ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), BAD_DTYPE),
    (dict(scale=0.0), BAD_SCALE),
    (dict(scale=-1.0), BAD_SCALE),
    (dict(scale=math.nan), BAD_SCALE),
    (dict(scale=math.inf), BAD_SCALE),
    (dict(chunk=32), UNSUPPORTED),
    (dict(K=48), UNSUPPORTED),
    (dict(K=256), UNSUPPORTED),
    (dict(K=16), UNSUPPORTED),          # bf16 needs K in {32, 64, 128}
    (dict(V=96), UNSUPPORTED),
    (dict(T=-1), BAD_SHAPE),
    (dict(H=0), BAD_SHAPE),
    (dict(n_seqs=3), BAD_SHAPE),        # without packing N must equal B
    (dict(packed=1), BAD_SHAPE),        # packing needs B == 1
    (dict(segment_chunks=-2), BAD_SHAPE),
])
def test_invalid_problems_are_rejected(lib, kw, code):
    p = prob(**kw)
    assert call(lib, p) == code
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) == ctypes.c_size_t(-1).value


def test_fp32_accepts_k16(lib):
    p = prob(dtype=gla.GLA_F32, K=16)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) != ctypes.c_size_t(-1).value


def test_null_arguments(lib):
    assert call(lib, None) == NULL_ARG
    assert call(lib, prob(), q=None) == NULL_ARG
    assert call(lib, prob(), o=None) == NULL_ARG
    # packed problem without offsets, offsets without a packed problem
    assert call(lib, prob(B=1, n_seqs=4, packed=1), cu=None) == NULL_ARG
    assert call(lib, prob(), cu=FAKE) == NULL_ARG


def test_workspace_size_and_check(lib):
    # B=2, T=1000 -> 16 chunks per sequence; 2 chunks per segment -> 8 segments each
    p = prob(T=1000, K=64, V=128, H=3, segment_chunks=2)
    up = lambda x: (x + 255) // 256 * 256
    slots = 2 * 8
    expect = up(slots * 3 * 64 * 128 * 4) + up(slots * 3 * 64 * 4)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p)) == expect
    assert call(lib, p, ws=None, ws_bytes=0) == WORKSPACE
    assert call(lib, p, ws=FAKE, ws_bytes=expect - 1) == WORKSPACE
    # one segment per sequence needs no workspace
    p1 = prob(T=1000, segment_chunks=16)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(p1)) == 0
    # packed: slots bounded by N + ceil((ceil(T/64) + N) / R), plus N+1 offsets
    pv = prob(B=1, T=1000, n_seqs=5, packed=1, segment_chunks=3)
    slots_v = 5 + -(-(16 + 5) // 3)
    expect_v = up(slots_v * 3 * 64 * 128 * 4) + up(slots_v * 3 * 64 * 4) + up(6 * 4)
    assert lib.gla_fwd_workspace_bytes(ctypes.byref(pv)) == expect_v


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
