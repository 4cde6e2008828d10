"""CPU oracle for the chunkwise gated linear attention forward (fp64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the GPU library and its Python binding never
do, and nothing here imports them.

``gla_reference`` runs the token-by-token recurrence of ``gla_oracle.c``
(S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T, o_t = scale q_t^T S_t, per sequence
and head, in double precision) on float32 inputs.  The definition and its
sources are stated in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

from .wy import wy_reference  # noqa: E402,F401  (WY-representation forward, numpy fp64)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.gla_oracle_fwd.argtypes = [i64, p, i64, i64, i64, p, p, p, p, p,
                                       ctypes.c_double, p, p, ctypes.c_int]
        lib.gla_oracle_fwd.restype = ctypes.c_int
        lib.gla_oracle_fwd_heads.argtypes = [i64, p, i64, i64, i64, i64, ctypes.c_int, p, p, p, p, p,
                                             ctypes.c_double, p, p, ctypes.c_int]
        lib.gla_oracle_fwd_heads.restype = ctypes.c_int
        lib.gla_oracle_bwd.argtypes = [i64, p, i64, i64, i64, p, p, p, p, p, ctypes.c_double, p, p,
                                       p, p, p, p, p, ctypes.c_int]
        lib.gla_oracle_bwd.restype = ctypes.c_int
        lib.gla_oracle_max_threads.argtypes = []
        lib.gla_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gla_oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def gla_reference(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                  h0: Optional[np.ndarray] = None, cu_seqlens: Optional[np.ndarray] = None,
                  scale: Optional[float] = None, output_final_state: bool = True,
                  threads: int = 0) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Token-by-token fp64 recurrence.

    q, k: [B, T, H, K]; v: [B, T, HV, V] with HV a multiple of H (value head hv
    reads key head hv // (HV // H)); g: [B, T, HV, K] (a decay per key) or
    [B, T, HV] (one decay per value head and token).  Any float dtype; converted
    to float32, which is exact for bf16 and fp32 data.  h0: [N, HV, K, V] or None.
    cu_seqlens: [N+1] offsets into the packed token axis (requires B == 1) or None.
    scale: None means K ** -0.5.
    Returns o [B, T, HV, V] float64 and ht [N, HV, K, V] float64 (or None).
    """
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    per_head = g.ndim == 3
    if k.shape != (B, T, H, K) or v.shape[:2] != (B, T) or HV % H != 0:
        raise ValueError("shape mismatch")
    if g.shape != ((B, T, HV) if per_head else (B, T, HV, K)):
        raise ValueError("g must be [B, T, HV, K] or [B, T, HV]")
    if scale is None:
        scale = K ** -0.5
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences need a batch of one")
        offsets = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        if offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    else:
        offsets = np.arange(B + 1, dtype=np.int64) * T
    N = len(offsets) - 1
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    qf, kf, vf, gf = f32(q), f32(k), f32(v), f32(g)
    hf = None
    if h0 is not None:
        if h0.shape != (N, HV, K, V):
            raise ValueError(f"h0 must be [{N}, {HV}, {K}, {V}]")
        hf = np.ascontiguousarray(h0, dtype=np.float64)
    o = np.zeros((B, T, HV, V), dtype=np.float64)
    ht = np.zeros((N, HV, K, V), dtype=np.float64) if output_final_state else None
    rc = _load().gla_oracle_fwd_heads(N, _ptr(offsets), H, HV, K, V, 1 if per_head else 0,
                                      _ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(hf), float(scale),
                                      _ptr(o), _ptr(ht), int(threads))
    if rc != 0:
        raise RuntimeError("oracle failed")
    return o, ht


def gla_reference_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, do: np.ndarray,
                      h0: Optional[np.ndarray] = None, dht: Optional[np.ndarray] = None,
                      cu_seqlens: Optional[np.ndarray] = None, scale: Optional[float] = None,
                      threads: int = 0):
    """Gradients of L = sum(do * o) + sum(dht * ht) by the reverse token recurrence (fp64).

    q, k: [B, T, H, K]; v, do: [B, T, HV, V]; g: [B, T, HV, K] (a decay per key)
    or [B, T, HV] (one per value head); h0, dht: [N, HV, K, V] or None.
    Returns dq, dk [B, T, H, K], dv [B, T, HV, V], dg (g's shape), dh0 [N, HV, K, V],
    float64.

    Value-head groups and per-head gates reduce exactly to the plain method
    (page "fla/ops/gated_delta_rule/backends/triton_ascend/wy_fast.py" maps value
    head hv to key head hv // (HV // H)): value head hv is an independent plain
    head whose q, k are key head hv // G's, and a per-head gate is the same
    decay on every key.  So the plain backward runs on q, k repeated per value
    head and the gate broadcast over keys, and the chain rule sums back: dq, dk
    of a key head over its G value heads, a per-head dg over keys.
    """
    B, T, H, K = q.shape
    HV = v.shape[2]
    if HV % H != 0 or v.shape[:2] != (B, T):
        raise ValueError("v must be [B, T, HV, V] with HV a multiple of H")
    per_head = g.shape == (B, T, HV)
    if not per_head and g.shape != (B, T, HV, K):
        raise ValueError("g must be [B, T, HV, K] or [B, T, HV]")
    if HV != H or per_head:
        G = HV // H
        qe = np.repeat(np.asarray(q), G, axis=2)
        ke = np.repeat(np.asarray(k), G, axis=2)
        ge = np.broadcast_to(np.asarray(g)[..., None], (B, T, HV, K)) if per_head else np.asarray(g)
        dq, dk, dv, dg, dh0 = _reference_bwd_plain(qe, ke, v, ge, do, h0, dht, cu_seqlens, scale, threads)
        dq = dq.reshape(B, T, H, G, K).sum(axis=3)
        dk = dk.reshape(B, T, H, G, K).sum(axis=3)
        if per_head:
            dg = dg.sum(axis=3)
        return dq, dk, dv, dg, dh0
    return _reference_bwd_plain(q, k, v, g, do, h0, dht, cu_seqlens, scale, threads)


def _reference_bwd_plain(q, k, v, g, do, h0, dht, cu_seqlens, scale, threads):
    """The plain method (HV = H, a decay per key) through gla_oracle_bwd.
    Memory is T * K * V doubles per (sequence, head) job: for test sizes."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, V) or do.shape != v.shape:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = K ** -0.5
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences need a batch of one")
        offsets = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        if offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    else:
        offsets = np.arange(B + 1, dtype=np.int64) * T
    N = len(offsets) - 1
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    f64 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float64)
    for a in (h0, dht):
        if a is not None and a.shape != (N, H, K, V):
            raise ValueError(f"h0 and dht must be [{N}, {H}, {K}, {V}]")
    dq = np.zeros((B, T, H, K)); dk = np.zeros((B, T, H, K)); dg = np.zeros((B, T, H, K))
    dv = np.zeros((B, T, H, V)); dh0 = np.zeros((N, H, K, V))
    qf, kf, vf, gf, dof = f32(q), f32(k), f32(v), f32(g), f32(do)
    h0d, dhtd = f64(h0), f64(dht)
    rc = _load().gla_oracle_bwd(N, _ptr(offsets), H, K, V, _ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf),
                                _ptr(h0d), float(scale), _ptr(dof), _ptr(dhtd), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(dg), _ptr(dh0), int(threads))
    if rc != 0:
        raise RuntimeError("oracle failed")
    return dq, dk, dv, dg, dh0
