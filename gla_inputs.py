"""Seeded synthetic inputs for the chunkwise gated linear attention forward.

This module is shared by the CPU oracle side (tests, the CPU baseline timing)
and the GPU side (tests, bench, smoke).  It only draws random numbers and
rounds them to the storage dtype; it contains none of the method's arithmetic.

Workloads (the five measured configurations; every input is synthetic):

  small   B=1  H=2  T=256   K=V=64        fp32 q/k/v, no h0
  c2048   B=8  H=16 T=2048  K=V=128       bf16 q/k/v, final state stored
  c4096   B=4  H=32 T=4096  K=128 V=256   bf16 q/k/v, h0 ~ 0.1*N(0,1), final state
  varlen  16 packed sequences, lengths uniform in [256, 4096], H=16 K=V=128 bf16
  long    B=1  H=32 T=65536 K=V=128       bf16 q/k/v, final state stored

Recipe, identical for every workload: one ``numpy.random.default_rng(seed)``
per workload, draws in the fixed order [lengths], q, k, v, z, [h0];
q, k, v ~ N(0,1) drawn in float32 then rounded to bf16 (round to nearest
even) when the workload is bf16; g = logsigmoid(z)/16 in float32 with
z ~ N(0,1) (one gate per key, per token and head); h0 = 0.1 * N(0,1) float32.
The gate formula is the workload's recipe for a per-key log decay in (-inf, 0).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "draw", "draw_wy", "logsigmoid_f32",
           "to_bf16_f32", "array_digest"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int           # tokens per sequence (fixed length); total tokens for varlen
    K: int
    V: int
    dtype: str       # "fp32" or "bf16": dtype of q, k, v and o
    h0: bool
    ht: bool
    seed: int
    n_seqs: int = 0  # >0 marks a packed variable-length workload (B must be 1)
    len_lo: int = 0
    len_hi: int = 0
    chunk: int = 64

    @property
    def varlen(self) -> bool:
        return self.n_seqs > 0


WORKLOADS = {
    "small": Workload("small", 1, 2, 256, 64, 64, "fp32", False, True, 1001),
    "c2048": Workload("c2048", 8, 16, 2048, 128, 128, "bf16", False, True, 1002),
    "c4096": Workload("c4096", 4, 32, 4096, 128, 256, "bf16", True, True, 1003),
    "varlen": Workload("varlen", 1, 16, 0, 128, 128, "bf16", False, False, 1004,
                       n_seqs=16, len_lo=256, len_hi=4096),
    "long": Workload("long", 1, 32, 65536, 128, 128, "bf16", False, True, 1005),
}


def logsigmoid_f32(z: np.ndarray) -> np.ndarray:
    """Numerically stable log(sigmoid(z)) = min(z, 0) - log1p(exp(-|z|)), in float32."""
    z = z.astype(np.float32, copy=False)
    return (np.minimum(z, 0) - np.log1p(np.exp(-np.abs(z)))).astype(np.float32)


def to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the values as float32.

    NaN is kept as NaN; the rounding is done on the bit pattern so it needs no torch.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def array_digest(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is None:
            h.update(b"none")
            continue
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()[:16]


def draw(seed: int, B: int, T: int, H: int, K: int, V: int, dtype: str = "bf16",
         h0: bool = False, lengths: Optional[list] = None, gate_scale: float = 1.0 / 16.0,
         HV: Optional[int] = None, gate: str = "key"):
    """Draw one input set from ``numpy.random.default_rng(seed)``.

    Returns a dict of float32 numpy arrays (q, k, v already rounded to bf16 when
    ``dtype == "bf16"``): q, k [B, T, H, K]; v [B, T, HV, V]; g [B, T, HV, K]
    (``gate == "key"``) or [B, T, HV] (``gate == "head"``); h0 [N, HV, K, V] or
    None; cu_seqlens int32 [N+1] or None.  HV defaults to H.  With ``lengths``
    the input is packed (B = 1, T = sum(lengths)).
    """
    return _draw_from(np.random.default_rng(seed), B, T, H, K, V, dtype, h0, lengths, gate_scale,
                      HV, gate)


def make_inputs(w: Workload):
    """Inputs of a named workload, drawn from its own seed in the documented order."""
    if w.varlen:
        rng = np.random.default_rng(w.seed)
        lengths = rng.integers(w.len_lo, w.len_hi, size=w.n_seqs, endpoint=True).tolist()
        d = _draw_from(rng, 1, 0, w.H, w.K, w.V, w.dtype, w.h0, lengths, 1.0 / 16.0, None, "key")
        d["lengths"] = lengths
        return d
    return draw(w.seed, w.B, w.T, w.H, w.K, w.V, w.dtype, w.h0)


def _draw_from(rng, B, T, H, K, V, dtype, h0, lengths, gate_scale, HV=None, gate="key"):
    HV = H if HV is None else HV
    if HV % H != 0 or gate not in ("key", "head"):
        raise ValueError("HV must be a multiple of H; gate is 'key' or 'head'")
    cu = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, T = 1, int(cu[-1])
    N = len(lengths) if lengths is not None else B
    q = rng.standard_normal((B, T, H, K), dtype=np.float32)
    k = rng.standard_normal((B, T, H, K), dtype=np.float32)
    v = rng.standard_normal((B, T, HV, V), dtype=np.float32)
    z = rng.standard_normal((B, T, HV, K) if gate == "key" else (B, T, HV), dtype=np.float32)
    g = (logsigmoid_f32(z) * np.float32(gate_scale)).astype(np.float32)
    del z
    h = None
    if h0:
        h = (np.float32(0.1) * rng.standard_normal((N, HV, K, V), dtype=np.float32)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = to_bf16_f32(q), to_bf16_f32(k), to_bf16_f32(v)
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype}")
    return {"q": q, "k": k, "v": v, "g": g, "h0": h, "cu_seqlens": cu}


def draw_wy(seed: int, B: int, T: int, H: int, K: int, V: int, dtype: str = "bf16",
            HV: Optional[int] = None, lengths: Optional[list] = None, use_g: bool = True,
            dense_A: bool = False, chunk: int = 64):
    """Inputs of the WY-representation forward, from ``numpy.random.default_rng(seed)``.

    Draw order: [lengths given], k, v, beta, A, [g].  k [B,T,H,K] and v
    [B,T,HV,V] ~ N(0,1); beta [B,T,HV] = sigmoid(N(0,1)); A [B,T,HV,chunk]: for
    each token, the row of its chunk's matrix, unit diagonal and N(0,1)/8 below
    it, zero above (a unit lower-triangular matrix, the shape of a WY inverse);
    with ``dense_A`` every entry of the row is N(0,1)/8 (columns past a partial
    chunk's rows included).  g [B,T,HV] = 4 logsigmoid(N(0,1)) (a log gate in
    (-inf, 0)).  k, v and A are rounded to bf16 for bf16; beta and g are float32.
    Returns k, v, beta, A, g (or None), cu_seqlens (or None).
    """
    rng = np.random.default_rng(seed)
    HV = H if HV is None else HV
    if HV % H != 0:
        raise ValueError("HV must be a multiple of H")
    cu = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, T = 1, int(cu[-1])
    k = rng.standard_normal((B, T, H, K), dtype=np.float32)
    v = rng.standard_normal((B, T, HV, V), dtype=np.float32)
    zb = rng.standard_normal((B, T, HV), dtype=np.float32)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    A = (rng.standard_normal((B, T, HV, chunk), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    if not dense_A:
        # position of each token inside its chunk (chunks restart per sequence)
        offs = cu if cu is not None else np.arange(B + 1, dtype=np.int64) * T
        pos = np.zeros(B * T, dtype=np.int64)
        for n in range(len(offs) - 1):
            pos[offs[n]:offs[n + 1]] = np.arange(offs[n + 1] - offs[n]) % chunk
        col = np.arange(chunk)[None, :]
        pos = pos.reshape(B, T)[:, :, None, None]
        A = np.where(col[None, None] < pos, A, np.where(col[None, None] == pos, np.float32(1.0),
                                                         np.float32(0.0))).astype(np.float32)
    g = (np.float32(4.0) * logsigmoid_f32(rng.standard_normal((B, T, HV), dtype=np.float32))).astype(
        np.float32) if use_g else None
    if dtype == "bf16":
        k, v, A = to_bf16_f32(k), to_bf16_f32(v), to_bf16_f32(A)
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype}")
    return {"k": k, "v": v, "beta": beta, "A": A, "g": g, "cu_seqlens": cu}
