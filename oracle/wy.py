"""fp64 CPU oracle for the WY-representation forward of the gated delta rule.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the tests, the smoke
check and the benchmark's CPU baseline may call it; the GPU library never does.

What is computed (page "fla/ops/gated_delta_rule/backends/triton_ascend/
wy_fast.py", recompute_w_u_fwd_kernel_npu and its wrapper
recompute_w_u_fwd_npu).  Tokens are cut into chunks of BT = 64 per sequence
(restarting at every packed sequence).  For chunk c of a sequence, value head
hv and the chunk's valid rows i, j (global token rows r0 + i, r0 + j):

    u[r0+i, hv, :] = sum_j A[r0+i, hv, j] * beta[r0+j, hv] * v[r0+j, hv, :]
    w[r0+i, hv, :] = sum_j A[r0+i, hv, j] * beta[r0+j, hv] * 2^g[r0+j, hv] * k[r0+j, hv // G, :]

with G = HV // H value heads per key head, and the factor 2^g dropped when no
g is given.  A holds, for each token row, that row of its chunk's BT x BT
matrix; columns j past the chunk's valid rows meet zero-padded rows and add
nothing.  The page applies exp2 to g, so g is a base-2 log gate here.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

BT = 64


def _offsets(B: int, T: int, cu_seqlens) -> np.ndarray:
    if cu_seqlens is None:
        return np.arange(B + 1, dtype=np.int64) * T
    if B != 1:
        raise ValueError("packed sequences need a batch of one")
    off = np.asarray(cu_seqlens, dtype=np.int64)
    if off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return off


def wy_reference(k: np.ndarray, v: np.ndarray, beta: np.ndarray, A: np.ndarray,
                 g: Optional[np.ndarray] = None,
                 cu_seqlens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """w [B, T, HV, K] and u [B, T, HV, V] in float64.

    k: [B, T, H, K]; v: [B, T, HV, V]; beta: [B, T, HV]; A: [B, T, HV, 64];
    g: [B, T, HV] or None.  Inputs of any float dtype are read as float64
    (exact for bf16 and fp32 data).  One matrix product per chunk and head
    (numpy's matmul in fp64), on exactly the rows the definition names.
    """
    B, T, H, K = k.shape
    HV, V = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, T) or HV % H != 0:
        raise ValueError("v must be [B, T, HV, V] with HV a multiple of H")
    if beta.shape != (B, T, HV) or A.shape != (B, T, HV, BT):
        raise ValueError("beta must be [B, T, HV] and A [B, T, HV, 64]")
    if g is not None and g.shape != (B, T, HV):
        raise ValueError("g must be [B, T, HV]")
    G = HV // H
    off = _offsets(B, T, cu_seqlens)
    kf = np.asarray(k, dtype=np.float64).reshape(B * T, H, K)
    vf = np.asarray(v, dtype=np.float64).reshape(B * T, HV, V)
    bf = np.asarray(beta, dtype=np.float64).reshape(B * T, HV)
    Af = np.asarray(A, dtype=np.float64).reshape(B * T, HV, BT)
    gf = None if g is None else np.asarray(g, dtype=np.float64).reshape(B * T, HV)
    w = np.zeros((B * T, HV, K))
    u = np.zeros((B * T, HV, V))
    for n in range(len(off) - 1):
        bos, eos = int(off[n]), int(off[n + 1])
        for r0 in range(bos, eos, BT):
            r1 = min(r0 + BT, eos)
            L = r1 - r0
            for hv in range(HV):
                Ac = Af[r0:r1, hv, :L]                      # rows i, columns j of the chunk
                scale = bf[r0:r1, hv]
                u[r0:r1, hv] = Ac @ (scale[:, None] * vf[r0:r1, hv])
                if gf is not None:
                    scale = scale * np.exp2(gf[r0:r1, hv])
                w[r0:r1, hv] = Ac @ (scale[:, None] * kf[r0:r1, hv // G])
    return w.reshape(B, T, HV, K), u.reshape(B, T, HV, V)
