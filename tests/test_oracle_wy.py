"""Pins for the fp64 WY-representation oracle (no GPU).

oracle.wy_reference (page "fla/ops/gated_delta_rule/backends/triton_ascend/
wy_fast.py", recompute_w_u_fwd_kernel_npu) is checked against things that
are not itself:

* A = the identity in every chunk: u = beta v and w = beta 2^g k (closed form);
* A = lower-triangular ones: u and w are chunk-wise cumulative sums, taken with
  numpy.cumsum;
* packed sequences equal the same sequences run one by one;
* value-head groups: value head hv reads key head hv // G (equal to a plain run
  whose k repeats each key head G times);
* columns of A past a partial chunk's rows do not matter;
* planted mistakes (A transposed within chunks, exp instead of exp2, the head
  mapping hv % H) each fail one of the pins above.
"""
import numpy as np
import pytest

import gla_inputs as gi
import oracle

C = 64


def chunk_pos(B, T, cu):
    offs = cu if cu is not None else np.arange(B + 1) * T
    pos = np.zeros(B * T, dtype=np.int64)
    start = np.zeros(B * T, dtype=np.int64)
    for n in range(len(offs) - 1):
        a, b = int(offs[n]), int(offs[n + 1])
        pos[a:b] = np.arange(b - a) % C
        start[a:b] = a + (np.arange(b - a) // C) * C
    return pos.reshape(B, T), start.reshape(B, T)


def structured_A(B, T, HV, cu, kind):
    pos, _ = chunk_pos(B, T, cu)
    col = np.arange(C)[None, None, None, :]
    p = pos[:, :, None, None]
    if kind == "identity":
        A = (col == p).astype(np.float64)
    else:  # lower-triangular ones
        A = (col <= p).astype(np.float64)
    return np.broadcast_to(A, (B, T, HV, C)).copy()


def chunk_cumsum(x, B, T, cu):
    """Inclusive cumulative sum over the tokens of each chunk (axis 1 of [B, T, HV, W])."""
    _, start = chunk_pos(B, T, cu)
    out = np.zeros_like(x)
    for b in range(B):
        t = 0
        while t < T:
            s = start[b, t]
            e = t
            while e < T and start[b, e] == s:
                e += 1
            out[b, t:e] = np.cumsum(x[b, t:e], axis=0)
            t = e
    return out


def close(a, b, tol=1e-12):
    return np.allclose(a, b, rtol=tol, atol=tol)


@pytest.mark.parametrize("packed", [False, True])
def test_identity_A_is_the_scaled_rows(packed):
    lengths = [70, 0, 5, 130] if packed else None
    d = gi.draw_wy(11, 2, 100, 2, 16, 8, dtype="fp32", HV=4, lengths=lengths)
    B, T = d["k"].shape[:2]
    A = structured_A(B, T, 4, d["cu_seqlens"], "identity")
    w, u = oracle.wy_reference(d["k"], d["v"], d["beta"], A, d["g"], cu_seqlens=d["cu_seqlens"])
    kk = np.repeat(d["k"].astype(np.float64), 2, axis=2)
    sc = d["beta"].astype(np.float64)
    assert close(u, sc[..., None] * d["v"])
    assert close(w, (sc * np.exp2(d["g"].astype(np.float64)))[..., None] * kk)


@pytest.mark.parametrize("packed", [False, True])
def test_lower_ones_A_is_a_chunk_cumsum(packed):
    lengths = [64, 65, 1, 200] if packed else None
    d = gi.draw_wy(12, 2, 150, 1, 8, 4, dtype="fp32", lengths=lengths)
    B, T = d["k"].shape[:2]
    cu = d["cu_seqlens"]
    A = structured_A(B, T, 1, cu, "ones")
    w, u = oracle.wy_reference(d["k"], d["v"], d["beta"], A, d["g"], cu_seqlens=cu)
    sc = d["beta"].astype(np.float64)
    assert close(u, chunk_cumsum(sc[..., None] * d["v"], B, T, cu), 1e-10)
    sg = sc * np.exp2(d["g"].astype(np.float64))
    assert close(w, chunk_cumsum(sg[..., None] * d["k"].astype(np.float64), B, T, cu), 1e-10)


def test_without_gate_w_uses_beta_only():
    d = gi.draw_wy(13, 1, 80, 1, 8, 8, dtype="fp32", use_g=False)
    B, T = d["k"].shape[:2]
    A = structured_A(B, T, 1, None, "identity")
    w, _ = oracle.wy_reference(d["k"], d["v"], d["beta"], A, None)
    assert close(w, d["beta"][..., None].astype(np.float64) * d["k"])


def test_packed_equals_separate_sequences():
    lengths = [30, 64, 129, 0, 7]
    d = gi.draw_wy(14, 1, 0, 2, 16, 8, dtype="fp32", HV=2, lengths=lengths, dense_A=True)
    w, u = oracle.wy_reference(d["k"], d["v"], d["beta"], d["A"], d["g"], cu_seqlens=d["cu_seqlens"])
    cu = d["cu_seqlens"]
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda x: None if x is None else x[:, a:b]
        ws, us = oracle.wy_reference(sl(d["k"]), sl(d["v"]), sl(d["beta"]), sl(d["A"]), sl(d["g"]))
        assert close(w[:, a:b], ws) and close(u[:, a:b], us)


def test_value_head_groups_read_key_head_hv_over_G():
    d = gi.draw_wy(15, 1, 90, 2, 8, 4, dtype="fp32", HV=6, dense_A=True)
    w, u = oracle.wy_reference(d["k"], d["v"], d["beta"], d["A"], d["g"])
    kk = np.repeat(d["k"], 3, axis=2)  # a plain run: every value head with its own copy of k
    w2, u2 = oracle.wy_reference(kk, d["v"], d["beta"], d["A"], d["g"])
    assert close(w, w2) and close(u, u2)


def test_columns_past_a_partial_chunk_do_not_matter():
    d = gi.draw_wy(16, 1, 100, 1, 8, 8, dtype="fp32", dense_A=True)
    A0 = d["A"].copy()
    A0[:, 64:, :, 36:] = 0.0          # the last chunk has 36 rows
    w1, u1 = oracle.wy_reference(d["k"], d["v"], d["beta"], d["A"], d["g"])
    w0, u0 = oracle.wy_reference(d["k"], d["v"], d["beta"], A0, d["g"])
    assert np.array_equal(w1, w0) and np.array_equal(u1, u0)


@pytest.mark.parametrize("mistake", ["A_transposed", "exp_not_exp2", "head_mod_H"])
def test_pins_catch_planted_mistakes(mistake):
    if mistake == "A_transposed":
        d = gi.draw_wy(17, 1, 128, 1, 8, 4, dtype="fp32")
        B, T = d["k"].shape[:2]
        A = structured_A(B, T, 1, None, "ones")
        At = A.copy()
        for c0 in range(0, T, C):       # transpose each chunk's matrix
            blk = A[0, c0:c0 + C, 0, :].copy()
            At[0, c0:c0 + C, 0, :] = blk.T
        _, u = oracle.wy_reference(d["k"], d["v"], d["beta"], At, d["g"])
        sc = d["beta"].astype(np.float64)
        assert not close(u, chunk_cumsum(sc[..., None] * d["v"], B, T, None), 1e-10)
    elif mistake == "exp_not_exp2":
        d = gi.draw_wy(18, 1, 64, 1, 8, 4, dtype="fp32")
        B, T = d["k"].shape[:2]
        A = structured_A(B, T, 1, None, "identity")
        g_nat = d["g"].astype(np.float64) * np.log2(np.e)   # 2^(g log2 e) = e^g
        w, _ = oracle.wy_reference(d["k"], d["v"], d["beta"], A, g_nat)
        sc = d["beta"].astype(np.float64) * np.exp2(d["g"].astype(np.float64))
        assert not close(w, sc[..., None] * d["k"])
    else:
        d = gi.draw_wy(19, 1, 70, 2, 8, 4, dtype="fp32", HV=4, dense_A=True)
        w, _ = oracle.wy_reference(d["k"], d["v"], d["beta"], d["A"], d["g"])
        kk = np.concatenate([d["k"], d["k"]], axis=2)          # value head hv with key head hv % H
        w2, _ = oracle.wy_reference(kk, d["v"], d["beta"], d["A"], d["g"])
        assert not close(w, w2)
