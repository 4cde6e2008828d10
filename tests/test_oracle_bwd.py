"""Pins for the fp64 backward oracle (no GPU).

oracle.gla_reference_bwd runs the chain rule of the token recurrence in
reverse.  It is checked against things that are not itself:

* central finite differences of the O(T^2) closed form (brute_force in
  test_oracle.py, a global-cumsum formula with no recurrence), in fp64, for
  every element of q, k, v, g, h0 on tiny inputs (fixed and packed lengths);
* g == 0, where the method is causal linear attention and every gradient is a
  plain product of matrices;
* planted mistakes (a dropped dht, a missing exp(g) factor in dg, dq taken
  from the state before the update) each fail the finite-difference pin;
* value-head groups and a per-head gate: central differences of the head-variant
  closed form (brute_force_heads), for every input element.
"""
import numpy as np
import pytest

import gla_inputs as gi
import oracle
from test_oracle import brute_force, brute_force_heads


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def loss(q, k, v, g, h0, do, dht, cu, scale):
    o, ht = brute_force(q, k, v, g, h0=h0, cu=cu, scale=scale)
    return float(np.sum(do * o) + np.sum(dht * ht))


def finite_difference(q, k, v, g, h0, do, dht, cu, scale, eps=1e-5):
    """Central differences of the closed-form loss for every input element (fp64)."""
    args = {"q": q.astype(np.float64), "k": k.astype(np.float64), "v": v.astype(np.float64),
            "g": g.astype(np.float64), "h0": h0.astype(np.float64)}
    grads = {}
    for name in ("q", "k", "v", "g", "h0"):
        x = args[name]
        gr = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = loss(args["q"], args["k"], args["v"], args["g"], args["h0"], do, dht, cu, scale)
            x[idx] = old - eps
            lm = loss(args["q"], args["k"], args["v"], args["g"], args["h0"], do, dht, cu, scale)
            x[idx] = old
            gr[idx] = (lp - lm) / (2 * eps)
        grads[name] = gr
    return grads


def tiny(seed, B=1, T=9, H=2, K=3, V=2, lengths=None):
    d = gi.draw(seed, B, T, H, K, V, dtype="fp32", h0=True, lengths=lengths, gate_scale=0.5)
    rng = np.random.default_rng(seed + 1)
    N = d["h0"].shape[0]
    do = rng.standard_normal(d["v"].shape).astype(np.float32).astype(np.float64)
    dht = rng.standard_normal((N, H, K, V)).astype(np.float32).astype(np.float64)
    return d, do, dht


def close(a, b, tol=1e-6):
    den = max(float(np.max(np.abs(b))), 1e-12)
    return float(np.max(np.abs(a - b))) / den < tol


@pytest.mark.parametrize("packed", [False, True])
def test_matches_finite_differences_of_the_closed_form(packed):
    lengths = [4, 0, 6, 1] if packed else None
    d, do, dht = tiny(31 + packed, B=1 if packed else 2, T=0 if packed else 7, lengths=lengths)
    scale = 0.7
    dq, dk, dv, dg, dh0 = oracle.gla_reference_bwd(d["q"], d["k"], d["v"], d["g"], do, h0=d["h0"],
                                                   dht=dht, cu_seqlens=d["cu_seqlens"], scale=scale)
    fd = finite_difference(d["q"], d["k"], d["v"], d["g"], d["h0"], do, dht, d["cu_seqlens"], scale)
    for name, got in (("q", dq), ("k", dk), ("v", dv), ("g", dg), ("h0", dh0)):
        assert close(got, fd[name]), f"d{name} disagrees with finite differences"


def test_zero_gate_gradients_are_matrix_products():
    # o = scale (tril(Q K^T) V + Q h0), ht = h0 + K^T V (per sequence and head)
    B, T, H, K, V = 2, 40, 2, 6, 5
    d = gi.draw(41, B, T, H, K, V, dtype="fp32", h0=True)
    g = np.zeros_like(d["g"])
    rng = np.random.default_rng(42)
    do = rng.standard_normal((B, T, H, V)).astype(np.float32)
    dht = rng.standard_normal((B, H, K, V))
    scale = 0.3
    dq, dk, dv, _, dh0 = oracle.gla_reference_bwd(d["q"], d["k"], d["v"], g, do, h0=d["h0"], dht=dht,
                                                  scale=scale)
    for b in range(B):
        for h in range(H):
            Q, Kk, Vv = (d[x][b, :, h].astype(np.float64) for x in ("q", "k", "v"))
            dO, h0 = do[b, :, h].astype(np.float64), d["h0"][b, h].astype(np.float64)
            M = np.tril(Q @ Kk.T)
            dM = scale * np.tril(dO @ Vv.T)
            np.testing.assert_allclose(dq[b, :, h], dM @ Kk + scale * dO @ h0.T, rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(dk[b, :, h], dM.T @ Q + Vv @ dht[b, h].T, rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(dv[b, :, h], scale * M.T @ dO + Kk @ dht[b, h], rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(dh0[b, h], scale * Q.T @ dO + dht[b, h], rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("mistake", ["drop_dht", "dg_without_exp", "dq_before_update"])
def test_finite_differences_catch_planted_mistakes(mistake):
    d, do, dht = tiny(51)
    scale = 0.9
    args = dict(h0=d["h0"], scale=scale)
    if mistake == "drop_dht":
        dq, dk, dv, dg, dh0 = oracle.gla_reference_bwd(d["q"], d["k"], d["v"], d["g"], do, dht=None, **args)
        got, name = dk, "k"
    elif mistake == "dg_without_exp":
        dq, dk, dv, dg, dh0 = oracle.gla_reference_bwd(d["q"], d["k"], d["v"], d["g"], do, dht=dht, **args)
        got, name = dg / np.exp(d["g"].astype(np.float64)), "g"
    else:
        # dq from the state before the token's update: the gradient of the
        # output read before the update, shifted by one token
        dq, dk, dv, dg, dh0 = oracle.gla_reference_bwd(d["q"], d["k"], d["v"], d["g"], do, dht=dht, **args)
        got, name = np.roll(dq, 1, axis=1), "q"
    fd = finite_difference(d["q"], d["k"], d["v"], d["g"], d["h0"], do, dht, None, scale)
    assert not close(got, fd[name]), f"planted mistake {mistake} slipped through"


@pytest.mark.parametrize("gate", ["key", "head"])
@pytest.mark.parametrize("HV", [1, 3])
def test_head_variants_match_finite_differences(gate, HV):
    B, T, H, K, V = 2, 6, 1, 3, 2
    d = gi.draw(61 + HV, B, T, H, K, V, dtype="fp32", h0=True, HV=HV, gate=gate, gate_scale=0.5)
    rng = np.random.default_rng(62)
    do = rng.standard_normal(d["v"].shape)
    dht = rng.standard_normal(d["h0"].shape)
    scale = 0.8
    got = oracle.gla_reference_bwd(d["q"], d["k"], d["v"], d["g"], do, h0=d["h0"], dht=dht, scale=scale)

    def lossf(q, k, v, g, h0):
        o, ht = brute_force_heads(q, k, v, g, h0=h0, scale=scale)
        return float(np.sum(do * o) + np.sum(dht * ht))

    args = {n: d[n].astype(np.float64) for n in ("q", "k", "v", "g", "h0")}
    eps = 1e-5
    for name, g_got in zip(("q", "k", "v", "g", "h0"), got):
        x = args[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = lossf(**args)
            x[idx] = old - eps
            lm = lossf(**args)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        assert g_got.shape == fd.shape, name
        assert close(g_got, fd), f"d{name} disagrees with finite differences (gate {gate}, HV {HV})"
