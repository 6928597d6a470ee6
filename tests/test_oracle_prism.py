"""Pins of the split-strength scan mode and of the PRISM write oracle.

Each expectation comes by a route other than the oracle's own code: dense
d x d monoid elements folded left to right, closed forms of special cases,
values of the normal distribution function, exact saturation of GELU in
float64, and the pages' statement that PRISM with no corrections is the gated
delta rule ("PRISM: Parallel Residual Iterative Sequence Model", gist.science
explainer, technical summary 2.1-2.2 and section 3; PRISM article,
banbantang.com, section 3(4)).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import prism


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _f32(*xs):
    return [None if x is None else np.asarray(x, dtype=np.float32) for x in xs]


def _ew_head(rng, T, dk, dv):
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.8, 1.0, T)
    be = rng.uniform(0.0, 1.0, T)
    bw = rng.uniform(0.0, 2.0, T)
    S0 = 0.3 * rng.standard_normal((dv, dk))
    q, k, v, alpha, be, bw = _f32(q, k, v, alpha, be, bw)
    return q, k, v, alpha, be, bw, S0


# --------------------------------------------------------------------------
# split erase / write strengths
# --------------------------------------------------------------------------


def test_split_strengths_match_dense_fold():
    """S_t = S_{t-1} alpha (I - be k k^T) + bw v k^T with explicit matrices."""
    rng = np.random.default_rng(11)
    T, dk, dv = 24, 6, 5
    q, k, v, alpha, be, bw, S0 = _ew_head(rng, T, dk, dv)
    o, ST = oracle.scan("gdn_ew", q, k, v, alpha, np.stack([be, bw]), S0)
    S = S0.copy()
    for t in range(T):
        kt = k[t].astype(np.float64)
        E = float(alpha[t]) * (np.eye(dk) - float(be[t]) * np.outer(kt, kt))
        S = S @ E + float(bw[t]) * np.outer(v[t].astype(np.float64), kt)
        np.testing.assert_allclose(o[t], S @ q[t].astype(np.float64), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST, S, rtol=1e-12, atol=1e-12)


def test_split_strengths_reduce_to_gdn_when_equal():
    rng = np.random.default_rng(12)
    q, k, v, alpha, be, _, S0 = _ew_head(rng, 40, 8, 8)
    o1, S1 = oracle.scan("gdn", q, k, v, alpha, be, S0)
    o2, S2 = oracle.scan("gdn_ew", q, k, v, alpha, np.stack([be, be]), S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_pure_writes_are_a_running_sum():
    """alpha = 1, erase 0: S_t = S_0 + sum_{s<=t} bw_s v_s k_s^T (closed form)."""
    rng = np.random.default_rng(13)
    T, dk, dv = 30, 5, 7
    q, k, v, _, _, bw, S0 = _ew_head(rng, T, dk, dv)
    ones, zeros = np.ones(T, np.float32), np.zeros(T, np.float32)
    o, ST = oracle.scan("gdn_ew", q, k, v, ones, np.stack([zeros, bw]), S0)
    outer = bw[:, None, None].astype(np.float64) * np.einsum("ti,tj->tij", v.astype(np.float64),
                                                              k.astype(np.float64))
    S_t = S0[None] + np.cumsum(outer, axis=0)
    np.testing.assert_allclose(o, np.einsum("tij,tj->ti", S_t, q.astype(np.float64)), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(ST, S_t[-1], rtol=1e-12, atol=1e-12)


def test_split_strength_decode_planes():
    """decode_step reads the erase plane then the write plane ([2, N])."""
    rng = np.random.default_rng(14)
    N, dk, dv = 6, 4, 3
    q, k = _unit(rng, N, dk).astype(np.float32), _unit(rng, N, dk).astype(np.float32)
    v = rng.standard_normal((N, dv)).astype(np.float32)
    alpha = rng.uniform(0.8, 1.0, N).astype(np.float32)
    be, bw = rng.uniform(0, 1, N).astype(np.float32), rng.uniform(0, 2, N).astype(np.float32)
    S = rng.standard_normal((N, dv, dk))
    expect = []
    for n in range(N):
        kt = k[n].astype(np.float64)
        Sn = S[n] @ (float(alpha[n]) * (np.eye(dk) - float(be[n]) * np.outer(kt, kt))) \
            + float(bw[n]) * np.outer(v[n].astype(np.float64), kt)
        expect.append(Sn)
    o = oracle.decode_step("gdn_ew", q, k, v, alpha, np.stack([be, bw]), S)
    for n in range(N):
        np.testing.assert_allclose(S[n], expect[n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o[n], expect[n] @ q[n].astype(np.float64), rtol=1e-12,
                                   atol=1e-12)


def test_split_strength_shape_checked():
    rng = np.random.default_rng(15)
    q, k, v, alpha, be, bw, S0 = _ew_head(rng, 8, 4, 4)
    with pytest.raises(ValueError):
        oracle.scan("gdn_ew", q, k, v, alpha, be, S0)


# --------------------------------------------------------------------------
# PRISM write factors
# --------------------------------------------------------------------------


def test_gelu_values():
    """GELU(x) = x Phi(x): Phi(1), Phi(2) from the normal table; odd part x."""
    g = prism.gelu(np.array([0.0, 1.0, -1.0, 2.0, -2.0]))
    phi1, phi2 = 0.8413447460685429, 0.9772498680518208
    np.testing.assert_allclose(g, [0.0, phi1, -(1 - phi1), 2 * phi2, -2 * (1 - phi2)],
                               rtol=1e-15, atol=1e-16)
    x = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(prism.gelu(x) - prism.gelu(-x), x, rtol=0, atol=1e-15)
    # slope 1/2 and curvature 2/sqrt(2 pi) at 0
    h = 1e-4
    assert abs(prism.gelu(h) - (h / 2 + h * h / math.sqrt(2 * math.pi))) < 1e-15


def test_short_conv_is_a_causal_shift_filter():
    rng = np.random.default_rng(21)
    T, d, w = 9, 3, 4
    x = rng.standard_normal((T, d))
    for j in range(w):
        c = np.zeros((w, d))
        c[j] = 1.0
        u = prism.short_conv(x, c)
        np.testing.assert_array_equal(u[j:], x[: T - j])
        np.testing.assert_array_equal(u[:j], 0.0)
    # linear in x and in c
    c1, c2 = rng.standard_normal((w, d)), rng.standard_normal((w, d))
    x2 = rng.standard_normal((T, d))
    np.testing.assert_allclose(prism.short_conv(x + x2, c1),
                               prism.short_conv(x, c1) + prism.short_conv(x2, c1), atol=1e-14)
    np.testing.assert_allclose(prism.short_conv(x, c1 + c2),
                               prism.short_conv(x, c1) + prism.short_conv(x, c2), atol=1e-14)
    # window shorter than the sequence start: the first tokens see fewer taps
    u = prism.short_conv(np.ones((T, d)), np.ones((w, d)))
    np.testing.assert_array_equal(u[:, 0], [1, 2, 3, 4, 4, 4, 4, 4, 4])


def test_residual_chain_closed_form_in_linear_regime():
    """With every p r >= 9, GELU(p r) = p r exactly in float64, so
    delta1 = p1 r1, r2 = r1 (1 - p1), delta2 = p2 r1 (1 - p1): a closed form
    that fixes the gain, the product with the residual and the sign of the
    residual update."""
    rng = np.random.default_rng(22)
    T, d = 5, 4
    x = rng.uniform(1.0, 2.0, (T, d))                 # u = x (identity taps)
    v = x + rng.uniform(6.0, 8.0, (T, d))             # r1 = v - u in [6, 8]
    c = np.zeros((4, d))
    c[0] = 1.0
    a1 = 1.5 / x.min()                                # p1 r1 >= 1.5 * 6 = 9
    a2 = -4.0 / x.min()                               # r2 = r1 (1 - p1) < 0, p2 < 0
    Wk = np.stack([np.eye(d), 2 * np.eye(d)])
    Wp = np.stack([a1 * np.eye(d), a2 * np.eye(d)])
    u, K, D = prism.write_factors(x, v, c, Wk, Wp)
    r1 = v - x
    p1, p2 = a1 * x, a2 * x
    assert np.all(p1 * r1 >= 9) and np.all(p2 * r1 * (1 - p1) >= 9)
    np.testing.assert_allclose(u, x, rtol=0, atol=0)
    np.testing.assert_allclose(D[:, 0], p1 * r1, rtol=1e-15)
    np.testing.assert_allclose(D[:, 1], p2 * r1 * (1 - p1), rtol=1e-14)
    np.testing.assert_allclose(K[:, 0], x, rtol=0)
    np.testing.assert_allclose(K[:, 1], 2 * x, rtol=0)


def test_negative_gain_switches_a_step_off():
    """p r <= -40: GELU = 0 exactly, the step writes nothing and the residual
    passes unchanged to the next step."""
    rng = np.random.default_rng(23)
    T, d = 6, 3
    x = rng.uniform(1.0, 2.0, (T, d))
    v = x + rng.uniform(5.0, 6.0, (T, d))
    c = np.zeros((3, d))
    c[0] = 1.0
    Wp = np.stack([-40.0 * np.eye(d), 0.3 * np.eye(d)])
    Wk = rng.standard_normal((2, 5, d))
    _, _, D = prism.write_factors(x, v, c, Wk, Wp)
    np.testing.assert_array_equal(D[:, 0], 0.0)
    np.testing.assert_allclose(D[:, 1], prism.gelu(0.3 * x * (v - x)), rtol=1e-15)


def test_gelu_argument_is_gain_times_residual():
    """GELU(z) - GELU(-z) = z, so flipping the gain's sign changes the first step
    by exactly p r (fails for GELU(p) r, GELU(p + r), ...)."""
    rng = np.random.default_rng(24)
    T, dk, dv = 7, 4, 5
    x, v = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    c = rng.standard_normal((4, dv))
    Wk, Wp = rng.standard_normal((1, dk, dv)), rng.standard_normal((1, dv, dv))
    u, _, D1 = prism.write_factors(x, v, c, Wk, Wp)
    _, _, D2 = prism.write_factors(x, v, c, Wk, -Wp)
    np.testing.assert_allclose(D1[:, 0] - D2[:, 0], (u @ Wp[0].T) * (v - u), atol=1e-13)


def _prism_head(rng, T, dk, dv, L, w=4):
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.8, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    x = rng.standard_normal((T, dv))
    c = rng.standard_normal((w, dv)) / w
    Wk = rng.standard_normal((L, dk, dv)) / np.sqrt(dv)
    Wp = rng.standard_normal((L, dv, dv)) / np.sqrt(dv)
    beta_l = rng.uniform(0.0, 1.0, (T, L))
    S0 = 0.3 * rng.standard_normal((dv, dk))
    q, k, v, alpha, beta, beta_l = _f32(q, k, v, alpha, beta, beta_l)
    return q, k, v, alpha, beta, x, c, Wk, Wp, beta_l, S0


@pytest.mark.parametrize("L", [1, 2, 3])
def test_prism_scan_matches_dense_rank_L_update(L):
    """S_t = S_{t-1} A_t + B_t with A_t the gated-delta forget and
    B_t = beta v k^T + sum_l beta^(l) delta^(l) k^(l)T as explicit matrices."""
    rng = np.random.default_rng(30 + L)
    T, dk, dv = 20, 6, 5
    q, k, v, alpha, beta, x, c, Wk, Wp, beta_l, S0 = _prism_head(rng, T, dk, dv, L)
    o, ST = prism.prism_scan(q, k, v, alpha, beta, x, c, Wk, Wp, beta_l, S0)
    _, K, D = prism.write_factors(x, v, c, Wk, Wp)
    K, D = K.astype(np.float32).astype(np.float64), D.astype(np.float32).astype(np.float64)
    S = S0.copy()
    for t in range(T):
        kt, vt = k[t].astype(np.float64), v[t].astype(np.float64)
        A = float(alpha[t]) * (np.eye(dk) - float(beta[t]) * np.outer(kt, kt))
        B = float(beta[t]) * np.outer(vt, kt)
        for l in range(L):
            B += float(beta_l[t, l]) * np.outer(D[t, l], K[t, l])
        if t == T // 2:  # generic inputs: the write has rank L + 1
            assert np.linalg.matrix_rank(B, tol=1e-9) == min(L + 1, dk, dv)
        S = S @ A + B
        np.testing.assert_allclose(o[t], S @ q[t].astype(np.float64), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(ST, S, rtol=1e-11, atol=1e-11)


def test_prism_without_corrections_is_gdn():
    """L = 0 (no refinement steps) gives the gated delta rule exactly."""
    rng = np.random.default_rng(40)
    q, k, v, alpha, beta, x, c, Wk, Wp, beta_l, S0 = _prism_head(rng, 33, 8, 8, 1)
    o, ST = prism.prism_scan(q, k, v, alpha, beta, x, c, Wk[:0], Wp[:0], beta_l[:, :0], S0)
    o0, S0T = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    np.testing.assert_array_equal(o, o0)
    np.testing.assert_array_equal(ST, S0T)


def test_prism_with_zero_gain_is_gdn():
    """W_p = 0: every step is GELU(0) = 0, the pure writes add nothing."""
    rng = np.random.default_rng(41)
    q, k, v, alpha, beta, x, c, Wk, Wp, beta_l, S0 = _prism_head(rng, 25, 8, 8, 2)
    o, ST = prism.prism_scan(q, k, v, alpha, beta, x, c, Wk, 0 * Wp, beta_l, S0)
    o0, S0T = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    np.testing.assert_array_equal(o, o0)
    np.testing.assert_array_equal(ST, S0T)


def test_expand_layout():
    """Sub-token order: gated-delta element first, corrections after, q last."""
    rng = np.random.default_rng(42)
    T, dk, dv, L = 3, 2, 2, 2
    q, k, v, alpha, beta, x, c, Wk, Wp, beta_l, S0 = _prism_head(rng, T, dk, dv, L)
    _, K, D = prism.write_factors(x, v, c, Wk, Wp)
    q2, k2, v2, a2, b2 = prism.expand(q, k, v, alpha, beta, K, D, beta_l)
    G = L + 1
    for t in range(T):
        np.testing.assert_array_equal(k2[t * G], k[t])
        np.testing.assert_array_equal(v2[t * G], v[t])
        assert a2[t * G] == alpha[t] and b2[0, t * G] == beta[t] and b2[1, t * G] == beta[t]
        for l in range(1, G):
            np.testing.assert_array_equal(k2[t * G + l], K[t, l - 1])
            np.testing.assert_array_equal(v2[t * G + l], D[t, l - 1])
            assert a2[t * G + l] == 1 and b2[0, t * G + l] == 0 and b2[1, t * G + l] == beta_l[t, l - 1]
        np.testing.assert_array_equal(q2[t * G + L], q[t])
        np.testing.assert_array_equal(q2[t * G: t * G + L], 0)
