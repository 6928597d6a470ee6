"""Pins of the oracle's gradient (oracle.scan_bwd).

The gradient of L = sum_t <dO_t, o_t> + <dST, S_T> is checked against things
other than the reverse sweep itself:
  * central finite differences of the scan written as a fold of dense d x d
    elements S_t = S_{t-1} E_t + f_t (the affine-scan form of the prefix-scan
    notes, key design 2), in float64, for every input;
  * Euler's identity for functions homogeneous of degree one: o and S_T are
    jointly linear in (v, S0), and o is linear in q, so the gradient dotted with
    those inputs returns L exactly, L taken from the forward oracle;
  * diagonal gates with equal channels against the scalar-gate modes;
  * ungated linear attention in closed form.
"""
import numpy as np
import pytest

import oracle

MODES = ["gdn", "gla", "gdn_diag", "gla_diag", "gdn_ew"]


def _inputs(rng, mode, T, dk, dv, f32=False):
    q = rng.standard_normal((T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = rng.uniform(0.6, 1.0, (T, dk) if mode.endswith("diag") else T)
    beta = rng.uniform(0.05, 1.0, (2, T) if mode == "gdn_ew" else T) if mode.startswith("gdn") else None
    S0 = 0.5 * rng.standard_normal((dv, dk))
    dO = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dv, dk))
    xs = [q, k, v, a, beta, S0, dO, dST]
    if f32:
        xs = [None if x is None else x.astype(np.float32).astype(np.float64) for x in xs]
    return xs


def _dense_loss(mode, q, k, v, a, beta, S0, dO, dST):
    T, dk = q.shape
    S = S0.copy()
    L = 0.0
    for t in range(T):
        d = a[t] if mode.endswith("diag") else np.full(dk, a[t])
        if mode == "gdn_ew":  # erase strength in E, write strength in f
            E = np.diag(d) @ (np.eye(dk) - beta[0, t] * np.outer(k[t], k[t]))
            f = beta[1, t] * np.outer(v[t], k[t])
        elif mode.startswith("gdn"):
            E = np.diag(d) @ (np.eye(dk) - beta[t] * np.outer(k[t], k[t]))
            f = beta[t] * np.outer(v[t], k[t])
        else:
            E = np.diag(d)
            f = np.outer(v[t], k[t])
        S = S @ E + f
        L += dO[t] @ (S @ q[t])
    return L + np.sum(dST * S)


@pytest.mark.parametrize("mode", MODES)
def test_finite_differences(mode):
    rng = np.random.default_rng(11)
    T, dk, dv = 7, 4, 3
    xs = _inputs(rng, mode, T, dk, dv)
    grads = oracle.scan_bwd(mode, *xs)
    names = ["q", "k", "v", "alpha", "beta", "S0"]
    for idx, (name, g) in enumerate(zip(names, grads)):
        if xs[idx] is None:
            assert g is None
            continue
        fd = np.empty_like(xs[idx])
        for pos in np.ndindex(xs[idx].shape):
            h = 1e-6
            plus = [x.copy() if x is not None else None for x in xs]
            minus = [x.copy() if x is not None else None for x in xs]
            plus[idx][pos] += h
            minus[idx][pos] -= h
            fd[pos] = (_dense_loss(mode, *plus) - _dense_loss(mode, *minus)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg=f"{mode} d{name}")


@pytest.mark.parametrize("mode", MODES)
def test_homogeneity_against_forward_oracle(mode):
    """L(v, S0) is linear in (v, S0) and L(q) linear in q: <grad, input> = L,
    with o and S_T from the forward oracle."""
    rng = np.random.default_rng(12)
    T, dk, dv = 40, 8, 6
    q, k, v, a, beta, S0, dO, dST = _inputs(rng, mode, T, dk, dv, f32=True)
    o, ST = oracle.scan(mode, q, k, v, a, beta, S0)
    L = np.sum(dO * o) + np.sum(dST * ST)
    gq, gk, gv, ga, gb, gS0 = oracle.scan_bwd(mode, q, k, v, a, beta, S0, dO, dST)
    np.testing.assert_allclose(np.sum(gv * v) + np.sum(gS0 * S0), L, rtol=1e-11)
    gq, *_ = oracle.scan_bwd(mode, q, k, v, a, beta, S0, dO, None)
    np.testing.assert_allclose(np.sum(gq * q), np.sum(dO * o), rtol=1e-11)


@pytest.mark.parametrize("delta", [True, False])
def test_equal_channels_are_the_scalar_gate(delta):
    rng = np.random.default_rng(13)
    T, dk, dv = 30, 5, 4
    scalar, diag = ("gdn", "gdn_diag") if delta else ("gla", "gla_diag")
    q, k, v, a, beta, S0, dO, dST = _inputs(rng, scalar, T, dk, dv)
    g1 = oracle.scan_bwd(scalar, q, k, v, a, beta, S0, dO, dST)
    g2 = oracle.scan_bwd(diag, q, k, v, np.repeat(a[:, None], dk, axis=1), beta, S0, dO, dST)
    for x, y in zip(g1[:3] + g1[4:], g2[:3] + g2[4:]):
        if x is None:
            assert y is None
        else:
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g1[3], g2[3].sum(axis=1), rtol=1e-12, atol=1e-12)


def test_linear_attention_closed_form():
    """alpha = 1, S0 = 0, no dST: o_t = sum_{s<=t} (q_t . k_s) v_s, so
    dv_s = sum_{t>=s} (q_t . k_s) dO_t, dq_t = sum_{s<=t} (dO_t . v_s) k_s and
    dk_s = sum_{t>=s} (dO_t . v_s) q_t."""
    rng = np.random.default_rng(14)
    T, dk, dv = 25, 6, 5
    q, k, v, _, _, _, dO, _ = _inputs(rng, "gla", T, dk, dv)
    gq, gk, gv, ga, gb, gS0 = oracle.scan_bwd("gla", q, k, v, np.ones(T), None, None, dO, None)
    M = np.tril(np.ones((T, T)))
    A = (q @ k.T) * M
    B = (dO @ v.T) * M
    np.testing.assert_allclose(gv, A.T @ dO, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gq, B @ k, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gk, B.T @ q, rtol=1e-12, atol=1e-12)
    assert gb is None
    # no decay: the gradient reaching S0 is the sum of every read-out's q_t
    np.testing.assert_allclose(gS0, dO.T @ q, rtol=1e-12, atol=1e-12)


def test_batched_heads_match_single_heads():
    rng = np.random.default_rng(15)
    T, dk, dv = 20, 4, 4
    heads = [_inputs(rng, "gdn", T, dk, dv) for _ in range(3)]
    st = lambda i: np.stack([h[i] for h in heads])  # noqa: E731
    g = oracle.scan_bwd("gdn", *[st(i) for i in range(8)], threads=3)
    for n, h in enumerate(heads):
        gh = oracle.scan_bwd("gdn", *h, threads=1)
        for x, y in zip(g, gh):
            np.testing.assert_array_equal(x[n], y)


def test_split_strengths_equal_planes_are_the_delta_rule():
    """Equal erase and write strengths give the delta rule's gradients, and the
    two planes of dbeta add up to its dbeta."""
    rng = np.random.default_rng(16)
    T, dk, dv = 30, 5, 4
    q, k, v, a, beta, S0, dO, dST = _inputs(rng, "gdn", T, dk, dv)
    g1 = oracle.scan_bwd("gdn", q, k, v, a, beta, S0, dO, dST)
    g2 = oracle.scan_bwd("gdn_ew", q, k, v, a, np.stack([beta, beta]), S0, dO, dST)
    for i in (0, 1, 2, 3, 5):
        np.testing.assert_allclose(g1[i], g2[i], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g1[4], g2[4][0] + g2[4][1], rtol=1e-12, atol=1e-12)

