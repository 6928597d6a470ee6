"""Pins of the diagonal-gate modes of the oracle ("gdn_diag": E_t = diag(a_t)
(I - beta_t k_t k_t^T), f_t = beta_t v_t k_t^T; "gla_diag": E_t = diag(a_t),
f_t = v_t k_t^T).  The prefix-scan notes (key design 2) list the diagonal gate
among the forms E_t takes; the expectations here come from dense d x d
elements folded left to right or combined in a tree, per-channel closed
forms, and the scalar-gate modes as special cases.
"""
import numpy as np
import pytest

import oracle


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _head(rng, T, dk, dv):
    f32 = lambda x: np.asarray(x, np.float32)  # noqa: E731
    q, k = f32(_unit(rng, T, dk)), f32(_unit(rng, T, dk))
    v = f32(rng.standard_normal((T, dv)))
    a = f32(rng.uniform(0.7, 1.0, (T, dk)))
    beta = f32(rng.uniform(0.0, 1.0, T))
    S0 = 0.3 * rng.standard_normal((dv, dk))
    return q, k, v, a, beta, S0


def _elements(mode, k, v, a, beta):
    Es, fs = [], []
    for t in range(k.shape[0]):
        kt, vt, at = (x[t].astype(np.float64) for x in (k, v, a))
        if mode == "gdn_diag":
            Es.append(np.diag(at) @ (np.eye(len(kt)) - float(beta[t]) * np.outer(kt, kt)))
            fs.append(float(beta[t]) * np.outer(vt, kt))
        else:
            Es.append(np.diag(at))
            fs.append(np.outer(vt, kt))
    return Es, fs


@pytest.mark.parametrize("mode", ["gdn_diag", "gla_diag"])
def test_dense_fold(mode):
    rng = np.random.default_rng(31)
    q, k, v, a, beta, S0 = _head(rng, 30, 6, 5)
    o, ST = oracle.scan(mode, q, k, v, a, beta if mode == "gdn_diag" else None, S0)
    Es, fs = _elements(mode, k, v, a, beta)
    S = S0.copy()
    for t in range(30):
        S = S @ Es[t] + fs[t]
        np.testing.assert_allclose(o[t], S @ q[t].astype(np.float64), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST, S, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["gdn_diag", "gla_diag"])
def test_tree_equals_fold(mode):
    """E_t is not symmetric here: the tree must keep the right-action order."""
    rng = np.random.default_rng(32)
    q, k, v, a, beta, S0 = _head(rng, 16, 4, 3)
    Es, fs = _elements(mode, k, v, a, beta)
    comb = lambda x, y: (x[0] @ y[0], x[1] @ y[0] + y[1])  # noqa: E731
    els = list(zip(Es, fs))
    while len(els) > 1:
        els = [comb(els[i], els[i + 1]) for i in range(0, len(els), 2)]
    _, ST = oracle.scan(mode, q, k, v, a, beta if mode == "gdn_diag" else None, S0)
    np.testing.assert_allclose(ST, S0 @ els[0][0] + els[0][1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("diag,scalar", [("gdn_diag", "gdn"), ("gla_diag", "gla")])
def test_uniform_channels_are_the_scalar_gate(diag, scalar):
    rng = np.random.default_rng(33)
    q, k, v, a, beta, S0 = _head(rng, 40, 8, 8)
    alpha = a[:, 0].copy()
    a_u = np.repeat(alpha[:, None], 8, axis=1)
    b = beta if diag == "gdn_diag" else None
    o1, S1 = oracle.scan(diag, q, k, v, a_u, b, S0)
    o2, S2 = oracle.scan(scalar, q, k, v, alpha, b, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-13)


def test_gla_diag_closed_form():
    """S_T[:, j] = S_0[:, j] prod_t a_tj + sum_s v_s k_sj prod_{r > s} a_rj:
    every key channel decays on its own."""
    rng = np.random.default_rng(34)
    T, dk, dv = 25, 5, 4
    q, k, v, a, _, S0 = _head(rng, T, dk, dv)
    _, ST = oracle.scan("gla_diag", q, k, v, a, None, S0)
    ad, kd, vd = a.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    expect = S0 * np.prod(ad, axis=0)[None, :]
    for s in range(T):
        tail = np.prod(ad[s + 1:], axis=0) if s + 1 < T else np.ones(dk)
        expect += np.outer(vd[s], kd[s] * tail)
    np.testing.assert_allclose(ST, expect, rtol=1e-12, atol=1e-12)


def test_decay_then_erase_order():
    """The gate scales the state before the erase reads it: with a key on one
    channel, the erase removes beta times the decayed component."""
    T, dk, dv = 1, 3, 1
    q = np.zeros((T, dk), np.float32)
    k = np.array([[1.0, 0.0, 0.0]], np.float32)
    v = np.zeros((T, dv), np.float32)
    a = np.array([[0.5, 0.25, 1.0]], np.float32)
    beta = np.array([0.5], np.float32)
    S0 = np.array([[2.0, 4.0, 8.0]])
    _, ST = oracle.scan("gdn_diag", q, k, v, a, beta, S0)
    # decay: [1, 1, 8]; erase along e_0 with beta = 1/2: [0.5, 1, 8]
    np.testing.assert_array_equal(ST, [[0.5, 1.0, 8.0]])


def test_decode_diag_matches_dense():
    rng = np.random.default_rng(35)
    N, dk, dv = 5, 4, 3
    q, k = _unit(rng, N, dk).astype(np.float32), _unit(rng, N, dk).astype(np.float32)
    v = rng.standard_normal((N, dv)).astype(np.float32)
    a = rng.uniform(0.5, 1.0, (N, dk)).astype(np.float32)
    beta = rng.uniform(0, 1, N).astype(np.float32)
    S = rng.standard_normal((N, dv, dk))
    expect = [S[n] @ (np.diag(a[n].astype(np.float64)) @ (np.eye(dk) - float(beta[n]) *
              np.outer(k[n].astype(np.float64), k[n].astype(np.float64)))) +
              float(beta[n]) * np.outer(v[n].astype(np.float64), k[n].astype(np.float64))
              for n in range(N)]
    o = oracle.decode_step("gdn_diag", q, k, v, a, beta, S)
    for n in range(N):
        np.testing.assert_allclose(S[n], expect[n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o[n], expect[n] @ q[n].astype(np.float64), rtol=1e-12, atol=1e-12)
