"""Pins of the large-chunk fast-weight update oracle (oracle/lact.py).

Expectations come by other routes: the gated-delta scan oracle (one-token
chunks are the delta rule), closed forms (one chunk over the whole sequence is
linear attention without a causal mask), fixed points of the loss, linearity,
and the block structure the update/apply order sets ("块级更新与端到端 TTT",
PaperTrace 5.2, opening section; LaCT news article, update/apply paragraph).
"""
import numpy as np
import pytest

import oracle
from oracle import lact as L


def _head(rng, T, dk, dv, eta_scale=0.5):
    q = rng.standard_normal((T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    eta = rng.uniform(0.0, eta_scale, T)
    W0 = 0.3 * rng.standard_normal((dv, dk))
    f32 = lambda x: x.astype(np.float32)  # noqa: E731
    return f32(q), f32(k), f32(v), f32(eta), W0


def test_one_token_chunks_are_the_delta_rule():
    """m = 1, update then apply: W_t = W_{t-1} - eta (W k - v) k^T is the gated
    delta rule with alpha = 1, beta = eta; o_t = W_t q_t."""
    rng = np.random.default_rng(1)
    T, dk, dv = 40, 6, 5
    q, k, v, eta, W0 = _head(rng, T, dk, dv)
    o, WT = L.lact(q, k, v, eta, 1, L.UPDATE_THEN_APPLY, W0)
    o2, S2 = oracle.scan("gdn", q, k, v, np.ones(T, np.float32), eta, W0)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(WT, S2, rtol=1e-12, atol=1e-12)


def test_one_token_chunks_apply_first_read_the_previous_state():
    """m = 1, apply then update: o_t = W_{t-1} q_t, the delta rule's state
    before token t."""
    rng = np.random.default_rng(2)
    T, dk, dv = 12, 4, 3
    q, k, v, eta, W0 = _head(rng, T, dk, dv)
    o, _ = L.lact(q, k, v, eta, 1, L.APPLY_THEN_UPDATE, W0)
    ones = np.ones(T, np.float32)
    for t in range(T):
        if t == 0:
            S = W0
        else:
            _, S = oracle.scan("gdn", q[:t], k[:t], v[:t], ones[:t], eta[:t], W0)
        np.testing.assert_allclose(o[t], S @ q[t].astype(np.float64), rtol=1e-12, atol=1e-12)


def test_whole_sequence_chunk_is_unmasked_linear_attention():
    """One chunk, W0 = 0, update then apply: o_i = sum_j eta_j (k_j . q_i) v_j
    over every j (no causal mask); apply then update reads W0 only."""
    rng = np.random.default_rng(3)
    T, dk, dv = 30, 8, 6
    q, k, v, eta, W0 = _head(rng, T, dk, dv)
    o, WT = L.lact(q, k, v, eta, T, L.UPDATE_THEN_APPLY, None)
    qd, kd, vd, ed = (x.astype(np.float64) for x in (q, k, v, eta))
    expect = (qd @ kd.T) @ (ed[:, None] * vd)
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(WT, (ed[:, None] * vd).T @ kd, rtol=1e-12, atol=1e-12)
    o2, _ = L.lact(q, k, v, eta, T + 5, L.APPLY_THEN_UPDATE, W0)
    np.testing.assert_allclose(o2, qd @ W0.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("order", [L.UPDATE_THEN_APPLY, L.APPLY_THEN_UPDATE])
def test_block_structure(order):
    """Changing chunk c's keys and values leaves every earlier chunk's output
    alone (update then apply) and also chunk c's own (apply then update)."""
    rng = np.random.default_rng(4)
    T, dk, dv, m = 50, 5, 4, 8
    q, k, v, eta, W0 = _head(rng, T, dk, dv)
    o, _ = L.lact(q, k, v, eta, m, order, W0)
    c = 3
    k2, v2 = k.copy(), v.copy()
    k2[c * m:(c + 1) * m] = rng.standard_normal((m, dk))
    v2[c * m:(c + 1) * m] += 1.0
    o2, _ = L.lact(q, k2, v2, eta, m, order, W0)
    same = c * m if order == L.UPDATE_THEN_APPLY else (c + 1) * m
    np.testing.assert_array_equal(o[:same], o2[:same])
    assert np.max(np.abs(o[same:same + m] - o2[same:same + m])) > 1e-3


def test_orders_are_one_chunk_apart():
    """Apply then update on chunk b uses the weight that update then apply used
    on chunk b - 1."""
    rng = np.random.default_rng(5)
    T, dk, dv, m = 48, 6, 6, 12
    q, k, v, eta, W0 = _head(rng, T, dk, dv)
    oa, Wa = L.lact(q, k, v, eta, m, L.APPLY_THEN_UPDATE, W0)
    qd = q.astype(np.float64)
    # weights after each chunk from the update-then-apply run, read back
    # through queries equal to the identity
    W = W0
    for b in range(T // m):
        np.testing.assert_allclose(oa[b * m:(b + 1) * m], qd[b * m:(b + 1) * m] @ W.T,
                                   rtol=1e-12, atol=1e-12)
        _, W = L.lact(q[: (b + 1) * m], k[: (b + 1) * m], v[: (b + 1) * m], eta[: (b + 1) * m],
                      m, L.UPDATE_THEN_APPLY, W0)
    np.testing.assert_allclose(Wa, W, rtol=1e-12, atol=1e-12)


def test_fixed_point_of_the_loss():
    """v_i = W* k_i for every token and W0 = W*: every gradient is zero."""
    rng = np.random.default_rng(6)
    T, dk, dv = 33, 7, 5
    q, k, _, eta, _ = _head(rng, T, dk, dv)
    Ws = rng.standard_normal((dv, dk))
    v = k.astype(np.float64) @ Ws.T
    o, WT = L.lact(q, k, v, eta, 10, L.UPDATE_THEN_APPLY, Ws)
    np.testing.assert_allclose(WT, Ws, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, q.astype(np.float64) @ Ws.T, rtol=1e-12, atol=1e-12)


def test_linear_in_values_and_initial_weight():
    rng = np.random.default_rng(7)
    T, dk, dv = 37, 6, 4
    q, k, v, eta, W0 = _head(rng, T, dk, dv)
    o1, W1 = L.lact(q, k, v, eta, 9, L.UPDATE_THEN_APPLY, W0)
    o2, W2 = L.lact(q, k, 2.5 * v.astype(np.float64), eta, 9, L.UPDATE_THEN_APPLY, 2.5 * W0)
    np.testing.assert_allclose(o2, 2.5 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W2, 2.5 * W1, rtol=1e-12, atol=1e-12)


def test_ragged_last_chunk_and_batch_wrapper():
    rng = np.random.default_rng(8)
    T, dk, dv, m = 29, 4, 4, 8
    heads = [_head(rng, T, dk, dv) for _ in range(3)]
    st = lambda i: np.stack([h[i] for h in heads])  # noqa: E731
    o, W = L.lact_batch(st(0), st(1), st(2), st(3), m, L.UPDATE_THEN_APPLY, st(4))
    for i, h in enumerate(heads):
        oi, Wi = L.lact(*h[:4], m, L.UPDATE_THEN_APPLY, h[4])
        np.testing.assert_array_equal(o[i], oi)
        np.testing.assert_array_equal(W[i], Wi)
    # the last chunk holds T mod m = 5 tokens: the same as a sequence padded
    # with eta = 0 tokens (which contribute no gradient)
    q, k, v, eta, W0 = heads[0]
    pad = lambda x: np.concatenate([x, np.zeros((3,) + x.shape[1:], x.dtype)])  # noqa: E731
    op, Wp = L.lact(pad(q), pad(k), pad(v), pad(eta), m, L.UPDATE_THEN_APPLY, W0)
    np.testing.assert_allclose(op[:T], o[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Wp, W[0], rtol=1e-12, atol=1e-12)
