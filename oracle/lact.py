"""float64 reference of the large-chunk fast-weight update (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module.  It shares no code with the GPU library and
never imports it.

What it computes ("块级更新与端到端 TTT", PaperTrace 5.2, opening section; the
LaCT news article on senqingzn.com, sections on the large-chunk test-time
training layer):

  * a fast weight W (d_v x d_k) per head is trained online on the sequence with
    a key-value reconstruction loss, l_i(W) = |W k_i - v_i|^2 / 2 (the early
    TTT layers' per-layer key-value reconstruction loss, section 2 of the
    PaperTrace page), so grad l_i(W) = (W k_i - v_i) k_i^T;
  * the sequence is cut into chunks B_b of m tokens, and every gradient of a
    chunk is taken at the chunk's starting weight (the parallel approximation
    of the opening section):
        W_{b+1} = W_b - sum_{i in B_b} eta_i (W_b k_i - v_i) k_i^T
    (eta is the page's learning rate; a per-token array, the page's scalar
    being the constant case);
  * the read-out applies a weight to each query, o_i = W q_i; the update and
    apply steps are decoupled and their order sets the mask (news article,
    update/apply paragraph): "update then apply" reads chunk b with W_{b+1}
    (every token sees its whole chunk: a block mask), "apply then update" with
    W_b (the mask shifted by one chunk, no token sees its own chunk).

Readings: the loss is the plain squared error above (the pages name a
key-value reconstruction loss and give no constant or normalisation); a
ragged last chunk holds the remaining tokens.
"""
from __future__ import annotations

import numpy as np

UPDATE_THEN_APPLY = 0
APPLY_THEN_UPDATE = 1


def lact(q, k, v, eta, chunk, order=UPDATE_THEN_APPLY, W0=None):
    """One head.  q, k: [T, dk]; v: [T, dv]; eta: [T]; W0: [dv, dk] or None.

    Returns (o [T, dv], W_T [dv, dk]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    eta = np.asarray(eta, dtype=np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    W = np.zeros((dv, dk)) if W0 is None else np.array(W0, dtype=np.float64)
    o = np.empty((T, dv))
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        Kb, Vb, eb = k[s:e], v[s:e], eta[s:e]
        grad = ((Kb @ W.T - Vb) * eb[:, None]).T @ Kb      # sum_i eta_i (W k_i - v_i) k_i^T
        W_next = W - grad
        o[s:e] = q[s:e] @ (W_next if order == UPDATE_THEN_APPLY else W).T
        W = W_next
    return o, W


def lact_batch(q, k, v, eta, chunk, order=UPDATE_THEN_APPLY, W0=None):
    """``lact`` over leading head dimensions ([..., T, d] arrays)."""
    lead = q.shape[:-2]
    n = int(np.prod(lead)) if lead else 1
    T = q.shape[-2]
    dv, dk = v.shape[-1], k.shape[-1]
    qf, kf, vf = q.reshape(n, T, -1), k.reshape(n, T, -1), v.reshape(n, T, -1)
    ef = np.asarray(eta).reshape(n, T)
    Wf = None if W0 is None else np.asarray(W0).reshape(n, dv, dk)
    o = np.empty((n, T, dv))
    WT = np.empty((n, dv, dk))
    for i in range(n):
        o[i], WT[i] = lact(qf[i], kf[i], vf[i], ef[i], chunk, order, None if Wf is None else Wf[i])
    return o.reshape(*lead, T, dv), WT.reshape(*lead, dv, dk)
