"""float64 reference of PRISM's rank-L write (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module.  It shares no code with the GPU library and
never imports it.

What PRISM adds to the gated delta rule ("PRISM: Parallel Residual Iterative
Sequence Model", gist.science explainer, technical summary 2.1 and 2.2; the
PRISM article on banbantang.com, section 3(2)-(4)):

  * the state update is S_t = S_{t-1} A_t + B_t with the forget operator A_t
    left exactly as in the gated delta rule, alpha_t (I - beta_t k_t k_t^T);
  * the write B_t is the gated-delta write beta_t v_t k_t^T plus L rank-1
    corrections computed from the input only (summary 2.2, step by step):
      anchor     u_t       = ShortConv(x)_t           (stands in for S_{t-1} k_t)
      direction  k_t^(l)   = W_k^(l) u_t
      gain       p_t^(l)   = W_p^(l) u_t
      step       delta^(l) = GELU(p_t^(l) * r_t^(l)),  r_t^(l+1) = r_t^(l) - delta^(l)
      write      B_t      += beta_t^(l) delta^(l) (k_t^(l))^T
    with L = 0 the gated delta rule itself (summary section 3);
  * everything on the right-hand side depends on the input alone, so the
    scan is unchanged: each correction is a pure-write element (E = I,
    f = beta^(l) delta^(l) k^(l)T) placed after the token's gated-delta
    element, and the token is read out after its last correction.

Readings where the pages leave a step open (each is one plain choice):
  * ShortConv: causal depthwise convolution over an anchor-source sequence x,
    window w including the current token, zero before the sequence start:
    u_t = sum_{j<w} c_j * x_{t-j} (elementwise per channel).
  * The residual chain starts from the delta-rule residual with the anchor in
    place of the recalled value: r^(1) = v_t - u_t.
  * GELU is the exact form x Phi(x) = x (1 + erf(x / sqrt 2)) / 2.
  * W_k^(l) is d_k x d_v and W_p^(l) is d_v x d_v, per head; beta^(l) is a
    given per-token gate.

Arithmetic is float64 throughout; inputs arrive as float32 (exact for
bfloat16 values).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from . import GDN_EW, scan


def gelu(x):
    """Exact GELU, x * Phi(x) (PRISM summary 2.2 names GELU as the step's nonlinearity)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def short_conv(x, c):
    """Causal depthwise short convolution: u_t = sum_{j<w} c[j] * x[t-j].

    x: [T, d]; c: [w, d].  Positions before the start contribute zero (the
    anchor of PRISM summary 2.2, computed from a short window of the input).
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    T = x.shape[0]
    u = np.zeros_like(x)
    for j in range(c.shape[0]):
        if j < T:
            u[j:] += c[j] * x[: T - j]
    return u


def write_factors(x, v, c, Wk, Wp):
    """PRISM's per-token write factors for one head (summary 2.2, in its order).

    x: [T, dv] anchor source; v: [T, dv] values; c: [w, dv] conv taps;
    Wk: [L, dk, dv]; Wp: [L, dv, dv].
    Returns (u [T, dv], K [T, L, dk], D [T, L, dv]) with K[:, l] = k^(l+1) and
    D[:, l] = delta^(l+1).
    """
    u = short_conv(x, c)
    Wk = np.asarray(Wk, dtype=np.float64)
    Wp = np.asarray(Wp, dtype=np.float64)
    L = Wk.shape[0]
    T = u.shape[0]
    K = np.empty((T, L, Wk.shape[1]))
    D = np.empty((T, L, Wp.shape[1]))
    r = np.asarray(v, dtype=np.float64) - u          # r^(1)
    for l in range(L):
        K[:, l] = u @ Wk[l].T                        # k^(l) = W_k^(l) u_t
        p = u @ Wp[l].T                              # p^(l) = W_p^(l) u_t
        d = gelu(p * r)                              # delta^(l) = GELU(p^(l) * r^(l))
        D[:, l] = d
        r = r - d                                    # r^(l+1) = r^(l) - delta^(l)
    return u, K, D


def expand(q, k, v, alpha, beta, K, D, beta_l):
    """The sub-token stream of one head: token t becomes L+1 scan elements.

    Element t(L+1) is the gated-delta element (alpha_t, erase = write =
    beta_t, k_t, v_t); element t(L+1)+l (l = 1..L) is the pure write
    (alpha = 1, erase 0, write beta_t^(l), k_t^(l), delta_t^(l)).  q_t sits on
    the last element of the group and q = 0 elsewhere, so the group's last
    output is o_t.
    Returns (q2, k2, v2, alpha2, beta2) with beta2 = [erase, write] of shape
    [2, T(L+1)], ready for ``oracle.scan("gdn_ew", ...)``.
    """
    T, dk = np.shape(k)
    dv = np.shape(v)[1]
    L = np.shape(K)[1]
    G = L + 1
    q2 = np.zeros((T, G, dk))
    q2[:, L] = q
    k2 = np.empty((T, G, dk))
    k2[:, 0] = k
    k2[:, 1:] = K
    v2 = np.empty((T, G, dv))
    v2[:, 0] = v
    v2[:, 1:] = D
    a2 = np.ones((T, G))
    a2[:, 0] = alpha
    be = np.zeros((T, G))
    be[:, 0] = beta
    bw = np.empty((T, G))
    bw[:, 0] = beta
    bw[:, 1:] = beta_l
    return (q2.reshape(T * G, dk), k2.reshape(T * G, dk), v2.reshape(T * G, dv),
            a2.reshape(T * G), np.stack([be.reshape(T * G), bw.reshape(T * G)]))


def prism_scan(q, k, v, alpha, beta, x, c, Wk, Wp, beta_l, S0=None, factor_round=None,
               threads=None):
    """PRISM layer read-out for one head: o_t = S_t q_t with S_t = S_{t-1} A_t + B_t.

    ``factor_round`` (optional) maps the float64 factors k^(l), delta^(l) to the
    values a storage format keeps (e.g. bfloat16 rounding); the scan then runs
    on those values, as it does when the factors are handed over in that
    format.  The scan takes float32 operands, so factors are handed to it
    rounded to float32 (exact when factor_round yields bfloat16 values).
    Returns (o [T, dv], S_T [dv, dk]) in float64.
    """
    _, K, D = write_factors(x, v, c, Wk, Wp)
    if factor_round is not None:
        K, D = factor_round(K), factor_round(D)
    q2, k2, v2, a2, b2 = expand(q, k, v, alpha, beta, K, D, beta_l)
    L = np.shape(K)[1]
    f32 = np.float32
    o2, ST = scan(GDN_EW, q2.astype(f32), k2.astype(f32), v2.astype(f32), a2.astype(f32),
                  b2.astype(f32), S0, threads=threads)
    return o2.reshape(-1, L + 1, o2.shape[-1])[:, L], ST
