"""Pins of the float64 oracle against facts the pages and the mathematics fix.

Each test computes its expectation by a route other than the oracle's
token-by-token row update: explicit d x d monoid elements combined in a tree,
dense unrolled products, closed forms of special cases, exact rational
arithmetic, or invariants of the affine map.  A dropped term, a wrong sign, a
transposed operand or a wrong index in the oracle fails at least one of them.

Sources (see oracle/oracle.c):
  * prefix-scan notes (papernotes.org), key design 2: the monoid (E, f), its
    combine and identity (I, 0); associativity makes a tree scan equal the
    left-to-right fold; key design 1: training and inference compute the same
    function; the worked example's Blelloch bracketing.
  * PRISM explainer (gist.science), 2.1-2.2: S_t = S_{t-1} A_t + B_t, with
    S_{t-1} k_t the recalled value; PRISM article section 1(4): scalar decay,
    rank-1 forgetting along k, rank-1 write.
"""
import fractions
import itertools

import numpy as np
import pytest

import oracle


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _head(rng, T, dk, dv, mode="gdn", s0=True, f32=True):
    q = _unit(rng, T, dk)
    k = _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(0.8, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T) if mode == "gdn" else None
    S0 = 0.3 * rng.standard_normal((dv, dk)) if s0 else None
    if f32:  # the oracle takes float32 operands; keep the exact float32 values
        q, k, v, alpha = (x.astype(np.float32) for x in (q, k, v, alpha))
        beta = None if beta is None else beta.astype(np.float32)
    return q, k, v, alpha, beta, S0


def _elements(mode, k, v, alpha, beta):
    """Explicit monoid elements: E_t (dk x dk) and f_t (dv x dk), float64."""
    k, v, alpha = k.astype(np.float64), v.astype(np.float64), alpha.astype(np.float64)
    dk = k.shape[1]
    Es, fs = [], []
    for t in range(k.shape[0]):
        kk = np.outer(k[t], k[t])
        if mode == "gdn":
            b = float(beta[t])
            Es.append(alpha[t] * (np.eye(dk) - b * kk))
            fs.append(b * np.outer(v[t], k[t]))
        else:
            Es.append(alpha[t] * np.eye(dk))
            fs.append(np.outer(v[t], k[t]))
    return Es, fs


def _combine(a, b):
    """(E_a, f_a) then (E_b, f_b) for the right action S -> S E + f."""
    return (a[0] @ b[0], a[1] @ b[0] + b[1])


def _blelloch_exclusive(xs, ident, comb=None):
    """Static Blelloch scan: up-sweep pairs adjacent nodes level by level, the
    down-sweep hands each right child (prefix of parent) then (left subtree).
    Leaf count padded to a power of two with the identity."""
    comb = comb or _combine
    n = len(xs)
    m = 1
    while m < n:
        m *= 2
    tree = list(xs) + [ident] * (m - n)
    d = 1
    while d < m:
        for i in range(2 * d - 1, m, 2 * d):
            tree[i] = comb(tree[i - d], tree[i])
        d *= 2
    tree[m - 1] = ident
    d = m // 2
    while d >= 1:
        for i in range(2 * d - 1, m, 2 * d):
            left = tree[i - d]
            tree[i - d] = tree[i]
            tree[i] = comb(tree[i], left)
        d //= 2
    return tree[:n]


def _check_close(x, ref, tol):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = max(np.linalg.norm(ref), 1e-300)
    assert np.linalg.norm(x - ref) / den <= tol, np.linalg.norm(x - ref) / den


# --------------------------------------------------------------------- P-1
@pytest.mark.parametrize("mode", ["gdn", "gla"])
@pytest.mark.parametrize("leaf", [1, 4])
def test_tree_scan_equals_fold(oracle_lib, mode, leaf):
    """Associativity: a Blelloch tree over explicit (E, f) elements, leaves of
    ``leaf`` tokens folded left to right, gives every prefix state and read-out
    the oracle's left-to-right recurrence gives."""
    rng = np.random.default_rng(101 + leaf)
    T, dk, dv = 37, 8, 6
    q, k, v, alpha, beta, S0 = _head(rng, T, dk, dv, mode)
    o_ref, ST_ref = oracle.scan(mode, q, k, v, alpha, beta, S0)
    Es, fs = _elements(mode, k, v, alpha, beta)
    xs = list(zip(Es, fs))
    ident = (np.eye(dk), np.zeros((dv, dk)))
    leaves = []
    for s in range(0, T, leaf):
        acc = ident
        for x in xs[s:s + leaf]:
            acc = _combine(acc, x)
        leaves.append(acc)
    prefixes = _blelloch_exclusive(leaves, ident)
    o_tree = np.empty((T, dv))
    S_t = None
    for li, s in enumerate(range(0, T, leaf)):
        acc = prefixes[li]
        for t in range(s, min(s + leaf, T)):
            acc = _combine(acc, xs[t])
            S_t = S0 @ acc[0] + acc[1]
            o_tree[t] = S_t @ q[t].astype(np.float64)
    _check_close(o_ref, o_tree, 1e-12)
    _check_close(ST_ref, S_t, 1e-12)


def test_blelloch_bracketing_matches_worked_example():
    """The prefix-scan notes' worked example (4 chunks): the up-sweep merges
    (x0,x1) and (x2,x3), then forms x_{0:3}; chunk 3 is predicted from the
    exclusive prefix x_{0:2} (the example's "x_{0:1}" for chunk 3 is read as a
    slip: the scheme and the binary-counter passage both give x_{0:2})."""
    golden = {}
    with open(__file__.replace("test_oracle_pins.py", "golden/blelloch_4chunks.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                key, val = line.split("=")
                golden[key.strip()] = val.strip()
    # symbolic run of the same scan routine: an element is the string of the
    # chunk range it covers, combine concatenates ranges.
    log = []

    def comb(a, b):
        if a == "I":
            return b
        if b == "I":
            return a
        r = f"{a.split(':')[0]}:{b.split(':')[-1]}"
        log.append(f"({a},{b})")
        return r

    pref = _blelloch_exclusive(["0:0", "1:1", "2:2", "3:3"], "I", comb)
    assert ",".join(log[:3]) == golden["upsweep"]
    assert ",".join(pref) == golden["exclusive"]


# --------------------------------------------------------------------- P-2
def test_identity_element_keeps_state(oracle_lib):
    """alpha = 1, beta = 0 makes every (E_t, f_t) the identity (I, 0): the
    state never changes and o_t = S_0 q_t."""
    rng = np.random.default_rng(2)
    T, dk, dv = 20, 16, 12
    q, k, v, _, _, S0 = _head(rng, T, dk, dv)
    alpha = np.ones(T, np.float32)
    beta = np.zeros(T, np.float32)
    o, ST = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    assert np.array_equal(ST, S0)
    _check_close(o, q.astype(np.float64) @ S0.T, 1e-14)


def test_decay_only_closed_form(oracle_lib):
    """beta = 0 leaves only the scalar decay: S_t = (prod_{r<=t} alpha_r) S_0."""
    rng = np.random.default_rng(3)
    T, dk, dv = 30, 8, 8
    q, k, v, alpha, _, S0 = _head(rng, T, dk, dv)
    beta = np.zeros(T, np.float32)
    o, ST = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    g = np.cumprod(alpha.astype(np.float64))
    _check_close(ST, g[-1] * S0, 1e-14)
    _check_close(o, g[:, None] * (q.astype(np.float64) @ S0.T), 1e-14)


# --------------------------------------------------------------------- P-3
def test_linear_attention_is_causal_masked_sum(oracle_lib):
    """E = I (ungated linear attention): O = tril(Q K^T) V + Q S_0^T and
    S_T = S_0 + V^T K."""
    rng = np.random.default_rng(4)
    T, dk, dv = 40, 16, 8
    q, k, v, _, _, S0 = _head(rng, T, dk, dv, "gla")
    alpha = np.ones(T, np.float32)
    o, ST = oracle.scan("gla", q, k, v, alpha, None, S0)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    _check_close(o, np.tril(Q @ K.T) @ V + Q @ S0.T, 1e-12)
    _check_close(ST, S0 + V.T @ K, 1e-12)


def test_gated_linear_attention_closed_form(oracle_lib):
    """E = alpha I: O = (Q K^T * D) V + diag(gamma) Q S_0^T with
    D_ts = prod_{s<r<=t} alpha_r (s <= t) and gamma_t = prod_{r<=t} alpha_r."""
    rng = np.random.default_rng(5)
    T, dk, dv = 33, 8, 12
    q, k, v, alpha, _, S0 = _head(rng, T, dk, dv, "gla")
    o, ST = oracle.scan("gla", q, k, v, alpha, None, S0)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    a = alpha.astype(np.float64)
    D = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            D[t, s] = np.prod(a[s + 1:t + 1])
    gamma = np.array([np.prod(a[:t + 1]) for t in range(T)])
    _check_close(o, (Q @ K.T * D) @ V + gamma[:, None] * (Q @ S0.T), 1e-12)
    _check_close(ST, gamma[-1] * S0 + (V.T * D[-1]) @ K, 1e-12)


# --------------------------------------------------------------------- P-4
@pytest.mark.parametrize("mode", ["gdn", "gla"])
def test_brute_force_unrolled_products(oracle_lib, mode):
    """S_t = S_0 prod_{r<=t} E_r + sum_{s<=t} f_s prod_{s<r<=t} E_r, with dense
    products, for every t <= 24."""
    rng = np.random.default_rng(6)
    T, dk, dv = 24, 6, 5
    q, k, v, alpha, beta, S0 = _head(rng, T, dk, dv, mode)
    o, ST = oracle.scan(mode, q, k, v, alpha, beta, S0)
    Es, fs = _elements(mode, k, v, alpha, beta)
    for t in range(T):
        P = np.eye(dk)
        for r in range(t + 1):
            P = P @ Es[r]
        S = S0 @ P
        for s in range(t + 1):
            Ps = np.eye(dk)
            for r in range(s + 1, t + 1):
                Ps = Ps @ Es[r]
            S = S + fs[s] @ Ps
        _check_close(o[t], S @ q[t].astype(np.float64), 1e-12)
        if t == T - 1:
            _check_close(ST, S, 1e-12)


# --------------------------------------------------------------------- P-5
def test_exact_rationals(oracle_lib):
    """Dyadic inputs, exact rational arithmetic over explicit E_t, f_t."""
    F = fractions.Fraction
    rng = np.random.default_rng(7)
    T, dk, dv = 6, 3, 2
    grid = np.array([-1.0, -0.5, -0.25, 0.0, 0.25, 0.5, 1.0])
    q = rng.choice(grid, (T, dk)).astype(np.float32)
    k = rng.choice(grid, (T, dk)).astype(np.float32)
    v = rng.choice(grid, (T, dv)).astype(np.float32)
    alpha = rng.choice([0.5, 0.75, 1.0], T).astype(np.float32)
    beta = rng.choice([0.0, 0.25, 0.5, 1.0], T).astype(np.float32)
    S0 = rng.choice(grid, (dv, dk))
    o, ST = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    S = [[F(float(S0[i, j])) for j in range(dk)] for i in range(dv)]
    for t in range(T):
        a, b = F(float(alpha[t])), F(float(beta[t]))
        kt = [F(float(x)) for x in k[t]]
        E = [[a * ((1 if i == j else 0) - b * kt[i] * kt[j]) for j in range(dk)] for i in range(dk)]
        S = [[sum(S[i][m] * E[m][j] for m in range(dk)) + b * F(float(v[t, i])) * kt[j]
              for j in range(dk)] for i in range(dv)]
        ot = [sum(S[i][j] * F(float(q[t, j])) for j in range(dk)) for i in range(dv)]
        for i in range(dv):
            assert abs(o[t, i] - float(ot[i])) <= 1e-14 * (1 + abs(float(ot[i])))
    for i, j in itertools.product(range(dv), range(dk)):
        assert abs(ST[i, j] - float(S[i][j])) <= 1e-14 * (1 + abs(float(S[i][j])))


# --------------------------------------------------------------------- P-6
def test_delta_rule_recall(oracle_lib):
    """alpha = beta = 1 and a unit key: the new state recalls exactly the
    written value for that key, S_t k_t = v_t, and leaves every direction
    orthogonal to k_t unchanged."""
    rng = np.random.default_rng(8)
    T, dk, dv = 10, 16, 16
    q, _, v, _, _, S0 = _head(rng, T, dk, dv)
    # keys of exactly unit norm in binary: +-1/2 on four random channels
    k = np.zeros((T, dk), np.float32)
    for t in range(T):
        k[t, rng.choice(dk, 4, replace=False)] = rng.choice([-0.5, 0.5], 4)
    alpha = np.ones(T, np.float32)
    beta = np.ones(T, np.float32)
    S_prev = S0.copy()
    for t in range(T):
        kt = k[t:t + 1]
        _, S_new = oracle.scan("gdn", q[t:t + 1], kt, v[t:t + 1], alpha[t:t + 1],
                               beta[t:t + 1], S_prev)
        k64 = kt[0].astype(np.float64)
        assert np.max(np.abs(S_new @ k64 - v[t].astype(np.float64))) < 1e-13
        x = rng.standard_normal(dk)
        x -= (x @ k64) / (k64 @ k64) * k64
        assert np.max(np.abs(S_new @ x - S_prev @ x)) < 1e-13
        S_prev = S_new


def test_delta_rule_basis_key_overwrites_column(oracle_lib):
    """k = e_j, alpha = beta = 1: column j of the state becomes v exactly and
    every other column is untouched, bit for bit."""
    rng = np.random.default_rng(9)
    dk, dv = 8, 5
    S0 = rng.standard_normal((dv, dk))
    for j in range(dk):
        k = np.zeros((1, dk), np.float32)
        k[0, j] = 1.0
        v = rng.standard_normal((1, dv)).astype(np.float32)
        _, ST = oracle.scan("gdn", k, k, v, np.ones(1, np.float32), np.ones(1, np.float32), S0)
        assert np.array_equal(ST[:, j], v[0].astype(np.float64))
        others = [c for c in range(dk) if c != j]
        assert np.array_equal(ST[:, others], S0[:, others])


# --------------------------------------------------------------------- P-7
@pytest.mark.parametrize("mode", ["gdn", "gla"])
def test_decode_steps_equal_scan(oracle_lib, mode):
    """Sequential view = parallel view: T single-token decode steps reproduce
    the full-sequence scan bit for bit."""
    rng = np.random.default_rng(10)
    N, T, dk, dv = 3, 17, 16, 8
    heads = [_head(rng, T, dk, dv, mode) for _ in range(N)]
    q = np.stack([h[0] for h in heads]); k = np.stack([h[1] for h in heads])
    v = np.stack([h[2] for h in heads]); alpha = np.stack([h[3] for h in heads])
    beta = np.stack([h[4] for h in heads]) if mode == "gdn" else None
    S0 = np.stack([h[5] for h in heads])
    o, ST = oracle.scan(mode, q, k, v, alpha, beta, S0)
    S = S0.copy()
    for t in range(T):
        ot = oracle.decode_step(mode, q[:, t], k[:, t], v[:, t], alpha[:, t],
                                None if beta is None else beta[:, t], S)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(S, ST)


# --------------------------------------------------------------------- P-8
@pytest.mark.parametrize("T1", [16, 23])
def test_split_resume(oracle_lib, T1):
    """Fixed-size state: scanning x[T1:] from the state left by x[:T1] equals
    scanning x, bit for bit."""
    rng = np.random.default_rng(11)
    T, dk, dv = 48, 8, 8
    q, k, v, alpha, beta, S0 = _head(rng, T, dk, dv)
    o, ST = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    o1, S1 = oracle.scan("gdn", q[:T1], k[:T1], v[:T1], alpha[:T1], beta[:T1], S0)
    o2, S2 = oracle.scan("gdn", q[T1:], k[T1:], v[T1:], alpha[T1:], beta[T1:], S1)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(S2, ST)


# --------------------------------------------------------------------- P-9
def test_linear_in_values_and_initial_state(oracle_lib):
    """For fixed (q, k, alpha, beta) the map (v, S_0) -> (o, S_T) is linear."""
    rng = np.random.default_rng(12)
    T, dk, dv = 25, 8, 6
    q, k, _, alpha, beta, _ = _head(rng, T, dk, dv)
    v1 = rng.integers(-8, 8, (T, dv)).astype(np.float32)
    v2 = rng.integers(-8, 8, (T, dv)).astype(np.float32)
    A1 = rng.standard_normal((dv, dk))
    A2 = rng.standard_normal((dv, dk))
    o1, S1 = oracle.scan("gdn", q, k, v1, alpha, beta, A1)
    o2, S2 = oracle.scan("gdn", q, k, v2, alpha, beta, A2)
    o3, S3 = oracle.scan("gdn", q, k, v1 + v2, alpha, beta, A1 + A2)
    _check_close(o3, o1 + o2, 1e-12)
    _check_close(S3, S1 + S2, 1e-12)
    o4, S4 = oracle.scan("gdn", q, k, 2 * v1, alpha, beta, 2 * A1)  # exact scaling
    assert np.array_equal(o4, 2 * o1) and np.array_equal(S4, 2 * S1)


# -------------------------------------------------------------------- P-10
def test_rows_and_heads_independent(oracle_lib):
    """Value channel i only ever touches row i of S: zeroing v[:, i] and row i
    of S_0 zeroes o[:, i] and S_T[i, :] exactly.  Heads are independent: a
    permutation of heads permutes the outputs, and the thread count does not
    change a single bit."""
    rng = np.random.default_rng(13)
    T, dk, dv = 21, 8, 8
    q, k, v, alpha, beta, S0 = _head(rng, T, dk, dv)
    i = 3
    v0 = v.copy(); v0[:, i] = 0
    S00 = S0.copy(); S00[i, :] = 0
    o, ST = oracle.scan("gdn", q, k, v0, alpha, beta, S00)
    assert np.all(o[:, i] == 0) and np.all(ST[i, :] == 0)
    H = 5
    hs = [_head(rng, T, dk, dv) for _ in range(H)]
    stack = [np.stack([h[j] for h in hs]) for j in range(6)]
    o, ST = oracle.scan("gdn", *stack, threads=1)
    perm = rng.permutation(H)
    op, STp = oracle.scan("gdn", *[x[perm] for x in stack], threads=7)
    assert np.array_equal(op, o[perm]) and np.array_equal(STp, ST[perm])


# -------------------------------------------------------------------- P-12
def test_state_norm_bound(oracle_lib):
    """Unit keys, beta in [0, 1], alpha <= 1: ||E_t||_2 <= 1 (eigenvalues
    alpha and alpha (1 - beta)), so ||S_t||_F <= ||S_{t-1}||_F + beta ||v_t||."""
    rng = np.random.default_rng(14)
    T, dk, dv = 60, 16, 16
    q, k, v, alpha, beta, S0 = _head(rng, T, dk, dv)
    S = S0[None].copy()
    for t in range(T):
        prev = np.linalg.norm(S)
        oracle.decode_step("gdn", q[t:t + 1], k[t:t + 1], v[t:t + 1], alpha[t:t + 1],
                           beta[t:t + 1], S)
        bound = prev + float(beta[t]) * np.linalg.norm(v[t].astype(np.float64))
        # keys are float32-rounded unit vectors, so allow their rounding
        assert np.linalg.norm(S) <= bound * (1 + 1e-6)


# ------------------------------------------------------------ chunk algebra
def _chunked_reference(mode, q, k, v, alpha, beta, S0, C):
    """Chunkwise UT/WY form of the same scan, written with numpy matmuls.

    Per chunk (tokens as rows; g = in-chunk cumulative log decay):
      A = strict_lower(diag(beta) (Gamma * K K^T)),  T = (I + A)^-1
      W = T diag(beta gamma) K,  U~ = T diag(beta) V,  U = U~ - W S^T
      O = diag(gamma) Q S^T + (Q K^T * Gamma * M) U
      S <- gamma_C S + U^T diag(exp(g_C - g)) K
    gla: U = V.  A ragged tail is padded with identity tokens (alpha = 1,
    beta = 0, q = k = v = 0)."""
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    a = alpha.astype(np.float64)
    b = beta.astype(np.float64) if beta is not None else None
    T = Q.shape[0]
    S = np.zeros((V.shape[1], K.shape[1])) if S0 is None else S0.copy()
    O = np.empty((T, V.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        n = e - s
        Qc, Kc, Vc = Q[s:e], K[s:e], V[s:e]
        g = np.cumsum(np.log(a[s:e]))
        gam = np.exp(g)
        Gam = np.exp(g[:, None] - g[None, :])
        M = np.tril(np.ones((n, n)))
        if mode == "gdn":
            bc = b[s:e]
            A = np.tril(bc[:, None] * Gam * (Kc @ Kc.T), -1)
            Tm = np.linalg.inv(np.eye(n) + A)
            W = Tm @ ((bc * gam)[:, None] * Kc)
            U = Tm @ (bc[:, None] * Vc) - W @ S.T
        else:
            U = Vc
        O[s:e] = gam[:, None] * (Qc @ S.T) + (Qc @ Kc.T * Gam * M) @ U
        S = gam[-1] * S + U.T @ (np.exp(g[-1] - g)[:, None] * Kc)
    return O, S


@pytest.mark.parametrize("mode", ["gdn", "gla"])
@pytest.mark.parametrize("T,C", [(64, 16), (100, 32), (130, 64)])
def test_chunkwise_form_equals_recurrence(oracle_lib, mode, T, C):
    """The chunkwise UT/WY identities the GPU kernels implement reproduce the
    token recurrence (including a ragged last chunk)."""
    rng = np.random.default_rng(15 + T)
    dk, dv = 16, 12
    q, k, v, alpha, beta, S0 = _head(rng, T, dk, dv, mode)
    o, ST = oracle.scan(mode, q, k, v, alpha, beta, S0)
    O, S = _chunked_reference(mode, q, k, v, alpha, beta, S0, C)
    _check_close(O, o, 1e-12)
    _check_close(S, ST, 1e-12)


def test_chunk_aggregate_composes(oracle_lib):
    """Chunk aggregates E_n = gamma_C I - W^T D K, f_n = U~^T D K satisfy
    S_n = S_{n-1} E_n + f_n and compose under the right-action combine."""
    rng = np.random.default_rng(16)
    T, C, dk, dv = 96, 32, 8, 8
    q, k, v, alpha, beta, S0 = _head(rng, T, dk, dv)
    _, ST = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    agg = (np.eye(dk), np.zeros((dv, dk)))
    for s in range(0, T, C):
        Kc = k[s:s + C].astype(np.float64); Vc = v[s:s + C].astype(np.float64)
        g = np.cumsum(np.log(alpha[s:s + C].astype(np.float64)))
        bc = beta[s:s + C].astype(np.float64)
        Gam = np.exp(g[:, None] - g[None, :])
        A = np.tril(bc[:, None] * Gam * (Kc @ Kc.T), -1)
        Tm = np.linalg.inv(np.eye(C) + A)
        W = Tm @ ((bc * np.exp(g))[:, None] * Kc)
        Ut = Tm @ (bc[:, None] * Vc)
        DK = np.exp(g[-1] - g)[:, None] * Kc
        agg = _combine(agg, (np.exp(g[-1]) * np.eye(dk) - W.T @ DK, Ut.T @ DK))
    _check_close(S0 @ agg[0] + agg[1], ST, 1e-12)


def test_zero_length_and_zero_state(oracle_lib):
    """T = 0 returns S_0 untouched; S_0 = None is the zero state."""
    rng = np.random.default_rng(17)
    q, k, v, alpha, beta, S0 = _head(rng, 0, 4, 4)
    o, ST = oracle.scan("gdn", q, k, v, alpha, beta, S0)
    assert o.shape == (0, 4) and np.array_equal(ST, S0)
    q, k, v, alpha, beta, _ = _head(rng, 5, 4, 4)
    o1, S1 = oracle.scan("gdn", q, k, v, alpha, beta, None)
    o2, S2 = oracle.scan("gdn", q, k, v, alpha, beta, np.zeros((4, 4)))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
