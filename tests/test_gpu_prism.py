"""GPU parity of split erase/write strengths (SCAN_GDN_EW) and of PRISM's
rank-L write (prism_expand, then the split-strength scan; and prism_scan, the
same stream scanned in place) against the float64 oracle, through the C ABI.

Gates as for the plain scan: relative Frobenius error per head <= 1e-5 for
float32 data, <= 5e-3 for bfloat16 data with float32 state.  The expanded
stream is also compared element by element: pass-through rows and gates
exactly, the computed factors k^(l), delta^(l) within their storage rounding
(bfloat16: 2^-8 relative) plus the float32 arithmetic of the kernel.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import prism as oprism
import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

from _parity import TOL, assert_local, assert_parity, dev, host, max_err, say

pytestmark = pytest.mark.gpu


def _batch(w, T=None, heads=None):
    """Inputs of the first B x H heads of w at length T, as [B, H, ...] arrays."""
    T = w.T if T is None else T
    B, H = heads or (w.B, w.H)
    hs = [[I.head_inputs(w, b, h, T) for h in range(H)] for b in range(B)]
    st = lambda f: np.stack([np.stack([f(x) for x in row]) for row in hs])  # noqa: E731
    S0 = st(lambda x: x.S0) if w.s0_var is not None else None
    return st(lambda x: x.q), st(lambda x: x.k), st(lambda x: x.v), st(lambda x: x.alpha), \
        st(lambda x: x.beta), S0


def _write_plane(w, B, H, T):
    return np.stack([np.stack([I.write_strengths(w, b, h, T) for h in range(H)]) for b in range(B)])


# --------------------------------------------------------------------------
# split erase / write strengths
# --------------------------------------------------------------------------

SPLIT_CASES = [
    # (workload, B, H, T, chunk, path)
    ("tiny-gdn", 1, 3, 77, 16, "sequential"),                 # float32 kernel, ragged
    ("tiny-gdn", 2, 1, 64, 32, "sequential"),
    ("gdn-b8h16t8192", 1, 3, 200, 64, "sequential"),          # bf16 MFMA kernel, ragged tail
    ("gdn-b8h16t8192", 1, 2, 64 * 40 + 17, 64, "blelloch"),   # leaf aggregates + tree
]


@pytest.mark.parametrize("name,B,H,T,chunk,path", SPLIT_CASES)
def test_split_strength_scan(name, B, H, T, chunk, path):
    w = I.WORKLOADS[name]
    say(f"split-strength scan {name} B{B} H{H} T{T} chunk {chunk} {path}")
    q, k, v, alpha, be, S0 = _batch(w, T, (B, H))
    bw = _write_plane(w, B, H, T)
    beta2 = np.stack([be, bw])
    o, ST = gds.scan_fwd(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(alpha),
                         dev(beta2), None if S0 is None else dev(S0), chunk=chunk, path=path,
                         leaf_chunks=8 if path == "blelloch" else 0)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.scan("gdn_ew", q, k, v, alpha, beta2,
                               None if S0 is None else S0.astype(np.float64))
    assert_parity(host(o), host(ST), o_ref, S_ref, w.dtype, what=f"{name} {path}")


@pytest.mark.parametrize("name,chunk", [("tiny-gdn", 16), ("gdn-b8h16t8192", 64)])
def test_split_strength_equal_planes_is_gdn_bitwise(name, chunk):
    """Equal erase and write planes give exactly the plain gated-delta result."""
    w = I.WORKLOADS[name]
    say(f"split strengths with equal planes vs gdn: {name}")
    q, k, v, alpha, be, S0 = _batch(w, 150, (1, 2))
    args = [dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(alpha)]
    S0d = None if S0 is None else dev(S0)
    o1, S1 = gds.scan_fwd(*args, dev(be), S0d, chunk=chunk, path="sequential")
    o2, S2 = gds.scan_fwd(*args, dev(np.stack([be, be])), S0d, chunk=chunk, path="sequential")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("bf16", 128)])
def test_split_strength_decode(dtype, d):
    say(f"split-strength decode {dtype} d{d}")
    rng = np.random.default_rng(5)
    N = 12
    q = I.cast(rng.standard_normal((N, d)) / np.sqrt(d), dtype)
    k = rng.standard_normal((N, d))
    k = I.cast(k / np.linalg.norm(k, axis=1, keepdims=True), dtype)
    v = I.cast(rng.standard_normal((N, d)), dtype)
    alpha = I.cast(rng.uniform(0.9, 1.0, N), "f32")
    beta2 = I.cast(np.stack([rng.uniform(0, 1, N), rng.uniform(0, 1.5, N)]), "f32")
    S = I.cast(0.1 * rng.standard_normal((N, d, d)), "f32")
    Sd = dev(S)
    o = gds.decode_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(alpha), dev(beta2), Sd)
    torch.cuda.synchronize()
    S_ref = S.astype(np.float64)
    o_ref = oracle.decode_step("gdn_ew", q, k, v, alpha, beta2, S_ref)
    assert_parity(host(o), host(Sd), o_ref, S_ref, dtype, head_dims=1, what="decode")


# --------------------------------------------------------------------------
# PRISM write factors and the PRISM layer
# --------------------------------------------------------------------------


def _prism_batch(w, T, B, H):
    q, k, v, alpha, beta, S0 = _batch(w, T, (B, H))
    tok = [[I.prism_token_inputs(w, b, h, T) for h in range(H)] for b in range(B)]
    x = np.stack([np.stack([t[0] for t in row]) for row in tok])
    beta_l = np.stack([np.stack([t[1] for t in row]) for row in tok])
    wts = [I.prism_weights(w, h) for h in range(H)]
    conv = np.stack([p.conv for p in wts])
    Wk = np.stack([p.Wk for p in wts])
    Wp = np.stack([p.Wp for p in wts])
    return q, k, v, alpha, beta, S0, x, beta_l, conv, Wk, Wp


def _prism_gpu_args(w, a):
    q, k, v, alpha, beta, S0, x, beta_l, conv, Wk, Wp = a
    dt = w.dtype
    return (dev(q, dt), dev(k, dt), dev(v, dt), dev(alpha), dev(beta), dev(x, dt), dev(beta_l),
            dev(conv), dev(Wk, dt), dev(Wp, dt)), None if S0 is None else dev(S0)


def _factor_round(dtype):
    return (lambda z: I.cast(z, "bf16").astype(np.float64)) if dtype == "bf16" else None


PRISM_CASES = [("tiny-prism", 1, 2, 64), ("tiny-prism", 2, 1, 45),
               ("prism-b8h16t8192-l2", 1, 2, 150)]


@pytest.mark.parametrize("name,B,H,T,W", [c + (None,) for c in PRISM_CASES] +
                         [("prism-b8h16t8192-l2", 1, 1, 70, 1), ("prism-b8h16t8192-l2", 1, 1, 70, 8)])
def test_prism_expand_stream(name, B, H, T, W):
    """Pass-through rows exact, factor rows within storage rounding; the last two
    cases take the anchor window to its ends (1 and the largest, 8 taps) over a
    ragged second tile."""
    w = I.WORKLOADS[name]
    if W is not None:
        w = w.replace(prism_window=W)
    L = w.prism_steps
    G = L + 1
    say(f"prism_expand {name} B{B} H{H} T{T} L{L} W{w.prism_window}")
    a = _prism_batch(w, T, B, H)
    q, k, v, alpha, beta, S0, x, beta_l, conv, Wk, Wp = a
    args, _ = _prism_gpu_args(w, a)
    q2, k2, v2, a2, b2 = [host(t) for t in gds.prism_expand(*args)]
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            _, K, D = oprism.write_factors(x[b, h], v[b, h], conv[h], Wk[h], Wp[h])
            rq, rk, rv, ra, rb = oprism.expand(q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h],
                                               K, D, beta_l[b, h])
            # pass-through rows and gates: exact
            np.testing.assert_array_equal(q2[b, h], rq)
            np.testing.assert_array_equal(k2[b, h, ::G], rk[::G])
            np.testing.assert_array_equal(v2[b, h, ::G], rv[::G])
            np.testing.assert_array_equal(a2[b, h], ra)
            np.testing.assert_array_equal(b2[:, b, h], rb)
            # computed factors: storage rounding plus float32 arithmetic
            rel = 2.0 ** -8 if w.dtype == "bf16" else 1e-5
            for got, ref in ((k2[b, h].reshape(T, G, -1)[:, 1:], K),
                             (v2[b, h].reshape(T, G, -1)[:, 1:], D)):
                scale = np.sqrt(np.mean(ref ** 2))
                err = np.abs(got - ref)
                bound = rel * np.abs(ref) + (2.0 ** -12 if w.dtype == "bf16" else 1e-6) * scale
                worst = float(np.max(err - bound))
                say(f"  head ({b},{h}) factor max err {float(np.max(err)):.3e} (scale {scale:.3e})")
                assert worst <= 0, f"factor error exceeds bound by {worst:.3e}"


@pytest.mark.parametrize("name,B,H,T", PRISM_CASES + [("prism-b8h16t8192-l2", 1, 2, 64 * 33 + 5)])
def test_prism_layer(name, B, H, T):
    w = I.WORKLOADS[name]
    say(f"prism layer {name} B{B} H{H} T{T}")
    a = _prism_batch(w, T, B, H)
    q, k, v, alpha, beta, S0, x, beta_l, conv, Wk, Wp = a
    args, S0d = _prism_gpu_args(w, a)
    o, ST = gds.prism_scan_fwd(*args, S0d, chunk=w.chunk)
    torch.cuda.synchronize()
    o_ref = np.empty(o.shape)
    S_ref = np.empty(ST.shape)
    for b in range(B):
        for h in range(H):
            o_ref[b, h], S_ref[b, h] = oprism.prism_scan(
                q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h], x[b, h], conv[h], Wk[h], Wp[h],
                beta_l[b, h], None if S0 is None else S0[b, h].astype(np.float64),
                factor_round=_factor_round(w.dtype))
    assert_parity(host(o), host(ST), o_ref, S_ref, w.dtype, what=name)


@pytest.mark.parametrize("L,T", [(1, 200), (2, 64 * 21 + 1), (3, 333), (8, 100), (2, 1)])
def test_prism_scan_in_place_equals_stream_scan_bitwise(L, T):
    """prism_scan reads PRISM's element stream in place (q only on a token's last
    element, k, v and gates from the token arrays or the factor rows, o once per
    token): its o and S_T equal the sequential scan_fwd over prism_expand's
    materialised stream, read at each token's last element, bit for bit.
    Ragged element counts, tokens that straddle chunks (L = 2, 3), the largest
    L (8: nine elements per token) and a single token."""
    w = I.WORKLOADS["prism-b8h16t8192-l2"].replace(prism_steps=L)
    say(f"prism_scan in place vs stream scan: L{L} T{T} (elements {T * (L + 1)})")
    a = _prism_batch(w, T, 1, 2)
    args, S0d = _prism_gpu_args(w, a)
    o1, S1 = gds.prism_scan(*args, S0d)
    # (the sequential path, as the in-place scan: the tree brackets differently)
    o2, S2 = gds.prism_scan_fwd(*args, S0d, stream=True, path="sequential")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.contiguous()), "o differs"
    assert torch.equal(S1, S2), "S_T differs"


def test_prism_scan_without_corrections_is_the_gdn_scan():
    """prism_scan with L = 0 is the gated-delta scan, bit for bit."""
    w = I.WORKLOADS["prism-b8h16t8192-l2"]
    say("prism_scan L=0 vs gdn scan (bitwise)")
    q, k, v, alpha, beta, S0 = _batch(w, 130, (1, 2))
    dt = w.dtype
    args = (dev(q, dt), dev(k, dt), dev(v, dt), dev(alpha), dev(beta))
    o1, S1 = gds.prism_scan(*args, S0=dev(S0))
    o2, S2 = gds.scan_fwd(*args, dev(S0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_prism_without_corrections_is_the_gdn_scan():
    """L = 0: the expanded stream is the input stream and the layer is the scan."""
    w = I.WORKLOADS["prism-b8h16t8192-l2"]
    say("prism L=0 vs gdn scan (bitwise)")
    q, k, v, alpha, beta, S0 = _batch(w, 130, (1, 2))
    dt = w.dtype
    args = (dev(q, dt), dev(k, dt), dev(v, dt), dev(alpha), dev(beta))
    o1, S1 = gds.prism_scan_fwd(*args, S0=dev(S0))
    o2, S2 = gds.scan_fwd(*args, dev(S0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_prism_full_workload_sampled_heads():
    """The PRISM workload at full size in the benchmark's launch configuration;
    two heads checked against the oracle."""
    w = I.WORKLOADS["prism-b8h16t8192-l2"]
    say(f"prism full workload {w.name}: B{w.B} H{w.H} T{w.T} L{w.prism_steps}")
    B, H, T = w.B, w.H, w.T
    b = I.batch_inputs(w)
    tok = [[I.prism_token_inputs(w, bb, hh) for hh in range(H)] for bb in range(B)]
    x = np.stack([np.stack([t[0] for t in row]) for row in tok])
    beta_l = np.stack([np.stack([t[1] for t in row]) for row in tok])
    del tok
    wts = [I.prism_weights(w, hh) for hh in range(H)]
    conv = np.stack([p.conv for p in wts])
    Wk = np.stack([p.Wk for p in wts])
    Wp = np.stack([p.Wp for p in wts])
    dt = w.dtype
    o, ST = gds.prism_scan_fwd(dev(b.q, dt), dev(b.k, dt), dev(b.v, dt), dev(b.alpha),
                               dev(b.beta), dev(x, dt), dev(beta_l), dev(conv), dev(Wk, dt),
                               dev(Wp, dt), dev(b.S0), chunk=w.chunk)
    torch.cuda.synchronize()
    o, ST = host(o), host(ST)
    for bb, hh in [(0, 0), (B - 1, H - 1)]:
        o_ref, S_ref = oprism.prism_scan(b.q[bb, hh], b.k[bb, hh], b.v[bb, hh], b.alpha[bb, hh],
                                         b.beta[bb, hh], x[bb, hh], conv[hh], Wk[hh], Wp[hh],
                                         beta_l[bb, hh], b.S0[bb, hh].astype(np.float64),
                                         factor_round=_factor_round(dt))
        eo = max_err(o[bb, hh][None], o_ref[None], 1)
        es = max_err(ST[bb, hh][None], S_ref[None], 1)
        say(f"  head ({bb},{hh}): o {eo:.3e}  S_T {es:.3e}  (gate {TOL[dt]:.0e})")
        assert eo <= TOL[dt] and es <= TOL[dt]
        assert_local(o[bb, hh][None], o_ref[None], 1, TOL[dt], f"head ({bb},{hh})")
