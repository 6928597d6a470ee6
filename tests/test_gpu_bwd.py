"""GPU parity of scan_bwd (the scan's gradient through the chunkwise form)
against the float64 oracle gradient (oracle.scan_bwd), through the C ABI.

Every gradient is float32 and is compared per head by relative Frobenius
error, gate 1e-4 for both input dtypes: the kernel works in float32 on the same
(bf16-exact) values the oracle sees, so no bf16 rounding enters the outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

from _parity import dev, host, max_err, say

pytestmark = pytest.mark.gpu
GATE = 1e-4
NAMES = ["dq", "dk", "dv", "dalpha", "dbeta", "dS0"]


def _batch(w, T, B, H, with_s0=True, with_dO=True, with_dST=True):
    hs = [[I.head_inputs(w, b, h, T) for h in range(H)] for b in range(B)]
    gs = [[I.output_grads(w, b, h, T) for h in range(H)] for b in range(B)]
    st = lambda f, rows: np.stack([np.stack([f(x) for x in r]) for r in rows])  # noqa: E731
    q, k, v = st(lambda x: x.q, hs), st(lambda x: x.k, hs), st(lambda x: x.v, hs)
    a = st(lambda x: x.alpha, hs)
    beta = st(lambda x: x.beta, hs) if w.beta is not None else None
    S0 = st(lambda x: x.S0, hs) if (with_s0 and w.s0_var is not None) else None
    dO = st(lambda g: g[0], gs) if with_dO else None
    dST = st(lambda g: g[1], gs) if with_dST else None
    return q, k, v, a, beta, S0, dO, dST


def _run(w, q, k, v, a, beta, S0, dO, dST):
    dt = w.dtype
    up = lambda x, d="f32": None if x is None else dev(x, d)  # noqa: E731
    g = gds.scan_bwd(up(q, dt), up(k, dt), up(v, dt), up(a), up(beta), up(S0), up(dO, dt), up(dST))
    torch.cuda.synchronize()
    return [None if x is None else host(x) for x in g]


def _check(got, ref, what, gate=GATE, head_dims=2):
    errs = {}
    for name, x, r in zip(NAMES, got, ref):
        if r is None:
            assert x is None, name
            continue
        errs[name] = max_err(x, r, head_dims)
    say(f"  {what}: " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= gate, f"{what}: {n} error {e:.3e} > {gate:.0e}"


CASES = [
    # (workload, mode, dtype, B, H, T, dk, dv)
    ("tiny-gdn", "gdn", "f32", 1, 2, 100, 32, 64),
    ("tiny-gdn", "gla", "f32", 1, 2, 77, 32, 64),
    ("tiny-gdn", "gdn", "f32", 2, 1, 64, 64, 128),
    ("tiny-gdn", "gdn", "f32", 1, 1, 33, 128, 64),
    ("tiny-gdn", "gla", "f32", 1, 1, 130, 128, 192),
    ("gdn-b8h16t8192", "gdn", "bf16", 1, 2, 200, 128, 128),
    ("gdn-b8h16t8192", "gla", "bf16", 1, 2, 97, 128, 128),
    ("gdn-b8h16t8192", "gdn", "bf16", 1, 1, 5, 128, 128),
    # bf16 at d_k = 64 (the stored state's permuted layout over 16 units of a
    # row) and GLA at d_k = 64, with ragged tails
    ("gdn-b8h16t8192", "gdn", "bf16", 1, 2, 150, 64, 64),
    ("tiny-gdn", "gla", "f32", 1, 1, 95, 64, 128),
]


@pytest.mark.parametrize("name,mode,dtype,B,H,T,dk,dv", CASES)
def test_scan_bwd(name, mode, dtype, B, H, T, dk, dv):
    w = I.WORKLOADS[name].replace(mode=mode, dtype=dtype, dk=dk, dv=dv,
                                  beta=I.WORKLOADS["gdn-b8h16t8192"].beta if mode == "gdn" else None,
                                  s0_var=0.01)
    say(f"scan_bwd {name} {mode} {dtype} B{B} H{H} T{T} dk{dk} dv{dv}")
    q, k, v, a, beta, S0, dO, dST = _batch(w, T, B, H)
    got = _run(w, q, k, v, a, beta, S0, dO, dST)
    ref = oracle.scan_bwd(mode, q, k, v, a, beta, S0, dO, dST)
    _check(got, ref, f"{mode} {dtype} T{T} dk{dk} dv{dv}")


@pytest.mark.parametrize("mode", ["gdn", "gla"])
def test_scan_bwd_missing_optionals(mode):
    """No S0, no dO (only dST), then no dST (only dO)."""
    w = I.WORKLOADS["tiny-gdn"].replace(mode=mode, dk=32, dv=64, s0_var=0.01,
                                        beta=I.WORKLOADS["gdn-b8h16t8192"].beta if mode == "gdn" else None)
    for with_s0, with_dO, with_dST in [(False, False, True), (True, True, False)]:
        say(f"scan_bwd optionals {mode}: S0 {with_s0} dO {with_dO} dST {with_dST}")
        q, k, v, a, beta, S0, dO, dST = _batch(w, 70, 1, 2, with_s0, with_dO, with_dST)
        got = _run(w, q, k, v, a, beta, S0, dO, dST)
        ref = oracle.scan_bwd(mode, q, k, v, a, beta, S0, dO, dST)
        _check(got, ref, f"{mode} S0 {with_s0} dO {with_dO} dST {with_dST}")


def test_scan_bwd_repeatable():
    """Two calls give bitwise identical gradients (fixed summation order)."""
    w = I.WORKLOADS["gdn-b8h16t8192"].replace(dtype="bf16")
    say("scan_bwd bitwise repeatability")
    q, k, v, a, beta, S0, dO, dST = _batch(w, 300, 1, 2)
    g1 = _run(w, q, k, v, a, beta, S0, dO, dST)
    g2 = _run(w, q, k, v, a, beta, S0, dO, dST)
    for n, x, y in zip(NAMES, g1, g2):
        np.testing.assert_array_equal(x, y, err_msg=n)


def test_scan_bwd_full_workload_sampled_heads():
    """The bench shape (B8 H16 T8192 d128, bf16), two heads recomputed by the
    oracle over their whole length (heads are independent)."""
    w = I.WORKLOADS["gdn-b8h16t8192"]
    say(f"scan_bwd full workload {w.name}: B{w.B} H{w.H} T{w.T}")
    b = I.batch_inputs(w)
    dO = np.empty((w.B, w.H, w.T, w.dv), np.float32)
    dST = np.empty((w.B, w.H, w.dv, w.dk), np.float32)
    for bb in range(w.B):
        for hh in range(w.H):
            dO[bb, hh], dST[bb, hh] = I.output_grads(w, bb, hh)
    got = _run(w, b.q, b.k, b.v, b.alpha, b.beta, b.S0, dO, dST)
    for bb, hh in [(0, 0), (w.B - 1, w.H - 1)]:
        ref = oracle.scan_bwd("gdn", b.q[bb, hh], b.k[bb, hh], b.v[bb, hh], b.alpha[bb, hh],
                              b.beta[bb, hh], b.S0[bb, hh], dO[bb, hh], dST[bb, hh])
        sel = [None if x is None else x[bb, hh][None] for x in got]
        refs = [None if r is None else r[None] for r in ref]
        _check(sel, refs, f"head ({bb},{hh})", head_dims=1)


@pytest.mark.parametrize("dtype,T,dk,dv", [("f32", 90, 64, 64), ("bf16", 133, 128, 128)])
def test_scan_bwd_split_strengths(dtype, T, dk, dv):
    """SCAN_GDN_EW: erase strengths beta, write strengths bw (as in PRISM's
    element stream); dbeta comes back in the same two planes."""
    w = I.WORKLOADS["gdn-b8h16t8192"].replace(dtype=dtype, dk=dk, dv=dv)
    B, H = 1, 2
    say(f"scan_bwd split strengths {dtype} B{B} H{H} T{T} dk{dk} dv{dv}")
    q, k, v, a, beta, S0, dO, dST = _batch(w, T, B, H)
    bw = np.stack([np.stack([I.write_strengths(w, b, h, T) for h in range(H)]) for b in range(B)])
    be2 = np.stack([beta, bw])
    got = _run(w, q, k, v, a, be2, S0, dO, dST)
    ref = oracle.scan_bwd("gdn_ew", q, k, v, a, be2, S0, dO, dST)
    # dbeta [2, B, H, T]: compare each plane per head
    _check(got[:4] + [None, got[5]], list(ref[:4]) + [None, ref[5]], f"ew {dtype} T{T}")
    for pl, name in ((0, "erase"), (1, "write")):
        e = max_err(got[4][pl], ref[4][pl], 2)
        say(f"  dbeta {name} plane: {e:.2e}")
        assert e <= GATE
    # equal planes reduce to the delta rule: dbeta planes add up to its dbeta
    g1 = _run(w, q, k, v, a, beta, S0, dO, dST)
    g2 = _run(w, q, k, v, a, np.stack([beta, beta]), S0, dO, dST)
    assert max_err(g2[4][0] + g2[4][1], g1[4], 2) <= GATE
