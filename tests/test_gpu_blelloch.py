"""The long-sequence path (leaf aggregates + fixed Blelloch tree + output pass)
against the float64 oracle, and against the sequential path on the same
inputs."""
import numpy as np
import pytest

import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

from _parity import assert_parity, gpu_scan, oracle_scan, say

pytestmark = pytest.mark.gpu


def _w(mode, T, B=1, H=3):
    base = I.WORKLOADS["long-b2h8t262144"]
    return base.replace(name="long-small", mode=mode, B=B, H=H, T=T,
                        beta=base.beta if mode == "gdn" else None,
                        alpha=base.alpha if mode == "gdn" else ("exp_uniform", -0.05, 0.0))


@pytest.mark.parametrize("mode", ["gdn", "gla"])
@pytest.mark.parametrize("T,leaf", [(64 * 37 + 5, 1), (64 * 37 + 5, 4), (64 * 64, 8),
                                    (64 * 2, 1), (64 * 5, 2), (100, 1), (64 * 130, 1)])
def test_blelloch_matches_oracle(mode, T, leaf):
    """Leaf counts that are and are not powers of two (identity padding), a
    ragged last chunk, a tree of one level, and a last leaf shorter than G.
    With gated linear attention up to 64 leaves take the per-element fold and
    more (256 here) the scaled sweeps."""
    w = _w(mode, T)
    b = I.batch_inputs(w)
    say(f"blelloch {mode} T={T} leaf_chunks={leaf}")
    o, ST = gpu_scan(w, b, path="blelloch", leaf_chunks=leaf)
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o, ST, o_ref, ST_ref, "bf16", what=f"blelloch {mode} T{T} G{leaf}")


def test_blelloch_and_sequential_agree():
    w = _w("gdn", 64 * 100 + 17, B=2, H=2)
    b = I.batch_inputs(w)
    say("blelloch vs sequential")
    o1, S1 = gpu_scan(w, b, path="blelloch", leaf_chunks=4)
    o2, S2 = gpu_scan(w, b, path="sequential")
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o1, S1, o_ref, ST_ref, "bf16", what="blelloch")
    assert_parity(o2, S2, o_ref, ST_ref, "bf16", what="sequential")


def test_blelloch_leaf_rows_of_E_that_reach_zero():
    """The rows of E in a leaf aggregate leave the chunk loop once their state is
    exactly zero.  Head 0 decays strongly everywhere (alpha ~ U(0.3, 0.5): E
    underflows within a few chunks of every 16-chunk leaf), head 1 has the long
    workload's mild gates (no leaf gets there), head 2 decays strongly in the
    first half of the sequence only; one launch holds all three.  Against the
    oracle and against the sequential path."""
    w = _w("gdn", 64 * 64 + 9, B=1, H=3)
    b = I.batch_inputs(w)
    rng = np.random.default_rng(17)
    T = w.T
    b.alpha[0, 0] = rng.uniform(0.3, 0.5, T).astype(b.alpha.dtype)
    b.alpha[0, 2, : T // 2] = rng.uniform(0.3, 0.5, T // 2).astype(b.alpha.dtype)
    say("blelloch, rows of E that reach zero")
    o1, S1 = gpu_scan(w, b, path="blelloch", leaf_chunks=16)
    o2, S2 = gpu_scan(w, b, path="sequential")
    o_ref, S_ref = oracle_scan(w, b)
    assert_parity(o1, S1, o_ref, S_ref, "bf16", what="blelloch, E rows reaching zero")
    assert_parity(o2, S2, o_ref, S_ref, "bf16", what="sequential, same gates")


def test_blelloch_zero_state_and_repeatable():
    w = _w("gdn", 64 * 20, B=1, H=2).replace(s0_var=None)
    b = I.batch_inputs(w)
    say("blelloch S0=None, bitwise repeat")
    runs = [gpu_scan(w, b, path="blelloch", leaf_chunks=2) for _ in range(2)]
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(runs[0][0], runs[0][1], o_ref, ST_ref, "bf16", what="blelloch S0 None")


def test_long_workload_sampled_heads():
    """B2 H8 T262144 in the launch configuration the benchmark would time
    (automatic path choice, default leaf size); two heads against the oracle
    over all 262144 tokens."""
    w = I.WORKLOADS["long-b2h8t262144"]
    nbytes = gds.scan_fwd_workspace_size(gds.SCAN_GDN, gds.SCAN_BF16, w.B, w.H, w.T, 128, 128, 64)
    assert nbytes > 0  # the automatic choice is the Blelloch path
    b = I.batch_inputs(w, threads=16)
    say(f"long workload, workspace {nbytes / 1e6:.0f} MB")
    o, ST = gpu_scan(w, b)
    heads = [(0, 0), (1, 7)]
    o_ref, ST_ref = oracle_scan(w, b, heads)
    sel = lambda x: np.stack([x[bb, hh] for bb, hh in heads])  # noqa: E731
    assert_parity(sel(o), sel(ST), o_ref, ST_ref, "bf16", head_dims=1, what=w.name)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
