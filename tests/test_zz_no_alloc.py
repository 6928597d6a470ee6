"""scan_fwd_noalloc (the entry point for callers that cannot allocate device
memory) against scan_fwd with a caller workspace, through the C ABI.

Both run the same kernels in the same order, so their outputs must agree bit
for bit.  Two calls in a row on the library's shared per-GPU scratch, the
second smaller than the first, catch a second call that depends on what the
first left there; the smaller call is also checked against the oracle."""
import numpy as np
import pytest
import torch

import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

from _parity import assert_parity, dev, host, oracle_scan, say

pytestmark = pytest.mark.gpu


def _w(mode, B, H, T):
    base = I.WORKLOADS["long-b2h8t262144"]
    return base.replace(name="noalloc", mode=mode, B=B, H=H, T=T,
                        beta=base.beta if mode == "gdn" else None,
                        alpha=base.alpha if mode == "gdn" else ("exp_uniform", -0.05, 0.0))


def _both(w, leaf):
    """(o, ST) of scan_fwd and of scan_fwd_noalloc on the same inputs, as host arrays."""
    b = I.batch_inputs(w)
    q, k, v = dev(b.q, w.dtype), dev(b.k, w.dtype), dev(b.v, w.dtype)
    alpha = dev(b.alpha)
    beta = dev(b.beta) if b.beta is not None else None
    S0 = dev(b.S0) if b.S0 is not None else None
    mode = gds.SCAN_GDN if w.mode == "gdn" else gds.SCAN_GLA
    need = gds.scan_fwd_workspace_size(mode, gds.SCAN_BF16, w.B, w.H, w.T, w.dk, w.dv, 64,
                                       "blelloch", leaf)
    assert 0 < need <= gds._lib.SCAN_NOALLOC_MAX_WORKSPACE, need
    o_ref, ST_ref = gds.scan_fwd(q, k, v, alpha, beta, S0, path="blelloch", leaf_chunks=leaf)
    # outputs filled with a pattern, so that anything left unwritten shows
    o = torch.full_like(o_ref, 7.0)
    ST = torch.full_like(ST_ref, 7.0)
    gds.scan_fwd_noalloc(q, k, v, alpha, beta, S0, o=o, ST=ST, path="blelloch", leaf_chunks=leaf)
    torch.cuda.synchronize()
    return b, need, (host(o_ref), host(ST_ref)), (host(o), host(ST))


@pytest.mark.parametrize("mode", ["gdn", "gla"])
def test_noalloc_matches_scan_fwd_on_two_calls(mode):
    cases = [(_w(mode, 2, 4, 64 * 128), 16),      # 8 heads x 8 leaves
             (_w(mode, 1, 2, 64 * 46 + 29), 16)]  # smaller: 2 heads x 3 leaves (+1 padding), ragged
    for i, (w, leaf) in enumerate(cases):
        say(f"noalloc {mode} call {i + 1}: B={w.B} H={w.H} T={w.T} leaf_chunks={leaf}")
        b, need, (o_ref, ST_ref), (o, ST) = _both(w, leaf)
        say(f"  workspace {need} bytes")
        assert np.array_equal(o, o_ref), "o differs"
        assert np.array_equal(ST, ST_ref), "S_T differs"
        if i == 1:
            o_or, ST_or = oracle_scan(w, b)
            assert_parity(o, ST, o_or, ST_or, "bf16", what=f"noalloc {mode}")


def test_noalloc_sequential_path_needs_no_scratch():
    """Where the plan needs no workspace the entry point is scan_fwd itself."""
    w = _w("gdn", 1, 2, 64 * 3 + 1)
    b = I.batch_inputs(w)
    q, k, v = dev(b.q, w.dtype), dev(b.k, w.dtype), dev(b.v, w.dtype)
    alpha, beta, S0 = dev(b.alpha), dev(b.beta), dev(b.S0)
    say("noalloc sequential path")
    o_ref, ST_ref = gds.scan_fwd(q, k, v, alpha, beta, S0, path="sequential")
    o = torch.empty_like(o_ref)
    ST = torch.empty_like(ST_ref)
    gds.scan_fwd_noalloc(q, k, v, alpha, beta, S0, o=o, ST=ST, path="sequential")
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ST, ST_ref)
