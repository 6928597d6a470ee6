"""GPU parity of the large-chunk fast-weight update (lact_fwd) against the
float64 oracle (oracle/lact.py), through the C ABI.

Gates: relative Frobenius error per head <= 1e-5 for float32 data (plain
kernel), <= 5e-3 for bfloat16 data (MFMA path: chunk statistics in split bf16,
float32 recursion, bf16 applied weight and output), for o and the final weight.
"""
import numpy as np
import pytest
import torch

from oracle import lact as olact
import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

from _parity import TOL, assert_local, assert_parity, dev, host, max_err, say

pytestmark = pytest.mark.gpu

ORDERS = {"update_then_apply": olact.UPDATE_THEN_APPLY, "apply_then_update": olact.APPLY_THEN_UPDATE}


def _batch(w, T, B, H):
    hs = [[I.head_inputs(w, b, h, T) for h in range(H)] for b in range(B)]
    st = lambda f: np.stack([np.stack([f(x) for x in row]) for row in hs])  # noqa: E731
    eta = np.stack([np.stack([I.lact_eta(w, b, h, T) for h in range(H)]) for b in range(B)])
    W0 = st(lambda x: x.S0) if w.s0_var is not None else None
    return st(lambda x: x.q), st(lambda x: x.k), st(lambda x: x.v), eta, W0


CASES = [
    # (workload, B, H, T, chunk, with W0)
    ("tiny-lact", 1, 2, 100, 16, True),          # plain kernel, ragged last chunk
    ("tiny-lact", 2, 1, 64, 64, False),          # one chunk = the sequence
    ("lact-b8h16t8192-m2048", 1, 2, 64 * 20 + 17, 256, True),   # MFMA path, ragged tile and chunk
    ("lact-b8h16t8192-m2048", 1, 2, 1000, 1024, False),         # one chunk, shorter than it
    ("lact-b8h16t8192-m2048", 1, 1, 5000, 4096, True),          # two splits per chunk, ragged
]


@pytest.mark.parametrize("order", ["update_then_apply", "apply_then_update"])
@pytest.mark.parametrize("name,B,H,T,chunk,w0", CASES)
def test_lact(name, B, H, T, chunk, w0, order):
    w = I.WORKLOADS[name].replace(chunk=chunk)
    say(f"lact {name} B{B} H{H} T{T} chunk {chunk} W0 {w0} {order}")
    q, k, v, eta, W0 = _batch(w, T, B, H)
    if not w0:
        W0 = None
    o, WT = gds.lact_fwd(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(eta),
                         None if W0 is None else dev(W0), chunk=chunk, order=order)
    torch.cuda.synchronize()
    o_ref, W_ref = olact.lact_batch(q, k, v, eta, chunk, ORDERS[order],
                                    None if W0 is None else W0.astype(np.float64))
    assert_parity(host(o), host(WT), o_ref, W_ref, w.dtype, what=f"{name} {order}")


def test_lact_in_place_weight_and_repeat_bitwise():
    """WT may be W0 itself; two identical calls give identical bits."""
    w = I.WORKLOADS["lact-b8h16t8192-m2048"]
    say("lact in-place weight, repeatability")
    q, k, v, eta, W0 = _batch(w, 640, 1, 2)
    args = (dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(eta))
    o1, W1 = gds.lact_fwd(*args, dev(W0), chunk=128)
    W = dev(W0)
    o2, W2 = gds.lact_fwd(*args, W, chunk=128, WT=W)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(W1, W2) and W2.data_ptr() == W.data_ptr()


def test_lact_full_workload_sampled_heads():
    w = I.WORKLOADS["lact-b8h16t8192-m2048"]
    say(f"lact full workload {w.name}: B{w.B} H{w.H} T{w.T} chunk {w.chunk}")
    b = I.batch_inputs(w)
    eta = np.stack([np.stack([I.lact_eta(w, bb, hh) for hh in range(w.H)]) for bb in range(w.B)])
    o, WT = gds.lact_fwd(dev(b.q, "bf16"), dev(b.k, "bf16"), dev(b.v, "bf16"), dev(eta),
                         dev(b.S0), chunk=w.chunk)
    torch.cuda.synchronize()
    o, WT = host(o), host(WT)
    for bb, hh in [(0, 0), (w.B - 1, w.H - 1)]:
        o_ref, W_ref = olact.lact(b.q[bb, hh], b.k[bb, hh], b.v[bb, hh], eta[bb, hh], w.chunk,
                                  olact.UPDATE_THEN_APPLY, b.S0[bb, hh].astype(np.float64))
        eo = max_err(o[bb, hh][None], o_ref[None], 1)
        ew = max_err(WT[bb, hh][None], W_ref[None], 1)
        say(f"  head ({bb},{hh}): o {eo:.3e}  W_T {ew:.3e}  (gate {TOL['bf16']:.0e})")
        assert eo <= TOL["bf16"] and ew <= TOL["bf16"]
        assert_local(o[bb, hh][None], o_ref[None], 1, TOL["bf16"], f"head ({bb},{hh})")
