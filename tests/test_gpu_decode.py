"""decode_step on the GPU against the float64 oracle (same seeded inputs)."""
import numpy as np
import pytest
import torch

import oracle
import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

from _parity import TOL, assert_local, dev, host, max_err, say

pytestmark = pytest.mark.gpu


def _run(w, N, steps, states=None):
    """Run ``steps`` decode steps on the GPU; compare the listed states with
    the oracle over all steps (o of every step, final S)."""
    S0, q, k, v, alpha, beta = I.decode_inputs(w, N=N, steps=steps)
    states = list(range(N)) if states is None else states
    S = dev(S0)
    outs = []
    for s in range(steps):
        o = gds.decode_step(dev(q[s], w.dtype), dev(k[s], w.dtype), dev(v[s], w.dtype),
                            dev(alpha[s]), None if beta is None else dev(beta[s]), S)
        outs.append(o[states].float())
    torch.cuda.synchronize()
    o_gpu = np.stack([host(x) for x in outs], axis=1)          # [n, steps, dv]
    S_gpu = host(S)[states]
    Sr = S0[states].astype(np.float64)
    o_ref = np.empty((len(states), steps, w.dv))
    for s in range(steps):
        o_ref[:, s] = oracle.decode_step(w.mode, q[s, states], k[s, states], v[s, states],
                                         alpha[s, states],
                                         None if beta is None else beta[s, states], Sr)
    return o_gpu, S_gpu, o_ref, Sr


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["gdn", "gla"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 48), (128, 128), (128, 200)])
def test_decode_small(mode, dtype, dk, dv):
    base = I.WORKLOADS["decode-4096x100"]
    w = base.replace(mode=mode, dtype=dtype, dk=dk, dv=dv,
                     beta=base.beta if mode == "gdn" else None)
    say(f"decode small {mode} {dtype} dk={dk} dv={dv}")
    o, S, o_ref, S_ref = _run(w, N=7, steps=12)
    eo, es = max_err(o, o_ref, 1), max_err(S, S_ref, 1)
    say(f"  o {eo:.3e} S {es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_full_workload_sampled():
    """4096 states x 100 in-place steps at the full size; 12 states checked
    against the oracle on every step."""
    w = I.WORKLOADS["decode-4096x100"]
    N = w.B * w.H
    states = [0, 1, 77, 1023, 1024, 2047, 2048, 3000, 4000, 4093, 4094, 4095]
    say(f"decode full {N} states x {w.steps} steps")
    o, S, o_ref, S_ref = _run(w, N=N, steps=w.steps, states=states)
    eo, es = max_err(o, o_ref, 1), max_err(S, S_ref, 1)
    say(f"  o {eo:.3e} S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    # o stacked [state, step, value]: blocks of 64 steps per state
    assert_local(o, o_ref, 1, TOL["bf16"], "decode")


def test_decode_repeatable_bitwise():
    w = I.WORKLOADS["decode-4096x100"]
    S0, q, k, v, alpha, beta = I.decode_inputs(w, N=64, steps=3)
    res = []
    for _ in range(3):
        S = dev(S0)
        for s in range(3):
            o = gds.decode_step(dev(q[s], "bf16"), dev(k[s], "bf16"), dev(v[s], "bf16"),
                                dev(alpha[s]), dev(beta[s]), S)
        torch.cuda.synchronize()
        res.append((host(o), host(S)))
    for o, S in res[1:]:
        assert np.array_equal(o, res[0][0]) and np.array_equal(S, res[0][1])
