"""scan_fwd on the GPU against the float64 oracle (same seeded inputs).

Small cases span several chunks and a ragged tail; the named full-size
workloads are checked on sampled heads (each head is independent, so the
oracle recomputes just those heads over their whole length)."""
import numpy as np
import pytest
import torch

import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

from _parity import TOL, assert_parity, dev, gpu_scan, host, oracle_scan, say

pytestmark = pytest.mark.gpu


def _small(mode, dtype, T, d, chunk, B=2, H=3, s0=True):
    base = I.WORKLOADS["gdn-b8h16t8192"]
    return base.replace(name="small", mode=mode, dtype=dtype, B=B, H=H, T=T, dk=d, dv=d,
                        chunk=chunk, beta=base.beta if mode == "gdn" else None,
                        alpha=base.alpha if mode == "gdn" else ("exp_uniform", -0.05, 0.0),
                        s0_var=0.01 if s0 else None)


def test_tiny_workload_f32():
    """B1 H1 T64 d16, float32, chunk 16: the 1e-5 gate."""
    w = I.WORKLOADS["tiny-gdn"]
    b = I.batch_inputs(w)
    say("tiny-gdn f32")
    o, ST = gpu_scan(w, b)
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o, ST, o_ref, ST_ref, "f32", what="tiny-gdn")


@pytest.mark.parametrize("mode", ["gdn", "gla"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_f32_sizes_and_chunks(mode, d, chunk):
    """float32 path: every supported head size and chunk, T with a ragged tail."""
    w = _small(mode, "f32", T=3 * chunk + 7, d=d, chunk=chunk)
    b = I.batch_inputs(w)
    say(f"f32 {mode} d={d} chunk={chunk} T={w.T}")
    o, ST = gpu_scan(w, b)
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o, ST, o_ref, ST_ref, "f32", what=f"{mode} d{d} C{chunk}")


@pytest.mark.parametrize("mode", ["gdn", "gla"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 1000])
def test_bf16_lengths(mode, T):
    """bfloat16 inputs at d = 128, chunk 64: lengths below, at and above a
    chunk, several chunks with ragged tails."""
    w = _small(mode, "bf16", T=T, d=128, chunk=64)
    b = I.batch_inputs(w)
    say(f"bf16 {mode} T={T}")
    o, ST = gpu_scan(w, b)
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o, ST, o_ref, ST_ref, "bf16", what=f"bf16 {mode} T{T}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bf16_chunk_size_invariance(chunk):
    """Chunking is exact algebra: every chunk size meets the gate on the same
    inputs."""
    w = _small("gdn", "bf16", T=512, d=128, chunk=chunk)
    b = I.batch_inputs(w)
    say(f"bf16 chunk {chunk}")
    o, ST = gpu_scan(w, b)
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o, ST, o_ref, ST_ref, "bf16", what=f"chunk {chunk}")


def test_zero_state_null_and_state_skip():
    w = _small("gdn", "bf16", T=130, d=128, chunk=64, s0=False)
    b = I.batch_inputs(w)
    say("S0=None, ST skipped")
    o, ST = gpu_scan(w, b, write_state=False)
    assert ST is None
    o_ref, _ = oracle_scan(w, b)
    assert_parity(o, None, o_ref, None, "bf16", what="S0 None")


def test_state_in_place_carry():
    """ST may alias S0: the library consumes S0 before writing ST."""
    w = _small("gdn", "bf16", T=200, d=128, chunk=64)
    b = I.batch_inputs(w)
    say("ST == S0")
    S = dev(b.S0)
    o, ST = gds.scan_fwd(dev(b.q, "bf16"), dev(b.k, "bf16"), dev(b.v, "bf16"), dev(b.alpha),
                         dev(b.beta), S, ST=S)
    torch.cuda.synchronize()
    o_ref, ST_ref = oracle_scan(w, b)
    assert ST.data_ptr() == S.data_ptr()
    assert_parity(host(o), host(S), o_ref, ST_ref, "bf16", what="in-place")


def test_split_resume_matches_whole():
    """scan(x) and scan(x[T1:], S0 = scan(x[:T1]).S_T) agree (T1 not a chunk
    multiple), both against the oracle."""
    w = _small("gdn", "bf16", T=300, d=128, chunk=64)
    b = I.batch_inputs(w)
    T1 = 157
    say("split/resume")
    q, k, v = dev(b.q, "bf16"), dev(b.k, "bf16"), dev(b.v, "bf16")
    al, be, S0 = dev(b.alpha), dev(b.beta), dev(b.S0)
    o1, S1 = gds.scan_fwd(q[:, :, :T1].contiguous(), k[:, :, :T1].contiguous(),
                          v[:, :, :T1].contiguous(), al[:, :, :T1].contiguous(),
                          be[:, :, :T1].contiguous(), S0)
    o2, S2 = gds.scan_fwd(q[:, :, T1:].contiguous(), k[:, :, T1:].contiguous(),
                          v[:, :, T1:].contiguous(), al[:, :, T1:].contiguous(),
                          be[:, :, T1:].contiguous(), S1)
    torch.cuda.synchronize()
    o = np.concatenate([host(o1), host(o2)], axis=2)
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o, host(S2), o_ref, ST_ref, "bf16", what="split/resume")


def test_decode_steps_match_scan():
    """Sequential view = parallel view on the GPU: T decode steps and one
    scan_fwd over the same tokens meet the gate against the same oracle."""
    w = _small("gdn", "bf16", T=40, d=128, chunk=64, B=1, H=4)
    b = I.batch_inputs(w)
    say("decode x T vs scan")
    o_scan, ST_scan = gpu_scan(w, b)
    S = dev(b.S0[0])
    outs = []
    for t in range(w.T):
        outs.append(host(gds.decode_step(dev(b.q[0, :, t], "bf16"), dev(b.k[0, :, t], "bf16"),
                                         dev(b.v[0, :, t], "bf16"), dev(b.alpha[0, :, t]),
                                         dev(b.beta[0, :, t]), S)))
    torch.cuda.synchronize()
    o_dec = np.stack(outs, axis=1)[None]
    o_ref, ST_ref = oracle_scan(w, b)
    assert_parity(o_dec, host(S)[None], o_ref, ST_ref, "bf16", what="decode x T")
    assert_parity(o_scan, ST_scan, o_ref, ST_ref, "bf16", what="scan")


def test_repeatable_bitwise():
    """Fixed order of every reduction: three runs give identical bits (this
    also exposes LDS races, which show up as run-to-run differences)."""
    w = _small("gdn", "bf16", T=777, d=128, chunk=64, B=2, H=4)
    b = I.batch_inputs(w)
    say("bitwise repeat")
    runs = [gpu_scan(w, b) for _ in range(3)]
    for o, ST in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(ST, runs[0][1])


@pytest.mark.parametrize("name", ["gla-b4h8t4096", "gdn-b8h16t8192"])
def test_full_workload_sampled_heads(name):
    """Full-size workloads in the launch configuration the benchmark times;
    sampled heads against the oracle over their whole length."""
    w = I.WORKLOADS[name]
    b = I.batch_inputs(w, threads=16)
    say(f"full {name}")
    o, ST = gpu_scan(w, b)
    heads = [(0, 0), (w.B // 2, w.H // 3), (w.B - 1, w.H - 1)]
    o_ref, ST_ref = oracle_scan(w, b, heads)
    sel = lambda x: np.stack([x[bb, hh] for bb, hh in heads])  # noqa: E731
    assert_parity(sel(o), sel(ST), o_ref, ST_ref, w.dtype, head_dims=1, what=name)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
