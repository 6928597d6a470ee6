"""Seeded synthetic input generators: determinism, independence, casts."""
import numpy as np
import torch

from scan_sequence_models_amd import inputs as I


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(I.bf16_round(x), back)


def test_head_inputs_deterministic_and_independent():
    w = I.WORKLOADS["gdn-b8h16t8192"].replace(T=256)
    a = I.head_inputs(w, 1, 2)
    b = I.head_inputs(w, 1, 2)
    c = I.head_inputs(w, 2, 1)
    for x, y in zip((a.q, a.k, a.v, a.alpha, a.beta, a.S0), (b.q, b.k, b.v, b.alpha, b.beta, b.S0)):
        assert x.tobytes() == y.tobytes()
    assert not np.array_equal(a.q, c.q)


def test_head_inputs_distributions():
    w = I.WORKLOADS["gdn-b8h16t8192"].replace(T=4096)
    x = I.head_inputs(w, 0, 0)
    # bf16-exact values, unit-norm keys and queries up to bf16 rounding
    assert np.array_equal(I.bf16_round(x.q), x.q)
    assert np.allclose(np.linalg.norm(x.k.astype(np.float64), axis=1), 1.0, atol=1e-2)
    assert 0.0 < x.alpha.min() and x.alpha.max() < 1.0 and 0.9 < x.alpha.mean() < 0.96
    assert 0.45 < x.beta.mean() < 0.55
    assert abs(x.S0.std() - 0.1) < 0.01  # N(0, 0.01) is variance 0.01
    g = I.head_inputs(I.WORKLOADS["gla-b4h8t4096"], 0, 0)
    assert g.beta is None and g.S0 is None
    la = np.log(g.alpha.astype(np.float64))
    assert la.min() >= -0.0500001 and la.max() <= 0.0


def test_batch_matches_heads():
    w = I.WORKLOADS["gdn-b8h16t8192"].replace(B=2, H=3, T=64)
    b = I.batch_inputs(w, threads=3)
    for bi in range(2):
        for h in range(3):
            x = I.head_inputs(w, bi, h)
            assert np.array_equal(b.q[bi, h], x.q) and np.array_equal(b.S0[bi, h], x.S0)


def test_decode_inputs_deterministic():
    w = I.WORKLOADS["decode-4096x100"]
    a = I.decode_inputs(w, N=8, steps=5, threads=2)
    b = I.decode_inputs(w, N=8, steps=5, threads=4)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()
    assert a[1].shape == (5, 8, 128) and a[0].shape == (8, 128, 128)
