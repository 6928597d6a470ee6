"""Pins of the comparison every parity gate uses.

``oracle.rel_err_per_head`` is the per-head relative Frobenius error
||x - ref||_F / ||ref||_F (the absolute norm where the reference is zero) that
the parity gates take the maximum of; ``_parity.block_err`` is the companion
check on 64-token blocks of o.  Both are checked here against values worked out
by hand, and two plausible mistakes in the metric (norms over the wrong axes,
the candidate's norm as the divisor) are shown to fail these pins.
"""
import numpy as np
import pytest

import oracle
from _parity import block_err


def _pins(fn):
    """Raise AssertionError unless ``fn`` behaves as the per-head relative
    Frobenius error with ``head_dims`` leading head axes."""
    # one head: ref = (3, 4) (norm 5), x = (3, 4) + (0, 1) -> 1/5
    r = fn(np.array([[3.0, 4.0]]), np.array([[3.0, 4.0]]), 1)
    assert np.allclose(r, [0.0])
    r = fn(np.array([[3.0, 5.0]]), np.array([[3.0, 4.0]]), 1)
    assert np.allclose(r, [0.2]), r
    # the divisor is the reference's norm, not the candidate's: x = 2 ref -> 1
    r = fn(np.array([[6.0, 8.0]]), np.array([[3.0, 4.0]]), 1)
    assert np.allclose(r, [1.0]), r
    # a zero reference reports the absolute norm: ||(1, 2, 2)|| = 3
    r = fn(np.array([[1.0, 2.0, 2.0]]), np.zeros((1, 3)), 1)
    assert np.allclose(r, [3.0]), r
    # head_dims = 2 on a 3-D array: heads (0,0), (0,1), (1,0), (1,1), norms over the last axis
    ref = np.array([[[1.0, 0.0], [0.0, 2.0]], [[0.0, 0.0], [3.0, 4.0]]])
    x = ref + np.array([[[0.5, 0.0], [0.0, 0.0]], [[0.0, 1.0], [0.0, 0.0]]])
    r = fn(x, ref, 2)
    assert r.shape == (2, 2), r.shape
    assert np.allclose(r, [[0.5, 0.0], [1.0, 0.0]]), r
    # head_dims = 1 on the same arrays: two heads, norms over both trailing axes
    r = fn(x, ref, 1)
    assert r.shape == (2,), r.shape
    assert np.allclose(r, [0.5 / np.sqrt(5.0), 1.0 / 5.0]), r
    # an error planted in one row of one head shows in that head only
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((3, 4, 16, 8))
    x = ref.copy()
    x[1, 2, 5] += 1.0  # one row of head (1, 2)
    r = fn(x, ref, 2)
    expect = np.zeros((3, 4))
    expect[1, 2] = np.sqrt(8.0) / np.linalg.norm(ref[1, 2])
    assert np.allclose(r, expect), r


def test_rel_err_per_head_pins():
    _pins(oracle.rel_err_per_head)


def _wrong_axes(x, ref, head_dims):
    """A plausible slip: the norms run over the head axes instead."""
    x, ref = np.asarray(x, float), np.asarray(ref, float)
    axes = tuple(range(ref.ndim - head_dims, ref.ndim))
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def _wrong_divisor(x, ref, head_dims):
    """A plausible slip: the candidate's norm as the divisor."""
    x, ref = np.asarray(x, float), np.asarray(ref, float)
    axes = tuple(range(head_dims, ref.ndim))
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(x ** 2, axis=axes))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


@pytest.mark.parametrize("mutant", [_wrong_axes, _wrong_divisor])
def test_planted_metric_mistakes_fail_the_pins(mutant):
    with pytest.raises(AssertionError):
        _pins(mutant)


def test_block_err_pins():
    """block_err: per 64-token block of o, ||x_b - ref_b|| over the head's RMS
    norm of a 64-token block, ||ref||_F sqrt(64 / T)."""
    T, dv = 256, 4
    ref = np.ones((1, T, dv))  # ||ref|| = sqrt(1024) = 32; RMS block norm = 32 * sqrt(64/256) = 16
    x = ref.copy()
    x[0, 130, :] += 2.0  # one token of block 2: ||delta|| = 4
    assert np.isclose(block_err(x, ref, 1), 4.0 / 16.0)
    # a uniform relative error e gives e in every block (equal to the head-wide error)
    assert np.isclose(block_err(ref * 1.01, ref, 1), 0.01)
    # a ragged tail block counts with its own tokens: T = 100, error in token 99
    ref = np.ones((2, 100, 4))
    x = ref.copy()
    x[1, 99, 0] += 1.0
    den = np.sqrt(400.0) * np.sqrt(64 / 100)
    assert np.isclose(block_err(x, ref, 1), 1.0 / den)
    # a zero reference head reports the absolute block norm
    assert np.isclose(block_err(np.full((1, 64, 1), 0.5), np.zeros((1, 64, 1)), 1), 4.0)
    # head axes: the maximum runs over all heads
    ref = np.ones((2, 3, 64, 2))
    x = ref.copy()
    x[1, 2, 10, 1] += 3.0
    assert np.isclose(block_err(x, ref, 2), 3.0 / np.sqrt(128.0))


def test_block_err_sees_a_local_mistake_the_head_norm_misses():
    """One wrong token in 8192 barely moves the head-wide error but fails the
    block check at its gate (4 x the head-wide gate)."""
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((1, 8192, 128))
    x = ref.copy()
    x[0, 4000] *= 0.7  # one token 30 % off
    head = float(np.max(oracle.rel_err_per_head(x, ref, 1)))
    assert head < 5e-3
    assert block_err(x, ref, 1) > 4 * 5e-3
