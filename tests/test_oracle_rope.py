"""Pins of the oracle's q/k RMSNorm and rotary embedding (oracle/qk_norm_rope.py)
against what the step-0 page ("第 0 步：一个能跑的最小推理引擎", its rmsnorm and
rope operators and the layer function) and the mathematics fix: RoPE is a
rotation of the (j, j + D/2) pairs (identity at position 0, norm-preserving,
additive in the position, inner products depending only on the position
difference); the frequencies form a geometric series starting at 1; RMSNorm is
scale invariant, gives unit RMS with unit weights, is linear in the weight,
and has a closed form on constant vectors; the norm comes before the rotation."""

import numpy as np
import pytest

import oracle
from oracle import qk_norm_rope, rmsnorm, rope, rope_angles, rope_inv_freq

THETA = 1_000_000.0
D = 128


def _x(seed, n=3, heads=2, d=D):
    return np.random.default_rng(seed).standard_normal((n, heads, d))


def test_position_zero_is_identity():
    x = _x(1)
    assert np.array_equal(rope(x, np.zeros(3, np.int32), THETA), x)


def test_halves_are_paired():
    """A unit vector at dimension j < D/2 turns into dimensions j and j + D/2
    only (not j + 1, the adjacent-pair convention), and one at j + D/2 turns
    back into j; dimension 0 turns by exactly the position (frequency 1)."""
    for j in (0, 1, 17, 63):
        for src in (j, j + D // 2):
            e = np.zeros((1, 1, D))
            e[0, 0, src] = 1.0
            y = rope(e, np.array([5]), THETA)[0, 0]
            nz = set(np.nonzero(np.abs(y) > 1e-15)[0].tolist())
            assert nz <= {j, j + D // 2}, (j, src, nz)
    e = np.zeros((1, 1, D))
    e[0, 0, 0] = 1.0
    for p in (1, 3, 1000):
        y = rope(e, np.array([p]), THETA)[0, 0]
        ang = np.arctan2(y[D // 2], y[0])
        want = np.float64(np.float32(p)) % (2 * np.pi)
        want = want - 2 * np.pi if want > np.pi else want
        assert abs(ang - want) < 1e-12


def test_frequencies_geometric_from_one():
    for d, th in ((128, 1e6), (128, 1e4), (4, 1e4)):
        f = rope_inv_freq(d, th).astype(np.float64)
        assert f[0] == 1.0
        ratios = f[1:] / f[:-1]
        assert np.allclose(ratios, ratios[0], rtol=2e-7, atol=0)   # fp32 rounding of each term
        assert 0 < ratios[0] < 1
        # theta^(-2/D) per step, so the D/2 - 1 steps span theta^(-(D-2)/D)
        assert abs(np.log(f[-1]) / np.log(th) + (d - 2) / d) < 1e-6


def test_angles_are_fp32_products():
    pos = np.array([0, 1, 7, 4096, 32767], np.int32)
    ang = rope_angles(pos, D, THETA)
    assert ang.dtype == np.float32
    assert np.array_equal(ang[1], rope_inv_freq(D, THETA))
    assert np.array_equal(ang[3], np.float32(4096) * rope_inv_freq(D, THETA))  # power of two: exact


def test_rotation_preserves_pair_norms():
    x = _x(2, n=4)
    pos = np.array([3, 100, 4095, 32000])
    y = rope(x, pos, THETA)
    nx = x[..., : D // 2] ** 2 + x[..., D // 2:] ** 2
    ny = y[..., : D // 2] ** 2 + y[..., D // 2:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("m,n,d", [(3, 9, 5), (0, 40, 17), (63, 2, 31)])
def test_inner_product_depends_on_position_difference(m, n, d):
    """<rope(q, m), rope(k, n)> = <rope(q, m + d), rope(k, n + d)> up to the
    fp32 rounding of the angles (|error| <= |angle| * 2^-24 rad each)."""
    q, k = _x(3, n=1, heads=1), _x(4, n=1, heads=1)
    a = np.sum(rope(q, [m], THETA) * rope(k, [n], THETA))
    b = np.sum(rope(q, [m + d], THETA) * rope(k, [n + d], THETA))
    scale = np.linalg.norm(q) * np.linalg.norm(k)
    assert abs(a - b) <= 1e-5 * scale


def test_rotations_compose():
    x = _x(5, n=1)
    a, b = 21, 34
    two = rope(rope(x, [a], THETA), [b], THETA)
    one = rope(x, [a + b], THETA)
    assert np.allclose(two, one, rtol=0, atol=1e-5 * np.abs(x).max())


def test_rmsnorm_unit_rms_scale_invariance_and_weight():
    x = _x(6, n=5)
    ones = np.ones(D)
    y = rmsnorm(x, ones, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(rmsnorm(37.5 * x, ones, 0.0), y, rtol=1e-13)
    w = np.random.default_rng(7).uniform(0.5, 1.5, D)
    assert np.allclose(rmsnorm(x, w, 1e-6), w * rmsnorm(x, ones, 1e-6), rtol=1e-15)


def test_rmsnorm_constant_vector_and_zero():
    """x = c in every dimension: mean(x^2) = c^2, so the output is c / sqrt(c^2 + eps);
    the zero vector stays zero (no NaN) for eps > 0."""
    for c, eps in ((2.0, 1e-6), (-0.5, 1e-2), (1e-3, 1e-6)):
        y = rmsnorm(np.full((1, 1, D), c), np.ones(D), eps)
        assert np.allclose(y, c / np.sqrt(c * c + eps), rtol=1e-14)
    assert np.array_equal(rmsnorm(np.zeros((1, D)), np.ones(D), 1e-6), np.zeros((1, D)))


def test_norm_comes_before_rotation():
    """With a non-uniform weight, norm-then-rotate (the page's order) differs
    from rotate-then-norm; the oracle is the former."""
    q, k = _x(8, n=2, heads=16), _x(9, n=2, heads=8)
    wq = np.random.default_rng(10).uniform(0.2, 2.0, D)
    wk = np.random.default_rng(11).uniform(0.2, 2.0, D)
    pos = np.array([11, 2000])
    qo, ko = qk_norm_rope(q, k, pos, wq, wk, 1e-6, THETA)
    assert np.array_equal(qo, rope(rmsnorm(q, wq, 1e-6), pos, THETA))
    assert np.array_equal(ko, rope(rmsnorm(k, wk, 1e-6), pos, THETA))
    other = rmsnorm(rope(q, pos, THETA), wq, 1e-6)
    assert np.max(np.abs(other - qo)) > 1e-2
