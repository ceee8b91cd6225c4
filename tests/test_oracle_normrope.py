"""Pins of the RMSNorm and RoPE oracle (oracle/normrope.py) against closed
forms, hand-worked values, invariants and finite differences -- nothing here
re-types the oracle's formulas."""
import math

import numpy as np
import pytest

from oracle import normrope as nr


# ---------------------------------------------------------------------------
# RMSNorm

def test_rmsnorm_hand_worked_row():
    # x = (3, 4): mean of squares 12.5, rms 5/sqrt(2); y = (3 sqrt2 / 5, 4 sqrt2 / 5)
    y, rstd = nr.rmsnorm_fwd(np.array([[3.0, 4.0]]), np.array([1.0, 1.0]), 0.0)
    assert rstd[0] == pytest.approx(math.sqrt(2.0) / 5.0, rel=1e-15)
    assert y[0, 0] == pytest.approx(3.0 * math.sqrt(2.0) / 5.0, rel=1e-15)
    assert y[0, 1] == pytest.approx(4.0 * math.sqrt(2.0) / 5.0, rel=1e-15)
    # the weight multiplies element-wise after the normalization
    y2, _ = nr.rmsnorm_fwd(np.array([[3.0, 4.0]]), np.array([2.0, -0.5]), 0.0)
    assert y2[0] == pytest.approx([6.0 * math.sqrt(2.0) / 5.0, -2.0 * math.sqrt(2.0) / 5.0], rel=1e-15)


def test_rmsnorm_eps_enters_under_the_root():
    # x = (1, 1, 1, 1), eps = 3: rstd = 1/sqrt(1 + 3) = 1/2
    _, rstd = nr.rmsnorm_fwd(np.ones((1, 4)), np.ones(4), 3.0)
    assert rstd[0] == pytest.approx(0.5, rel=1e-15)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 96))
    w = np.ones(96)
    y, _ = nr.rmsnorm_fwd(x, w, 0.0)
    # unit root-mean-square rows, and scale invariance without eps
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    y3, _ = nr.rmsnorm_fwd(7.5 * x, w, 0.0)
    assert np.allclose(y3, y, rtol=1e-13, atol=0)


def test_rmsnorm_zero_row():
    eps = 1e-5
    dy = np.arange(8, dtype=np.float64)[None, :] - 3.0
    w = np.linspace(0.5, 2.0, 8)
    y, rstd = nr.rmsnorm_fwd(np.zeros((1, 8)), w, eps)
    assert rstd[0] == pytest.approx(1.0 / math.sqrt(eps), rel=1e-15) and not y.any()
    # with x = 0 the normalized row is 0, so dx = rstd * w * dy
    dx = nr.rmsnorm_bwd(dy, np.zeros((1, 8)), w, eps)
    assert np.allclose(dx, w * dy / math.sqrt(eps), rtol=1e-14)


def test_rmsnorm_backward_matches_finite_differences():
    rng = np.random.default_rng(2)
    M, H, eps = 3, 24, 1e-3
    x = rng.standard_normal((M, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.standard_normal((M, H))
    dx = nr.rmsnorm_bwd(dy, x, w, eps)
    h = 1e-6
    num = np.zeros_like(x)
    for m in range(M):
        for k in range(H):
            xp, xm = x.copy(), x.copy()
            xp[m, k] += h
            xm[m, k] -= h
            num[m, k] = (np.sum(dy * nr.rmsnorm_fwd(xp, w, eps)[0]) - np.sum(dy * nr.rmsnorm_fwd(xm, w, eps)[0])) / (2 * h)
    assert np.allclose(dx, num, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------------------
# RoPE

def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((4, 3 * 16))
    assert np.array_equal(nr.rope(v, np.zeros(4, np.int64), 16, 10000.0), v)


def test_rope_hand_worked_pairs():
    # d = 4: pairs are (0, 2) and (1, 3); theta = (1, base^-1/2) = (1, 0.01) for base 1e4
    p = np.array([1])
    y = nr.rope(np.array([[1.0, 0.0, 0.0, 0.0]]), p, 4, 10000.0)
    assert y[0] == pytest.approx([math.cos(1.0), 0.0, math.sin(1.0), 0.0], abs=1e-15)
    y = nr.rope(np.array([[0.0, 1.0, 0.0, 0.0]]), p, 4, 10000.0)
    assert y[0] == pytest.approx([0.0, math.cos(0.01), 0.0, math.sin(0.01)], abs=1e-15)
    # the second half rotates the other way into the first: (0, 0, 1, 0) -> (-sin, 0, cos, 0)
    y = nr.rope(np.array([[0.0, 0.0, 1.0, 0.0]]), np.array([3]), 4, 10000.0)
    assert y[0] == pytest.approx([-math.sin(3.0), 0.0, math.cos(3.0), 0.0], abs=1e-15)
    # d = 2 at p = pi/2 turns (1, 0) into (0, 1)
    y = nr.rope(np.array([[1.0, 0.0]]), np.array([math.pi / 2]), 2, 500000.0)
    assert y[0] == pytest.approx([0.0, 1.0], abs=1e-15)


def test_rope_rotation_properties():
    rng = np.random.default_rng(4)
    d, base, M = 128, 500000.0, 6
    q = rng.standard_normal((M, 4 * d))
    k = rng.standard_normal((M, 2 * d))
    p1 = rng.integers(0, 20000, M)
    p2 = rng.integers(0, 20000, M)
    # pair norms are kept
    rq = nr.rope(q, p1, d, base).reshape(M, 4, d)
    qq = q.reshape(M, 4, d)
    assert np.allclose(rq[..., :64] ** 2 + rq[..., 64:] ** 2, qq[..., :64] ** 2 + qq[..., 64:] ** 2, rtol=1e-12)
    # composition adds positions
    assert np.allclose(nr.rope(nr.rope(q, p1, d, base), p2, d, base), nr.rope(q, p1 + p2, d, base), atol=1e-9)
    # scores depend on the position difference only
    q0, k0 = q[:, :d], k[:, :d]

    def score(a, b):
        return np.sum(nr.rope(q0, a, d, base) * nr.rope(k0, b, d, base), axis=1)
    assert np.allclose(score(p1, p2), score(p1 + 777, p2 + 777), atol=1e-9)


def test_rope_backward_is_the_adjoint_and_the_inverse():
    rng = np.random.default_rng(5)
    d, base, M = 64, 10000.0, 5
    x = rng.standard_normal((M, 3 * d))
    g = rng.standard_normal((M, 3 * d))
    p = rng.integers(0, 4096, M)
    assert np.sum(nr.rope(x, p, d, base) * g) == pytest.approx(np.sum(x * nr.rope_bwd(g, p, d, base)), rel=1e-12)
    assert np.allclose(nr.rope_bwd(nr.rope(x, p, d, base), p, d, base), x, atol=1e-12)
