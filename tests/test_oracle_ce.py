"""Pins of the cross-entropy oracle (oracle/ce.py): closed forms, ignored rows,
shift invariance, stability and finite differences."""
import math

import numpy as np
import pytest

from oracle import ce


def test_zero_head_gives_log_v():
    rng = np.random.default_rng(1)
    M, H, V = 5, 8, 37
    h = rng.standard_normal((M, H))
    t = rng.integers(0, V, M)
    loss, rows, dh = ce.ce_fwd_bwd(h, np.zeros((V, H)), t)
    assert loss == pytest.approx(math.log(V), rel=1e-15)
    assert np.allclose(rows, math.log(V), rtol=1e-15) and not dh.any()


def test_two_classes_softplus():
    # V = 2, H = 1, W = (1, 0): logits (x, 0); target 0 -> log(1 + e^-x), target 1 -> log(1 + e^x)
    h = np.array([[0.7], [-2.0], [3.0]])
    W = np.array([[1.0], [0.0]])
    loss, rows, dh = ce.ce_fwd_bwd(h, W, np.array([0, 1, 1]))
    want = [math.log1p(math.exp(-0.7)), math.log1p(math.exp(-2.0)), math.log1p(math.exp(3.0))]
    assert rows == pytest.approx(want, rel=1e-14)
    assert loss == pytest.approx(sum(want) / 3, rel=1e-14)
    # d/dx log(1 + e^-x) = -1/(1 + e^x), divided by n = 3
    assert dh[0, 0] == pytest.approx(-1.0 / (1.0 + math.exp(0.7)) / 3, rel=1e-14)


def test_ignored_rows():
    rng = np.random.default_rng(2)
    M, H, V = 6, 4, 11
    h, W = rng.standard_normal((M, H)), rng.standard_normal((V, H))
    t = rng.integers(0, V, M)
    t2 = t.copy()
    t2[[1, 4]] = -100
    loss_all, rows_all, dh_all = ce.ce_fwd_bwd(h, W, t)
    loss, rows, dh = ce.ce_fwd_bwd(h, W, t2)
    keep = t2 >= 0
    assert rows[1] == 0 and rows[4] == 0 and not dh[[1, 4]].any()
    assert np.allclose(rows[keep], rows_all[keep], rtol=1e-14)
    assert loss == pytest.approx(rows_all[keep].sum() / 4, rel=1e-14)
    assert np.allclose(dh[keep], dh_all[keep] * 6 / 4, rtol=1e-12)
    assert ce.ce_fwd_bwd(h, W, np.full(M, -100))[0] == 0.0


def test_shift_invariance_and_stability():
    rng = np.random.default_rng(3)
    M, H, V = 4, 6, 23
    h, W = rng.standard_normal((M, H)), rng.standard_normal((V, H))
    t = rng.integers(0, V, M)
    loss, rows, dh = ce.ce_fwd_bwd(h, W, t)
    # adding one vector u to every head row shifts all logits of a row by h.u: nothing changes
    u = rng.standard_normal(H)
    loss2, rows2, dh2 = ce.ce_fwd_bwd(h, W + u[None, :], t)
    assert loss2 == pytest.approx(loss, rel=1e-12) and np.allclose(dh2, dh, atol=1e-12)
    # logits of a thousand do not overflow
    loss3, _, dh3 = ce.ce_fwd_bwd(300.0 * h, W, t)
    assert np.isfinite(loss3) and np.isfinite(dh3).all()


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(4)
    M, H, V = 3, 5, 9
    h, W = rng.standard_normal((M, H)), rng.standard_normal((V, H))
    t = np.array([2, -100, 7])
    _, _, dh = ce.ce_fwd_bwd(h, W, t)
    eps = 1e-6
    num = np.zeros_like(h)
    for m in range(M):
        for k in range(H):
            hp, hm = h.copy(), h.copy()
            hp[m, k] += eps
            hm[m, k] -= eps
            num[m, k] = (ce.ce_fwd_bwd(hp, W, t)[0] - ce.ce_fwd_bwd(hm, W, t)[0]) / (2 * eps)
    assert np.allclose(dh, num, rtol=1e-6, atol=1e-9)
