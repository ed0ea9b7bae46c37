"""Pins for the oracle's adapter dropout: central differences of <Y, dY>
with the mask fixed, the no-drop and all-drop special cases against the
pinned plain layer, and the inverted-dropout expectation over many masks."""
import numpy as np
import pytest

from oracle import dropout as OD
from oracle import linear as OL


def tiny(seed, m=3, n=5, k=64, r=2, p=0.25):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((m, k))
    w = rng.standard_normal((n, k)) * 0.02
    a = rng.standard_normal((r, k)) / r
    b = rng.standard_normal((n, r)) * 0.1
    dy = rng.standard_normal((m, n))
    keep = rng.random((m, k)) >= p
    return x, w, a, b, dy, keep


def loss(x, w, a, b, dy, alpha, r, keep, p):
    y, _ = OD.linear_fwd_dropout(x, w, a, b, alpha, r, keep, p)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("p", [0.05, 0.25, 0.5])
def test_central_differences_with_fixed_mask(p):
    x, w, a, b, dy, keep = tiny(3, p=p)
    alpha, r = 4.0, 2
    dx, da, db = OD.linear_bwd_dropout(x, w, a, b, dy, alpha, r, keep, p)
    eps = 1e-6
    for name, t, g in (("x", x, dx), ("a", a, da), ("b", b, db)):
        rows, cols = t.shape
        idxs = [(0, 0), (min(1, rows - 1), min(3, cols - 1)), (rows - 1, cols - 1), (0, cols // 2)]
        if name == "x":  # a dropped and a kept input element
            idxs += [tuple(np.argwhere(~keep)[0]), tuple(np.argwhere(keep)[0])]
        for idx in idxs:
            tp, tm = t.copy(), t.copy()
            tp[idx] += eps
            tm[idx] -= eps
            lp = loss(*[tp if v is t else v for v in (x, w, a, b, dy)], alpha, r, keep, p)
            lm = loss(*[tm if v is t else v for v in (x, w, a, b, dy)], alpha, r, keep, p)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])
    # the frozen path is not dropped: a dropped element still gets dY W
    i, j = np.argwhere(~keep)[0]
    assert abs(dx[i, j] - (dy @ w)[i, j]) <= 1e-15


def test_keep_all_with_p0_is_the_plain_layer():
    x, w, a, b, dy, _ = tiny(5, m=4, n=8, k=128, r=4)
    keep = np.ones_like(x, dtype=bool)
    y, h = OD.linear_fwd_dropout(x, w, a, b, 8.0, 4, keep, 0.0)
    y0, h0 = OL.linear_fwd(x, w, a, b, 8.0, 4)
    assert np.array_equal(y, y0) and np.array_equal(h, h0)
    g = OD.linear_bwd_dropout(x, w, a, b, dy, 8.0, 4, keep, 0.0)
    g0 = OL.linear_bwd(x, w, a, b, dy, 8.0, 4)
    for u, v in zip(g, g0):
        assert np.allclose(u, v, rtol=1e-14, atol=1e-15)


def test_drop_all_leaves_the_frozen_path():
    x, w, a, b, dy, _ = tiny(6, m=4, n=8, k=128, r=4)
    keep = np.zeros_like(x, dtype=bool)
    y, h = OD.linear_fwd_dropout(x, w, a, b, 8.0, 4, keep, 0.1)
    assert np.array_equal(y, x @ w.T) and not np.any(h)
    dx, da, db = OD.linear_bwd_dropout(x, w, a, b, dy, 8.0, 4, keep, 0.1)
    assert np.array_equal(dx, dy @ w) and not np.any(da) and not np.any(db)


def test_inverted_dropout_expectation():
    """Averaged over many masks, H equals the undropped H (the 1/(1 - p)
    scaling), within a few standard errors."""
    rng = np.random.Generator(np.random.PCG64(9))
    x, w, a, b, _, _ = tiny(7, m=2, n=4, k=256, r=2)
    p, trials = 0.1, 4000
    acc = np.zeros((2, 2))
    acc2 = np.zeros((2, 2))
    for _ in range(trials):
        keep = rng.random(x.shape) >= p
        _, h = OD.linear_fwd_dropout(x, w, a, b, 4.0, 2, keep, p)
        acc += h
        acc2 += h * h
    mean = acc / trials
    se = np.sqrt(np.maximum(acc2 / trials - mean ** 2, 0) / trials)
    _, h0 = OL.linear_fwd(x, w, a, b, 4.0, 2)
    assert np.all(np.abs(mean - h0) <= 5 * se + 1e-12)
