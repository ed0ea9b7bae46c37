"""Pins for the oracle's linear layer: finite differences, adjoint identities,
the B = 0 init, the merged-weight identity, a literal triple loop, and the
parameter counts and scale the pages print."""
import os

import numpy as np
import pytest

from oracle import linear as OL
from oracle import nf4 as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()[:2]
            vals[k] = v
    return vals


def tiny(seed=0, m=3, n=5, k=64, r=2):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((m, k))
    w = rng.standard_normal((n, k)) * 0.02
    a = rng.standard_normal((r, k)) / r
    b = rng.standard_normal((n, r)) * 0.01
    dy = rng.standard_normal((m, n))
    return x, w, a, b, dy


def loss(x, w, a, b, dy, alpha, r):
    y, _ = OL.linear_fwd(x, w, a, b, alpha, r)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("alpha,r", [(4.0, 2), (1.0, 2), (16.0, 8)])
def test_backward_central_differences(alpha, r):
    """L = <Y, dY> is linear in each of X, A, B separately, so a central
    difference equals the gradient up to rounding."""
    x, w, a, b, dy = tiny(r=r)
    dx, da, db = OL.linear_bwd(x, w, a, b, dy, alpha, r)
    h = 1e-3
    for name, arr, grad in (("x", x, dx), ("a", a, da), ("b", b, db)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, q = arr.copy(), arr.copy()
            p[idx] += h
            q[idx] -= h
            args = {"x": x, "a": a, "b": b}
            args[name] = p
            lp = loss(args["x"], w, args["a"], args["b"], dy, alpha, r)
            args[name] = q
            lm = loss(args["x"], w, args["a"], args["b"], dy, alpha, r)
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(num, grad, rtol=1e-7, atol=1e-10), name


def test_backward_adjoint_identity():
    """<dY, J v> = <J^T dY, v> for a random direction v in (X, A, B)."""
    x, w, a, b, dy = tiny(seed=3, m=4, n=6, k=128, r=4)
    alpha, r = 8.0, 4
    rng = np.random.Generator(np.random.PCG64(99))
    vx, va, vb = rng.standard_normal(x.shape), rng.standard_normal(a.shape), rng.standard_normal(b.shape)
    s = OL.lora_scale(alpha, r)
    # J v: directional derivative of Y, written from the product rule
    jv = vx @ w.T + s * ((vx @ a.T + x @ va.T) @ b.T + (x @ a.T) @ vb.T)
    dx, da, db = OL.linear_bwd(x, w, a, b, dy, alpha, r)
    lhs = np.sum(dy * jv)
    rhs = np.sum(dx * vx) + np.sum(da * va) + np.sum(db * vb)
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_b_zero_init_gives_base_output_and_zero_da():
    """B = 0 at init means the adapter adds nothing and dA vanishes."""
    x, w, a, b, dy = tiny(seed=5, m=4, n=8, k=128, r=4)
    b = np.zeros_like(b)
    y, _ = OL.linear_fwd(x, w, a, b, 8.0, 4)
    assert np.array_equal(y, x @ w.T)
    dx, da, db = OL.linear_bwd(x, w, a, b, dy, 8.0, 4)
    assert np.array_equal(da, np.zeros_like(da))
    assert np.array_equal(dx, dy @ w)
    assert np.any(db != 0)


def test_merged_weight_equivalence():
    """X (W + s B A)^T equals the two-path forward."""
    x, w, a, b, dy = tiny(seed=6, m=8, n=16, k=256, r=8)
    y, _ = OL.linear_fwd(x, w, a, b, 16.0, 8)
    ym = x @ OL.merged_weight(w, a, b, 16.0, 8).T
    assert np.max(np.abs(y - ym)) <= 1e-12 * np.max(np.abs(y))


def test_blas_equals_triple_loop_small():
    """The library matmul the oracle leans on agrees with a literal loop on a
    slice of the 256 x 256 single-layer case."""
    rng = np.random.Generator(np.random.PCG64(12))
    m, n, k, r = 3, 7, 256, 8
    x = rng.standard_normal((m, k))
    w = rng.standard_normal((n, k)) * 0.02
    a = rng.standard_normal((r, k)) / r
    b = rng.standard_normal((n, r)) * 0.01
    s = OL.lora_scale(16.0, r)
    y, h = OL.linear_fwd(x, w, a, b, 16.0, r)
    for i in range(m):
        hh = [sum(x[i, t] * a[j, t] for t in range(k)) for j in range(r)]
        for o in range(n):
            base = sum(x[i, t] * w[o, t] for t in range(k))
            lo = sum(hh[j] * b[o, j] for j in range(r))
            assert abs(y[i, o] - (base + s * lo)) <= 1e-12 * (1 + abs(y[i, o]))


def test_scale_values():
    assert OL.lora_scale(16.0, 8) == 2.0
    assert OL.lora_scale(32.0, 16) == 2.0
    assert OL.lora_scale(16.0, 64) == 0.25
    assert OL.lora_scale(64.0, 32) == OL.lora_scale(32.0, 16)  # only the ratio matters


def test_lora_parameter_counts():
    g = golden("storage_figures.txt")
    assert 16 * (4096 + 4096) == int(g["LORA_PARAMS_4096_R16"])
    assert 4096 * 4096 == int(g["FULL_PARAMS_4096"])
    assert round(100 * (1 - 131072 / 16777216), 1) == float(g["REDUCTION_PERCENT"])
    for r, key in ((8, "LORA_PARAMS_4096_R8"), (32, "LORA_PARAMS_4096_R32"), (64, "LORA_PARAMS_4096_R64")):
        assert r * (4096 + 4096) == int(g[key])


def test_rank_zero_is_base_only():
    x, w, a, b, dy = tiny()
    y, h = OL.linear_fwd(x, w, None, None, 0.0, 0)
    assert np.array_equal(y, x @ w.T) and h.shape == (3, 0)


def test_rel_err_semantics():
    assert OL.rel_err(np.zeros(3), np.zeros(3)) == 0.0
    assert OL.rel_err(np.ones(3) * 1e-30, np.zeros(3)) == float("inf")
    assert OL.rel_err([1.0, 2.01], [1.0, 2.0]) == pytest.approx(0.005)


def test_forward_through_quantizer_small_case():
    """End to end on the 256 x 256 case: quantize, dequantize to bf16, forward.
    The bf16 dequantized weight stays within the NF4 step of the original."""
    import synth
    wl = synth.SMALL
    lay = wl.layers[0]
    w = synth.weight(wl, lay)
    q = O.quantize(w.reshape(-1), True)
    w32, bits = O.dequantize(q)
    w16 = O.bf16_bits_to_f32(bits).reshape(lay.n, lay.k)
    step = np.repeat(q["scales"], 64).reshape(lay.n, lay.k) * 0.33  # widest half-gap ~0.3
    assert np.all(np.abs(w16 - w) <= step * 1.02 + np.abs(w) * 2 ** -8)
