"""Pins for the oracle's merge / unmerge / re-quantize: exact rational
arithmetic in the stated order, the float64 definition within the float32
summation bound, the B = 0 and r = 0 cases, the merged forward against the
two-path forward, and the unmerge round trip."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import linear as OL
from oracle import merge as OM
from oracle import nf4 as O
from test_oracle_nf4 import round_fp32

U = 2.0 ** -24  # unit roundoff of float32


def bf16_values(shape, std, seed):
    """Random values that are exactly representable in bf16 (as float32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    return O.bf16_bits_to_f32(O.bf16_rne_bits(v)).reshape(shape)


def inputs(n, k, r, seed):
    w16 = bf16_values((n, k), 0.02, seed)
    a = bf16_values((r, k), 1.0 / max(r, 1), seed + 1)
    b = bf16_values((n, r), 0.01, seed + 2)
    return w16, a, b


@pytest.mark.parametrize("r,alpha", [(1, 2.0), (3, 6.0), (4, 1.0)])
def test_merge_equals_exact_rationals_in_stated_order(r, alpha):
    """Every step redone in exact rationals with one float32 rounding where
    the stated order rounds: d_j = fl32(d_{j-1} + b_pj a_jq), t = fl32(s d),
    m = fl32(w16 + t)."""
    n, k = 3, 5
    w16, a, b = inputs(n, k, r, 40 + r)
    m, bits = OM.merge(w16, a, b, alpha, r)
    s = round_fp32(Fraction(float(np.float32(alpha))) / Fraction(r))
    for p in range(n):
        for q in range(k):
            d = Fraction(0)
            for j in range(r):
                d = round_fp32(d + round_fp32(Fraction(float(b[p, j])) * Fraction(float(a[j, q]))))
            t = round_fp32(s * d)
            want = round_fp32(Fraction(float(w16[p, q])) + t)
            assert Fraction(float(m[p, q])) == want, (p, q)
            u = round_fp32(Fraction(float(m[p, q])) - t)
            assert Fraction(float(OM.unmerge(m, a, b, alpha, r)[0][p, q])) == u
    assert np.array_equal(bits, O.bf16_rne_bits(m))


@pytest.mark.parametrize("r,alpha", [(16, 32.0), (64, 16.0), (5, 10.0)])
def test_merge_within_summation_bound_of_float64_definition(r, alpha):
    """|m - (w16 + s B A)| is within the float32 error bound of recursive
    summation: u|exact| + s (r + 1) u sum_j |b_pj a_jq| (+ slack)."""
    n, k = 48, 320
    w16, a, b = inputs(n, k, r, 7 * r)
    m, _ = OM.merge(w16, a, b, alpha, r)
    s = OL.lora_scale(alpha, r)
    exact = OL.merged_weight(w16, a, b, alpha, r)
    mag = np.abs(b.astype(np.float64)) @ np.abs(a.astype(np.float64))
    bound = U * np.abs(exact) + s * (r + 1) * U * mag * 1.01 + 1e-30
    assert np.all(np.abs(m - exact) <= bound)
    # the update is visible: a dropped rank-1 term would exceed the bound
    drop = exact - s * np.outer(b[:, 0], a[0, :]).astype(np.float64)
    assert np.any(np.abs(m - drop) > bound)


def test_zero_adapter_and_rank_zero_return_the_base():
    w16, a, b = inputs(32, 128, 8, 3)
    m, bits = OM.merge(w16, a, np.zeros_like(b), 16.0, 8)
    assert np.array_equal(m.view(np.uint32), w16.view(np.uint32))
    assert np.array_equal(bits, O.bf16_rne_bits(w16))
    m0, _ = OM.merge(w16, a[:0], b[:, :0], 0.0, 0)
    assert np.array_equal(m0, w16)


def test_merged_forward_equals_two_path_forward():
    """[L]: the merged layer computes what the adapted layer computes."""
    n, k, r, alpha = 64, 256, 16, 32.0
    w16, a, b = inputs(n, k, r, 11)
    x = bf16_values((8, k), 1.0, 12).astype(np.float64)
    y, _ = OL.linear_fwd(x, w16, a, b, alpha, r)
    m, _ = OM.merge(w16, a, b, alpha, r)
    ym = x @ m.astype(np.float64).T
    assert np.max(np.abs(ym - y)) <= 1e-6 * np.max(np.abs(y))


def test_unmerge_round_trip_within_two_roundings():
    n, k, r, alpha = 40, 192, 8, 16.0
    w16, a, b = inputs(n, k, r, 21)
    m, _ = OM.merge(w16, a, b, alpha, r)
    u, _ = OM.unmerge(m, a, b, alpha, r)
    assert np.all(np.abs(u - w16) <= 2 * U * (np.abs(m) + np.abs(w16)))
    # the adapter really comes out: unmerging the base moves it by -t
    v, _ = OM.unmerge(w16, a, b, alpha, r)
    t = OM.update32(a, b, alpha, r)
    assert np.all(np.abs(v - (w16 - t)) <= U * np.abs(w16 - t))


def test_requantize_is_quantize_of_the_merged_weight():
    n, k, r, alpha = 16, 512, 8, 16.0
    w16, a, b = inputs(n, k, r, 31)
    q = OM.requantize(w16, a, b, alpha, r, True)
    m, _ = OM.merge(w16, a, b, alpha, r)
    ref = O.quantize(m.reshape(-1), True)
    for key in ("codes", "scale_codes", "group_scale", "absmax"):
        assert np.array_equal(q[key], ref[key]), key
    # B = 0: the base quantized again
    q0 = OM.requantize(w16, a, np.zeros_like(b), alpha, r, False)
    assert np.array_equal(q0["codes"], O.quantize(w16.reshape(-1), False)["codes"])
    # the reconstruction stays within half the widest level gap of each block's absmax
    w32, _ = O.dequantize(q)
    amax = np.repeat(q["absmax"], O.BLOCK)
    gap = np.max(np.diff(O.nf4_levels()))
    assert np.all(np.abs(w32 - m.reshape(-1)) <= (gap / 2 + 0.01) * amax + 1e-12)
