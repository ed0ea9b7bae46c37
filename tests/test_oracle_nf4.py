"""Pins for the oracle's quantizer, each against something other than the
oracle itself: the values the pages print, two independent quantile
functions, exact rational arithmetic, torch's bf16 rounding, and invariants
(round trip, ties, zero blocks, error bounds)."""
import math
import os
import statistics
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

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


# --- exact-arithmetic helpers, written independently of the oracle ----------
def round_fp32(q: Fraction) -> Fraction:
    """Round a rational to the nearest IEEE binary32 value, ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n, rem = divmod(q, quantum)
    half = quantum / 2
    if rem > half or (rem == half and n % 2 == 1):
        n += 1
    return sign * n * quantum


def exact_nearest(x: Fraction, levels) -> int:
    """argmin_k fl32(|x - L_k|) with exact subtraction and one fp32 rounding,
    first index on ties."""
    best, best_d = None, None
    for k, lv in enumerate(levels):
        d = round_fp32(abs(x - Fraction(float(lv))))
        if best_d is None or d < best_d:
            best, best_d = k, d
    return best


# --- codebook ---------------------------------------------------------------
def test_levels_structure():
    L = O.nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L) > 0)
    assert L[0] == np.float32(-1.0) and L[15] == np.float32(1.0)
    assert L.view(np.uint32)[7] == 0  # +0.0 exactly
    assert (L < 0).sum() == 7 and (L > 0).sum() == 8


def test_levels_two_independent_inverse_cdfs():
    a = O.nf4_levels()  # Python's statistics (Wichura AS241)
    b = O.nf4_levels(scipy.special.ndtri)  # cephes ndtri
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_levels_are_normal_quantiles():
    """Each nonzero level times Phi^-1(offset) sits at the intended probability:
    8 evenly spaced in [0.5, o) above zero, 7 below; checked with the normal
    CDF (scipy ndtr), not the quantile function."""
    L = O.nf4_levels().astype(np.float64)
    o = O.NF4_QUANTILE_OFFSET
    top = statistics.NormalDist().inv_cdf(o)
    pos = np.sort(scipy.special.ndtr(L[8:] * top))[::-1]
    neg = np.sort(scipy.special.ndtr(-L[:7] * top))[::-1]
    assert np.allclose(pos, [o - i * (o - 0.5) / 8 for i in range(8)], atol=1e-6)
    assert np.allclose(neg, [o - j * (o - 0.5) / 7 for j in range(7)], atol=1e-6)


def test_offset_literal_matches_closed_form():
    """The printed offset is the mean of 1-1/30 and 1-1/32 to 7 digits; a table
    built from the closed form differs by at most 2 ulp per level."""
    closed = ((1 - 1 / 30) + (1 - 1 / 32)) / 2
    assert abs(closed - O.NF4_QUANTILE_OFFSET) < 1e-7
    inv = statistics.NormalDist().inv_cdf
    vals = [inv(p) for p in np.linspace(closed, 0.5, 9)[:-1]] + [0.0] + [-inv(p) for p in np.linspace(closed, 0.5, 8)[:-1]]
    vals.sort()
    alt = (np.array(vals) / vals[-1]).astype(np.float32)
    diff = np.abs(alt.view(np.int32).astype(np.int64) - O.nf4_levels().view(np.int32).astype(np.int64))
    assert diff.max() <= 2


def test_page_example_mse():
    """Reproduce the page's printed NF4 and INT4 reconstruction errors on the
    page's own data (torch CPU generator, seed 0)."""
    torch = pytest.importorskip("torch")
    g = golden("ultralytics_nf4_vs_int4_mse.txt")
    torch.manual_seed(0)
    w = (torch.randn(4096, 64) * 0.02).numpy().reshape(-1)
    res = {}
    for name, lv in (("NF4", O.nf4_levels()), ("INT4", O.int4_levels())):
        q = O.quantize(w, double_quant=False, levels=lv)
        w32, _ = O.dequantize(q, lv)
        mse = float(np.mean((w32.astype(np.float64) - w.astype(np.float64)) ** 2))
        res[name] = mse
        assert f"{mse:.3e}" == g[name]
    reduction = 100 * (1 - res["NF4"] / res["INT4"])
    assert abs(reduction - float(g["REDUCTION_PERCENT_APPROX"])) < 1.0


def test_mse_other_generator_nf4_below_int4():
    """With a different RNG the two errors stay within 2% of the page's and in
    the same order."""
    rng = np.random.Generator(np.random.PCG64(1234))
    w = (rng.standard_normal(4096 * 64) * 0.02).astype(np.float32)
    out = {}
    for name, lv in (("NF4", O.nf4_levels()), ("INT4", O.int4_levels())):
        w32, _ = O.dequantize(O.quantize(w, False, lv), lv)
        out[name] = float(np.mean((w32.astype(np.float64) - w) ** 2))
    assert out["NF4"] < out["INT4"]
    assert abs(out["NF4"] / 3.395e-06 - 1) < 0.02 and abs(out["INT4"] / 4.053e-06 - 1) < 0.02


# --- encoder ----------------------------------------------------------------
def _near_midpoint_values(levels, rng, span=4):
    """Every float32 within +-span ulp of each decision midpoint, plus randoms."""
    xs = []
    for k in range(15):
        v = np.float32((np.float64(levels[k]) + np.float64(levels[k + 1])) / 2)
        for _ in range(span):
            v = np.nextafter(v, np.float32(-2))
        for _ in range(2 * span + 1):
            xs.append(v)
            v = np.nextafter(v, np.float32(2))
    xs += list(rng.uniform(-1, 1, 200).astype(np.float32))
    return np.array(xs, dtype=np.float32)


def test_encode_matches_exact_rational_argmin():
    """x = w / a (correctly rounded), then nearest level by fp32 distance with
    ties to the low index -- checked against exact rational arithmetic, on
    random values and values within a few ulp of every decision midpoint."""
    L = O.nf4_levels()
    rng = np.random.Generator(np.random.PCG64(7))
    targets = _near_midpoint_values(L, rng)
    a = np.float32(0.0371)  # block absmax
    # w chosen so that w / a lands near each target
    w = (targets.astype(np.float64) * np.float64(a)).astype(np.float32)
    w = np.clip(w, -a, a)
    block = np.concatenate([w, np.zeros((-w.size) % 64, np.float32)])
    # force every 64-run to have absmax exactly a
    block = block.reshape(-1, 64)
    block[:, 0] = a
    block = block.reshape(-1)
    q = O.quantize(block, double_quant=False)
    codes = O.unpack_nibbles(q["codes"], block.size)
    assert np.all(q["absmax"] == a)
    for i in range(block.size):
        x = round_fp32(Fraction(float(block[i])) / Fraction(float(a)))
        assert codes[i] == exact_nearest(x, L), i


def test_int4_levels_are_correctly_rounded_even_spacing():
    """The evenly spaced table of the NF4-vs-INT4 example: level k is
    -1 + 2k/15 rounded once to float32 (exact rationals), symmetric about 0,
    with exact endpoints and no zero level."""
    L = O.int4_levels()
    assert L.dtype == np.float32 and L.size == 16
    for k in range(16):
        assert Fraction(float(L[k])) == round_fp32(Fraction(-1) + Fraction(2 * k, 15)), k
        assert L[k] == -L[15 - k]
    assert L[0] == -1.0 and L[15] == 1.0 and not np.any(L == 0)


def test_int4_encode_matches_exact_rational_argmin():
    """The encoder with the evenly spaced table, against exact rationals, on
    values near every decision midpoint; x = 0 sits exactly between levels 7
    and 8 and takes the low one."""
    L = O.int4_levels()
    rng = np.random.Generator(np.random.PCG64(17))
    xs = np.concatenate([_near_midpoint_values(L, rng), np.zeros(1, np.float32)])
    codes = O.encode_nearest(xs, L)
    for i, x in enumerate(xs):
        assert codes[i] == exact_nearest(Fraction(float(x)), L), i
    assert codes[-1] == 7
    # an all-zero block: code 7 everywhere, and L_7 * 0 decodes to -0.0
    q = O.quantize(np.zeros(64, np.float32), True, L)
    assert np.all(O.unpack_nibbles(q["codes"], 64) == 7)
    w32, bits = O.dequantize(q, L)
    assert np.all(w32 == 0) and np.all(np.signbit(w32)) and np.all(bits == 0x8000)


def test_division_not_reciprocal_product():
    """Pick w where fl(w/a) and fl(w*fl(1/a)) differ and the difference moves
    the code; the oracle must follow the correctly rounded quotient."""
    L = O.nf4_levels()
    rng = np.random.Generator(np.random.PCG64(3))
    found = 0
    for _ in range(20000):
        a = np.float32(rng.uniform(0.01, 0.05))
        k = int(rng.integers(0, 15))
        mid = np.float32((np.float64(L[k]) + np.float64(L[k + 1])) / 2)
        w = np.float32(np.float64(mid) * np.float64(a))
        for _s in range(4):
            q_div = np.float32(w / a)
            q_rcp = np.float32(w * np.float32(np.float32(1) / a))
            if q_div != q_rcp:
                c_div = exact_nearest(Fraction(float(q_div)), L)
                c_rcp = exact_nearest(Fraction(float(q_rcp)), L)
                if c_div != c_rcp:
                    blk = np.zeros(64, np.float32)
                    blk[0], blk[1] = a, w
                    got = O.unpack_nibbles(O.quantize(blk, False)["codes"], 64)[1]
                    assert got == c_div
                    found += 1
            w = np.nextafter(w, np.float32(1))
        if found >= 3:
            break
    assert found >= 1


def test_exact_ties_resolve_low():
    """Exact fp32 distance ties exist near the midpoints; they take the lower code."""
    L = O.nf4_levels()
    ties = 0
    for k in range(15):
        mid = np.float32((np.float64(L[k]) + np.float64(L[k + 1])) / 2)
        v = mid
        for _ in range(4):
            v = np.nextafter(v, np.float32(-1))
        for _ in range(9):
            dlo, dhi = np.abs(v - L[k]), np.abs(v - L[k + 1])
            if dlo == dhi:
                ties += 1
                assert O.encode_nearest(np.array([v]), L)[0] == k
            v = np.nextafter(v, np.float32(1))
    assert ties >= 1


def test_roundtrip_of_level_values():
    """A block made of L_k * 2^e (one element at 2^e) encodes to k and dequantizes
    exactly -- with and without double quantization (that block's absmax is its
    group's max, so U_255 = 1 reproduces it)."""
    L = O.nf4_levels()
    for e in (-20, -7, 0, 3):
        codes = np.arange(64) % 16
        w = (L[codes].astype(np.float64) * 2.0 ** e).astype(np.float32)
        w[15] = np.float32(2.0 ** e)
        for dq in (False, True):
            q = O.quantize(w, dq)
            got = O.unpack_nibbles(q["codes"], 64)
            assert np.array_equal(got, codes)
            w32, _ = O.dequantize(q)
            assert np.array_equal(w32, w)


def test_zero_block_and_group():
    w = np.zeros(64 * 300, np.float32)
    w[64 * 256 + 5] = 0.25  # second group nonzero
    q = O.quantize(w, True)
    codes = O.unpack_nibbles(q["codes"], w.size)
    assert np.all(codes[:64 * 256] == O.ZERO_CODE)
    assert q["group_scale"][0] == 0 and np.all(q["scale_codes"][:256] == 0)
    w32, bits = O.dequantize(q)
    assert np.all(w32[:64 * 256] == 0)
    assert w32[64 * 256 + 5] == np.float32(0.25)


def test_absmax_element_is_extreme_code():
    rng = np.random.Generator(np.random.PCG64(11))
    w = (rng.standard_normal(64 * 40) * 0.02).astype(np.float32)
    q = O.quantize(w, False)
    codes = O.unpack_nibbles(q["codes"], w.size).reshape(-1, 64)
    wb = w.reshape(-1, 64)
    for b in range(wb.shape[0]):
        i = int(np.argmax(np.abs(wb[b])))
        assert codes[b, i] == (15 if wb[b, i] > 0 else 0)


def test_partial_tail_and_odd_numel():
    rng = np.random.Generator(np.random.PCG64(5))
    n = 64 * 257 + 37  # partial block and partial group, odd count
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    q = O.quantize(w, True)
    assert q["codes"].size == (n + 1) // 2 and (q["codes"][-1] >> 4) == 0
    assert q["absmax"].size == 258 and q["group_scale"].size == 2
    assert q["absmax"][-1] == np.max(np.abs(w[64 * 257:]))


# --- double quantization ----------------------------------------------------
def test_bits_per_param_matches_pages():
    g = golden("storage_figures.txt")
    for n, k in ((4096, 4096), (11008, 4096), (8192, 8192), (22016, 8192)):
        assert O.bits_per_param(n * k, True) == 0.126953125
        assert O.bits_per_param(n * k, False) == float(g["SCALE_BITS_PLAIN"])
    dq = O.bits_per_param(4096 * 4096, True)
    assert abs(dq - float(g["SCALE_BITS_DQ_APPROX"])) < 0.001
    saving = 0.5 - dq
    assert abs(saving - float(g["DQ_SAVING_BITS_APPROX"])) < 0.005
    # 65B model: ~3 GB saved, ~34 GB stored (4-bit codes + DQ scales)
    assert abs(65e9 * saving / 8 / 1e9 - float(g["SAVED_GB_65B_APPROX"])) < 0.2
    assert abs(65e9 * (4 + dq) / 8 / 1e9 - float(g["STORED_GB_65B_APPROX"])) < 1.0
    # 7B: 28 GB fp32 -> 3.5 GB at 4 bit
    assert 7e9 * 4 / 1e9 == float(g["FP32_GB_7B_APPROX"])
    assert 7e9 * 0.5 / 1e9 == float(g["INT4_GB_7B_APPROX"])


def test_dq_scale_error_bound_and_top_code():
    rng = np.random.Generator(np.random.PCG64(21))
    w = (rng.standard_normal(64 * 256 * 6) * 0.02).astype(np.float32)
    idx = rng.choice(w.size, 100, replace=False)
    w[idx] *= 10  # outliers
    q = O.quantize(w, True)
    a, s = q["absmax"].astype(np.float64), q["scales"].astype(np.float64)
    mg = np.repeat(q["group_scale"].astype(np.float64), 256)[: a.size]
    assert np.all(np.abs(s - a) <= mg / 510 * (1 + 1e-5))
    top = q["scale_codes"] == 255
    assert np.all((s == mg) == top)
    assert top.sum() == q["group_scale"].size


def test_dq_codes_match_exact_rational_argmin():
    rng = np.random.Generator(np.random.PCG64(8))
    a = (np.abs(rng.standard_normal(256 * 2)) * 0.03 + 1e-4).astype(np.float32)
    # push some ratios onto code midpoints
    a[:100] = (a[:100].max() * (np.arange(100) + 0.5) / 255).astype(np.float32)
    c2, mg = O.double_quantize(a)
    U = [Fraction(float(u)) for u in O.u8_scale_levels()]
    for b in range(a.size):
        M = Fraction(float(mg[b // 256]))
        x = round_fp32(Fraction(float(a[b])) / M)
        best, bd = None, None
        for k, u in enumerate(U):
            d = round_fp32(abs(x - u))
            if bd is None or d < bd:
                best, bd = k, d
        assert c2[b] == best


def test_e4m4_scale_table():
    """The float-like scale code: strictly increasing, 0 at code 0, exactly 1
    at code 240 (codes above exceed 1), powers of two at each exponent step,
    every value the exact dyadic rational of its definition, and a relative
    spacing of at most 1/16 above the subnormal codes."""
    E = O.e4m4_scale_levels()
    assert E.dtype == np.float32 and E.size == 256
    assert np.all(np.diff(E.astype(np.float64)) > 0)
    assert E[0] == 0 and E[240] == 1.0 and np.all(E[241:] > 1)
    for e in range(1, 16):
        assert E[16 * e] == np.float32(2.0 ** (e - 15))
    for c in range(256):
        e, m = c >> 4, c & 15
        want = Fraction(m, 2 ** 18) if e == 0 else Fraction(16 + m) * Fraction(2) ** (e - 19)
        assert Fraction(float(E[c])) == want, c
    rel = np.diff(E[16:241].astype(np.float64)) / E[16:240].astype(np.float64)
    assert rel.max() <= 1 / 16 + 1e-12


def test_e4m4_codes_match_exact_rational_argmin_and_bound():
    """Double quantization with the float-like code: codes equal the exact
    rational argmin (ties low), the decoded scale is within 1/32 relative of
    a_b wherever a_b / M_g >= 2^-14, and the group maximum decodes exactly."""
    rng = np.random.Generator(np.random.PCG64(23))
    a = (np.abs(rng.standard_normal(256 * 2)) * 0.03 + 1e-6).astype(np.float32)
    a[:60] = (a.max() * np.float32(2.0) ** -rng.uniform(0, 16, 60)).astype(np.float32)  # many binades
    E = O.e4m4_scale_levels()
    c2, mg = O.double_quantize(a, E)
    EF = [Fraction(float(v)) for v in E]
    for b in range(a.size):
        M = Fraction(float(mg[b // 256]))
        x = round_fp32(Fraction(float(a[b])) / M)
        best, bd = None, None
        for k, u in enumerate(EF):
            d = round_fp32(abs(x - u))
            if bd is None or d < bd:
                best, bd = k, d
        assert c2[b] == best, b
    s = O.decode_scales(c2, mg, E).astype(np.float64)
    mgr = np.repeat(mg.astype(np.float64), 256)[: a.size]
    big = a / mgr >= 2.0 ** -14
    assert np.all(np.abs(s[big] - a[big]) <= a[big] / 32 * (1 + 1e-6))
    assert np.all(c2[a == mgr] == 240)


def test_e4m4_beats_linear_on_small_ratios():
    """Where an outlier makes most blocks small next to the group maximum
    (ratios below 1/16), the float-like code's worst relative scale error is
    below the linear code's -- the reason for the variant."""
    rng = np.random.Generator(np.random.PCG64(24))
    w = (rng.standard_normal(64 * 256 * 4) * 0.02).astype(np.float32)
    w[rng.choice(w.size, 4, replace=False)] = 2.0  # one huge outlier per group, ratios about 0.03
    errs = {}
    for mode in (1, 2):
        q = O.quantize(w, mode)
        a, s = q["absmax"].astype(np.float64), q["scales"].astype(np.float64)
        errs[mode] = float(np.max(np.abs(s - a) / a))
    assert errs[2] < errs[1]


def test_dq_mse_increase_is_small():
    rng = np.random.Generator(np.random.PCG64(9))
    w = (rng.standard_normal(64 * 256 * 8) * 0.02).astype(np.float32)
    e = {}
    for dq in (False, True):
        w32, _ = O.dequantize(O.quantize(w, dq))
        e[dq] = float(np.mean((w32.astype(np.float64) - w) ** 2))
    assert e[False] <= e[True] < e[False] * 1.01


# --- bf16 rounding ----------------------------------------------------------
def test_f16_rounding_matches_torch():
    """The half rounding of the fp16 variant against torch's conversion, on
    random values, ties, subnormals and values past the half range."""
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(19))
    x = np.concatenate([
        (rng.standard_normal(20000) * 0.02).astype(np.float32),
        (rng.standard_normal(2000) * 1e-6).astype(np.float32),             # half subnormals
        np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24, 2 ** -25, 3 * 2 ** -26, 65504.0, 65520.0,
                  -0.0, 0.0, 6.1e-5], dtype=np.float32),                  # ties, smallest subnormal, overflow edge
    ])
    got = O.f16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(2))
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000  # exact ties
    bits[1000:2000] &= 0x807FFFFF  # subnormals
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = O.bf16_rne_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_dequant_value_is_level_times_scale():
    """w32 = fl32(L[c] * s) -- a single float32 product, checked with exact
    rationals on a random block set."""
    rng = np.random.Generator(np.random.PCG64(4))
    w = (rng.standard_normal(64 * 512) * 0.02).astype(np.float32)
    q = O.quantize(w, True)
    w32, _ = O.dequantize(q)
    codes = O.unpack_nibbles(q["codes"], w.size)
    L = O.nf4_levels()
    for i in rng.choice(w.size, 300, replace=False):
        s = Fraction(float(q["scales"][i // 64]))
        assert Fraction(float(w32[i])) == round_fp32(Fraction(float(L[codes[i]])) * s)
    # the scale itself: fl32(fl32(c2/255) * M_g)
    for b in rng.choice(q["absmax"].size, 100, replace=False):
        u = round_fp32(Fraction(int(q["scale_codes"][b]), 255))
        assert Fraction(float(q["scales"][b])) == round_fp32(u * Fraction(float(q["group_scale"][b // 256])))
