"""CPU oracle: NF4 codebook, blockwise absmax quantizer, double quantization
of the scales, and dequantization -- written step by step from the pages.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The GPU library
never calls it and shares no code, table or constant generator with it.

Sources (cited by page title and section):
  [U] Ultralytics glossary "QLoRA", section "Come funziona QLoRA": the NF4
      bullet (16 levels at normal quantiles, one absmax scale per block of 64),
      the double-quantization bullet (scales to 8 bit in blocks of 256,
      0.5 -> ~0.127 bit/param), the forward/backward paragraph (dequantize to
      bfloat16 just before the matmul) and the printed NF4-vs-INT4 example
      (level construction, absmax per block, nearest-level encode, restore).
  [M] "Modulo 4: QLoRA" (courses.eduardonacimiento.com), section 4.3 b)
      "Cuantizacion Doble": weights are quantized to 4 bit first, then the
      scale constants to 8 bit.

Precision: every quantizer step is carried out in IEEE float32 exactly as
stated (numpy float32 ops are correctly rounded, keep denormals and never
contract), except the codebook itself, which is computed in float64 and
rounded once to float32.

Readings where the pages are silent:
  * the quantile offset is the printed literal 0.9677083, levels built in
    float64 and rounded once to float32;
  * nearest level = argmin of the float32 distance |x - L_k|, ties to the
    lowest index (what numpy/torch ``argmin`` return);
  * x = w / absmax is a correctly rounded float32 division;
  * an all-zero block encodes to the exact-zero level (code 7) with scale 0;
  * blocks are runs of 64 consecutive elements of the row-major flattening,
    the last run may be partial; double-quant groups are runs of 256 blocks;
  * two codes per byte, element 2i in the low nibble, 2i+1 in the high nibble
    (parity unpinned: a storage convention no page fixes); an odd element
    count leaves the final high nibble 0;
  * the 8-bit scale code is the unsigned linear codebook U_k = k/255 on
    [0, 1] times the group absmax M_g, encoded by the same nearest-level rule
    (parity unpinned: the pages say only "8 bit in blocks of 256");
  * an alternative, float-like 8-bit scale code (double_quant = 2): the
    unsigned 4-bit-exponent / 4-bit-mantissa values E_c, c = 16 e + m,
    E = m 2^-18 for e = 0 and (16 + m) 2^(e - 19) otherwise, so E_240 = 1 and
    codes 241..255 (above 1) are never chosen; same nearest-level rule
    (parity unpinned like the linear code: the pages fix only "8 bit");
  * the weights are encoded with their exact block absmax; the decoded scale
    s_b = fl32(U[c2_b] * M_g) is what dequantization uses;
  * dequantized value = fl32(L[code] * s_b), then round-to-nearest-even bf16.
"""
from __future__ import annotations

import math
import statistics

import numpy as np

NF4_QUANTILE_OFFSET = 0.9677083  # the literal printed in [U]'s example
BLOCK = 64                       # weights per absmax block [U]
DQ_GROUP = 256                   # blocks per second-level group [U]
ZERO_CODE = 7                    # index of the exact-zero level


# ---------------------------------------------------------------------------
# Codebooks
# ---------------------------------------------------------------------------
def nf4_levels(inv_cdf=None) -> np.ndarray:
    """16 NF4 levels, ascending, float32 [U].

    With Phi^-1 the standard-normal quantile function and o the quantile
    offset, the levels are, before normalisation,
        Phi^-1(p)  for p = o - i (o - 1/2) / 8,  i = 0 .. 7   (8 positive),
        0                                                      (exact zero),
        -Phi^-1(p) for p = o - j (o - 1/2) / 7,  j = 0 .. 6   (7 negative),
    i.e. probabilities evenly spaced from o towards 1/2 with 1/2 itself left
    out on each side (its quantile is the zero level). All 16 are divided by
    the largest, Phi^-1(o), so the table spans [-1, 1] with 1 at the top;
    the values are formed in float64 and rounded once to float32.
    ``inv_cdf`` is the float64 standard-normal quantile function; by default
    Python's ``statistics.NormalDist().inv_cdf``.
    """
    if inv_cdf is None:
        inv_cdf = statistics.NormalDist(0.0, 1.0).inv_cdf
    o = NF4_QUANTILE_OFFSET

    def side(count):
        # quantiles at `count` probabilities stepping from o towards 1/2
        return [float(inv_cdf(o - i * (o - 0.5) / count)) for i in range(count)]

    positive, negative = side(8), side(7)
    top = positive[0]  # Phi^-1(o), the largest level
    raw = sorted([-q for q in negative] + [0.0] + positive)
    return np.array([q / top for q in raw], dtype=np.float64).astype(np.float32)


def int4_levels() -> np.ndarray:
    """16 evenly spaced levels on [-1, 1] -- [U]'s comparison baseline.
    Level k is -1 + 2k/15 rounded once to float32 (numpy forms the float64
    value and rounds it; a float32-stepped linspace may differ in the last
    bits)."""
    return np.linspace(-1.0, 1.0, 16, dtype=np.float32)


def e4m4_scale_levels() -> np.ndarray:
    """E_c for c = 0..255: a float-like unsigned 8-bit code with 4 exponent
    and 4 mantissa bits whose code 240 is exactly 1 (the group maximum).
    Every value is a small integer times a power of two, so float32 holds it
    exactly."""
    c = np.arange(256)
    e, m = c >> 4, c & 15
    val = np.where(e == 0, m * 2.0 ** -18, (16 + m) * np.exp2(e - 19.0))
    return val.astype(np.float32)


def scale_levels(double_quant: int) -> np.ndarray:
    """The 8-bit scale codebook of a double-quantization mode: 1 linear k/255,
    2 the float-like E4M4 values."""
    return e4m4_scale_levels() if int(double_quant) == 2 else u8_scale_levels()


def u8_scale_levels() -> np.ndarray:
    """U_k = fl32(k / 255), k = 0..255: the 8-bit code for a scale relative to
    its group absmax (the plain reading of "8 bit" in [U] and [M])."""
    return np.arange(256, dtype=np.float32) / np.float32(255.0)


# ---------------------------------------------------------------------------
# Nearest-level encoder shared by both quantization levels (same rule twice)
# ---------------------------------------------------------------------------
def encode_nearest(x: np.ndarray, levels: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """code_i = argmin_k fl32(|x_i - L_k|), first index on ties. uint8."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    levels = np.asarray(levels, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint8)
    for s in range(0, x.size, chunk):
        d = np.abs(x[s:s + chunk, None] - levels[None, :])   # float32
        out[s:s + chunk] = np.argmin(d, axis=1)
    return out


# ---------------------------------------------------------------------------
# Blockwise absmax quantization [U]
# ---------------------------------------------------------------------------
def num_blocks(numel: int) -> int:
    return -(-numel // BLOCK)


def num_groups(numel: int) -> int:
    return -(-num_blocks(numel) // DQ_GROUP)


def block_absmax(w: np.ndarray) -> np.ndarray:
    """a_b = max |w| over each run of 64 consecutive elements (fp32, exact)."""
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    nb = num_blocks(w.size)
    padded = np.zeros(nb * BLOCK, dtype=np.float32)   # |0| never raises a max
    padded[: w.size] = np.abs(w)
    return padded.reshape(nb, BLOCK).max(axis=1)


def normalize(w: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """x = fl32(w / a_b); an all-zero block gives x = 0."""
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    a = np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK)[: w.size]
    x = np.zeros_like(w)
    nz = a > 0
    x[nz] = w[nz] / a[nz]
    return x


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Byte i = code[2i] | code[2i+1] << 4; a missing last code counts as 0."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if codes.size % 2:
        codes = np.concatenate([codes, np.zeros(1, dtype=np.uint8)])
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, numel: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out[:numel]


def double_quantize(absmax: np.ndarray, scale_table: np.ndarray | None = None):
    """Second level [U], [M]: per group of 256 blocks, M_g = max a_b; each
    a_b / M_g is encoded to the nearest U_k. Returns (c2 uint8, M_g float32)."""
    absmax = np.asarray(absmax, dtype=np.float32)
    nb = absmax.size
    ng = -(-nb // DQ_GROUP)
    padded = np.zeros(ng * DQ_GROUP, dtype=np.float32)
    padded[:nb] = absmax
    group_max = padded.reshape(ng, DQ_GROUP).max(axis=1)
    mg = np.repeat(group_max, DQ_GROUP)[:nb]
    x2 = np.zeros(nb, dtype=np.float32)
    nz = mg > 0
    x2[nz] = absmax[nz] / mg[nz]
    c2 = encode_nearest(x2, u8_scale_levels() if scale_table is None else scale_table)
    return c2, group_max


def decode_scales(c2: np.ndarray, group_max: np.ndarray, scale_table: np.ndarray | None = None) -> np.ndarray:
    """s_b = fl32(U[c2_b] * M_g)."""
    c2 = np.asarray(c2, dtype=np.uint8)
    mg = np.repeat(np.asarray(group_max, dtype=np.float32), DQ_GROUP)[: c2.size]
    return (u8_scale_levels() if scale_table is None else scale_table)[c2] * mg


def quantize(w: np.ndarray, double_quant: bool | int = True, levels: np.ndarray | None = None) -> dict:
    """Full quantizer. Weights first (with exact a_b), then the scales [M].
    double_quant: 0/False none, 1/True the linear 8-bit code, 2 the
    float-like E4M4 code."""
    if levels is None:
        levels = nf4_levels()
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    absmax = block_absmax(w)
    codes = encode_nearest(normalize(w, absmax), levels)
    out = {"numel": w.size, "codes": pack_nibbles(codes), "absmax": absmax, "double_quant": bool(double_quant)}
    out["dq_mode"] = int(double_quant)
    if double_quant:
        table = scale_levels(double_quant)
        c2, mg = double_quantize(absmax, table)
        out["scale_codes"] = c2
        out["group_scale"] = mg
        out["scales"] = decode_scales(c2, mg, table)
    else:
        out["scales"] = absmax
    return out


# ---------------------------------------------------------------------------
# Dequantization [U]
# ---------------------------------------------------------------------------
def f16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE half, nearest-even (subnormals kept), returned as
    uint16 bit patterns: the weight of the fp16 compute variant."""
    with np.errstate(over="ignore"):  # past 65504 rounds to infinity, as IEEE says
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returned as uint16 bit patterns
    (finite inputs only)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    return ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dequantize(q: dict, levels: np.ndarray | None = None):
    """w32 = fl32(L[code] * s_b) and its bf16 rounding (as uint16 bits)."""
    if levels is None:
        levels = nf4_levels()
    numel = q["numel"]
    codes = unpack_nibbles(q["codes"], numel)
    s = np.repeat(np.asarray(q["scales"], dtype=np.float32), BLOCK)[:numel]
    w32 = levels[codes] * s
    return w32, bf16_rne_bits(w32)


def bits_per_param(numel: int, double_quant: bool) -> float:
    """Scale storage per weight: 32-bit absmax per block, or an 8-bit code per
    block plus one 32-bit M_g per 256 blocks [U]."""
    nb, ng = num_blocks(numel), num_groups(numel)
    return (8.0 * nb + 32.0 * ng) / numel if double_quant else 32.0 * nb / numel
