"""CPU oracle: a counter-based generator for dropout keep masks.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.

Dropout ("LoRA y QLoRA en Profundidad", section "Dropout (lora_dropout)")
needs random keep masks. To let the GPU draw them while the oracle checks
them bit for bit, both sides implement the same published counter-based
generator: Philox4x64 with 10 rounds (J. K. Salmon, M. A. Moraes,
R. O. Dror and D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011). One round maps the counter (x0, x1, x2, x3) under the key (k0, k1)
to (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)), with
64 x 64 -> 128-bit products; the key advances by two Weyl constants between
rounds. The multipliers and Weyl constants are the paper's.

Mask reading (this design's, documented with the C ABI): element g of the
global element stream lives in block b = g // 16, whose four output words
Philox4x64-10((b, 0, 0, 0), (seed, 0)) give sixteen 16-bit chunks, chunk
j = g % 16 being bits 16 (j % 4) .. 16 (j % 4) + 15 of word j // 4. The
element is dropped when float32(chunk) < float32(p) * 65536, so the drop
probability is ceil(65536 p) / 65536.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
W0, W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
ROUNDS = 10
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.ndarray, m: int):
    """(hi, lo) of the 128-bit product of uint64 arrays a and the constant m,
    from four 32 x 32 -> 64-bit partial products."""
    a = a.astype(np.uint64)
    m64 = np.uint64(m)
    a0, a1 = a & _LO32, a >> _S32
    m0, m1 = m64 & _LO32, m64 >> _S32
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = a * m64  # wraps modulo 2^64
    return hi, lo


def philox4x64_10(ctr, key):
    """ctr: uint64 array (..., 4), key: (k0, k1). Returns uint64 (..., 4)."""
    ctr = np.asarray(ctr, dtype=np.uint64)
    x0, x1, x2, x3 = (ctr[..., i].copy() for i in range(4))
    k0, k1 = int(key[0]), int(key[1])
    mask = (1 << 64) - 1
    with np.errstate(over="ignore"):
        for _ in range(ROUNDS):
            hi0, lo0 = _mulhilo(x0, M0)
            hi1, lo1 = _mulhilo(x2, M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ np.uint64(k0), lo1, hi0 ^ x3 ^ np.uint64(k1), lo0
            k0, k1 = (k0 + W0) & mask, (k1 + W1) & mask
    return np.stack([x0, x1, x2, x3], axis=-1)


def chunks16(seed: int, offset: int, count: int) -> np.ndarray:
    """The 16-bit chunks of elements offset .. offset + count - 1 (uint16)."""
    g0, g1 = offset, offset + count
    b0, b1 = g0 // 16, (g1 + 15) // 16
    ctr = np.zeros((b1 - b0, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(b0, b1, dtype=np.uint64)
    words = philox4x64_10(ctr, (seed, 0))                       # (blocks, 4)
    shifts = np.array([0, 16, 32, 48], dtype=np.uint64)
    ch = (words[:, :, None] >> shifts[None, None, :]) & np.uint64(0xFFFF)  # (blocks, 4 words, 4 chunks)
    flat = ch.reshape(-1).astype(np.uint16)                    # chunk j of a block at 4 (j // 4) + j % 4 = j
    return flat[g0 - 16 * b0: g1 - 16 * b0]


def keep_mask(seed: int, offset: int, count: int, p: float) -> np.ndarray:
    """uint8 keep mask: 0 where float32(chunk) < float32(p) * 65536, else 1."""
    thr = np.float32(p) * np.float32(65536.0)
    return (chunks16(seed, offset, count).astype(np.float32) >= thr).astype(np.uint8)
