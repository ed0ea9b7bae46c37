"""CPU oracle: merging a trained adapter into the weight, taking it back out,
and re-quantizing the merged weight.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.

Sources (cited by page title and section):
  [L] "LoRA y QLoRA en Profundidad", section "La Idea Central: Descomposicion
      de Bajo Rango": for inference the adapter is folded into the weight,
      W_final = W + (alpha/r) B @ A, after which the layer has the plain
      architecture and cost.
  [U] Ultralytics glossary "QLoRA", sections "QLoRA e metodi correlati" and
      "Compromessi": an adapted model is merged into the 16-bit weights and
      then quantized again for distribution; merging needs the base weight
      dequantized to 16 bit first. Adapters are small and are stored and
      swapped per task (so the update must also come back out: unmerge).

Readings (where the pages give no precision):
  * The 16-bit base is the bf16 dequantized weight w16 the layer computes
    with, so the merged layer equals the adapted one up to rounding.
  * The update t = s * (B @ A), s = fl32(alpha / r), is formed in float32:
    d = sum over j = 0, 1, ..., r-1 in that order of fl32(b_pj * a_jq), each
    step one float32 addition; then t = fl32(s * d). The merged weight is
    m = fl32(w16 + t) (float32), or its bf16 round-to-nearest-even. The
    re-quantizer encodes this float32 m, so both sides decide every code
    from the same float32 values.
  * Unmerge of a merged weight W' (bf16 or float32 values) is fl32(W' - t)
    with the same t.
  * r = 0 means no adapter: t = 0.
"""
from __future__ import annotations

import numpy as np

from . import nf4


def _scale32(alpha: float, r: int) -> np.float32:
    return np.float32(np.float32(alpha) / np.float32(r))


def update32(a, b, alpha: float, r: int) -> np.ndarray:
    """t = fl32(s * d), d the float32 running sum of the rank-1 terms
    b[:, j] a[j, :] taken in ascending j (each product rounded to float32;
    for bf16 inputs it is exact). a: r x k, b: n x r, values as float32."""
    b = np.asarray(b, dtype=np.float32)
    a = np.asarray(a, dtype=np.float32)
    n, k = b.shape[0], a.shape[1]
    d = np.zeros((n, k), dtype=np.float32)
    for j in range(r):
        d = d + np.outer(b[:, j], a[j, :]).astype(np.float32)
    if r == 0:
        return d
    return (_scale32(alpha, r) * d).astype(np.float32)


def merge(w16, a, b, alpha: float, r: int):
    """m = fl32(w16 + t) [L]. Returns (m float32 n x k, bf16 bits of m)."""
    w16 = np.asarray(w16, dtype=np.float32)
    m = (w16 + update32(a, b, alpha, r)).astype(np.float32)
    return m, nf4.bf16_rne_bits(m)


def unmerge(w_merged, a, b, alpha: float, r: int):
    """fl32(W' - t): the adapter taken back out of a merged weight.
    Returns (float32 n x k, its bf16 bits)."""
    w = np.asarray(w_merged, dtype=np.float32)
    u = (w - update32(a, b, alpha, r)).astype(np.float32)
    return u, nf4.bf16_rne_bits(u)


def requantize(w16, a, b, alpha: float, r: int, double_quant: bool = True, levels=None) -> dict:
    """The merged float32 weight quantized again [U]: the packed weight of
    ``nf4.quantize`` (blocks, codes, scales exactly as for any float32
    weight), plus the merged values under key "merged"."""
    m, _ = merge(w16, a, b, alpha, r)
    q = nf4.quantize(m.reshape(-1), double_quant, levels)
    q["merged"] = m
    return q
