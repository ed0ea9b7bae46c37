"""CPU oracle: the QLoRA linear layer with dropout on the adapter path, in
float64.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.

Sources (cited by page title and section):
  [L] "LoRA y QLoRA en Profundidad", section "Dropout (lora_dropout)": during
      training the LoRA layers randomly zero elements as regularisation
      (0.0, 0.05 and 0.1 are the values the page discusses); section
      "Configuracion Completa" sets lora_dropout=0.05.
  [U] Ultralytics glossary "QLoRA", section "Come funziona QLoRA": the frozen
      path is the dequantized weight, and only the adapters get gradients.

Readings (the page names the effect, not the formula):
  * Dropout acts on the adapter's input: H = D(X) A^T with D(X) = X * keep /
    (1 - p) (inverted dropout: the kept elements are scaled so that the
    expected input is X). The frozen path X W^T is not dropped.
  * The keep mask (m x k, true = kept) is an explicit input, so the oracle
    and the GPU see the same mask; p is the drop probability.
  * Everything follows by the chain rule, with the mask held fixed:
        Y  = X W^T + s H B^T
        dH = s dY B
        dX = dY W + (dH A) * keep / (1 - p)
        dA = dH^T D(X)
        dB = s dY^T H
"""
from __future__ import annotations

import numpy as np

from .linear import lora_scale


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def dropped_input(x, keep, p: float):
    """D(X) = X * keep / (1 - p), p taken as the float32 value the layer gets."""
    q = 1.0 / (1.0 - float(np.float32(p)))
    return _f64(x) * (np.asarray(keep) != 0) * q


def linear_fwd_dropout(x, w, a, b, alpha, r, keep, p):
    """Returns (Y m x n, H m x r) with H from the dropped input."""
    x, w = _f64(x), _f64(w)
    y = x @ w.T
    if r == 0:
        return y, np.zeros((x.shape[0], 0))
    s = lora_scale(alpha, r)
    h = dropped_input(x, keep, p) @ _f64(a).T
    return y + s * (h @ _f64(b).T), h


def linear_bwd_dropout(x, w, a, b, dy, alpha, r, keep, p):
    """Gradients of <Y, dY> with Y from ``linear_fwd_dropout`` and the mask
    fixed. Returns (dX m x k, dA r x k, dB n x r)."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    dx = dy @ w
    if r == 0:
        return dx, np.zeros((0, x.shape[1])), np.zeros((w.shape[0], 0))
    a, b = _f64(a), _f64(b)
    s = lora_scale(alpha, r)
    xd = dropped_input(x, keep, p)
    h = xd @ a.T
    dh = s * (dy @ b)
    q = 1.0 / (1.0 - float(np.float32(p)))
    dx = dx + (dh @ a) * (np.asarray(keep) != 0) * q
    return dx, dh.T @ xd, s * (dy.T @ h)
