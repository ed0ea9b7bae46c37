"""CPU oracle: the QLoRA linear layer forward and backward, in float64.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.

Sources (cited by page title and section):
  [L] "LoRA y QLoRA en Profundidad" (skyvanguard.com.py), section "La Idea
      Central: Descomposicion de Bajo Rango": W is d_out x d_in, the update is
      B @ A with A r x d_in and B d_out x r; merged weight W + (alpha/r) B @ A.
      Section "Alpha (lora_alpha)": the effective update is (alpha/r) B @ A.
      Section "Inicializacion": A Gaussian, B zero, so the update starts at 0.
  [U] Ultralytics glossary "QLoRA", section "Come funziona QLoRA": each frozen
      layer dequantizes its NF4 weights to bfloat16 right before the matmul and
      adds the LoRA path output; backpropagation computes gradients through the
      dequantized weights but updates only the two LoRA matrices.

Inputs are the exact values the GPU sees (bf16 X, A, B, dY and the bf16
dequantized weight, all widened exactly to float64). Everything is computed in
float64 with library matmuls; there is no blocking or reordering beyond the
plain formulas. No bias, no dropout (bias="none" in the pages' LoraConfig).
"""
from __future__ import annotations

import numpy as np


def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / r [L], rounded once to float32 (the precision the layer
    receives it in)."""
    return float(np.float32(alpha) / np.float32(r))


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def linear_fwd(x, w, a, b, alpha, r):
    """H = X A^T and Y = X W^T + s H B^T [L], [U].

    x: m x k, w: n x k (dequantized bf16 values), a: r x k, b: n x r.
    Returns (Y m x n, H m x r) in float64.
    """
    x, w = _f64(x), _f64(w)
    y = x @ w.T
    if r == 0:
        return y, np.zeros((x.shape[0], 0))
    s = lora_scale(alpha, r)
    h = x @ _f64(a).T
    return y + s * (h @ _f64(b).T), h


def linear_bwd(x, w, a, b, dy, alpha, r):
    """Gradients of L = <Y, dY> with Y from ``linear_fwd`` [U]: the weight W
    is frozen (no dW); the adapters get dA and dB.

      H  = X A^T
      dH = s dY B
      dX = dY W + dH A
      dA = dH^T X
      dB = s dY^T H
    Returns (dX m x k, dA r x k, dB n x r) in float64.
    """
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    dx = dy @ w
    if r == 0:
        return dx, np.zeros((0, x.shape[1])), np.zeros((w.shape[0], 0))
    a, b = _f64(a), _f64(b)
    s = lora_scale(alpha, r)
    h = x @ a.T
    dh = s * (dy @ b)
    dx = dx + dh @ a
    da = dh.T @ x
    db = s * (dy.T @ h)
    return dx, da, db


def merged_weight(w, a, b, alpha, r):
    """W + (alpha/r) B @ A [L] -- used as an identity check on the forward."""
    return _f64(w) + lora_scale(alpha, r) * (_f64(b) @ _f64(a))


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over one tensor; an all-zero reference
    demands an exact zero (returns 0 or inf)."""
    got, ref = _f64(got), _f64(ref)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
