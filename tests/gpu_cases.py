"""Shared helpers for the GPU parity tests: seeded inputs (from ``synth``),
bf16 marshalling, and the oracle's expected values."""
from __future__ import annotations

import sys

import numpy as np

import synth
from oracle import linear as OL
from oracle import nf4 as O

TOL = 1e-2  # max|gpu - ref| / max|ref| per output tensor (bf16 inputs, fp32 accumulation)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_bf16(a: np.ndarray):
    """float32 numpy -> torch bf16 (CPU, round-to-nearest-even by torch)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_levels(codebook: int = 0) -> np.ndarray:
    """The oracle's table for a codebook id (0: NF4, 1: evenly spaced INT4)."""
    return O.int4_levels() if codebook == 1 else O.nf4_levels()


def oracle_weight(w: np.ndarray, dq: bool = True, codebook: int = 0):
    """Oracle quantization of an n x k fp32 weight and its bf16 dequantized values."""
    lv = oracle_levels(codebook)
    q = O.quantize(w.reshape(-1), dq, lv)
    _, bits = O.dequantize(q, lv)
    return q, O.bf16_bits_to_f32(bits).reshape(w.shape)


def oracle_weight_f16(w: np.ndarray, dq: bool = True):
    """The fp16 compute variant's weight: the half rounding of fl32(L s)."""
    w32, _ = O.dequantize(O.quantize(w.reshape(-1), dq))
    return O.f16_rne_bits(w32).view(np.float16).astype(np.float64).reshape(w.shape)


def to_f16(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float16)


def layer_inputs(n, k, m, r, tag, std_w=0.02):
    """W (fp32), X, A, B, dY as bf16 torch CPU tensors (values also used by the oracle)."""
    w = synth.normal((n, k), std_w, tag, "W")
    x = to_bf16(synth.normal((m, k), 1.0, tag, "X"))
    a = to_bf16(synth.normal((r, k), 1.0 / max(r, 1), tag, "A")) if r else None
    b = to_bf16(synth.normal((n, r), 0.01, tag, "B")) if r else None
    dy = to_bf16(synth.normal((m, n), 1.0, tag, "dY"))
    return w, x, a, b, dy


def rel(got, ref) -> float:
    return OL.rel_err(got, ref)
