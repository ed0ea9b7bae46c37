"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

This module only draws random numbers and describes workload shapes. It holds
none of the method's arithmetic (no codebook, no quantizer, no matmul), so both
the CPU oracle and the GPU path can take their inputs from it without sharing
any of the computation.

Every tensor comes from its own ``numpy.random.Generator(PCG64(seed))`` where the
seed is derived from a stable name (config / layer / tensor), so the same call
always returns the same array on any machine. Values are returned as float32;
callers that need bf16 tensors round them to bf16 themselves (that rounding is
a property of the input dtype, done once, and both sides then read the very
same bf16 values).

Distributions follow the workloads the pages describe:
  * frozen weights roughly normal with std 0.02 (Ultralytics glossary "QLoRA",
    the NF4-vs-INT4 example under "Come funziona QLoRA");
  * LoRA A Gaussian and B at zero at init ("LoRA y QLoRA en Profundidad",
    section "Inicializacion"); for parity we draw B small but non-zero so the
    adapter path is exercised, and test B = 0 separately;
  * a heavy-tailed Student-t(4) variant for the 65B-shaped set;
  * Bernoulli keep masks for adapter dropout ("LoRA y QLoRA en Profundidad",
    section "Dropout (lora_dropout)").
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np


def seed_of(*parts) -> int:
    """Stable 32-bit seed from a tuple of names/ints."""
    return zlib.crc32("/".join(str(p) for p in parts).encode()) & 0xFFFFFFFF


def rng(*parts) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_of(*parts)))


def normal(shape, std, *parts) -> np.ndarray:
    """float32 N(0, std^2) samples (std is the standard deviation)."""
    return (rng(*parts).standard_normal(shape, dtype=np.float64) * std).astype(np.float32)


def with_outliers(w: np.ndarray, frac: float, mul: float, *parts) -> np.ndarray:
    """Multiply round(frac * w.size) distinct, uniformly drawn entries by ``mul``."""
    out = np.array(w, dtype=np.float32, copy=True)
    cnt = int(round(frac * out.size))
    if cnt:
        idx = rng(*parts, "outliers").choice(out.size, size=cnt, replace=False)
        flat = out.reshape(-1)
        flat[idx] = flat[idx] * np.float32(mul)
    return out


def student_t(shape, df, scale, *parts) -> np.ndarray:
    return (rng(*parts).standard_t(df, size=shape) * scale).astype(np.float32)


def keep_mask(shape, p: float, *parts) -> np.ndarray:
    """Dropout keep mask: uint8, 1 with probability 1 - p, else 0 (one
    uniform draw per element; the pages' dropout rates are 0.05 and 0.1)."""
    return (rng(*parts).random(shape) >= p).astype(np.uint8)


# ----------------------------------------------------------------------------
# Workload descriptions (shapes only).
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    n: int  # d_out
    k: int  # d_in


def layer_set(hidden: int, ffn: int):
    """The seven adapted linears of one decoder block: q/k/v/o, gate/up, down."""
    return (
        Linear("q_proj", hidden, hidden),
        Linear("k_proj", hidden, hidden),
        Linear("v_proj", hidden, hidden),
        Linear("o_proj", hidden, hidden),
        Linear("gate_proj", ffn, hidden),
        Linear("up_proj", ffn, hidden),
        Linear("down_proj", hidden, ffn),
    )


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: tuple
    m: int            # tokens (batch x seq)
    r: int
    alpha: float
    weight_dist: str  # "normal" | "normal_outliers" | "student_t"


SMALL = Workload("single_256x256_m16_r8", (Linear("single", 256, 256),), 16, 8, 16.0, "normal")
DECODE_7B = Workload("decode_7b_4096x4096_11008x4096", (Linear("attn", 4096, 4096), Linear("mlp_up", 11008, 4096),
                                                       Linear("mlp_down", 4096, 11008)),
                     1, 16, 32.0, "normal_outliers")
LAYERS_7B = Workload("llama7b_layer_set_m2048_r16", layer_set(4096, 11008), 2048, 16, 32.0, "normal")
LAYERS_65B = Workload("llama65b_layer_set_m4096_r64", layer_set(8192, 22016), 4096, 64, 16.0, "student_t")


def weight(wl: Workload, layer: Linear, copy: int = 0) -> np.ndarray:
    """Frozen fp32 weight (n x k) for one linear of a workload."""
    tag = (wl.name, layer.name, copy, "W")
    if wl.weight_dist == "student_t":
        return student_t((layer.n, layer.k), 4, 0.02, *tag)
    w = normal((layer.n, layer.k), 0.02, *tag)
    if wl.weight_dist == "normal_outliers":
        w = with_outliers(w, 0.001, 10.0, *tag)
    return w


def activations(wl: Workload, layer: Linear, m: int | None = None) -> np.ndarray:
    """X (m x k), N(0,1), float32 values to be rounded to bf16 by the caller."""
    return normal((wl.m if m is None else m, layer.k), 1.0, wl.name, layer.name, "X")


def grad_output(wl: Workload, layer: Linear, m: int | None = None) -> np.ndarray:
    """dY (m x n), N(0,1)."""
    return normal((wl.m if m is None else m, layer.n), 1.0, wl.name, layer.name, "dY")


def lora_a(wl: Workload, layer: Linear) -> np.ndarray:
    """A (r x k), N(0, (1/r)^2) -- std 1/r."""
    return normal((wl.r, layer.k), 1.0 / wl.r, wl.name, layer.name, "A")


def lora_b(wl: Workload, layer: Linear) -> np.ndarray:
    """B (n x r), N(0, 0.01^2)."""
    return normal((layer.n, wl.r), 0.01, wl.name, layer.name, "B")
