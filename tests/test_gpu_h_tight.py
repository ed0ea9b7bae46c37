"""H = X A^T, as the forward returns it, held to 1e-5 of the fp64 product.

Each product of two 16-bit values is exact in fp32 and every path sums
them in fp32, so H carries only fp32 accumulation rounding. Every path that
forms H is covered: the prefill projection (r <= 64) and the skinny kernel
(r > 64) before the GEMM, the row-per-wave GEMV with H inside and with H
from split partials, the matrix-core GEMV with H inside (one and several
passes over k) and from partials, the grouped forms and fp16. A slip that
cost H a few bits (a 16-bit rounding of a partial sum, a dropped ragged
tail with small values) would pass the 1e-2 parity bound but not this one."""
import numpy as np
import pytest

import synth
from gpu_cases import f64, rel, say, to_bf16, to_f16

pytestmark = pytest.mark.gpu

TIGHT = 1e-5

# (name, m, n, k, r, half)
CASES = [
    ("prefill_proj_m300_k320_r8", 300, 272, 320, 8, "bf16"),
    ("prefill_proj_m520_k1088_r64", 520, 256, 1088, 64, "bf16"),
    ("prefill_skinny_m48_k256_r128", 48, 256, 256, 128, "bf16"),
    ("rows_fused_m1_k4096_r16", 1, 160, 4096, 16, "bf16"),
    ("rows_fused_m2_k2112_r20", 2, 48, 2112, 20, "bf16"),
    ("rows_partials_m1_k11008_r16", 1, 96, 11008, 16, "bf16"),
    ("mfma_fused_m3_k4160_r16", 3, 64, 4160, 16, "bf16"),
    ("mfma_fused_m2_k16384_r16", 2, 64, 16384, 16, "bf16"),
    ("mfma_partials_m4_k4096_r32", 4, 160, 4096, 32, "bf16"),
    ("mfma_partials_m8_k256_r24", 8, 128, 256, 24, "bf16"),
    ("rows_fused_m1_k4096_r16_f16", 1, 160, 4096, 16, "f16"),
    ("prefill_proj_m300_k320_r8_f16", 300, 272, 320, 8, "f16"),
]


def _inputs(m, n, k, r, tag, conv, ra=None):
    w = synth.normal((n, k), 0.02, tag, "W")
    x = conv(synth.normal((m, k), 1.0, tag, "X"))
    a = conv(synth.normal((ra or r, k), 1.0 / r, tag, "A"))
    b = conv(synth.normal((n, r), 0.01, tag, "B"))
    return w, x, a, b


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_h_tight(gpu_lib, case):
    import torch

    name, m, n, k, r, half = case
    conv = to_f16 if half == "f16" else to_bf16
    w, x, a, b = _inputs(m, n, k, r, f"h_tight_{name}", conv)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    _, h = gpu_lib.linear_fwd(q, x.cuda(), a.cuda(), b.cuda(), 2.0 * r)
    torch.cuda.synchronize()
    e = rel(f64(h), f64(x) @ f64(a).T)
    say(f"[h_tight] {name}: rel err H={e:.2e}")
    assert e <= TIGHT


@pytest.mark.parametrize("m", [1, 2, 4, 64])
def test_h_tight_grouped(gpu_lib, m):
    """Three parts of 256 rows, 16 slots each (48 slots of H)."""
    import torch

    parts, r, k = [256, 256, 256], 16, 4096
    w, x, a, b = _inputs(m, sum(parts), k, r, f"h_tight_grouped_m{m}", to_bf16, ra=len(parts) * r)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    _, h = gpu_lib.linear_fwd_grouped(q, parts, x.cuda(), a.cuda(), b.cuda(), 32.0)
    torch.cuda.synchronize()
    e = rel(f64(h), f64(x) @ f64(a).T)
    say(f"[h_tight] grouped m={m}: rel err H={e:.2e}")
    assert e <= TIGHT
    assert np.isfinite(f64(h)).all()
