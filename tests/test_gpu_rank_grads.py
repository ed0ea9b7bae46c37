"""dA and dB held to the precision of their product kernel.

dA = dH^T X and dB = s dY^T H contract the fp32 dH and H with the 16-bit X
and dY over the token rows. With bf16 compute each fp32 element enters the
matrix cores as a hi and a lo bf16 term (16 significant bits together) and
the sums stay fp32; with fp16 compute the products are fp32. A lo term that
was dropped or formed wrongly would leave about 2^-8 relative error, which
the 1e-2 parity bound lets through, so here dA and dB must be within 1e-4.

dB is compared with s dY^T H for the H that the forward returned, in fp64,
so only the gradient kernels' own rounding is measured; dA with the oracle's
fp64 dH^T X (the device's dH carries fp32 rounding only)."""
import numpy as np
import pytest

import synth
from gpu_cases import f64, rel, say, to_bf16, to_f16
from oracle import linear as OL

pytestmark = pytest.mark.gpu

TIGHT = 1e-4

# (name, m, n, k, r, alpha, half): r % 16 == 0 takes the fused dA/dB kernel
CASES = [
    ("m512_n1040_k960_r16", 512, 1040, 960, 16, 32.0, "bf16"),     # ragged 256-column blocks
    ("m300_n272_k320_r32", 300, 272, 320, 32, 64.0, "bf16"),       # ragged row split, two rank tiles
    ("m2048_n512_k4096_r64", 2048, 512, 4096, 64, 16.0, "bf16"),   # four rank tiles, several splits
    ("m512_n1040_k960_r16_f16", 512, 1040, 960, 16, 32.0, "f16"),
]


def _check(name, da, db, x64, dy64, b64, h_dev, s):
    dh_ref = s * (dy64 @ b64)
    da_ref = dh_ref.T @ x64
    db_ref = s * (dy64.T @ f64(h_dev))
    eda, edb = rel(f64(da), da_ref), rel(f64(db), db_ref)
    say(f"[rank_grads] {name}: rel err dA={eda:.2e} dB={edb:.2e}")
    assert eda <= TIGHT and edb <= TIGHT


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rank_grads_tight(gpu_lib, case):
    import torch

    name, m, n, k, r, alpha, half = case
    conv = to_f16 if half == "f16" else to_bf16
    tag = f"rank_grads_{name}"
    w = synth.normal((n, k), 0.02, tag, "W")
    x = conv(synth.normal((m, k), 1.0, tag, "X"))
    a = conv(synth.normal((r, k), 1.0 / r, tag, "A"))
    b = conv(synth.normal((n, r), 0.01, tag, "B"))
    dy = conv(synth.normal((m, n), 1.0, tag, "dY"))
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    xc, ac, bc = x.cuda(), a.cuda(), b.cuda()
    _, h = gpu_lib.linear_fwd(q, xc, ac, bc, alpha)
    _, da, db = gpu_lib.linear_bwd(q, xc, dy.cuda(), ac, bc, alpha, h=h, need_dx=False)
    torch.cuda.synchronize()
    _check(name, da, db, f64(x), f64(dy), f64(b), h, OL.lora_scale(alpha, r))


def test_rank_grads_tight_grouped(gpu_lib):
    """Two parts of 256 and 512 rows, 16 slots each: per-part U columns."""
    import torch

    parts, r, alpha, m, k = [256, 512], 16, 32.0, 384, 640
    n, tag = sum(parts), "rank_grads_grouped"
    w = synth.normal((n, k), 0.02, tag, "W")
    x = to_bf16(synth.normal((m, k), 1.0, tag, "X"))
    a = to_bf16(synth.normal((len(parts) * r, k), 1.0 / r, tag, "A"))
    b = to_bf16(synth.normal((n, r), 0.01, tag, "B"))
    dy = to_bf16(synth.normal((m, n), 1.0, tag, "dY"))
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    xc, ac, bc = x.cuda(), a.cuda(), b.cuda()
    _, h = gpu_lib.linear_fwd_grouped(q, parts, xc, ac, bc, alpha)
    _, da, db = gpu_lib.linear_bwd_grouped(q, parts, xc, dy.cuda(), ac, bc, alpha, h=h, need_dx=False)
    torch.cuda.synchronize()
    s = OL.lora_scale(alpha, r)
    x64, dy64, b64, h64 = f64(x), f64(dy), f64(b), f64(h)
    # dH slots of part l: s dY[:, rows of l] B_l; dB rows of part l: s dY[:, rows]^T H[:, slots of l]
    dh = np.zeros((m, len(parts) * r))
    db_ref = np.zeros((n, r))
    row = 0
    for l, rows in enumerate(parts):
        sl = slice(l * r, (l + 1) * r)
        dh[:, sl] = s * (dy64[:, row:row + rows] @ b64[row:row + rows])
        db_ref[row:row + rows] = s * (dy64[:, row:row + rows].T @ h64[:, sl])
        row += rows
    eda, edb = rel(f64(da), dh.T @ x64), rel(f64(db), db_ref)
    say(f"[rank_grads] grouped: rel err dA={eda:.2e} dB={edb:.2e}")
    assert eda <= TIGHT and edb <= TIGHT
