"""GPU parity of the fp16 compute variant: dequantization to IEEE half is
bit-exact, and qlora_linear_fwd_f16 / qlora_linear_bwd_f16 agree with the
float64 oracle on the fp16 values (max|gpu - ref| / max|ref| <= 1e-2)."""
import numpy as np
import pytest

import synth
from gpu_cases import TOL, f64, rel, say
from oracle import linear as OL
from oracle import nf4 as O

pytestmark = pytest.mark.gpu


def to_f16(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float16)


def inputs(n, k, m, r, tag):
    w = synth.normal((n, k), 0.02, tag, "W")
    x = to_f16(synth.normal((m, k), 1.0, tag, "X"))
    a = to_f16(synth.normal((r, k), 1.0 / max(r, 1), tag, "A")) if r else None
    b = to_f16(synth.normal((n, r), 0.01, tag, "B")) if r else None
    dy = to_f16(synth.normal((m, n), 1.0, tag, "dY"))
    return w, x, a, b, dy


def w16_f16(w, dq):
    q = O.quantize(w.reshape(-1), dq)
    w32, _ = O.dequantize(q)
    return O.f16_rne_bits(w32).view(np.float16).astype(np.float64).reshape(w.shape)


@pytest.mark.parametrize("shape,dq", [((256, 256), True), ((4096, 4096), True), ((37, 50), False),
                                      ((11008, 4096), True)])
def test_dequantize_f16_bit_exact(gpu_lib, shape, dq):
    import torch

    w = synth.with_outliers(synth.normal(shape, 0.02, "f16dq", str(shape)), 0.001, 10.0, "f16dq", str(shape))
    say(f"[dequantize f16] shape={shape} dq={dq}")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda(), double_quant=dq)
    d = gpu_lib.dequantize(q, torch.float16)
    torch.cuda.synchronize()
    w32, _ = O.dequantize(O.quantize(w.reshape(-1), dq))
    assert np.array_equal(d.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16), O.f16_rne_bits(w32))


# (name, m, n, k, r, alpha, dq)
CASES = [
    ("ragged_m300_n272_k320_r8", 300, 272, 320, 8, 16.0, True),   # matmul path
    ("m1_r8", 1, 256, 256, 8, 16.0, True),                         # decode, H inside the GEMV
    ("m16_r16", 16, 512, 320, 16, 32.0, True),
    ("decode_rank24_m8", 8, 128, 256, 24, 48.0, True),             # decode, H from the skinny kernel
    ("decode_k4608_m3_r16", 3, 256, 4608, 16, 32.0, True),         # decode, k > 4096: two passes
    ("rank5_m40", 40, 128, 256, 5, 10.0, True),                    # rank gradients without the fused kernel
    ("rank64_m64", 64, 256, 512, 64, 16.0, True),
    ("no_dq_m96", 96, 384, 448, 16, 32.0, False),
    ("base_only_m33", 33, 256, 192, 0, 0.0, True),
    ("attn_4096x4096_m2048_r16", 2048, 4096, 4096, 16, 32.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_linear_f16_parity(gpu_lib, case):
    import torch

    name, m, n, k, r, alpha, dq = case
    say(f"[linear f16] case={name} m={m} n={n} k={k} r={r} dq={dq}")
    w, x, a, b, dy = inputs(n, k, m, r, "f16_" + name)
    w16 = w16_f16(w, dq)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda(), double_quant=dq)
    xc, dyc = x.cuda(), dy.cuda()
    ac = a.cuda() if r else None
    bc = b.cuda() if r else None
    y, h = gpu_lib.linear_fwd(q, xc, ac, bc, alpha)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    fa = f64(a) if r else None
    fb = f64(b) if r else None
    y_ref, h_ref = OL.linear_fwd(f64(x), w16, fa, fb, alpha, r)
    ey = rel(f64(y), y_ref)
    msg = f"   fwd rel err y={ey:.2e}"
    assert ey <= TOL, msg
    if r:
        assert rel(f64(h), h_ref) <= TOL
    dx, da, db = gpu_lib.linear_bwd(q, xc, dyc, ac, bc, alpha, h=h)
    torch.cuda.synchronize()
    assert dx.dtype == torch.float16
    dx_ref, da_ref, db_ref = OL.linear_bwd(f64(x), w16, fa, fb, f64(dy), alpha, r)
    edx = rel(f64(dx), dx_ref)
    msg += f" bwd dx={edx:.2e}"
    assert edx <= TOL, msg
    if r:
        eda, edb = rel(f64(da), da_ref), rel(f64(db), db_ref)
        msg += f" da={eda:.2e} db={edb:.2e}"
        assert eda <= TOL and edb <= TOL, msg
    say(msg)
