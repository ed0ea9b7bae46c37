"""GPU parity at the size limits of the linear calls.

The largest weight, n k = 2^31 (32768 x 65536): the fp32 source is 8 GiB, so its last rows lie past every
32-bit byte offset, and the packed codes fill 1 GiB. Sampled weight rows are
checked against the oracle: codes, scale codes, group scales and the
dequantized bf16 values bit for bit, the outputs of those rows in the
forward (one token: the matrix-core GEMV, 32 tokens: the fused GEMM) within
the 1e-2 bound, and the backward with dY non-zero only on those rows (so dX
depends on no other weight row, while the dX GEMM still contracts over all
32768 of them); dA and dB in full.

The longest row, k = 2^22 (n = 16): every output of the forward and
backward at one and 32 tokens."""
import numpy as np
import pytest

import synth
from gpu_cases import TOL, f64, rel, say, to_bf16
from oracle import linear as OL
from oracle import nf4 as O

pytestmark = pytest.mark.gpu

N, K = 32768, 65536
ROWS = [0, 1, N // 2 + 7, N - 1]  # the last one starts 8 GiB - 256 KiB into the fp32 source
R, ALPHA = 16, 32.0


def test_max_size_sampled(gpu_lib):
    import torch

    tag = "max_size"
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2031)
    say(f"[max] draw a {N} x {K} fp32 weight on the device")
    w = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32).mul_(0.02)
    w_rows = w[ROWS].cpu().numpy()  # the oracle's inputs: torch's draw, not a kernel of this library
    say("[max] quantize")
    q = gpu_lib.quantize(w)
    torch.cuda.synchronize()
    del w
    torch.cuda.empty_cache()

    # every row holds 1024 blocks = 4 whole double-quantization groups
    codes = q.codes.view(N, K // 2)
    scodes = q.scale_codes.view(N, K // 64)
    gscale = q.group_scale.view(N, K // (64 * 256))
    w16 = np.empty((len(ROWS), K), dtype=np.float64)
    ref_bits = []
    for i, row in enumerate(ROWS):
        ref = O.quantize(w_rows[i], True)
        assert np.array_equal(codes[row].cpu().numpy(), ref["codes"]), f"codes of row {row}"
        assert np.array_equal(scodes[row].cpu().numpy(), ref["scale_codes"]), f"scale codes of row {row}"
        assert np.array_equal(gscale[row].cpu().numpy().view(np.uint32),
                              np.asarray(ref["group_scale"], dtype=np.float32).view(np.uint32)), f"group scales of row {row}"
        _, bits = O.dequantize(ref)
        ref_bits.append(bits)
        w16[i] = O.bf16_bits_to_f32(bits)

    say("[max] dequantize to bf16 (4 GiB)")
    wd = gpu_lib.dequantize(q, torch.bfloat16)
    torch.cuda.synchronize()
    for i, row in enumerate(ROWS):
        got = wd[row].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref_bits[i]), f"dequantized row {row}"
    del wd
    torch.cuda.empty_cache()

    a = to_bf16(synth.normal((R, K), 1.0 / R, tag, "A"))
    b = to_bf16(synth.normal((N, R), 0.01, tag, "B"))
    a64, b64 = f64(a), f64(b)
    ac, bc = a.cuda(), b.cuda()
    for m in (1, 32):
        x = to_bf16(synth.normal((m, K), 1.0, tag, f"X{m}"))
        say(f"[max] forward m={m}")
        y, h = gpu_lib.linear_fwd(q, x.cuda(), ac, bc, ALPHA)
        torch.cuda.synchronize()
        x64 = f64(x)
        y_ref, h_ref = OL.linear_fwd(x64, w16, a64, b64[ROWS], ALPHA, R)
        ey, eh = rel(f64(y)[:, ROWS], y_ref), rel(f64(h), h_ref)
        say(f"   rel err y={ey:.2e} h={eh:.2e}")
        assert max(ey, eh) <= TOL

    # backward (32 tokens): dY zero outside the sampled rows' output columns
    m = 32
    x = to_bf16(synth.normal((m, K), 1.0, tag, f"X{m}"))
    dy_s = synth.normal((m, len(ROWS)), 1.0, tag, "dY")
    dy = np.zeros((m, N), dtype=np.float32)
    dy[:, ROWS] = dy_s
    dy = to_bf16(dy)
    say("[max] backward m=32")
    xc = x.cuda()
    _, h = gpu_lib.linear_fwd(q, xc, ac, bc, ALPHA)
    dx, da, db = gpu_lib.linear_bwd(q, xc, dy.cuda(), ac, bc, ALPHA, h=h)
    torch.cuda.synchronize()
    x64, dy64 = f64(x), f64(dy)
    dx_ref, _, _ = OL.linear_bwd(x64, w16, a64, b64[ROWS], dy64[:, ROWS], ALPHA, R)
    s = OL.lora_scale(ALPHA, R)
    h_ref = x64 @ a64.T
    dh_ref = s * (dy64 @ b64)
    da_ref = dh_ref.T @ x64
    db_ref = s * (dy64.T @ h_ref)
    edx, eda, edb = rel(f64(dx), dx_ref), rel(f64(da), da_ref), rel(f64(db), db_ref)
    say(f"   rel err dx={edx:.2e} da={eda:.2e} db={edb:.2e}")
    assert max(edx, eda, edb) <= TOL


def test_max_k_full(gpu_lib):
    """The longest accepted row, k = 2^22, with n = 16 (64 M weights): the
    one-token GEMV makes 1024 passes over k, the 32-token GEMM 65536 K-steps
    in one workgroup, the dX GEMM 32768 output tiles of one ragged step.
    Every output is checked against the oracle."""
    import torch

    n, k, tag = 16, 1 << 22, "max_k"
    w = synth.normal((n, k), 0.02, tag, "W")
    say(f"[max_k] oracle quantization of {n} x {k}")
    ref = O.quantize(w.reshape(-1), True)
    _, bits = O.dequantize(ref)
    w16 = O.bf16_bits_to_f32(bits).reshape(n, k).astype(np.float64)
    say("[max_k] quantize")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(q.scale_codes.cpu().numpy(), ref["scale_codes"])
    del w
    a = to_bf16(synth.normal((R, k), 1.0 / R, tag, "A"))
    b = to_bf16(synth.normal((n, R), 0.01, tag, "B"))
    a64, b64 = f64(a), f64(b)
    ac, bc = a.cuda(), b.cuda()
    for m in (1, 32):
        x = to_bf16(synth.normal((m, k), 1.0, tag, f"X{m}"))
        dy = to_bf16(synth.normal((m, n), 1.0, tag, f"dY{m}"))
        say(f"[max_k] forward and backward m={m}")
        xc = x.cuda()
        y, h = gpu_lib.linear_fwd(q, xc, ac, bc, ALPHA)
        dx, da, db = gpu_lib.linear_bwd(q, xc, dy.cuda(), ac, bc, ALPHA, h=h)
        torch.cuda.synchronize()
        x64, dy64 = f64(x), f64(dy)
        y_ref, h_ref = OL.linear_fwd(x64, w16, a64, b64, ALPHA, R)
        dx_ref, da_ref, db_ref = OL.linear_bwd(x64, w16, a64, b64, dy64, ALPHA, R)
        errs = [rel(f64(y), y_ref), rel(f64(h), h_ref), rel(f64(dx), dx_ref), rel(f64(da), da_ref),
                rel(f64(db), db_ref)]
        say("   rel err y/h/dx/dA/dB = " + " ".join(f"{e:.2e}" for e in errs))
        assert max(errs) <= TOL
