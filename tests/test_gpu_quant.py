"""GPU parity of qlora_nf4_quantize / qlora_nf4_dequantize: codes, scale codes,
group maxima, exact absmax and dequantized bf16/fp32 values must be bit-equal
to the oracle's."""
import numpy as np
import pytest

import synth
from oracle import nf4 as O
from gpu_cases import say

pytestmark = pytest.mark.gpu


def _ties_case():
    """Blocks whose normalised values sit within a few ulp of every decision
    midpoint (exact fp32 distance ties included)."""
    L = O.nf4_levels()
    a = np.float32(0.0371)
    xs = []
    for k in range(15):
        v = np.float32((np.float64(L[k]) + np.float64(L[k + 1])) / 2)
        for _ in range(4):
            v = np.nextafter(v, np.float32(-2))
        for _ in range(9):
            xs.append(v)
            v = np.nextafter(v, np.float32(2))
    w = (np.array(xs, np.float64) * np.float64(a)).astype(np.float32)
    w = np.clip(w, -a, a)
    w = np.concatenate([w, np.zeros((-w.size) % 63, np.float32)]).reshape(-1, 63)
    w = np.concatenate([np.full((w.shape[0], 1), a, np.float32), w], axis=1)  # absmax a in every block
    return w.reshape(-1)


def _denormal_case():
    rng = np.random.Generator(np.random.PCG64(31))
    w = (rng.standard_normal(64 * 512) * 1e-39).astype(np.float32)  # subnormal weights and scales
    w[64 * 100: 64 * 101] = 0.0
    w[64 * 200: 64 * 300] *= np.float32(1e30)
    return w


def _zeros_case():
    w = synth.normal(64 * 256 * 3 + 64 * 5, 0.02, "zeros")
    w[: 64 * 256] = 0.0           # a whole zero group
    w[64 * 600: 64 * 601] = 0.0   # a zero block
    w[-10:] = -0.0
    return w


CASES = {
    "single_256x256": lambda: synth.normal((256, 256), 0.02, "q", "single"),
    "attn_4096x4096_outliers": lambda: synth.with_outliers(synth.normal((4096, 4096), 0.02, "q", "attn"),
                                                            0.001, 10.0, "q", "attn"),
    "mlp_11008x4096_outliers": lambda: synth.with_outliers(synth.normal((11008, 4096), 0.02, "q", "mlp"),
                                                            0.001, 10.0, "q", "mlp"),
    "student_t_2048x8192": lambda: synth.student_t((2048, 8192), 4, 0.02, "q", "t"),
    "ragged_1d": lambda: synth.normal(64 * 257 + 37, 0.02, "q", "ragged"),
    "numel_1": lambda: np.array([0.3], np.float32),
    "numel_3": lambda: np.array([0.3, -1.0, 2e-3], np.float32),
    "numel_63": lambda: synth.normal(63, 1.0, "q", "63"),
    "numel_65": lambda: synth.normal(65, 1.0, "q", "65"),
    "ties": _ties_case,
    "denormals": _denormal_case,
    "zeros": _zeros_case,
}


def _u8(t):
    return t.cpu().numpy().view(np.uint8)


def _f32bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("dq", [True, False])
@pytest.mark.parametrize("name", list(CASES))
def test_quantize_dequantize_bit_exact(gpu_lib, name, dq):
    import torch

    w = CASES[name]()
    say(f"[quantize] case={name} dq={dq} numel={w.size}")
    ref = O.quantize(w.reshape(-1), dq)
    wt = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    q = gpu_lib.quantize(wt, double_quant=dq, keep_absmax=True)
    torch.cuda.synchronize()
    assert np.array_equal(_u8(q.codes), ref["codes"])
    assert np.array_equal(_f32bits(q.absmax), ref["absmax"].view(np.uint32))
    if dq:
        assert np.array_equal(_u8(q.scale_codes), ref["scale_codes"])
        assert np.array_equal(_f32bits(q.group_scale), ref["group_scale"].view(np.uint32))
    # dequantize (without the exact absmax in DQ mode: the kernel must use c2 and M_g)
    if dq:
        q.absmax = None
    w32_ref, bits_ref = O.dequantize(ref)
    say(f"[dequantize] case={name} dq={dq}")
    d16 = gpu_lib.dequantize(q, torch.bfloat16)
    d32 = gpu_lib.dequantize(q, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(d16.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16), bits_ref)
    assert np.array_equal(d32.reshape(-1).cpu().numpy().view(np.uint32), w32_ref.view(np.uint32))


INT4_CASES = ["single_256x256", "attn_4096x4096_outliers", "ragged_1d", "numel_3", "numel_65", "denormals", "zeros"]


def _int4_ties_case():
    """Values within a few ulp of every midpoint of the evenly spaced table."""
    L = O.int4_levels()
    a = np.float32(0.0371)
    xs = []
    for k in range(15):
        v = np.float32((np.float64(L[k]) + np.float64(L[k + 1])) / 2)
        for _ in range(4):
            v = np.nextafter(v, np.float32(-2))
        for _ in range(9):
            xs.append(v)
            v = np.nextafter(v, np.float32(2))
    w = np.clip((np.array(xs, np.float64) * np.float64(a)).astype(np.float32), -a, a)
    w = np.concatenate([w, np.zeros((-w.size) % 63, np.float32)]).reshape(-1, 63)
    return np.concatenate([np.full((w.shape[0], 1), a, np.float32), w], axis=1).reshape(-1)


@pytest.mark.parametrize("dq", [True, False])
@pytest.mark.parametrize("name", INT4_CASES + ["int4_ties"])
def test_int4_codebook_bit_exact(gpu_lib, name, dq):
    """The evenly spaced codebook: same kernels with the other level table,
    codes and dequantized values bit-equal to the oracle with that table."""
    import torch

    w = _int4_ties_case() if name == "int4_ties" else CASES[name]()
    L = O.int4_levels()
    say(f"[quantize int4] case={name} dq={dq} numel={w.size}")
    ref = O.quantize(w.reshape(-1), dq, L)
    q = gpu_lib.quantize(torch.from_numpy(np.ascontiguousarray(w)).cuda(), double_quant=dq, keep_absmax=True,
                         codebook=gpu_lib.CODEBOOK_INT4)
    torch.cuda.synchronize()
    assert q.codebook == gpu_lib.CODEBOOK_INT4
    assert np.array_equal(_u8(q.codes), ref["codes"])
    assert np.array_equal(_f32bits(q.absmax), ref["absmax"].view(np.uint32))
    if dq:
        assert np.array_equal(_u8(q.scale_codes), ref["scale_codes"])
        q.absmax = None
    w32_ref, bits_ref = O.dequantize(ref, L)
    d16 = gpu_lib.dequantize(q, torch.bfloat16)
    d32 = gpu_lib.dequantize(q, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(d16.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16), bits_ref)
    assert np.array_equal(d32.reshape(-1).cpu().numpy().view(np.uint32), w32_ref.view(np.uint32))


def test_dequantize_2d_non_multiple_of_64(gpu_lib):
    """Dequantize takes any n x k; blocks still follow the flattened order."""
    import torch

    w = synth.normal((37, 50), 0.02, "q", "37x50")
    say("[dequantize] 37x50")
    ref = O.quantize(w.reshape(-1), True)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    w32_ref, bits_ref = O.dequantize(ref)
    d16 = gpu_lib.dequantize(q, torch.bfloat16)
    assert d16.shape == (37, 50)
    assert np.array_equal(d16.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16), bits_ref)


def test_quantize_deterministic(gpu_lib):
    import torch

    w = torch.from_numpy(synth.normal((1024, 1024), 0.02, "q", "det")).cuda()
    say("[quantize] determinism")
    a = gpu_lib.quantize(w)
    b = gpu_lib.quantize(w)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scale_codes, b.scale_codes)


@pytest.mark.parametrize("name", ["single_256x256", "attn_4096x4096_outliers", "ragged_1d", "numel_65", "denormals",
                                  "zeros", "ties"])
def test_float8_scale_code_bit_exact(gpu_lib, name):
    """double_quant = 2 (the float-like scale code): scale codes, group
    maxima, codes and dequantized values bit-equal to the oracle's."""
    import torch

    w = CASES[name]()
    say(f"[quantize dq=2] case={name} numel={w.size}")
    ref = O.quantize(w.reshape(-1), 2)
    q = gpu_lib.quantize(torch.from_numpy(np.ascontiguousarray(w)).cuda(), double_quant=2, keep_absmax=True)
    torch.cuda.synchronize()
    assert np.array_equal(_u8(q.codes), ref["codes"])
    assert np.array_equal(_u8(q.scale_codes), ref["scale_codes"])
    assert np.array_equal(_f32bits(q.group_scale), ref["group_scale"].view(np.uint32))
    q.absmax = None
    w32_ref, bits_ref = O.dequantize(ref)
    d16 = gpu_lib.dequantize(q, torch.bfloat16)
    d32 = gpu_lib.dequantize(q, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(d16.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16), bits_ref)
    assert np.array_equal(d32.reshape(-1).cpu().numpy().view(np.uint32), w32_ref.view(np.uint32))


@pytest.mark.parametrize("dq", [1, 0])
def test_saved_weight_reloads_bit_exact(gpu_lib, tmp_path, dq):
    """A weight quantized on the GPU, written with save_packed and read back
    with load_packed, dequantizes to the same bits as before and gives the
    same forward output; both are checked against the oracle's dequantized
    weight."""
    import torch

    n, k = 272, 640
    w = synth.normal((n, k), 0.02, "storage", "W")
    say(f"[quant] case=storage_round_trip dq={dq}")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda(), double_quant=bool(dq))
    path = tmp_path / "w.npz"
    gpu_lib.save_packed(path, q)
    r = gpu_lib.load_packed(path)
    w_before = gpu_lib.dequantize(q, torch.float32)
    w_after = gpu_lib.dequantize(r, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(w_before, w_after)
    lv = O.nf4_levels()
    ref, _ = O.dequantize(O.quantize(w.reshape(-1), dq, lv), lv)
    assert np.array_equal(w_after.cpu().numpy().reshape(-1).view(np.uint32), ref.view(np.uint32))
    x = torch.from_numpy(synth.normal((5, k), 1.0, "storage", "X")).to(torch.bfloat16).cuda()
    y0, _ = gpu_lib.linear_fwd(q, x)
    y1, _ = gpu_lib.linear_fwd(r, x)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
