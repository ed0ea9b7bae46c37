"""GPU parity of qlora_merge / qlora_unmerge / qlora_requantize: merged and
unmerged values (float32 and bf16) and the re-quantized weight are bit-equal
to the oracle's, which forms the update in the same stated float32 order."""
import numpy as np
import pytest

from gpu_cases import layer_inputs, oracle_levels, oracle_weight, say
from oracle import merge as OM
from oracle import nf4 as O

pytestmark = pytest.mark.gpu

# (name, n, k, r, alpha, dq, codebook)
CASES = [
    ("ragged_n50_k320_r8", 50, 320, 8, 16.0, True, 0),      # n not a multiple of 16, k of 512
    ("r1", 32, 576, 1, 2.0, True, 0),
    ("r5_no_dq", 48, 256, 5, 10.0, False, 0),
    ("r64", 64, 1024, 64, 16.0, True, 0),
    ("r128", 40, 512, 128, 64.0, True, 0),
    ("r0", 24, 192, 0, 0.0, True, 0),
    ("int4_r16", 80, 640, 16, 32.0, True, 1),
    ("float8_scales_r16", 64, 512, 16, 32.0, 2, 0),
    ("attn_4096x4096_r16", 4096, 4096, 16, 32.0, True, 0),
    ("mlp_11008x4096_r16", 11008, 4096, 16, 32.0, True, 0),
]


def _bits16(t):
    import torch

    return t.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)


def _bits32(t):
    return t.reshape(-1).cpu().numpy().view(np.uint32)


def _setup(gpu_lib, name, n, k, r, dq, codebook):
    import torch

    w, _, a, b, _ = layer_inputs(n, k, 1, r, "merge_" + name)
    _, w16 = oracle_weight(w, dq, codebook)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda(), double_quant=dq, codebook=codebook)
    af = a.float().numpy() if r else np.zeros((0, k), np.float32)
    bf = b.float().numpy() if r else np.zeros((n, 0), np.float32)
    ac = a.cuda() if r else None
    bc = b.cuda() if r else None
    return q, w16.astype(np.float32), af, bf, ac, bc


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_merge_unmerge_bit_exact(gpu_lib, case):
    import torch

    name, n, k, r, alpha, dq, codebook = case
    say(f"[merge] case={name} n={n} k={k} r={r} dq={dq} codebook={codebook}")
    q, w16, af, bf, ac, bc = _setup(gpu_lib, name, n, k, r, dq, codebook)
    m32 = gpu_lib.merge(q, ac, bc, alpha, torch.float32)
    m16 = gpu_lib.merge(q, ac, bc, alpha, torch.bfloat16)
    torch.cuda.synchronize()
    ref32, ref16 = OM.merge(w16, af, bf, alpha, r)
    assert np.array_equal(_bits32(m32), ref32.reshape(-1).view(np.uint32))
    assert np.array_equal(_bits16(m16), ref16.reshape(-1))
    say(f"[unmerge] case={name}")
    u32 = gpu_lib.unmerge(m32, ac, bc, alpha)
    u16 = gpu_lib.unmerge(m16, ac, bc, alpha)
    torch.cuda.synchronize()
    uref32, _ = OM.unmerge(ref32, af, bf, alpha, r)
    _, uref16 = OM.unmerge(O.bf16_bits_to_f32(ref16).reshape(n, k), af, bf, alpha, r)
    assert np.array_equal(_bits32(u32), uref32.reshape(-1).view(np.uint32))
    assert np.array_equal(_bits16(u16), uref16.reshape(-1))
    # in place gives the same bits
    gpu_lib.unmerge(m32, ac, bc, alpha, out=m32)
    torch.cuda.synchronize()
    assert torch.equal(m32, u32)


@pytest.mark.parametrize("case", [c for c in CASES if c[1] * c[2] <= 1 << 20] + [CASES[7]],
                         ids=[c[0] for c in CASES if c[1] * c[2] <= 1 << 20] + [CASES[7][0]])
@pytest.mark.parametrize("dq_out,cb_out", [(True, 0), (False, 1)])
def test_requantize_bit_exact(gpu_lib, case, dq_out, cb_out):
    import torch

    name, n, k, r, alpha, dq, codebook = case
    say(f"[requantize] case={name} n={n} k={k} r={r} -> dq={dq_out} codebook={cb_out}")
    q, w16, af, bf, ac, bc = _setup(gpu_lib, name, n, k, r, dq, codebook)
    q2, merged = gpu_lib.requantize(q, ac, bc, alpha, double_quant=dq_out, codebook=cb_out, keep_absmax=True)
    torch.cuda.synchronize()
    lv = oracle_levels(cb_out)
    ref = OM.requantize(w16, af, bf, alpha, r, dq_out, lv)
    assert np.array_equal(_bits32(merged), ref["merged"].reshape(-1).view(np.uint32))
    assert np.array_equal(q2.codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(_bits32(q2.absmax), ref["absmax"].view(np.uint32))
    if dq_out:
        assert np.array_equal(q2.scale_codes.cpu().numpy(), ref["scale_codes"])
        assert np.array_equal(_bits32(q2.group_scale), ref["group_scale"].view(np.uint32))
    # the new packed weight dequantizes like the oracle's
    _, bits = O.dequantize(ref, lv)
    assert np.array_equal(_bits16(gpu_lib.dequantize(q2, torch.bfloat16)), bits)


def test_merged_layer_matches_adapted_layer(gpu_lib):
    """The merged bf16 weight used as a plain weight gives the adapted
    forward within the layer tolerance (the pages' reason to merge)."""
    import torch

    from gpu_cases import TOL, f64, rel
    from oracle import linear as OL

    n, k, m, r, alpha = 256, 512, 64, 16, 32.0
    w, x, a, b, _ = layer_inputs(n, k, m, r, "merge_fwd")
    _, w16 = oracle_weight(w, True)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    say("[merge] merged forward vs adapted forward")
    mw = gpu_lib.merge(q, a.cuda(), b.cuda(), alpha, torch.bfloat16)
    ym = x.cuda().float() @ mw.float().t()
    torch.cuda.synchronize()
    y_ref, _ = OL.linear_fwd(f64(x), w16, f64(a), f64(b), alpha, r)
    assert rel(f64(ym), y_ref) <= TOL
