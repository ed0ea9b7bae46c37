"""The binding refuses tensors that do not match what a call assumes (shape,
dtype, device, contiguity) before anything reaches the library: the C ABI
takes raw pointers and sizes, so a mismatch would otherwise be read out of
bounds. CPU tensors stand in for device tensors: every case here raises
before the first library call."""
import pytest
import torch

from bit_nf4_quantized_18_amd import binding as B


def _packed(n=32, k=128):
    numel = n * k
    nb = numel // B.BLOCK
    return B.PackedNF4(n, k, torch.zeros(numel // 2, dtype=torch.uint8), True,
                       torch.zeros(nb, dtype=torch.uint8), torch.zeros(1, dtype=torch.float32))


def _inputs(m=4, n=32, k=128, r=8, dtype=torch.bfloat16):
    return (torch.zeros(m, k, dtype=dtype), torch.zeros(r, k, dtype=dtype), torch.zeros(n, r, dtype=dtype),
            torch.zeros(m, n, dtype=dtype))


def test_fwd_rejects_bad_shapes_dtypes_and_layouts():
    q = _packed()
    x, a, b, _ = _inputs()
    with pytest.raises(ValueError, match="x has shape"):
        B.linear_fwd(q, x[:, :64].contiguous(), a, b, 16.0)
    with pytest.raises(ValueError, match="a has shape"):
        B.linear_fwd(q, x, a[:, :64].contiguous(), b, 16.0)
    with pytest.raises(ValueError, match="b has shape"):
        B.linear_fwd(q, x, a, b[:16].contiguous(), 16.0)
    with pytest.raises(TypeError, match="a has dtype"):
        B.linear_fwd(q, x, a.float(), b, 16.0)
    with pytest.raises(TypeError, match="x must be bfloat16 or float16"):
        B.linear_fwd(q, x.float(), a, b, 16.0)
    with pytest.raises(ValueError, match="must be contiguous"):
        B.linear_fwd(q, torch.zeros(128, 4, dtype=torch.bfloat16).t(), a, b, 16.0)
    with pytest.raises(ValueError, match="together"):
        B.linear_fwd(q, x, a, None, 16.0)
    with pytest.raises(ValueError, match="out has shape"):
        B.linear_fwd(q, x, a, b, 16.0, out=torch.zeros(4, 16, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="h_out has dtype"):
        B.linear_fwd(q, x, a, b, 16.0, h_out=torch.zeros(4, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="ws must be"):
        B.linear_fwd(q, x, a, b, 16.0, ws=torch.zeros(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="x has shape"):
        B.linear_fwd_noalloc(q, x[:, :64].contiguous(), a, b, 16.0)


def test_bwd_rejects_bad_tensors():
    q = _packed()
    x, a, b, dy = _inputs()
    with pytest.raises(ValueError, match="dy has shape"):
        B.linear_bwd(q, x, dy[:, :16].contiguous(), a, b, 16.0)
    with pytest.raises(ValueError, match="h has shape"):
        B.linear_bwd(q, x, dy, a, b, 16.0, h=torch.zeros(4, 4))
    with pytest.raises(ValueError, match="da has shape"):
        B.linear_bwd(q, x, dy, a, b, 16.0, da=torch.zeros(8, 64))
    with pytest.raises(TypeError, match="db has dtype"):
        B.linear_bwd(q, x, dy, a, b, 16.0, db=torch.zeros(32, 8, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="x has dtype"):
        B.linear_bwd(q, x.half(), dy, a, b, 16.0)


def test_grouped_and_dropout_reject_bad_tensors():
    q = _packed(48, 128)
    x, a, b, dy = _inputs(n=48)
    a3 = torch.zeros(24, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="a has shape"):
        B.linear_fwd_grouped(q, [16, 16, 16], x, a, b, 16.0)  # a must stack 3 x 8 rows
    with pytest.raises(ValueError, match="h_out has shape"):
        B.linear_fwd_grouped(q, [16, 16, 16], x, a3, b, 16.0, h_out=torch.zeros(4, 8))
    with pytest.raises(ValueError, match="da has shape"):
        B.linear_bwd_grouped(q, [16, 16, 16], x, dy, a3, b, 16.0, da=torch.zeros(8, 128))
    keep = torch.ones(4, 128, dtype=torch.uint8)
    with pytest.raises(TypeError, match="keep has dtype"):
        B.linear_fwd_dropout(q, x, a, b, 16.0, keep.bool(), 0.1)
    with pytest.raises(ValueError, match="keep has shape"):
        B.linear_bwd_dropout(q, x, dy, a, b, 16.0, keep[:2].contiguous(), 0.1)


def test_packed_weight_buffers_checked():
    q = _packed()
    q.scale_codes = None
    with pytest.raises(ValueError, match="scale_codes is required"):
        B.dequantize(q)
    q = _packed()
    q.codes = q.codes[:100]
    with pytest.raises(ValueError, match="codes must be"):
        B.linear_fwd(q, *_inputs()[:3], 16.0)
    q = _packed()
    q.group_scale = q.group_scale.double()
    with pytest.raises(ValueError, match="group_scale must be"):
        B.merge(q, None, None, 0.0)
