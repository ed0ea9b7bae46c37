"""save_packed / load_packed on the host: the .npz holds the packed buffers
byte for byte and the sizes; a file whose buffers are too short for n x k is
refused on load."""
import numpy as np
import pytest
import torch

from bit_nf4_quantized_18_amd import binding as B


def _packed(dq):
    rng = np.random.Generator(np.random.PCG64(11))
    n, k = 48, 320
    nb = n * k // 64
    codes = torch.from_numpy(rng.integers(0, 256, n * k // 2, dtype=np.uint8))
    if dq:
        return B.PackedNF4(n, k, codes, dq, torch.from_numpy(rng.integers(0, 256, nb, dtype=np.uint8)),
                           torch.from_numpy(rng.random(1, dtype=np.float32)), None, B.CODEBOOK_NF4)
    return B.PackedNF4(n, k, codes, 0, None, None, torch.from_numpy(rng.random(nb, dtype=np.float32)),
                       B.CODEBOOK_INT4)


@pytest.mark.parametrize("dq", [0, 1, 2])
def test_round_trip_is_byte_exact(tmp_path, dq):
    q = _packed(dq)
    path = tmp_path / "w.npz"
    B.save_packed(path, q)
    r = B.load_packed(path, device="cpu")
    assert (r.n, r.k, int(r.double_quant), r.codebook) == (q.n, q.k, dq, q.codebook)
    for name in ("codes", "scale_codes", "group_scale", "absmax"):
        a, b = getattr(q, name), getattr(r, name)
        assert (a is None) == (b is None), name
        if a is not None:
            assert a.dtype == b.dtype and torch.equal(a, b), name


def test_truncated_buffers_are_refused(tmp_path):
    q = _packed(1)
    q.codes = q.codes[:100]
    with pytest.raises(ValueError, match="codes"):
        B.save_packed(tmp_path / "bad.npz", q)
    # a file written by hand with a short scale-code buffer
    np.savez(tmp_path / "short.npz", n=np.int64(48), k=np.int64(320), double_quant=np.int32(1),
             codebook=np.int32(0), codes=np.zeros(48 * 320 // 2, np.uint8), scale_codes=np.zeros(10, np.uint8),
             group_scale=np.zeros(1, np.float32))
    with pytest.raises(ValueError, match="scale_codes"):
        B.load_packed(tmp_path / "short.npz", device="cpu")
