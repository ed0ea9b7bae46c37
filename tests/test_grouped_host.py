"""Grouped linears on the host: the stacked-weight encoding is the parts'
encodings laid end to end (an oracle property that the grouped calls rely
on), and the grouped C-ABI entry points reject bad part lists before any
launch."""
import ctypes

import numpy as np

import synth
from bit_nf4_quantized_18_amd import binding

# Every call below fails its argument checks (or has m = 0) before anything
# is launched: the pointers are placeholders, never dereferenced.
from oracle import nf4 as O

P = 1 << 20


def wstruct(n, k):
    return binding.NF4WeightC(n=n, k=k, codes=P, scale_codes=P, group_scale=P, absmax=None, double_quant=1)


def test_stacked_quantization_is_concatenation():
    """Parts of 256 rows at k = 128 span whole double-quantization groups
    (256 blocks of 64), so quantizing the stacked matrix gives each part's
    codes, scale codes and group maxima unchanged, in order."""
    k = 128
    parts = [256, 512, 256]
    ws = [synth.normal((n, k), 0.02, "grouped_pin", f"W{i}") for i, n in enumerate(parts)]
    ws[1][3, 5] = 0.9  # an outlier in one part only
    whole = O.quantize(np.concatenate(ws, axis=0).reshape(-1), True)
    each = [O.quantize(w.reshape(-1), True) for w in ws]
    assert np.array_equal(whole["codes"], np.concatenate([q["codes"] for q in each]))
    assert np.array_equal(whole["scale_codes"], np.concatenate([q["scale_codes"] for q in each]))
    assert np.array_equal(whole["group_scale"], np.concatenate([q["group_scale"] for q in each]))


def test_grouped_workspace_sizes():
    f = binding.grouped_workspace_bytes
    assert f(2048, 12288, 4096, 3, 16) > 0
    assert f(2048, 12288, 4096, 0, 16) == 0
    assert f(2048, 12288, 4096, 5, 16) == 0
    assert f(2048, 12288, 4096, 3, 0) == 0
    assert f(2048, 12288, 4096, 3, 64) == 0  # 3 * 64 > QLORA_MAX_RANK


def test_grouped_argument_errors():
    lib = binding.load()
    fwd, bwd = lib.qlora_linear_fwd_grouped, lib.qlora_linear_bwd_grouped
    w = wstruct(768, 128)
    ws_need = binding.grouped_workspace_bytes(32, 768, 128, 3, 16)

    def parts(*v):
        return (ctypes.c_int64 * len(v))(*v)

    good = parts(256, 256, 256)
    args = lambda pa, g=3, r=16: (ctypes.byref(w), g, pa, P, 32, P, P, r, 32.0, P, None, P, ws_need, None)  # noqa: E731
    assert fwd(*args(parts(256, 256, 128))) == -2     # part not a multiple of 256, sum short
    assert fwd(*args(parts(256, 256, 512))) == -2     # sum past n
    assert fwd(*args(good, g=0)) == -2
    assert fwd(*args(good, g=5)) == -2
    assert fwd(*args(good, r=0)) == -2
    assert fwd(*args(good, r=48)) == -4               # 3 * 48 > QLORA_MAX_RANK
    assert fwd(ctypes.byref(w), 3, None, P, 32, P, P, 16, 32.0, P, None, P, ws_need, None) == -1
    assert fwd(ctypes.byref(w), 3, good, P, 32, P, P, 16, 32.0, P, None, P, ws_need - 1, None) == -5
    assert fwd(ctypes.byref(w), 3, good, P, 0, None, None, 16, 32.0, None, None, None, 0, None) == 0  # m = 0
    bargs = lambda pa, r=16: (ctypes.byref(w), 3, pa, P, P, 32, P, P, r, 32.0, None, P, P, P, P, ws_need, None)  # noqa: E731
    assert bwd(*bargs(parts(256, 256, 128))) == -2
    assert bwd(*bargs(good, r=8)) == -4               # the backward needs r % 16 == 0
    assert bwd(ctypes.byref(w), 3, good, P, None, 32, P, P, 16, 32.0, None, P, P, P, P, ws_need, None) == -1
