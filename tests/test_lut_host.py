"""The kernels' register lookup (nf4_lut.h), built for the host with a model
of the byte-permute instruction, against the oracle's dequantized values."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from oracle import nf4 as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def emul(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("lut") / "lut_emul.so")
    cmd = ["hipcc", "-O2", "-fPIC", "-shared", "-std=c++17", f"-I{ROOT}/bit_nf4_quantized_18_amd/csrc",
           f"-I{ROOT}/include", os.path.join(ROOT, "tests", "native", "lut_emul.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return ctypes.CDLL(out)


def run_lut(emul, levels, scale, words):
    words = np.ascontiguousarray(words, dtype=np.uint32)
    dec = np.zeros(words.size * 4, np.uint32)
    nat = np.zeros(words.size * 4, np.uint32)
    f = emul.lut_emul
    f.argtypes = [ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f(levels.ctypes.data, ctypes.c_float(scale), words.ctypes.data, words.size, dec.ctypes.data, nat.ctypes.data)
    return dec.view(np.uint16).reshape(-1, 8), nat.view(np.uint16).reshape(-1, 8)


def expected_bits(levels, scale, words):
    codes = np.stack([(words >> (4 * i)) & 0xF for i in range(8)], axis=1).astype(np.int64)
    w32 = levels[codes] * np.float32(scale)
    return O.bf16_rne_bits(w32).reshape(-1, 8)


@pytest.mark.parametrize("scale", [0.0, 1.0, 0.0371, 3.7e-3, 1e-30, 250.0])
def test_lookup_matches_oracle(emul, scale):
    L = O.nf4_levels()
    rng = np.random.Generator(np.random.PCG64(17))
    words = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    # every code in every nibble position
    rep = np.array([sum(c << (4 * i) for i in range(8)) for c in range(16)], dtype=np.uint32)
    words = np.concatenate([rep, words])
    dec, nat = run_lut(emul, L, scale, words)
    exp = expected_bits(L, scale, words)
    assert np.array_equal(nat, exp)
    order = [0, 2, 4, 6, 1, 3, 5, 7]
    assert np.array_equal(dec, exp[:, order])


def test_decode_order_permutation(emul):
    rng = np.random.Generator(np.random.PCG64(3))
    x = rng.integers(0, 2 ** 16, 8 * 100, dtype=np.uint64).astype(np.uint16)
    out = np.zeros_like(x)
    f = emul.decode_order_emul
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    f(x.ctypes.data, 100, out.ctypes.data)
    assert np.array_equal(out.reshape(-1, 8), x.reshape(-1, 8)[:, [0, 2, 4, 6, 1, 3, 5, 7]])


def test_scale_code_unit_is_correctly_rounded(emul):
    """The kernels' 3-instruction k/255 equals the oracle's double-quant
    levels fl32(k/255) for every 8-bit code."""
    out = np.zeros(256, np.float32)
    f = emul.u8_unit_emul
    f.argtypes = [ctypes.c_void_p]
    assert f(out.ctypes.data) == 256
    assert np.array_equal(out.view(np.uint32), O.u8_scale_levels().astype(np.float32).view(np.uint32))


def test_e4m4_unit_matches_oracle_table(emul):
    """The kernels' bit-built float-like scale values equal the oracle's."""
    out = np.zeros(256, np.float32)
    f = emul.e4m4_unit_emul
    f.argtypes = [ctypes.c_void_p]
    assert f(out.ctypes.data) == 256
    assert np.array_equal(out.view(np.uint32), O.e4m4_scale_levels().view(np.uint32))
