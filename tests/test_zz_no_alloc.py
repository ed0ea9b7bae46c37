"""qlora_linear_fwd_noalloc (the forward on the library's own scratch array,
for callers that cannot allocate) against qlora_linear_fwd with a caller
workspace: the same kernels, so Y and H must be bit-identical; also within the
1e-2 bar of the float64 oracle. Calls run back to back on one stream, each
later one smaller than the one before, so the shared array holds the previous
call's contents when the next one starts."""
import ctypes

import numpy as np
import pytest

from gpu_cases import TOL, f64, layer_inputs, oracle_weight, rel, say
from oracle import linear as OL

pytestmark = pytest.mark.gpu

# (name, m, n, k, r, alpha): matmul path with a large scratch use first, then
# a smaller matmul-path call, then decode calls whose H partial sums live in
# the scratch array (r > 16; one token at k > 4096)
CASES = [
    ("noalloc_m300_n272_k320_r16", 300, 272, 320, 16, 32.0),
    ("noalloc_m40_n128_k256_r24", 40, 128, 256, 24, 48.0),
    ("noalloc_decode_m1_n96_k6144_r16", 1, 96, 6144, 16, 32.0),
    ("noalloc_decode_m8_n128_k256_r24", 8, 128, 256, 24, 48.0),
]


def test_noalloc_matches_workspace_call(gpu_lib):
    import torch

    for name, m, n, k, r, alpha in CASES:
        say(f"[noalloc] case={name} m={m} n={n} k={k} r={r}")
        w, x, a, b, _ = layer_inputs(n, k, m, r, name)
        _, w16 = oracle_weight(w, True)
        q = gpu_lib.quantize(torch.from_numpy(w).cuda())
        xc, ac, bc = x.cuda(), a.cuda(), b.cuda()
        y_ws, h_ws = gpu_lib.linear_fwd(q, xc, ac, bc, alpha)
        h_na = torch.empty((m, r), dtype=torch.float32, device="cuda")
        y_na, _ = gpu_lib.linear_fwd_noalloc(q, xc, ac, bc, alpha, h_out=h_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), name
        assert torch.equal(h_na, h_ws), name
        y_ref, h_ref = OL.linear_fwd(f64(x), w16, f64(a), f64(b), alpha, r)
        ey, eh = rel(f64(y_na), y_ref), rel(f64(h_na), h_ref)
        say(f"   bit-equal to the workspace call; rel err y={ey:.2e} h={eh:.2e}")
        assert ey <= TOL and eh <= TOL


def test_noalloc_rejects_sizes_beyond_the_array(gpu_lib):
    import torch

    lib = gpu_lib.load()
    n, k = 256, 256
    w, _, _, _, _ = layer_inputs(n, k, 1, 0, "noalloc_limit")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    wc = q.c_struct()
    x = torch.zeros((16, k), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((16, n), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((128, k), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((n, 128), dtype=torch.bfloat16, device="cuda")
    # m = 2^20 tokens at r = 128 needs far more than 16 MiB of scratch: the
    # host check refuses it before anything is enqueued
    st = lib.qlora_linear_fwd_noalloc(ctypes.byref(wc), ctypes.c_void_p(x.data_ptr()), 1 << 20,
                                      ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), 128, 16.0,
                                      ctypes.c_void_p(y.data_ptr()), None,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -5
    assert np.all(y.cpu().float().numpy() == 0.0)
