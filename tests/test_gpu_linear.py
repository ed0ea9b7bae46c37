"""GPU parity of qlora_linear_fwd / qlora_linear_bwd against the float64
oracle (tolerance: max|gpu - ref| / max|ref| <= 1e-2 per tensor), plus the
invariants that hold exactly on the GPU (B = 0 equals the base-only call,
run-to-run determinism, saved vs recomputed H)."""
import numpy as np
import pytest

import synth
from gpu_cases import TOL, f64, layer_inputs, oracle_weight, rel, say
from oracle import linear as OL

pytestmark = pytest.mark.gpu

# (name, m, n, k, r, alpha, dq)
FWD_BWD_CASES = [
    ("single_256_m16_r8", 16, 256, 256, 8, 16.0, True),         # decode path (m <= 16)
    ("single_256_m17_r8", 17, 256, 256, 8, 16.0, True),         # smallest prefill-path m
    ("m1_r8", 1, 256, 256, 8, 16.0, True),
    ("m4_r16", 4, 512, 320, 16, 32.0, True),
    ("ragged_m300_n272_k320_r8", 300, 272, 320, 8, 16.0, True),  # ragged m, n tail, odd number of k-steps
    ("base_only_m33", 33, 256, 192, 0, 0.0, True),
    ("rank24", 40, 128, 256, 24, 48.0, True),                   # r not a multiple of 32
    ("rank5_unaligned", 40, 128, 256, 5, 10.0, True),           # r % 8 != 0: guarded loads
    ("rank64_alpha16", 64, 256, 512, 64, 16.0, True),            # s = 0.25
    ("rank128", 48, 256, 256, 128, 64.0, True),
    ("no_dq", 96, 384, 448, 16, 32.0, False),
    ("decode_no_dq_m3", 3, 384, 448, 16, 32.0, False),
    ("decode_m16_r0", 16, 256, 256, 0, 0.0, True),
    ("decode_rank5_m2", 2, 96, 192, 5, 10.0, True),              # H inside the GEMV, ragged rank
    ("decode_k8192_r4_m5", 5, 48, 8192, 4, 8.0, True),           # H inside the GEMV, two passes over k
    ("decode_rank24_m8", 8, 128, 256, 24, 48.0, True),           # r > 16: H from the skinny kernel
    ("decode_long_k_m2", 2, 64, 16384, 16, 32.0, True),          # k > 12288 at two tokens: the matrix-core multi-pass GEMV, H fused
    ("decode_rank32_m1", 1, 160, 4096, 32, 64.0, True),          # one token, two fused H tiles, full k
    ("decode_rank20_m2_k2112", 2, 48, 2112, 20, 40.0, True),     # two tokens, ragged k past one 2048 half
    ("decode_xl_m1_k11008_r16", 1, 96, 11008, 16, 32.0, True),   # k > 4096 at one token: X read from LDS per row
    ("decode_xl_m2_k4160_r8", 2, 64, 4160, 8, 16.0, True),       # ragged third half
    ("decode_xl_m2_k12288_r0", 2, 48, 12288, 0, 0.0, True),      # the largest k of that form, base only
    ("decode_xl_m1_k6144_r40_nodq", 1, 80, 6144, 40, 80.0, False),
    # the row-per-wave GEMV at every rows-per-wave count (n / (16 x 256 CUs), rounded up to 1, 2, 3, 4, 6, 8)
    ("decode_rpw2_m1_k320", 1, 8192, 320, 16, 32.0, True),           # two rows per wave, fused H
    ("decode_rpw2_xl_m1_k6144", 1, 8192, 6144, 16, 32.0, True),      # two rows per wave, X from LDS, H partials
    ("decode_rpw4_m2_k256", 2, 16384, 256, 16, 32.0, True),          # four rows per wave, two tokens
    ("decode_rpw8_m1_k256_nodq", 1, 40960, 256, 8, 16.0, False),     # eight rows per wave, 320 workgroups
    # three or four tokens: the matrix-core GEMV
    ("decode_m4_k4096_r32", 4, 160, 4096, 32, 64.0, True),           # r > 16: H from split partials
    ("decode_m3_k2112_r40", 3, 48, 2112, 40, 80.0, True),            # H from partials, ragged k
    ("decode_m4_k256_r0_nodq", 4, 272, 256, 0, 0.0, False),          # base only, one pass
    ("decode_m3_k4160_r16", 3, 64, 4160, 16, 32.0, True),            # fused H, two passes over k
    # several GEMM tiles with ragged tails in m and n, and every remainder of
    # the k-step count modulo the three-stage ring, forward (k / 64 steps)
    # and dX (n / 64 steps)
    ("gemm_ragged_m300_n400_k1024_r16", 300, 400, 1024, 16, 32.0, True),        # 16 and 7 steps
    ("gemm_ragged_m520_n272_k1088_r24_nodq", 520, 272, 1088, 24, 48.0, False),  # 17 and 5 steps
    ("gemm_ragged_m257_n1040_k960_r8", 257, 1040, 960, 8, 16.0, True),          # 15 and 17 steps
]


def _run_case(gpu_lib, name, m, n, k, r, alpha, dq, check_bwd=True, codebook=0):
    import torch

    w, x, a, b, dy = layer_inputs(n, k, m, r, name)
    q_ref, w16 = oracle_weight(w, dq, codebook)
    say(f"[linear] case={name} m={m} n={n} k={k} r={r} dq={dq} codebook={codebook}")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda(), double_quant=dq, codebook=codebook)
    xc, dyc = x.cuda(), dy.cuda()
    ac = a.cuda() if r else None
    bc = b.cuda() if r else None
    y, h = gpu_lib.linear_fwd(q, xc, ac, bc, alpha)
    torch.cuda.synchronize()
    y_ref, h_ref = OL.linear_fwd(f64(x), w16, f64(a) if r else None, f64(b) if r else None, alpha, r)
    ey = rel(f64(y), y_ref)
    say(f"   fwd rel err y={ey:.2e}")
    assert ey <= TOL
    if r:
        eh = rel(f64(h), h_ref)
        assert eh <= TOL, eh
    if not check_bwd:
        return
    dx, da, db = gpu_lib.linear_bwd(q, xc, dyc, ac, bc, alpha, h=h)
    torch.cuda.synchronize()
    dx_ref, da_ref, db_ref = OL.linear_bwd(f64(x), w16, f64(a) if r else None, f64(b) if r else None, f64(dy),
                                           alpha, r)
    edx = rel(f64(dx), dx_ref)
    msg = f"   bwd rel err dx={edx:.2e}"
    assert edx <= TOL, msg
    if r:
        eda, edb = rel(f64(da), da_ref), rel(f64(db), db_ref)
        msg += f" da={eda:.2e} db={edb:.2e}"
        assert eda <= TOL and edb <= TOL, msg
        # H recomputed inside the backward gives the same gradients bit for bit
        dx2, da2, db2 = gpu_lib.linear_bwd(q, xc, dyc, ac, bc, alpha, h=None)
        torch.cuda.synchronize()
        assert rel(f64(da2), da_ref) <= TOL and rel(f64(db2), db_ref) <= TOL
        assert torch.equal(dx2, dx)
    say(msg)


@pytest.mark.parametrize("case", FWD_BWD_CASES, ids=[c[0] for c in FWD_BWD_CASES])
def test_linear_parity(gpu_lib, case):
    _run_case(gpu_lib, *case)


# Weights on the evenly spaced INT4 table: every path (GEMM, GEMV with H
# inside, GEMV with H from the skinny kernel, no double quantization).
INT4_CASES = [
    ("int4_ragged_m300_n272_k320_r8", 300, 272, 320, 8, 16.0, True),
    ("int4_decode_m1_r8", 1, 256, 256, 8, 16.0, True),
    ("int4_decode_rank24_m8", 8, 128, 256, 24, 48.0, True),
    ("int4_decode_k4608_m16", 16, 256, 4608, 16, 32.0, True),   # k > 4096: two passes
    ("int4_no_dq_m96", 96, 384, 448, 16, 32.0, False),
]


@pytest.mark.parametrize("case", INT4_CASES, ids=[c[0] for c in INT4_CASES])
def test_linear_parity_int4(gpu_lib, case):
    _run_case(gpu_lib, *case, codebook=1)


# The float-like 8-bit scale code (double_quant = 2) on every path.
FLOAT8_CASES = [
    ("f8scale_ragged_m300_n272_k320_r8", 300, 272, 320, 8, 16.0, 2),
    ("f8scale_decode_m1_r8", 1, 256, 256, 8, 16.0, 2),
    ("f8scale_decode_long_k_m2", 2, 64, 16384, 16, 32.0, 2),
]


@pytest.mark.parametrize("case", FLOAT8_CASES, ids=[c[0] for c in FLOAT8_CASES])
def test_linear_parity_float8_scales(gpu_lib, case):
    _run_case(gpu_lib, *case)


@pytest.mark.parametrize("m", [1, 4, 16])
@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_decode_7b_shapes(gpu_lib, m, n, k):
    """The decode (GEMV) path at the 7B layer shapes, forward only (k = 11008:
    the multi-pass form, three passes, the last one partial)."""
    _run_case(gpu_lib, f"decode_{n}x{k}_m{m}", m, n, k, 16, 32.0, True, check_bwd=False)


@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_7b_layer_full(gpu_lib, n, k):
    """A full 2048-token 7B-shaped layer, forward and backward, checked on
    every output element."""
    _run_case(gpu_lib, f"layer7b_{n}x{k}", 2048, n, k, 16, 32.0, True)


@pytest.mark.parametrize("proj,n,k", [("q", 8192, 8192), ("down", 8192, 22016), ("gate", 22016, 8192)],
                         ids=["q_k_v_o_8192x8192", "down_8192x22016", "gate_up_22016x8192"])
def test_65b_layer_sampled(gpu_lib, proj, n, k):
    """The 65B-shaped layer set at its training size (4096 tokens, r = 64,
    alpha = 16, Student-t(4) weights scaled by 0.02): the 8192 x 8192 shape of
    q/k/v/o, down (8192 x 22016: the longest k) and gate/up (22016 x 8192).
    dA and dB are checked in full, Y and dX on 64 sampled token rows."""
    import torch

    m, r, alpha = 4096, 64, 16.0
    tag = f"layer65b_{proj}"
    w = synth.student_t((n, k), 4, 0.02, tag, "W")
    from gpu_cases import to_bf16
    x = to_bf16(synth.normal((m, k), 1.0, tag, "X"))
    a = to_bf16(synth.normal((r, k), 1.0 / r, tag, "A"))
    b = to_bf16(synth.normal((n, r), 0.01, tag, "B"))
    dy = to_bf16(synth.normal((m, n), 1.0, tag, "dY"))
    say(f"[linear] case={tag} quantize")
    _, w16 = oracle_weight(w, True)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    del w
    xc, ac, bc, dyc = x.cuda(), a.cuda(), b.cuda(), dy.cuda()
    say(f"[linear] case={tag} fwd")
    y, h = gpu_lib.linear_fwd(q, xc, ac, bc, alpha)
    say(f"[linear] case={tag} bwd")
    dx, da, db = gpu_lib.linear_bwd(q, xc, dyc, ac, bc, alpha, h=h)
    torch.cuda.synchronize()
    rows = np.random.Generator(np.random.PCG64(5)).choice(m, 64, replace=False)
    xs, dys = f64(x)[rows], f64(dy)[rows]
    a64, b64 = f64(a), f64(b)
    y_ref, _ = OL.linear_fwd(xs, w16, a64, b64, alpha, r)
    dx_ref, _, _ = OL.linear_bwd(xs, w16, a64, b64, dys, alpha, r)
    ey, edx = rel(f64(y)[rows], y_ref), rel(f64(dx)[rows], dx_ref)
    s = OL.lora_scale(alpha, r)
    x64 = f64(x)
    h_ref = x64 @ a64.T
    dh_ref = s * (f64(dy) @ b64)
    da_ref = dh_ref.T @ x64
    db_ref = s * (f64(dy).T @ h_ref)
    eda, edb = rel(f64(da), da_ref), rel(f64(db), db_ref)
    say(f"   rel err y={ey:.2e} dx={edx:.2e} da={eda:.2e} db={edb:.2e}")
    assert max(ey, edx, eda, edb) <= TOL


def test_b_zero_equals_base_only(gpu_lib):
    """B = 0 (the LoRA init) gives exactly the base-only output, on both paths."""
    import torch

    for m in (8, 200):
        w, x, a, b, dy = layer_inputs(256, 320, m, 16, f"bzero{m}")
        say(f"[linear] B=0 m={m}")
        q = gpu_lib.quantize(torch.from_numpy(w).cuda())
        xc = x.cuda()
        y0, _ = gpu_lib.linear_fwd(q, xc)
        y1, _ = gpu_lib.linear_fwd(q, xc, a.cuda(), torch.zeros_like(b).cuda(), 32.0)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)
        _, da, db = gpu_lib.linear_bwd(q, xc, dy.cuda(), a.cuda(), torch.zeros_like(b).cuda(), 32.0)
        torch.cuda.synchronize()
        assert torch.count_nonzero(da).item() == 0 and torch.count_nonzero(db).item() > 0


def test_run_twice_bit_equal(gpu_lib):
    import torch

    w, x, a, b, dy = layer_inputs(512, 512, 600, 16, "det")
    say("[linear] determinism")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    args = (x.cuda(), a.cuda(), b.cuda())
    y1, h1 = gpu_lib.linear_fwd(q, *args, 32.0)
    y2, h2 = gpu_lib.linear_fwd(q, *args, 32.0)
    g1 = gpu_lib.linear_bwd(q, args[0], dy.cuda(), args[1], args[2], 32.0, h=h1)
    g2 = gpu_lib.linear_bwd(q, args[0], dy.cuda(), args[1], args[2], 32.0, h=h1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    for u, v in zip(g1, g2):
        assert torch.equal(u, v)


def test_empty_batch(gpu_lib):
    """m = 0: the forward is a no-op; the backward writes zero dA and dB."""
    import torch

    w, x, a, b, dy = layer_inputs(128, 128, 4, 8, "empty")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    say("[linear] m=0")
    x0 = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dy0 = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    y, h = gpu_lib.linear_fwd(q, x0, a.cuda(), b.cuda(), 16.0)
    assert y.shape == (0, 128)
    dx, da, db = gpu_lib.linear_bwd(q, x0, dy0, a.cuda(), b.cuda(), 16.0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(da).item() == 0 and torch.count_nonzero(db).item() == 0


def test_fused_gemm_matches_dequantize_then_matmul(gpu_lib):
    """The fused kernel's base product equals an fp32 matmul of the separately
    dequantized bf16 weight (a check of the in-loop dequantization)."""
    import torch

    w, x, _, _, _ = layer_inputs(1024, 1024, 512, 0, "fusedvsdeq")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    xc = x.cuda()
    say("[linear] fused vs dequantize+matmul")
    y, _ = gpu_lib.linear_fwd(q, xc)
    w16 = gpu_lib.dequantize(q, torch.bfloat16)
    ref = xc.float() @ w16.float().t()
    torch.cuda.synchronize()
    assert rel(f64(y), f64(ref)) <= 4e-3


@pytest.mark.parametrize("m,k,r", [(4, 320, 16), (300, 320, 16), (4, 4608, 32), (1, 4096, 16), (2, 8192, 16)],
                         ids=["gemv_fused_h", "gemm", "gemv_multipass_split_h", "gemv_rows_fused_h",
                              "gemv_rows_x_lds_split_h"])
def test_graph_replay_matches_eager(gpu_lib, m, k, r):
    """Forward + backward captured in a HIP graph: every replay (with eager
    work and synchronisation in between, outputs and workspace overwritten)
    reproduces the eager results."""
    import torch

    n = 256
    w, x, a, b, dy = layer_inputs(n, k, m, r, f"graph{m}_{k}_{r}")
    say(f"[linear] graph replay m={m} k={k} r={r}")
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    xc, ac, bc, dyc = x.cuda(), a.cuda(), b.cuda(), dy.cuda()
    ws = torch.empty(gpu_lib.workspace_bytes(m, n, k, r), dtype=torch.uint8, device="cuda")
    bufs = dict(y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                h=torch.empty((m, r), dtype=torch.float32, device="cuda"),
                dx=torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
                da=torch.empty((r, k), dtype=torch.float32, device="cuda"),
                db=torch.empty((n, r), dtype=torch.float32, device="cuda"))

    def step():
        gpu_lib.linear_fwd(q, xc, ac, bc, 32.0, out=bufs["y"], h_out=bufs["h"], ws=ws)
        gpu_lib.linear_bwd(q, xc, dyc, ac, bc, 32.0, h=bufs["h"], dx=bufs["dx"], da=bufs["da"], db=bufs["db"], ws=ws)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        eager = {key: v.clone() for key, v in bufs.items()}
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        for rep in range(3):
            for v in bufs.values():
                v.fill_(7)  # eager work between replays
            ws.fill_(0xA5)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for key in bufs:
                assert torch.equal(bufs[key], eager[key]), (rep, key)


def _random_cases(count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for c in range(count):
        m = int(rng.choice([1, 2, 5, 16, 17, 33, 64, 130, 257]))
        n = 16 * int(rng.integers(1, 30))
        k = 64 * int(rng.integers(1, 11))
        r = int(rng.choice([0, 1, 3, 8, 16, 17, 31, 32, 48, 64, 65, 96]))
        alpha = float(rng.choice([1.0, 8.0, 16.0, 32.0]))
        dq = bool(rng.integers(0, 2))
        cases.append((f"rand{c}_m{m}_n{n}_k{k}_r{r}_dq{int(dq)}", m, n, k, r, alpha, dq))
    return cases


RANDOM_CASES = _random_cases(24, 2026)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_linear_parity_random_shapes(gpu_lib, case):
    """Seeded random shapes across both paths: m from 1 to 257, n and k on
    their 16 / 64 grids, ranks from 0 to 96 (ragged and tile-aligned), DQ on
    and off."""
    _run_case(gpu_lib, *case)
