"""GPU parity of qlora_linear_fwd_dropout / qlora_linear_bwd_dropout against
the float64 oracle with the same explicit keep mask (tolerance as for the
plain layer: max|gpu - ref| / max|ref| <= 1e-2 per tensor), plus the exact
relations to the plain call (keep everything with p = 0; drop everything)."""
import numpy as np
import pytest

import synth
from gpu_cases import TOL, f64, layer_inputs, oracle_weight, rel, say
from oracle import dropout as OD

pytestmark = pytest.mark.gpu

# (name, m, n, k, r, alpha, p)
CASES = [
    ("ragged_m300_n272_k320_r8_p0.1", 300, 272, 320, 8, 16.0, 0.1),
    ("m17_r16_p0.05", 17, 256, 256, 16, 32.0, 0.05),
    ("m1_r8_p0.05", 1, 256, 256, 8, 16.0, 0.05),
    ("rank5_p0.1", 40, 128, 256, 5, 10.0, 0.1),          # rank gradients without the fused kernel
    ("rank64_p0.5", 64, 256, 512, 64, 16.0, 0.5),
    ("attn_4096x4096_m2048_r16_p0.05", 2048, 4096, 4096, 16, 32.0, 0.05),
]


def _inputs(gpu_lib, name, m, n, k, r, p):
    import torch

    w, x, a, b, dy = layer_inputs(n, k, m, r, "drop_" + name)
    keep = synth.keep_mask((m, k), p, "drop_" + name, "keep")
    _, w16 = oracle_weight(w, True)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    return q, w16, x, a, b, dy, keep


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dropout_parity(gpu_lib, case):
    import torch

    name, m, n, k, r, alpha, p = case
    say(f"[dropout] case={name} m={m} n={n} k={k} r={r} p={p}")
    q, w16, x, a, b, dy, keep = _inputs(gpu_lib, name, m, n, k, r, p)
    xc, dyc, ac, bc = x.cuda(), dy.cuda(), a.cuda(), b.cuda()
    kc = torch.from_numpy(keep).cuda()
    y, h = gpu_lib.linear_fwd_dropout(q, xc, ac, bc, alpha, kc, p)
    torch.cuda.synchronize()
    y_ref, h_ref = OD.linear_fwd_dropout(f64(x), w16, f64(a), f64(b), alpha, r, keep, p)
    ey, eh = rel(f64(y), y_ref), rel(f64(h), h_ref)
    say(f"   fwd rel err y={ey:.2e} h={eh:.2e}")
    assert ey <= TOL and eh <= TOL
    dx, da, db = gpu_lib.linear_bwd_dropout(q, xc, dyc, ac, bc, alpha, kc, p, h=h)
    torch.cuda.synchronize()
    dx_ref, da_ref, db_ref = OD.linear_bwd_dropout(f64(x), w16, f64(a), f64(b), f64(dy), alpha, r, keep, p)
    edx, eda, edb = rel(f64(dx), dx_ref), rel(f64(da), da_ref), rel(f64(db), db_ref)
    say(f"   bwd rel err dx={edx:.2e} da={eda:.2e} db={edb:.2e}")
    assert edx <= TOL and eda <= TOL and edb <= TOL
    # H recomputed from the mask inside the backward gives the same results
    dx2, da2, db2 = gpu_lib.linear_bwd_dropout(q, xc, dyc, ac, bc, alpha, kc, p, h=None)
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx) and torch.equal(da2, da) and torch.equal(db2, db)


@pytest.mark.parametrize("case", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_dropout_parity_f16(gpu_lib, case):
    """The dropout calls with fp16 compute (qlora_linear_*_dropout_f16)."""
    import torch

    from gpu_cases import oracle_weight_f16, to_f16

    name, m, n, k, r, alpha, p = case
    say(f"[dropout f16] case={name}")
    tag = "dropf16_" + name
    w = synth.normal((n, k), 0.02, tag, "W")
    x, a, b, dy = (to_f16(synth.normal(sh, sd, tag, nm)) for sh, sd, nm in
                   (((m, k), 1.0, "X"), ((r, k), 1.0 / r, "A"), ((n, r), 0.01, "B"), ((m, n), 1.0, "dY")))
    keep = synth.keep_mask((m, k), p, tag, "keep")
    w16 = oracle_weight_f16(w, True)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    xc, dyc, ac, bc, kc = x.cuda(), dy.cuda(), a.cuda(), b.cuda(), torch.from_numpy(keep).cuda()
    y, h = gpu_lib.linear_fwd_dropout(q, xc, ac, bc, alpha, kc, p)
    dx, da, db = gpu_lib.linear_bwd_dropout(q, xc, dyc, ac, bc, alpha, kc, p, h=h)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16 and dx.dtype == torch.float16
    y_ref, h_ref = OD.linear_fwd_dropout(f64(x), w16, f64(a), f64(b), alpha, r, keep, p)
    dx_ref, da_ref, db_ref = OD.linear_bwd_dropout(f64(x), w16, f64(a), f64(b), f64(dy), alpha, r, keep, p)
    errs = [rel(f64(y), y_ref), rel(f64(h), h_ref), rel(f64(dx), dx_ref), rel(f64(da), da_ref), rel(f64(db), db_ref)]
    say("   rel errs " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= TOL


def test_keep_all_p0_matches_plain_call(gpu_lib):
    """Keeping every element with p = 0: the forward and dA, dB are the plain
    call's bit for bit (same kernels on the same values); dX takes another
    route (frozen GEMM, then the adapter term) and agrees within tolerance."""
    import torch

    m, n, k, r, alpha = 96, 256, 512, 16, 32.0
    q, w16, x, a, b, dy, _ = _inputs(gpu_lib, "keep_all", m, n, k, r, 0.0)
    xc, dyc, ac, bc = x.cuda(), dy.cuda(), a.cuda(), b.cuda()
    kc = torch.ones((m, k), dtype=torch.uint8, device="cuda")
    say("[dropout] keep all, p = 0, vs the plain call")
    y, h = gpu_lib.linear_fwd_dropout(q, xc, ac, bc, alpha, kc, 0.0)
    y0, h0 = gpu_lib.linear_fwd(q, xc, ac, bc, alpha)
    dx, da, db = gpu_lib.linear_bwd_dropout(q, xc, dyc, ac, bc, alpha, kc, 0.0, h=h)
    dx0, da0, db0 = gpu_lib.linear_bwd(q, xc, dyc, ac, bc, alpha, h=h0)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(h, h0)
    assert torch.equal(da, da0) and torch.equal(db, db0)
    assert rel(f64(dx), f64(dx0)) <= TOL


def test_drop_all_leaves_frozen_path(gpu_lib):
    """Dropping every element: H = 0, Y = the base-only call's output, dA = 0,
    dB = 0, and dX = the base-only call's dX (bit for bit: the adapter term
    adds exact zeros)."""
    import torch

    m, n, k, r, alpha = 64, 256, 256, 8, 16.0
    q, w16, x, a, b, dy, _ = _inputs(gpu_lib, "drop_all", m, n, k, r, 0.5)
    xc, dyc, ac, bc = x.cuda(), dy.cuda(), a.cuda(), b.cuda()
    kc = torch.zeros((m, k), dtype=torch.uint8, device="cuda")
    say("[dropout] drop all")
    y, h = gpu_lib.linear_fwd_dropout(q, xc, ac, bc, alpha, kc, 0.5)
    y0, _ = gpu_lib.linear_fwd(q, xc)
    dx, da, db = gpu_lib.linear_bwd_dropout(q, xc, dyc, ac, bc, alpha, kc, 0.5, h=h)
    dx0, _, _ = gpu_lib.linear_bwd(q, xc, dyc)
    torch.cuda.synchronize()
    assert not torch.any(h) and not torch.any(da) and not torch.any(db)
    assert torch.equal(y, y0) and torch.equal(dx, dx0)


@pytest.mark.parametrize("seed,offset,count,p", [
    (0, 0, 2048 * 4096, 0.05),          # one 7B activation tile's mask
    (12345, 16 * 7, 1000 + 37, 0.1),    # ragged tail
    (2**64 - 1, 2**40, 16, 0.5),
    (7, 0, 5, 0.999),
    (7, 32, 4096, 0.0),
])
def test_dropout_mask_bit_exact(gpu_lib, seed, offset, count, p):
    """Keep masks drawn on the GPU equal the oracle's Philox4x64-10 masks."""
    import torch

    from oracle import philox as OP

    say(f"[dropout mask] seed={seed} offset={offset} count={count} p={p}")
    got = gpu_lib.dropout_mask(seed, offset, (count,), p)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), OP.keep_mask(seed, offset, count, p))


def test_dropout_step_with_generated_mask(gpu_lib):
    """A layer step whose mask is drawn on the device: parity with the oracle
    given the oracle's mask for the same (seed, offset)."""
    import torch

    from oracle import philox as OP

    m, n, k, r, alpha, p = 300, 256, 320, 16, 32.0, 0.1
    q, w16, x, a, b, dy, _ = _inputs(gpu_lib, "gen_mask", m, n, k, r, p)
    say("[dropout] step with a device-drawn mask")
    kc = gpu_lib.dropout_mask(42, 16 * 1000, (m, k), p)
    keep = OP.keep_mask(42, 16 * 1000, m * k, p).reshape(m, k)
    xc, dyc, ac, bc = x.cuda(), dy.cuda(), a.cuda(), b.cuda()
    y, h = gpu_lib.linear_fwd_dropout(q, xc, ac, bc, alpha, kc, p)
    dx, da, db = gpu_lib.linear_bwd_dropout(q, xc, dyc, ac, bc, alpha, kc, p, h=h)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), keep)
    y_ref, _ = OD.linear_fwd_dropout(f64(x), w16, f64(a), f64(b), alpha, r, keep, p)
    dx_ref, da_ref, db_ref = OD.linear_bwd_dropout(f64(x), w16, f64(a), f64(b), f64(dy), alpha, r, keep, p)
    assert max(rel(f64(y), y_ref), rel(f64(dx), dx_ref), rel(f64(da), da_ref), rel(f64(db), db_ref)) <= TOL


def test_dropout_step_graph_replay_matches_eager(gpu_lib):
    """Mask drawing + dropout forward + backward captured in a HIP graph: every
    replay, with eager work and synchronisation in between, reproduces the
    eager results bit for bit (the bench times this step as a graph)."""
    import torch

    m, n, k, r, alpha, p = 300, 256, 320, 16, 32.0, 0.1
    q, w16, x, a, b, dy, _ = _inputs(gpu_lib, "graph_drop", m, n, k, r, p)
    xc, dyc, ac, bc = x.cuda(), dy.cuda(), a.cuda(), b.cuda()
    say("[dropout] graph replay")
    ws = torch.empty(gpu_lib.dropout_workspace_bytes(m, n, k, r), dtype=torch.uint8, device="cuda")
    bufs = dict(keep=torch.empty((m, k), dtype=torch.uint8, device="cuda"),
                y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                h=torch.empty((m, r), dtype=torch.float32, device="cuda"),
                dx=torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
                da=torch.empty((r, k), dtype=torch.float32, device="cuda"),
                db=torch.empty((n, r), dtype=torch.float32, device="cuda"))

    def step():
        gpu_lib.dropout_mask(5, 16 * 64, (m, k), p, out=bufs["keep"])
        gpu_lib.linear_fwd_dropout(q, xc, ac, bc, alpha, bufs["keep"], p, out=bufs["y"], h_out=bufs["h"], ws=ws)
        gpu_lib.linear_bwd_dropout(q, xc, dyc, ac, bc, alpha, bufs["keep"], p, h=bufs["h"], dx=bufs["dx"],
                                   da=bufs["da"], db=bufs["db"], ws=ws)

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
                v.fill_(7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for key in bufs:
                assert torch.equal(bufs[key], eager[key]), (rep, key)
