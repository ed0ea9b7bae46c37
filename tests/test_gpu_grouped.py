"""GPU parity of the grouped linear calls (q/k/v or gate/up over one stacked
weight) against the oracle run part by part: Y and H per part, dX summed over
the parts, dA and dB per part (tolerance: max|gpu - ref| / max|ref| <= 1e-2)."""
import numpy as np
import pytest

import synth
from gpu_cases import TOL, f64, oracle_weight, oracle_weight_f16, rel, say, to_bf16, to_f16
from oracle import linear as OL

pytestmark = pytest.mark.gpu

# (name, m, parts, k, r, alpha)
CASES = [
    ("qkv_ragged_m300", 300, (256, 512, 256), 320, 16, 32.0),  # ragged m, odd number of k-steps
    ("gateup_m17", 17, (512, 256), 192, 16, 16.0),             # smallest m on the GEMM path
    ("qkv_r32", 64, (256, 256, 256), 256, 32, 64.0),           # g r = 96: the general projection
    ("four_parts_m40", 40, (256, 256, 256, 256), 128, 16, 32.0),
    ("qkv_m260_k1088", 260, (256, 512, 512), 1088, 16, 32.0),  # 17 forward and 20 dX steps, ragged m
]

# Decode sizes (m <= 16, the GEMV): H in the kernel when g r <= 16, else from
# split partial sums; k <= 4096 takes the persistent form, larger k the
# multi-pass one. The backward needs r % 16 == 0, so r = 4 cases check the
# forward only.
DECODE_CASES = [
    ("qkv_decode_m1", 1, (256, 512, 256), 320, 4, 32.0),
    ("four_parts_decode_m5", 5, (256, 256, 256, 256), 192, 4, 16.0),
    ("gateup_decode_m16_k4160", 16, (512, 256), 4160, 16, 32.0),
    ("qkv_decode_r32_m7", 7, (256, 256, 256), 256, 32, 64.0),
    ("qkv_decode_r4_m3_k4608", 3, (256, 256, 512), 4608, 4, 8.0),
    ("qkv_decode_r7_m2", 2, (256, 512, 256), 320, 7, 14.0),  # g r = 21: split partials, padded to 32 slots
    ("gateup_decode_m1_k6208", 1, (512, 256), 6208, 16, 32.0),    # one token, k > 4096: X from LDS, H partials
    ("qkv_decode_m2_k8192", 2, (256, 256, 256), 8192, 8, 16.0),
    ("qkv_decode_m4", 4, (256, 512, 256), 320, 16, 32.0),          # four tokens: g r = 48, H from split partials
    ("gateup_decode_m3_r24", 3, (512, 256), 448, 24, 48.0),
]


def run_case(gpu_lib, name, m, parts, k, r, alpha, check_bwd=True, f16=False):
    import torch

    tag = f"grouped_{name}"
    say(f"[grouped] case={name} m={m} parts={parts} k={k} r={r} f16={f16}")
    cv = to_f16 if f16 else to_bf16
    ws = [synth.normal((n, k), 0.02, tag, f"W{l}") for l, n in enumerate(parts)]
    x = cv(synth.normal((m, k), 1.0, tag, "X"))
    a = [cv(synth.normal((r, k), 1.0 / r, tag, f"A{l}")) for l in range(len(parts))]
    b = [cv(synth.normal((n, r), 0.01, tag, f"B{l}")) for l, n in enumerate(parts)]
    dy = [cv(synth.normal((m, n), 1.0, tag, f"dY{l}")) for l, n in enumerate(parts)]
    q = gpu_lib.quantize(torch.from_numpy(np.concatenate(ws, axis=0)).cuda())
    xc, ac, bc = x.cuda(), torch.cat(a).cuda(), torch.cat(b).cuda()
    y, h = gpu_lib.linear_fwd_grouped(q, parts, xc, ac, bc, alpha)
    if check_bwd:
        dx, da, db = gpu_lib.linear_bwd_grouped(q, parts, xc, torch.cat(dy, dim=1).cuda(), ac, bc, alpha, h=h)
    torch.cuda.synchronize()
    off, dx_ref, errs = 0, None, []
    x64 = f64(x)
    for l, n in enumerate(parts):
        w16 = oracle_weight_f16(ws[l], True) if f16 else oracle_weight(ws[l], True)[1]
        y_ref, h_ref = OL.linear_fwd(x64, w16, f64(a[l]), f64(b[l]), alpha, r)
        errs.append(("y", l, rel(f64(y)[:, off:off + n], y_ref)))
        errs.append(("h", l, rel(f64(h)[:, l * r:(l + 1) * r], h_ref)))
        if check_bwd:
            dxl, dal, dbl = OL.linear_bwd(x64, w16, f64(a[l]), f64(b[l]), f64(dy[l]), alpha, r)
            dx_ref = dxl if dx_ref is None else dx_ref + dxl
            errs.append(("da", l, rel(f64(da)[l * r:(l + 1) * r], dal)))
            errs.append(("db", l, rel(f64(db)[off:off + n], dbl)))
        off += n
    if check_bwd:
        errs.append(("dx", -1, rel(f64(dx), dx_ref)))
    worst = max(errs, key=lambda e: e[2])
    say(f"   worst rel err {worst[0]}[{worst[1]}] = {worst[2]:.2e}")
    assert all(e[2] <= TOL for e in errs), errs


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_parity(gpu_lib, case):
    run_case(gpu_lib, *case)


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_grouped_parity_decode(gpu_lib, case):
    run_case(gpu_lib, *case, check_bwd=case[4] % 16 == 0)


F16_CASES = CASES[:2] + DECODE_CASES[2:3]


@pytest.mark.parametrize("case", F16_CASES, ids=[c[0] for c in F16_CASES])
def test_grouped_parity_f16(gpu_lib, case):
    """The grouped calls with fp16 compute (qlora_linear_*_grouped_f16)."""
    run_case(gpu_lib, *case, f16=True)


@pytest.mark.parametrize("parts", [(4096, 4096, 4096), (11008, 11008)], ids=["qkv_7b", "gateup_7b"])
def test_grouped_7b_layers(gpu_lib, parts):
    """The 7B block's grouped projections at 2048 tokens, every output element."""
    run_case(gpu_lib, f"7b_{len(parts)}", 2048, parts, 4096, 16, 32.0)


@pytest.mark.parametrize("m", [1, 2])
@pytest.mark.parametrize("parts", [(4096, 4096, 4096), (11008, 11008)], ids=["qkv_7b", "gateup_7b"])
def test_grouped_7b_decode(gpu_lib, parts, m):
    """The 7B q/k/v and gate/up groups at one and two tokens: the row-per-wave
    GEMV with 48 and 96 rows per workgroup, so the workgroups at the part
    boundaries hold rows of two parts and form both parts' H slots."""
    run_case(gpu_lib, f"7b_decode_{len(parts)}_m{m}", m, parts, 4096, 16, 32.0)


@pytest.mark.parametrize("m", [96, 3], ids=["gemm_m96", "gemv_m3"])
def test_grouped_equals_separate_calls(gpu_lib, m):
    """One part of a grouped call and the single-linear call on that part's
    own packed weight give the same Y within float32 accumulation order."""
    import torch

    parts, k, r, alpha = (256, 512), 256, 16, 32.0
    ws = [synth.normal((n, k), 0.02, "grouped_sep", f"W{l}") for l, n in enumerate(parts)]
    x = to_bf16(synth.normal((m, k), 1.0, "grouped_sep", "X")).cuda()
    a = [to_bf16(synth.normal((r, k), 1.0 / r, "grouped_sep", f"A{l}")).cuda() for l in range(2)]
    b = [to_bf16(synth.normal((n, r), 0.01, "grouped_sep", f"B{l}")).cuda() for l, n in enumerate(parts)]
    qg = gpu_lib.quantize(torch.from_numpy(np.concatenate(ws, axis=0)).cuda())
    yg, _ = gpu_lib.linear_fwd_grouped(qg, parts, x, torch.cat(a), torch.cat(b), alpha)
    q1 = gpu_lib.quantize(torch.from_numpy(ws[1]).cuda())
    y1, _ = gpu_lib.linear_fwd(q1, x, a[1], b[1], alpha)
    torch.cuda.synchronize()
    assert rel(f64(yg)[:, parts[0]:], f64(y1)) <= 1e-3


@pytest.mark.parametrize("m", [96, 3], ids=["gemm_m96", "gemv_m3"])
def test_grouped_graph_replay_matches_eager(gpu_lib, m):
    """Grouped forward + backward captured in a HIP graph: every replay
    reproduces the eager results bit for bit, with the outputs and the
    workspace overwritten between replays (m = 3: the decode GEMV with H from
    split partials in the workspace)."""
    import torch

    parts, k, r = (256, 256, 256), 256, 16
    tag = f"grouped_graph_m{m}"
    w = np.concatenate([synth.normal((n, k), 0.02, tag, f"W{l}") for l, n in enumerate(parts)], axis=0)
    q = gpu_lib.quantize(torch.from_numpy(w).cuda())
    x = to_bf16(synth.normal((m, k), 1.0, tag, "X")).cuda()
    a = to_bf16(synth.normal((3 * r, k), 1.0 / r, tag, "A")).cuda()
    b = to_bf16(synth.normal((sum(parts), r), 0.01, tag, "B")).cuda()
    dy = to_bf16(synth.normal((m, sum(parts)), 1.0, tag, "dY")).cuda()
    say("[grouped] graph replay")
    ws = torch.empty(gpu_lib.grouped_workspace_bytes(m, sum(parts), k, 3, r), dtype=torch.uint8, device="cuda")
    bufs = dict(y=torch.empty((m, sum(parts)), dtype=torch.bfloat16, device="cuda"),
                h=torch.empty((m, 3 * r), dtype=torch.float32, device="cuda"),
                dx=torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
                da=torch.empty((3 * r, k), dtype=torch.float32, device="cuda"),
                db=torch.empty((sum(parts), r), dtype=torch.float32, device="cuda"))

    def step():
        gpu_lib.linear_fwd_grouped(q, parts, x, a, b, 32.0, out=bufs["y"], h_out=bufs["h"], ws=ws)
        gpu_lib.linear_bwd_grouped(q, parts, x, dy, a, b, 32.0, h=bufs["h"], dx=bufs["dx"], da=bufs["da"],
                                   db=bufs["db"], ws=ws)

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
            ws.fill_(0xA5)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for key in bufs:
                assert torch.equal(bufs[key], eager[key]), (rep, key)
