"""The timed training step, at its full size and in its launch form.

The 7B layer set at 2048 tokens, r = 16: q/k/v as one grouped call on their
shared input, o single, gate/up grouped, down single, forward then backward
of each, captured in one HIP graph as the benchmark times it. Every replay
(outputs and workspaces overwritten in between) must equal the eager run bit
for bit, and sampled output columns of the graph's result must match the
oracle within the parity bound."""
import numpy as np
import pytest

import synth
from gpu_cases import TOL, f64, rel, say
from oracle import linear as OL
from oracle import nf4 as O

pytestmark = pytest.mark.gpu

GROUPS = (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",))


def group_slice(w, row):
    """The whole double-quantization groups (256 blocks of 64 consecutive
    weights of the row-major weight) that hold weight row ``row``, and the
    row's offset in them: the oracle quantizes these so that the row's group
    maxima are the device's."""
    n, k = w.shape
    gsz = 256 * 64
    g0, g1 = row * k // gsz, ((row + 1) * k - 1) // gsz
    flat = w.reshape(-1)
    return flat[g0 * gsz:min((g1 + 1) * gsz, n * k)].copy(), row * k - g0 * gsz


def test_7b_grouped_step_graph(gpu_lib):
    import torch

    wl = synth.LAYERS_7B
    M, R, ALPHA = wl.m, wl.r, wl.alpha
    dev = "cuda"
    byname = {lay.name: lay for lay in wl.layers}
    bf = torch.bfloat16

    def t16(a):
        return torch.from_numpy(a).to(bf).to(dev)

    say("[step] build the grouped 7B step")
    calls = []
    for names in GROUPS:
        lays = [byname[nm] for nm in names]
        k = lays[0].k
        w = np.concatenate([synth.weight(wl, lay) for lay in lays], axis=0)
        n = w.shape[0]
        g = len(lays)
        c = dict(names=names, parts=[lay.n for lay in lays], w_rows=[group_slice(w, row) for row in (0, n - 1)],
                 q=gpu_lib.quantize(torch.from_numpy(w).to(dev)),
                 x=t16(synth.activations(wl, lays[0])),
                 a=torch.cat([t16(synth.lora_a(wl, lay)) for lay in lays]),
                 b=torch.cat([t16(synth.lora_b(wl, lay)) for lay in lays]),
                 dy=torch.cat([t16(synth.grad_output(wl, lay)) for lay in lays], dim=1))
        del w
        ws_bytes = (gpu_lib.grouped_workspace_bytes(M, n, k, g, R) if g > 1 else gpu_lib.workspace_bytes(M, n, k, R))
        c["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        c["out"] = dict(y=torch.empty((M, n), dtype=bf, device=dev),
                        h=torch.empty((M, g * R), dtype=torch.float32, device=dev),
                        dx=torch.empty((M, k), dtype=bf, device=dev),
                        da=torch.empty((g * R, k), dtype=torch.float32, device=dev),
                        db=torch.empty((n, R), dtype=torch.float32, device=dev))
        calls.append(c)
    torch.cuda.synchronize()

    def step():
        for c in calls:
            o = c["out"]
            if len(c["parts"]) == 1:
                gpu_lib.linear_fwd(c["q"], c["x"], c["a"], c["b"], ALPHA, out=o["y"], h_out=o["h"], ws=c["ws"])
                gpu_lib.linear_bwd(c["q"], c["x"], c["dy"], c["a"], c["b"], ALPHA, h=o["h"], dx=o["dx"],
                                   da=o["da"], db=o["db"], ws=c["ws"])
            else:
                gpu_lib.linear_fwd_grouped(c["q"], c["parts"], c["x"], c["a"], c["b"], ALPHA, out=o["y"],
                                           h_out=o["h"], ws=c["ws"])
                gpu_lib.linear_bwd_grouped(c["q"], c["parts"], c["x"], c["dy"], c["a"], c["b"], ALPHA, h=o["h"],
                                           dx=o["dx"], da=o["da"], db=o["db"], ws=c["ws"])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        eager = [{key: v.clone() for key, v in c["out"].items()} for c in calls]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step()
        for rep in range(3):
            for c in calls:
                for v in c["out"].values():
                    v.fill_(3)
                c["ws"].fill_(0x5A)
            torch.cuda.synchronize()
            say(f"[step] replay {rep}")
            graph.replay()
            torch.cuda.synchronize()
            for c, e in zip(calls, eager):
                for key, v in c["out"].items():
                    assert torch.equal(v, e[key]), (rep, c["names"], key)

    # the graph's Y against the oracle on each call's first and last weight row
    # (the last row lies in the last part of a grouped call)
    s_lora = OL.lora_scale(ALPHA, R)
    for c in calls:
        n = c["out"]["y"].shape[1]
        cols = [0, n - 1]
        k = c["x"].shape[1]
        w16 = np.stack([O.bf16_bits_to_f32(O.dequantize(O.quantize(sl, True))[1])[off:off + k]
                        for sl, off in c["w_rows"]])
        x64 = f64(c["x"])
        a64, b64 = f64(c["a"]), f64(c["b"])
        # row 0 belongs to part 0 (A rows 0..R-1), row n-1 to the last part
        g = len(c["parts"])
        ref = np.empty((M, 2))
        for j, (col, part) in enumerate(zip(cols, (0, g - 1))):
            h = x64 @ a64[part * R:(part + 1) * R].T
            ref[:, j] = x64 @ w16[j].astype(np.float64) + s_lora * (h @ b64[col])
        e = rel(f64(c["out"]["y"])[:, cols], ref)
        say(f"[step] {'/'.join(c['names'])}: rel err of sampled Y columns {e:.2e}")
        assert e <= TOL
