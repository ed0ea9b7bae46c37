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


def sample_rows(parts):
    """About 30 weight rows of a (stacked) weight: every part's first and last
    row and evenly spaced ones between, so that the sampled outputs' largest
    magnitude is typical of the layer even at one token."""
    n = sum(parts)
    edges = np.cumsum([0] + list(parts))
    rows = set(np.linspace(0, n - 1, 24).astype(int).tolist())
    for l in range(len(parts)):
        rows.update((int(edges[l]), int(edges[l + 1]) - 1))
    return sorted(rows)


def _build(gpu_lib, M, R):
    """The grouped 7B calls (q/k/v, o, gate/up, down) at M tokens, with their
    inputs, output buffers and workspaces, from the benchmark's seeded data."""
    import torch

    wl = synth.LAYERS_7B
    dev = "cuda"
    byname = {lay.name: lay for lay in wl.layers}
    bf = torch.bfloat16

    def t16(a):
        return torch.from_numpy(a).to(bf).to(dev)

    calls = []
    for names in GROUPS:
        lays = [byname[nm] for nm in names]
        k = lays[0].k
        w = np.concatenate([synth.weight(wl, lay) for lay in lays], axis=0)
        n = w.shape[0]
        g = len(lays)
        c = dict(names=names, parts=[lay.n for lay in lays],
                 rows=sample_rows([lay.n for lay in lays]),
                 q=gpu_lib.quantize(torch.from_numpy(w).to(dev)),
                 x=t16(synth.activations(wl, lays[0], M)),
                 a=torch.cat([t16(synth.lora_a(wl, lay)) for lay in lays]),
                 b=torch.cat([t16(synth.lora_b(wl, lay)) for lay in lays]),
                 dy=torch.cat([t16(synth.grad_output(wl, lay, M)) for lay in lays], dim=1))
        c["w_rows"] = [group_slice(w, row) for row in c["rows"]]
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
    return calls


def _step(gpu_lib, calls, alpha, bwd):
    for c in calls:
        o = c["out"]
        if len(c["parts"]) == 1:
            gpu_lib.linear_fwd(c["q"], c["x"], c["a"], c["b"], alpha, out=o["y"], h_out=o["h"], ws=c["ws"])
            if bwd:
                gpu_lib.linear_bwd(c["q"], c["x"], c["dy"], c["a"], c["b"], alpha, h=o["h"], dx=o["dx"],
                                   da=o["da"], db=o["db"], ws=c["ws"])
        else:
            gpu_lib.linear_fwd_grouped(c["q"], c["parts"], c["x"], c["a"], c["b"], alpha, out=o["y"],
                                       h_out=o["h"], ws=c["ws"])
            if bwd:
                gpu_lib.linear_bwd_grouped(c["q"], c["parts"], c["x"], c["dy"], c["a"], c["b"], alpha, h=o["h"],
                                           dx=o["dx"], da=o["da"], db=o["db"], ws=c["ws"])


def _graph_equals_eager(calls, step, keys):
    """Eager run, then one graph of the same calls replayed three times with
    outputs and workspaces overwritten in between: every replay equals the
    eager run bit for bit."""
    import torch

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        eager = [{key: c["out"][key].clone() for key in keys} for c in calls]
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
                for key in keys:
                    assert torch.equal(c["out"][key], e[key]), (rep, c["names"], key)


def _check_sampled_y(calls, M, R, alpha):
    """The sampled weight rows' output columns of each call against the
    oracle (a row of part l takes slots l R .. (l + 1) R - 1 of H)."""
    s_lora = OL.lora_scale(alpha, R)
    for c in calls:
        k = c["x"].shape[1]
        x64 = f64(c["x"])
        a64, b64 = f64(c["a"]), f64(c["b"])
        edges = np.cumsum([0] + c["parts"])
        ref = np.empty((M, len(c["rows"])))
        for j, (row, (sl, off)) in enumerate(zip(c["rows"], c["w_rows"])):
            w16 = O.bf16_bits_to_f32(O.dequantize(O.quantize(sl, True))[1])[off:off + k].astype(np.float64)
            part = int(np.searchsorted(edges, row, side="right")) - 1
            h = x64 @ a64[part * R:(part + 1) * R].T
            ref[:, j] = x64 @ w16 + s_lora * (h @ b64[row])
        e = rel(f64(c["out"]["y"])[:, c["rows"]], ref)
        say(f"[step] m={M} {'/'.join(c['names'])}: rel err of {len(c['rows'])} sampled Y columns {e:.2e}")
        assert e <= TOL


def test_7b_grouped_step_graph(gpu_lib):
    wl = synth.LAYERS_7B
    M, R, ALPHA = wl.m, wl.r, wl.alpha
    say("[step] build the grouped 7B training step")
    calls = _build(gpu_lib, M, R)
    _graph_equals_eager(calls, lambda: _step(gpu_lib, calls, ALPHA, True), ("y", "h", "dx", "da", "db"))
    _check_sampled_y(calls, M, R, ALPHA)


@pytest.mark.parametrize("m", [1, 2])
def test_7b_grouped_decode_graph(gpu_lib, m):
    """One layer set of the decode token: the four grouped forward calls at
    one or two tokens (the row-per-wave GEMV, H inside or from the
    projection) as one graph."""
    wl = synth.LAYERS_7B
    R, ALPHA = wl.r, wl.alpha
    say(f"[step] build the grouped 7B decode calls, m={m}")
    calls = _build(gpu_lib, m, R)
    _graph_equals_eager(calls, lambda: _step(gpu_lib, calls, ALPHA, False), ("y", "h"))
    _check_sampled_y(calls, m, R, ALPHA)
