"""Benchmark of the QLoRA NF4 linear layer on one MI355X.

Step = one training step of the 7B-shaped layer set (q/k/v/o 4096x4096,
gate/up 11008x4096, down 4096x11008; 2048 tokens; LoRA r=16, alpha=32 on all
seven): forward (H saved) + backward (dX, dA, dB) of every linear, captured in
one HIP graph and replayed. ``value`` is its algorithmic TFLOP/s.

In the same run (reported under "parts"):
  * decode GEMV GB/s at 1/4/16 tokens on 4096x4096 and 11008x4096 (LoRA r=16),
    rotating over > 2 GB of distinct packed copies so the 256 MB
    Infinity Cache cannot serve the weights;
  * dequantize (bf16) and quantize (double quant) GB/s on the same shapes;
  * the fused dequant-GEMM kernels timed per launch with HIP events (base-only
    calls, which launch exactly that kernel) against the bf16 MFMA peak;
  * the CPU oracle on a bounded sample (the "cpu_baseline").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NF4 linear fwd+bwd TFLOP/s and GEMV GB/s (7B-shaped), % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROT_BYTES = 2.2e9  # > 8x the 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemv_bytes(m, n, k, r):
    nk = n * k
    return nk * (0.5 + 1 / 64 + 1 / 4096) + 2 * m * k + 2 * m * n + 2 * r * (k + n)


def fwd_flops(m, n, k, r):
    return 2 * m * n * k + 2 * m * r * (k + n)


def bwd_flops(m, n, k, r):
    # dX = dY W (2mnk) + dH A (2mrk); dH = s dY B (2mnr); dA = dH^T X (2mrk); dB = s dY^T H (2mnr)
    return 2 * m * n * k + 4 * m * r * k + 4 * m * n * r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--counters", action="store_true",
                    help="launch once each, in a fixed order, the kernels whose HBM counters are summarised under "
                         "profiles/ (a 256 MiB copy, quantize, dequantize, decode GEMV), print the order to stderr "
                         "and exit; meant to run under rocprofv3 --pmc")
    ap.add_argument("--only", default="", help="comma list of parts to run (train,f16,dropout,c5,gemm,library,copy,decode,decode_token,dequant,quant,merge,cpu)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    only = set(filter(None, args.only.split(",")))
    want = (lambda p: not only or p in only)

    import numpy as np
    import torch

    import bit_nf4_quantized_18_amd as qn
    import synth

    qn.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    if args.counters:
        counter_sequence(qn, synth, torch, dev)
        return

    wl = synth.LAYERS_7B
    M, R, ALPHA = wl.m, wl.r, wl.alpha
    parts = {}

    # ---------------------------------------------------------------- setup
    log("[bench] quantizing the 7B layer set")
    layers = []
    for lay in wl.layers:
        w = torch.from_numpy(synth.weight(wl, lay)).to(dev)
        q = qn.quantize(w)
        del w
        x = torch.from_numpy(synth.activations(wl, lay)).to(torch.bfloat16).to(dev)
        a = torch.from_numpy(synth.lora_a(wl, lay)).to(torch.bfloat16).to(dev)
        b = torch.from_numpy(synth.lora_b(wl, lay)).to(torch.bfloat16).to(dev)
        dy = torch.from_numpy(synth.grad_output(wl, lay)).to(torch.bfloat16).to(dev)
        nbytes = qn.workspace_bytes(M, lay.n, lay.k, R)
        layers.append(dict(
            lay=lay, q=q, x=x, a=a, b=b, dy=dy,
            y=torch.empty((M, lay.n), dtype=torch.bfloat16, device=dev),
            h=torch.empty((M, R), dtype=torch.float32, device=dev),
            dx=torch.empty((M, lay.k), dtype=torch.bfloat16, device=dev),
            da=torch.empty((R, lay.k), dtype=torch.float32, device=dev),
            db=torch.empty((lay.n, R), dtype=torch.float32, device=dev),
            ws=torch.empty(nbytes, dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()

    def train_step():
        for L in layers:
            qn.linear_fwd(L["q"], L["x"], L["a"], L["b"], ALPHA, out=L["y"], h_out=L["h"], ws=L["ws"])
            qn.linear_bwd(L["q"], L["x"], L["dy"], L["a"], L["b"], ALPHA, h=L["h"], dx=L["dx"], da=L["da"],
                          db=L["db"], ws=L["ws"])

    # Grouped step: the linears that read the same input in the model run as
    # one call over their stacked weight (q/k/v on one X, gate/up on one X).
    byname = {L["lay"].name: L for L in layers}
    groups = []
    for names in (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",)):
        Ls = [byname[nm] for nm in names]
        if len(Ls) == 1:
            groups.append(dict(single=Ls[0]))
            continue
        k = Ls[0]["lay"].k
        parts_n = [L["lay"].n for L in Ls]
        ntot = sum(parts_n)
        w = torch.cat([torch.from_numpy(synth.weight(wl, L["lay"])) for L in Ls], dim=0).to(dev)
        qg = qn.quantize(w)
        del w
        nbytes = qn.grouped_workspace_bytes(M, ntot, k, len(Ls), R)
        groups.append(dict(
            parts=parts_n, q=qg, x=Ls[0]["x"], a=torch.cat([L["a"] for L in Ls]), b=torch.cat([L["b"] for L in Ls]),
            dy=torch.cat([L["dy"] for L in Ls], dim=1),
            y=torch.empty((M, ntot), dtype=torch.bfloat16, device=dev),
            h=torch.empty((M, len(Ls) * R), dtype=torch.float32, device=dev),
            dx=torch.empty((M, k), dtype=torch.bfloat16, device=dev),
            da=torch.empty((len(Ls) * R, k), dtype=torch.float32, device=dev),
            db=torch.empty((ntot, R), dtype=torch.float32, device=dev),
            ws=torch.empty(nbytes, dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()

    def train_step_grouped():
        for G in groups:
            if "single" in G:
                L = G["single"]
                qn.linear_fwd(L["q"], L["x"], L["a"], L["b"], ALPHA, out=L["y"], h_out=L["h"], ws=L["ws"])
                qn.linear_bwd(L["q"], L["x"], L["dy"], L["a"], L["b"], ALPHA, h=L["h"], dx=L["dx"], da=L["da"],
                              db=L["db"], ws=L["ws"])
                continue
            qn.linear_fwd_grouped(G["q"], G["parts"], G["x"], G["a"], G["b"], ALPHA, out=G["y"], h_out=G["h"],
                                  ws=G["ws"])
            qn.linear_bwd_grouped(G["q"], G["parts"], G["x"], G["dy"], G["a"], G["b"], ALPHA, h=G["h"], dx=G["dx"],
                                  da=G["da"], db=G["db"], ws=G["ws"])

    step_fwd = sum(fwd_flops(M, L["lay"].n, L["lay"].k, R) for L in layers)
    step_bwd = sum(bwd_flops(M, L["lay"].n, L["lay"].k, R) for L in layers)
    step_flops = step_fwd + step_bwd

    # ------------------------------------------------------- training step
    def time_step(fn, label):
        log(f"[bench] {label}: capture")
        fn()  # eager warm-up (also loads every kernel)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        log(f"[bench] {label}: timing {args.steps} steps")
        t0 = time.perf_counter()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / args.steps
        tf = step_flops / (ms * 1e-3) / 1e12
        log(f"[bench] {label} {ms:.3f} ms  {tf:.1f} TFLOP/s")
        del g
        return {"ms_per_step": ms, "tflops": tf, "gflop_per_step": step_flops / 1e9,
                "frac_bf16_peak": tf / BF16_PEAK_TFLOPS, "wall_s": wall}

    value = ms_step = None
    if want("train"):
        parts["train_step_per_linear"] = time_step(train_step, "training step, one call per linear")
        parts["train_step"] = time_step(train_step_grouped, "training step (q/k/v and gate/up grouped)")
        ms_step, value = parts["train_step"]["ms_per_step"], parts["train_step"]["tflops"]

    # The same per-linear step with IEEE half as the compute type (fp16 X, A,
    # B, dY; the weight unpacked to half inside the matmuls).
    if want("f16"):
        for L in layers:
            for key in ("x", "a", "b", "dy"):
                L[key + "16"] = L[key].float().to(torch.float16)
            L["y16"] = torch.empty_like(L["y"], dtype=torch.float16)
            L["dx16"] = torch.empty_like(L["dx"], dtype=torch.float16)

        def train_step_f16():
            for L in layers:
                qn.linear_fwd(L["q"], L["x16"], L["a16"], L["b16"], ALPHA, out=L["y16"], h_out=L["h"], ws=L["ws"])
                qn.linear_bwd(L["q"], L["x16"], L["dy16"], L["a16"], L["b16"], ALPHA, h=L["h"], dx=L["dx16"],
                              da=L["da"], db=L["db"], ws=L["ws"])

        parts["train_step_f16"] = time_step(train_step_f16, "training step, fp16 compute, one call per linear")
        for L in layers:
            for key in ("x16", "a16", "b16", "dy16", "y16", "dx16"):
                del L[key]

    # Training step with adapter dropout (p = 0.05, one keep mask per linear
    # drawn on the device each step): the same algorithmic flops plus the mask,
    # the masked copy of X and the masked dX update; every linear its own call.
    if want("dropout"):
        p_drop = 0.05
        mask_off = 0
        for L in layers:
            lay = L["lay"]
            L["keep"] = torch.empty((M, lay.k), dtype=torch.uint8, device=dev)
            L["mask_off"] = mask_off  # disjoint windows of one Philox stream
            mask_off += M * lay.k
            L["wsd"] = torch.empty(qn.dropout_workspace_bytes(M, lay.n, lay.k, R), dtype=torch.uint8, device=dev)

        def train_step_dropout():
            for L in layers:
                qn.dropout_mask(2024, L["mask_off"], (M, L["lay"].k), p_drop, out=L["keep"])
                qn.linear_fwd_dropout(L["q"], L["x"], L["a"], L["b"], ALPHA, L["keep"], p_drop, out=L["y"],
                                      h_out=L["h"], ws=L["wsd"])
                qn.linear_bwd_dropout(L["q"], L["x"], L["dy"], L["a"], L["b"], ALPHA, L["keep"], p_drop, h=L["h"],
                                      dx=L["dx"], da=L["da"], db=L["db"], ws=L["wsd"])

        parts["train_step_dropout"] = time_step(train_step_dropout, "training step with adapter dropout p=0.05")
        parts["train_step_dropout"]["p"] = p_drop
        for L in layers:
            del L["keep"], L["wsd"]

    # ----------------------------------------- 65B-shaped layer set (C5)
    # q/k/v/o 8192x8192, gate/up 22016x8192, down 8192x22016; 4096 tokens;
    # LoRA r=64, alpha=16; Student-t(4) x 0.02 weights. Inputs are drawn on
    # the device from one seeded generator (Student-t(4) as z / sqrt(chi2_4 /
    # 4) from five normals), quantized there, and the fwd+bwd step of the
    # seven linears (gate/up grouped) is captured in one graph and replayed.
    if want("c5"):
        wl5 = synth.LAYERS_65B
        M5, R5, A5 = wl5.m, wl5.r, wl5.alpha
        log("[bench] 65B layer set: drawing and quantizing the weights on the device")
        gen = torch.Generator(device=dev)
        gen.manual_seed(6504)

        def dnormal(shape, std):
            return torch.randn(shape, generator=gen, device=dev) * std

        def dstudent_t4(shape, scale):
            chi2 = torch.zeros(shape, device=dev)
            for _ in range(4):
                chi2.add_(torch.randn(shape, generator=gen, device=dev).square_())
            return torch.randn(shape, generator=gen, device=dev).div_(chi2.div_(4.0).sqrt_()).mul_(scale)

        def pack_cat(qs):
            return qn.PackedNF4(sum(q.n for q in qs), qs[0].k, torch.cat([q.codes for q in qs]), True,
                                torch.cat([q.scale_codes for q in qs]), torch.cat([q.group_scale for q in qs]))

        by5 = {lay.name: lay for lay in wl5.layers}
        x_h = dnormal((M5, 8192), 1.0).to(torch.bfloat16)
        x_f = dnormal((M5, 22016), 1.0).to(torch.bfloat16)
        groups5 = []
        # at r = 64 three stacked adapters would take 192 H slots, beyond the
        # 128 of one call: q, k and v run as single calls
        for names in (("q_proj",), ("k_proj",), ("v_proj",), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",)):
            lays = [by5[nm] for nm in names]
            k5 = lays[0].k
            qs = []
            for lay in lays:
                w = dstudent_t4((lay.n, k5), 0.02)
                qs.append(qn.quantize(w))
                del w
            ntot = sum(lay.n for lay in lays)
            G = dict(parts=[lay.n for lay in lays], q=pack_cat(qs) if len(qs) > 1 else qs[0],
                     x=x_f if k5 == 22016 else x_h,
                     a=dnormal((len(lays) * R5, k5), 1.0 / R5).to(torch.bfloat16),
                     b=dnormal((ntot, R5), 0.01).to(torch.bfloat16),
                     dy=dnormal((M5, ntot), 1.0).to(torch.bfloat16),
                     y=torch.empty((M5, ntot), dtype=torch.bfloat16, device=dev),
                     h=torch.empty((M5, len(lays) * R5), dtype=torch.float32, device=dev),
                     dx=torch.empty((M5, k5), dtype=torch.bfloat16, device=dev),
                     da=torch.empty((len(lays) * R5, k5), dtype=torch.float32, device=dev),
                     db=torch.empty((ntot, R5), dtype=torch.float32, device=dev))
            nbytes = (qn.grouped_workspace_bytes(M5, ntot, k5, len(lays), R5) if len(lays) > 1
                      else qn.workspace_bytes(M5, ntot, k5, R5))
            G["ws"] = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
            groups5.append(G)
            del qs
        torch.cuda.synchronize()

        def step65():
            for G in groups5:
                if len(G["parts"]) == 1:
                    qn.linear_fwd(G["q"], G["x"], G["a"], G["b"], A5, out=G["y"], h_out=G["h"], ws=G["ws"])
                    qn.linear_bwd(G["q"], G["x"], G["dy"], G["a"], G["b"], A5, h=G["h"], dx=G["dx"], da=G["da"],
                                  db=G["db"], ws=G["ws"])
                else:
                    qn.linear_fwd_grouped(G["q"], G["parts"], G["x"], G["a"], G["b"], A5, out=G["y"], h_out=G["h"],
                                          ws=G["ws"])
                    qn.linear_bwd_grouped(G["q"], G["parts"], G["x"], G["dy"], G["a"], G["b"], A5, h=G["h"],
                                          dx=G["dx"], da=G["da"], db=G["db"], ws=G["ws"])

        fl65 = sum(fwd_flops(M5, lay.n, lay.k, R5) + bwd_flops(M5, lay.n, lay.k, R5) for lay in wl5.layers)
        step65()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step65()
        g.replay()
        torch.cuda.synchronize()
        reps65 = 10
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps65):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms65 = e0.elapsed_time(e1) / reps65
        tf65 = fl65 / (ms65 * 1e-3) / 1e12
        parts["train_step_65b"] = {"ms_per_step": ms65, "tflops": tf65, "gflop_per_step": fl65 / 1e9,
                                   "frac_bf16_peak": tf65 / BF16_PEAK_TFLOPS, "replays": reps65,
                                   "workload": "llama65b_layer_set_m4096_r64", "tokens": M5, "lora_r": R5,
                                   "lora_alpha": A5, "weights": "Student-t(4) x 0.02, drawn on the device",
                                   "launches": "gate/up grouped; q, k, v, o and down single"}
        log(f"[bench] 65B layer set fwd+bwd (graph): {ms65:.3f} ms  {tf65:.1f} TFLOP/s "
            f"({100 * tf65 / BF16_PEAK_TFLOPS:.1f}% of bf16 peak)")
        del g, groups5, x_h, x_f
        torch.cuda.empty_cache()

    # ------------------------------------------- fused dequant-GEMM kernels
    roofline = None
    if want("gemm"):
        log("[bench] fused dequant-GEMM kernels, per launch")
        res = {}
        for kind in ("fwd", "dx"):
            tot_flops, tot_ms, per = 0.0, 0.0, []
            for L in layers:
                lay = L["lay"]
                reps = 10
                call = (lambda: qn.linear_fwd(L["q"], L["x"], out=L["y"], ws=L["ws"])) if kind == "fwd" else \
                    (lambda: qn.linear_bwd(L["q"], L["x"], L["dy"], dx=L["dx"], ws=L["ws"]))
                call()
                torch.cuda.synchronize()
                # reps launches captured back to back in one graph, replayed
                # between one pair of events on the kernel's stream: the mean
                # is the kernel's duration plus the graph's dispatch gap, with
                # no host time in between
                gg = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gg, stream=stream):
                    for _ in range(reps):
                        call()
                gg.replay()
                torch.cuda.synchronize()
                s0, s1 = ev(), ev()
                s0.record()
                gg.replay()
                s1.record()
                torch.cuda.synchronize()
                ms = s0.elapsed_time(s1) / reps
                del gg
                fl = 2.0 * M * lay.n * lay.k
                tot_flops += fl
                tot_ms += ms
                per.append({"layer": lay.name, "n": lay.n, "k": lay.k, "ms": ms, "tflops": fl / ms / 1e9})
            ach = tot_flops / tot_ms / 1e9
            res[kind] = {"kernel": f"nf4_gemm_kernel<{'true' if kind == 'dx' else 'false'}, true, false>",
                         "achieved_tflops": ach,
                         "frac": ach / BF16_PEAK_TFLOPS, "avg_launch_ms": tot_ms / len(layers), "per_layer": per}
            log(f"[bench] gemm {kind}: {ach:.1f} TFLOP/s ({100 * ach / BF16_PEAK_TFLOPS:.1f}% of bf16 peak)")
        parts["fused_gemm"] = res
        traffic, traffic_src = measured_traffic()
        roofline = {"bound": "mfma", "achieved": res["fwd"]["achieved_tflops"], "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": res["fwd"]["frac"], "traffic": traffic,
                    "traffic_unit": "bytes per launch (HBM fetch + write, calibrated)", "traffic_source": traffic_src,
                    "kernel": res["fwd"]["kernel"],
                    "per_launch_gflop": step_fwd_base(layers, M) / len(layers) / 1e9,
                    "avg_launch_ms": res["fwd"]["avg_launch_ms"]}

    # Context, not the product: the vendor library's dense bf16 GEMM
    # (torch.matmul -> hipBLASLt) on the same shapes with a bf16 weight that
    # is already dequantized (no NF4 unpack), timed the same way.
    if want("library"):
        lib_res = []
        for L in layers:
            lay = L["lay"]
            wd = qn.dequantize(L["q"], torch.bfloat16)
            for kind, fn in (("fwd", lambda: L["x"] @ wd.t()), ("dx", lambda: L["dy"] @ wd)):
                fn()
                torch.cuda.synchronize()
                pairs = []
                for _ in range(10):
                    s0, s1 = ev(), ev()
                    s0.record()
                    fn()
                    s1.record()
                    pairs.append((s0, s1))
                torch.cuda.synchronize()
                ms = sum(a.elapsed_time(b) for a, b in pairs) / 10
                lib_res.append({"layer": lay.name, "kind": kind, "n": lay.n, "k": lay.k, "ms": ms,
                                "tflops": 2.0 * M * lay.n * lay.k / ms / 1e9})
            del wd
        for kind in ("fwd", "dx"):
            rows = [e for e in lib_res if e["kind"] == kind]
            tf = sum(2.0 * M * e["n"] * e["k"] for e in rows) / sum(e["ms"] for e in rows) / 1e9
            log(f"[bench] library dense bf16 GEMM {kind} (hipBLASLt, weight pre-dequantized): {tf:.1f} TFLOP/s")
        parts["library_dense_bf16_gemm"] = {"note": "torch.matmul on a pre-dequantized bf16 weight, same shapes",
                                            "per_layer": lib_res}

    # ------------------------------------- plain copy (counter calibration)
    if want("copy"):
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 5
        parts["plain_copy"] = {"bytes_read": nbytes, "bytes_written": nbytes, "us": us,
                               "GBps_read_plus_write": 2 * nbytes / (us * 1e-6) / 1e9}
        log(f"[bench] plain 1 GiB device copy: {us:.1f} us  {2 * nbytes / (us * 1e-6) / 1e9:.0f} GB/s (read+write)")
        del src, dst

    # ---------------------------------------------------------- decode GEMV
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]

    def dlay(n, k):
        return next(l for l in synth.DECODE_7B.layers if (l.n, l.k) == (n, k))

    if want("decode"):
        dec = []
        for (n, k) in shapes:
            lay = dlay(n, k)
            w = torch.from_numpy(synth.weight(synth.DECODE_7B, lay))
            q0 = qn.quantize(w.to(dev))
            del w
            per_copy = q0.codes.numel() + q0.scale_codes.numel() + 4 * q0.group_scale.numel()
            copies = int(ROT_BYTES // per_copy) + 1
            log(f"[bench] decode {n}x{k}: {copies} packed copies ({copies * per_copy / 1e9:.2f} GB)")
            pool = [qn.PackedNF4(n, k, q0.codes.clone(), True, q0.scale_codes.clone(), q0.group_scale.clone())
                    for _ in range(copies)]
            a = torch.from_numpy(synth.lora_a(synth.DECODE_7B, lay)).to(torch.bfloat16).to(dev)
            b = torch.from_numpy(synth.lora_b(synth.DECODE_7B, lay)).to(torch.bfloat16).to(dev)
            for m in (1, 2, 4, 16):
                x = torch.from_numpy(synth.activations(synth.DECODE_7B, lay, m)).to(torch.bfloat16).to(dev)
                y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                ws = torch.empty(qn.workspace_bytes(m, n, k, 16), dtype=torch.uint8, device=dev)
                for q in pool[:2]:
                    qn.linear_fwd(q, x, a, b, 32.0, want_h=False, out=y, ws=ws)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for q in pool:
                        qn.linear_fwd(q, x, a, b, 32.0, want_h=False, out=y, ws=ws)
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = ev(), ev()
                reps = 3
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (reps * len(pool))
                byt = gemv_bytes(m, n, k, 16)
                gbs = byt / (us * 1e-6) / 1e9
                dec.append({"n": n, "k": k, "m": m, "us_per_call": us, "bytes": byt, "GBps": gbs,
                            "frac_hbm_peak": gbs / HBM_PEAK_GBS})
                log(f"[bench] decode {n}x{k} m={m}: {us:.2f} us/call  {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
                del g
            # dequantize on the same pool
            if want("dequant"):
                out = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
                nsub = min(len(pool), 64)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for q in pool[:nsub]:
                        qn.binding._check(qn.load().qlora_nf4_dequantize(
                            qn.binding.ctypes.byref(q.c_struct()), 0, qn.binding._ptr(out), qn.binding._stream()),
                            "dequantize")
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = ev(), ev()
                e0.record()
                for _ in range(3):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (3 * nsub)
                byt = n * k * (2.5 + 1 / 64 + 1 / 4096)
                parts.setdefault("dequantize_bf16", []).append(
                    {"n": n, "k": k, "us_per_call": us, "GBps": byt / (us * 1e-6) / 1e9,
                     "frac_hbm_peak": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS})
                log(f"[bench] dequantize {n}x{k}: {us:.2f} us  {byt / (us * 1e-6) / 1e9:.0f} GB/s")
                del g, out
            del pool
            torch.cuda.empty_cache()
        parts["decode_gemv"] = dec

    # One decode token through a 7B-shaped model: 32 distinct copies of the
    # layer set (q/k/v/o, gate/up, down) at m = 1, every linear with its
    # adapter (r = 16), captured as one graph. 3.4 GB of NF4 weights per
    # token, far beyond the 256 MB Infinity Cache. Two launch plans: q/k/v
    # and gate/up as grouped calls on their shared input (4 calls per layer
    # set, the headline), and one call per linear (7 per layer set).
    if want("decode_token"):
        nlayers = 32
        base_q = {}
        for lay in wl.layers:
            key = (lay.n, lay.k)
            if key not in base_q:
                base_q[key] = qn.quantize(torch.from_numpy(synth.weight(wl, lay)).to(dev))
        byname = {lay.name: lay for lay in wl.layers}
        plans = {"grouped": [("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",)],
                 "per_linear": [(lay.name,) for lay in wl.layers]}
        for plan, groups in plans.items():
            model = []
            for li in range(nlayers):
                for grp in groups:
                    lays = [byname[nm] for nm in grp]
                    k = lays[0].k
                    qs = [base_q[(lay.n, lay.k)] for lay in lays]
                    qc = qn.PackedNF4(sum(lay.n for lay in lays), k, torch.cat([q.codes for q in qs]), True,
                                      torch.cat([q.scale_codes for q in qs]), torch.cat([q.group_scale for q in qs]))
                    a = torch.cat([torch.from_numpy(synth.lora_a(wl, lay)) for lay in lays]).to(torch.bfloat16).to(dev)
                    b = torch.cat([torch.from_numpy(synth.lora_b(wl, lay)) for lay in lays]).to(torch.bfloat16).to(dev)
                    x = torch.from_numpy(synth.normal((1, k), 1.0, "decode_token", grp[0])).to(torch.bfloat16).to(dev)
                    y = torch.empty((1, qc.n), dtype=torch.bfloat16, device=dev)
                    parts_n = [lay.n for lay in lays]
                    nbytes = (qn.grouped_workspace_bytes(1, qc.n, k, len(lays), R) if len(lays) > 1
                              else qn.workspace_bytes(1, qc.n, k, R))
                    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
                    # bytes: codes, scales, X, Y, the stacked A (g r x k) and B (n x r)
                    nb = gemv_bytes(1, qc.n, k, R) + 2 * (len(lays) - 1) * R * k
                    model.append((qc, parts_n, x, a, b, y, ws, nb))
            tot_bytes = sum(e[-1] for e in model)
            log(f"[bench] decode token ({plan}): {len(model)} GEMV calls over {tot_bytes / 1e9:.2f} GB")

            def token():
                for q, parts_n, x, a, b, y, ws, _ in model:
                    if len(parts_n) > 1:
                        qn.linear_fwd_grouped(q, parts_n, x, a, b, ALPHA, want_h=False, out=y, ws=ws)
                    else:
                        qn.linear_fwd(q, x, a, b, ALPHA, want_h=False, out=y, ws=ws)

            token()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                token()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            reps = 5
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            gbs = tot_bytes / (ms * 1e-3) / 1e9
            key = "decode_token_7b" if plan == "grouped" else "decode_token_7b_per_linear"
            parts[key] = {"layers": nlayers, "launch_plan": plan, "calls": len(model), "bytes": tot_bytes,
                          "ms_per_token": ms, "tokens_per_s": 1e3 / ms, "GBps": gbs,
                          "frac_hbm_peak": gbs / HBM_PEAK_GBS}
            log(f"[bench] decode token ({plan}, 32 layer sets, m=1, r=16): {ms:.3f} ms  {1e3 / ms:.0f} tokens/s  "
                f"{gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
            del model, g
            torch.cuda.empty_cache()
        del base_q

    if want("quant"):
        qres = []
        for (n, k) in shapes[:2]:
            w = torch.from_numpy(synth.weight(synth.DECODE_7B, dlay(n, k))).to(dev)
            copies = max(2, int(1.2e9 // (4 * n * k)))
            ws_pool = [w.clone() for _ in range(copies)]
            codes = torch.empty(n * k // 2, dtype=torch.uint8, device=dev)
            sc = torch.empty(n * k // 64, dtype=torch.uint8, device=dev)
            gs = torch.empty(-(-(n * k // 64) // 256), dtype=torch.float32, device=dev)
            lib = qn.load()
            P = qn.binding._ptr

            def qcall(src):
                qn.binding._check(lib.qlora_nf4_quantize(P(src), n * k, 1, P(codes), P(sc), P(gs), None,
                                                         qn.binding._stream()), "quantize")
            qcall(ws_pool[0])
            torch.cuda.synchronize()
            # one graph over the pool (distinct sources), replayed: launch
            # gaps are the graph's, not the Python loop's
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for src in ws_pool:
                    qcall(src)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(3):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            del g
            us = e0.elapsed_time(e1) * 1e3 / (3 * len(ws_pool))
            byt = n * k * (4 + 0.5 + 1 / 64 + 1 / 4096)
            qres.append({"n": n, "k": k, "us_per_call": us, "GBps": byt / (us * 1e-6) / 1e9,
                         "weights_per_s": n * k / (us * 1e-6),
                         "frac_hbm_peak": byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS})
            log(f"[bench] quantize {n}x{k}: {us:.2f} us  {byt / (us * 1e-6) / 1e9:.0f} GB/s")
            del ws_pool, w
            torch.cuda.empty_cache()
        parts["quantize_dq"] = qres

    # ------------------------------------------- merge / unmerge / re-quantize
    if want("merge"):
        mres = []
        for (n, k) in shapes[:2]:
            lay = dlay(n, k)
            q = qn.quantize(torch.from_numpy(synth.weight(synth.DECODE_7B, lay)).to(dev))
            a = torch.from_numpy(synth.lora_a(synth.DECODE_7B, lay)).to(torch.bfloat16).to(dev)
            b = (torch.from_numpy(synth.lora_b(synth.DECODE_7B, lay)) + 0.01).to(torch.bfloat16).to(dev)
            o16 = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
            o32 = torch.empty((n, k), dtype=torch.float32, device=dev)
            packed = n * k * (0.5 + 1 / 64 + 1 / 4096)
            calls = {
                "merge_bf16": (lambda: qn.merge(q, a, b, 32.0, torch.bfloat16, out=o16), packed + 2 * n * k),
                "merge_f32": (lambda: qn.merge(q, a, b, 32.0, torch.float32, out=o32), packed + 4 * n * k),
                "unmerge_bf16_in_place": (lambda: qn.unmerge(o16, a, b, 32.0, out=o16), 4 * n * k),
                "requantize_dq": (lambda: qn.requantize(q, a, b, 32.0), 2 * packed + 8 * n * k),
            }
            for name, (fn, byt) in calls.items():
                fn()
                torch.cuda.synchronize()
                reps = 20
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for _ in range(reps):
                        fn()
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = ev(), ev()
                e0.record()
                for _ in range(3):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (3 * reps)
                gbs = byt / (us * 1e-6) / 1e9
                mres.append({"op": name, "n": n, "k": k, "r": 16, "us_per_call": us, "bytes": byt, "GBps": gbs,
                             "frac_hbm_peak": gbs / HBM_PEAK_GBS})
                log(f"[bench] {name} {n}x{k} r=16: {us:.2f} us  {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
                del g
            del q, o16, o32
            torch.cuda.empty_cache()
        parts["merge"] = mres

    # -------------------------------------------------------- CPU baseline
    cpu = None
    if want("cpu") and not args.no_cpu:
        cpu = cpu_baseline(layers, M, R, ALPHA, wl, parts)
        log(f"[bench] cpu oracle: {cpu['value']:.4f} {cpu['unit']} ({cpu['blas_threads']} BLAS threads, "
            f"{cpu['host_cpus']} host CPUs)")
        for name, leg in cpu["legs"].items():
            log(f"[bench] cpu oracle {name}: " + ", ".join(f"{k}={v:.4g}" for k, v in leg.items()
                                                            if isinstance(v, float)))

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama7b_layer_set_fwd_bwd", "layers": "q/k/v/o 4096x4096, gate/up 11008x4096, "
                   "down 4096x11008", "tokens": M, "lora_r": R, "lora_alpha": ALPHA, "nf4_block": 64,
                   "double_quant_block": 256, "global_batch": 4, "seq_len": 512, "parallelism": "none (1 GPU)",
                   "launches": "q/k/v one grouped call on a shared input, gate/up likewise; o and down single"},
        "roofline": roofline, "cpu_baseline": cpu, "parts": parts,
    }
    print(json.dumps(line), flush=True)


def counter_sequence(qn, synth, torch, dev):
    """Setup first (weights quantized, inputs drawn), then exactly one launch
    per line below, in this order and with nothing launched in between, so
    the last dispatches of a counter trace map onto these lines one to one.
    Algorithmic bytes (read, written) are printed with each line."""
    MiB = 1 << 20
    src = torch.ones(256 * MiB, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ops = []
    ops.append(("copy 256 MiB", lambda: dst.copy_(src), 256 * MiB, 256 * MiB))
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]
    layers = {(l.n, l.k): l for l in synth.DECODE_7B.layers}
    packed, w32 = {}, {}
    for (n, k) in shapes:
        w32[(n, k)] = torch.from_numpy(synth.weight(synth.DECODE_7B, layers[(n, k)])).to(dev)
        packed[(n, k)] = qn.quantize(w32[(n, k)])
    scratch_q = {key: (torch.empty(key[0] * key[1] // 2, dtype=torch.uint8, device=dev),
                       torch.empty(key[0] * key[1] // 64, dtype=torch.uint8, device=dev),
                       torch.empty(-(-(key[0] * key[1] // 64) // 256), dtype=torch.float32, device=dev))
                 for key in shapes[:2]}
    lib = qn.load()
    P = qn.binding._ptr
    for (n, k) in shapes[:2]:
        c, sc, gs = scratch_q[(n, k)]

        def qcall(n=n, k=k, c=c, sc=sc, gs=gs):
            qn.binding._check(lib.qlora_nf4_quantize(P(w32[(n, k)]), n * k, 1, P(c), P(sc), P(gs), None,
                                                     qn.binding._stream()), "quantize")
        ops.append((f"quantize {n}x{k}", qcall, 4 * n * k, n * k * (0.5 + 1 / 64 + 1 / 4096)))
    outs = {key: torch.empty(key, dtype=torch.bfloat16, device=dev) for key in shapes[:2]}
    for (n, k) in shapes[:2]:
        def dcall(n=n, k=k):
            qn.binding._check(lib.qlora_nf4_dequantize(qn.binding.ctypes.byref(packed[(n, k)].c_struct()), 0,
                                                       P(outs[(n, k)]), qn.binding._stream()), "dequantize")
        ops.append((f"dequantize bf16 {n}x{k}", dcall, n * k * (0.5 + 1 / 64 + 1 / 4096), 2 * n * k))
    gemv_in = {}
    for (n, k) in shapes:
        lay = layers[(n, k)]
        a = torch.from_numpy(synth.lora_a(synth.DECODE_7B, lay)).to(torch.bfloat16).to(dev)
        b = torch.from_numpy(synth.lora_b(synth.DECODE_7B, lay)).to(torch.bfloat16).to(dev)
        for m in (1, 16):
            x = torch.from_numpy(synth.activations(synth.DECODE_7B, lay, m)).to(torch.bfloat16).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(1, qn.workspace_bytes(m, n, k, 16)), dtype=torch.uint8, device=dev)
            gemv_in[(n, k, m)] = (x, a, b, y, ws)

            def gcall(n=n, k=k, m=m):
                x, a, b, y, ws = gemv_in[(n, k, m)]
                qn.linear_fwd(packed[(n, k)], x, a, b, 32.0, want_h=False, out=y, ws=ws)
            rd = n * k * (0.5 + 1 / 64 + 1 / 4096) + 2 * m * k + 2 * 16 * (k + n)
            ops.append((f"decode GEMV {n}x{k} m={m} r=16", gcall, rd, 2 * m * n))
    torch.cuda.synchronize()
    for name, fn, rd, wr in ops:
        fn()
        log(f"[counters] {name}: algorithmic read {rd:.0f} B, write {wr:.0f} B")
    torch.cuda.synchronize()
    log(f"[counters] {len(ops)} launches")


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "nf4_gemm_fwd_7b_layers_traffic.md")
GEMM_SOURCES = ["gemm_kernels.hip", "nf4_lut.h", "mfma.h", "internal.h"]


def gemm_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "bit_nf4_quantized_18_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the forward fused GEMM from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    (its sha256 is recorded there); otherwise None."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None, "no counter summary"
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            key, _, v = line[2:].partition(": ")
            vals[key.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != gemm_source_hash():
        return None, "kernel source changed since the counters were taken"
    try:
        return float(vals["traffic_bytes_per_launch"]), os.path.relpath(TRAFFIC_FILE, ROOT)
    except (KeyError, ValueError):
        return None, "counter summary unreadable"


def step_fwd_base(layers, M):
    return sum(2.0 * M * L["lay"].n * L["lay"].k for L in layers)


def cpu_threads():
    """(host CPUs this process may run on, threads of the BLAS that numpy uses)."""
    host = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = None
    return host, blas


def timed_passes(fn, min_s, max_passes):
    """Run fn() in whole passes until at least min_s seconds (at most
    max_passes); returns (seconds, passes)."""
    t, n = 0.0, 0
    while n < max_passes and (n == 0 or t < min_s):
        t0 = time.perf_counter()
        fn()
        t += time.perf_counter() - t0
        n += 1
    return t, n


def cpu_baseline(layers, M, R, ALPHA, wl, parts, min_s=10.0, max_passes=24):
    """The oracle, untouched, on bounded samples of the benchmarked work,
    each leg next to the GPU figure it compares with.

    Headline (value): the training step of the 7B layer set -- for every
    linear, the first 2048 weight rows (output features) and all 2048 token
    rows; oracle quantization (once, untimed), then oracle dequantization,
    float64 forward and backward, timed over whole passes until at least
    min_s seconds have run. Scaled to TFLOP/s with the sample's algorithmic
    flops. The legs: quantization of the 11008x4096 decode weight (a row
    sample), the one-token decode forward of the 4096x4096 weight (whole),
    and a sample of the 65B layer set (extrapolated to its full step)."""
    import numpy as np

    import synth
    from oracle import linear as OL
    from oracle import nf4 as O

    host, blas = cpu_threads()
    ms, ns = 2048, 2048
    sample = []
    for L in layers:
        lay = L["lay"]
        w = synth.weight(wl, lay)[:ns]
        sample.append((lay, O.quantize(w.reshape(-1), True),
                       L["x"][:ms].float().cpu().numpy().astype(np.float64),
                       L["dy"][:ms, :ns].float().cpu().numpy().astype(np.float64),
                       L["a"].float().cpu().numpy().astype(np.float64),
                       L["b"][:ns].float().cpu().numpy().astype(np.float64)))
    flops_pass = sum(fwd_flops(ms, ns, lay.k, R) + bwd_flops(ms, ns, lay.k, R) for lay, *_ in sample)

    def train_pass():
        for lay, q, x, dy, a, b in sample:
            _, bits = O.dequantize(q)
            w16 = O.bf16_bits_to_f32(bits).reshape(ns, lay.k)
            OL.linear_fwd(x, w16, a, b, ALPHA, R)
            OL.linear_bwd(x, w16, a, b, dy, ALPHA, R)

    t_total, passes = timed_passes(train_pass, min_s, max_passes)
    flops = flops_pass * passes
    del sample
    legs = {}

    # quantize (double quant) of the 11008x4096 decode weight: 512 of its rows
    lay_up = next(l for l in synth.DECODE_7B.layers if (l.n, l.k) == (11008, 4096))
    wq = synth.weight(synth.DECODE_7B, lay_up)[:512].reshape(-1)
    tq, nq = timed_passes(lambda: O.quantize(wq, True), 2.0, 8)
    gpu_q = next((e for e in parts.get("quantize_dq", []) if (e["n"], e["k"]) == (11008, 4096)), None)
    legs["quantize_11008x4096"] = {
        "oracle_weights_per_s": wq.size * nq / tq, "sample": f"512 of 11008 rows ({wq.size} weights), {nq} pass(es)",
        "gpu_weights_per_s": gpu_q["weights_per_s"] if gpu_q else None}

    # one-token decode forward of the 4096x4096 weight with its adapter
    # (r = 16): oracle dequantization + float64 matvec and LoRA, per call
    lay_at = next(l for l in synth.DECODE_7B.layers if (l.n, l.k) == (4096, 4096))
    q_at = O.quantize(synth.weight(synth.DECODE_7B, lay_at).reshape(-1), True)
    x1 = synth.activations(synth.DECODE_7B, lay_at, 1).astype(np.float64)
    a1 = synth.lora_a(synth.DECODE_7B, lay_at).astype(np.float64)
    b1 = synth.lora_b(synth.DECODE_7B, lay_at).astype(np.float64)

    def gemv_call():
        _, bits = O.dequantize(q_at)
        OL.linear_fwd(x1, O.bf16_bits_to_f32(bits).reshape(4096, 4096), a1, b1, 32.0, 16)

    tg, ng = timed_passes(gemv_call, 2.0, 8)
    gpu_g = next((e for e in parts.get("decode_gemv", []) if (e["n"], e["k"], e["m"]) == (4096, 4096, 1)), None)
    legs["decode_gemv_4096x4096_m1"] = {
        "oracle_us_per_call": tg / ng * 1e6, "sample": f"whole weight, {ng} call(s); quantization untimed",
        "gpu_us_per_call": gpu_g["us_per_call"] if gpu_g else None}

    # 65B layer set, sampled: q_proj (8192 x 8192) with 1024 of its weight
    # rows; forward and dX on 64 token rows, dA and dB on all 4096; the rate
    # is extrapolated to the full fwd+bwd step of the seven linears
    wl5 = synth.LAYERS_65B
    lay5 = wl5.layers[0]
    n5, m5s = 1024, 64
    tag = "cpu_sample_65b"
    q5 = O.quantize(synth.student_t((n5, lay5.k), 4, 0.02, tag, "W").reshape(-1), True)
    x5 = synth.normal((wl5.m, lay5.k), 1.0, tag, "X").astype(np.float64)
    dy5 = synth.normal((wl5.m, n5), 1.0, tag, "dY").astype(np.float64)
    a5 = synth.normal((wl5.r, lay5.k), 1.0 / wl5.r, tag, "A").astype(np.float64)
    b5 = synth.normal((n5, wl5.r), 0.01, tag, "B").astype(np.float64)
    s5 = OL.lora_scale(wl5.alpha, wl5.r)

    def c5_pass():
        _, bits = O.dequantize(q5)
        w16 = O.bf16_bits_to_f32(bits).reshape(n5, lay5.k)
        OL.linear_fwd(x5[:m5s], w16, a5, b5, wl5.alpha, wl5.r)
        OL.linear_bwd(x5[:m5s], w16, a5, b5, dy5[:m5s], wl5.alpha, wl5.r)
        h = x5 @ a5.T
        dh = s5 * (dy5 @ b5)
        _ = dh.T @ x5, s5 * (dy5.T @ h)

    t5, n5p = timed_passes(c5_pass, 2.0, 8)
    # flops of one pass: forward and backward on the sampled token rows, then
    # H, dH, dA and dB on all token rows (dequantization counts none)
    fl5 = (fwd_flops(m5s, n5, lay5.k, wl5.r) + bwd_flops(m5s, n5, lay5.k, wl5.r)
           + 4 * wl5.m * wl5.r * lay5.k + 4 * wl5.m * n5 * wl5.r) * n5p
    rate5 = fl5 / t5
    step5 = sum(fwd_flops(wl5.m, lay.n, lay.k, wl5.r) + bwd_flops(wl5.m, lay.n, lay.k, wl5.r) for lay in wl5.layers)
    gpu5 = parts.get("train_step_65b")
    legs["train_step_65b"] = {
        "oracle_tflops_on_sample": rate5 / 1e12,
        "oracle_step_s_extrapolated": step5 / rate5,
        "extrapolation": True,
        "sample": f"q_proj, {n5} of 8192 weight rows; forward and dX on {m5s} of {wl5.m} token rows, dA and dB "
                  f"on all {wl5.m}; {n5p} pass(es), {fl5 / 1e9:.1f} GFLOP in {t5:.2f} s; the full step's "
                  f"{step5 / 1e12:.2f} TFLOP divided by the sample's rate",
        "gpu_step_s": gpu5["ms_per_step"] * 1e-3 if gpu5 else None}

    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(blas or host), "kind": "oracle",
            "host_cpus": host, "blas_threads": blas,
            "sample": f"7B layer set: per linear the first {ns} weight rows and {ms} of {M} token rows; "
                      f"oracle dequantization + float64 forward and backward timed over {passes} pass(es) "
                      f"({flops / 1e9:.2f} GFLOP in {t_total:.2f} s), oracle quantization untimed",
            "legs": legs}


if __name__ == "__main__":
    main()
