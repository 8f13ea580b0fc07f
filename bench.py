#!/usr/bin/env python3
"""Benchmark of the BitLinear W1.58A8 hot path on one MI355X.

Headline (one JSON line on stdout):
  workload  decode at M=1 through the 30-layer BitNet b1.58 2B4T-shaped linear
            stack (each layer: the 7 projections q,k,v,o,gate,up,down with the
            per-token int8 quantization, subln / ffn_sub_norm RMSNorm and
            ReLU^2(gate)*up between them; attention excluded).  One step = one
            token through all 30 layers.  521 MB of packed weights, so every
            step streams its weights from HBM (no cache residency).
  metric    decode HBM GB/s = algorithmic bytes of one step / step time.
            Algorithmic bytes: packed weights + every BitLinear's input and
            output activations (fp32; bf16 for the first input).
The same line carries the dominant kernel's roofline, the oracle's CPU
baseline, and secondary figures (prefill int8 TOPS, batched decode, the
single-layer decode, ternarization) under "extra".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def layer_bytes(M: int, in_bytes: int, H: int, I: int, KV: int) -> int:
    """Algorithmic HBM bytes of one layer's linear path at M tokens."""
    packed = ((H + 2 * KV) * H + H * H + 2 * I * H + H * I) // 4
    act = (M * H * in_bytes + M * (H + 2 * KV) * 4      # qkv: x in, q|k|v out
           + M * H * 4 + M * H * 4                      # o: q in, o out
           + M * H * 4 + M * I * 4                      # gate|up: h in, p out
           + M * I * 4 + M * H * 4)                     # down: p in, y out
    return packed + act


def layer_ops(M: int, H: int, I: int, KV: int) -> int:
    return 2 * M * ((H + 2 * KV) * H + H * H + 2 * I * H + H * I)


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps      # ms per call

    def per_launch(self, fns, warmup=3):
        """Average duration of single launches, each bracketed by its own events."""
        torch = self.torch
        for f in fns[:warmup]:
            f()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
        for (s, e), f in zip(evs, fns):
            s.record()
            f()
            e.record()
        torch.cuda.synchronize()
        ts = sorted(s.elapsed_time(e) for s, e in evs)
        return sum(ts) / len(ts), ts[len(ts) // 2]


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def cpu_baseline(seconds: float = 12.0):
    """The oracle as it stands, single thread, M=1 layers on two distinct layers' codes."""
    import numpy as np

    import oracle
    from bit_ternary_weight_amd import synth
    H, I, KV = synth.HIDDEN, synth.INTERMEDIATE, synth.KV_DIM
    layers = []
    for l in range(2):
        codes, wms = {}, {}
        for p, _, _ in synth.PROJECTIONS:
            _, wm, c = oracle.ternarize_pack(synth.layer_weight(l, p))
            codes[p], wms[p] = c, wm
        layers.append((codes, wms))
    x = synth.bf16_to_f32(synth.act_outliers_bf16(0, 1, H))
    n = 0
    nbytes = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        codes, wms = layers[n % 2]
        out = oracle.layer(x, codes, wms)
        nbytes += layer_bytes(1, 2 if n == 0 else 4, H, I, KV)
        x = out["y"]
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} single-token (M=1) layer forwards of the 2B4T layer shape, alternating two "
                      f"seeded layers' codes, {dt:.1f} s on one host thread (same bytes accounting as the GPU)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernel-only", action="store_true",
                    help="only the dominant-kernel loop (for profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build has no "
              "multi-GPU path; see the sharding notes in DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_ternary_weight_amd import binding as bl
    from bit_ternary_weight_amd import stack, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H, I, KV = synth.HIDDEN, synth.INTERMEDIATE, synth.KV_DIM
    timer = Timer(torch)
    t_build = time.perf_counter()
    layers = stack.build_layers(args.layers, dev, workers=16)
    log(f"built {args.layers} layers in {time.perf_counter() - t_build:.1f} s")
    packed_total = sum(lw.nbytes_packed() for lw in layers)

    # ---------------------------------------------------------------- dominant kernel
    # decode GEMV over the largest projection group (gate|up, 2 x 6912 outputs,
    # K=2560) on int8 codes, so the launch is that one kernel; weights rotate
    # over the layers so each launch reads them from HBM.
    xq = torch.from_numpy(synth.act_outliers_bf16(1, 1, H).view(np.int16)).to(dev).view(torch.bfloat16)
    q1, a1 = bl.quant_act(xq)
    ygu = torch.empty((1, 2 * I), dtype=torch.float32, device=dev)
    launches = []
    for rep in range(4):
        for lw in layers:
            launches.append(lambda lw=lw: bl.gemv_w2a8(q1, lw.packed_gu, lw.w_gu, seg_n=[I, I], a=a1, y=ygu))
    avg_ms, med_ms = timer.per_launch(launches)
    gu_bytes = 2 * I * H // 4 + H + 2 * I * 4 + 4
    achieved = gu_bytes / (avg_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "k_gemv (decode GEMV, gate|up 2x6912 x 2560, M=1, int8 codes in)",
                "bytes_per_launch": gu_bytes, "avg_launch_us": round(avg_ms * 1e3, 3),
                "median_launch_us": round(med_ms * 1e3, 3)}
    log(f"dominant kernel: {roofline}")
    if args.kernel_only:
        return

    # ---------------------------------------------------------------- headline: M=1 decode, 30 layers
    x1 = torch.from_numpy(synth.act_outliers_bf16(0, 1, H).view(np.int16)).to(dev).view(torch.bfloat16)
    bufs1 = {}
    step_fn = lambda: stack.stack_forward(x1, layers, bufs=bufs1)
    eager_ms = timer.run(step_fn, max(2, args.steps // 4), 1)
    graph = capture(torch, step_fn)
    # a replay must reproduce the eager result bit for bit
    ref = stack.stack_forward(x1, layers, bufs={}).clone()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(bufs1["outs"][(len(layers) - 1) & 1], ref):
        raise RuntimeError("graph replay differs from the eager decode pass")
    ms = timer.run(graph.replay, args.steps, args.warmup)
    step_bytes = layer_bytes(1, 2, H, I, KV) + (len(layers) - 1) * layer_bytes(1, 4, H, I, KV)
    value = step_bytes / (ms * 1e-3) / 1e9
    log(f"decode M=1 x {len(layers)} layers: {ms * 1e3:.1f} us/step (graph), eager {eager_ms * 1e3:.1f} us, "
        f"{value:.1f} GB/s")

    extra = {"decode_m1_eager_us_per_step": round(eager_ms * 1e3, 2),
             "decode_m1_graph_us_per_layer": round(ms * 1e3 / len(layers), 3),
             "packed_weight_bytes": packed_total}

    if not args.no_extras:
        # batched decode (M=16, 64) through the stack
        for M in (16, 64):
            xb = torch.from_numpy(synth.act_heavy_tail_bf16(0, M, H).view(np.int16)).to(dev).view(torch.bfloat16)
            bb = {}
            fn = lambda: stack.stack_forward(xb, layers, bufs=bb)
            g = capture(torch, fn)
            t = timer.run(g.replay, max(5, args.steps // 2), 2)
            by = layer_bytes(M, 2, H, I, KV) + (len(layers) - 1) * layer_bytes(M, 4, H, I, KV)
            extra[f"decode_m{M}_gbs"] = round(by / (t * 1e-3) / 1e9, 1)
            extra[f"decode_m{M}_us_per_step"] = round(t * 1e3, 2)
            del g
        # single layer, MALL-resident (warm) and the kernel-level split per layer
        l0 = layers[:1]
        b0 = {}
        g = capture(torch, lambda: stack.stack_forward(x1, l0, bufs=b0))
        t = timer.run(g.replay, 200, 10)
        extra["decode_m1_one_layer_warm_gbs"] = round(layer_bytes(1, 2, H, I, KV) / (t * 1e-3) / 1e9, 1)
        extra["decode_m1_one_layer_warm_us"] = round(t * 1e3, 2)
        del g
        # prefill GEMM: fused gate|up (2560 -> 2x6912) then down (6912 -> 2560), M=2048
        M = 2048
        xg = torch.from_numpy(synth.act_normal_bf16(0, M, H).view(np.int16)).to(dev).view(torch.bfloat16)
        xd = torch.from_numpy(synth.act_normal_bf16(1, M, I).view(np.int16)).to(dev).view(torch.bfloat16)
        qg, ag = bl.quant_act(xg)
        qd, ad = bl.quant_act(xd)
        yg = torch.empty((M, 2 * I), dtype=torch.float32, device=dev)
        yd = torch.empty((M, H), dtype=torch.float32, device=dev)
        lw = layers[0]
        f_gu = lambda: bl.gemm_w2a8(qg, lw.packed_gu, lw.w_gu, seg_n=[I, I], a=ag, y=yg)
        f_dn = lambda: bl.gemm_w2a8(qd, lw.packed_down, lw.w_down, a=ad, y=yd)
        t_gu = timer.run(f_gu, 20, 3)
        t_dn = timer.run(f_dn, 20, 3)
        ops_gu = 2 * M * 2 * I * H
        ops_dn = 2 * M * H * I
        f_all = lambda: (bl.gemm_w2a8(xg, lw.packed_gu, lw.w_gu, seg_n=[I, I], y=yg),
                         bl.gemm_w2a8(xd, lw.packed_down, lw.w_down, y=yd))
        t_all = timer.run(f_all, 20, 3)
        tops = (ops_gu + ops_dn) / (t_all * 1e-3) / 1e12
        extra["prefill_m2048_ffn_tops"] = round(tops, 1)
        extra["prefill_m2048_ffn_frac_of_int8_peak"] = round(tops / INT8_PEAK_TOPS, 4)
        extra["prefill_m2048_gateup_gemm_tops"] = round(ops_gu / (t_gu * 1e-3) / 1e12, 1)
        extra["prefill_m2048_down_gemm_tops"] = round(ops_dn / (t_dn * 1e-3) / 1e12, 1)
        extra["prefill_m2048_ffn_us"] = round(t_all * 1e3, 1)
        # prefill through the 30-layer stack, M=4096
        M = 4096
        xp = torch.from_numpy(synth.act_normal_bf16(0, M, H).view(np.int16)).to(dev).view(torch.bfloat16)
        bp = {}
        t = timer.run(lambda: stack.stack_forward(xp, layers, bufs=bp), 3, 1)
        ops = layer_ops(M, H, I, KV) * len(layers)
        extra["prefill_m4096_stack_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
        extra["prefill_m4096_stack_frac_of_int8_peak"] = round(ops / (t * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
        extra["prefill_m4096_stack_ms"] = round(t, 2)
        del bp
        # offline ternarization (absmean + pack) of one 6912 x 2560 master
        W = torch.from_numpy(synth.layer_weight(0, "gate")).to(dev)
        pk = torch.empty((I // 4, H), dtype=torch.uint8, device=dev)
        wm = torch.empty(1, dtype=torch.float32, device=dev)
        t = timer.run(lambda: bl.ternarize_pack(W, packed=pk, w_mean=wm), 20, 3)
        extra["ternarize_pack_gbs"] = round((W.numel() * 4 + pk.numel()) / (t * 1e-3) / 1e9, 1)
        del W

    cpu = None if args.no_cpu else cpu_baseline()
    line = {
        "metric": "W1.58A8 BitLinear decode HBM GB/s (M=1 through the 30-layer 2B4T linear stack)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xternary->int32, fp32 scales",
        "data": "synthetic (seeded N(0,0.02) fp32 masters ternarized on the device; bf16 x with 1% x20 outliers)",
        "config": {"workload": f"decode M=1, {len(layers)}-layer BitNet-2B4T linear stack (hidden 2560, "
                               f"intermediate 6912, q/k/v/o/gate/up/down + subln, ReLU^2, ffn_sub_norm), "
                               f"{packed_total} packed weight bytes, HIP graph of one token pass",
                   "M": 1, "layers": len(layers), "bytes_per_step": step_bytes, "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
