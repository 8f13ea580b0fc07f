#!/usr/bin/env python3
"""Benchmark of the BitLinear W1.58A8 hot path on one MI355X.

Headline (one JSON line on stdout):
  workload  decode GEMV at M=1 over the 7 projections of one BitNet b1.58
            2B4T-shaped layer (q/o 2560->2560, k/v 2560->640, gate/up
            2560->6912, down 6912->2560), each projection with its own bf16
            activations (N(0,1), 1% x20 outliers), quantized per token inside
            the kernel.  One step = the 7 projections of one layer in one
            batched launch.  Consecutive steps walk through 30 distinct seeded
            layers (521 MB of packed weights, twice the 256 MB Infinity
            Cache), so every step streams its weights from HBM.
  metric    decode HBM GB/s = algorithmic bytes of one step / step time, with
            algorithmic bytes = packed weights + bf16 inputs + fp32 outputs.
The same line carries the kernel's roofline, the oracle's CPU baseline, and
secondary figures under "extra": the chained 30-layer decode (quantize ->
q|k|v -> o -> RMSNorm -> gate|up -> ReLU^2 -> RMSNorm -> down per layer),
batched decode at M=16 and M=64, decode attention over a 4096-token cache and
the whole decode step with attention, prefill int8 TOPS, the prefill with
attention and the prefill attention alone, the straight-through backward of
quantization-aware training, ternarization.

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

    def trials(self, fn, min_trials=5, min_total_ms=50.0, max_trials=2000):
        """Times whole calls of fn (each one timed region between two events)
        until at least min_trials calls and min_total_ms of timed work; returns
        (median ms per call, number of calls timed)."""
        torch = self.torch
        times = []
        total = 0.0
        while len(times) < max_trials and (len(times) < min_trials or total < min_total_ms):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            t = s.elapsed_time(e)
            times.append(t)
            total += t
        times.sort()
        return times[len(times) // 2], len(times)

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


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_gemv_v1_decode_m1_7proj_traffic.md")
TRAFFIC_SOURCES = ("bit_ternary_weight_amd/csrc/k_gemv.hip", "bit_ternary_weight_amd/csrc/bl_common.h")


def profiled_traffic():
    """HBM bytes per launch of the headline kernel from the committed
    FETCH_SIZE/WRITE_SIZE summary, or None when the kernel sources have
    changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    h = re.search(r"^source_sha256: ([0-9a-f]+)$", text, re.M)
    if not t or not h:
        return None
    d = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        d.update(open(os.path.join(ROOT, f), "rb").read())
    return int(t.group(1)) if d.hexdigest() == h.group(1) else None


TRACE_PROFILE = os.path.join(ROOT, "profiles", "k_gemv_v1_decode_m1_7proj_kernel_trace.md")


def profiled_duration_us():
    """Average duration of the headline kernel in the committed rocprofv3
    kernel trace of this command, or None when the kernel sources have
    changed since it was taken."""
    import hashlib
    import re
    try:
        text = open(TRACE_PROFILE).read()
    except OSError:
        return None
    t = re.search(r"^headline_kernel_avg_us: ([0-9.]+)$", text, re.M)
    h = re.search(r"^source_sha256: ([0-9a-f]+)$", text, re.M)
    if not t or not h:
        return None
    d = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        d.update(open(os.path.join(ROOT, f), "rb").read())
    return float(t.group(1)) if d.hexdigest() == h.group(1) else None


def cpu_baseline():
    """The oracle as it stands (plain single-threaded C), pinned to one host
    core, on bounded samples of each workload; tokens are independent after
    ternarization, so a row sample's rate is the workload's rate.  Returns the
    cpu_baseline object: the headline (M=1, 7 projections of a layer) in
    GB/s, the other workloads under per_workload."""
    import numpy as np

    import oracle
    from bit_ternary_weight_amd import synth
    H, I, KV = synth.HIDDEN, synth.INTERMEDIATE, synth.KV_DIM
    try:
        allowed = os.sched_getaffinity(0)
        core = min(allowed)
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        allowed, core = None, None
    try:
        layers = []
        for l in range(2):
            codes, wms = {}, {}
            for p, _, _ in synth.PROJECTIONS:
                _, wm, c = oracle.ternarize_pack(synth.layer_weight(l, p))
                codes[p], wms[p] = c, wm
            layers.append((codes, wms))

        def seven(M, kind, reps):
            """M tokens through the 7 projections, each with its own input."""
            xs = {}
            for j, (p, N, K) in enumerate(synth.PROJECTIONS):
                b = synth.act_heavy_tail_bf16(100 + j, M, K) if kind == "heavy" else synth.act_outliers_bf16(100 + j, M, K)
                xs[p] = synth.bf16_to_f32(b)
            t0 = time.perf_counter()
            for r in range(reps):
                codes, wms = layers[r % 2]
                for p, N, K in synth.PROJECTIONS:
                    oracle.bitlinear(xs[p], codes[p], None, wms[p])
            dt = time.perf_counter() - t0
            nbytes = reps * sum(N * K // 4 + M * K * 2 + M * N * 4 for _, N, K in synth.PROJECTIONS)
            return nbytes / dt / 1e9, dt

        out = {}
        W1, x1 = synth.bitlinear_m4_k256_n256()
        t0 = time.perf_counter()
        for _ in range(20):
            _, wm1, c1 = oracle.ternarize_pack(W1)
            oracle.bitlinear(x1, c1, None, wm1)
        t1 = (time.perf_counter() - t0) / 20
        out["bitlinear_m4_k256_n256_us_per_forward"] = round(t1 * 1e6, 1)
        g2, t2 = seven(1, "outliers", 40)
        out["decode_m1_7proj_gbs"] = round(g2, 4)
        g16, t16 = seven(16, "heavy", 2)
        out["decode_m16_7proj_gbs"] = round(g16, 4)
        g64, t64 = seven(64, "heavy", 1)
        out["decode_m64_7proj_gbs"] = round(g64, 4)
        # the M=2048 FFN prefill (gate|up then down) on 128 of its 2048 rows
        rows4 = 128
        codes, wms = layers[0]
        cgu = np.concatenate([codes["gate"], codes["up"]])
        wgu = np.array([wms["gate"], wms["up"]], np.float32)
        xg = synth.bf16_to_f32(synth.act_normal_bf16(0, rows4, H))
        xd = synth.bf16_to_f32(synth.act_normal_bf16(1, rows4, I))
        t0 = time.perf_counter()
        oracle.bitlinear(xg, cgu, [I, I], wgu)
        oracle.bitlinear(xd, codes["down"], None, wms["down"])
        t4 = time.perf_counter() - t0
        out["prefill_m2048_ffn_tops"] = round(2 * rows4 * (2 * I * H + H * I) / t4 / 1e12, 6)
        # the 30-layer stack: the chained decode (two layers' codes
        # alternating) and the prefill on 12 of 4096 rows through 30 layers
        x = synth.bf16_to_f32(synth.act_outliers_bf16(0, 1, H))
        t0 = time.perf_counter()
        for l in range(30):
            codes, wms = layers[l % 2]
            x = oracle.layer(x, codes, wms)["y"]
        t5d = time.perf_counter() - t0
        out["chained_decode_30layers_m1_gbs"] = round((layer_bytes(1, 2, H, I, KV) + 29 * layer_bytes(1, 4, H, I, KV))
                                             / t5d / 1e9, 4)
        rows5 = 12
        x = synth.bf16_to_f32(synth.act_normal_bf16(0, rows5, H))
        t0 = time.perf_counter()
        for l in range(30):
            codes, wms = layers[l % 2]
            x = oracle.layer(x, codes, wms)["y"]
        t5p = time.perf_counter() - t0
        out["prefill_m4096_30layers_tops"] = round(30 * layer_ops(rows5, H, I, KV) / t5p / 1e12, 6)
        total = t2 + t16 + t64 + t4 + t5d + t5p
    finally:
        if allowed is not None:
            os.sched_setaffinity(0, allowed)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": out["decode_m1_7proj_gbs"], "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": (f"oracle (gcc {' '.join(oracle.CFLAGS[:4])}), one thread pinned to core {core}: "
                       f"the M=4, K=256, N=256 BitLinear in full (ternarize + forward, 20 times), the M=1 decode of a layer's 7 projections in full (40 single-token passes, two seeded layers' "
                       f"codes alternating), the batched decode in full (M=16 twice, M=64 once), the M=2048 FFN prefill on {rows4} of "
                       f"2048 rows, the 30-layer chained decode in full, the 30-layer M=4096 prefill on {rows5} of 4096 "
                       f"rows through 30 layers; rates scale with the rows (tokens are independent); "
                       f"{total:.1f} s of CPU work"),
            "per_workload": out, "cpu_model": model, "host_cpus": os.cpu_count(),
            "flags": " ".join(oracle.CFLAGS)}


def q1_disagreement_count(W, m) -> int:
    """Weights whose ternary code differs between the two readings of the
    weight quantization ("Transformers 实战 BitNet 1.58 位量化", section
    "BitLinear 的三步量化"): W / m rounded half to even, against W * fl(1/m),
    both in fp32 and clamped to [-1, 1].  They differ only where |W| / m lies
    within about an ulp of 0.5 (m = 0.023221396, W one ulp above m / 2: the
    quotient rounds to 0.50000006, code 1; the product to 0.5, code 0)."""
    import numpy as np
    W = np.asarray(W, np.float32)
    m = np.float32(m)
    a = np.clip(np.rint(W / m), -1, 1)
    b = np.clip(np.rint(W * (np.float32(1.0) / m)), -1, 1)
    return int(np.count_nonzero(a != b))


def absmean_f32(W) -> "np.float32":
    """mean |W| with an fp64 sum, floored at 1e-5, rounded to fp32."""
    import numpy as np
    return np.float32(max(float(np.abs(W).astype(np.float64).sum()) / W.size, 1e-5))


ATTN_CTX = 4096


def attn_bytes(S: int, H: int, KV: int) -> int:
    """Algorithmic bytes of one decode attention call for the token at
    position S - 1: the cached key and value rows read, q, k, v in, the
    appended rows and the output written (fp32)."""
    return 2 * KV * (S - 1) * 4 + (H + 2 * KV) * 4 + 2 * KV * 4 + H * 4


def attn_decode_timing(torch, bl, stack, timer, dev, n_layers, H, KV, keep=False):
    """Decode attention for the token at position 4095 over n_layers layers'
    fp32 caches (N(0,1)), replayed from a graph; returns (ms per layer, GB/s)
    and, with keep, the caches."""
    S = ATTN_CTX
    cache = stack.alloc_kv(n_layers, S, dev)
    gen = torch.Generator(device=dev).manual_seed(5)
    for kc, vc in zip(cache.k, cache.v):
        kc.normal_(generator=gen)
        vc.normal_(generator=gen)
    qa = torch.randn(H, generator=gen, device=dev)
    ka = torch.randn(KV, generator=gen, device=dev)
    va = torch.randn(KV, generator=gen, device=dev)
    oa = torch.empty(H, device=dev)
    g = capture(torch, lambda: [bl.attn_decode(qa, ka, va, S - 1, kc, vc, cache.rope_cos, cache.rope_sin,
                                               stack.N_HEADS, stack.N_KV_HEADS, out=oa)
                                for kc, vc in zip(cache.k, cache.v)])
    t = timer.run(g.replay, 5, 1) / n_layers
    del g
    gbs = round(attn_bytes(S, H, KV) / (t * 1e-3) / 1e9, 1)
    return (t, gbs, cache) if keep else (t, gbs)


def attn_prefill_timing(torch, bl, stack, timer, dev, H, KV, qkv=None, cache=None):
    """Prefill attention over a 4096-token prompt (20 query / 5 key-value
    heads): ms per call and causal TFLOPS.  qkv defaults to N(0,1)."""
    M = ATTN_CTX
    if qkv is None:
        qkv = torch.randn((M, H + 2 * KV), generator=torch.Generator(device=dev).manual_seed(6), device=dev)
    if cache is None:
        cache = stack.alloc_kv(1, M, dev)
    att = torch.empty((M, H), dtype=torch.float32, device=dev)
    t = timer.run(lambda: bl.attn_prefill(qkv[:, :H], qkv[:, H:H + KV], qkv[:, H + KV:], cache.k[0], cache.v[0],
                                          cache.rope_cos, cache.rope_sin, stack.N_HEADS, stack.N_KV_HEADS,
                                          out=att), 10, 2)
    flops = 4 * 128 * stack.N_HEADS * M * (M + 1) / 2
    return t, round(flops / (t * 1e-3) / 1e12, 1)


def ste_timing(torch, dev, timer, H, I, M=2048):
    """The straight-through backward (dX and dW) of the gate|up pair and of
    down at M tokens, bf16 output gradients: µs and TFLOPS per backward."""
    from bit_ternary_weight_amd import qat
    out = {}
    for name, N, K in (("gateup", 2 * I, H), ("down", H, I)):
        W = torch.randn((N, K), generator=torch.Generator(device=dev).manual_seed(7), device=dev) * 0.02
        xb = torch.randn((M, K), generator=torch.Generator(device=dev).manual_seed(8), device=dev)
        _, saved = qat.forward(xb, W)
        dy = torch.randn((M, N), generator=torch.Generator(device=dev).manual_seed(9), device=dev).to(torch.bfloat16)
        t = timer.run(lambda: qat.backward(dy, saved), 5, 2)
        out[f"ste_backward_m{M}_{name}_tflops"] = round(2 * 2 * M * N * K / (t * 1e-3) / 1e12, 1)
        out[f"ste_backward_m{M}_{name}_us"] = round(t * 1e3, 1)
        del W, xb, saved, dy
    return out


def w1_build(torch, bl, synth, dev, n_layers):
    """Binarized weights of n_layers layers of the 2B4T shape: seeded N(0, 0.02)
    masters drawn on the device (one projection at a time), sign-packed."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    out = []
    for _ in range(n_layers):
        lay = []
        for name, N, K in synth.PROJECTIONS:
            W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
            lay.append(bl.binarize_pack(W))
            del W
        out.append(lay)
    torch.cuda.synchronize()
    return out


def w1_timing(torch, bl, synth, timer, dev, n_layers, steps=None):
    """The 1-bit BitLinear: decode M=1 over a layer's 7 projections (one call:
    the norm launch, then the contraction launch) stepping through n_layers
    layers, and the prefill of the FFN shapes at M=2048 (gate, up and down
    as three problems of one call; and the contraction alone)."""
    import numpy as np
    res = {}
    wl = w1_build(torch, bl, synth, dev, n_layers)
    xs = [torch.from_numpy(synth.act_outliers_bf16(300 + j, 1, K).view(np.int16)).to(dev).view(torch.bfloat16)
          for j, (_, N, K) in enumerate(synth.PROJECTIONS)]
    ys = [torch.empty((1, N), dtype=torch.float32, device=dev) for _, N, K in synth.PROJECTIONS]
    probs = [[dict(x=xs[j], packed=lay[j][0], w_scale=lay[j][1], y=ys[j]) for j in range(len(ys))] for lay in wl]
    g = capture(torch, lambda: [bl.bitlinear_w1_batched(pl) for pl in probs])
    t = timer.run(g.replay, steps or 10, 2) / n_layers
    by = sum(N * K // 8 + K * 2 + N * 4 for _, N, K in synth.PROJECTIONS)
    res["w1_decode_m1_7proj_us_per_layer"] = round(t * 1e3, 2)
    res["w1_decode_m1_7proj_gbs"] = round(by / (t * 1e-3) / 1e9, 1)
    res["w1_decode_m1_7proj_bytes"] = by
    del g
    H, I = synth.HIDDEN, synth.INTERMEDIATE
    M = 2048
    lay = wl[0]
    names = [n for n, _, _ in synth.PROJECTIONS]
    gi, ui, di = names.index("gate"), names.index("up"), names.index("down")
    xh = torch.from_numpy(synth.act_normal_bf16(0, M, H).view(np.int16)).to(dev).view(torch.bfloat16)
    xi = torch.from_numpy(synth.act_normal_bf16(1, M, I).view(np.int16)).to(dev).view(torch.bfloat16)
    yg = torch.empty((M, I), dtype=torch.float32, device=dev)
    yu = torch.empty((M, I), dtype=torch.float32, device=dev)
    yd = torch.empty((M, H), dtype=torch.float32, device=dev)
    pf = [dict(x=xh, packed=lay[gi][0], w_scale=lay[gi][1], y=yg), dict(x=xh, packed=lay[ui][0], w_scale=lay[ui][1], y=yu),
          dict(x=xi, packed=lay[di][0], w_scale=lay[di][1], y=yd)]
    ops = 2 * M * (2 * I * H + H * I)
    t = timer.run(lambda: bl.bitlinear_w1_batched(pf), 20, 3)
    res["w1_prefill_m2048_ffn_us"] = round(t * 1e3, 1)
    res["w1_prefill_m2048_ffn_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
    qh, ah = bl.layernorm_quant(xh)
    qi, ai = bl.layernorm_quant(xi)
    f = lambda: (bl.gemm_w1a8(qh, ah, lay[gi][0], lay[gi][1], y=yg), bl.gemm_w1a8(qh, ah, lay[ui][0], lay[ui][1], y=yu),
                 bl.gemm_w1a8(qi, ai, lay[di][0], lay[di][1], y=yd))
    t = timer.run(f, 20, 3)
    res["w1_prefill_m2048_ffn_gemm_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
    res["w1_prefill_m2048_ffn_gemm_frac_of_int8_peak"] = round(ops / (t * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
    return res


def unpacked_timing(torch, bl, stack, synth, timer, dev, layers, probs1, H, I):
    """The offline-unpacked baseline: the 30 layers' weights unpacked to bf16
    codes (about 4.2 GB), decode M=1 over each layer's 7 projections (the
    headline's inputs, one launch per projection, graph replay), and the
    M=2048 FFN prefill (gate|up then down, quantization included)."""
    import numpy as np
    out = {}
    unp = []
    for lw in layers:
        d = {}
        for name, N, K in synth.PROJECTIONS:
            packed, _ = stack._dest(lw, name)
            d[name] = bl.unpack_bf16(packed)        # one tensor each
        unp.append(d)
    torch.cuda.synchronize()
    ys = [[torch.empty((1, N), dtype=torch.float32, device=dev) for _, N, _ in synth.PROJECTIONS] for _ in layers]

    def one_pass():
        for l, pl in enumerate(probs1):
            for j, (name, N, K) in enumerate(synth.PROJECTIONS):
                bl.gemm_unpacked(pl[j]["x"], unp[l][name], pl[j]["w_mean"], y=ys[l][j])

    one_pass()
    ok = all(torch.equal(ys[l][j], bl.gemv_w2a8(probs1[l][j]["x"], probs1[l][j]["packed"], probs1[l][j]["w_mean"]))
             for l in (0, len(layers) - 1) for j in range(7))
    if not ok:
        raise RuntimeError("the unpacked path differs from the packed one")
    g = capture(torch, one_pass)
    t = timer.run(g.replay, 5, 1) / len(layers)
    wbytes = sum(2 * N * K for _, N, K in synth.PROJECTIONS)
    out["unpacked_decode_m1_us_per_layer"] = round(t * 1e3, 2)
    out["unpacked_decode_m1_weight_gbs"] = round(wbytes / (t * 1e-3) / 1e9, 1)
    del g
    M = 2048
    lw = layers[0]
    gu = torch.cat([unp[0]["gate"], unp[0]["up"]])
    dn = unp[0]["down"]
    xg = torch.from_numpy(synth.act_normal_bf16(0, M, H).view(np.int16)).to(dev).view(torch.bfloat16)
    xd = torch.from_numpy(synth.act_normal_bf16(1, M, I).view(np.int16)).to(dev).view(torch.bfloat16)
    yg = torch.empty((M, 2 * I), dtype=torch.float32, device=dev)
    yd = torch.empty((M, H), dtype=torch.float32, device=dev)
    f = lambda: (bl.gemm_unpacked(xg, gu, lw.w_gu, seg_n=[I, I], y=yg), bl.gemm_unpacked(xd, dn, lw.w_down, y=yd))
    t = timer.run(f, 10, 2)
    out["unpacked_prefill_m2048_ffn_tops"] = round(2 * M * 3 * I * H / (t * 1e-3) / 1e12, 1)
    out["unpacked_prefill_m2048_ffn_us"] = round(t * 1e3, 1)
    del unp, gu
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernel-only", action="store_true",
                    help="only the dominant-kernel loop (for profiler runs)")
    ap.add_argument("--attn-only", action="store_true",
                    help="only the decode attention loop at position 4095 over 30 layers' caches (for profiler runs)")
    ap.add_argument("--attn-prefill-only", action="store_true",
                    help="only the prefill attention over a 4096-token prompt (for profiler runs)")
    ap.add_argument("--ste-only", action="store_true",
                    help="only the straight-through backward at M=2048 (for profiler runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the M=2048 FFN prefill GEMMs (gate|up, then down, int8 codes given) (for profiler runs)")
    ap.add_argument("--chain-only", action="store_true",
                    help="only the persistent 30-layer decode step (for profiler runs)")
    ap.add_argument("--mt-only", type=int, default=0, metavar="M",
                    help="only the batched decode at M rows, 7 projections per launch over 30 layers (for profiler runs)")
    ap.add_argument("--w1-only", action="store_true",
                    help="only the 1-bit BitLinear decode (7 projections x 30 layers) and prefill (for profiler runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer 5 times (calibrates profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the library has no "
              "multi-GPU path (each GPU would hold its own shard of the weight rows)", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    # the oracle's CPU baseline first, before anything touches the GPU (its
    # core is pinned and nothing else runs meanwhile)
    run_cpu = not (args.no_cpu or args.copy_probe or args.kernel_only or args.attn_only or args.ste_only
                   or args.attn_prefill_only or args.prefill_only or args.mt_only or args.chain_only
                   or args.w1_only)
    cpu = cpu_baseline() if run_cpu else None
    if cpu is not None:
        log(f"cpu baseline (oracle, 1 core): {cpu['value']} GB/s decode; {cpu['per_workload']}")

    import torch

    from bit_ternary_weight_amd import binding as bl
    from bit_ternary_weight_amd import stack, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(7)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}), flush=True)
        return
    H, I, KV = synth.HIDDEN, synth.INTERMEDIATE, synth.KV_DIM
    timer = Timer(torch)
    if args.attn_only:
        t, gbs = attn_decode_timing(torch, bl, stack, timer, dev, args.layers, H, KV)
        print(json.dumps({"attn_decode_ctx4096_us_per_layer": round(t * 1e3, 3), "attn_decode_ctx4096_gbs": gbs}),
              flush=True)
        return
    if args.ste_only:
        print(json.dumps(ste_timing(torch, dev, timer, H, I)), flush=True)
        return
    if args.attn_prefill_only:
        t, tf = attn_prefill_timing(torch, bl, stack, timer, dev, H, KV)
        print(json.dumps({"attn_prefill_m4096_us": round(t * 1e3, 1), "attn_prefill_m4096_tflops": tf}), flush=True)
        return
    if args.w1_only:
        print(json.dumps(w1_timing(torch, bl, synth, timer, dev, args.layers, steps=max(1, args.steps // args.layers))),
              flush=True)
        return
    if args.prefill_only:
        lw = stack.build_layers(1, dev)[0]
        M = 2048
        qg, ag = bl.quant_act(torch.from_numpy(synth.act_normal_bf16(0, M, H).view(np.int16)).to(dev).view(torch.bfloat16))
        qd, ad = bl.quant_act(torch.from_numpy(synth.act_normal_bf16(1, M, I).view(np.int16)).to(dev).view(torch.bfloat16))
        yg = torch.empty((M, 2 * I), dtype=torch.float32, device=dev)
        yd = torch.empty((M, H), dtype=torch.float32, device=dev)
        f = lambda: (bl.gemm_w2a8(qg, lw.packed_gu, lw.w_gu, seg_n=[I, I], a=ag, y=yg),
                     bl.gemm_w2a8(qd, lw.packed_down, lw.w_down, a=ad, y=yd))
        t = timer.run(f, max(1, args.steps), 3)
        print(json.dumps({"prefill_m2048_gateup_then_down_us": round(t * 1e3, 1),
                          "tops": round((2 * M * 2 * I * H + 2 * M * H * I) / (t * 1e-3) / 1e12, 1)}), flush=True)
        return
    t_build = time.perf_counter()
    layers = stack.build_layers(args.layers, dev, workers=16)
    log(f"built {args.layers} layers in {time.perf_counter() - t_build:.1f} s")
    packed_total = sum(lw.nbytes_packed() for lw in layers)

    # ---------------------------------------------------------------- headline: one-row decode, 7 projections a launch
    def seven_problems(M, layer_list, kind):
        probs = []
        for l, lw in enumerate(layer_list):
            xs = []
            for j, (name, N, K) in enumerate(synth.PROJECTIONS):
                if kind == "heavy":
                    bits = synth.act_heavy_tail_bf16(100 + j, M, K)
                else:
                    bits = synth.act_outliers_bf16(100 + j, M, K)
                xs.append(torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16))
            pl = []
            for j, (name, N, K) in enumerate(synth.PROJECTIONS):
                packed, wm = stack._dest(lw, name)
                pl.append(dict(x=xs[j], packed=packed, w_mean=wm,
                               y=torch.empty((M, N), dtype=torch.float32, device=dev)))
            probs.append(pl)
        return probs

    def step_bytes7(M):
        return sum(N * K // 4 + M * K * 2 + M * N * 4 for _, N, K in synth.PROJECTIONS)

    if args.chain_only:
        x1 = torch.from_numpy(synth.act_outliers_bf16(0, 1, H).view(np.int16)).to(dev).view(torch.bfloat16)
        yp = torch.empty((1, H), dtype=torch.float32, device=dev)
        g = capture(torch, lambda: stack.stack_decode(x1, layers, out=yp))
        t = timer.run(g.replay, max(1, args.steps), 2)
        by = layer_bytes(1, 2, H, I, KV) + (len(layers) - 1) * layer_bytes(1, 4, H, I, KV)
        print(json.dumps({"persistent_decode_us_per_layer": round(t * 1e3 / len(layers), 2),
                          "persistent_decode_gbs": round(by / (t * 1e-3) / 1e9, 1)}), flush=True)
        return
    if args.mt_only:
        M = args.mt_only
        pm = seven_problems(M, layers, "heavy")
        g = capture(torch, lambda: [bl.gemv_w2a8_batched(pl) for pl in pm])
        t = timer.run(g.replay, max(1, args.steps // len(layers)), 1) / len(layers)
        print(json.dumps({f"decode_m{M}_us_per_layer": round(t * 1e3, 2),
                          f"decode_m{M}_gbs": round(step_bytes7(M) / (t * 1e-3) / 1e9, 1)}), flush=True)
        return
    probs1 = seven_problems(1, layers, "outliers")
    # One step = one layer's 7 projections in one launch; step i uses layer
    # i mod 30, so consecutive steps read different weights.  The timed region
    # is a graph of exactly K steps (after W untimed steps); it is replayed
    # until at least 5 regions and 50 ms have been timed, and the median
    # region gives the step time.
    steps = max(1, args.steps)
    nl = len(layers)
    warm_fn = lambda: [bl.gemv_w2a8_batched(probs1[i % nl]) for i in range(max(0, args.warmup))]
    timed_fn = lambda: [bl.gemv_w2a8_batched(probs1[i % nl]) for i in range(steps)]
    warm_fn()
    g1 = capture(torch, timed_fn)
    g1.replay()
    ms_region, n_regions = timer.trials(g1.replay)
    ms = ms_region / steps
    sb = step_bytes7(1)
    value = sb / (ms * 1e-3) / 1e9
    log(f"decode M=1, 7 projections: {ms * 1e3:.2f} us/step, {value:.1f} GB/s ({value / HBM_PEAK_GBS:.1%} of HBM peak); "
        f"median of {n_regions} timed regions of {steps} steps")

    # The headline kernel is the only launch of a step: its average launch
    # duration over the timed region is the step time (back-to-back launches
    # from a graph, gaps included), so the roofline uses the same bytes and
    # time.  The committed kernel trace of this command gives the kernel's
    # duration under the tracer; both are reported.
    traffic = profiled_traffic()
    prof_us = profiled_duration_us()
    roofline = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_gemv_v1<false, bf16 one row, 10 units> (batched one-row decode GEMV, fused per-token quantization)",
                "bytes_per_launch": sb, "avg_launch_us": round(ms * 1e3, 3), "timing": "hip events, graph replay",
                "traffic_over_algorithmic": None if traffic is None else round(traffic / sb, 4),
                "rocprof_avg_us": prof_us,
                "rocprof_frac": None if prof_us is None else round(sb / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if args.kernel_only:
        print(json.dumps({"roofline": roofline}), flush=True)
        return
    del g1

    extra = {"packed_weight_bytes": packed_total}
    # ---------------------------------------------------------------- chained decode through the stack
    x1 = torch.from_numpy(synth.act_outliers_bf16(0, 1, H).view(np.int16)).to(dev).view(torch.bfloat16)
    bufs1 = {}
    step_fn = lambda: stack.stack_forward(x1, layers, bufs=bufs1)
    eager_ms = timer.run(step_fn, 3, 1)
    graph = capture(torch, step_fn)
    ref = stack.stack_forward(x1, layers, bufs={}).clone()
    for _ in range(3):   # every replay must reproduce the eager result bit for bit
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(bufs1["outs"][(len(layers) - 1) & 1], ref):
            raise RuntimeError("graph replay differs from the eager decode pass")
        torch.cuda.synchronize()
    t = timer.run(graph.replay, 10, 2)
    by = layer_bytes(1, 2, H, I, KV) + (len(layers) - 1) * layer_bytes(1, 4, H, I, KV)
    extra["chained_decode_m1_gbs"] = round(by / (t * 1e-3) / 1e9, 1)
    extra["chained_decode_m1_us_per_layer"] = round(t * 1e3 / len(layers), 2)
    extra["chained_decode_m1_eager_us_per_layer"] = round(eager_ms * 1e3 / len(layers), 2)
    log(f"chained decode M=1: {t * 1e3 / len(layers):.2f} us/layer, {extra['chained_decode_m1_gbs']} GB/s")
    del graph
    # the same decode step as one persistent launch (bl_stack_decode): every
    # replay checked against the eager launch chain's output
    yp = torch.empty((1, H), dtype=torch.float32, device=dev)
    pers = lambda: stack.stack_decode(x1, layers, out=yp)
    pers()
    torch.cuda.synchronize()
    if not torch.equal(yp, ref):
        log("persistent decode differs from the launch chain (RMSNorm fp64 sum order)")
    gp = capture(torch, pers)
    for _ in range(3):
        gp.replay()
        torch.cuda.synchronize()
        if not torch.equal(yp, ref):
            raise RuntimeError("persistent decode graph replay differs from the eager decode pass")
    t = timer.run(gp.replay, 20, 2)
    extra["chained_decode_m1_persistent_gbs"] = round(by / (t * 1e-3) / 1e9, 1)
    extra["chained_decode_m1_persistent_us_per_layer"] = round(t * 1e3 / len(layers), 2)
    log(f"persistent chained decode M=1: {t * 1e3 / len(layers):.2f} us/layer, "
        f"{extra['chained_decode_m1_persistent_gbs']} GB/s")
    del gp

    if not args.no_extras:
        # batched decode: M=16 and M=64, 7 projections per launch
        for M in (16, 64):
            pm = seven_problems(M, layers, "heavy")
            g = capture(torch, lambda pm=pm: [bl.gemv_w2a8_batched(pl) for pl in pm])
            t = timer.run(g.replay, 3, 1) / len(layers)
            extra[f"decode_m{M}_gbs"] = round(step_bytes7(M) / (t * 1e-3) / 1e9, 1)
            extra[f"decode_m{M}_us_per_layer"] = round(t * 1e3, 2)
            log(f"batched decode M={M}: {t * 1e3:.2f} us/layer, {extra[f'decode_m{M}_gbs']} GB/s")
            del g, pm
        # decode attention at the full 4096-token context: 30 layers' fp32
        # caches (20 query / 5 key-value heads x 128), the token at position
        # 4095; bytes = the caches read + q, k, v in + the row appended + the
        # output.  Then the whole decode step with attention through the 30
        # layers (q|k|v -> attention -> attn_sub_norm + quantize -> o -> FFN).
        S = ATTN_CTX
        t, gbs, cache = attn_decode_timing(torch, bl, stack, timer, dev, len(layers), H, KV, keep=True)
        ab = attn_bytes(S, H, KV)
        extra["attn_decode_ctx4096_gbs"] = gbs
        extra["attn_decode_ctx4096_us_per_layer"] = round(t * 1e3, 2)
        log(f"decode attention, context 4096: {t * 1e3:.2f} us/layer, {gbs} GB/s")
        bufs_a = {}
        g = capture(torch, lambda: stack.decode_step_attn(x1, layers, cache, S - 1, bufs=bufs_a))
        ref = stack.decode_step_attn(x1, layers, cache, S - 1, bufs={}).clone()
        for _ in range(3):   # replays must reproduce the eager step bit for bit
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(bufs_a["outs1"][(len(layers) - 1) & 1], ref):
                raise RuntimeError("graph replay differs from the eager decode step with attention")
        t = timer.run(g.replay, 5, 1) / len(layers)
        extra["decode_step_attn_ctx4096_us_per_layer"] = round(t * 1e3, 2)
        extra["decode_step_attn_ctx4096_gbs"] = round((layer_bytes(1, 4, H, I, KV) + ab) / (t * 1e-3) / 1e9, 1)
        log(f"decode step with attention, context 4096: {t * 1e3:.2f} us/layer")
        del g, cache
        # one layer, weights resident in the Infinity Cache (warm), for
        # contrast: 30 back-to-back launches on the same layer per replay
        g = capture(torch, lambda: [bl.gemv_w2a8_batched(probs1[0]) for _ in range(len(layers))])
        t = timer.run(g.replay, 20, 2) / len(layers)
        extra["decode_m1_one_layer_warm_gbs"] = round(sb / (t * 1e-3) / 1e9, 1)
        del g
        # prefill GEMMs: fused gate|up (2560 -> 2x6912) then down (6912 -> 2560), M=2048
        M = M2 = 2048
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
        log(f"prefill FFN M=2048: {tops:.1f} TOPS ({tops / INT8_PEAK_TOPS:.1%} of int8 peak)")
        # prefill through the 30-layer stack, M=4096
        M = 4096
        xp = torch.from_numpy(synth.act_normal_bf16(0, M, H).view(np.int16)).to(dev).view(torch.bfloat16)
        bp = {}
        t = timer.run(lambda: stack.stack_forward(xp, layers, bufs=bp), 3, 1)
        ops = layer_ops(M, H, I, KV) * len(layers)
        extra["prefill_m4096_stack_tops"] = round(ops / (t * 1e-3) / 1e12, 1)
        extra["prefill_m4096_stack_frac_of_int8_peak"] = round(ops / (t * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
        extra["prefill_m4096_stack_ms"] = round(t, 2)
        log(f"30-layer prefill M=4096: {extra['prefill_m4096_stack_tops']} TOPS")
        del bp
        # the same prompt with attention (positions 0 .. 4095, caches filled),
        # and the prefill attention alone on one layer's q|k|v
        cache = stack.alloc_kv(len(layers), M, dev)
        bp = {}
        t = timer.run(lambda: stack.prefill_attn(xp, layers, cache, bufs=bp), 3, 1)
        extra["prefill_m4096_attn_stack_ms"] = round(t, 2)
        t, tf = attn_prefill_timing(torch, bl, stack, timer, dev, H, KV, qkv=bp["p_qkv"], cache=cache)
        extra["attn_prefill_m4096_us"] = round(t * 1e3, 1)
        extra["attn_prefill_m4096_tflops"] = tf
        log(f"prefill with attention, M=4096: {extra['prefill_m4096_attn_stack_ms']} ms; attention alone "
            f"{t * 1e3:.1f} us/layer, {tf} TFLOPS (bf16 products, causal)")
        del bp, cache
        # the straight-through backward at M=2048 (quantization-aware
        # training): dX and dW of the gate|up pair and of down
        extra.update(ste_timing(torch, dev, timer, H, I))
        log(f"straight-through backward M=2048: gate|up {extra['ste_backward_m2048_gateup_tflops']} TFLOPS, "
            f"down {extra['ste_backward_m2048_down_tflops']} TFLOPS (bf16 products)")
        # the offline-unpacked path (weights expanded once to bf16 codes, dense
        # bf16 products; the same output bits): decode M=1 over the 7
        # projections of each of the 30 layers (one launch per projection),
        # and the M=2048 FFN prefill
        extra.update(unpacked_timing(torch, bl, stack, synth, timer, dev, layers, probs1, H, I))
        log(f"offline-unpacked: decode M=1 {extra['unpacked_decode_m1_us_per_layer']} us/layer "
            f"({extra['unpacked_decode_m1_weight_gbs']} GB/s of bf16 codes), prefill M=2048 "
            f"{extra['unpacked_prefill_m2048_ffn_tops']} TOPS")
        # the 1-bit BitLinear (binarized weights, layer norm): decode over the
        # 7 projections of 30 layers and the FFN prefill at M=2048
        extra.update(w1_timing(torch, bl, synth, timer, dev, len(layers)))
        log(f"1-bit BitLinear: decode M=1 {extra['w1_decode_m1_7proj_us_per_layer']} us/layer "
            f"({extra['w1_decode_m1_7proj_gbs']} GB/s), prefill FFN M=2048 {extra['w1_prefill_m2048_ffn_tops']} TOPS "
            f"(contraction alone {extra['w1_prefill_m2048_ffn_gemm_tops']} TOPS)")
        # offline ternarization (absmean + pack) of one 6912 x 2560 master
        W = torch.from_numpy(synth.layer_weight(0, "gate")).to(dev)
        pk = torch.empty((I // 4, H), dtype=torch.uint8, device=dev)
        wm = torch.empty(1, dtype=torch.float32, device=dev)
        t = timer.run(lambda: bl.ternarize_pack(W, packed=pk, w_mean=wm), 20, 3)
        extra["ternarize_pack_gbs"] = round((W.numel() * 4 + pk.numel()) / (t * 1e-3) / 1e9, 1)
        del W
        # the two readings of the weight quantization (divide by the mean,
        # multiply by its reciprocal) over one layer's 7 masters, on the host
        nq, nw = 0, 0
        for p, _, _ in synth.PROJECTIONS:
            Wh = synth.layer_weight(0, p)
            nq += q1_disagreement_count(Wh, absmean_f32(Wh))
            nw += Wh.size
        extra["divide_vs_reciprocal_code_disagreements"] = {"weights": nw, "disagree": nq}
        log(f"weight codes that differ between W / mean and W * (1 / mean): {nq} of {nw}")

    line = {
        "metric": "W1.58A8 BitLinear decode GEMV HBM GB/s (M=1, 7 projections of a 2B4T layer per step)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xternary->int32, fp32 scales",
        "data": "synthetic (seeded N(0,0.02) fp32 masters ternarized on the device; bf16 x with 1% x20 outliers)",
        "config": {"workload": f"decode GEMV M=1 over the 7 projections of a BitNet-2B4T layer (hidden 2560, "
                               f"intermediate 6912, 20/5 heads x 128) in one batched launch per layer, stepping "
                               f"through {len(layers)} distinct layers ({packed_total} packed bytes) so weights "
                               f"stream from HBM; bf16 in, fp32 out, quantization inside the kernel",
                   "M": 1, "layers": len(layers), "bytes_per_step": sb, "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
