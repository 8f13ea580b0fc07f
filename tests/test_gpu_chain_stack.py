"""GPU parity: bl_ffn_chain stage by stage, and the 30-layer linear stack.

The chain's stage outputs (codes and scales after each RMSNorm, the
ReLU^2(gate)*up tensor) are compared bit-exactly; final outputs by the fp32
tolerance (and expected bit-identical).  The stack is checked layer by layer:
each layer's GPU output is compared with the oracle's layer run on the same
input (the GPU's input of that layer), so a difference cannot cascade.
Every output and stage buffer is pre-filled with a pattern no result can
hold and followed by a canary tail (gpu_helpers.Guarded).
"""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import (F32_TOL, BF16_TOL, assert_exact, assert_rows_close, bf16_dev, dev, f32_of_bf16, guarded,
                         host, max_ulp_diff, requires_gpu, to_dev)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


def _chain_weights(seed, H, I):
    pg, wg, cg = oracle.ternarize_pack(synth.master_weight(seed, I, H))
    pu, wu, cu = oracle.ternarize_pack(synth.master_weight(seed + 1, I, H))
    pd, wd, cd = oracle.ternarize_pack(synth.master_weight(seed + 2, H, I))
    return (np.concatenate([pg, pu]), np.array([wg, wu], np.float32), pd, np.array([wd], np.float32),
            np.concatenate([cg, cu]), cd)


def _check_chain(M, H, I, seed=0, gains=False, h_kind="f32", rows=None, y_dtype=torch.float32):
    pgu, wgu, pd, wd, cgu, cd = _chain_weights(100 + seed, H, I)
    if h_kind == "bf16":
        bits = synth.act_outliers_bf16(seed, M, H)
        h_host, h_dev = f32_of_bf16(bits), bf16_dev(bits)
    else:
        h_host = synth.act_normal_f32(seed, M, H)
        h_dev = to_dev(h_host)
    gs = gf = None
    if gains:
        rng = np.random.default_rng(seed)
        gs = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
        gf = rng.uniform(0.5, 1.5, size=I).astype(np.float32)
    gy = guarded((M, H), y_dtype)
    gst = dict(q1=guarded((M, H), torch.int8), a1=guarded((M,)), p=guarded((M, I)), q2=guarded((M, I), torch.int8),
               a2=guarded((M,)))
    y, st = _bl().ffn_chain(h_dev, to_dev(pgu), to_dev(wgu), to_dev(pd), to_dev(wd),
                            g_subln=None if gs is None else to_dev(gs), g_ffn=None if gf is None else to_dev(gf),
                            debug={k: g.t for k, g in gst.items()}, y_dtype=y_dtype, y=gy.t)
    gy.check("y")
    for k, g in gst.items():
        g.check(k)
    rows = list(range(M)) if rows is None else rows
    if M * I > 4096 * 1024 and len(rows) > 8:
        ref = oracle.ffn_chain_f64gemm(h_host[rows], cgu, wgu, cd, wd[0], g_subln=gs, g_ffn=gf)
    else:
        ref = oracle.ffn_chain(h_host[rows], cgu, wgu, cd, wd[0], g_subln=gs, g_ffn=gf)
    for k in ("q1", "a1", "q2", "a2"):
        assert_exact(host(st[k])[rows], ref[k], k)
    assert_exact(host(st["p"])[rows].view(np.uint32), ref["p"].view(np.uint32), "p bits")
    yh = host(y)[rows]
    if y_dtype == torch.float32:
        assert_rows_close(yh, ref["y"], F32_TOL)
        assert max_ulp_diff(yh, ref["y"]) == 0
    else:
        assert_rows_close(f32_of_bf16(yh), ref["y"], BF16_TOL)
        assert_exact(yh, oracle.to_bf16(ref["y"]), "bf16 y")


@pytest.mark.parametrize("M", [1, 4, 16, 17, 64, 65, 200])
def test_chain_small(M):
    _check_chain(M, 256, 512, seed=M)


def test_chain_gains_bf16_in_out():
    _check_chain(8, 256, 512, seed=3, gains=True, h_kind="bf16")
    _check_chain(130, 256, 512, seed=4, gains=True, h_kind="bf16", y_dtype=torch.bfloat16)


@pytest.mark.parametrize("M,H,I", [(3, 20, 36), (70, 20, 36), (2, 64, 100)])
def test_chain_ragged(M, H, I):
    _check_chain(M, H, I, seed=5)


@pytest.mark.parametrize("M", [1, 4, 64])
def test_chain_full_size_decode(M):
    _check_chain(M, 2560, 6912, seed=7, h_kind="bf16")


@pytest.mark.timeout(600)
def test_chain_full_size_prefill_all_rows():
    _check_chain(2048, 2560, 6912, seed=8, h_kind="bf16")


def test_chain_zero_row():
    """A zero row through both sub-norms and quantizers (decode and prefill
    sizes): every stage is exactly zero for it, the other rows as usual."""
    for M in (3, 130):
        from bit_ternary_weight_amd import binding as bl
        pgu, wgu, pd, wd, cgu, cd = _chain_weights(300 + M, 256, 512)
        h = synth.act_normal_f32(60 + M, M, 256)
        h[1] = 0.0
        y, st = bl.ffn_chain(to_dev(h), to_dev(pgu), to_dev(wgu), to_dev(pd), to_dev(wd), debug=True)
        ref = oracle.ffn_chain(h, cgu, wgu, cd, wd[0])
        for k in ("q1", "a1", "q2", "a2"):
            assert_exact(host(st[k]), ref[k], k)
        assert (host(st["q1"])[1] == 0).all() and (host(y)[1] == 0).all()
        assert_exact(host(y).view(np.uint32), ref["y"].view(np.uint32), "y bits")


# ----------------------------------------------------------------------------- the stack
def _oracle_layer_codes(layer):
    codes, wms = {}, {}
    for p, _, _ in synth.PROJECTIONS:
        _, wm, c = oracle.ternarize_pack(synth.layer_weight(layer, p))
        codes[p] = c
        wms[p] = wm
    return codes, wms


def _check_stack(M, n_layers, rows):
    """Each layer's stage outputs (q|k|v, o, the layer output) at `rows`
    against the oracle's layer on the GPU's own input to that layer; every
    buffer guarded over all M rows."""
    from bit_ternary_weight_amd import stack
    layers = stack.build_layers(n_layers, dev())
    if M == 1:
        bits = synth.act_outliers_bf16(0, M, synth.HIDDEN)
    else:
        bits = synth.act_normal_bf16(0, M, synth.HIDDEN)
    x = bf16_dev(bits)
    x_host = f32_of_bf16(bits)
    H = synth.HIDDEN
    layer_ref = oracle.layer if len(rows) <= 4 else oracle.layer_f64gemm
    for l, lw in enumerate(layers):
        codes, wms = _oracle_layer_codes(l)
        # the device ternarization must reproduce the oracle's packing
        for p in ("q", "gate", "down"):
            packed, wm = stack._dest(lw, p)
            assert host(wm)[0] == wms[p]
            assert_exact(host(packed), oracle.pack(codes[p]), f"layer {l} {p} packed")
        g_qkv, g_o, g_y = guarded((M, H + 2 * synth.KV_DIM)), guarded((M, H)), guarded((M, H))
        bufs = {"y_qkv": g_qkv.t, "y_o": g_o.t}
        y = stack.layer_forward(x, lw, bufs=bufs, out=g_y.t)
        for g, what in ((g_qkv, "q|k|v"), (g_o, "o"), (g_y, "layer output")):
            g.check(f"layer {l} {what}")
        ref = layer_ref(x_host[rows], codes, wms)
        for key, t in (("y_qkv", g_qkv.t), ("y_o", g_o.t), ("y", y)):
            got = host(t)[rows]
            assert_rows_close(got, ref[key], F32_TOL, f"layer {l} {key}")
            assert max_ulp_diff(got, ref[key]) == 0, f"layer {l} {key}"
        x = y.clone()
        x_host = host(y)
        print(f"[stack M={M}] layer {l} matches the oracle on {len(rows)} rows", flush=True)


@pytest.mark.timeout(900)
def test_stack_decode_30_layers():
    _check_stack(1, 30, [0])


@pytest.mark.timeout(1200)
def test_stack_prefill_30_layers_one_row_per_token_tile():
    """M=4096 through all 30 layers: one row in every 32-token block (so in
    every 96- and 128-token tile of the prefill GEMM), at a different offset
    in each block, plus the last row."""
    M = 4096
    rows = sorted(set([32 * t + (13 * t) % 32 for t in range(M // 32)] + [M - 1]))
    _check_stack(M, 30, rows)


# ----------------------------------------------------------------------------- the persistent decode step
def _check_stack_decode(n_layers, x_kind="outliers", seed=0, gains=False):
    """bl_stack_decode over n_layers: every stage of every layer (q|k|v, o,
    ReLU^2(gate)*up, down) against the oracle's layer on the GPU's own input
    to that layer; all stage buffers and the output guarded.  gains: every
    layer gets seeded RMSNorm gains U(0.5, 1.5) for both sub-norms."""
    from bit_ternary_weight_amd import stack
    H, KV, I = synth.HIDDEN, synth.KV_DIM, synth.INTERMEDIATE
    layers = stack.build_layers(n_layers, dev())
    host_gains = [(None, None)] * n_layers
    if gains:
        rng = np.random.default_rng(1000 + seed)
        host_gains = [(rng.uniform(0.5, 1.5, size=H).astype(np.float32),
                       rng.uniform(0.5, 1.5, size=I).astype(np.float32)) for _ in range(n_layers)]
        for lw, (gs, gf) in zip(layers, host_gains):
            lw.g_subln, lw.g_ffn = to_dev(gs), to_dev(gf)
    bits = synth.act_outliers_bf16(seed, 1, H) if x_kind == "outliers" else synth.act_normal_bf16(seed, 1, H)
    x = bf16_dev(bits)
    Sw = (H + 2 * KV) + H + I + H
    gst = guarded((n_layers, Sw))
    gy = guarded((1, H))
    stack.stack_decode(x, layers, out=gy.t, stages=gst.t)
    gst.check("stages")
    gy.check("y")
    st = host(gst.t)
    assert np.array_equal(host(gy.t)[0].view(np.uint32), st[-1, Sw - H:].view(np.uint32))
    x_host = f32_of_bf16(bits)
    offs = {"y_qkv": (0, H + 2 * KV), "y_o": (H + 2 * KV, H), "p": (2 * H + 2 * KV, I), "y": (2 * H + 2 * KV + I, H)}
    for l in range(n_layers):
        codes, wms = _oracle_layer_codes(l)
        ref = oracle.layer(x_host, codes, wms, g_subln=host_gains[l][0], g_ffn=host_gains[l][1])
        for key, (o, n) in offs.items():
            got = st[l:l + 1, o:o + n]
            assert_exact(got.view(np.uint32), np.ascontiguousarray(ref[key]).view(np.uint32), f"layer {l} {key}")
        x_host = st[l:l + 1, Sw - H:].copy()
        print(f"[stack_decode] layer {l} stages bit-exact", flush=True)


@pytest.mark.timeout(900)
def test_stack_decode_persistent_30_layers():
    _check_stack_decode(30)


def test_stack_decode_persistent_odd_and_short():
    """One layer (a phantom second layer in the pair loop) and three layers."""
    _check_stack_decode(1, seed=3)
    _check_stack_decode(3, x_kind="normal", seed=4)


def test_stack_decode_persistent_with_gains():
    """Both sub-norms with gains: the absmax is taken after the gain, so the
    kernel's gain path (a separate max pass) runs in every FFN stage."""
    _check_stack_decode(3, seed=5, gains=True)


def test_stack_decode_persistent_matches_the_launch_chain():
    """The persistent step and the separate launches give the same output."""
    from bit_ternary_weight_amd import stack
    layers = stack.build_layers(4, dev())
    x = bf16_dev(synth.act_outliers_bf16(9, 1, synth.HIDDEN))
    a = stack.stack_decode(x, layers).clone()
    b = stack.stack_forward(x, layers, bufs={}).clone()
    assert torch.equal(a, b)
    # repeated calls on the same buffers stay identical
    assert torch.equal(stack.stack_decode(x, layers), a)
