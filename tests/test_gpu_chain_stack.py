"""GPU parity: bl_ffn_chain stage by stage, and the 30-layer linear stack.

The chain's stage outputs (codes and scales after each RMSNorm, the
ReLU^2(gate)*up tensor) are compared bit-exactly; final outputs by the fp32
tolerance (and expected bit-identical).  The stack is checked layer by layer:
each layer's GPU output is compared with the oracle's layer run on the same
input (the GPU's input of that layer), so a difference cannot cascade.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import (F32_TOL, BF16_TOL, assert_exact, assert_rows_close, bf16_dev, dev, f32_of_bf16, host,
                         max_ulp_diff, requires_gpu, to_dev)

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
    y, st = _bl().ffn_chain(h_dev, to_dev(pgu), to_dev(wgu), to_dev(pd), to_dev(wd),
                            g_subln=None if gs is None else to_dev(gs), g_ffn=None if gf is None else to_dev(gf),
                            debug=True, y_dtype=y_dtype)
    rows = list(range(M)) if rows is None else rows
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
    _check_chain(M, 2560, 6912, seed=7, h_kind="bf16", rows=None if M <= 4 else [0, 31, 63])


def test_chain_full_size_prefill_sampled():
    _check_chain(2048, 2560, 6912, seed=8, h_kind="bf16", rows=[0, 5, 1023, 2047])


# ----------------------------------------------------------------------------- the stack
def _oracle_layer_codes(layer):
    codes, wms = {}, {}
    for p, _, _ in synth.PROJECTIONS:
        _, wm, c = oracle.ternarize_pack(synth.layer_weight(layer, p))
        codes[p] = c
        wms[p] = wm
    return codes, wms


def _check_stack(M, n_layers, rows):
    from bit_ternary_weight_amd import stack
    layers = stack.build_layers(n_layers, dev())
    if M == 1:
        bits = synth.act_outliers_bf16(0, M, synth.HIDDEN)
    else:
        bits = synth.act_normal_bf16(0, M, synth.HIDDEN)
    x = bf16_dev(bits)
    bufs = {}
    x_host = f32_of_bf16(bits)
    for l, lw in enumerate(layers):
        codes, wms = _oracle_layer_codes(l)
        # the device ternarization must reproduce the oracle's packing
        for p in ("q", "gate", "down"):
            packed, wm = stack._dest(lw, p)
            assert host(wm)[0] == wms[p]
            assert_exact(host(packed), oracle.pack(codes[p]), f"layer {l} {p} packed")
        y = stack.layer_forward(x, lw, bufs=bufs)
        ref = oracle.layer(x_host[rows], codes, wms)
        yh = host(y)
        assert_rows_close(yh[rows], ref["y"], F32_TOL, f"layer {l}")
        assert max_ulp_diff(yh[rows], ref["y"]) == 0, f"layer {l}"
        x = y.clone()
        x_host = yh


@pytest.mark.timeout(900)
def test_stack_decode_30_layers():
    _check_stack(1, 30, [0])


@pytest.mark.timeout(600)
def test_stack_prefill_sampled_rows():
    _check_stack(4096, 3, [0, 2049, 4095])
