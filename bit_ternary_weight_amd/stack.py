"""Linear path of a BitNet b1.58 2B4T-shaped decoder stack.

Per layer (shapes from the "BitNetConfig" section of the BitNet model
documentation pages: hidden 2560, intermediate 6912, 20 query / 5 key-value
heads of 128):
  x -> fused q|k|v BitLinear (three segments, one launch)
    -> o BitLinear fed with q's output (layer_forward: attention left out, a
       convention the pages give no wiring for)
    -> FFN chain: subln RMSNorm -> quantize -> gate|up -> ReLU^2(gate)*up ->
       ffn_sub_norm RMSNorm -> quantize -> down          (bl_ffn_chain)
  and down's output is the next layer's input (no residual additions).

decode_layer_attn is the same layer at one token with the attention side in
place of the stand-in ("BitNet" model documentation, "模型详情": rotary
position embeddings, grouped-query attention, subln before o_proj):
  x -> q|k|v -> RoPE, key/value cache append and attention over positions
    0..pos (bl_attn_decode) -> attn_sub_norm RMSNorm -> quantize -> o
    BitLinear (bl_subln_gemv_w2a8, one launch at decode size) -> FFN chain.
prefill_layer_attn is the same at M prompt tokens (positions 0 .. M-1): the
causal attention of bl_attn_prefill, which also fills the caches that the
decode steps then extend.  Input norms and residual additions stay out, as in
layer_forward.

Every step runs in libbitlinear through the binding; this module only holds
weights and orders calls.  Weights are ternarized on the device from seeded
fp32 masters (bl_ternarize_pack), so the packed bytes match what the oracle
packs from the same masters.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import torch

from . import binding as bl
from . import synth

H = synth.HIDDEN
I = synth.INTERMEDIATE
KV = synth.KV_DIM
QKV_SEGS = (H, KV, KV)
DECODE_MAX_M = 64
HEAD_DIM = 128
N_HEADS = H // HEAD_DIM
N_KV_HEADS = KV // HEAD_DIM
ROPE_BASE = 500000.0   # rope_theta: a parameter on the pages (no value given); any base works


@dataclass
class LayerWeights:
    packed_qkv: torch.Tensor    # [(H+2KV)/4, H]
    w_qkv: torch.Tensor         # [3]
    packed_o: torch.Tensor      # [H/4, H]
    w_o: torch.Tensor           # [1]
    packed_gu: torch.Tensor     # [2I/4, H]
    w_gu: torch.Tensor          # [2]
    packed_down: torch.Tensor   # [H/4, I]
    w_down: torch.Tensor        # [1]

    def nbytes_packed(self) -> int:
        return sum(t.numel() for t in (self.packed_qkv, self.packed_o, self.packed_gu, self.packed_down))


def _alloc_layer(device) -> LayerWeights:
    u8, f32 = torch.uint8, torch.float32
    return LayerWeights(
        packed_qkv=torch.empty(((H + 2 * KV) // 4, H), dtype=u8, device=device),
        w_qkv=torch.empty(3, dtype=f32, device=device),
        packed_o=torch.empty((H // 4, H), dtype=u8, device=device),
        w_o=torch.empty(1, dtype=f32, device=device),
        packed_gu=torch.empty((2 * I // 4, H), dtype=u8, device=device),
        w_gu=torch.empty(2, dtype=f32, device=device),
        packed_down=torch.empty((H // 4, I), dtype=u8, device=device),
        w_down=torch.empty(1, dtype=f32, device=device),
    )


def _dest(lw: LayerWeights, proj: str):
    """(packed rows view, w_mean view) where projection `proj` lives."""
    r_h, r_kv, r_i = H // 4, KV // 4, I // 4
    return {
        "q": (lw.packed_qkv[0:r_h], lw.w_qkv[0:1]),
        "k": (lw.packed_qkv[r_h:r_h + r_kv], lw.w_qkv[1:2]),
        "v": (lw.packed_qkv[r_h + r_kv:r_h + 2 * r_kv], lw.w_qkv[2:3]),
        "o": (lw.packed_o, lw.w_o),
        "gate": (lw.packed_gu[0:r_i], lw.w_gu[0:1]),
        "up": (lw.packed_gu[r_i:2 * r_i], lw.w_gu[1:2]),
        "down": (lw.packed_down, lw.w_down),
    }[proj]


def build_layers(n_layers: int, device, masters=None, workers: int = 8):
    """Ternarize and pack `n_layers` seeded layers on the device.

    masters: optional callable (layer, proj) -> fp32 numpy [N,K]; defaults to
    the seeded generator.  Masters are drawn on host threads and ternarized
    one projection at a time, so at most a few projections sit in memory.
    """
    gen = masters or synth.layer_weight
    layers = [_alloc_layer(device) for _ in range(n_layers)]
    jobs = [(l, p) for l in range(n_layers) for p, _, _ in synth.PROJECTIONS]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(gen, l, p) for l, p in jobs[: 2 * workers]]
        nxt = len(futs)
        for i, (l, p) in enumerate(jobs):
            W = futs[i].result()
            futs[i] = None
            if nxt < len(jobs):
                futs.append(ex.submit(gen, *jobs[nxt]))
                nxt += 1
            Wd = torch.from_numpy(W).to(device, non_blocking=False)
            packed, wm = _dest(layers[l], p)
            bl.ternarize_pack(Wd, packed=packed, w_mean=wm)
            del Wd
    torch.cuda.synchronize(device)
    return layers


def _contract(M):
    return bl.gemv_w2a8 if M <= DECODE_MAX_M else bl.gemm_w2a8


def layer_forward(x: torch.Tensor, lw: LayerWeights, eps: float = 1e-5, out: torch.Tensor = None,
                  bufs: dict = None):
    """One layer's linear path.  x [M,H] fp32 or bf16 -> y [M,H] fp32.

    bufs: optional dict of preallocated intermediates (y_qkv, y_o) reused
    across calls (keeps the allocator out of timed loops).
    """
    M = x.shape[0]
    fn = _contract(M)
    dev = x.device
    if bufs is None:
        bufs = {}
    y_qkv = bufs.get("y_qkv")
    if y_qkv is None or y_qkv.shape[0] != M:
        y_qkv = torch.empty((M, sum(QKV_SEGS)), dtype=torch.float32, device=dev)
        bufs["y_qkv"] = y_qkv
    y_o = bufs.get("y_o")
    if y_o is None or y_o.shape[0] != M:
        y_o = torch.empty((M, H), dtype=torch.float32, device=dev)
        bufs["y_o"] = y_o
    fn(x, lw.packed_qkv, lw.w_qkv, seg_n=QKV_SEGS, y=y_qkv)
    fn(y_qkv[:, :H], lw.packed_o, lw.w_o, y=y_o)
    return bl.ffn_chain(y_o, lw.packed_gu, lw.w_gu, lw.packed_down, lw.w_down, eps=eps, y=out)


def stack_decode(x: torch.Tensor, layers, eps: float = 1e-5, out: torch.Tensor = None, stages: torch.Tensor = None):
    """The same linear path as stack_forward at one token, every layer's
    stages in one persistent launch per 32 layers (bl_stack_decode).
    x [1,H] fp32 or bf16 -> [1,H] fp32; stages, when given, is
    [len(layers), (H+2KV)+H+I+H] fp32 and receives each stage's output."""
    if x.shape[0] != 1:
        raise ValueError("stack_decode takes one token")
    n = bl.STACK_DECODE_MAX_LAYERS
    if out is None:
        out = torch.empty((1, H), dtype=torch.float32, device=x.device)
    cur = x
    for i in range(0, len(layers), n):
        part = layers[i:i + n]
        st = None if stages is None else stages[i:i + len(part)]
        y = out if i + n >= len(layers) else torch.empty((1, H), dtype=torch.float32, device=x.device)
        bl.stack_decode(cur, part, H, KV, I, eps=eps, y=y, stages=st)
        cur = y
    return out


def stack_forward(x: torch.Tensor, layers, eps: float = 1e-5, bufs: dict = None):
    """All layers in sequence; returns the last layer's output [M,H] fp32."""
    if bufs is None:
        bufs = {}
    M = x.shape[0]
    outs = bufs.get("outs")
    if outs is None or outs[0].shape[0] != M:
        outs = [torch.empty((M, H), dtype=torch.float32, device=x.device) for _ in range(2)]
        bufs["outs"] = outs
    cur = x
    for i, lw in enumerate(layers):
        cur = layer_forward(cur, lw, eps, out=outs[i & 1], bufs=bufs)
    return cur



@dataclass
class KVCache:
    """Per-layer fp32 key/value caches [N_KV_HEADS, max_seq, 128] and the
    RoPE tables [max_seq, 64] they share."""
    k: list
    v: list
    rope_cos: torch.Tensor
    rope_sin: torch.Tensor
    max_seq: int


def alloc_kv(n_layers: int, max_seq: int, device, base: float = ROPE_BASE) -> KVCache:
    rc, rs = bl.rope_table(max_seq, HEAD_DIM, base, device=device)
    shape = (N_KV_HEADS, max_seq, HEAD_DIM)
    return KVCache([torch.zeros(shape, dtype=torch.float32, device=device) for _ in range(n_layers)],
                   [torch.zeros(shape, dtype=torch.float32, device=device) for _ in range(n_layers)],
                   rc, rs, max_seq)


def decode_layer_attn(x: torch.Tensor, lw: LayerWeights, cache: KVCache, layer: int, pos: int,
                      eps: float = 1e-5, out: torch.Tensor = None, bufs: dict = None, debug: dict = None):
    """One layer at one token with attention.  x [1,H] fp32 or bf16 -> [1,H]
    fp32; the token's rotated key and its value go into the layer's cache at
    pos.  debug: optional dict that receives the stage outputs."""
    if x.shape[0] != 1:
        raise ValueError("decode_layer_attn takes one token")
    dev = x.device
    if bufs is None:
        bufs = {}
    if "att" not in bufs:
        bufs["a_qkv"] = torch.empty((1, sum(QKV_SEGS)), dtype=torch.float32, device=dev)
        bufs["att"] = torch.empty(H, dtype=torch.float32, device=dev)
        bufs["q_o"] = torch.empty((1, H), dtype=torch.int8, device=dev)
        bufs["a_o"] = torch.empty(1, dtype=torch.float32, device=dev)
        bufs["a_y_o"] = torch.empty((1, H), dtype=torch.float32, device=dev)
    y_qkv, att, q_o, a_o, y_o = bufs["a_qkv"], bufs["att"], bufs["q_o"], bufs["a_o"], bufs["a_y_o"]
    bl.gemv_w2a8(x, lw.packed_qkv, lw.w_qkv, seg_n=QKV_SEGS, y=y_qkv)
    row = y_qkv[0]
    bl.attn_decode(row[:H], row[H:H + KV], row[H + KV:], pos, cache.k[layer], cache.v[layer],
                   cache.rope_cos, cache.rope_sin, N_HEADS, N_KV_HEADS, out=att)
    bl.subln_gemv_w2a8(att.view(1, H), lw.packed_o, lw.w_o, eps=eps, y=y_o,
                       q_out=q_o if debug is not None else None, a_out=a_o if debug is not None else None)
    if debug is not None:
        debug.update(y_qkv=y_qkv.clone(), att=att.clone(), q_o=q_o.clone(), a_o=a_o.clone(), y_o=y_o.clone())
    return bl.ffn_chain(y_o, lw.packed_gu, lw.w_gu, lw.packed_down, lw.w_down, eps=eps, y=out)


def decode_step_attn(x: torch.Tensor, layers, cache: KVCache, pos: int, eps: float = 1e-5, bufs: dict = None):
    """All layers at one token with attention; returns the last layer's output."""
    if bufs is None:
        bufs = {}
    outs = bufs.get("outs1")
    if outs is None:
        outs = [torch.empty((1, H), dtype=torch.float32, device=x.device) for _ in range(2)]
        bufs["outs1"] = outs
    cur = x
    for i, lw in enumerate(layers):
        cur = decode_layer_attn(cur, lw, cache, i, pos, eps, out=outs[i & 1], bufs=bufs)
    return cur


def prefill_layer_attn(x: torch.Tensor, lw: LayerWeights, cache: KVCache, layer: int, eps: float = 1e-5,
                       out: torch.Tensor = None, bufs: dict = None, debug: dict = None):
    """One layer over a prompt of M tokens at positions 0 .. M-1 with
    attention (the prefill counterpart of decode_layer_attn): x [M,H] ->
    [M,H] fp32; the layer's caches receive positions 0 .. M-1."""
    M = x.shape[0]
    if M > cache.max_seq:
        raise ValueError("the prompt is longer than the cache")
    dev = x.device
    if bufs is None:
        bufs = {}
    if bufs.get("p_m") != M:
        bufs["p_m"] = M
        bufs["p_qkv"] = torch.empty((M, sum(QKV_SEGS)), dtype=torch.float32, device=dev)
        bufs["p_att"] = torch.empty((M, H), dtype=torch.float32, device=dev)
        bufs["p_y_o"] = torch.empty((M, H), dtype=torch.float32, device=dev)
    y_qkv, att, y_o = bufs["p_qkv"], bufs["p_att"], bufs["p_y_o"]
    _contract(M)(x, lw.packed_qkv, lw.w_qkv, seg_n=QKV_SEGS, y=y_qkv)
    bl.attn_prefill(y_qkv[:, :H], y_qkv[:, H:H + KV], y_qkv[:, H + KV:], cache.k[layer], cache.v[layer],
                    cache.rope_cos, cache.rope_sin, N_HEADS, N_KV_HEADS, out=att)
    q_o = a_o = None
    if debug is not None:
        q_o = torch.empty((M, H), dtype=torch.int8, device=dev)
        a_o = torch.empty(M, dtype=torch.float32, device=dev)
    bl.subln_gemv_w2a8(att, lw.packed_o, lw.w_o, eps=eps, y=y_o, q_out=q_o, a_out=a_o)
    if debug is not None:
        debug.update(y_qkv=y_qkv.clone(), att=att.clone(), q_o=q_o, a_o=a_o, y_o=y_o.clone())
    return bl.ffn_chain(y_o, lw.packed_gu, lw.w_gu, lw.packed_down, lw.w_down, eps=eps, y=out)


def prefill_attn(x: torch.Tensor, layers, cache: KVCache, eps: float = 1e-5, bufs: dict = None):
    """All layers over a prompt with attention; returns the last layer's output."""
    if bufs is None:
        bufs = {}
    M = x.shape[0]
    outs = bufs.get("p_outs")
    if outs is None or outs[0].shape[0] != M:
        outs = [torch.empty((M, H), dtype=torch.float32, device=x.device) for _ in range(2)]
        bufs["p_outs"] = outs
    cur = x
    for i, lw in enumerate(layers):
        cur = prefill_layer_attn(cur, lw, cache, i, eps, out=outs[i & 1], bufs=bufs)
    return cur
