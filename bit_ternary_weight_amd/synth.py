"""Seeded synthetic inputs for the BitLinear W1.58A8 hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scales, no rounding to codes, no packing).  Both the
HIP path (through the tests and the benchmark) and the CPU oracle are fed from
here, so the two sides always see the same bits.

Shapes follow the BitNet b1.58 2B4T configuration listed on the Transformers
model-doc pages for BitNet ("BitNetConfig": hidden 2560, intermediate 6912,
30 layers, 20 query heads / 5 key-value heads, head_dim 128).

Generators
----------
Every array comes from ``numpy.random.default_rng`` (PCG64) seeded with a
``SeedSequence(seed, spawn_key=(stream,))``; stream 0 draws weights and
stream 1 draws activations, so "seed 0 for both" still gives two independent
streams.

* master weights: fp32 normal with mean 0 and std 0.02 (the model config's
  initializer range; drawn plain, not truncated).
* plain activations: fp32 standard normal.
* outlier activations: fp32 standard normal, each element independently
  multiplied by 20 with probability 0.01, then rounded to bf16
  (round-to-nearest-even on the fp32 bit pattern).
* heavy-tail activations: the outlier recipe, except that 8 evenly spaced
  token rows (row ``j*M//8`` for j = 0..7) are Student-t with 3 degrees of
  freedom.

Layer weights use seed ``1000 + 16*layer + j`` with j the projection index in
the order q, k, v, o, gate, up, down.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HIDDEN = 2560
INTERMEDIATE = 6912
N_LAYERS = 30
N_HEADS = 20
N_KV_HEADS = 5
HEAD_DIM = 128
KV_DIM = N_KV_HEADS * HEAD_DIM  # 640

WEIGHT_STD = 0.02

# (name, N = out features, K = in features) of one decoder layer.
PROJECTIONS = (
    ("q", HIDDEN, HIDDEN),
    ("k", KV_DIM, HIDDEN),
    ("v", KV_DIM, HIDDEN),
    ("o", HIDDEN, HIDDEN),
    ("gate", INTERMEDIATE, HIDDEN),
    ("up", INTERMEDIATE, HIDDEN),
    ("down", HIDDEN, INTERMEDIATE),
)
PROJ_INDEX = {name: j for j, (name, _, _) in enumerate(PROJECTIONS)}

STREAM_WEIGHTS = 0
STREAM_ACTS = 1


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream,)))


def layer_seed(layer: int, proj: str) -> int:
    return 1000 + 16 * layer + PROJ_INDEX[proj]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Finite input."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def master_weight(seed: int, N: int, K: int, std: float = WEIGHT_STD) -> np.ndarray:
    g = rng(seed, STREAM_WEIGHTS)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def layer_weight(layer: int, proj: str) -> np.ndarray:
    _, N, K = PROJECTIONS[PROJ_INDEX[proj]]
    return master_weight(layer_seed(layer, proj), N, K)


def act_normal_f32(seed: int, M: int, K: int) -> np.ndarray:
    return rng(seed, STREAM_ACTS).standard_normal((M, K), dtype=np.float32)


def act_outliers_bf16(seed: int, M: int, K: int, p: float = 0.01, mult: float = 20.0) -> np.ndarray:
    """bf16 bits [M,K]: N(0,1) with per-element Bernoulli(p) outliers times `mult`."""
    g = rng(seed, STREAM_ACTS)
    x = g.standard_normal((M, K), dtype=np.float32)
    hit = g.random((M, K), dtype=np.float32) < np.float32(p)
    x[hit] *= np.float32(mult)
    return bf16_bits(x)


def act_heavy_tail_bf16(seed: int, M: int, K: int, nu: float = 3.0, rows: int = 8) -> np.ndarray:
    """bf16 bits [M,K]: the outlier recipe, with `rows` evenly spaced Student-t rows."""
    g = rng(seed, STREAM_ACTS)
    x = g.standard_normal((M, K), dtype=np.float32)
    hit = g.random((M, K), dtype=np.float32) < np.float32(0.01)
    x[hit] *= np.float32(20.0)
    heavy = sorted({j * M // rows for j in range(rows)})
    for r in heavy:
        x[r] = g.standard_t(nu, size=K).astype(np.float32)
    return bf16_bits(x)


def act_heavy_in_row_bf16(seed: int, M: int, K: int, nu: float = 3.0, per_row: int = 8) -> np.ndarray:
    """Alternative reading of the heavy-tail mix: `per_row` Student-t entries inside every row."""
    g = rng(seed, STREAM_ACTS)
    x = g.standard_normal((M, K), dtype=np.float32)
    for r in range(M):
        cols = g.choice(K, size=min(per_row, K), replace=False)
        x[r, cols] = g.standard_t(nu, size=cols.size).astype(np.float32)
    return bf16_bits(x)


def act_normal_bf16(seed: int, M: int, K: int) -> np.ndarray:
    return bf16_bits(act_normal_f32(seed, M, K))


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    desc: str


CONFIGS = (
    Config(1, "single", "single BitLinear M=4 K=256 N=256, fp32 weights N(0,0.02), fp32 x N(0,1), seed 0"),
    Config(2, "decode_m1", "decode GEMV M=1 over the 7 projections of one 2B4T layer, bf16 x with 1% x20 outliers"),
    Config(3, "decode_m16_m64", "batched decode M=16 and M=64, same shapes, 8 Student-t(3) rows per batch"),
    Config(4, "prefill_ffn_m2048", "prefill M=2048: fused gate|up 2560->2x6912, then down 6912->2560"),
    Config(5, "stack30", "30-layer linear stack (attention excluded) at M=4096 prefill and M=1 decode"),
)


def bitlinear_m4_k256_n256():
    """The small parity case's inputs: (W fp32 [256,256], x fp32 [4,256])."""
    W = master_weight(0, 256, 256)
    x = act_normal_f32(0, 4, 256)
    return W, x
