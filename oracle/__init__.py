"""CPU oracle for the BitLinear W1.58A8 forward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never does.

The arithmetic lives in ``bitlinear_oracle.c`` (plain single-threaded C, each
function citing the page passage it follows); this module builds it with gcc
and marshals numpy arrays through ctypes.  Every function here takes and
returns numpy arrays.

One step is evaluated by a library routine: ``contract_f64`` forms the
integer contraction with numpy's fp64 matrix product.  Every product and
every partial sum there is an integer below 2^53 in magnitude, so the result
is exact in any summation order; it is pinned against the C loop
(``ora_contract``) and brute force.  It serves the full-size parity checks,
where the C loop would take minutes.

Parity status: every function is pinned by tests under ``tests/`` (worked
examples, closed forms, exact rationals, invariants, brute force; the prefill
attention rows against the separately written decode attention).  The layer
wiring used for the 30-layer stack (q output feeding o in place of
attention, no residual) is a convention with no passage behind it: parity
unpinned for that wiring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_int64
    F = ctypes.c_float
    sig = {
        "ora_weight_mean": (F, [P, L]),
        "ora_ternarize": (None, [P, L, F, P]),
        "ora_fake_quant_weight": (None, [P, L, F, P]),
        "ora_pack": (None, [P, I, I, P]),
        "ora_unpack": (L, [P, I, I, P]),
        "ora_quant_act": (None, [P, I, I, P, P]),
        "ora_contract": (L, [P, I, I, P, I, P]),
        "ora_rescale": (None, [P, I, I, P, I, P, P, P]),
        "ora_to_bf16": (None, [P, L, P]),
        "ora_dequant_f64": (None, [P, P, I, I, P, I, I, P, P, P]),
        "ora_rmsnorm": (None, [P, I, I, P, F, P]),
        "ora_relu2_mul": (None, [P, P, L, P]),
        "ora_bitlinear": (None, [P, I, I, P, I, I, P, P, P, P, P, P]),
        "ora_ffn_chain": (None, [P, I, I, I, P, P, F, P, P, P, P, P, P, P, P, P, P]),
        "ora_rope_f64": (None, [P, I, I, I, ctypes.c_double, P]),
        "ora_attn_decode": (None, [P, P, P, I, I, I, I, P, P, I, ctypes.c_double, P]),
        "ora_attn_prefill_f64": (None, [P, P, P, I, I, I, I, ctypes.c_double, P, I, P]),
        "ora_ste_grad_input_rows": (None, [P, I, I, P, I, F, P, I, P]),
        "ora_ste_grad_weight_rows": (None, [P, I, I, P, P, I, P, I, P]),
        "ora_binarize": (None, [P, L, P]),
        "ora_pack_bits": (None, [P, I, I, P]),
        "ora_unpack_bits": (None, [P, I, I, P]),
        "ora_layernorm": (None, [P, I, I, P, P, F, P]),
        "ora_bitlinear_w1": (None, [P, I, I, P, P, F, P, I, F, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def weight_mean(W) -> np.float32:
    W = _c(W, np.float32)
    return np.float32(_load().ora_weight_mean(_p(W), W.size))


def ternarize(W, w_mean) -> np.ndarray:
    W = _c(W, np.float32)
    out = np.empty(W.shape, np.int8)
    _load().ora_ternarize(_p(W), W.size, float(np.float32(w_mean)), _p(out))
    return out


def fake_quant_weight(codes, w_mean) -> np.ndarray:
    codes = _c(codes, np.int8)
    out = np.empty(codes.shape, np.float32)
    _load().ora_fake_quant_weight(_p(codes), codes.size, float(np.float32(w_mean)), _p(out))
    return out


def pack(codes) -> np.ndarray:
    codes = _c(codes, np.int8)
    N, K = codes.shape
    assert N % 4 == 0
    out = np.empty((N // 4, K), np.uint8)
    _load().ora_pack(_p(codes), N, K, _p(out))
    return out


def unpack(packed, N=None):
    packed = _c(packed, np.uint8)
    R, K = packed.shape
    N = 4 * R if N is None else N
    out = np.empty((N, K), np.int8)
    bad = _load().ora_unpack(_p(packed), N, K, _p(out))
    return out, int(bad)


def ternarize_pack(W):
    """(packed [N/4,K] uint8, w_mean float32, codes [N,K] int8) for one tensor."""
    wm = weight_mean(W)
    codes = ternarize(W, wm)
    return pack(codes), wm, codes


def quant_act(x):
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    a = np.empty(M, np.float32)
    _load().ora_quant_act(_p(x), M, K, _p(q), _p(a))
    return q, a


def contract(q, codes) -> np.ndarray:
    q = _c(q, np.int8)
    codes = _c(codes, np.int8)
    M, K = q.shape
    N, K2 = codes.shape
    assert K == K2
    A = np.empty((M, N), np.int32)
    ovf = _load().ora_contract(_p(q), M, K, _p(codes), N, _p(A))
    assert ovf == 0, "int32 overflow in the contraction"
    return A


def contract_f64(q, codes) -> np.ndarray:
    """The same integer contraction as ``contract`` (sum_k q[m,k] c[n,k]),
    evaluated by numpy's fp64 matrix product.  |q| <= 128 and |c| <= 1, so
    every partial sum is an integer of magnitude <= 128 K < 2^53 for K < 2^45:
    each addition is exact and the order the library takes does not matter."""
    q = np.asarray(q, np.int8)
    codes = np.asarray(codes, np.int8)
    assert q.shape[1] == codes.shape[1] and q.shape[1] < (1 << 45)
    A = q.astype(np.float64) @ codes.astype(np.float64).T
    assert np.abs(A).max(initial=0) < 2.0 ** 31, "int32 overflow in the contraction"
    return A.astype(np.int32)


def bitlinear_f64gemm(x, codes, seg_n=None, w_mean=None):
    """``bitlinear`` with the contraction taken by ``contract_f64``: the C
    quantizer, the exact integer product, the C rescale.  Returns (q, a, A, y)."""
    q, a = quant_act(x)
    A = contract_f64(q, codes)
    N = codes.shape[0]
    return q, a, A, rescale(A, a, seg_n if seg_n is not None else [N], w_mean)


def _segs(seg_n, N):
    seg = np.ascontiguousarray(np.asarray(seg_n if seg_n is not None else [N], dtype=np.int32))
    assert int(seg.sum()) == N
    return seg


def rescale(A, a, seg_n, w_mean) -> np.ndarray:
    A = _c(A, np.int32)
    a = _c(a, np.float32)
    M, N = A.shape
    seg = _segs(seg_n, N)
    wm = _c(np.atleast_1d(w_mean), np.float32)
    y = np.empty((M, N), np.float32)
    _load().ora_rescale(_p(A), M, N, _p(a), seg.size, _p(seg), _p(wm), _p(y))
    return y


def to_bf16(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint16)
    _load().ora_to_bf16(_p(y), y.size, _p(out))
    return out


def dequant_f64(q, a, codes, seg_n, w_mean) -> np.ndarray:
    q = _c(q, np.int8)
    a = _c(a, np.float32)
    codes = _c(codes, np.int8)
    M, K = q.shape
    N = codes.shape[0]
    seg = _segs(seg_n, N)
    wm = _c(np.atleast_1d(w_mean), np.float32)
    y = np.empty((M, N), np.float64)
    _load().ora_dequant_f64(_p(q), _p(a), M, K, _p(codes), N, seg.size, _p(seg), _p(wm), _p(y))
    return y


def rmsnorm(h, g=None, eps=1e-5) -> np.ndarray:
    h = _c(h, np.float32)
    M, K = h.shape
    g = None if g is None else _c(g, np.float32)
    out = np.empty((M, K), np.float32)
    _load().ora_rmsnorm(_p(h), M, K, _p(g), float(np.float32(eps)), _p(out))
    return out


def relu2_mul(gate, up) -> np.ndarray:
    gate = _c(gate, np.float32)
    up = _c(up, np.float32)
    assert gate.shape == up.shape
    p = np.empty(gate.shape, np.float32)
    _load().ora_relu2_mul(_p(gate), _p(up), gate.size, _p(p))
    return p


def bitlinear(x, codes, seg_n=None, w_mean=None):
    """(q, a, A, y) of one BitLinear forward on fp32 x [M,K], codes [N,K]."""
    x = _c(x, np.float32)
    codes = _c(codes, np.int8)
    M, K = x.shape
    N = codes.shape[0]
    seg = _segs(seg_n, N)
    wm = _c(np.atleast_1d(w_mean), np.float32)
    q = np.empty((M, K), np.int8)
    a = np.empty(M, np.float32)
    A = np.empty((M, N), np.int32)
    y = np.empty((M, N), np.float32)
    _load().ora_bitlinear(_p(x), M, K, _p(codes), N, seg.size, _p(seg), _p(wm),
                          _p(q), _p(a), _p(A), _p(y))
    return q, a, A, y


def ffn_chain(h, codes_gu, w_mean_gu, codes_down, w_mean_down, g_subln=None, g_ffn=None, eps=1e-5):
    """dict(q1, a1, p, q2, a2, y) of the FFN chain on fp32 h [M,H]."""
    h = _c(h, np.float32)
    M, H = h.shape
    codes_gu = _c(codes_gu, np.int8)
    codes_down = _c(codes_down, np.int8)
    I = codes_gu.shape[0] // 2
    assert codes_gu.shape == (2 * I, H) and codes_down.shape == (H, I)
    wgu = _c(np.asarray(w_mean_gu).reshape(2), np.float32)
    wd = _c(np.atleast_1d(w_mean_down), np.float32)
    gs = None if g_subln is None else _c(g_subln, np.float32)
    gf = None if g_ffn is None else _c(g_ffn, np.float32)
    out = dict(q1=np.empty((M, H), np.int8), a1=np.empty(M, np.float32),
               p=np.empty((M, I), np.float32), q2=np.empty((M, I), np.int8),
               a2=np.empty(M, np.float32), y=np.empty((M, H), np.float32))
    _load().ora_ffn_chain(_p(h), M, H, I, _p(gs), _p(gf), float(np.float32(eps)),
                          _p(codes_gu), _p(wgu), _p(codes_down), _p(wd),
                          _p(out["q1"]), _p(out["a1"]), _p(out["p"]), _p(out["q2"]),
                          _p(out["a2"]), _p(out["y"]))
    return out


def ffn_chain_f64gemm(h, codes_gu, w_mean_gu, codes_down, w_mean_down, g_subln=None, g_ffn=None, eps=1e-5):
    """``ffn_chain`` composed from the C stage functions with the two
    contractions taken by ``contract_f64`` (same stages, same order, the
    exact integer products): dict(q1, a1, p, q2, a2, y)."""
    h = _c(h, np.float32)
    I = np.asarray(codes_gu).shape[0] // 2
    wgu = _c(np.asarray(w_mean_gu).reshape(2), np.float32)
    q1, a1, _, ygu = bitlinear_f64gemm(rmsnorm(h, g_subln, eps), codes_gu, [I, I], wgu)
    p = relu2_mul(np.ascontiguousarray(ygu[:, :I]), np.ascontiguousarray(ygu[:, I:]))
    q2, a2, _, y = bitlinear_f64gemm(rmsnorm(p, g_ffn, eps), codes_down, None, w_mean_down)
    return dict(q1=q1, a1=a1, p=p, q2=q2, a2=a2, y=y)


def layer_f64gemm(x, codes, w_means, eps=1e-5):
    """``layer`` with every contraction taken by ``contract_f64``."""
    qkv_codes = np.concatenate([codes["q"], codes["k"], codes["v"]], axis=0)
    segs = [codes["q"].shape[0], codes["k"].shape[0], codes["v"].shape[0]]
    wm = np.array([w_means["q"], w_means["k"], w_means["v"]], np.float32)
    q0, a0, _, y_qkv = bitlinear_f64gemm(x, qkv_codes, segs, wm)
    y_q = np.ascontiguousarray(y_qkv[:, :segs[0]])
    q_o, a_o, _, y_o = bitlinear_f64gemm(y_q, codes["o"], None, w_means["o"])
    gu = np.concatenate([codes["gate"], codes["up"]], axis=0)
    ch = ffn_chain_f64gemm(y_o, gu, np.array([w_means["gate"], w_means["up"]], np.float32),
                           codes["down"], w_means["down"], eps=eps)
    return dict(q_in=q0, a_in=a0, y_qkv=y_qkv, q_o=q_o, a_o=a_o, y_o=y_o, **ch)


def layer(x, codes, w_means, eps=1e-5, g_subln=None, g_ffn=None):
    """One decoder layer's linear path (attention excluded), fp32 x [M,2560].

    codes: dict proj -> [N,K] int8; w_means: dict proj -> float32; g_subln,
    g_ffn: the FFN chain's RMSNorm gains, or None (unit gain).
    Wiring (a convention, parity unpinned by the pages): quantize x -> fused
    q|k|v -> q's output is re-quantized and fed to o -> FFN chain on o's
    output.  No residual additions.  Returns dict of stage outputs.
    """
    qkv_codes = np.concatenate([codes["q"], codes["k"], codes["v"]], axis=0)
    segs = [codes["q"].shape[0], codes["k"].shape[0], codes["v"].shape[0]]
    wm = np.array([w_means["q"], w_means["k"], w_means["v"]], np.float32)
    q0, a0, A0, y_qkv = bitlinear(x, qkv_codes, segs, wm)
    y_q = np.ascontiguousarray(y_qkv[:, :segs[0]])
    q_o, a_o, A_o, y_o = bitlinear(y_q, codes["o"], None, w_means["o"])
    gu = np.concatenate([codes["gate"], codes["up"]], axis=0)
    ch = ffn_chain(y_o, gu, np.array([w_means["gate"], w_means["up"]], np.float32),
                   codes["down"], w_means["down"], g_subln=g_subln, g_ffn=g_ffn, eps=eps)
    return dict(q_in=q0, a_in=a0, y_qkv=y_qkv, q_o=q_o, a_o=a_o, y_o=y_o, **ch)


def rope(x, pos, base):
    """RoPE (split-half pairing) of x [heads, D] at position pos, fp64."""
    x = _c(x, np.float64)
    nh, D = x.shape
    y = np.empty((nh, D), np.float64)
    _load().ora_rope_f64(_p(x), nh, D, int(pos), float(base), _p(y))
    return y


def attn_decode(q, k_new, v_new, pos, k_cache, v_cache, base, n_heads, n_kv_heads):
    """fp64 attention output [n_heads, D] of one new token at position pos.

    q [H*D], k_new / v_new [KVH*D] fp32 (before RoPE); k_cache / v_cache
    [KVH, max_seq, D] fp32, positions < pos used (rotated keys)."""
    q = _c(np.asarray(q).reshape(-1), np.float32)
    k_new = _c(np.asarray(k_new).reshape(-1), np.float32)
    v_new = _c(np.asarray(v_new).reshape(-1), np.float32)
    k_cache = _c(k_cache, np.float32)
    v_cache = _c(v_cache, np.float32)
    KVH, S, D = k_cache.shape
    assert KVH == n_kv_heads and q.size == n_heads * D and 0 <= pos < S
    out = np.empty((n_heads, D), np.float64)
    _load().ora_attn_decode(_p(q), _p(k_new), _p(v_new), int(pos), n_heads, n_kv_heads, D,
                            _p(k_cache), _p(v_cache), S, float(base), _p(out))
    return out


def bf16_round(x) -> np.ndarray:
    """fp32 values of x rounded to bf16 (nearest even), via to_bf16."""
    b = to_bf16(np.asarray(x, np.float32))
    return (b.astype(np.uint32) << 16).view(np.float32)


def attn_prefill_rows(q, k, v, base, n_heads, n_kv_heads, rows):
    """fp64 causal attention outputs [len(rows), n_heads*D] of a prompt whose
    tokens sit at positions 0 .. M-1: the plain definition, nothing rounded.

    q [M, n_heads*D], k / v [M, n_kv_heads*D] fp32, before RoPE.  Row p
    attends to positions 0 .. p with scores q'.k'/sqrt(D) of the fp64
    rotations; query head h reads key/value head h // (n_heads/n_kv_heads)."""
    q = _c(q, np.float32)
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    M = q.shape[0]
    D = q.shape[1] // n_heads
    assert k.shape == (M, n_kv_heads * D) and v.shape == k.shape and n_heads % n_kv_heads == 0
    r = _c(np.asarray(rows).reshape(-1), np.int32)
    assert r.size and r.min() >= 0 and r.max() < M
    out = np.empty((r.size, n_heads * D), np.float64)
    _load().ora_attn_prefill_f64(_p(q), _p(k), _p(v), M, n_heads, n_kv_heads, D, float(base), _p(r), r.size,
                                 _p(out))
    return out


def _rows(rows, n):
    r = np.arange(n, dtype=np.int32) if rows is None else _c(np.asarray(rows).reshape(-1), np.int32)
    assert r.size == 0 or (r.min() >= 0 and r.max() < n)
    return r


def ste_grad_input(dy, codes, w_mean, rows=None) -> np.ndarray:
    """fp64 rows of dX = dY . W~ of BitLinear's straight-through backward,
    W~ = codes * w_mean: dx[m,k] = sum_n dy[m,n] (codes[n,k] w_mean) for the
    token rows m in `rows` (all when None).  dy [M,N] fp32; codes [N,K]."""
    dy = _c(dy, np.float32)
    codes = _c(codes, np.int8)
    M, N = dy.shape
    N2, K = codes.shape
    assert N == N2
    r = _rows(rows, M)
    out = np.empty((r.size, K), np.float64)
    _load().ora_ste_grad_input_rows(_p(dy), M, N, _p(codes), K, float(np.float32(w_mean)), _p(r), r.size, _p(out))
    return out


def ste_grad_weight(dy, q, a, rows=None) -> np.ndarray:
    """fp64 rows of dW = dY^T . x~ of the straight-through backward,
    x~ = q / a: dw[n,k] = sum_m dy[m,n] (q[m,k] / a[m]) for the weight rows n
    in `rows` (all when None).  dy [M,N] fp32; q [M,K] int8; a [M] fp32."""
    dy = _c(dy, np.float32)
    q = _c(q, np.int8)
    a = _c(a, np.float32)
    M, N = dy.shape
    M2, K = q.shape
    assert M == M2 and a.shape == (M,)
    r = _rows(rows, N)
    out = np.empty((r.size, K), np.float64)
    _load().ora_ste_grad_weight_rows(_p(dy), M, N, _p(q), _p(a), K, _p(r), r.size, _p(out))
    return out


# ---------------------------------------------------------------------------
# The 1-bit BitLinear (binarized weights): layer norm, signs with one scale
# per tensor, absmax int8 activations.
# ---------------------------------------------------------------------------
def binarize_pack(W):
    """(packed [N/8,K] uint8, w_scale float32, signs [N,K] int8) for one tensor."""
    W = _c(W, np.float32)
    N, K = W.shape
    assert N % 8 == 0
    signs = np.empty((N, K), np.int8)
    _load().ora_binarize(_p(W), W.size, _p(signs))
    packed = np.empty((N // 8, K), np.uint8)
    _load().ora_pack_bits(_p(signs), N, K, _p(packed))
    return packed, weight_mean(W), signs


def unpack_bits(packed, N=None):
    packed = _c(packed, np.uint8)
    R, K = packed.shape
    N = 8 * R if N is None else N
    signs = np.empty((N, K), np.int8)
    _load().ora_unpack_bits(_p(packed), N, K, _p(signs))
    return signs


def layernorm(x, gamma=None, beta=None, eps=1e-5) -> np.ndarray:
    x = _c(x, np.float32)
    M, K = x.shape
    gamma = None if gamma is None else _c(gamma, np.float32)
    beta = None if beta is None else _c(beta, np.float32)
    out = np.empty((M, K), np.float32)
    _load().ora_layernorm(_p(x), M, K, _p(gamma), _p(beta), float(np.float32(eps)), _p(out))
    return out


def bitlinear_w1(x, signs, w_scale, gamma=None, beta=None, eps=1e-5):
    """(q, a, A, y) of one 1-bit BitLinear forward on fp32 x [M,K], signs [N,K]."""
    x = _c(x, np.float32)
    signs = _c(signs, np.int8)
    M, K = x.shape
    N = signs.shape[0]
    gamma = None if gamma is None else _c(gamma, np.float32)
    beta = None if beta is None else _c(beta, np.float32)
    q = np.empty((M, K), np.int8)
    a = np.empty(M, np.float32)
    A = np.empty((M, N), np.int32)
    y = np.empty((M, N), np.float32)
    _load().ora_bitlinear_w1(_p(x), M, K, _p(gamma), _p(beta), float(np.float32(eps)), _p(signs), N,
                             float(np.float32(w_scale)), _p(q), _p(a), _p(A), _p(y))
    return q, a, A, y


def bitlinear_w1_f64gemm(x, signs, w_scale, gamma=None, beta=None, eps=1e-5):
    """``bitlinear_w1`` with the contraction taken by ``contract_f64`` (exact:
    |q| <= 128, |sign| = 1, integer partial sums below 2^53)."""
    q, a = quant_act(layernorm(x, gamma, beta, eps))
    A = contract_f64(q, signs)
    return q, a, A, rescale(A, a, [signs.shape[0]], w_scale)
