"""Thin Python binding of libbitlinear (include/bitlinear.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  Importing this module fails loudly when libbitlinear.so has not been
built -- there is no CPU fallback.

The functions keep the names of the C entry points (ternarize_pack,
quant_act, gemv_w2a8, gemm_w2a8, ffn_chain); ``raw`` exposes the ctypes
handle for callers that want the C signatures directly.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# BL_LIBRARY names another build of the same library (for example one whose
# host code carries sanitizers); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("BL_LIBRARY") or os.path.join(_HERE, "libbitlinear.so")

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_SEGMENTS, BL_ERR_WORKSPACE, BL_ERR_HIP = range(8)
BL_F32, BL_BF16, BL_I8, BL_I32 = range(4)
MAX_SEGMENTS = 8

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libbitlinear.so not found at {LIB_PATH}; build it first "
        "(python -m bit_ternary_weight_amd.build or __graft_entry__.build())")

raw = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_S = ctypes.c_size_t
_F = ctypes.c_float


class FfnDebug(ctypes.Structure):
    _fields_ = [("q1", _P), ("a1", _P), ("p", _P), ("q2", _P), ("a2", _P)]


class Layer(ctypes.Structure):
    _fields_ = [("packed_qkv", _P), ("w_qkv", _P), ("packed_o", _P), ("w_o", _P), ("packed_gu", _P), ("w_gu", _P),
                ("packed_down", _P), ("w_down", _P), ("g_subln", _P), ("g_ffn", _P)]


class GemvProblem(ctypes.Structure):
    _fields_ = [("x", _P), ("x_dtype", _I), ("ldx", _I), ("a", _P), ("M", _I), ("K", _I),
                ("packed", _P), ("N", _I), ("n_seg", _I), ("seg_n", ctypes.POINTER(_I)), ("w_mean", _P),
                ("y", _P), ("y_dtype", _I)]


class W1Problem(ctypes.Structure):
    _fields_ = [("x", _P), ("x_dtype", _I), ("M", _I), ("K", _I), ("gamma", _P), ("beta", _P),
                ("packed", _P), ("N", _I), ("w_scale", _P), ("y", _P)]


MAX_PROBLEMS = 8


_SIGS = {
    "bl_abi_version": (_I, []),
    "bl_device_errors": (_I, [ctypes.POINTER(ctypes.c_uint), _I]),
    "bl_status_string": (ctypes.c_char_p, [_I]),
    "bl_last_error": (ctypes.c_char_p, []),
    "bl_ternarize_workspace_bytes": (_S, [_L, _L]),
    "bl_ternarize_pack": (_I, [_P, _I, _I, _P, _P, _P, _S, _P]),
    "bl_quant_act": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "bl_rmsnorm_quant": (_I, [_P, _I, _I, _I, _P, ctypes.c_float, _P, _P, _P]),
    "bl_attn_prefill_workspace_bytes": (_S, [_I, _I, _I]),
    "bl_ste_grad_input_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "bl_ste_grad_weight_workspace_bytes": (_S, [_I, _I, _I]),
    "bl_ste_grad_input": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _S, _P]),
    "bl_ste_grad_weight": (_I, [_P, _I, _P, _P, _I, _I, _I, _P, _P, _S, _P]),
    "bl_attn_prefill": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _I, _P, _S, _P]),
    "bl_subln_gemv_workspace_bytes": (_S, [_I, _I]),
    "bl_subln_gemv_w2a8": (_I, [_P, _I, _I, _I, _P, ctypes.c_float, _P, _I, _P, _P, _I, _P, _P, _P, _S, _P]),
    "bl_gemv_workspace_bytes": (_S, [_I, _I, _I]),
    "bl_gemv_w2a8": (_I, [_P, _I, _I, _P, _I, _I, _P, _I, _I, _P, _P, _P, _I, _P, _S, _P]),
    "bl_gemv_batched_workspace_bytes": (_S, [_I, ctypes.POINTER(GemvProblem)]),
    "bl_gemv_w2a8_batched": (_I, [_I, ctypes.POINTER(GemvProblem), _P, _S, _P]),
    "bl_gemm_workspace_bytes": (_S, [_I, _I, _I]),
    "bl_gemm_w2a8": (_I, [_P, _I, _I, _P, _I, _I, _P, _I, _I, _P, _P, _P, _I, _P, _S, _P]),
    "bl_ffn_chain_workspace_bytes": (_S, [_I, _I, _I]),
    "bl_ffn_chain": (_I, [_P, _I, _I, _I, _I, _P, _P, _F, _P, _P, _P, _P, _P, _I, _P, _S,
                          ctypes.POINTER(FfnDebug), _P]),
    "bl_unpack_bf16": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "bl_stack_decode_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "bl_stack_decode": (_I, [_P, _I, _I, ctypes.POINTER(Layer), _I, _I, _I, _F, _P, _P, _P, _S, _P]),
    "bl_gemm_unpacked_workspace_bytes": (_S, [_I, _I, _I]),
    "bl_gemm_unpacked": (_I, [_P, _I, _I, _P, _I, _I, _P, _I, _I, _P, _P, _P, _I, _P, _S, _P]),
    "bl_ffn_chain_noalloc_max_bytes": (_S, []),
    "bl_ffn_chain_noalloc": (_I, [_P, _I, _I, _I, _I, _P, _P, _F, _P, _P, _P, _P, _P, _I,
                                  ctypes.POINTER(FfnDebug), _P]),
    "bl_rope_table": (_I, [_I, _I, ctypes.c_double, _P, _P]),
    "bl_attn_decode_workspace_bytes": (_S, [_I, _I]),
    "bl_attn_decode": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _S, _P]),
    "bl_binarize_workspace_bytes": (_S, [_L, _L]),
    "bl_binarize_pack": (_I, [_P, _I, _I, _P, _P, _P, _S, _P]),
    "bl_layernorm_quant": (_I, [_P, _I, _I, _I, _I, _P, _P, _F, _P, _P, _P]),
    "bl_gemm_w1a8": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _P]),
    "bl_bitlinear_w1_workspace_bytes": (_S, [ctypes.POINTER(W1Problem), _I]),
    "bl_bitlinear_w1": (_I, [ctypes.POINTER(W1Problem), _I, _F, _P, _S, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(raw, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class BitLinearError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{raw.bl_status_string(status).decode()}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != BL_OK:
        raise BitLinearError(status, raw.bl_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_DT = {torch.float32: BL_F32, torch.bfloat16: BL_BF16, torch.int8: BL_I8, torch.int32: BL_I32}
_TORCH = {v: k for k, v in _DT.items()}


def _dt(t) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on a HIP device")
    return ts[0].device


# ---------------------------------------------------------------------------
# Workspace: one scratch buffer per device, grown on demand.  Calls never read
# what an earlier call left in it.
# ---------------------------------------------------------------------------
_ws_lock = threading.Lock()
_ws: dict = {}


def workspace(device, nbytes: int) -> torch.Tensor:
    key = torch.device(device).index if torch.device(device).index is not None else torch.cuda.current_device()
    with _ws_lock:
        buf = _ws.get(key)
        if buf is None or buf.numel() < nbytes:
            size = max(int(nbytes), 16 << 20)
            buf = torch.empty(size, dtype=torch.uint8, device=device)
            _ws[key] = buf
        return buf


def _need(t, shape, dtypes, name, contiguous=True):
    """Host-side check of a tensor handed to the library: the C ABI takes bare
    pointers, so a buffer of the wrong size would be read or written out of
    bounds on the device instead of failing here."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_OUT_DT = (torch.float32, torch.bfloat16, torch.int32)


def _check_weight(packed, w_mean, N4, K, n_seg, name="packed"):
    _need(packed, (N4, K), (torch.uint8,), name)
    if w_mean.dtype != torch.float32 or w_mean.numel() < n_seg:
        raise ValueError(f"w_mean must be float32 with at least {n_seg} elements")


def _segs(seg_n, N):
    if seg_n is None:
        return 1, None
    seg = (ctypes.c_int * len(seg_n))(*[int(v) for v in seg_n])
    return len(seg_n), seg


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def device_errors(reset: bool = True) -> int:
    """Expired bounded waits counted by the kernels on the current device
    since the last reset (synchronizes the device; see bl_device_errors)."""
    n = ctypes.c_uint(0)
    _check(raw.bl_device_errors(ctypes.byref(n), int(reset)))
    return int(n.value)


def ternarize_pack(W: torch.Tensor, packed: torch.Tensor = None, w_mean: torch.Tensor = None):
    """W fp32 [N,K] -> (packed uint8 [N/4,K], w_mean fp32 [1])."""
    dev = _dev(W)
    N, K = W.shape
    _need(W, (N, K), (torch.float32,), "W")
    if packed is None:
        packed = torch.empty((N // 4, K), dtype=torch.uint8, device=dev)
    if w_mean is None:
        w_mean = torch.empty(1, dtype=torch.float32, device=dev)
    _need(packed, (N // 4, K), (torch.uint8,), "packed")
    _need(w_mean, (1,), (torch.float32,), "w_mean")
    nbytes = raw.bl_ternarize_workspace_bytes(N, K)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(raw.bl_ternarize_pack(_ptr(W), N, K, _ptr(packed), _ptr(w_mean), _ptr(ws), ws.numel(), _stream(dev)))
    return packed, w_mean


def quant_act(x: torch.Tensor, q: torch.Tensor = None, a: torch.Tensor = None):
    """x [M,K] fp32/bf16 (row stride may exceed K) -> (q int8 [M,K], a fp32 [M])."""
    dev = _dev(x)
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
    if a is None:
        a = torch.empty(M, dtype=torch.float32, device=dev)
    _need(q, (M, K), (torch.int8,), "q")
    _need(a, (M,), (torch.float32,), "a")
    _check(raw.bl_quant_act(_ptr(x), _dt(x), M, K, x.stride(0), _ptr(q), _ptr(a), _stream(dev)))
    return q, a


def rmsnorm_quant(h: torch.Tensor, gain: torch.Tensor = None, eps: float = 1e-5, q: torch.Tensor = None,
                  a: torch.Tensor = None):
    """RMSNorm of each row of h [M,K] (contiguous fp32/bf16, optional gain
    [K]) then per-token int8 quantization -> (q int8 [M,K], a fp32 [M])."""
    dev = _dev(h)
    M, K = h.shape
    if not h.is_contiguous():
        raise ValueError("h must be contiguous")
    if gain is not None:
        _need(gain, (K,), (torch.float32,), "gain")
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
    if a is None:
        a = torch.empty(M, dtype=torch.float32, device=dev)
    _need(q, (M, K), (torch.int8,), "q")
    _need(a, (M,), (torch.float32,), "a")
    _check(raw.bl_rmsnorm_quant(_ptr(h), _dt(h), M, K, None if gain is None else _ptr(gain), float(eps),
                                _ptr(q), _ptr(a), _stream(dev)))
    return q, a


def subln_gemv_w2a8(h: torch.Tensor, packed: torch.Tensor, w_mean: torch.Tensor, gain: torch.Tensor = None,
                    eps: float = 1e-5, y_dtype=torch.float32, y: torch.Tensor = None, q_out: torch.Tensor = None,
                    a_out: torch.Tensor = None):
    """y = BitLinear(RMSNorm(h)) for h [M,K] contiguous fp32/bf16, one weight
    segment; q_out / a_out optionally receive the codes and scales."""
    dev = _dev(h, packed, w_mean)
    M, K = h.shape
    if not h.is_contiguous():
        raise ValueError("h must be contiguous")
    N = packed.shape[0] * 4
    _need(packed, (N // 4, K), (torch.uint8,), "packed")
    _need(w_mean, (1,), (torch.float32,), "w_mean")
    if gain is not None:
        _need(gain, (K,), (torch.float32,), "gain")
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=dev)
    _need(y, (M, N), (y_dtype,), "y")
    if q_out is not None:
        _need(q_out, (M, K), (torch.int8,), "q_out")
    if a_out is not None:
        _need(a_out, (M,), (torch.float32,), "a_out")
    ws = workspace(dev, raw.bl_subln_gemv_workspace_bytes(M, K))
    _check(raw.bl_subln_gemv_w2a8(_ptr(h), _dt(h), M, K, None if gain is None else _ptr(gain), float(eps),
                                  _ptr(packed), N, _ptr(w_mean), _ptr(y), _dt(y),
                                  None if q_out is None else _ptr(q_out), None if a_out is None else _ptr(a_out),
                                  _ptr(ws), ws.numel(), _stream(dev)))
    return y


def _contract(fn_name, ws_query, x, packed, w_mean, seg_n=None, y_dtype=torch.float32, a=None, y=None):
    dev = _dev(x, packed, w_mean)
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    N = packed.shape[0] * 4
    n_seg, seg = _segs(seg_n, N)
    _check_weight(packed, w_mean, N // 4, K, n_seg)
    if a is not None and (a.dtype != torch.float32 or a.numel() < M):
        raise ValueError("a must be float32 with at least M elements")
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=dev)
    _need(y, (M, N), _OUT_DT, "y")
    nbytes = ws_query(M, N, K)
    ws = workspace(dev, nbytes)
    fn = getattr(raw, fn_name)
    _check(fn(_ptr(x), _dt(x), x.stride(0), _ptr(a), M, K, _ptr(packed), N, n_seg, seg, _ptr(w_mean),
              _ptr(y), _dt(y), _ptr(ws), ws.numel(), _stream(dev)))
    return y


def gemv_w2a8(x, packed, w_mean, seg_n=None, y_dtype=torch.float32, a=None, y=None):
    """Decode BitLinear (M <= 64): y = rescale(quant(x) @ unpack(packed)^T)."""
    return _contract("bl_gemv_w2a8", raw.bl_gemv_workspace_bytes, x, packed, w_mean, seg_n, y_dtype, a, y)


def gemv_w2a8_batched(problems):
    """Up to 8 independent decode contractions in one launch.

    problems: list of dicts with keys x, packed, w_mean and optional seg_n,
    a, y, y_dtype.  Returns the list of outputs (allocated when y is absent).
    """
    if not 1 <= len(problems) <= MAX_PROBLEMS:
        raise ValueError(f"1..{MAX_PROBLEMS} problems per launch")
    arr = (GemvProblem * len(problems))()
    keep, outs = [], []
    dev = None
    for i, pr in enumerate(problems):
        x, packed, w_mean = pr["x"], pr["packed"], pr["w_mean"]
        dev = _dev(x, packed, w_mean)
        if x.stride(1) != 1:
            raise ValueError("x rows must be contiguous")
        M, K = x.shape
        N = packed.shape[0] * 4
        y = pr.get("y")
        if y is None:
            y = torch.empty((M, N), dtype=pr.get("y_dtype", torch.float32), device=dev)
        n_seg, seg = _segs(pr.get("seg_n"), N)
        _check_weight(packed, w_mean, N // 4, K, n_seg)
        _need(y, (M, N), _OUT_DT, "y")
        keep.append(seg)
        a = pr.get("a")
        if a is not None and (a.dtype != torch.float32 or a.numel() < M):
            raise ValueError("a must be float32 with at least M elements")
        arr[i] = GemvProblem(x.data_ptr(), _dt(x), x.stride(0), a.data_ptr() if a is not None else None, M, K,
                             packed.data_ptr(), N, n_seg, seg, w_mean.data_ptr(), y.data_ptr(), _dt(y))
        outs.append(y)
    ws = workspace(dev, raw.bl_gemv_batched_workspace_bytes(len(problems), arr))
    _check(raw.bl_gemv_w2a8_batched(len(problems), arr, _ptr(ws), ws.numel(), _stream(dev)))
    return outs


def gemm_w2a8(x, packed, w_mean, seg_n=None, y_dtype=torch.float32, a=None, y=None):
    """Prefill BitLinear (any M), same arithmetic as gemv_w2a8."""
    return _contract("bl_gemm_w2a8", raw.bl_gemm_workspace_bytes, x, packed, w_mean, seg_n, y_dtype, a, y)


def ffn_chain(h, packed_gu, w_mean_gu, packed_down, w_mean_down, g_subln=None, g_ffn=None, eps=1e-5,
              y_dtype=torch.float32, debug=False, y=None):
    """FFN half of a layer.  Returns y, or (y, dict of stage outputs) with
    debug=True; debug may also be a dict of preallocated stage buffers (q1,
    a1, p, q2, a2; missing ones are allocated)."""
    dev = _dev(h, packed_gu, packed_down)
    M, H = h.shape
    I = packed_gu.shape[0] * 2
    if h.stride(1) != 1 or h.stride(0) != H:
        raise ValueError("h must be contiguous")
    _check_weight(packed_gu, w_mean_gu, I // 2, H, 2, "packed_gu")
    _check_weight(packed_down, w_mean_down, H // 4, I, 1, "packed_down")
    for g, n, name in ((g_subln, H, "g_subln"), (g_ffn, I, "g_ffn")):
        if g is not None:
            _need(g, (n,), (torch.float32,), name)
    if y is None:
        y = torch.empty((M, H), dtype=y_dtype, device=dev)
    _need(y, (M, H), (torch.float32, torch.bfloat16), "y")
    stages = None
    dbg = None
    if debug:
        shapes = dict(q1=((M, H), torch.int8), a1=((M,), torch.float32), p=((M, I), torch.float32),
                      q2=((M, I), torch.int8), a2=((M,), torch.float32))
        given = debug if isinstance(debug, dict) else {}
        stages = {}
        for k, (shp, dt) in shapes.items():
            t = given.get(k)
            if t is None:
                t = torch.empty(shp, dtype=dt, device=dev)
            _need(t, shp, (dt,), k)
            stages[k] = t
        dbg = FfnDebug(*[stages[k].data_ptr() for k in ("q1", "a1", "p", "q2", "a2")])
    nbytes = raw.bl_ffn_chain_workspace_bytes(M, H, I)
    ws = workspace(dev, nbytes)
    _check(raw.bl_ffn_chain(_ptr(h), _dt(h), M, H, I, _ptr(g_subln), _ptr(g_ffn), float(eps),
                            _ptr(packed_gu), _ptr(w_mean_gu), _ptr(packed_down), _ptr(w_mean_down),
                            _ptr(y), _dt(y), _ptr(ws), ws.numel(),
                            ctypes.byref(dbg) if dbg is not None else None, _stream(dev)))
    return (y, stages) if debug else y


STACK_DECODE_MAX_LAYERS = 32


def stack_decode(x, layers, H, KV, I, eps=1e-5, y=None, stages=None):
    """The linear path of len(layers) <= 32 layers at one token in one
    persistent launch (see bl_stack_decode).  x [H] or [1,H] fp32/bf16;
    layers: objects with packed_qkv, w_qkv, packed_o, w_o, packed_gu, w_gu,
    packed_down, w_down (and optional g_subln, g_ffn) device tensors.
    Returns y [1,H] fp32; stages, when given, is [L, (H+2KV)+H+I+H] fp32 and
    receives every stage's output."""
    dev = _dev(x)
    L = len(layers)
    if not 1 <= L <= STACK_DECODE_MAX_LAYERS:
        raise ValueError(f"1..{STACK_DECODE_MAX_LAYERS} layers per call")
    if x.numel() != H or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous tensor of {H} elements")
    arr = (Layer * L)()
    for i, lw in enumerate(layers):
        _need(lw.packed_qkv, ((H + 2 * KV) // 4, H), (torch.uint8,), "packed_qkv")
        _need(lw.packed_o, (H // 4, H), (torch.uint8,), "packed_o")
        _need(lw.packed_gu, (2 * I // 4, H), (torch.uint8,), "packed_gu")
        _need(lw.packed_down, (H // 4, I), (torch.uint8,), "packed_down")
        for t, n, name in ((lw.w_qkv, 3, "w_qkv"), (lw.w_o, 1, "w_o"), (lw.w_gu, 2, "w_gu"), (lw.w_down, 1, "w_down")):
            if t.dtype != torch.float32 or t.numel() < n:
                raise ValueError(f"{name} must be float32 with at least {n} elements")
        gs, gf = getattr(lw, "g_subln", None), getattr(lw, "g_ffn", None)
        if gs is not None:
            _need(gs, (H,), (torch.float32,), "g_subln")
        if gf is not None:
            _need(gf, (I,), (torch.float32,), "g_ffn")
        arr[i] = Layer(lw.packed_qkv.data_ptr(), lw.w_qkv.data_ptr(), lw.packed_o.data_ptr(), lw.w_o.data_ptr(),
                       lw.packed_gu.data_ptr(), lw.w_gu.data_ptr(), lw.packed_down.data_ptr(), lw.w_down.data_ptr(),
                       None if gs is None else gs.data_ptr(), None if gf is None else gf.data_ptr())
    if y is None:
        y = torch.empty((1, H), dtype=torch.float32, device=dev)
    _need(y, tuple(y.shape), (torch.float32,), "y")
    if y.numel() != H:
        raise ValueError(f"y must hold {H} elements")
    if stages is not None:
        _need(stages, (L, (H + 2 * KV) + H + I + H), (torch.float32,), "stages")
    ws = workspace(dev, raw.bl_stack_decode_workspace_bytes(L, H, KV, I))
    _check(raw.bl_stack_decode(_ptr(x), _dt(x), L, arr, H, KV, I, float(eps), _ptr(y), _ptr(stages), _ptr(ws),
                               ws.numel(), _stream(dev)))
    return y


def unpack_bf16(packed, seg_n=None, w_codes=None):
    """Offline unpack (see bl_unpack_bf16): packed uint8 [N/4,K] (segments
    stacked, widths seg_n) -> bf16 codes [N,K] (-1, 0, +1) in output-column
    order."""
    dev = _dev(packed)
    R, K = packed.shape
    _need(packed, (R, K), (torch.uint8,), "packed")
    n_seg, seg = _segs(seg_n, 4 * R)
    if w_codes is None:
        w_codes = torch.empty((4 * R, K), dtype=torch.bfloat16, device=dev)
    _need(w_codes, (4 * R, K), (torch.bfloat16,), "w_codes")
    _check(raw.bl_unpack_bf16(_ptr(packed), 4 * R, K, n_seg, seg, _ptr(w_codes), _stream(dev)))
    return w_codes


def gemm_unpacked(x, w_codes, w_mean, seg_n=None, y_dtype=torch.float32, a=None, y=None):
    """BitLinear on offline-unpacked bf16 codes [N,K] (see bl_gemm_unpacked):
    the same bits as gemm_w2a8 on the packed weight."""
    dev = _dev(x, w_codes, w_mean)
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    N = w_codes.shape[0]
    n_seg, seg = _segs(seg_n, N)
    _need(w_codes, (N, K), (torch.bfloat16,), "w_codes")
    if w_mean.dtype != torch.float32 or w_mean.numel() < n_seg:
        raise ValueError(f"w_mean must be float32 with at least {n_seg} elements")
    if a is not None and (a.dtype != torch.float32 or a.numel() < M):
        raise ValueError("a must be float32 with at least M elements")
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=dev)
    _need(y, (M, N), _OUT_DT, "y")
    ws = workspace(dev, raw.bl_gemm_unpacked_workspace_bytes(M, N, K))
    _check(raw.bl_gemm_unpacked(_ptr(x), _dt(x), x.stride(0), _ptr(a), M, K, _ptr(w_codes), N, n_seg, seg,
                                _ptr(w_mean), _ptr(y), _dt(y), _ptr(ws), ws.numel(), _stream(dev)))
    return y


def ffn_chain_noalloc(h, packed_gu, w_mean_gu, packed_down, w_mean_down, y, g_subln=None, g_ffn=None, eps=1e-5):
    """ffn_chain through the allocation-free entry point: the library's fixed
    per-device scratch, no workspace; y [M,H] fp32/bf16 is the caller's.
    Calls that overlap on one device race (they share the scratch)."""
    dev = _dev(h, packed_gu, packed_down, y)
    M, H = h.shape
    I = packed_gu.shape[0] * 2
    if h.stride(1) != 1 or h.stride(0) != H:
        raise ValueError("h must be contiguous")
    _check_weight(packed_gu, w_mean_gu, I // 2, H, 2, "packed_gu")
    _check_weight(packed_down, w_mean_down, H // 4, I, 1, "packed_down")
    for g, n, name in ((g_subln, H, "g_subln"), (g_ffn, I, "g_ffn")):
        if g is not None:
            _need(g, (n,), (torch.float32,), name)
    _need(y, (M, H), (torch.float32, torch.bfloat16), "y")
    _check(raw.bl_ffn_chain_noalloc(_ptr(h), _dt(h), M, H, I, _ptr(g_subln), _ptr(g_ffn), float(eps),
                                    _ptr(packed_gu), _ptr(w_mean_gu), _ptr(packed_down), _ptr(w_mean_down),
                                    _ptr(y), _dt(y), None, _stream(dev)))
    return y


def rope_table(max_pos: int, head_dim: int, base: float, device=None):
    """(cos, sin) [max_pos, head_dim/2] fp32 of the library's RoPE table, on
    `device` (host arrays when None)."""
    import numpy as np
    c = np.empty((max_pos, head_dim // 2), np.float32)
    sn = np.empty((max_pos, head_dim // 2), np.float32)
    _check(raw.bl_rope_table(int(max_pos), int(head_dim), float(base), c.ctypes.data_as(_P), sn.ctypes.data_as(_P)))
    if device is None:
        return c, sn
    return torch.from_numpy(c).to(device), torch.from_numpy(sn).to(device)


def attn_decode(q, k_new, v_new, pos, k_cache, v_cache, rope_cos, rope_sin, n_heads, n_kv_heads, out=None):
    """Decode attention of one token at position `pos` (see bl_attn_decode):
    q [n_heads*128], k_new / v_new [n_kv_heads*128] fp32; k_cache / v_cache
    [n_kv_heads, max_seq, 128] fp32 (updated at `pos`); returns out [n_heads*128]."""
    dev = _dev(q, k_new, v_new, k_cache, v_cache, rope_cos, rope_sin)
    D = 128
    kvh, max_seq, d = k_cache.shape
    if d != D or kvh != n_kv_heads or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [n_kv_heads, max_seq, 128]")
    for t, n, name in ((q, n_heads * D, "q"), (k_new, n_kv_heads * D, "k_new"), (v_new, n_kv_heads * D, "v_new")):
        if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 tensor of {n} elements")
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32")
    if rope_cos.shape[0] < max_seq or rope_cos.shape[-1] != D // 2 or rope_sin.shape != rope_cos.shape:
        raise ValueError("rope tables must be [>= max_seq, 64]")
    if out is None:
        out = torch.empty(n_heads * D, dtype=torch.float32, device=dev)
    ws = workspace(dev, raw.bl_attn_decode_workspace_bytes(int(n_heads), int(max_seq)))
    _check(raw.bl_attn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), int(pos), int(n_heads), int(n_kv_heads), D,
                              _ptr(k_cache), _ptr(v_cache), int(max_seq), _ptr(rope_cos), _ptr(rope_sin),
                              _ptr(out), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def attn_prefill(q, k, v, k_cache, v_cache, rope_cos, rope_sin, n_heads, n_kv_heads, out=None):
    """Causal attention of a prompt at positions 0 .. M-1 (see bl_attn_prefill):
    q [M, n_heads*128], k / v [M, n_kv_heads*128] fp32 with one row stride
    (views into a q|k|v output are fine); k_cache / v_cache [n_kv_heads,
    max_seq, 128] fp32 (positions < M written); returns out [M, n_heads*128]."""
    dev = _dev(q, k, v, k_cache, v_cache, rope_cos, rope_sin)
    D = 128
    M = q.shape[0]
    for t, w, name in ((q, n_heads * D, "q"), (k, n_kv_heads * D, "k"), (v, n_kv_heads * D, "v")):
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape != (M, w) or t.stride(1) != 1:
            raise ValueError(f"{name} must be fp32 [{M}, {w}] with contiguous rows")
    if not (q.stride(0) == k.stride(0) == v.stride(0)):
        raise ValueError("q, k and v must share one row stride")
    kvh, max_seq, d = k_cache.shape
    if d != D or kvh != n_kv_heads or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [n_kv_heads, max_seq, 128]")
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32")
    if rope_cos.shape[0] < M or rope_cos.shape[-1] != D // 2 or rope_sin.shape != rope_cos.shape:
        raise ValueError("rope tables must be [>= M, 64]")
    if out is None:
        out = torch.empty((M, n_heads * D), dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or out.shape != (M, n_heads * D) or out.stride(1) != 1:
        raise ValueError("out must be fp32 [M, n_heads*128] with contiguous rows")
    ws = workspace(dev, raw.bl_attn_prefill_workspace_bytes(M, int(n_heads), int(n_kv_heads)))
    _check(raw.bl_attn_prefill(_ptr(q), _ptr(k), _ptr(v), q.stride(0), M, int(n_heads), int(n_kv_heads), D,
                               _ptr(k_cache), _ptr(v_cache), int(max_seq), _ptr(rope_cos), _ptr(rope_sin),
                               _ptr(out), out.stride(0), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def ste_grad_input(dy, packed, w_mean, dx=None, dx_dtype=torch.float32):
    """dX = dY . (codes * w_mean) for dy [M,N] bf16 or fp32 (rounded to bf16
    on the device) and one packed weight segment [N/4,K] (see
    bl_ste_grad_input); returns dx [M,K] in dx_dtype (fp32, or bf16 rounded
    on the device), or in dx's dtype when dx is given."""
    dev = _dev(dy, packed, w_mean)
    M, N = dy.shape
    K = packed.shape[1]
    _need(dy, (M, N), (torch.bfloat16, torch.float32), "dy")
    _need(packed, (N // 4, K), (torch.uint8,), "packed")
    _need(w_mean, (1,), (torch.float32,), "w_mean")
    if dx is None:
        dx = torch.empty((M, K), dtype=dx_dtype, device=dev)
    _need(dx, (M, K), (torch.float32, torch.bfloat16), "dx")
    ws = workspace(dev, raw.bl_ste_grad_input_workspace_bytes(M, N, K, _dt(dy)))
    _check(raw.bl_ste_grad_input(_ptr(dy), _dt(dy), M, N, K, _ptr(packed), _ptr(w_mean), _ptr(dx), _dt(dx),
                                 _ptr(ws), ws.numel(), _stream(dev)))
    return dx


def ste_grad_weight(dy, q, a, dw=None):
    """dW = sum_m bf16(dY[m] / a[m]) (x) q[m] for dy [M,N] bf16 or fp32 and the
    forward's activation codes q [M,K] int8 and scales a [M] (see
    bl_ste_grad_weight); returns dw [N,K] fp32."""
    dev = _dev(dy, q, a)
    M, N = dy.shape
    K = q.shape[1]
    _need(dy, (M, N), (torch.bfloat16, torch.float32), "dy")
    _need(q, (M, K), (torch.int8,), "q")
    _need(a, (M,), (torch.float32,), "a")
    if dw is None:
        dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    _need(dw, (N, K), (torch.float32,), "dw")
    ws = workspace(dev, raw.bl_ste_grad_weight_workspace_bytes(M, N, K))
    _check(raw.bl_ste_grad_weight(_ptr(dy), _dt(dy), _ptr(q), _ptr(a), M, N, K, _ptr(dw), _ptr(ws), ws.numel(),
                                  _stream(dev)))
    return dw


# ---------------------------------------------------------------------------
# The 1-bit BitLinear.
# ---------------------------------------------------------------------------
def binarize_pack(W: torch.Tensor, packed: torch.Tensor = None, w_scale: torch.Tensor = None):
    """W fp32 [N,K] -> (packed uint8 [N/8,K], w_scale fp32 [1])."""
    dev = _dev(W)
    N, K = W.shape
    _need(W, (N, K), (torch.float32,), "W")
    if packed is None:
        packed = torch.empty((N // 8, K), dtype=torch.uint8, device=dev)
    if w_scale is None:
        w_scale = torch.empty(1, dtype=torch.float32, device=dev)
    _need(packed, (N // 8, K), (torch.uint8,), "packed")
    _need(w_scale, (1,), (torch.float32,), "w_scale")
    ws = workspace(dev, raw.bl_binarize_workspace_bytes(N, K))
    _check(raw.bl_binarize_pack(_ptr(W), N, K, _ptr(packed), _ptr(w_scale), _ptr(ws), ws.numel(), _stream(dev)))
    return packed, w_scale


def layernorm_quant(x: torch.Tensor, gamma=None, beta=None, eps: float = 1e-5, q=None, a=None):
    """x [M,K] fp32/bf16 (row stride may exceed K) -> (q int8 [M,K], a fp32 [M])."""
    dev = _dev(x)
    M, K = x.shape
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
    if a is None:
        a = torch.empty(M, dtype=torch.float32, device=dev)
    _need(q, (M, K), (torch.int8,), "q")
    _need(a, (M,), (torch.float32,), "a")
    for t, nm in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _need(t, (K,), (torch.float32,), nm)
    _check(raw.bl_layernorm_quant(_ptr(x), _dt(x), M, K, x.stride(0), _ptr(gamma), _ptr(beta), float(eps),
                                  _ptr(q), _ptr(a), _stream(dev)))
    return q, a


def gemm_w1a8(q: torch.Tensor, a: torch.Tensor, packed: torch.Tensor, w_scale: torch.Tensor, N: int = None,
              y: torch.Tensor = None):
    """Codes q int8 [M,K] with scales a [M] times packed signs [N/8,K] -> y fp32 [M,N]."""
    dev = _dev(q, a, packed, w_scale)
    M, K = q.shape
    N = 8 * packed.shape[0] if N is None else N
    _need(q, (M, K), (torch.int8,), "q")
    _need(a, (M,), (torch.float32,), "a")
    _need(packed, (N // 8, K), (torch.uint8,), "packed")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(y, (M, N), (torch.float32,), "y")
    _check(raw.bl_gemm_w1a8(_ptr(q), _ptr(a), M, K, _ptr(packed), N, _ptr(w_scale), _ptr(y), _stream(dev)))
    return y


def bitlinear_w1_batched(problems, eps: float = 1e-5):
    """Up to 8 forwards in two launches; each problem a dict with x [M,K]
    (fp32/bf16, contiguous), packed [N/8,K], w_scale [1], y fp32 [M,N] and
    optional gamma / beta [K]."""
    if not 1 <= len(problems) <= MAX_PROBLEMS:
        raise ValueError(f"1..{MAX_PROBLEMS} problems per call")
    arr = (W1Problem * len(problems))()
    dev = None
    for i, pr in enumerate(problems):
        x, packed, y = pr["x"], pr["packed"], pr["y"]
        dev = _dev(x, packed, y, pr["w_scale"])
        M, K = x.shape
        N = y.shape[1]
        _need(x, (M, K), (torch.float32, torch.bfloat16), "x")
        _need(packed, (N // 8, K), (torch.uint8,), "packed")
        _need(y, (M, N), (torch.float32,), "y")
        arr[i] = W1Problem(x.data_ptr(), _dt(x), M, K, _ptr(pr.get("gamma")), _ptr(pr.get("beta")),
                           packed.data_ptr(), N, pr["w_scale"].data_ptr(), y.data_ptr())
    ws = workspace(dev, raw.bl_bitlinear_w1_workspace_bytes(arr, len(problems)))
    _check(raw.bl_bitlinear_w1(arr, len(problems), float(eps), _ptr(ws), ws.numel(), _stream(dev)))
    return [pr["y"] for pr in problems]


def bitlinear_w1(x: torch.Tensor, packed: torch.Tensor, w_scale: torch.Tensor, gamma=None, beta=None,
                 eps: float = 1e-5, y: torch.Tensor = None):
    """One 1-bit BitLinear forward: x [M,K] -> y fp32 [M, 8 * packed rows]."""
    M = x.shape[0]
    N = 8 * packed.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    bitlinear_w1_batched([dict(x=x, packed=packed, w_scale=w_scale, y=y, gamma=gamma, beta=beta)], eps)
    return y
