"""C-ABI contract of libbitlinear, checked without a GPU.

Every call here fails argument validation on the host, before anything is
enqueued, so no kernel is ever launched (the pointers are fake).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")
LIB = os.environ.get("BL_LIBRARY") or os.path.join(ROOT, "bit_ternary_weight_amd", "libbitlinear.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bl_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libbitlinear.so is not built (run __graft_entry__.build())")
    from bit_ternary_weight_amd import binding
    return binding


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for name in ("bl_ternarize_pack", "bl_quant_act", "bl_gemv_w2a8", "bl_gemm_w2a8", "bl_ffn_chain"):
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    handle = ctypes.CDLL(LIB)
    missing = [f for f in declared_functions() if not hasattr(handle, f)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    raw = lib.raw
    assert raw.bl_abi_version() == 2
    names = [raw.bl_status_string(i).decode() for i in range(8)]
    assert names == ["BL_OK", "BL_ERR_NULL", "BL_ERR_SHAPE", "BL_ERR_ALIGN", "BL_ERR_DTYPE",
                     "BL_ERR_SEGMENTS", "BL_ERR_WORKSPACE", "BL_ERR_HIP"]
    assert raw.bl_status_string(99).decode() == "BL_ERR_UNKNOWN"
    assert raw.bl_device_errors(None, 0) == lib.BL_ERR_NULL


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p(0x10004)   # 4-byte aligned only
BIG = 1 << 40


def _gemv(raw, fn="bl_gemv_w2a8", x=FAKE, x_dt=1, ldx=0, a=None, M=1, K=256, packed=FAKE, N=256,
          n_seg=1, seg=None, w_mean=FAKE, y=FAKE, y_dt=0, ws=FAKE, ws_bytes=BIG):
    return getattr(raw, fn)(x, x_dt, ldx, a, M, K, packed, N, n_seg, seg, w_mean, y, y_dt, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["bl_gemv_w2a8", "bl_gemm_w2a8"])
def test_contract_validation(lib, fn):
    raw = lib.raw
    segs = lambda *v: (ctypes.c_int * len(v))(*v)
    cases = [
        (dict(x=None), lib.BL_ERR_NULL),
        (dict(packed=None), lib.BL_ERR_NULL),
        (dict(w_mean=None), lib.BL_ERR_NULL),
        (dict(y=None), lib.BL_ERR_NULL),
        (dict(ws=None, M=8), lib.BL_ERR_WORKSPACE),       # 8 bf16 rows need scratch
        (dict(x_dt=2, a=None), lib.BL_ERR_NULL),          # int8 codes need scales
        (dict(x_dt=3), lib.BL_ERR_DTYPE),
        (dict(y_dt=2), lib.BL_ERR_DTYPE),
        (dict(M=0), lib.BL_ERR_SHAPE),
        (dict(K=0), lib.BL_ERR_SHAPE),
        (dict(N=254), lib.BL_ERR_SHAPE),
        (dict(K=1 << 19), lib.BL_ERR_SHAPE),
        (dict(ldx=100), lib.BL_ERR_SHAPE),
        (dict(x=FAKE_MIS), lib.BL_ERR_ALIGN),
        (dict(packed=FAKE_MIS), lib.BL_ERR_ALIGN),
        (dict(y=FAKE_MIS), lib.BL_ERR_ALIGN),
        (dict(n_seg=0), lib.BL_ERR_SEGMENTS),
        (dict(n_seg=9, seg=segs(*([32] * 8 + [0]))), lib.BL_ERR_SEGMENTS),
        (dict(n_seg=2, seg=None), lib.BL_ERR_SEGMENTS),
        (dict(n_seg=2, seg=segs(128, 64)), lib.BL_ERR_SEGMENTS),   # sums to 192
        (dict(n_seg=2, seg=segs(126, 130)), lib.BL_ERR_SEGMENTS),  # not multiples of 4
        (dict(ws_bytes=1024, M=8), lib.BL_ERR_WORKSPACE),
    ]
    if fn == "bl_gemv_w2a8":
        cases.append((dict(M=65), lib.BL_ERR_SHAPE))
    for kw, want in cases:
        st = _gemv(raw, fn=fn, **kw)
        # a case that passed validation would have reached a launch: never allowed here
        assert st not in (lib.BL_OK, lib.BL_ERR_HIP), (kw, st)
        assert st == want, (kw, st, raw.bl_last_error())
        assert raw.bl_last_error().decode() != ""


def test_workspace_queries(lib):
    raw = lib.raw
    assert raw.bl_gemv_workspace_bytes(1, 2560, 2560) >= 2560 + 4
    assert raw.bl_gemm_workspace_bytes(2048, 13824, 2560) >= 2048 * 2560 + 4 * 2048
    assert raw.bl_ffn_chain_workspace_bytes(4, 2560, 6912) >= 4 * (2560 + 6912 + 4 * 6912)
    assert raw.bl_gemv_workspace_bytes(0, 4, 4) == 0
    assert raw.bl_ternarize_workspace_bytes(2560, 2560) >= 8
    assert raw.bl_ternarize_workspace_bytes(2560, 2560) % 256 == 0


def test_ternarize_and_quant_validation(lib):
    raw = lib.raw
    B = lib
    assert raw.bl_ternarize_pack(None, 8, 8, FAKE, FAKE, FAKE, BIG, None) == B.BL_ERR_NULL
    assert raw.bl_ternarize_pack(FAKE, 6, 8, FAKE, FAKE, FAKE, BIG, None) == B.BL_ERR_SHAPE
    assert raw.bl_ternarize_pack(FAKE, 8, 0, FAKE, FAKE, FAKE, BIG, None) == B.BL_ERR_SHAPE
    assert raw.bl_ternarize_pack(FAKE_MIS, 8, 8, FAKE, FAKE, FAKE, BIG, None) == B.BL_ERR_ALIGN
    assert raw.bl_ternarize_pack(FAKE, 2560, 2560, FAKE, FAKE, FAKE, 8, None) == B.BL_ERR_WORKSPACE
    assert raw.bl_quant_act(None, 0, 4, 8, 0, FAKE, FAKE, None) == B.BL_ERR_NULL
    assert raw.bl_quant_act(FAKE, 2, 4, 8, 0, FAKE, FAKE, None) == B.BL_ERR_DTYPE
    assert raw.bl_quant_act(FAKE, 0, 0, 8, 0, FAKE, FAKE, None) == B.BL_ERR_SHAPE
    assert raw.bl_quant_act(FAKE, 0, 4, 8, 4, FAKE, FAKE, None) == B.BL_ERR_SHAPE
    assert raw.bl_quant_act(FAKE_MIS, 0, 4, 8, 0, FAKE, FAKE, None) == B.BL_ERR_ALIGN
    assert raw.bl_rmsnorm_quant(None, 0, 4, 8, None, 1e-5, FAKE, FAKE, None) == B.BL_ERR_NULL
    assert raw.bl_rmsnorm_quant(FAKE, 2, 4, 8, None, 1e-5, FAKE, FAKE, None) == B.BL_ERR_DTYPE
    assert raw.bl_rmsnorm_quant(FAKE, 0, 0, 8, None, 1e-5, FAKE, FAKE, None) == B.BL_ERR_SHAPE
    assert raw.bl_rmsnorm_quant(FAKE, 0, 4, 8, None, -1.0, FAKE, FAKE, None) == B.BL_ERR_SHAPE
    assert raw.bl_rmsnorm_quant(FAKE_MIS, 0, 4, 8, None, 1e-5, FAKE, FAKE, None) == B.BL_ERR_ALIGN
    sg = raw.bl_subln_gemv_w2a8
    need = raw.bl_subln_gemv_workspace_bytes(4, 64)
    assert need >= 4 * 64 + 16 and raw.bl_subln_gemv_workspace_bytes(0, 64) == 0
    ok = dict(h=FAKE, dt=0, M=4, K=64, g=None, eps=1e-5, P=FAKE, N=16, w=FAKE, y=FAKE, ydt=0, q=None, a=None,
              ws=FAKE, wsb=need)
    call = lambda **kw: sg(*{**ok, **kw}.values(), None)
    assert call(h=None) == B.BL_ERR_NULL
    assert call(dt=2) == B.BL_ERR_DTYPE                       # int8 input has no norm to apply
    assert call(N=18) == B.BL_ERR_SHAPE
    assert call(eps=-1.0) == B.BL_ERR_SHAPE
    assert call(q=FAKE_MIS) == B.BL_ERR_ALIGN
    assert call(wsb=need - 1) == B.BL_ERR_WORKSPACE


def test_ffn_chain_validation(lib):
    raw = lib.raw
    B = lib

    def call(h=FAKE, h_dt=0, M=1, H=256, I=512, eps=1e-5, gu=FAKE, wgu=FAKE, dn=FAKE, wd=FAKE, y=FAKE,
             y_dt=0, ws=FAKE, ws_bytes=BIG):
        return raw.bl_ffn_chain(h, h_dt, M, H, I, None, None, eps, gu, wgu, dn, wd, y, y_dt, ws, ws_bytes,
                                None, None)

    assert call(h=None) == B.BL_ERR_NULL
    assert call(gu=None) == B.BL_ERR_NULL
    assert call(h_dt=2) == B.BL_ERR_DTYPE
    assert call(y_dt=3) == B.BL_ERR_DTYPE
    assert call(H=254) == B.BL_ERR_SHAPE
    assert call(I=0) == B.BL_ERR_SHAPE
    assert call(M=0) == B.BL_ERR_SHAPE
    assert call(eps=-1.0) == B.BL_ERR_SHAPE
    assert call(y=FAKE_MIS) == B.BL_ERR_ALIGN
    assert call(ws_bytes=16) == B.BL_ERR_WORKSPACE
    assert call(ws=None) == B.BL_ERR_WORKSPACE


def test_batched_validation(lib):
    raw = lib.raw
    P = lib.GemvProblem

    def prob(**kw):
        d = dict(x=0x10000, x_dtype=1, ldx=0, a=None, M=1, K=256, packed=0x20000, N=256, n_seg=1,
                 seg_n=None, w_mean=0x30000, y=0x40000, y_dtype=0)
        d.update(kw)
        return P(**d)

    arr = (P * 2)(prob(), prob(M=0))
    assert raw.bl_gemv_w2a8_batched(2, arr, FAKE, BIG, None) == lib.BL_ERR_SHAPE
    arr = (P * 2)(prob(), prob(x=None))
    assert raw.bl_gemv_w2a8_batched(2, arr, FAKE, BIG, None) == lib.BL_ERR_NULL
    arr = (P * 1)(prob(M=65))
    assert raw.bl_gemv_w2a8_batched(1, arr, FAKE, BIG, None) == lib.BL_ERR_SHAPE
    assert raw.bl_gemv_w2a8_batched(0, arr, FAKE, BIG, None) == lib.BL_ERR_SHAPE
    assert raw.bl_gemv_w2a8_batched(9, arr, FAKE, BIG, None) == lib.BL_ERR_SHAPE
    assert raw.bl_gemv_w2a8_batched(1, None, FAKE, BIG, None) == lib.BL_ERR_NULL
    arr = (P * 2)(prob(M=8), prob(M=8, K=512))      # M > 4: codes go to the workspace
    need = raw.bl_gemv_batched_workspace_bytes(2, arr)
    assert need >= 8 * 256 + 8 * 512
    assert raw.bl_gemv_w2a8_batched(2, arr, FAKE, need - 1, None) == lib.BL_ERR_WORKSPACE
    assert raw.bl_gemv_w2a8_batched(2, arr, None, 0, None) == lib.BL_ERR_WORKSPACE


def test_last_error_is_per_thread(lib):
    import threading
    raw = lib.raw
    assert _gemv(raw, M=0) == lib.BL_ERR_SHAPE
    msg_main = raw.bl_last_error().decode()
    seen = {}

    def worker():
        seen["before"] = raw.bl_last_error().decode()
        _gemv(raw, x=None)
        seen["after"] = raw.bl_last_error().decode()

    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert seen["before"] == ""
    assert "NULL" in seen["after"]
    assert raw.bl_last_error().decode() == msg_main


def _attn(raw, q=FAKE, kn=FAKE, vn=FAKE, pos=5, H=20, KVH=5, D=128, kc=FAKE, vc=FAKE, S=2048,
          rc=FAKE, rs=FAKE, out=FAKE, ws=FAKE, ws_bytes=BIG):
    return raw.bl_attn_decode(q, kn, vn, pos, H, KVH, D, kc, vc, S, rc, rs, out, ws, ws_bytes, None)


def test_attn_decode_validation(lib):
    raw = lib.raw
    assert _attn(raw, q=None) == lib.BL_ERR_NULL
    assert _attn(raw, out=None) == lib.BL_ERR_NULL
    assert _attn(raw, D=64) == lib.BL_ERR_SHAPE
    assert _attn(raw, H=20, KVH=3) == lib.BL_ERR_SHAPE          # not a multiple
    assert _attn(raw, H=20, KVH=2) == lib.BL_ERR_SHAPE          # 10 query heads per key/value head
    assert _attn(raw, pos=2048) == lib.BL_ERR_SHAPE
    assert _attn(raw, pos=-1) == lib.BL_ERR_SHAPE
    assert _attn(raw, kc=FAKE_MIS) == lib.BL_ERR_ALIGN
    assert _attn(raw, S=32769, pos=5) == lib.BL_ERR_SHAPE      # beyond the longest cache
    need = raw.bl_attn_decode_workspace_bytes(20, 2048)
    assert need >= 20 * 32 * 132 * 4                            # partial results per head and chunk
    assert _attn(raw, ws_bytes=need - 1) == lib.BL_ERR_WORKSPACE
    assert _attn(raw, ws=None, ws_bytes=0) == lib.BL_ERR_WORKSPACE
    assert raw.bl_attn_decode_workspace_bytes(0, 2048) == 0


def test_rope_table_values(lib):
    import numpy as np
    import math
    # closed form: head_dim 8, base 100 -> pair i turns by 100^(-2i/8) = 1,
    # 10^-0.5, 0.1, 10^-1.5 radians per position
    c, s = lib.rope_table(4, 8, 100.0)
    assert c.shape == (4, 4) and (c[0] == 1).all() and (s[0] == 0).all()
    for p in range(1, 4):
        for i, t in enumerate([1.0, 10 ** -0.5, 0.1, 10 ** -1.5]):
            for got, want in ((c[p, i], math.cos(p * t)), (s[p, i], math.sin(p * t))):
                assert abs(float(got) - want) <= float(np.spacing(np.float32(abs(want)))), (p, i)
    raw = lib.raw
    assert raw.bl_rope_table(4, 7, 10000.0, FAKE, FAKE) == lib.BL_ERR_SHAPE
    assert raw.bl_rope_table(4, 8, 0.0, FAKE, FAKE) == lib.BL_ERR_SHAPE
    assert raw.bl_rope_table(4, 8, 10000.0, None, FAKE) == lib.BL_ERR_NULL


def test_attn_prefill_validation(lib):
    raw = lib.raw
    pf = raw.bl_attn_prefill
    need = raw.bl_attn_prefill_workspace_bytes(100, 20, 5)
    assert need >= 128 * 128 * 2 * 30 and raw.bl_attn_prefill_workspace_bytes(0, 20, 5) == 0
    ok = dict(q=FAKE, k=FAKE, v=FAKE, ldx=3840, M=100, H=20, KVH=5, D=128, kc=FAKE, vc=FAKE, S=4096, rc=FAKE,
              rs=FAKE, out=FAKE, ldo=2560, ws=FAKE, wsb=need)
    call = lambda **kw: pf(*{**ok, **kw}.values(), None)
    assert call(q=None) == lib.BL_ERR_NULL
    assert call(D=64) == lib.BL_ERR_SHAPE
    assert call(KVH=3) == lib.BL_ERR_SHAPE
    assert call(M=4097) == lib.BL_ERR_SHAPE
    assert call(M=0) == lib.BL_ERR_SHAPE
    assert call(ldx=2000) == lib.BL_ERR_SHAPE
    assert call(ldo=2562) == lib.BL_ERR_SHAPE
    assert call(out=FAKE_MIS) == lib.BL_ERR_ALIGN
    assert call(wsb=need - 1) == lib.BL_ERR_WORKSPACE


def test_ste_validation(lib):
    raw = lib.raw
    gi, gw = raw.bl_ste_grad_input, raw.bl_ste_grad_weight
    BF, F = lib.BL_BF16, lib.BL_F32
    ni = raw.bl_ste_grad_input_workspace_bytes(128, 256, 384, BF)
    nw = raw.bl_ste_grad_weight_workspace_bytes(128, 256, 384)
    assert ni >= 256 * 384 * 2 and nw >= (256 * 128 + 384 * 128) * 2
    # whole tiles of a bf16 gradient are used in place; fp32 or ragged ones get a padded bf16 copy
    assert raw.bl_ste_grad_input_workspace_bytes(128, 256, 384, F) >= ni + 128 * 256 * 2
    assert raw.bl_ste_grad_input_workspace_bytes(100, 256, 384, BF) >= ni + 128 * 256 * 2
    assert raw.bl_ste_grad_input_workspace_bytes(128, 256, 384, 2) == 0
    ni100 = raw.bl_ste_grad_input_workspace_bytes(100, 200, 300, F)
    assert gi(None, BF, 128, 256, 384, FAKE, FAKE, FAKE, F, FAKE, ni, None) == lib.BL_ERR_NULL
    assert gi(FAKE, BF, 0, 256, 384, FAKE, FAKE, FAKE, F, FAKE, ni, None) == lib.BL_ERR_SHAPE
    assert gi(FAKE, F, 100, 202, 300, FAKE, FAKE, FAKE, F, FAKE, ni100, None) == lib.BL_ERR_SHAPE   # N % 4
    assert gi(FAKE, 2, 128, 256, 384, FAKE, FAKE, FAKE, F, FAKE, ni, None) == lib.BL_ERR_DTYPE
    assert gi(FAKE_MIS, BF, 128, 256, 384, FAKE, FAKE, FAKE, F, FAKE, ni, None) == lib.BL_ERR_ALIGN
    assert gi(FAKE, BF, 128, 256, 384, FAKE, FAKE, FAKE, F, FAKE, ni - 1, None) == lib.BL_ERR_WORKSPACE
    assert gi(FAKE, BF, 1 << 16, 1 << 16, 128, FAKE, FAKE, FAKE, F, FAKE, BIG, None) == lib.BL_ERR_SHAPE
    assert gi(FAKE, BF, 128, 256, 384, FAKE, FAKE, FAKE, 2, FAKE, ni, None) == lib.BL_ERR_DTYPE   # dx int8
    assert gi(FAKE, BF, 128, 256, 384, FAKE, FAKE, FAKE_MIS, BF, FAKE, ni, None) == lib.BL_ERR_ALIGN
    assert gw(FAKE, BF, None, FAKE, 128, 256, 384, FAKE, FAKE, nw, None) == lib.BL_ERR_NULL
    assert gw(FAKE, BF, FAKE, FAKE, 128, 256, -1, FAKE, FAKE, nw, None) == lib.BL_ERR_SHAPE
    assert gw(FAKE, BF, FAKE, FAKE, 128, 256, 384, FAKE_MIS, FAKE, nw, None) == lib.BL_ERR_ALIGN
    assert gw(FAKE, BF, FAKE, FAKE, 128, 256, 384, FAKE, FAKE, nw - 1, None) == lib.BL_ERR_WORKSPACE
    assert gw(FAKE, 3, FAKE, FAKE, 128, 256, 384, FAKE, FAKE, nw, None) == lib.BL_ERR_DTYPE


def test_unpacked_validation(lib):
    raw = lib.raw
    assert raw.bl_unpack_bf16(None, 8, 8, 1, None, FAKE, None) == lib.BL_ERR_NULL
    assert raw.bl_unpack_bf16(FAKE, 6, 8, 1, None, FAKE, None) == lib.BL_ERR_SHAPE
    assert raw.bl_unpack_bf16(FAKE, 8, 8, 2, None, FAKE, None) == lib.BL_ERR_SEGMENTS
    assert raw.bl_unpack_bf16(FAKE, 8, 8, 1, None, ctypes.c_void_p(0x10001), None) == lib.BL_ERR_ALIGN
    need = raw.bl_gemm_unpacked_workspace_bytes(130, 256, 2560)
    assert need >= 130 * 2560 + 256 * 2560 * 2
    g = raw.bl_gemm_unpacked
    ok = dict(x=FAKE, xdt=1, ldx=0, a=None, M=130, K=2560, w=FAKE, N=256, ns=1, seg=None, wm=FAKE, y=FAKE, ydt=0,
              ws=FAKE, wsb=need)
    call = lambda **kw: g(*{**ok, **kw}.values(), None)
    assert call(x=None) == lib.BL_ERR_NULL
    assert call(xdt=3) == lib.BL_ERR_DTYPE
    assert call(xdt=2) == lib.BL_ERR_NULL          # int8 codes need their scales
    assert call(N=254) == lib.BL_ERR_SHAPE
    assert call(K=100, wsb=1 << 30) == lib.BL_ERR_SHAPE   # neither kernel takes K = 100 at M = 130
    assert call(y=FAKE_MIS) == lib.BL_ERR_ALIGN
    assert call(wsb=need - 1) == lib.BL_ERR_WORKSPACE


def test_stack_decode_validation(lib):
    raw = lib.raw
    L = lib.Layer
    ok = L(*[FAKE.value] * 8, None, None)
    arr = (L * 2)(ok, ok)
    H, KV, I = 2560, 640, 6912
    need = raw.bl_stack_decode_workspace_bytes(2, H, KV, I)
    assert need >= 2 * ((H + 2 * KV) + H + I + H) * 4
    call = lambda **kw: raw.bl_stack_decode(*{**dict(x=FAKE, xdt=1, L=2, layers=arr, H=H, KV=KV, I=I, eps=1e-5, y=FAKE,
                                                      st=None, ws=FAKE, wsb=need), **kw}.values(), None)
    assert call(x=None) == lib.BL_ERR_NULL
    assert call(xdt=2) == lib.BL_ERR_DTYPE
    assert call(L=0) == lib.BL_ERR_SHAPE
    assert call(L=33) == lib.BL_ERR_SHAPE
    assert call(eps=-1.0) == lib.BL_ERR_SHAPE


def test_w1_validation(lib):
    raw = lib.raw
    assert raw.bl_binarize_workspace_bytes(2560, 2560) == raw.bl_ternarize_workspace_bytes(2560, 2560)
    need = raw.bl_binarize_workspace_bytes(64, 32)
    bp = lambda **kw: raw.bl_binarize_pack(*{**dict(W=FAKE, N=64, K=32, P=FAKE, s=FAKE, ws=FAKE, wsb=need),
                                            **kw}.values(), None)
    assert bp(W=None) == lib.BL_ERR_NULL
    assert bp(N=60) == lib.BL_ERR_SHAPE
    assert bp(K=30) == lib.BL_ERR_SHAPE
    assert bp(P=FAKE_MIS) == lib.BL_ERR_ALIGN
    assert bp(wsb=need - 1) == lib.BL_ERR_WORKSPACE
    ln = lambda **kw: raw.bl_layernorm_quant(*{**dict(x=FAKE, xdt=0, M=4, K=2560, ldx=0, g=None, b=None, eps=1e-5,
                                                      q=FAKE, a=FAKE), **kw}.values(), None)
    assert ln(x=None) == lib.BL_ERR_NULL
    assert ln(xdt=2) == lib.BL_ERR_DTYPE
    assert ln(K=2562) == lib.BL_ERR_SHAPE
    assert ln(K=16388) == lib.BL_ERR_SHAPE         # above the norm's 16384
    assert ln(ldx=2561) == lib.BL_ERR_SHAPE
    assert ln(eps=-1.0) == lib.BL_ERR_SHAPE
    assert ln(g=FAKE_MIS) == lib.BL_ERR_ALIGN
    gm = lambda **kw: raw.bl_gemm_w1a8(*{**dict(q=FAKE, a=FAKE, M=3, K=2560, P=FAKE, N=2560, s=FAKE, y=FAKE),
                                         **kw}.values(), None)
    assert gm(q=None) == lib.BL_ERR_NULL
    assert gm(P=None) == lib.BL_ERR_NULL
    assert gm(K=2568) == lib.BL_ERR_SHAPE          # K a multiple of 16
    assert gm(N=2564) == lib.BL_ERR_SHAPE          # N a multiple of 8
    assert gm(M=0) == lib.BL_ERR_SHAPE
    assert gm(P=FAKE_MIS) == lib.BL_ERR_ALIGN
    W1 = lib.W1Problem
    ok = W1(FAKE.value, 1, 1, 2560, None, None, FAKE.value, 3840, FAKE.value, FAKE.value)
    arr = (W1 * 2)(ok, ok)
    need = raw.bl_bitlinear_w1_workspace_bytes(arr, 2)
    assert need >= 2 * (2560 + 4)
    assert raw.bl_bitlinear_w1_workspace_bytes(arr, 9) == 0
    bw = lambda arr=arr, n=2, eps=1e-5, ws=FAKE, wsb=need: raw.bl_bitlinear_w1(arr, n, eps, ws, wsb, None)
    assert bw(n=0) == lib.BL_ERR_SHAPE
    assert bw(n=9) == lib.BL_ERR_SHAPE
    assert bw(wsb=need - 1) == lib.BL_ERR_WORKSPACE
    bad = (W1 * 2)(ok, W1(FAKE.value, 3, 1, 2560, None, None, FAKE.value, 3840, FAKE.value, FAKE.value))
    assert bw(arr=bad) == lib.BL_ERR_DTYPE
    bad = (W1 * 2)(ok, W1(FAKE.value, 1, 1, 2560, None, None, FAKE.value, 3844, FAKE.value, FAKE.value))
    assert bw(arr=bad) == lib.BL_ERR_SHAPE


def test_loaded_library_is_the_requested_build(lib):
    """BL_LIBRARY, when set, names the build the binding loads (the sanitizer
    run relies on it); otherwise the in-tree library."""
    assert os.path.abspath(lib.LIB_PATH) == os.path.abspath(LIB)
