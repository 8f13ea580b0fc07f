"""GPU parity: bl_gemv_w2a8 (decode) and bl_gemm_w2a8 (prefill) against the oracle.

Weights are always packed by the oracle (its bytes go to the device), so the
contraction is checked on its own.  int32 accumulators (y dtype int32) are
compared bit-exactly; fp32 / bf16 outputs by the per-row tolerance, and the
fp32 path is additionally expected to be bit-identical (it replays the same
fp32 operations).  Every output buffer is pre-filled with a pattern no
result can hold and followed by a canary tail (gpu_helpers.Guarded): no
element may be left unwritten and nothing written past the end.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import (BF16_TOL, F32_TOL, assert_exact, assert_rows_close, bf16_dev, f32_of_bf16, guarded, host,
                         max_ulp_diff, requires_gpu, to_dev)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


def _weights(seed, seg_n, K):
    """Oracle-packed segmented weight: (packed [N/4,K], w_means [S], codes [N,K])."""
    packs, wms, codes = [], [], []
    for i, n in enumerate(seg_n):
        p, wm, c = oracle.ternarize_pack(synth.master_weight(seed + 17 * i, n, K))
        packs.append(p)
        wms.append(wm)
        codes.append(c)
    return np.concatenate(packs), np.array(wms, np.float32), np.concatenate(codes)


def _run(fn, x_dev, packed, wms, seg_n, y_dtype, a=None):
    f = getattr(_bl(), fn)
    M, N = x_dev.shape[0], packed.shape[0] * 4
    out = guarded((M, N), y_dtype)
    f(x_dev, packed if isinstance(packed, torch.Tensor) else to_dev(packed), wms if isinstance(wms, torch.Tensor)
      else to_dev(wms), seg_n=list(seg_n) if len(seg_n) > 1 else None, y_dtype=y_dtype, a=a, y=out.t)
    out.check(f"{fn} y {y_dtype}")
    return out.t


def _check(fn, M, K, seg_n, x_kind="bf16", seed=0, check_all_dtypes=True):
    packed, wms, codes = _weights(1000 + seed, seg_n, K)
    if x_kind == "bf16":
        bits = synth.act_outliers_bf16(seed, M, K)
        x_host = f32_of_bf16(bits)
        x_dev = bf16_dev(bits)
    else:
        x_host = synth.act_normal_f32(seed, M, K)
        x_dev = to_dev(x_host)
    q, a, A, y = oracle.bitlinear(x_host, codes, seg_n, wms)
    a_dev = None
    if x_kind == "i8":
        x_dev = to_dev(q)
        a_dev = to_dev(a)
    # raw accumulators
    Ag = _run(fn, x_dev, packed, wms, seg_n, torch.int32, a=a_dev)
    assert_exact(host(Ag), A, f"{fn} int32 accumulators")
    if not check_all_dtypes:
        return
    yg = host(_run(fn, x_dev, packed, wms, seg_n, torch.float32, a=a_dev))
    assert_rows_close(yg, y, F32_TOL, "fp32 y")
    assert max_ulp_diff(yg, y) == 0, "fp32 output differs from the oracle's bits"
    yb = host(_run(fn, x_dev, packed, wms, seg_n, torch.bfloat16, a=a_dev))
    assert_rows_close(f32_of_bf16(yb), y, BF16_TOL, "bf16 y")
    assert_exact(yb, oracle.to_bf16(y), "bf16 bits")


# ----------------------------------------------------------------------------- decode path
GEMV_SHAPES = [  # (M, K, seg_n)
    (1, 64, (4,)), (1, 256, (256,)), (2, 256, (64,)), (3, 128, (12,)), (4, 256, (256,)),
    (5, 320, (36,)), (16, 512, (128,)), (17, 256, (68,)), (33, 192, (64,)), (64, 256, (256,)),
    (1, 2560, (2560, 640, 640)), (4, 2560, (64, 16, 16)), (64, 1024, (128, 32, 32)),
    (1, 6912, (2560,)), (1, 6912, (64,)), (2, 4096, (16,)), (64, 6912, (32,)),
    # batched-decode streaming kernel: one 256-byte block (most waves idle), a
    # 10-row tensor, 49..64 rows over fused q|k|v; K not a multiple of 256
    # (the register kernel)
    (8, 256, (16,)), (24, 768, (40,)), (50, 2560, (2560, 640, 640)), (8, 64, (16,)), (20, 128, (8,)),
    (16, 272, (32,)),
]


@pytest.mark.parametrize("M,K,seg_n", GEMV_SHAPES)
def test_gemv_parity(M, K, seg_n):
    _check("gemv_w2a8", M, K, seg_n, seed=M + K)


@pytest.mark.parametrize("M,K,seg_n", [(1, 17, (8,)), (3, 100, (16,)), (2, 4, (4,)), (4, 33, (12, 4))])
def test_gemv_ragged_k(M, K, seg_n):
    _check("gemv_w2a8", M, K, seg_n, seed=3)


@pytest.mark.parametrize("x_kind", ["f32", "i8"])
def test_gemv_input_kinds(x_kind):
    _check("gemv_w2a8", 4, 2560, (640, 160), x_kind=x_kind, seed=9)


@pytest.mark.parametrize("M,x_kind", [(16, "i8"), (50, "i8"), (33, "f32"), (64, "f32")])
def test_gemv_batched_input_kinds(M, x_kind):
    """More than 4 rows: int8 codes given row-major take the register kernel,
    fp32 rows are quantized into the tiled layout of the streaming kernel."""
    _check("gemv_w2a8", M, 2560, (640, 160), x_kind=x_kind, seed=10 + M)


# 5 to 17 token rows through the row quantizer and the batched streaming
# kernel: one 256-byte block, fused q|k|v, K = 6912, 7168 and 7424, fp32
# rows, one token tile and a second one; 36 output rows leave a partial row
# group of 9 packed rows.
@pytest.mark.parametrize("M,K,seg_n,x_kind", [
    (5, 256, (16,), "bf16"), (8, 2560, (2560, 640, 640), "bf16"), (13, 6912, (2560,), "bf16"),
    (16, 7168, (68,), "bf16"), (16, 6912, (36,), "bf16"), (16, 7424, (68,), "bf16"),
    (16, 2560, (640, 160), "f32"), (17, 2560, (640, 160), "bf16")])
def test_gemv_batched_rows(M, K, seg_n, x_kind):
    _check("gemv_w2a8", M, K, seg_n, x_kind=x_kind, seed=20 + M + K % 7)


def test_gemv_batched_strided_rows():
    """16 bf16 rows read with a row stride larger than K (a column slice of a
    wider activation tensor): every output bit-identical to the oracle."""
    M, K, seg_n = 16, 2560, (640, 160)
    packed, wms, codes = _weights(77, seg_n, K)
    bits = synth.act_heavy_tail_bf16(77, M, K + 64)
    wide = bf16_dev(bits)
    x = wide[:, 32:32 + K]
    assert x.stride(0) == K + 64
    _, _, A, y = oracle.bitlinear(f32_of_bf16(bits[:, 32:32 + K]), codes, seg_n, wms)
    Ag = _run("gemv_w2a8", x, packed, wms, seg_n, torch.int32)
    assert_exact(host(Ag), A, "int32 accumulators")
    yg = host(_run("gemv_w2a8", x, packed, wms, seg_n, torch.float32))
    assert max_ulp_diff(yg, y) == 0


def test_batched_mixed_rows():
    """Problems of 3, 9 and 16 bf16 rows (K 6912, 2560 with three segments,
    256) in one call: the 16-row problem keeps the batch off the one-row and
    LDS kernels, so every problem goes through the row quantizer and the
    batched streaming kernel, the 3-row one included."""
    specs = [(3, 6912, (2560,)), (9, 2560, (640, 160, 160)), (16, 256, (64,))]
    probs, refs = [], []
    for i, (M, K, seg_n) in enumerate(specs):
        packed, wms, codes = _weights(400 + i, seg_n, K)
        bits = synth.act_outliers_bf16(90 + i, M, K)
        _, _, _, y = oracle.bitlinear(f32_of_bf16(bits), codes, seg_n, wms)
        probs.append(dict(x=bf16_dev(bits), packed=to_dev(packed), w_mean=to_dev(wms),
                          seg_n=list(seg_n) if len(seg_n) > 1 else None))
        refs.append(y)
    outs = _bl().gemv_w2a8_batched(probs)
    for y, yr in zip(outs, refs):
        assert max_ulp_diff(host(y), yr) == 0


# The one-row decode kernel stages the row's codes in a 12288-byte LDS buffer:
# K at that limit takes it, one k-range more takes the register kernel; fp32
# rows carry half as many elements per load.
@pytest.mark.parametrize("K,x_kind", [(12288, "bf16"), (12544, "bf16"), (12288, "f32"), (8192, "f32")])
def test_gemv_one_row_kernel_k_limits(K, x_kind):
    _check("gemv_w2a8", 1, K, (256,), x_kind=x_kind, seed=K % 97, check_all_dtypes=False)


# Large single problems: each stream wave of the one-row kernel then holds the
# most weight units (12 and 16 in flight, the two largest instantiations).
# Codes are drawn uniformly from {-1, 0, 1} and packed by the oracle.
@pytest.mark.parametrize("N,K", [(13312, 6144), (13312, 8192)])
def test_gemv_one_row_kernel_many_units(N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    packed = oracle.pack(codes)
    wms = np.array([0.0173], np.float32)
    bits = synth.act_outliers_bf16(5, 1, K)
    x_host = f32_of_bf16(bits)
    _, _, A, y = oracle.bitlinear(x_host, codes, (N,), wms)
    Ag = _run("gemv_w2a8", bf16_dev(bits), packed, wms, (N,), torch.int32)
    assert_exact(host(Ag), A, "int32 accumulators")
    yg = host(_run("gemv_w2a8", bf16_dev(bits), packed, wms, (N,), torch.float32))
    assert_rows_close(yg, y, F32_TOL, "fp32 y")


def test_gemv_long_k_repeated():
    """Long K over a single tile (one workgroup streams all of it); repeated
    calls on the same workspace stay exact."""
    for seed in (1, 2):
        _check("gemv_w2a8", 1, 6912, (64,), seed=seed, check_all_dtypes=False)
        _check("gemv_w2a8", 2, 6912, (128,), seed=seed + 5, check_all_dtypes=False)


# ----------------------------------------------------------------------------- prefill path
GEMM_SHAPES = [
    (1, 64, (4,)), (7, 256, (256,)), (64, 256, (128,)), (65, 256, (128,)), (128, 512, (64,)),
    (129, 320, (36,)), (200, 1024, (256, 64, 64)), (300, 2560, (160,)), (256, 6912, (128,)),
    # segments of 3 and 2 packed rows: the large-tile kernel with per-column stores
    (130, 512, (12, 8)),
]


@pytest.mark.parametrize("M,K,seg_n", GEMM_SHAPES)
def test_gemm_parity(M, K, seg_n):
    _check("gemm_w2a8", M, K, seg_n, seed=2 * M + K)


@pytest.mark.parametrize("M,K,seg_n", [(130, 17, (8,)), (70, 100, (16,))])
def test_gemm_ragged_k(M, K, seg_n):
    _check("gemm_w2a8", M, K, seg_n, seed=4)


@pytest.mark.parametrize("x_kind", ["f32", "i8"])
def test_gemm_input_kinds(x_kind):
    _check("gemm_w2a8", 150, 2560, (256, 64), x_kind=x_kind, seed=10)


# ----------------------------------------------------------------------------- properties
@pytest.mark.parametrize("fn,M", [("gemv_w2a8", 4), ("gemm_w2a8", 130)])
def test_identity_weight_pins_orientation(fn, M):
    K = 256
    packed, wm, codes = oracle.ternarize_pack(np.eye(K, dtype=np.float32))
    x = synth.act_normal_f32(6, M, K)
    q, a = oracle.quant_act(x)
    A = host(getattr(_bl(), fn)(to_dev(x), to_dev(packed), to_dev(np.array([wm])), y_dtype=torch.int32))
    assert_exact(A, q.astype(np.int32), "identity weight accumulators")


@pytest.mark.parametrize("fn,M", [("gemv_w2a8", 64), ("gemm_w2a8", 300)])
def test_row_permutation_and_determinism(fn, M):
    K, seg_n = 2560, (256,)
    packed, wms, _ = _weights(5, seg_n, K)
    bits = synth.act_heavy_tail_bf16(8, M, K)
    x = bf16_dev(bits)
    y1 = _run(fn, x, packed, wms, seg_n, torch.float32)
    y2 = _run(fn, x, packed, wms, seg_n, torch.float32)
    assert torch.equal(y1, y2)
    perm = torch.randperm(M, generator=torch.Generator().manual_seed(1)).to(x.device)
    y3 = _run(fn, x[perm].contiguous(), packed, wms, seg_n, torch.float32)
    assert torch.equal(y3, y1[perm])


def test_gemv_equals_gemm():
    K, seg_n = 2560, (2560, 640, 640)
    packed, wms, _ = _weights(6, seg_n, K)
    bits = synth.act_outliers_bf16(13, 64, K)
    x = bf16_dev(bits)
    yv = _run("gemv_w2a8", x, packed, wms, seg_n, torch.int32)
    ym = _run("gemm_w2a8", x, packed, wms, seg_n, torch.int32)
    assert torch.equal(yv, ym)


def test_extreme_accumulators():
    K = 6912
    M = 2
    x = np.full((M, K), 1.0, np.float32)
    x[1] = -1.0
    W = np.ones((8, K), np.float32)
    W[1::2] = -1.0
    packed, wm, codes = oracle.ternarize_pack(W)
    for fn in ("gemv_w2a8", "gemm_w2a8"):
        A = host(getattr(_bl(), fn)(to_dev(x), to_dev(packed), to_dev(np.array([wm])), y_dtype=torch.int32))
        exp = np.array([[127 * K, -127 * K] * 4, [-127 * K, 127 * K] * 4], np.int64)
        # plane order: output column n is weight row n
        assert_exact(A, exp.astype(np.int32), fn)


# ----------------------------------------------------------------------------- full-size shapes
@pytest.mark.parametrize("proj", [p for p, _, _ in synth.PROJECTIONS])
def test_decode_m1_projection(proj):
    """M=1 decode over each projection of one 2B4T layer, oracle-packed weights."""
    _, N, K = synth.PROJECTIONS[synth.PROJ_INDEX[proj]]
    packed, wm, codes = oracle.ternarize_pack(synth.layer_weight(0, proj))
    bits = synth.act_outliers_bf16(0, 1, K)
    q, a, A, y = oracle.bitlinear(f32_of_bf16(bits), codes, None, wm)
    yg = host(_bl().gemv_w2a8(bf16_dev(bits), to_dev(packed), to_dev(np.array([wm]))))
    assert_rows_close(yg, y, F32_TOL)
    assert max_ulp_diff(yg, y) == 0


@pytest.mark.parametrize("M", [16, 64])
def test_batched_decode_seven_projections(M):
    """M=16/64 with Student-t rows over the fused q|k|v and gate|up shapes and down."""
    bits = synth.act_heavy_tail_bf16(0, M, 2560)
    for projs in (("q", "k", "v"), ("gate", "up")):
        packs, wms, codes = [], [], []
        for p in projs:
            pk, wm, c = oracle.ternarize_pack(synth.layer_weight(0, p))
            packs.append(pk); wms.append(wm); codes.append(c)
        seg_n = [c.shape[0] for c in codes]
        rows = [0, M // 8, M // 2, M - 1]   # sample rows incl. Student-t rows
        q, a, A, y = oracle.bitlinear(f32_of_bf16(bits[rows]), np.concatenate(codes), seg_n, np.array(wms))
        yg = host(_bl().gemv_w2a8(bf16_dev(bits), to_dev(np.concatenate(packs)), to_dev(np.array(wms)),
                                  seg_n=seg_n))
        assert_rows_close(yg[rows], y, F32_TOL)
        assert max_ulp_diff(yg[rows], y) == 0


@pytest.mark.timeout(600)
def test_prefill_m2048_ffn_all_rows():
    """M=2048 prefill: fused gate|up (K=2560 -> 2x6912) and down (6912 -> 2560),
    every row and column: the int32 accumulators bit-exact against the exact
    integer product, the fp32 outputs bit-identical to the oracle's rescale."""
    M = 2048
    pg, wg, cg = oracle.ternarize_pack(synth.layer_weight(0, "gate"))
    pu, wu, cu = oracle.ternarize_pack(synth.layer_weight(0, "up"))
    wms = np.array([wg, wu], np.float32)
    cgu = np.concatenate([cg, cu])
    pgu = to_dev(np.concatenate([pg, pu]))
    bits = synth.act_normal_bf16(0, M, 2560)
    q, a, A, y = oracle.bitlinear_f64gemm(f32_of_bf16(bits), cgu, [6912, 6912], wms)
    Ag = _run("gemm_w2a8", bf16_dev(bits), pgu, to_dev(wms), (6912, 6912), torch.int32)
    assert_exact(host(Ag), A, "gate|up accumulators")
    yg = host(_run("gemm_w2a8", bf16_dev(bits), pgu, to_dev(wms), (6912, 6912), torch.float32))
    assert_exact(yg.view(np.uint32), y.view(np.uint32), "gate|up fp32 bits")
    del A, Ag, yg, y
    pd, wd, cd = oracle.ternarize_pack(synth.layer_weight(0, "down"))
    bits2 = synth.act_normal_bf16(1, M, 6912)
    _, _, A2, y2 = oracle.bitlinear_f64gemm(f32_of_bf16(bits2), cd, None, np.array([wd], np.float32))
    Ad = _run("gemm_w2a8", bf16_dev(bits2), pd, np.array([wd], np.float32), (2560,), torch.int32)
    assert_exact(host(Ad), A2, "down accumulators")
    yd = host(_run("gemm_w2a8", bf16_dev(bits2), pd, np.array([wd], np.float32), (2560,), torch.float32))
    assert_exact(yd.view(np.uint32), y2.view(np.uint32), "down fp32 bits")


# ----------------------------------------------------------------------------- degenerate rows and ties
def _zero_and_tie_rows(M, K):
    """Rows of x: an all-zero row, a row whose codes hit the half-way ties
    (max 127 so a = 1: +-63.5, 0.5, 1.5, 2.5, -2.5), a tiny row (max below the
    1e-5 floor) and N(0,1) rows."""
    x = synth.act_normal_f32(123 + K, M, K)
    x[0] = 0.0
    ties = np.array([127.0, 63.5, -63.5, 0.5, -0.5, 1.5, 2.5, -2.5, 3.5, -126.5], np.float32)
    x[1] = 0.0
    x[1, :min(K, ties.size)] = ties[:min(K, ties.size)]
    x[2] = 0.0
    x[2, ::7] = np.float32(3e-6)
    x[M - 1] = 0.0
    return x


@pytest.mark.parametrize("fn,M,K,seg_n,kind", [("gemv_w2a8", 4, 2560, (2560, 640, 640), "bf16"),
                                               ("gemv_w2a8", 3, 2560, (64,), "f32"),
                                               ("gemv_w2a8", 16, 2560, (128, 32), "bf16"),
                                               ("gemm_w2a8", 130, 2560, (256, 64), "bf16"),
                                               ("gemm_w2a8", 300, 6912, (128,), "f32")])
def test_zero_rows_and_ties(fn, M, K, seg_n, kind):
    """Zero rows, exact .5 ties and sub-floor rows through the quantizing
    prologues (the decode kernel's fused quantizer, the row kernel before the
    prefill GEMM): codes, accumulators and outputs exact; zero rows give +0."""
    packed, wms, codes = _weights(900 + M, seg_n, K)
    x = _zero_and_tie_rows(M, K)
    if kind == "bf16":
        bits = synth.bf16_bits(x)
        x_host, x_dev = f32_of_bf16(bits), bf16_dev(bits)
    else:
        x_host, x_dev = x, to_dev(x)
    q, a, A, y = oracle.bitlinear(x_host, codes, seg_n, wms)
    assert (q[0] == 0).all() and (q[M - 1] == 0).all() and (A[0] == 0).all()
    Ag = _run(fn, x_dev, packed, wms, seg_n, torch.int32)
    assert_exact(host(Ag), A, "accumulators")
    yg = host(_run(fn, x_dev, packed, wms, seg_n, torch.float32))
    assert_exact(yg.view(np.uint32), y.view(np.uint32), "fp32 bits (zero rows +0)")


# ----------------------------------------------------------------------------- batched decode
def _proj_case(layer, proj, M, seed, kind="outliers"):
    _, N, K = synth.PROJECTIONS[synth.PROJ_INDEX[proj]]
    packed, wm, codes = oracle.ternarize_pack(synth.layer_weight(layer, proj))
    if kind == "heavy":
        bits = synth.act_heavy_tail_bf16(seed, M, K)
    else:
        bits = synth.act_outliers_bf16(seed, M, K)
    return packed, wm, codes, bits


@pytest.mark.parametrize("M", [1, 2, 4, 16, 64])
def test_batched_seven_projections(M):
    """The 7 projections of a layer, each with its own activations, in one call."""
    cases = [_proj_case(0, p, M, 50 + j, "heavy" if M >= 16 else "outliers")
             for j, (p, _, _) in enumerate(synth.PROJECTIONS)]
    probs = [dict(x=bf16_dev(bits), packed=to_dev(pk), w_mean=to_dev(np.array([wm]))) for pk, wm, _, bits in cases]
    outs = _bl().gemv_w2a8_batched(probs)
    rows = list(range(M)) if M <= 4 else [0, M // 8, M - 1]
    for (pk, wm, codes, bits), y in zip(cases, outs):
        _, _, _, yr = oracle.bitlinear(f32_of_bf16(bits[rows]), codes, None, wm)
        yh = host(y)[rows]
        assert_rows_close(yh, yr, F32_TOL)
        assert max_ulp_diff(yh, yr) == 0


def test_batched_mixed_kinds():
    """Fused-prologue, int8-input, larger-M and ragged-K problems in one call."""
    specs = [(1, 2560, (64, 16, 16), "bf16"), (8, 512, (128,), "f32"), (3, 256, (32,), "i8"),
             (2, 100, (16,), "bf16"), (1, 6912, (64,), "bf16")]
    probs, refs = [], []
    for i, (M, K, seg_n, kind) in enumerate(specs):
        packed, wms, codes = _weights(300 + i, seg_n, K)
        if kind == "bf16":
            bits = synth.act_outliers_bf16(70 + i, M, K)
            xh, xd = f32_of_bf16(bits), bf16_dev(bits)
        else:
            xh = synth.act_normal_f32(70 + i, M, K)
            xd = to_dev(xh)
        q, a, A, y = oracle.bitlinear(xh, codes, seg_n, wms)
        pr = dict(x=xd, packed=to_dev(packed), w_mean=to_dev(wms), seg_n=list(seg_n) if len(seg_n) > 1 else None)
        if kind == "i8":
            pr.update(x=to_dev(q), a=to_dev(a))
        probs.append(pr)
        refs.append(y)
    outs = _bl().gemv_w2a8_batched(probs)
    for y, yr in zip(outs, refs):
        assert_rows_close(host(y), yr, F32_TOL)
        assert max_ulp_diff(host(y), yr) == 0
    # each problem alone gives the same bits
    for pr, y in zip(probs, outs):
        kw = {k: v for k, v in pr.items() if k in ("seg_n", "a")}
        y1 = _bl().gemv_w2a8(pr["x"], pr["packed"], pr["w_mean"], **kw)
        assert torch.equal(y1, y)
