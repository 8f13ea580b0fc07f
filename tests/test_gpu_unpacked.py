"""GPU parity of the offline-unpacked path (bl_unpack_bf16, bl_gemm_unpacked)
against the oracle: the unpacked codes equal the oracle's unpack (plane
order) bit for bit, and the dense bf16 product gives the same int32
accumulators and the same fp32 / bf16 output bits as the oracle's BitLinear
(every partial sum is an exact integer in fp32).  Outputs guarded."""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import assert_exact, bf16_dev, f32_of_bf16, guarded, host, requires_gpu, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


def _weights(seed, seg_n, K):
    packs, wms, codes = [], [], []
    for i, n in enumerate(seg_n):
        p, wm, c = oracle.ternarize_pack(synth.master_weight(seed + 17 * i, n, K))
        packs.append(p)
        wms.append(wm)
        codes.append(c)
    return np.concatenate(packs), np.array(wms, np.float32), np.concatenate(codes)


def _unpacked(packed, seg_n=None):
    bl = _bl()
    R, K = packed.shape
    out = guarded((4 * R, K), torch.bfloat16)
    bl.unpack_bf16(to_dev(packed), seg_n=list(seg_n) if seg_n is not None and len(seg_n) > 1 else None, w_codes=out.t)
    out.check("w_codes")
    return out.t


@pytest.mark.parametrize("seg_n,K", [((8,), 1), ((12,), 7), ((4,), 33), ((256,), 256), ((640,), 2560),
                                     ((2560,), 6912), ((16, 8, 8), 64), ((2560, 640, 640), 256), ((6912, 6912), 96)])
def test_unpack_matches_the_oracle(seg_n, K):
    """Each segment packed on its own by the oracle, stacked; the unpacked rows
    are the segments' codes in output-column order."""
    rng = np.random.default_rng(sum(seg_n) + K)
    codes = [rng.integers(-1, 2, size=(n, K)).astype(np.int8) for n in seg_n]
    packed = np.concatenate([oracle.pack(c) for c in codes])
    w = _unpacked(packed, seg_n)
    ref = []
    for c in codes:
        back, bad = oracle.unpack(oracle.pack(c))
        assert bad == 0 and np.array_equal(back, c)
        ref.append(back)
    want = synth.bf16_bits(np.concatenate(ref).astype(np.float32))
    assert_exact(host(w), want, "bf16 codes")


CASES = [  # (M, K, seg_n, x kind)
    (1, 2560, (2560,), "bf16"), (1, 2560, (2560, 640, 640), "bf16"), (1, 6912, (2560,), "bf16"),
    (3, 264, (36,), "f32"), (4, 2560, (64, 16, 16), "bf16"), (5, 256, (12,), "f32"),
    (64, 2560, (256, 128), "bf16"), (130, 6912, (256,), "f32"), (300, 2560, (640, 128, 128), "i8"),
]


@pytest.mark.parametrize("M,K,seg_n,kind", CASES)
def test_gemm_unpacked_equals_the_oracle(M, K, seg_n, kind):
    bl = _bl()
    packed, wms, codes = _weights(500 + M + K, seg_n, K)
    if kind == "bf16":
        bits = synth.act_outliers_bf16(M + 7, M, K)
        xh, xd = f32_of_bf16(bits), bf16_dev(bits)
    else:
        xh = synth.act_normal_f32(M + 7, M, K)
        xd = to_dev(xh)
    q, a, A, y = oracle.bitlinear(xh, codes, seg_n, wms)
    ad = None
    if kind == "i8":
        xd, ad = to_dev(q), to_dev(a)
    w = _unpacked(packed, seg_n)
    N = sum(seg_n)
    sn = list(seg_n) if len(seg_n) > 1 else None
    for ydt in (torch.int32, torch.float32, torch.bfloat16):
        out = guarded((M, N), ydt)
        bl.gemm_unpacked(xd, w, to_dev(wms), seg_n=sn, y_dtype=ydt, a=ad, y=out.t)
        out.check(f"y {ydt}")
        got = host(out.t)
        if ydt == torch.int32:
            assert_exact(got, A, "int32 accumulators")
        elif ydt == torch.float32:
            assert_exact(got.view(np.uint32), y.view(np.uint32), "fp32 bits")
        else:
            assert_exact(got, oracle.to_bf16(y), "bf16 bits")
    # and the packed path gives the same bits
    yp = bl.gemm_w2a8(xd, to_dev(packed), to_dev(wms), seg_n=sn, a=ad)
    assert torch.equal(yp, bl.gemm_unpacked(xd, w, to_dev(wms), seg_n=sn, a=ad))


@pytest.mark.timeout(600)
def test_gemm_unpacked_prefill_m2048_all_rows():
    """M=2048 gate|up (K=2560 -> 2x6912) on the bf16 MFMA GEMM, every row."""
    bl = _bl()
    M = 2048
    pg, wg, cg = oracle.ternarize_pack(synth.layer_weight(0, "gate"))
    pu, wu, cu = oracle.ternarize_pack(synth.layer_weight(0, "up"))
    wms = np.array([wg, wu], np.float32)
    bits = synth.act_normal_bf16(0, M, 2560)
    _, _, A, y = oracle.bitlinear_f64gemm(f32_of_bf16(bits), np.concatenate([cg, cu]), [6912, 6912], wms)
    w = _unpacked(np.concatenate([pg, pu]), (6912, 6912))
    out = guarded((M, 13824))
    bl.gemm_unpacked(bf16_dev(bits), w, to_dev(wms), seg_n=[6912, 6912], y=out.t)
    out.check("y")
    assert_exact(host(out.t).view(np.uint32), y.view(np.uint32), "fp32 bits")


def test_gemm_unpacked_rejects_unsupported_shapes():
    bl = _bl()
    x = torch.zeros((2, 100), dtype=torch.float32, device="cuda")     # K = 100: not a multiple of 8
    w = torch.zeros((8, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bl.BitLinearError):
        bl.gemm_unpacked(x, w, torch.ones(1, dtype=torch.float32, device="cuda"))
