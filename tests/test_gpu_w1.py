"""GPU parity of the 1-bit BitLinear (bl_binarize_pack, bl_layernorm_quant,
bl_gemm_w1a8, bl_bitlinear_w1) against the oracle.

Acceptance: packed bytes, weight scales, int8 codes and activation scales
bit-exact; fp32 outputs bit-exact too (the accumulator is an exact integer
and the rescale is the same two fp32 roundings on both sides).  The layer
norm's fp64 sums run in a different order on the device (a tree) than in the
oracle (index order); the fp32 results they feed agree unless a sum lands
within one fp64 ulp of an fp32 rounding boundary, which the seeded inputs
below do not hit.  Outputs guarded (never-written elements, writes past the
end)."""
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


def _pack_dev(W: np.ndarray):
    """bl_binarize_pack twice, into buffers pre-filled with 0x00 and 0xFF:
    every byte must come out the same both times (so every byte was written)."""
    bl = _bl()
    N, K = W.shape
    Wd = to_dev(W)
    outs = []
    for fill in (0x00, 0xFF):
        g = guarded((N // 8, K), torch.uint8, fill=fill)
        s = guarded((1,), torch.float32)
        bl.binarize_pack(Wd, packed=g.t, w_scale=s.t)
        g.check("packed")
        s.check("w_scale")
        outs.append((host(g.t), host(s.t)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    return outs[0][0], outs[0][1][0]


@pytest.mark.parametrize("N,K", [(8, 4), (24, 20), (64, 36), (2560, 2560), (6912, 2560), (2560, 6912)])
def test_binarize_pack_matches_the_oracle(N, K):
    W = synth.master_weight(N + 7 * K, N, K)
    W[0, :min(K, 3)] = [0.0, -0.0, 1e-30][:min(K, 3)]   # zeros and a tiny value: +1
    p, s = _pack_dev(W)
    rp, rs, _ = oracle.binarize_pack(W)
    assert_exact(p, rp, "packed")
    assert s.view(np.uint32) == np.float32(rs).view(np.uint32)


def _ln_case(M, K, kind, seed):
    if kind == "bf16":
        bits = synth.act_outliers_bf16(seed, M, K)
        return bits, f32_of_bf16(bits)
    x = (2.0 + 3.0 * synth.act_normal_f32(seed, M, K)).astype(np.float32)
    return x, x


@pytest.mark.parametrize("M,K,kind,affine", [(1, 4, "f32", False), (3, 20, "bf16", True), (1, 2560, "bf16", False),
                                             (5, 2560, "f32", True), (2, 6912, "bf16", True), (130, 2560, "bf16", False),
                                             (4, 16384, "f32", True), (17, 1028, "f32", False)])
def test_layernorm_quant_matches_the_oracle(M, K, kind, affine):
    bl = _bl()
    raw, x32 = _ln_case(M, K, kind, M * 31 + K)
    xd = bf16_dev(raw) if kind == "bf16" else to_dev(raw)
    gamma = beta = None
    if affine:
        r = np.random.default_rng(K)
        gamma = (1.0 + 0.25 * r.standard_normal(K)).astype(np.float32)
        beta = (0.1 * r.standard_normal(K)).astype(np.float32)
    q = guarded((M, K), torch.int8)
    a = guarded((M,), torch.float32)
    bl.layernorm_quant(xd, None if gamma is None else to_dev(gamma), None if beta is None else to_dev(beta),
                       1e-5, q=q.t, a=a.t)
    q.check("q")
    a.check("a")
    rq, ra = oracle.quant_act(oracle.layernorm(x32, gamma, beta, 1e-5))
    assert_exact(host(q.t), rq, "codes")
    assert_exact(host(a.t).view(np.uint32), ra.view(np.uint32), "scales")


def test_layernorm_quant_row_stride_and_constant_rows():
    """Rows read with a stride above K; a constant row normalizes to zeros
    (codes 0, scale 127 / 1e-5)."""
    bl = _bl()
    M, K, ld = 4, 256, 320
    x = synth.act_normal_f32(3, M, ld)
    x[2, :] = 5.5
    xd = to_dev(x)[:, :K]
    q, a = bl.layernorm_quant(xd)
    rq, ra = oracle.quant_act(oracle.layernorm(np.ascontiguousarray(x[:, :K])))
    assert_exact(host(q), rq, "codes")
    assert_exact(host(a).view(np.uint32), ra.view(np.uint32), "scales")
    assert (host(q)[2] == 0).all() and host(a)[2] == np.float32(127.0) / np.float32(1e-5)


def _codes(rng, M, K):
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    q[0, :min(K, 8)] = [-128, 127, -128, 127, 0, -1, 1, -128][:min(K, 8)]
    a = (127.0 / rng.uniform(0.5, 30.0, size=M)).astype(np.float32)
    return q, a


@pytest.mark.parametrize("M,N,K", [(1, 8, 16), (1, 136, 48), (5, 2560, 2560), (16, 128, 64), (17, 264, 80),
                                   (33, 2560, 2560), (64, 6912, 2560), (1, 2560, 6912), (300, 1024, 2560),
                                   (2, 8, 16384),
                                   # at least one 128 x 32 tile per CU: the LDS-staged kernel (ragged token
                                   # and row tiles; N/8 not a multiple of 4: scalar stores)
                                   (1200, 8008, 256), (1000, 8000, 384), (2048, 6912, 2560)])
def test_gemm_w1a8_matches_the_oracle(M, N, K):
    bl = _bl()
    rng = np.random.default_rng(M * 7 + N + K)
    W = synth.master_weight(N * 3 + K, N, K)
    packed, ws, signs = oracle.binarize_pack(W)
    q, a = _codes(rng, M, K)
    y = guarded((M, N), torch.float32)
    bl.gemm_w1a8(to_dev(q), to_dev(a), to_dev(packed), to_dev(np.array([ws], np.float32)), N=N, y=y.t)
    y.check("y")
    A = oracle.contract_f64(q, signs)
    ref = oracle.rescale(A, a, [N], ws)
    assert_exact(host(y.t).view(np.uint32), ref.view(np.uint32), "y")


def test_gemm_w1a8_extreme_accumulators():
    """Every code -128 against all-(+1) and all-(-1) rows: |A| = 128 K, the
    largest the accumulator sees."""
    bl = _bl()
    M, N, K = 3, 16, 16384
    W = np.ones((N, K), np.float32)
    W[N // 2:] = -1.0
    packed, ws, signs = oracle.binarize_pack(W)
    q = np.full((M, K), -128, np.int8)
    a = np.array([1.0, 2.0, 0.5], np.float32)
    y = bl.gemm_w1a8(to_dev(q), to_dev(a), to_dev(packed), to_dev(np.array([ws], np.float32)))
    ref = oracle.rescale(oracle.contract_f64(q, signs), a, [N], ws)
    assert_exact(host(y).view(np.uint32), ref.view(np.uint32), "y")


def test_bitlinear_w1_seven_projections_decode():
    """A layer's seven projection shapes (q, k, v, o, gate, up, down of the
    2B4T configuration) at one token, each with its own input: one call (the
    fused single-token launch), every output bit against the oracle."""
    bl = _bl()
    probs, refs = [], []
    for j, (name, N, K) in enumerate(synth.PROJECTIONS):
        W = synth.master_weight(1000 + j, N, K)
        packed, ws, signs = oracle.binarize_pack(W)
        bits = synth.act_outliers_bf16(200 + j, 1, K)
        y = guarded((1, N), torch.float32)
        probs.append(dict(x=bf16_dev(bits), packed=to_dev(packed), w_scale=to_dev(np.array([ws], np.float32)),
                          y=y.t, guard=y))
        refs.append(oracle.bitlinear_w1_f64gemm(f32_of_bf16(bits), signs, ws)[3])
    bl.bitlinear_w1_batched([{k: v for k, v in p.items() if k != "guard"} for p in probs])
    for j, (p, ref) in enumerate(zip(probs, refs)):
        p["guard"].check(f"y {j}")
        assert_exact(host(p["y"]).view(np.uint32), ref.view(np.uint32), f"projection {j}")


@pytest.mark.parametrize("M,N,K", [(2048, 2560, 2560), (64, 6912, 2560), (200, 2560, 6912), (2048, 6912, 2560)])
def test_bitlinear_w1_prefill_all_rows(M, N, K):
    """Prefill sizes, every output row, with gain and bias."""
    bl = _bl()
    r = np.random.default_rng(M + N)
    W = synth.master_weight(M + N + K, N, K)
    packed, ws, signs = oracle.binarize_pack(W)
    bits = synth.act_outliers_bf16(M, M, K)
    gamma = (1.0 + 0.25 * r.standard_normal(K)).astype(np.float32)
    beta = (0.1 * r.standard_normal(K)).astype(np.float32)
    y = guarded((M, N), torch.float32)
    bl.bitlinear_w1(bf16_dev(bits), to_dev(packed), to_dev(np.array([ws], np.float32)), to_dev(gamma), to_dev(beta),
                    y=y.t)
    y.check("y")
    ref = oracle.bitlinear_w1_f64gemm(f32_of_bf16(bits), signs, ws, gamma, beta)[3]
    assert_exact(host(y.t).view(np.uint32), ref.view(np.uint32), "y")


@pytest.mark.parametrize("N,K,kind,affine", [(8, 16, "f32", True), (136, 48, "bf16", False), (2560, 8192, "f32", True),
                                             (640, 2560, "bf16", True), (2560, 8208, "bf16", False),
                                             (24, 4112, "f32", False)])
def test_bitlinear_w1_single_token(N, K, kind, affine):
    """One token: the fused decode launch (K <= 8192), or the two-launch path
    beyond it (K = 8208)."""
    bl = _bl()
    r = np.random.default_rng(N * 3 + K)
    W = synth.master_weight(N + 5 * K, N, K)
    packed, ws, signs = oracle.binarize_pack(W)
    raw, x32 = _ln_case(1, K, kind, N + K)
    gamma = beta = None
    if affine:
        gamma = (1.0 + 0.25 * r.standard_normal(K)).astype(np.float32)
        beta = (0.1 * r.standard_normal(K)).astype(np.float32)
    y = guarded((1, N), torch.float32)
    bl.bitlinear_w1(bf16_dev(raw) if kind == "bf16" else to_dev(raw), to_dev(packed), to_dev(np.array([ws], np.float32)),
                    None if gamma is None else to_dev(gamma), None if beta is None else to_dev(beta), y=y.t)
    y.check("y")
    ref = oracle.bitlinear_w1_f64gemm(x32, signs, ws, gamma, beta)[3]
    assert_exact(host(y.t).view(np.uint32), ref.view(np.uint32), "y")


def test_bitlinear_w1_mixed_batch():
    """A batch mixing input types and a two-row problem takes the two-launch
    path; the same outputs as the oracle."""
    bl = _bl()
    probs, refs = [], []
    for j, (M, N, K, kind) in enumerate([(1, 256, 512, "bf16"), (1, 128, 256, "f32"), (2, 64, 1024, "bf16")]):
        W = synth.master_weight(77 + j, N, K)
        packed, ws, signs = oracle.binarize_pack(W)
        raw, x32 = _ln_case(M, K, kind, 40 + j)
        y = guarded((M, N), torch.float32)
        probs.append((dict(x=bf16_dev(raw) if kind == "bf16" else to_dev(raw), packed=to_dev(packed),
                           w_scale=to_dev(np.array([ws], np.float32)), y=y.t), y))
        refs.append(oracle.bitlinear_w1_f64gemm(x32, signs, ws)[3])
    bl.bitlinear_w1_batched([p for p, _ in probs])
    for j, ((p, g), ref) in enumerate(zip(probs, refs)):
        g.check(f"y {j}")
        assert_exact(host(p["y"]).view(np.uint32), ref.view(np.uint32), f"problem {j}")
