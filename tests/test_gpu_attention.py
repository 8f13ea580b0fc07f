"""GPU parity of the decode-step attention (bl_attn_decode) against the oracle.

The oracle rotates and attends in fp64; the kernels work in fp32 (RoPE from
the fp32 table, fp32 scores, exponentials and sums).  Acceptance, derived
from fp32 rounding over a 128-term dot product and a softmax over at most
2048 positions: max |out - ref| <= 1e-4 * max(1, max |ref|) per call; the
cached value at pos is bit-exact (a copy) and the cached key within 1e-6 of
the fp64 rotation (relative to its row's maximum).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev, host, requires_gpu, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]

ATTN_TOL = 1e-4


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


def _inputs(seed, H, KVH, S, D=128):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(H * D).astype(np.float32)
    kn = rng.standard_normal(KVH * D).astype(np.float32)
    vn = rng.standard_normal(KVH * D).astype(np.float32)
    kc = rng.standard_normal((KVH, S, D)).astype(np.float32)
    vc = rng.standard_normal((KVH, S, D)).astype(np.float32)
    return q, kn, vn, kc, vc


def _run(q, kn, vn, pos, kc, vc, base, H, KVH):
    bl = _bl()
    S = kc.shape[1]
    rc, rs = bl.rope_table(S, 128, base, device=dev())
    kcd, vcd = to_dev(kc), to_dev(vc)
    out = bl.attn_decode(to_dev(q), to_dev(kn), to_dev(vn), pos, kcd, vcd, rc, rs, H, KVH)
    torch.cuda.synchronize()
    return host(out).reshape(H, 128), host(kcd), host(vcd)


def _check(seed, H, KVH, S, positions, base=500000.0):
    q, kn, vn, kc, vc = _inputs(seed, H, KVH, S)
    for pos in positions:
        out, kcg, vcg = _run(q, kn, vn, pos, kc, vc, base, H, KVH)
        ref = oracle.attn_decode(q, kn, vn, pos, kc, vc, base, H, KVH)
        err = np.abs(out - ref).max()
        assert err <= ATTN_TOL * max(1.0, np.abs(ref).max()), (pos, err)
        # the token's value copied and its rotated key written at pos; the rest untouched
        assert np.array_equal(vcg[:, pos], vn.reshape(KVH, 128))
        kr = oracle.rope(kn.reshape(KVH, 128), pos, base)
        assert np.abs(kcg[:, pos] - kr).max() <= 1e-6 * max(1.0, np.abs(kr).max())
        mask = np.ones(S, bool)
        mask[pos] = False
        assert np.array_equal(kcg[:, mask], kc[:, mask]) and np.array_equal(vcg[:, mask], vc[:, mask])


@pytest.mark.parametrize("H,KVH", [(4, 1), (4, 4), (6, 3), (8, 2)])
def test_attn_decode_small(H, KVH):
    # chunk edges (64 positions), a single position, the last one
    _check(11, H, KVH, 200, [0, 1, 63, 64, 65, 127, 128, 199])


def test_attn_decode_model_shape():
    # 20 query heads, 5 key/value heads, 128 dimensions, 2048 positions
    _check(12, 20, 5, 2048, [0, 700, 2047], base=500000.0)


def test_attn_decode_many_chunks():
    # 79 and 512 chunks of 64 positions: merges over several batches, and the
    # longest cache the kernel serves
    _check(15, 8, 2, 5000, [4999, 4160])
    _check(16, 4, 1, 32768, [32767])


def test_attn_decode_other_base_and_peaked_scores():
    H, KVH, S, pos = 20, 5, 300, 257
    q, kn, vn, kc, vc = _inputs(13, H, KVH, S)
    # one cached key per group nearly parallel to the group's rotated queries:
    # a sharply peaked softmax
    qr = oracle.rope(q.reshape(H, 128), pos, 10000.0)
    for g in range(KVH):
        kc[g, 42] = (6.0 * qr[4 * g] / np.linalg.norm(qr[4 * g]) * np.sqrt(128)).astype(np.float32)
    out, _, _ = _run(q, kn, vn, pos, kc, vc, 10000.0, H, KVH)
    ref = oracle.attn_decode(q, kn, vn, pos, kc, vc, 10000.0, H, KVH)
    assert np.abs(out - ref).max() <= ATTN_TOL * max(1.0, np.abs(ref).max())


def test_attn_decode_sequence_from_empty_cache():
    """Decode 70 tokens from an empty cache; the oracle keeps its own cache
    (its fp64 rotations rounded to fp32), so no GPU value feeds it."""
    bl = _bl()
    H, KVH, S, base = 8, 2, 96, 500000.0
    rng = np.random.default_rng(14)
    rc, rs = bl.rope_table(S, 128, base, device=dev())
    kcd = torch.zeros((KVH, S, 128), dtype=torch.float32, device=dev())
    vcd = torch.zeros_like(kcd)
    kc_ref = np.zeros((KVH, S, 128), np.float32)
    vc_ref = np.zeros((KVH, S, 128), np.float32)
    for pos in range(70):
        q = rng.standard_normal(H * 128).astype(np.float32)
        kn = rng.standard_normal(KVH * 128).astype(np.float32)
        vn = rng.standard_normal(KVH * 128).astype(np.float32)
        out = host(bl.attn_decode(to_dev(q), to_dev(kn), to_dev(vn), pos, kcd, vcd, rc, rs, H, KVH)).reshape(H, 128)
        ref = oracle.attn_decode(q, kn, vn, pos, kc_ref, vc_ref, base, H, KVH)
        assert np.abs(out - ref).max() <= ATTN_TOL * max(1.0, np.abs(ref).max()), pos
        kc_ref[:, pos] = oracle.rope(kn.reshape(KVH, 128), pos, base).astype(np.float32)
        vc_ref[:, pos] = vn.reshape(KVH, 128)


# ----------------------------------------------------------------------------- sub-norm + quantization
@pytest.mark.parametrize("M,K,kind,gain", [(1, 2560, "bf16", False), (4, 2560, "f32", True),
                                           (65, 6912, "f32", False), (3, 100, "f32", True), (1, 20, "bf16", True)])
def test_rmsnorm_quant(M, K, kind, gain):
    from bit_ternary_weight_amd import synth
    from gpu_helpers import assert_exact, bf16_dev, f32_of_bf16
    bl = _bl()
    if kind == "bf16":
        bits = synth.act_outliers_bf16(20 + M, M, K)
        h_host, h_dev = f32_of_bf16(bits), bf16_dev(bits)
    else:
        h_host = synth.act_normal_f32(20 + M, M, K)
        h_dev = to_dev(h_host)
    g = np.random.default_rng(K).uniform(0.5, 1.5, size=K).astype(np.float32) if gain else None
    q, a = bl.rmsnorm_quant(h_dev, gain=None if g is None else to_dev(g), eps=1e-5)
    rq, ra = oracle.quant_act(oracle.rmsnorm(h_host, g, 1e-5))
    assert_exact(host(q), rq, "codes")
    assert_exact(host(a), ra, "scales")


# ----------------------------------------------------------------------------- one layer with attention
def test_decode_layer_with_attention_stagewise():
    """stack.decode_layer_attn over 3 layers and several positions, each stage
    against the oracle on the GPU's own input to that stage (no cascade):
    q|k|v, attention (and the cache rows it appends), attn_sub_norm +
    quantization, o, the FFN chain."""
    from bit_ternary_weight_amd import stack, synth
    from gpu_helpers import F32_TOL, assert_exact, assert_rows_close, bf16_dev, f32_of_bf16, max_ulp_diff
    H, KV, S, L = synth.HIDDEN, synth.KV_DIM, 300, 3
    layers = stack.build_layers(L, dev())
    cache = stack.alloc_kv(L, S, dev())
    rng = np.random.default_rng(21)
    # earlier tokens: random rotated keys and values at positions < 257
    for l in range(L):
        cache.k[l][:, :257] = torch.from_numpy(rng.standard_normal((5, 257, 128)).astype(np.float32)).to(dev())
        cache.v[l][:, :257] = torch.from_numpy(rng.standard_normal((5, 257, 128)).astype(np.float32)).to(dev())
    codes_l = []
    for l in range(L):
        codes, wms = {}, {}
        for p, _, _ in synth.PROJECTIONS:
            _, wm, c = oracle.ternarize_pack(synth.layer_weight(l, p))
            codes[p], wms[p] = c, wm
        codes_l.append((codes, wms))
    for step, pos in enumerate((257, 258, 259)):
        bits = synth.act_outliers_bf16(30 + step, 1, H)
        x, x_host = bf16_dev(bits), f32_of_bf16(bits)
        for l, lw in enumerate(layers):
            codes, wms = codes_l[l]
            kc0, vc0 = host(cache.k[l]).copy(), host(cache.v[l]).copy()
            dbg = {}
            y = stack.decode_layer_attn(x, lw, cache, l, pos, debug=dbg)
            qkv_codes = np.concatenate([codes["q"], codes["k"], codes["v"]])
            wq = np.array([wms["q"], wms["k"], wms["v"]], np.float32)
            _, _, _, r_qkv = oracle.bitlinear(x_host, qkv_codes, [H, KV, KV], wq)
            g_qkv = host(dbg["y_qkv"])
            assert_rows_close(g_qkv, r_qkv, F32_TOL, f"qkv {l}")
            assert max_ulp_diff(g_qkv, r_qkv) == 0
            r_att = oracle.attn_decode(g_qkv[0, :H], g_qkv[0, H:H + KV], g_qkv[0, H + KV:], pos, kc0, vc0,
                                       stack.ROPE_BASE, 20, 5).reshape(-1)
            g_att = host(dbg["att"])
            assert np.abs(g_att - r_att).max() <= ATTN_TOL * max(1.0, np.abs(r_att).max()), (l, pos)
            assert np.array_equal(host(cache.v[l])[:, pos], g_qkv[0, H + KV:].reshape(5, 128))
            rq, ra = oracle.quant_act(oracle.rmsnorm(g_att.reshape(1, H), None, 1e-5))
            assert_exact(host(dbg["q_o"]), rq, f"attn_sub_norm codes {l}")
            assert_exact(host(dbg["a_o"]), ra, f"attn_sub_norm scale {l}")
            r_o = oracle.rescale(oracle.contract(rq, codes["o"]), ra, None, wms["o"])
            assert_exact(host(dbg["y_o"]).view(np.uint32), r_o.view(np.uint32), f"o {l}")
            gu = np.concatenate([codes["gate"], codes["up"]])
            ch = oracle.ffn_chain(r_o, gu, np.array([wms["gate"], wms["up"]], np.float32), codes["down"], wms["down"])
            yh = host(y)
            assert_rows_close(yh, ch["y"], F32_TOL, f"layer {l}")
            x, x_host = y.clone(), yh


@pytest.mark.parametrize("M,K,N,kind,gain,ydt", [(1, 2560, 2560, "f32", False, torch.float32),
                                                 (4, 2560, 640, "bf16", True, torch.float32),
                                                 (1, 6912, 2560, "f32", True, torch.bfloat16),
                                                 (3, 100, 64, "f32", False, torch.float32),
                                                 (70, 256, 128, "f32", True, torch.float32)])
def test_subln_gemv(M, K, N, kind, gain, ydt):
    """bl_subln_gemv_w2a8 = RMSNorm -> quantize -> BitLinear: the fused decode
    launch, the two-launch fallback (K not a multiple of 16) and the prefill
    path (M > 64), against the oracle's rmsnorm, quant_act, contract, rescale."""
    from bit_ternary_weight_amd import synth
    from gpu_helpers import assert_exact, bf16_dev, f32_of_bf16
    bl = _bl()
    if kind == "bf16":
        bits = synth.act_outliers_bf16(40 + M, M, K)
        h_host, h_dev = f32_of_bf16(bits), bf16_dev(bits)
    else:
        h_host = synth.act_normal_f32(40 + M, M, K)
        h_dev = to_dev(h_host)
    g = np.random.default_rng(K + 1).uniform(0.5, 1.5, size=K).astype(np.float32) if gain else None
    packed, wm, codes = oracle.ternarize_pack(synth.master_weight(50 + K, N, K))
    q = torch.empty((M, K), dtype=torch.int8, device=dev())
    a = torch.empty(M, dtype=torch.float32, device=dev())
    y = bl.subln_gemv_w2a8(h_dev, to_dev(packed), to_dev(np.array([wm], np.float32)),
                           gain=None if g is None else to_dev(g), y_dtype=ydt, q_out=q, a_out=a)
    rq, ra = oracle.quant_act(oracle.rmsnorm(h_host, g, 1e-5))
    assert_exact(host(q), rq, "codes")
    assert_exact(host(a), ra, "scales")
    ref = oracle.rescale(oracle.contract(rq, codes), ra, None, wm)
    if ydt == torch.float32:
        assert_exact(host(y).view(np.uint32), ref.view(np.uint32), "y bits")
    else:
        yb = host(y.view(torch.int16)).view(np.uint16)
        assert_exact(yb, oracle.to_bf16(ref), "bf16 y")


# ----------------------------------------------------------------------------- prefill attention
# The oracle is the plain fp64 attention (nothing rounded).  The kernel rotates
# in fp32 from the fp32 table, rounds the rotated queries and keys, the values
# and the (unnormalized) probabilities to bf16 (unit roundoff u = 2^-8), and
# sums in fp32.  Tolerance derived from that, per output element (row p, head
# h, dimension d), with a_ji = q'_i k'_ji / sqrt(D) the fp64 score terms and
# w the fp64 softmax weights:
#   * score error  |ds_j| <= Delta_j = (2u + u^2) sum_i |a_ji|
#                                      + 2^-19 sum_i r(q)_i r(k_j)_i / sqrt(D),
#     r(x)_i = |x_i| + |x_(i +- 64)| bounding the fp32 rotation's error
#     (table and arithmetic, a few 2^-24) and the fp32 score sums and scaling;
#   * weights: a shift of every score by at most Delta moves each normalized
#     weight by a factor within exp(+-2 Delta), Delta = max_j Delta_j;
#   * probabilities and values rounded to bf16 (1 + u each), fp32 sums of
#     n = p + 1 terms in the numerator and in the normalizer (g = (n + 8) 2^-24);
#   => worst case  |got - ref| <= sum_j w_j |v_jd| (e^{2 Delta} (1+u)^2 (1+g)^2/(1-g) - 1).
#   * rounding model: independent roundings with E[e^2] <= u^2/3 give the
#     variance  (u^2/3) [ sum_j w_j^2 (v_jd - o_d)^2 sum_i a_ji^2
#                         + sum_i (q'_i / sqrt(D))^2 C_id^2 + 2 sum_j w_j^2 v_jd^2 ],
#     C_id = sum_j w_j k'_ji (v_jd - o_d) (the query's rounding, shared by all
#     keys); the mean of err^2 / variance over a call must stay below 2.
U = 2.0 ** -8


def _attn_prefill_bounds(q, k, v, base, H, KVH, rows):
    """(worst-case bound, model variance), each [len(rows), H*128]."""
    D = 128
    M = q.shape[0]
    G = H // KVH
    pmax = max(rows)
    kr = np.stack([oracle.rope(k[j].reshape(KVH, D), j, base) for j in range(pmax + 1)])     # [P, KVH, D]
    kk = k[:pmax + 1].astype(np.float64).reshape(-1, KVH, D)
    rk = np.abs(kk) + np.abs(np.roll(kk, D // 2, axis=2))                                  # |k_i| + |k_(i+-64)|
    vv = v[:pmax + 1].astype(np.float64).reshape(-1, KVH, D)
    bound = np.empty((len(rows), H * D))
    var = np.empty((len(rows), H * D))
    for n, p in enumerate(rows):
        qr = oracle.rope(q[p].reshape(H, D), p, base)
        qq = q[p].astype(np.float64).reshape(H, D)
        rq = np.abs(qq) + np.abs(np.roll(qq, D // 2, axis=1))
        g = (p + 1 + 8) * 2.0 ** -24
        for h in range(H):
            kv = h // G
            K_, V_ = kr[:p + 1, kv], vv[:p + 1, kv]
            a = (K_ * qr[h]) / np.sqrt(D)                                  # [n, D]
            s = a.sum(axis=1)
            w = np.exp(s - s.max())
            w /= w.sum()
            o = w @ V_
            delta = ((2 * U + U * U) * np.abs(a).sum(axis=1)
                     + 2.0 ** -19 * (rk[:p + 1, kv] @ rq[h]) / np.sqrt(D)).max()
            fac = np.exp(2 * delta) * (1 + U) ** 2 * (1 + g) ** 2 / (1 - g) - 1
            bound[n, h * D:(h + 1) * D] = fac * (w @ np.abs(V_))
            dv = V_ - o                                                    # [n, D]
            C = (K_ * w[:, None]).T @ dv                                   # [i, d]
            var[n, h * D:(h + 1) * D] = (U * U / 3) * (
                (w ** 2 * (a ** 2).sum(axis=1)) @ (dv ** 2)
                + ((qr[h] / np.sqrt(D)) ** 2) @ (C ** 2)
                + 2 * (w ** 2) @ (V_ ** 2))
    return bound, var


def _assert_attn_prefill(got, ref, q, k, v, base, H, KVH, rows, what):
    bound, var = _attn_prefill_bounds(q, k, v, base, H, KVH, rows)
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the worst-case bound, max err {err.max():.3e}"
    if err.size >= 1024:
        z2 = float((err ** 2 / np.maximum(var, 1e-300)).mean())
        assert z2 < 2.0, f"{what}: mean z^2 {z2:.3f} above the rounding model"


def _prefill_check(seed, M, H, KVH, rows=None, S=None, base=500000.0):
    from gpu_helpers import guarded
    bl = _bl()
    S = S or M
    rng = np.random.default_rng(seed)
    qkv = rng.standard_normal((M, (H + 2 * KVH) * 128)).astype(np.float32)
    q, k, v = qkv[:, :H * 128], qkv[:, H * 128:(H + KVH) * 128], qkv[:, (H + KVH) * 128:]
    d_qkv = to_dev(qkv)
    rc, rs = bl.rope_table(S, 128, base, device=dev())
    kc = torch.full((KVH, S, 128), 7.0, dtype=torch.float32, device=dev())
    vc = torch.full((KVH, S, 128), 7.0, dtype=torch.float32, device=dev())
    out = guarded((M, H * 128))
    bl.attn_prefill(d_qkv[:, :H * 128], d_qkv[:, H * 128:(H + KVH) * 128], d_qkv[:, (H + KVH) * 128:],
                    kc, vc, rc, rs, H, KVH, out=out.t)
    out.check("attention output")
    rows = list(range(M)) if rows is None else rows
    ref = oracle.attn_prefill_rows(q, k, v, base, H, KVH, rows)
    got = host(out.t)[rows].astype(np.float64)
    _assert_attn_prefill(got, ref, q, k, v, base, H, KVH, rows, f"M={M} H={H} KVH={KVH}")
    # caches: rotated fp32 keys and the values at positions < M, nothing else
    kch, vch = host(kc), host(vc)
    for p in sorted(set([0, M - 1] + [r for r in rows if r < M])):
        kr = oracle.rope(k[p].reshape(KVH, 128), p, base)
        assert np.abs(kch[:, p] - kr).max() <= 1e-6 * max(1.0, np.abs(kr).max()), p
        assert np.array_equal(vch[:, p], v[p].reshape(KVH, 128)), p
    assert np.all(kch[:, M:] == 7.0) and np.all(vch[:, M:] == 7.0)


@pytest.mark.parametrize("M,H,KVH", [(1, 4, 1), (5, 4, 1), (64, 8, 2), (70, 8, 2), (127, 2, 2), (128, 4, 1),
                                     (129, 4, 1), (130, 4, 4), (200, 20, 5), (257, 6, 3)])
def test_attn_prefill_small(M, H, KVH):
    _prefill_check(60 + M, M, H, KVH, S=M + 17)


@pytest.mark.timeout(600)
def test_attn_prefill_model_shape_sampled_rows():
    # 4096 tokens, 20 query / 5 key-value heads: one row in every 128-query
    # tile (at a different offset in each) and the block edges; the whole
    # output is guarded against unwritten elements
    rows = sorted(set([0, 1, 63, 64, 65, 2047, 2048, 4094, 4095] + [128 * t + (37 * t) % 128 for t in range(32)]))
    _prefill_check(61, 4096, 20, 5, rows=rows)


def test_attn_prefill_then_decode():
    """The caches a prefill writes carry on into decode steps: the token at
    position M against the oracle's decode over its own fp32 rotations."""
    bl = _bl()
    M, H, KVH, S, base = 100, 20, 5, 160, 10000.0
    rng = np.random.default_rng(62)
    qkv = rng.standard_normal((M, (H + 2 * KVH) * 128)).astype(np.float32)
    d_qkv = to_dev(qkv)
    rc, rs = bl.rope_table(S, 128, base, device=dev())
    kc = torch.zeros((KVH, S, 128), dtype=torch.float32, device=dev())
    vc = torch.zeros_like(kc)
    bl.attn_prefill(d_qkv[:, :H * 128], d_qkv[:, H * 128:(H + KVH) * 128], d_qkv[:, (H + KVH) * 128:],
                    kc, vc, rc, rs, H, KVH)
    kc_ref = np.zeros((KVH, S, 128), np.float32)
    vc_ref = np.zeros((KVH, S, 128), np.float32)
    for p in range(M):
        kc_ref[:, p] = oracle.rope(qkv[p, H * 128:(H + KVH) * 128].reshape(KVH, 128), p, base).astype(np.float32)
        vc_ref[:, p] = qkv[p, (H + KVH) * 128:].reshape(KVH, 128)
    for pos in (M, M + 1):
        qn = rng.standard_normal(H * 128).astype(np.float32)
        kn = rng.standard_normal(KVH * 128).astype(np.float32)
        vn = rng.standard_normal(KVH * 128).astype(np.float32)
        o = host(bl.attn_decode(to_dev(qn), to_dev(kn), to_dev(vn), pos, kc, vc, rc, rs, H, KVH)).reshape(H, 128)
        r = oracle.attn_decode(qn, kn, vn, pos, kc_ref, vc_ref, base, H, KVH)
        assert np.abs(o - r).max() <= ATTN_TOL * max(1.0, np.abs(r).max()), pos
        kc_ref[:, pos] = oracle.rope(kn.reshape(KVH, 128), pos, base).astype(np.float32)
        vc_ref[:, pos] = vn.reshape(KVH, 128)


@pytest.mark.timeout(600)
def test_prefill_layer_with_attention_stagewise():
    """stack.prefill_layer_attn over 2 layers of a 130-token prompt, each stage
    against the oracle on the GPU's own input to it; then one decode step
    continues from the caches the prefill wrote."""
    from bit_ternary_weight_amd import stack, synth
    from gpu_helpers import F32_TOL, assert_exact, assert_rows_close, bf16_dev, f32_of_bf16, max_ulp_diff
    H, KV, M, L = synth.HIDDEN, synth.KV_DIM, 130, 2
    layers = stack.build_layers(L, dev())
    cache = stack.alloc_kv(L, 256, dev())
    bits = synth.act_normal_bf16(70, M, H)
    x, x_host = bf16_dev(bits), f32_of_bf16(bits)
    rows = [0, 1, 63, 64, 129]
    for l, lw in enumerate(layers):
        codes, wms = {}, {}
        for p, _, _ in synth.PROJECTIONS:
            _, wm, c = oracle.ternarize_pack(synth.layer_weight(l, p))
            codes[p], wms[p] = c, wm
        dbg = {}
        y = stack.prefill_layer_attn(x, lw, cache, l, debug=dbg)
        qkv_codes = np.concatenate([codes["q"], codes["k"], codes["v"]])
        wq = np.array([wms["q"], wms["k"], wms["v"]], np.float32)
        _, _, _, r_qkv = oracle.bitlinear(x_host[rows], qkv_codes, [H, KV, KV], wq)
        g_qkv = host(dbg["y_qkv"])
        assert_rows_close(g_qkv[rows], r_qkv, F32_TOL, f"qkv {l}")
        assert max_ulp_diff(g_qkv[rows], r_qkv) == 0
        g_att = host(dbg["att"])
        r_att = oracle.attn_prefill_rows(g_qkv[:, :H], g_qkv[:, H:H + KV], g_qkv[:, H + KV:], stack.ROPE_BASE,
                                         20, 5, rows)
        _assert_attn_prefill(g_att[rows].astype(np.float64), r_att, g_qkv[:, :H], g_qkv[:, H:H + KV],
                             g_qkv[:, H + KV:], stack.ROPE_BASE, 20, 5, rows, f"layer {l} attention")
        rq, ra = oracle.quant_act(oracle.rmsnorm(g_att[rows], None, 1e-5))
        assert_exact(host(dbg["q_o"])[rows], rq, f"attn_sub_norm codes {l}")
        assert_exact(host(dbg["a_o"])[rows], ra, f"attn_sub_norm scales {l}")
        r_o = oracle.rescale(oracle.contract(rq, codes["o"]), ra, None, wms["o"])
        assert_exact(host(dbg["y_o"])[rows].view(np.uint32), r_o.view(np.uint32), f"o {l}")
        gu = np.concatenate([codes["gate"], codes["up"]])
        ch = oracle.ffn_chain(r_o, gu, np.array([wms["gate"], wms["up"]], np.float32), codes["down"], wms["down"])
        yh = host(y)
        assert_rows_close(yh[rows], ch["y"], F32_TOL, f"layer {l}")
        x, x_host = y.clone(), yh
    # a decode step at position M reads the caches the prefill wrote
    dbg = {}
    stack.decode_layer_attn(x[-1:].contiguous(), layers[0], cache, 0, M, debug=dbg)
    assert np.isfinite(host(dbg["att"])).all()
