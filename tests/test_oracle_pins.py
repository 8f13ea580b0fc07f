"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked examples (tests/golden), closed forms, exact rational arithmetic,
invariants and brute force on tiny inputs.  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_ternary_weight_amd import synth

F32_EPS_SCALE = float(np.float32(1e-5))


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _ulp(v: float) -> float:
    return float(np.spacing(np.float32(abs(v)))) if v != 0 else float(np.float32(1.4e-45))


# ----------------------------------------------------------------------------- worked examples
def test_a1_worked_example_end_to_end(golden_dir):
    g = _golden(golden_dir, "a1_worked_example.json")
    W = np.array(g["W"], np.float32)
    wm = oracle.weight_mean(W)
    assert wm == np.float32(g["w_mean"])
    codes = oracle.ternarize(W, wm)
    assert codes.tolist() == g["codes"]
    packed = oracle.pack(codes)
    assert packed.tolist() == g["packed"]
    x = np.array(g["x"], np.float32)
    q, a = oracle.quant_act(x)
    assert q.tolist() == g["q"]
    assert a.tolist() == g["a"]
    A = oracle.contract(q, codes)
    assert A.tolist() == g["A"]
    y = oracle.rescale(A, a, None, wm)
    for m in range(4):
        for n in range(4):
            num, den = g["y_rational"][m][n]
            exact = Fraction(num, den)
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(_ulp(float(exact)))
    # rows 0 and 2 are exact in fp32
    assert y[0].tolist() == [32.25, -16.0, -48.25, 16.5]
    assert y[2].tolist() == [0.0, 0.0, 0.0, 0.0]
    # composite entry point agrees with the stage functions
    q2, a2, A2, y2 = oracle.bitlinear(x, codes, None, wm)
    assert (q2 == q).all() and (a2 == a).all() and (A2 == A).all() and (y2 == y).all()


def test_a2_plane_order(golden_dir):
    g = _golden(golden_dir, "a2_plane_order.json")
    codes = np.array(g["codes"], np.int8).reshape(8, 1)
    packed = oracle.pack(codes)
    assert packed.ravel().tolist() == g["packed_plane_order"]
    back, bad = oracle.unpack(packed)
    assert bad == 0 and back.ravel().tolist() == g["codes"]


# ----------------------------------------------------------------------------- packing
def test_pack_unpack_exhaustive_81():
    combos = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).astype(np.int8)
    assert combos.shape == (4, 81)
    packed = oracle.pack(combos)                      # N=4 -> one packed row, K=81
    assert packed.shape == (1, 81)
    assert len(set(packed.ravel().tolist())) == 81     # injective
    for b in packed.ravel().tolist():                  # never uses the field value 3
        assert all(((b >> (2 * i)) & 3) != 3 for i in range(4))
    back, bad = oracle.unpack(packed)
    assert bad == 0 and (back == combos).all()
    # field i of the byte is code row i (+1): value of the byte is base-4 number
    for k in range(81):
        digits = [int(combos[i, k]) + 1 for i in range(4)]
        assert int(packed[0, k]) == sum(d * 4 ** i for i, d in enumerate(digits))


def test_unpack_reports_value_3():
    _, bad = oracle.unpack(np.array([[0xFF, 0x03]], np.uint8))
    assert bad == 5


def test_pack_plane_order_larger():
    # N=12: packed row r field i must hold weight row i*3 + r
    rng = np.random.default_rng(5)
    codes = rng.integers(-1, 2, size=(12, 7)).astype(np.int8)
    packed = oracle.pack(codes)
    for r in range(3):
        for k in range(7):
            for i in range(4):
                assert ((int(packed[r, k]) >> (2 * i)) & 3) - 1 == codes[i * 3 + r, k]


# ----------------------------------------------------------------------------- weight scale / codes
def test_weight_stats_closed_form():
    """N(0, s^2) masters: E|W| = s*sqrt(2/pi); P(code 0) = erf(1/(2 sqrt(pi)))."""
    W = synth.master_weight(1000, 2560, 2560)
    wm = float(oracle.weight_mean(W))
    s = synth.WEIGHT_STD
    expect = s * math.sqrt(2 / math.pi)
    n = W.size
    se_mean = s * math.sqrt(1 - 2 / math.pi) / math.sqrt(n)
    assert abs(wm - expect) < 5 * se_mean
    codes = oracle.ternarize(W, wm)
    p0 = math.erf(1 / (2 * math.sqrt(math.pi)))
    assert abs(p0 - 0.310064) < 1e-6
    frac0 = float((codes == 0).mean())
    se = math.sqrt(p0 * (1 - p0) / n)
    assert abs(frac0 - p0) < 6 * se + 2e-4   # + effect of the sample mean on the threshold
    pp = (1 - p0) / 2
    assert abs(float((codes == 1).mean()) - pp) < 6 * se + 2e-4
    assert abs(float((codes == -1).mean()) - pp) < 6 * se + 2e-4
    assert set(np.unique(codes).tolist()) <= {-1, 0, 1}


def test_weight_mean_exact_small():
    W = np.array([[1.0, -2.0], [0.5, -0.25]], np.float32)
    assert oracle.weight_mean(W) == np.float32(3.75 / 4)


def test_zero_weight_floor():
    W = np.zeros((8, 16), np.float32)
    wm = oracle.weight_mean(W)
    assert wm == np.float32(1e-5)
    assert (oracle.ternarize(W, wm) == 0).all()


def test_const_weight_sign():
    for c in (0.3, -0.7, 1e-3):
        W = np.full((4, 6), c, np.float32)
        codes = oracle.ternarize(W, oracle.weight_mean(W))
        assert (codes == np.sign(c)).all()


def test_identity_weight_codes():
    N = 256
    W = np.eye(N, dtype=np.float32)
    wm = oracle.weight_mean(W)
    assert wm == np.float32(1.0 / N)
    assert (oracle.ternarize(W, wm) == np.eye(N, dtype=np.int8)).all()


def test_ternarize_matches_exact_rounding_near_half():
    """rne(fl32(w/m)) == 0 exactly when the exact quotient |w|/m <= 1/2 + 2^-25.

    Tests fp32 division followed by half-even rounding against exact rational
    arithmetic, on values a few ulps around the half-way point."""
    rng = np.random.default_rng(7)
    means = rng.uniform(1e-3, 1.0, size=64).astype(np.float32)
    thr = Fraction(1, 2) + Fraction(1, 2 ** 25)
    checked = 0
    for m in means:
        half = np.float32(m) * np.float32(0.5)
        vals = [half]
        up = dn = half
        for _ in range(6):
            up = np.nextafter(up, np.float32(1e9))
            dn = np.nextafter(dn, np.float32(0))
            vals += [up, dn]
        W = np.array(vals + [-v for v in vals], np.float32)
        codes = oracle.ternarize(W, m)
        for w, c in zip(W.tolist(), codes.tolist()):
            q = abs(Fraction(w)) / Fraction(float(m))
            expect = 0 if q <= thr else int(math.copysign(1, w))
            assert c == expect, (w, float(m), c)
            checked += 1
    assert checked > 1000


def test_ternarize_ties_half_even():
    W = np.array([0.5, -0.5, 1.5, -1.5, 2.5, 0.49999997], np.float32)
    assert oracle.ternarize(W, np.float32(1.0)).tolist() == [0, 0, 1, -1, 1, 0]


# ----------------------------------------------------------------------------- activation quantization
def test_quant_act_scale_is_correctly_rounded_division():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 33)) * rng.uniform(1e-3, 1e3, size=(64, 1))).astype(np.float32)
    q, a = oracle.quant_act(x)
    for m in range(64):
        amax = max(Fraction(abs(float(v))) for v in x[m])
        amax = max(amax, Fraction(F32_EPS_SCALE))
        exact = Fraction(127) / amax
        assert abs(Fraction(float(a[m])) - exact) <= Fraction(_ulp(float(a[m]))) / 2


def test_quant_act_codes_exact_rounding():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((16, 40)).astype(np.float32)
    q, a = oracle.quant_act(x)
    for m in range(16):
        for k in range(40):
            prod = np.float32(x[m, k]) * np.float32(a[m])   # one fp32 rounding
            t = Fraction(float(prod))
            fl = math.floor(t)
            d = t - fl
            r = fl + 1 if d > Fraction(1, 2) else (fl if d < Fraction(1, 2) else (fl if fl % 2 == 0 else fl + 1))
            assert q[m, k] == max(-128, min(127, r))


def test_quant_act_invariants():
    x = synth.bf16_to_f32(synth.act_heavy_tail_bf16(0, 64, 2560))
    q, a = oracle.quant_act(x)
    assert q.min() >= -127 and q.max() <= 127                       # I2
    am = np.abs(x).argmax(axis=1)
    assert (np.abs(q[np.arange(64), am]) == 127).all()               # I3
    # I6: scaling a row by a power of two keeps q and scales a exactly
    for e in (-7, 3, 20):
        q2, a2 = oracle.quant_act(x * np.float32(2.0 ** e))
        assert (q2 == q).all()
        assert (a2 == a * np.float32(2.0 ** -e)).all()
    # I7: permuting rows permutes outputs
    perm = np.random.default_rng(3).permutation(64)
    q3, a3 = oracle.quant_act(x[perm])
    assert (q3 == q[perm]).all() and (a3 == a[perm]).all()


def test_quant_act_zero_and_tiny_rows():
    x = np.zeros((3, 8), np.float32)
    x[1, 2] = 1e-7          # below the 1e-5 floor
    x[2, 5] = -1e-45        # denormal
    q, a = oracle.quant_act(x)
    assert (a == np.float32(127.0) / np.float32(1e-5)).all()
    assert a[0] == np.float32(12700000.0)
    assert (q[0] == 0).all()
    assert q[1, 2] == 1     # 1e-7 * 1.27e7 = 1.27 -> 1
    assert (q[2] == 0).all()


def test_quant_act_per_token_not_per_channel():
    x = np.array([[1.0, 100.0], [100.0, 1.0]], np.float32)
    q, a = oracle.quant_act(x)
    assert a.tolist() == [1.27, 1.27] or np.allclose(a, 1.27)
    assert q.tolist() == [[1, 127], [127, 1]]


# ----------------------------------------------------------------------------- contraction
def test_contract_brute_force_python_ints():
    rng = np.random.default_rng(21)
    M, K, N = 3, 5, 8
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    c = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    A = oracle.contract(q, c)
    for m in range(M):
        for n in range(N):
            assert A[m, n] == sum(int(q[m, k]) * int(c[n, k]) for k in range(K))


def test_contract_extremes_and_identity():
    K = 6912
    q = np.full((2, K), 127, np.int8)
    q[1] = -127
    c = np.ones((4, K), np.int8)
    c[1] = -1
    A = oracle.contract(q, c)
    assert A.tolist() == [[127 * K, -127 * K, 127 * K, 127 * K], [-127 * K, 127 * K, -127 * K, -127 * K]]
    # identity weights: A == q (pins which index of the weight is the output)
    rng = np.random.default_rng(2)
    q = rng.integers(-127, 128, size=(4, 256)).astype(np.int8)
    A = oracle.contract(q, np.eye(256, dtype=np.int8))
    assert (A == q.astype(np.int32)).all()


# ----------------------------------------------------------------------------- rescale
def _rne32(fr: Fraction) -> float:
    """Exact rational -> nearest fp32 (ties to even), by exact comparison with
    the two fp32 neighbours; independent of any floating-point evaluation."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    fr = abs(fr)
    lo = np.float32(float(fr))                      # within an ulp of fr
    while Fraction(float(lo)) > fr:
        lo = np.nextafter(lo, np.float32(0))
    while Fraction(float(np.nextafter(lo, np.float32(np.inf)))) <= fr:
        lo = np.nextafter(lo, np.float32(np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dl, dh = fr - Fraction(float(lo)), Fraction(float(hi)) - fr
    if dl < dh or (dl == dh and (int(np.array(lo).view(np.uint32)) & 1) == 0):
        return sign * float(lo)
    return sign * float(hi)


def test_rescale_against_exact_rationals_segments():
    """y = fl32(float(A) * fl32(w_mean / a)): the scale is the correctly rounded
    quotient, then one rounding of the product (exact rationals, no float
    evaluation of the formula)."""
    rng = np.random.default_rng(31)
    M, segs = 5, [8, 4, 12]
    N = sum(segs)
    A = rng.integers(-877824, 877825, size=(M, N)).astype(np.int32)
    a = rng.uniform(0.5, 300, size=M).astype(np.float32)
    wm = rng.uniform(0.01, 0.03, size=3).astype(np.float32)
    y = oracle.rescale(A, a, segs, wm)
    seg_of = np.repeat(np.arange(3), segs)
    for m in range(M):
        for n in range(N):
            sc = _rne32(Fraction(float(wm[seg_of[n]])) / Fraction(float(a[m])))
            assert float(y[m, n]) == _rne32(Fraction(int(A[m, n])) * Fraction(sc)), (m, n)


def test_rescale_divides_once_not_by_reciprocal():
    """A pair (w_mean, a) for which fl(w_mean / a) and w_mean * fl(1 / a) are
    different fp32 numbers: with A = 1 the output is the scale itself and must
    be the correctly rounded quotient."""
    rng = np.random.default_rng(77)
    found = 0
    for _ in range(20000):
        w = np.float32(rng.uniform(0.01, 0.03))
        a = np.float32(rng.uniform(1.0, 300.0))
        quot = _rne32(Fraction(float(w)) / Fraction(float(a)))
        recip = _rne32(Fraction(float(w)) * Fraction(_rne32(1 / Fraction(float(a)))))
        if quot != recip:
            y = oracle.rescale(np.ones((1, 4), np.int32), np.array([a]), None, np.float32(w))
            assert (y == np.float32(quot)).all() and (y != np.float32(recip)).all()
            found += 1
            if found == 5:
                break
    assert found == 5


def test_rescale_vs_dequant_f64():
    W = synth.master_weight(5, 64, 96)
    packed, wm, codes = oracle.ternarize_pack(W)
    x = synth.act_normal_f32(5, 6, 96)
    q, a, A, y = oracle.bitlinear(x, codes, None, wm)
    yd = oracle.dequant_f64(q, a, codes, None, wm)
    scale = np.abs(yd).max(axis=1, keepdims=True)
    assert (np.abs(y - yd) <= 1e-6 * scale).all()


def test_to_bf16_closed_forms():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 0.0], np.float32)
    assert oracle.to_bf16(vals).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000]


# ----------------------------------------------------------------------------- RMSNorm / ReLU^2
def test_rmsnorm_closed_forms():
    eps = float(np.float32(1e-5))
    K = 64
    for c in (0.5, -3.0, 1e-3):
        h = np.full((1, K), c, np.float32)
        out = oracle.rmsnorm(h)
        expect = c / math.sqrt(c * c + eps)
        assert abs(float(out[0, 0]) - expect) <= 2 * _ulp(expect)
    h = np.zeros((1, K), np.float32)
    h[0, 3] = 2.0
    out = oracle.rmsnorm(h)
    expect = 2.0 / math.sqrt(4.0 / K + eps)
    assert abs(float(out[0, 3]) - expect) <= 2 * _ulp(expect)
    assert (out[0, :3] == 0).all() and (out[0, 4:] == 0).all()
    # scale invariance (eps negligible at this norm)
    rng = np.random.default_rng(8)
    h = rng.standard_normal((4, 100)).astype(np.float32) * 10
    o1 = oracle.rmsnorm(h)
    o2 = oracle.rmsnorm(h * np.float32(8.0))
    assert np.allclose(o1, o2, rtol=2e-6, atol=0)
    # gain multiplies elementwise
    g = rng.uniform(0.5, 2, size=100).astype(np.float32)
    og = oracle.rmsnorm(h, g)
    assert np.allclose(og, o1 * g, rtol=1e-6, atol=0)
    # zero row stays zero
    assert (oracle.rmsnorm(np.zeros((1, 16), np.float32)) == 0).all()


def test_rmsnorm_sum_of_squares_is_exact_fp64():
    """A row of one 4096 followed by 4096 ones: sum h^2 = 4096^2 + 4096 =
    4096 * 4097 exactly, so the mean square over K = 4097 is exactly 4096.
    Summed in fp32 the ones vanish (2^24 + 1 is not representable), which
    would give a mean of 2^24 / 4097 instead.  r = fl32(1 / sqrt(4096 + eps))
    to within rounding of the exact value."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    K = 4097
    h = np.ones((1, K), np.float32)
    h[0, 0] = 4096.0
    out = oracle.rmsnorm(h)
    eps = Decimal(float(np.float32(1e-5)))
    r_exact = Decimal(1) / (Decimal(4096) + eps).sqrt()
    r = Fraction(float(out[0, 1]))                  # h = 1 there: out = fl32(r)
    # one fp32 rounding of a value computed in fp64: within 0.5 ulp + 1e-15
    assert abs(r - Fraction(r_exact)) <= Fraction(_ulp(float(r_exact))) / 2 + Fraction(1, 10 ** 15)
    assert float(out[0, 0]) == float(np.float32(np.float32(4096.0) * np.float32(out[0, 1])))
    # the fp32 sum's answer is far outside that
    r_f32sum = 1 / math.sqrt(2.0 ** 24 / K + 1e-5)
    assert abs(float(r) - r_f32sum) > 1000 * _ulp(r_f32sum)


def test_relu2_mul_closed_forms():
    g = np.array([-1.0, 2.0, 0.5, -0.0, 3.0], np.float32)
    u = np.array([5.0, 3.0, -4.0, 7.0, 0.0], np.float32)
    assert oracle.relu2_mul(g, u).tolist() == [0.0, 12.0, -1.0, 0.0, 0.0]


# ----------------------------------------------------------------------------- FFN chain wiring
def _chain_weights(H, I, gate_sign=1):
    cg = gate_sign * np.eye(I, H, dtype=np.int8)
    cu = np.eye(I, H, dtype=np.int8)
    cd = np.eye(H, I, dtype=np.int8)
    return np.concatenate([cg, cu]), cd


def test_ffn_chain_identity_weights_closed_form():
    """h = ones, identity gate/up/down: y = w_down * 127/a2 * ... ~= w_down."""
    H = I = 8
    cgu, cd = _chain_weights(H, I)
    h = np.ones((1, H), np.float32)
    wgu = np.array([0.25, 0.5], np.float32)
    wd = np.float32(0.125)
    out = oracle.ffn_chain(h, cgu, wgu, cd, wd)
    assert (out["q1"] == 127).all()
    assert (out["q2"] == 127).all()
    # closed form: the normalized input is r1 = 1/sqrt(1+eps) everywhere, so
    # q1 = 127, a1 = 127/r1 and each branch gives w*r1; p = (wg*r1)^2*(wu*r1)
    # is constant, normalizes to p/sqrt(p^2+eps), and y = wd * that.
    eps = float(np.float32(1e-5))
    r1 = 1 / math.sqrt(1 + eps)
    p = (0.25 * r1) ** 2 * (0.5 * r1)
    assert np.allclose(out["p"], p, rtol=1e-6, atol=0)
    assert np.allclose(out["y"], 0.125 * p / math.sqrt(p * p + eps), rtol=1e-6, atol=0)


def test_ffn_chain_negative_gate_is_zero():
    """gate outputs all <= 0 -> ReLU kills them -> y == 0 exactly.  Swapping
    the roles of gate and up would give a non-zero result here."""
    H = I = 8
    cgu, cd = _chain_weights(H, I, gate_sign=-1)
    h = np.ones((2, H), np.float32)
    out = oracle.ffn_chain(h, cgu, np.array([0.25, 0.5], np.float32), cd, np.float32(0.1))
    assert (out["p"] == 0).all() and (out["q2"] == 0).all() and (out["y"] == 0).all()
    # swapped roles would not vanish
    cgu_sw = np.concatenate([cgu[I:], cgu[:I]])
    out2 = oracle.ffn_chain(h, cgu_sw, np.array([0.5, 0.25], np.float32), cd, np.float32(0.1))
    assert (out2["y"] != 0).any()


def test_ffn_chain_random_stagewise_consistency():
    rng = np.random.default_rng(44)
    H, I, M = 32, 48, 3
    Wg = synth.master_weight(1, I, H)
    Wu = synth.master_weight(2, I, H)
    Wd = synth.master_weight(3, H, I)
    _, wg, cg = oracle.ternarize_pack(Wg)
    _, wu, cu = oracle.ternarize_pack(Wu)
    _, wd, cd = oracle.ternarize_pack(Wd)
    h = rng.standard_normal((M, H)).astype(np.float32)
    out = oracle.ffn_chain(h, np.concatenate([cg, cu]), np.array([wg, wu]), cd, wd)
    hn = oracle.rmsnorm(h)
    q1, a1, _, ygu = oracle.bitlinear(hn, np.concatenate([cg, cu]), [I, I], [wg, wu])
    assert (q1 == out["q1"]).all() and (a1 == out["a1"]).all()
    p = oracle.relu2_mul(ygu[:, :I], ygu[:, I:])
    assert (p == out["p"]).all()
    q2, a2, _, y = oracle.bitlinear(oracle.rmsnorm(p), cd, None, wd)
    assert (q2 == out["q2"]).all() and (a2 == out["a2"]).all() and (y == out["y"]).all()


# ----------------------------------------------------------------------------- attention (decode)
def _attn_inputs(seed, H, KVH, D, S):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(H * D).astype(np.float32)
    kn = rng.standard_normal(KVH * D).astype(np.float32)
    vn = rng.standard_normal(KVH * D).astype(np.float32)
    kc = rng.standard_normal((KVH, S, D)).astype(np.float32)
    vc = rng.standard_normal((KVH, S, D)).astype(np.float32)
    return q, kn, vn, kc, vc


def test_rope_position_zero_is_identity_and_d2_is_a_plane_rotation():
    x = np.random.default_rng(1).standard_normal((3, 16))
    assert np.array_equal(oracle.rope(x, 0, 10000.0), x)
    # D = 2: one pair rotated by exactly pos radians (base^0 = 1)
    v = np.array([[0.6, -0.8]])
    for pos in (1, 5, 77):
        c, s = math.cos(pos), math.sin(pos)
        assert np.allclose(oracle.rope(v, pos, 500000.0), [[0.6 * c + 0.8 * s, -0.8 * c + 0.6 * s]], atol=1e-15)


def test_rope_angle_schedule_closed_form():
    """D = 8, base = 100, position 1: the four pairs turn by 100^(-2i/8) =
    1, 10^-0.5, 0.1, 10^-1.5 radians.  Unit vectors e_i and e_(i+4) give the
    cosines and sines of exactly those angles."""
    D, base = 8, 100.0
    angles = [1.0, 10 ** -0.5, 0.1, 10 ** -1.5]
    eye = np.eye(D)
    r = oracle.rope(eye, 1, base)
    for i, t in enumerate(angles):
        # e_i -> cos t at i, sin t at i + 4;  e_(i+4) -> -sin t at i, cos t at i + 4
        assert abs(r[i, i] - math.cos(t)) < 1e-15 and abs(r[i, i + 4] - math.sin(t)) < 1e-15
        assert abs(r[i + 4, i] + math.sin(t)) < 1e-15 and abs(r[i + 4, i + 4] - math.cos(t)) < 1e-15
    # position 3: three times the angles
    r3 = oracle.rope(eye, 3, base)
    for i, t in enumerate(angles):
        assert abs(r3[i, i + 4] - math.sin(3 * t)) < 1e-14


def test_rope_invariants():
    rng = np.random.default_rng(2)
    D = 128
    x = rng.standard_normal((4, D))
    y = rng.standard_normal((4, D))
    for base in (10000.0, 500000.0):
        r = oracle.rope(x, 37, base)
        # each (i, i + D/2) pair keeps its length
        assert np.allclose(r[:, :D // 2] ** 2 + r[:, D // 2:] ** 2, x[:, :D // 2] ** 2 + x[:, D // 2:] ** 2, rtol=1e-12)
        # angles add
        assert np.allclose(oracle.rope(oracle.rope(x, 11, base), 26, base), r, atol=1e-12)
        # the dot product of a rotated query and key depends on their distance only
        d1 = np.sum(oracle.rope(x, 40, base) * oracle.rope(y, 13, base), axis=1)
        d2 = np.sum(oracle.rope(x, 1040, base) * oracle.rope(y, 1013, base), axis=1)
        assert np.allclose(d1, d2, rtol=1e-9, atol=1e-9)


def test_attn_single_position_returns_the_value():
    H, KVH, D = 8, 2, 16
    q, kn, vn, kc, vc = _attn_inputs(3, H, KVH, D, 4)
    out = oracle.attn_decode(q, kn, vn, 0, kc, vc, 10000.0, H, KVH)
    for h in range(H):
        assert np.allclose(out[h], vn.reshape(KVH, D)[h // (H // KVH)], rtol=1e-14)


def test_attn_equal_keys_average_the_values():
    H, KVH, D, pos = 4, 1, 8, 5
    q, kn, vn, kc, vc = _attn_inputs(4, H, KVH, D, 8)
    # every cached key equal to the new token's rotated key: uniform weights
    kr = oracle.rope(kn.reshape(KVH, D).astype(np.float64), pos, 10000.0)
    kc[:, :pos, :] = kr.astype(np.float32)[:, None, :]
    out = oracle.attn_decode(q, kn, vn, pos, kc, vc, 10000.0, H, KVH)
    mean_v = (vc[0, :pos].astype(np.float64).sum(0) + vn.astype(np.float64)) / (pos + 1)
    # the cached keys are the new key's fp32 rounding (<= 1 ulp apart): the
    # weights are equal to ~1e-6
    assert np.allclose(out, mean_v[None, :], rtol=0, atol=1e-5 * np.abs(mean_v).max())


def test_attn_scale_and_softmax_closed_form():
    # one cached key of zeros (score 0) and the new key with q.k = sqrt(D) ln 3
    # (RoPE rotates q and the new key by the same angle: their dot product is
    # unchanged): weights 1/4, 3/4
    H, KVH, D, pos = 1, 1, 16, 1
    q = np.zeros(D, np.float32)
    q[0] = 1.0
    kn = np.zeros(D, np.float32)
    kn[0] = np.float32(math.sqrt(D) * math.log(3.0))
    vn = np.random.default_rng(5).standard_normal(D).astype(np.float32)
    kc = np.zeros((1, 4, D), np.float32)
    vc = np.random.default_rng(6).standard_normal((1, 4, D)).astype(np.float32)
    out = oracle.attn_decode(q, kn, vn, pos, kc, vc, 10000.0, H, KVH)
    w1 = math.exp(float(kn[0]) / math.sqrt(D))      # exp(score of the new key), ~3
    exp = (vc[0, 0].astype(np.float64) + w1 * vn.astype(np.float64)) / (1.0 + w1)
    assert abs(w1 - 3.0) < 1e-6
    assert np.allclose(out[0], exp, rtol=1e-12, atol=1e-12)


def test_attn_grouped_query_equals_repeated_heads():
    # GQA with H / KVH query heads per key/value head equals multi-head
    # attention with each key/value head repeated for its group
    H, KVH, D, S, pos = 8, 2, 16, 12, 9
    q, kn, vn, kc, vc = _attn_inputs(7, H, KVH, D, S)
    G = H // KVH
    gqa = oracle.attn_decode(q, kn, vn, pos, kc, vc, 10000.0, H, KVH)
    rep = lambda a: np.repeat(a, G, axis=0)
    mha = oracle.attn_decode(q, rep(kn.reshape(KVH, D)).reshape(-1), rep(vn.reshape(KVH, D)).reshape(-1), pos,
                             rep(kc), rep(vc), 10000.0, H, H)
    assert np.array_equal(gqa, mha)
    # and per head it is the textbook softmax attention (numpy, fp64)
    qr = oracle.rope(q.reshape(H, D), pos, 10000.0)
    kr = oracle.rope(kn.reshape(KVH, D), pos, 10000.0)
    for h in range(H):
        g = h // G
        keys = np.concatenate([kc[g, :pos].astype(np.float64), kr[g:g + 1]], axis=0)
        vals = np.concatenate([vc[g, :pos].astype(np.float64), vn.reshape(KVH, D)[g:g + 1].astype(np.float64)], axis=0)
        s = keys @ qr[h] / math.sqrt(D)
        p = np.exp(s - s.max())
        assert np.allclose(gqa[h], p @ vals / p.sum(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- prefill attention
def _prefill_inputs(seed, M, H, KVH, D=128):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, H * D)).astype(np.float32),
            rng.standard_normal((M, KVH * D)).astype(np.float32),
            rng.standard_normal((M, KVH * D)).astype(np.float32))


def test_attn_prefill_rows_match_the_decode_oracle():
    """Row p of the prompt against one decode step at position p over a cache
    of the earlier tokens' rotated keys: two separate writings of the same
    attention.  The decode cache holds fp32 keys (rounded once), the prefill
    definition none, hence the 1e-6."""
    M, H, KVH, D, base = 40, 8, 2, 128, 10000.0
    q, k, v = _prefill_inputs(21, M, H, KVH)
    rows = [0, 1, 17, 39]
    got = oracle.attn_prefill_rows(q, k, v, base, H, KVH, rows)
    kc = np.zeros((KVH, M, D), np.float32)
    vc = np.zeros((KVH, M, D), np.float32)
    for p in range(M):
        kc[:, p] = oracle.rope(k[p].reshape(KVH, D), p, base).astype(np.float32)
        vc[:, p] = v[p].reshape(KVH, D)
    for n, p in enumerate(rows):
        ref = oracle.attn_decode(q[p], k[p], v[p], p, kc, vc, base, H, KVH).reshape(-1)
        assert np.abs(got[n] - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max()), p


def test_attn_prefill_first_row_and_causality():
    M, H, KVH, D = 12, 4, 1, 128
    q, k, v = _prefill_inputs(22, M, H, KVH)
    out = oracle.attn_prefill_rows(q, k, v, 500000.0, H, KVH, [0, 5])
    # position 0 sees only itself: every head returns the value, unrounded
    for h in range(H):
        assert np.array_equal(out[0, h * D:(h + 1) * D], v[0].astype(np.float64))
    # later tokens do not change row 5
    k2, v2 = k.copy(), v.copy()
    k2[6:] += 3.0
    v2[6:] -= 2.0
    assert np.array_equal(oracle.attn_prefill_rows(q, k2, v2, 500000.0, H, KVH, [5]), out[1:2])


def test_attn_prefill_zero_query_averages_the_values():
    """q = 0 gives every score 0, whatever the rotation: token p returns the
    plain mean of the values of positions 0 .. p (its key/value head's)."""
    M, H, KVH, D = 30, 4, 2, 128
    _, k, v = _prefill_inputs(23, M, H, KVH)
    q = np.zeros((M, H * D), np.float32)
    rows = [0, 7, 29]
    out = oracle.attn_prefill_rows(q, k, v, 10000.0, H, KVH, rows)
    vh = v.astype(np.float64).reshape(M, KVH, D)
    for n, p in enumerate(rows):
        for h in range(H):
            mean = vh[:p + 1, h // (H // KVH)].sum(axis=0) / (p + 1)
            assert np.allclose(out[n, h * D:(h + 1) * D], mean, rtol=0, atol=1e-14)


def test_attn_prefill_grouped_query_equals_repeated_heads():
    M, H, KVH, D = 20, 6, 3, 128
    q, k, v = _prefill_inputs(24, M, H, KVH)
    G = H // KVH
    rep = lambda a: np.repeat(a.reshape(M, KVH, D), G, axis=1).reshape(M, H * D)
    rows = [3, 19]
    gqa = oracle.attn_prefill_rows(q, k, v, 10000.0, H, KVH, rows)
    mha = oracle.attn_prefill_rows(q, rep(k), rep(v), 10000.0, H, H, rows)
    assert np.array_equal(gqa, mha)


def test_bf16_round_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5, 3.0e-3], np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5, 0.0030059814453125], np.float32)
    assert np.array_equal(oracle.bf16_round(x), want)


# ----------------------------------------------------------------------------- straight-through backward
def test_ste_grad_input_is_the_gradient_through_the_fake_quantized_weight():
    rng = np.random.default_rng(31)
    W = rng.normal(0, 0.02, size=(12, 20)).astype(np.float32)
    _, wm, codes = oracle.ternarize_pack(W)
    dy = rng.standard_normal((3, 12)).astype(np.float32)
    # against the matmul with the fake-quantized weight itself
    Wq = oracle.fake_quant_weight(codes, wm).astype(np.float64)
    assert np.allclose(oracle.ste_grad_input(dy, codes, wm), dy.astype(np.float64) @ Wq, rtol=1e-12, atol=1e-15)
    # brute force in exact rationals, element by element
    got = oracle.ste_grad_input(dy, codes, wm)
    for m in range(3):
        for k in range(20):
            ref = sum(Fraction(float(dy[m, n])) * int(codes[n, k]) for n in range(12)) * Fraction(float(wm))
            assert abs(Fraction(float(got[m, k])) - ref) <= Fraction(1, 2 ** 48) * (abs(ref) + 1)
    # a row subset gives the same rows
    assert np.array_equal(oracle.ste_grad_input(dy, codes, wm, rows=[2, 0]), got[[2, 0]])


def test_ste_grad_weight_is_dy_transposed_times_fake_quant_activations():
    rng = np.random.default_rng(32)
    # one token: an outer product of dy and x~ = q / a
    x = rng.standard_normal((1, 16)).astype(np.float32)
    q, a = oracle.quant_act(x)
    dy = np.array([[0.5, -1.25, 3.0]], np.float32)
    got = oracle.ste_grad_weight(dy, q, a)
    for n in range(3):
        for k in range(16):
            exact = Fraction(float(dy[0, n])) * Fraction(int(q[0, k])) / Fraction(float(a[0]))
            assert abs(Fraction(float(got[n, k])) - exact) <= Fraction(1, 2 ** 50) * abs(exact)
    # several tokens, brute force in exact rationals: dW[n,k] = sum_m dy[m,n] q[m,k] / a[m]
    xs = rng.standard_normal((7, 5)).astype(np.float32)
    q2, a2 = oracle.quant_act(xs)
    dy2 = rng.standard_normal((7, 4)).astype(np.float32)
    got2 = oracle.ste_grad_weight(dy2, q2, a2)
    assert got2.shape == (4, 5)
    for n in range(4):
        for k in range(5):
            exact = sum(Fraction(float(dy2[m, n])) * int(q2[m, k]) / Fraction(float(a2[m])) for m in range(7))
            assert abs(Fraction(float(got2[n, k])) - exact) <= Fraction(1, 2 ** 48) * (abs(exact) + 1)
    assert np.array_equal(oracle.ste_grad_weight(dy2, q2, a2, rows=[3, 1]), got2[[3, 1]])


# ----------------------------------------------------------------------------- exact contraction by fp64 product
def test_contract_f64_equals_the_integer_loop():
    rng = np.random.default_rng(55)
    for M, K, N in ((3, 7, 8), (17, 300, 12), (64, 2560, 40)):
        q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        c = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        assert np.array_equal(oracle.contract_f64(q, c), oracle.contract(q, c))
    # the extremes: |A| = 127 K and -128 K at K = 6912
    K = 6912
    q = np.full((2, K), 127, np.int8)
    q[1] = -128
    c = np.ones((4, K), np.int8)
    c[1] = -1
    A = oracle.contract_f64(q, c)
    assert A[0, 0] == 127 * K and A[0, 1] == -127 * K and A[1, 0] == -128 * K and A[1, 1] == 128 * K
    # and the whole forward agrees with the C forward bit for bit
    W = synth.master_weight(9, 48, 256)
    _, wm, codes = oracle.ternarize_pack(W)
    x = synth.act_normal_f32(9, 5, 256)
    r1 = oracle.bitlinear(x, codes, None, wm)
    r2 = oracle.bitlinear_f64gemm(x, codes, None, wm)
    for u, w in zip(r1, r2):
        assert np.array_equal(u, w)


def test_chain_and_layer_f64gemm_equal_the_c_composition():
    """The fast compositions (contractions by the exact fp64 product) give the
    C chain's and layer's bits at every stage."""
    Wg, Wu, Wd = synth.master_weight(11, 48, 32), synth.master_weight(12, 48, 32), synth.master_weight(13, 32, 48)
    _, wg, cg = oracle.ternarize_pack(Wg)
    _, wu, cu = oracle.ternarize_pack(Wu)
    _, wd, cd = oracle.ternarize_pack(Wd)
    h = synth.act_normal_f32(14, 5, 32)
    g1 = np.linspace(0.5, 1.5, 32).astype(np.float32)
    a = oracle.ffn_chain(h, np.concatenate([cg, cu]), np.array([wg, wu]), cd, wd, g_subln=g1)
    b = oracle.ffn_chain_f64gemm(h, np.concatenate([cg, cu]), np.array([wg, wu]), cd, wd, g_subln=g1)
    for key in ("q1", "a1", "p", "q2", "a2", "y"):
        assert np.array_equal(a[key], b[key]), key
    codes, wms = {}, {}
    for j, (p, n, k) in enumerate([("q", 32, 32), ("k", 8, 32), ("v", 8, 32), ("o", 32, 32), ("gate", 48, 32),
                                   ("up", 48, 32), ("down", 32, 48)]):
        _, wms[p], codes[p] = oracle.ternarize_pack(synth.master_weight(20 + j, n, k))
    x = synth.act_normal_f32(15, 3, 32)
    la, lb = oracle.layer(x, codes, wms), oracle.layer_f64gemm(x, codes, wms)
    for key in la:
        assert np.array_equal(la[key], lb[key]), key
