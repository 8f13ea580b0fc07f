"""Pins of the 1-bit BitLinear oracle (layer norm, sign binarization with one
scale per tensor, absmax int8 activations) against facts that do not come
from the oracle: hand-worked bytes and products, closed forms, exact scaling
and shifting invariances, exact rationals.  CPU only.

The page ("How It Works" of the PyTorch 1-bit BitNet summary) names the steps
but prints no formula; the readings pinned here are the ones the oracle's
header states.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _ulp(v: float) -> float:
    return float(np.spacing(np.float32(abs(v)))) if v != 0 else float(np.float32(1.4e-45))


# ----------------------------------------------------------------------------- binarization and packing
# Hand-worked: N = 8 rows (one packed row, bit i = row i), K = 4.
_W8 = np.array([[1, -1, 2, -0.0],
                [0.5, -3, 0, 1],
                [-1, -1, -1, -1],
                [2, 2, 2, 2],
                [0.125, -0.125, 0.125, -0.125],
                [1, 1, -1, -1],
                [-5, 5, -5, 5],
                [0, 0, 0, 0]], np.float32)
# signs per column k (rows 0..7), zero and -0.0 -> +1:
#   k0: + + - + + + - +  -> bits 1,1,0,1,1,1,0,1 -> 0b10111011 = 0xBB
#   k1: - - - + - + + +  -> 0b11101000 = 0xE8
#   k2: + + - + + - - +  -> 0b10011011 = 0x9B
#   k3: + + - + - - + +  -> 0b11001011 = 0xCB
# sum |W| = 4 + 4.5 + 4 + 8 + 0.5 + 4 + 20 + 0 = 45, / 32 = 1.40625 (exact)
def test_w1_binarize_pack_hand_worked():
    packed, ws, signs = oracle.binarize_pack(_W8)
    assert packed.tolist() == [[0xBB, 0xE8, 0x9B, 0xCB]]
    assert ws == np.float32(1.40625)
    assert signs[0].tolist() == [1, -1, 1, 1]      # -0.0 -> +1
    assert signs[7].tolist() == [1, 1, 1, 1]       # zeros -> +1
    assert (oracle.unpack_bits(packed) == signs).all()


@pytest.mark.parametrize("N", [8, 16, 24, 64])
def test_w1_plane_order_one_hot(N):
    """A single negative weight at row n lands in bit n // (N/8) of packed
    row n % (N/8); every other bit is set."""
    R = N // 8
    for n in range(N):
        W = np.ones((N, 3), np.float32)
        W[n, 1] = -2.0
        packed, _, _ = oracle.binarize_pack(W)
        want = np.full((R, 3), 0xFF, np.uint8)
        want[n % R, 1] = 0xFF ^ (1 << (n // R))
        assert (packed == want).all(), n


def test_w1_unpack_inverts_pack_random():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((40, 33)).astype(np.float32)
    packed, _, signs = oracle.binarize_pack(W)
    assert (oracle.unpack_bits(packed) == signs).all()
    assert (signs == np.where(W < 0, -1, 1)).all()


# ----------------------------------------------------------------------------- layer norm
@pytest.mark.parametrize("c", [0.5, 3.0, 1000.0])
def test_layernorm_two_values_eps0(c):
    """x = [-c, c]: mean 0, variance c^2, so with eps = 0 the output is [-1, 1]
    (c r rounds to 1 for these c)."""
    out = oracle.layernorm(np.array([[-c, c]], np.float32), eps=0.0)
    assert out.tolist() == [[-1.0, 1.0]]


def test_layernorm_constant_row_is_zero():
    out = oracle.layernorm(np.full((2, 16), 7.25, np.float32), eps=1e-5)
    assert (out == 0).all()


def test_layernorm_scale_invariance_exact_eps0():
    """With eps = 0 every step scales exactly by powers of two, so LN(2x) and
    LN(x) are bit-identical."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 37)).astype(np.float32)
    assert np.array_equal(oracle.layernorm(2 * x, eps=0.0).view(np.uint32),
                          oracle.layernorm(x, eps=0.0).view(np.uint32))


def test_layernorm_shift_invariance_exact():
    """Integer-valued rows, K a power of two: the mean is exact, so shifting
    the row by an integer leaves every output bit unchanged."""
    rng = np.random.default_rng(2)
    x = rng.integers(-50, 50, size=(4, 64)).astype(np.float32)
    for c in (1.0, -17.0, 1000.0):
        assert np.array_equal(oracle.layernorm(x + np.float32(c)).view(np.uint32),
                              oracle.layernorm(x).view(np.uint32))


def test_layernorm_gain_and_bias():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 24)).astype(np.float32)
    plain = oracle.layernorm(x)
    assert np.array_equal(oracle.layernorm(x, np.ones(24, np.float32), np.zeros(24, np.float32)), plain)
    assert np.array_equal(oracle.layernorm(x, np.full(24, 2.0, np.float32)), 2 * plain)
    g = rng.standard_normal(24).astype(np.float32)
    b = rng.standard_normal(24).astype(np.float32)
    out = oracle.layernorm(x, g, b)
    # each output is one fp32 product and one fp32 sum away from plain * g + b
    ref = plain.astype(np.float64) * g + b
    assert np.all(np.abs(out - ref) <= 2 * np.spacing(np.abs(ref).astype(np.float32)) + 1e-7)


def test_layernorm_moments():
    rng = np.random.default_rng(4)
    x = (3 + 5 * rng.standard_normal((6, 2560))).astype(np.float32)
    out = oracle.layernorm(x, eps=1e-5).astype(np.float64)
    assert np.all(np.abs(out.mean(axis=1)) < 1e-6)
    var = x.astype(np.float64).var(axis=1)
    assert np.all(np.abs(out.var(axis=1) - var / (var + 1e-5)) < 1e-5)


def test_layernorm_exact_rational_small():
    """K = 3 with eps = 0 against the exact value (x - mu) / sqrt(var) worked
    out in 50-digit decimal arithmetic: the oracle's float(x - mu), its
    rounded r and the product are each within half an ulp, so the result
    lies within 2 ulps."""
    getcontext().prec = 50
    x = np.array([[0.7, -2.25, 1.3]], np.float32)
    out = oracle.layernorm(x, eps=0.0)[0]
    xs = [Fraction(float(v)) for v in x[0]]
    mu = sum(xs) / 3
    var = sum((v - mu) ** 2 for v in xs) / 3
    sd = Decimal(var.numerator) / Decimal(var.denominator)
    sd = sd.sqrt()
    for k in range(3):
        d = xs[k] - mu
        exact = (Decimal(d.numerator) / Decimal(d.denominator)) / sd
        assert abs(Decimal(float(out[k])) - exact) <= Decimal(2 * _ulp(float(exact)))


# ----------------------------------------------------------------------------- the 1-bit BitLinear
def test_w1_hand_worked_end_to_end():
    """x = [3, -1, 1, -3] (K = 4): mean 0, variance 5; the normalized row is
    [3r, -r, r, -3r] with r ~ 1/sqrt(5), so amax = 3r and the codes are
    127, rint(-127/3) = -42, 42, -127 whatever the rounding of r.  With
    |W| = 0.25 everywhere the scale is 0.25 and A[n] = sum_k q_k s_nk:
      + + + +: 0;  + - + -: 338;  - + - +: -338;  + + - -: 170;
      + - - +: 0;  - - - -: 0;    + + + -: 254;   - + + +: -254."""
    S = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [-1, 1, -1, 1], [1, 1, -1, -1],
                  [1, -1, -1, 1], [-1, -1, -1, -1], [1, 1, 1, -1], [-1, 1, 1, 1]], np.int8)
    W = (0.25 * S).astype(np.float32)
    packed, ws, signs = oracle.binarize_pack(W)
    assert ws == np.float32(0.25) and (signs == S).all()
    x = np.array([[3, -1, 1, -3]], np.float32)
    q, a, A, y = oracle.bitlinear_w1(x, signs, ws, eps=0.0)
    assert q.tolist() == [[127, -42, 42, -127]]
    assert A.tolist() == [[0, 338, -338, 170, 0, 0, 254, -254]]
    # y = A * 0.25 / a with a = 127 / amax and amax ~ 3 / sqrt(5)
    getcontext().prec = 50
    amax = Decimal(3) / Decimal(5).sqrt()
    for n in range(8):
        exact = Decimal(int(A[0, n])) * Decimal("0.25") * amax / Decimal(127)
        assert abs(Decimal(float(y[0, n])) - exact) <= Decimal(4 * _ulp(float(exact))), n


def test_w1_all_positive_weights_give_code_sums():
    rng = np.random.default_rng(6)
    W = np.abs(rng.standard_normal((16, 48))).astype(np.float32)
    x = rng.standard_normal((3, 48)).astype(np.float32)
    _, ws, signs = oracle.binarize_pack(W)
    q, a, A, y = oracle.bitlinear_w1(x, signs, ws)
    qs = q.astype(np.int64).sum(axis=1)
    assert (A == qs[:, None]).all()


def test_w1_negated_weights_negate_the_output():
    rng = np.random.default_rng(7)
    W = rng.standard_normal((24, 40)).astype(np.float32)
    W[W == 0] = 1.0
    x = rng.standard_normal((4, 40)).astype(np.float32)
    _, ws, s1 = oracle.binarize_pack(W)
    _, ws2, s2 = oracle.binarize_pack(-W)
    assert ws == ws2
    _, _, A1, y1 = oracle.bitlinear_w1(x, s1, ws)
    _, _, A2, y2 = oracle.bitlinear_w1(x, s2, ws)
    assert (A2 == -A1).all() and (y2 == -y1).all()


def test_w1_one_negative_weight():
    """All weights positive except one: that output loses twice its code."""
    rng = np.random.default_rng(8)
    N, K = 16, 32
    x = rng.standard_normal((2, K)).astype(np.float32)
    for n0, k0 in ((0, 0), (5, 31), (15, 7), (9, 16)):
        W = np.ones((N, K), np.float32)
        W[n0, k0] = -1.0
        packed, ws, _ = oracle.binarize_pack(W)
        q, a, A, y = oracle.bitlinear_w1(x, oracle.unpack_bits(packed), ws)
        qs = q.astype(np.int64).sum(axis=1)
        want = np.repeat(qs[:, None], N, axis=1)
        want[:, n0] -= 2 * q[:, k0].astype(np.int64)
        assert (A == want).all(), (n0, k0)


def test_w1_f64gemm_matches_the_c_loop():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((32, 80)).astype(np.float32)
    x = rng.standard_normal((5, 80)).astype(np.float32)
    g = rng.standard_normal(80).astype(np.float32)
    b = rng.standard_normal(80).astype(np.float32)
    _, ws, s = oracle.binarize_pack(W)
    r1 = oracle.bitlinear_w1(x, s, ws, g, b)
    r2 = oracle.bitlinear_w1_f64gemm(x, s, ws, g, b)
    for u, v in zip(r1, r2):
        assert np.array_equal(u, v)
