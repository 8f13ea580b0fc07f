"""GPU parity: bl_quant_act and bl_ternarize_pack against the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import assert_exact, bf16_dev, dev, f32_of_bf16, host, requires_gpu, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


# ----------------------------------------------------------------------------- activation quantization
def _check_quant_f32(x: np.ndarray):
    q, a = _bl().quant_act(to_dev(x))
    qr, ar = oracle.quant_act(x)
    assert_exact(host(q), qr, "q")
    assert_exact(host(a).view(np.uint32), ar.view(np.uint32), "a bits")


def _check_quant_bf16(bits: np.ndarray):
    q, a = _bl().quant_act(bf16_dev(bits))
    qr, ar = oracle.quant_act(f32_of_bf16(bits))
    assert_exact(host(q), qr, "q")
    assert_exact(host(a).view(np.uint32), ar.view(np.uint32), "a bits")


def test_quant_m4_k256_fp32():
    _, x = synth.bitlinear_m4_k256_n256()
    _check_quant_f32(x)


@pytest.mark.parametrize("M,K", [(1, 2560), (1, 6912), (4, 256), (16, 2560), (64, 6912), (4096, 2560)])
def test_quant_bf16_outliers(M, K):
    _check_quant_bf16(synth.act_outliers_bf16(M * 7 + K, M, K))


@pytest.mark.parametrize("M", [16, 64])
def test_quant_bf16_heavy_tail(M):
    _check_quant_bf16(synth.act_heavy_tail_bf16(3, M, 2560))
    _check_quant_bf16(synth.act_heavy_in_row_bf16(4, M, 2560))


@pytest.mark.parametrize("M,K", [(3, 17), (5, 1), (2, 4), (7, 100), (1, 6913)])
def test_quant_ragged_fp32_and_bf16(M, K):
    _check_quant_f32(synth.act_normal_f32(11, M, K))
    _check_quant_bf16(synth.act_outliers_bf16(12, M, K))


# Row lengths at and just past what the register-resident kernel holds
# (8 loads of 16 bytes per lane: 16384 bf16 or 8192 fp32 elements), a last
# load that only some lanes make, and lengths that take the re-reading kernel.
@pytest.mark.parametrize("M,K", [(2, 16384), (2, 16392), (3, 2056), (3, 8192), (2, 8196), (1, 24)])
def test_quant_register_kernel_bounds(M, K):
    _check_quant_f32(synth.act_normal_f32(13 + K, M, K))
    _check_quant_bf16(synth.act_outliers_bf16(14 + K, M, K))


def test_quant_edge_rows():
    x = np.zeros((6, 64), np.float32)
    x[1, 3] = 1e-7                      # below the floor
    x[2, 5] = -1e-45                    # denormal
    x[3] = np.linspace(-2, 2, 64, dtype=np.float32)
    x[4, :] = 3.0                       # constant
    x[5, 7] = -127.0                    # single spike
    x[5, 8] = 63.5                      # tie after scaling: 63.5 -> 64 (even)
    _check_quant_f32(x)


def test_quant_strided_rows():
    full = synth.act_normal_f32(21, 8, 3840)
    xs = to_dev(full)[:, :2560]
    q, a = _bl().quant_act(xs)
    qr, ar = oracle.quant_act(np.ascontiguousarray(full[:, :2560]))
    assert_exact(host(q), qr, "q")
    assert_exact(host(a), ar, "a")


def test_quant_invariants_on_gpu():
    bits = synth.act_heavy_tail_bf16(5, 64, 2560)
    x = to_dev(f32_of_bf16(bits))
    q, a = _bl().quant_act(x)
    q2, a2 = _bl().quant_act(x * 8.0)
    assert torch.equal(q, q2) and torch.equal(a2 * 8.0, a)
    perm = torch.randperm(64, generator=torch.Generator().manual_seed(0)).to(dev())
    q3, a3 = _bl().quant_act(x[perm].contiguous())
    assert torch.equal(q3, q[perm]) and torch.equal(a3, a[perm])


# ----------------------------------------------------------------------------- ternarize + pack
def _check_ternarize(W: np.ndarray):
    packed, wm = _bl().ternarize_pack(to_dev(W))
    pr, wr, _ = oracle.ternarize_pack(W)
    assert_exact(host(wm).view(np.uint32), np.array([wr], np.float32).view(np.uint32), "w_mean bits")
    assert_exact(host(packed), pr, "packed")
    return host(packed), host(wm)


def test_ternarize_m4_k256_n256():
    W, _ = synth.bitlinear_m4_k256_n256()
    _check_ternarize(W)


@pytest.mark.parametrize("proj", ["q", "k", "gate", "down"])
def test_ternarize_layer_projection(proj):
    _check_ternarize(synth.layer_weight(0, proj))


@pytest.mark.parametrize("N,K", [(4, 1), (4, 17), (8, 3), (12, 100), (64, 6913), (256, 256)])
def test_ternarize_ragged(N, K):
    _check_ternarize(synth.master_weight(N + K, N, K))


def test_ternarize_special_cases():
    p, w = _check_ternarize(np.zeros((8, 16), np.float32))
    assert w[0] == np.float32(1e-5) and (p == 0x55).all()
    p, w = _check_ternarize(np.full((8, 16), -0.3, np.float32))
    assert (p == 0).all()
    p, w = _check_ternarize(np.eye(256, dtype=np.float32))
    back, bad = oracle.unpack(p)
    assert bad == 0 and (back == np.eye(256, dtype=np.int8)).all()
    # entries exactly at and one or two ulps around half the scale: groups whose
    # magnitudes average to exactly 0.5 keep w_mean at exactly 0.5
    u25, u24 = 2.0 ** -25, 2.0 ** -24
    groups = [0.25 + u25, 0.25 - u25, 0.75, 0.75, 0.25, 0.75,
              0.25 + u24, 0.75 - u24, 0.25 - u24, 0.75 + u24]
    vals = np.full(256, 0.5, np.float64)
    vals[:10] = groups
    vals[10:20] = [-v for v in groups]
    vals[20::3] *= -1
    W = vals.astype(np.float32).reshape(4, 64)
    assert float(np.abs(W.astype(np.float64)).mean()) == 0.5
    p, w = _check_ternarize(W)
    assert w[0] == np.float32(0.5)
    codes, _ = oracle.unpack(p)
    assert codes.ravel()[:10].tolist() == [1, 0, 1, 1, 0, 1, 1, 1, 0, 1]


def test_ternarize_deterministic():
    W = to_dev(synth.layer_weight(1, "up"))
    p1, w1 = _bl().ternarize_pack(W)
    p2, w2 = _bl().ternarize_pack(W)
    assert torch.equal(p1, p2) and torch.equal(w1, w2)
