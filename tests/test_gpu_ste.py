"""GPU parity of the straight-through backward (bl_ste_grad_input /
bl_ste_grad_weight) against the oracle.

Both sides take the same bf16 operands (the gradient as given, the codes and
the activation codes exactly, bf16(dy / a) by the same fp32 division and
round-to-nearest-even); the products of two bf16 values are exact in fp32, so
what remains is the order of the fp32 sums.  The matrix cores add 32 products
per step and the steps in fp32: |got - ref| <= 2^-14 * sum |terms| (about
L/32 roundings of 2^-24 for L up to 2^14 terms), plus one rounding of the
w_mean scaling for dX.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import bf16_dev, dev, f32_of_bf16, host, requires_gpu, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 640, 384), (384, 256, 1024), (2048, 2560, 6912)])
def test_ste_grad_input(M, N, K):
    bl = _bl()
    packed, wm, codes = oracle.ternarize_pack(synth.master_weight(80 + K, N, K))
    bits = synth.act_normal_bf16(81 + M, M, N)
    dy = f32_of_bf16(bits)
    dx = host(bl.ste_grad_input(bf16_dev(bits), to_dev(packed), to_dev(np.array([wm], np.float32))))
    ref = oracle.ste_grad_input(dy, codes, wm)
    bound = 2.0 ** -14 * (np.abs(dy).astype(np.float64) @ np.abs(codes).astype(np.float64)) * float(wm) \
        + 2.0 ** -23 * np.abs(ref)
    bad = np.abs(dx - ref) > bound
    assert not bad.any(), (int(bad.sum()), float(np.abs(dx - ref).max()))


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 384, 640), (512, 128, 256), (2048, 6912, 2560)])
def test_ste_grad_weight(M, N, K):
    bl = _bl()
    q, a = oracle.quant_act(synth.act_normal_f32(90 + K, M, K))
    bits = synth.act_normal_bf16(91 + N, M, N)
    dy = f32_of_bf16(bits)
    dw = host(bl.ste_grad_weight(bf16_dev(bits), to_dev(q), to_dev(a)))
    ref = oracle.ste_grad_weight(dy, q, a)
    s = oracle.bf16_round(dy / a[:, None]).astype(np.float64)
    bound = 2.0 ** -14 * (np.abs(s).T @ np.abs(q).astype(np.float64))
    bad = np.abs(dw - ref) > bound
    assert not bad.any(), (int(bad.sum()), float(np.abs(dw - ref).max()))


def test_ste_shapes_rejected():
    bl = _bl()
    dy = torch.zeros((100, 128), dtype=torch.bfloat16, device=dev())
    with pytest.raises(RuntimeError):
        bl.ste_grad_input(dy, torch.zeros((32, 128), dtype=torch.uint8, device=dev()),
                          torch.ones(1, dtype=torch.float32, device=dev()))


def test_qat_forward_backward_autograd():
    """The online path end to end through torch.autograd: the forward equals
    the oracle's BitLinear on W ternarized this step (bit-exact), the
    gradients equal the straight-through oracle on the forward's own codes."""
    from bit_ternary_weight_amd import qat
    from gpu_helpers import F32_TOL, assert_rows_close
    M, N, K = 256, 384, 640
    W = synth.master_weight(95, N, K)
    x = synth.act_normal_f32(96, M, K)
    Wd = to_dev(W).requires_grad_(True)
    xd = to_dev(x).requires_grad_(True)
    y = qat.BitLinearFunction.apply(xd, Wd)
    _, wm, codes = oracle.ternarize_pack(W)
    q, a, A, ref = oracle.bitlinear(x, codes, None, wm)
    yh = host(y.detach())
    assert_rows_close(yh, ref, F32_TOL)
    assert np.array_equal(yh.view(np.uint32), ref.view(np.uint32))
    bits = synth.act_normal_bf16(97, M, N)
    y.backward(bf16_dev(bits).float())
    dy = f32_of_bf16(bits)
    rx = oracle.ste_grad_input(dy, codes, wm)
    rw = oracle.ste_grad_weight(dy, q, a)
    bx = 2.0 ** -14 * (np.abs(dy).astype(np.float64) @ np.abs(codes).astype(np.float64)) * float(wm) + 2.0 ** -23 * np.abs(rx)
    s = oracle.bf16_round(dy / a[:, None]).astype(np.float64)
    bw = 2.0 ** -14 * (np.abs(s).T @ np.abs(q).astype(np.float64))
    assert np.all(np.abs(host(xd.grad) - rx) <= bx)
    assert np.all(np.abs(host(Wd.grad) - rw) <= bw)
