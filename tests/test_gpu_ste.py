"""GPU parity of the straight-through backward (bl_ste_grad_input /
bl_ste_grad_weight) against the oracle's plain fp64 definitions,
dX = dY . (codes * w_mean) and dW = dY^T . (q / a), nothing rounded.

Tolerance, derived from what the kernels round (u = 2^-8, the unit roundoff
of bf16):
  * the products take bf16 operands.  The codes and q are exact in bf16; the
    gradient is exact when it comes in bf16, else rounded once (relative u);
    for dW the kernel forms fp32(dy / a) (relative 2^-24) and rounds it to bf16
    (relative u).  Each term t of a sum is therefore taken as t (1 + d) with
    |d| <= u_in, u_in = 0 (dX, bf16 gradient) or u + 2^-23;
  * the matrix cores add 32 exact bf16 products per step and the steps in
    fp32: at most L/32 + 2 roundings of 2^-24 on sum |t| for L <= 2^14 terms,
    bounded by 2^-14 sum |t|; dX adds one rounding of the w_mean scaling;
  => worst case, per element:  |got - ref| <= (u_in + 2^-14) sum |t| + 2^-23 |ref|.
  * rounding model: the bf16 rounding errors of distinct terms are independent
    with E[d^2] <= u^2/3, so sum_t t d has variance <= (u^2/3) sum t^2; the
    mean of z^2 = err^2 / ((u^2/3) sum t^2) over a tested block of at least
    1024 elements must stay below 2 (its expectation is about 0.54).  A dropped or doubled term moves
    z^2 by about 3 / (u^2 M), hundreds at these sizes.
Every output is pre-filled with NaN and followed by a canary tail.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import assert_exact, bf16_dev, dev, f32_of_bf16, guarded, host, requires_gpu, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]

U = 2.0 ** -8


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


def _rows(n, full):
    """All rows of small problems; else tile edges and a spread of others."""
    if n <= 512:
        return np.arange(n)
    r = {0, 1, n - 1, n - 2}
    for e in range(128, n, 128):
        r.update((e - 1, e))
    r = sorted(r)
    return np.array(r[:: max(1, len(r) // full)] + [n - 1])


def _check_bounds(got, ref, abs_terms, sq_terms, u_in, extra, what):
    bound = (u_in + 2.0 ** -14) * abs_terms + 2.0 ** -23 * np.abs(ref) + extra
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the worst-case bound, max err {err.max():.3e}"
    if u_in and err.size >= 1024:   # a mean over enough elements to hold the model to
        z2 = (err ** 2) / np.maximum((U * U / 3.0) * sq_terms, 1e-300)
        assert float(z2.mean()) < 2.0, f"{what}: mean z^2 {float(z2.mean()):.3f} above the rounding model"


SHAPES = [(128, 128, 128), (256, 640, 384), (384, 256, 1024), (100, 200, 300), (1, 4, 1), (130, 36, 70),
          (257, 132, 129), (2048, 2560, 6912)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("dy_kind", ["bf16", "f32"])
def test_ste_grad_input(M, N, K, dy_kind):
    bl = _bl()
    packed, wm, codes = oracle.ternarize_pack(synth.master_weight(80 + K, N, K))
    if dy_kind == "bf16":
        bits = synth.act_normal_bf16(81 + M, M, N)
        dy, dyd, u_in = f32_of_bf16(bits), bf16_dev(bits), 0.0
    else:
        dy = synth.act_normal_f32(81 + M, M, N)
        dyd, u_in = to_dev(dy), U + 2.0 ** -23
    out = guarded((M, K))
    bl.ste_grad_input(dyd, to_dev(packed), to_dev(np.array([wm], np.float32)), dx=out.t)
    out.check("dx")
    rows = _rows(M, 32)
    ref = oracle.ste_grad_input(dy, codes, wm, rows=rows)
    got = host(out.t)[rows].astype(np.float64)
    c = np.abs(codes).astype(np.float64) * float(wm)
    abs_t = np.abs(dy[rows]).astype(np.float64) @ c
    sq_t = (dy[rows].astype(np.float64) ** 2) @ (c ** 2)
    _check_bounds(got, ref, abs_t, sq_t, u_in, 0.0, "dx")


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (100, 200, 300), (257, 132, 129), (1, 4, 1)])
def test_ste_grad_input_bf16_output(M, N, K):
    """dx requested in bf16 is the fp32 result rounded to nearest even
    (oracle.to_bf16), element by element: the same products and sums, only
    the store differs.  Whole and ragged tiles."""
    bl = _bl()
    packed, wm, codes = oracle.ternarize_pack(synth.master_weight(70 + K, N, K))
    dyd = bf16_dev(synth.act_normal_bf16(71 + M, M, N))
    P, W = to_dev(packed), to_dev(np.array([wm], np.float32))
    f32 = guarded((M, K))
    b16 = guarded((M, K), torch.bfloat16)
    bl.ste_grad_input(dyd, P, W, dx=f32.t)
    bl.ste_grad_input(dyd, P, W, dx=b16.t)
    f32.check("dx fp32")
    b16.check("dx bf16")
    assert_exact(host(b16.t), oracle.to_bf16(host(f32.t)), "bf16 dx")


@pytest.mark.parametrize("M,N,K", SHAPES[:-1] + [(2048, 6912, 2560)])
@pytest.mark.parametrize("dy_kind", ["bf16", "f32"])
def test_ste_grad_weight(M, N, K, dy_kind):
    bl = _bl()
    q, a = oracle.quant_act(synth.act_normal_f32(90 + K, M, K))
    if dy_kind == "bf16":
        bits = synth.act_normal_bf16(91 + N, M, N)
        dy, dyd = f32_of_bf16(bits), bf16_dev(bits)
    else:
        dy = synth.act_normal_f32(91 + N, M, N)
        dyd = to_dev(dy)
    out = guarded((N, K))
    bl.ste_grad_weight(dyd, to_dev(q), to_dev(a), dw=out.t)
    out.check("dw")
    rows = _rows(N, 32)
    ref = oracle.ste_grad_weight(dy, q, a, rows=rows)
    got = host(out.t)[rows].astype(np.float64)
    s = dy[:, rows].astype(np.float64) / a.astype(np.float64)[:, None]        # [M, rows]
    qa = q.astype(np.float64)
    abs_t = np.abs(s).T @ np.abs(qa)
    sq_t = (s ** 2).T @ (qa ** 2)
    _check_bounds(got, ref, abs_t, sq_t, U + 2.0 ** -23, 0.0, "dw")


def test_ste_shapes_rejected():
    bl = _bl()
    dy = torch.zeros((100, 130), dtype=torch.bfloat16, device=dev())   # N = 130: not a packed width
    with pytest.raises(RuntimeError):
        bl.ste_grad_input(dy, torch.zeros((32, 128), dtype=torch.uint8, device=dev()),
                          torch.ones(1, dtype=torch.float32, device=dev()))


def test_qat_forward_backward_autograd():
    """The online path end to end through torch.autograd: the forward equals
    the oracle's BitLinear on W ternarized this step (bit-exact), the
    gradients the straight-through definitions on the forward's own codes
    (an fp32 output gradient, rounded to bf16 inside the library)."""
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
    dy = synth.act_normal_f32(97, M, N)
    y.backward(to_dev(dy))
    rx = oracle.ste_grad_input(dy, codes, wm)
    rw = oracle.ste_grad_weight(dy, q, a)
    c = np.abs(codes).astype(np.float64) * float(wm)
    _check_bounds(host(xd.grad).astype(np.float64), rx, np.abs(dy).astype(np.float64) @ c,
                  (dy.astype(np.float64) ** 2) @ (c ** 2), U + 2.0 ** -23, 0.0, "dx")
    s = dy.astype(np.float64) / a.astype(np.float64)[:, None]
    qa = q.astype(np.float64)
    _check_bounds(host(Wd.grad).astype(np.float64), rw, np.abs(s).T @ np.abs(qa), (s ** 2).T @ (qa ** 2),
                  U + 2.0 ** -23, 0.0, "dw")


def test_qat_backward_bf16_input():
    """A bf16 input gets its gradient in bf16 from the library (no cast
    after it): the fp32 input gradient of the same call, rounded to nearest
    even."""
    from bit_ternary_weight_amd import qat
    M, N, K = 128, 256, 384
    W = to_dev(synth.master_weight(98, N, K)).requires_grad_(True)
    xb = bf16_dev(synth.act_normal_bf16(99, M, K)).requires_grad_(True)
    y = qat.BitLinearFunction.apply(xb, W)
    dy = to_dev(synth.act_normal_f32(100, M, N))
    y.backward(dy)
    assert xb.grad.dtype == torch.bfloat16
    _, saved = qat.forward(xb.detach(), W.detach())
    dx32, _ = qat.backward(dy, saved)
    assert_exact(host(xb.grad), oracle.to_bf16(host(dx32)), "bf16 input gradient")
