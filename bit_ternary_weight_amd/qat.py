"""BitLinear for quantization-aware training (the online path).

Article "Transformers 实战 BitNet 1.58 位量化", "BitLinear 的三步量化": in
training the weight is ternarized from its fp32 master at every forward
(absmean scale) and the activations are quantized per token (absmax); both
quantizers pass gradients straight through in the backward.  So:

  forward   y  = x~ . W~^T with W~ = codes * w_mean, x~ = q / a: the same bits
               as the inference forward (int8 x ternary contraction, rescale
               by w_mean / a), computed from W freshly ternarized;
  backward  dX = dY . W~ and dW = dY^T . x~ (the gradient of the master W).

Every step runs in libbitlinear: bl_ternarize_pack, bl_quant_act,
bl_gemv_w2a8 / bl_gemm_w2a8, bl_ste_grad_input, bl_ste_grad_weight.  The
backward takes the output gradient as it comes (bf16 or fp32); the library
rounds an fp32 one to bf16, the products' operand type, on the device.
"""
from __future__ import annotations

import torch

from . import binding as bl

DECODE_MAX_M = 64


def forward(x: torch.Tensor, W: torch.Tensor):
    """x [M,K] fp32/bf16, W [N,K] fp32 master -> (y [M,N] fp32, saved), where
    saved = (packed, w_mean, q, a) is what the backward needs."""
    packed, w_mean = bl.ternarize_pack(W)
    q, a = bl.quant_act(x)
    fn = bl.gemv_w2a8 if x.shape[0] <= DECODE_MAX_M else bl.gemm_w2a8
    y = fn(q, packed, w_mean, a=a)
    return y, (packed, w_mean, q, a)


def backward(dy: torch.Tensor, saved, dx_dtype=torch.float32):
    """dy [M,N] bf16 or fp32 -> (dx [M,K] in dx_dtype (fp32 or bf16, rounded on
    the device), dW [N,K] fp32)."""
    packed, w_mean, q, a = saved
    if not dy.is_contiguous():
        raise ValueError("dy must be contiguous")
    return bl.ste_grad_input(dy, packed, w_mean, dx_dtype=dx_dtype), bl.ste_grad_weight(dy, q, a)


class BitLinearFunction(torch.autograd.Function):
    """autograd wrapper: y = BitLinearFunction.apply(x, W)."""

    @staticmethod
    def forward(ctx, x, W):
        y, saved = forward(x, W)
        ctx.saved = saved
        ctx.x_dtype = x.dtype
        return y

    @staticmethod
    def backward(ctx, dy):
        dx, dW = backward(dy, ctx.saved, dx_dtype=ctx.x_dtype)
        ctx.saved = None
        return dx, dW
