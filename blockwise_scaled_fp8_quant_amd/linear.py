"""FP8 linear layer with autograd, on the blockwise-scaled kernels of this library.

The method trains a Transformer's linear layers through FP8 from random initialisation:
activations grouped by 128 along the contraction axis, weights in 128x128 blocks, master
weights and optimizer state kept in BF16/FP32 (agihunt digest "清华用消费级 5090 花 6890
美元从零训 2B，15 项均分超过 Qwen2", section 方法, FP8 bullet; the matmuls of the main
linear layers on the FP8 path after DeepSeek-V3, ModelScope write-up on Puro-2B, section
精度).  Y = X W^T for X [..., Din] and W [Dout, Din], both bf16:

    forward   W -> 128x128 codes + transposed copy      (puro_fp8_quant_w_128x128)
              X -> 1x128 codes and 128x1 codes, one read (puro_fp8_quant_act_dual)
              Y = FWD(X 1x128, W)                        bf16
    backward  dY -> 1x128 and 128x1 codes, one read      (puro_fp8_quant_act_dual)
              dX = DGRAD(dY 1x128, W^T copy)             bf16
              dW = WGRAD(dY 128x1, X 128x1)              fp32

Every arithmetic step runs in the library's HIP kernels; this module allocates buffers,
orders the calls and keeps the codes backward needs (the 128x1 codes of X and the
transposed weight codes; X itself is not kept).  If the weight carries an fp32 `main_grad`
tensor (see Fp8Linear.enable_main_grad), dW is added into it with
puro_fp8_gemm_accumulate and no .grad is produced; otherwise the fp32 dW is returned and
autograd stores it in the weight's dtype.

Shapes follow the kernels: Din, Dout and the number of tokens (product of X's leading
dimensions) must be multiples of 128; anything else raises PuroError (PURO_ERR_SHAPE).
"""
from __future__ import annotations

import math

import torch

from . import (DGRAD, FWD, OUT_BF16, OUT_FP32, WGRAD, puro_fp8_gemm, puro_fp8_gemm_accumulate,
               puro_fp8_quant_act_dual, puro_fp8_quant_w_128x128)

__all__ = ["Fp8LinearFunction", "Fp8Linear", "fp8_linear"]


def _rows(t: torch.Tensor, width: int) -> torch.Tensor:
    """View as [rows, width] with unit column stride (copies only a non-viewable layout)."""
    t2 = t.reshape(-1, width)
    return t2 if t2.stride(1) == 1 else t2.contiguous()


class Fp8LinearFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor) -> torch.Tensor:
        if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
            raise TypeError("Fp8Linear takes bf16 activations and bf16 weights")
        dout, din = weight.shape
        if x.shape[-1] != din:
            raise ValueError(f"x has {x.shape[-1]} features, weight expects {din}")
        x2 = _rows(x, din)
        wq, ws, wqT, wsT = puro_fp8_quant_w_128x128(_rows(weight, din))
        xq, xs, xqT, xsT = puro_fp8_quant_act_dual(x2)
        y = puro_fp8_gemm(FWD, xq, xs, wq, ws, out_dtype=OUT_BF16)
        ctx.save_for_backward(xqT, xsT, wqT, wsT)
        ctx.weight = weight
        ctx.x_shape = x.shape
        return y.view(*x.shape[:-1], dout)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        xqT, xsT, wqT, wsT = ctx.saved_tensors
        weight = ctx.weight
        dout = weight.shape[0]
        if dy.dtype != torch.bfloat16:
            raise TypeError("Fp8Linear expects a bf16 output gradient")
        dy2 = _rows(dy, dout)
        gq, gs, gqT, gsT = puro_fp8_quant_act_dual(dy2)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = puro_fp8_gemm(DGRAD, gq, gs, wqT, wsT, out_dtype=OUT_BF16).view(ctx.x_shape)
        if ctx.needs_input_grad[1]:
            main = getattr(weight, "main_grad", None)
            if main is not None:
                puro_fp8_gemm_accumulate(WGRAD, gqT, gsT, xqT, xsT, main)
            else:
                dw = puro_fp8_gemm(WGRAD, gqT, gsT, xqT, xsT, out_dtype=OUT_FP32)
        return dx, dw


def fp8_linear(x: torch.Tensor, weight: torch.Tensor) -> torch.Tensor:
    """Y = X W^T through the blockwise-scaled FP8 path (differentiable)."""
    return Fp8LinearFunction.apply(x, weight)


class Fp8Linear(torch.nn.Module):
    """Bias-free linear layer (the layers of the pages' Qwen3-like model carry none) whose
    forward and backward matmuls run on the blockwise-scaled FP8 kernels."""

    def __init__(self, in_features: int, out_features: int, device=None):
        super().__init__()
        self.in_features, self.out_features = in_features, out_features
        w = torch.empty((out_features, in_features), dtype=torch.float32, device=device)
        torch.nn.init.kaiming_uniform_(w, a=math.sqrt(5))       # nn.Linear's default
        self.weight = torch.nn.Parameter(w.to(torch.bfloat16))

    def enable_main_grad(self) -> torch.Tensor:
        """Give the weight an fp32 gradient buffer that backward accumulates into."""
        self.weight.main_grad = torch.zeros(self.weight.shape, dtype=torch.float32, device=self.weight.device)
        return self.weight.main_grad

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return Fp8LinearFunction.apply(x, self.weight)

    def extra_repr(self) -> str:
        return f"in_features={self.in_features}, out_features={self.out_features}, fp8=blockwise"
