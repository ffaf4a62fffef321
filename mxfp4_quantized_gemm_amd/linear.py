"""A linear layer whose three products run through the fused MXFP4 entry
points ([P1] "Pretraining Large Language Models with MXFP4 on Native FP4
Hardware", architecture section: the MXFP4 GEMM replaces the GEMM of each
linear-layer product, Fprop, Dgrad and Wgrad, and is called from standard
linear modules; quick-read block: both GEMM inputs are rotated along the
reduction axis before quantization).

    forward   Y  = X W^T      mxfp4_fprop  (X, W rotated along K)
    backward  dX = dY W       mxfp4_dgrad  (dY, W rotated along N)
              dW = dY^T X     mxfp4_wgrad  (dY, X rotated along T)

Marshalling only: the autograd function allocates the workspace and the
outputs with torch and calls the C ABI; every step of each product runs in
the library's kernels. Tensors are bf16 and row-major; T (tokens), N (out
features) and K (in features) must be multiples of 32 (each is the
reduction axis of one product). Outputs and gradients are bf16 (rounded to
nearest even from the fp32 accumulators), matching bf16 parameters. No bias:
the products of a Llama block have none.
"""
from __future__ import annotations

import torch

from . import (OP_DGRAD, OP_FPROP, OP_WGRAD, OUT_BF16, SCALE_OCP_FLOOR, mxfp4_dgrad,
               mxfp4_fprop, mxfp4_wgrad, mxfp4_workspace_bytes)

_ENTRY = {OP_FPROP: mxfp4_fprop, OP_DGRAD: mxfp4_dgrad, OP_WGRAD: mxfp4_wgrad}


def _product(op, P, Q, T, N, K, hadamard, scale_mode, out_shape):
    ws = torch.empty(mxfp4_workspace_bytes(op, T, N, K), dtype=torch.uint8, device=P.device)
    out = torch.empty(out_shape, dtype=torch.bfloat16, device=P.device)
    _ENTRY[op](P, Q, T, N, K, hadamard, scale_mode, ws, out, OUT_BF16)
    return out


class MXFP4LinearFunction(torch.autograd.Function):
    """Y = X W^T with MXFP4 products; modes = (fprop, dgrad, wgrad) scale rules."""

    @staticmethod
    def forward(ctx, X, W, hadamard, modes):
        T, K = X.shape
        N = W.shape[0]
        X, W = X.contiguous(), W.contiguous()
        ctx.save_for_backward(X, W)
        ctx.hadamard, ctx.modes = hadamard, modes
        return _product(OP_FPROP, X, W, T, N, K, hadamard, modes[0], (T, N))

    @staticmethod
    def backward(ctx, dY):
        X, W = ctx.saved_tensors
        T, K = X.shape
        N = W.shape[0]
        dY = dY.contiguous()
        dX = dW = None
        if ctx.needs_input_grad[0]:
            dX = _product(OP_DGRAD, dY, W, T, N, K, ctx.hadamard, ctx.modes[1], (T, K))
        if ctx.needs_input_grad[1]:
            dW = _product(OP_WGRAD, dY, X, T, N, K, ctx.hadamard, ctx.modes[2], (N, K))
        return dX, dW, None, None


class MXFP4Linear(torch.nn.Module):
    """Bias-free linear layer, weight [out_features][in_features] in bf16.

    hadamard: 16 (the method's H16), 32 or 0. modes: the E8M0 rule of the
    Fprop, Dgrad and Wgrad products (SCALE_OCP_FLOOR or SCALE_CEIL each);
    the ceiling rule keeps heavy-tailed Wgrad operands from clipping.
    Inputs of shape [..., in_features] are flattened to T rows.
    """

    def __init__(self, in_features, out_features, hadamard=16,
                 modes=(SCALE_OCP_FLOOR, SCALE_OCP_FLOOR, SCALE_OCP_FLOOR), device=None):
        super().__init__()
        if in_features % 32 or out_features % 32:
            raise ValueError("in_features and out_features must be multiples of 32")
        self.hadamard, self.modes = hadamard, tuple(modes)
        w = torch.empty(out_features, in_features, dtype=torch.bfloat16, device=device)
        torch.nn.init.normal_(w, std=in_features ** -0.5)
        self.weight = torch.nn.Parameter(w)

    def forward(self, x):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1])
        if x2.shape[0] % 32:
            raise ValueError("the number of input rows must be a multiple of 32")
        y = MXFP4LinearFunction.apply(x2, self.weight, self.hadamard, self.modes)
        return y.reshape(*lead, self.weight.shape[0])
