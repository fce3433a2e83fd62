"""PyTorch autograd wrapper of the fused convolution (fixed path weights).

The forward calls eqtp_conv_fused and the backward eqtp_conv_backward; all
arithmetic runs in the HIP library.  Gradients flow to the edge vectors (for
forces), the node features and the path weights.
"""
from __future__ import annotations

import torch

from . import eqtp as _eq


class EquivariantConvFunction(torch.autograd.Function):
    """out = conv(vec, x, weights) over dst-sorted (row_ptr) or unsorted (dst) edges."""

    @staticmethod
    def forward(ctx, vec, x, weights, src, row_ptr, dst, lmax, path_set):
        out = _eq.eqtp_conv_fused(vec, src, x, weights, lmax, row_ptr=row_ptr, dst=dst, path_set=path_set)
        ctx.save_for_backward(vec, x, weights, src, row_ptr, dst)
        ctx.lmax = lmax
        ctx.path_set = path_set
        return out

    @staticmethod
    def backward(ctx, grad_out):
        vec, x, weights, src, row_ptr, dst = ctx.saved_tensors
        need_vec, need_x, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1], ctx.needs_input_grad[2]
        gx = gw = gv = None
        if need_vec or need_x or need_w:
            gx, gw, gv = _eq.eqtp_conv_backward(vec, src, x, weights, grad_out.contiguous(), ctx.lmax,
                                                row_ptr=row_ptr, dst=dst, path_set=ctx.path_set, need_x=need_x,
                                                need_w=need_w, need_vec=need_vec)
        return gv, gx, gw, None, None, None, None, None


def equivariant_conv(vec, x, weights, src, lmax: int, row_ptr=None, dst=None, path_set: int = _eq.EQTP_PATHS_PARITY):
    """Differentiable fused convolution (see eqtp_conv_fused for the layouts)."""
    return EquivariantConvFunction.apply(vec, x, weights, src, row_ptr, dst, lmax, path_set)
