"""PyTorch autograd wrapper of the fused convolution.

The forward calls eqtp_conv_fused.  The backward groups the edges by source
node on the GPU (eqtp_edge_rows, eqtp_sort_edges) so that grad_x is summed per
source without atomics, and
  * with fixed weights at lmax <= 3: grad_x and grad_w with
    eqtp_conv_backward_by_source (the adjoint of the node-factored forward, on
    the matrix cores) and grad_vec (for forces) with eqtp_conv_backward;
  * with radial weights (weight_mode = EQTP_W_RADIAL) or above lmax 3: all
    three with eqtp_conv_backward_by_source (one walk in each edge's frame;
    grad_vec back in the caller's edge order through the sort's permutation).
``grad_x_mode="edge"`` takes all three from eqtp_conv_backward on the edges as
given instead (grad_x by fp32 atomics).  All arithmetic runs in the HIP
library; this module only marshals arguments.
"""
from __future__ import annotations

import torch

from . import eqtp as _eq


def group_by_source(N: int, src, vec, dst=None, row_ptr=None, with_perm: bool = False):
    """(src_ptr [N+1], vec_s [E,3], dst_s [E]) and, with_perm, perm [E] (the
    caller's index of each grouped edge): the edges grouped by source node (the
    input of eqtp_conv_backward_by_source), each source's edges in input order,
    so grad_x, summed per source over them, is the same from call to call.
    Destinations come from dst, or from a dst-sorted CSR (row_ptr)."""
    E = src.shape[0]
    if dst is None:
        dst = _eq.eqtp_edge_rows(row_ptr, E)
    src_ptr, perm, vec_s, dst_s = _eq.eqtp_sort_edges_stable(src, N, vec=vec, src=dst)
    return (src_ptr, vec_s, dst_s, perm) if with_perm else (src_ptr, vec_s, dst_s)


class EquivariantConvFunction(torch.autograd.Function):
    """out = conv(vec, x, weights) over dst-sorted (row_ptr) or unsorted (dst) edges."""

    @staticmethod
    def forward(ctx, vec, x, weights, src, row_ptr, dst, lmax, path_set, grad_x_mode, weight_mode=_eq.EQTP_W_FIXED,
                r_cut=0.0):
        out = _eq.eqtp_conv_fused(vec, src, x, weights, lmax, row_ptr=row_ptr, dst=dst, path_set=path_set,
                                  weight_mode=weight_mode, r_cut=r_cut)
        ctx.save_for_backward(vec, x, weights, src, row_ptr, dst)
        ctx.lmax = lmax
        ctx.path_set = path_set
        ctx.grad_x_mode = grad_x_mode
        ctx.weight_mode = weight_mode
        ctx.r_cut = r_cut
        return out

    @staticmethod
    def backward(ctx, grad_out):
        vec, x, weights, src, row_ptr, dst = ctx.saved_tensors
        need_vec, need_x, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1], ctx.needs_input_grad[2]
        g = grad_out.contiguous()
        gx = gw = gv = None
        walk = ctx.weight_mode == _eq.EQTP_W_RADIAL or ctx.lmax > 3  # one walk over the edges gives all three
        if walk and ctx.grad_x_mode == "by_source":
            if need_vec or need_x or need_w:
                src_ptr, vec_s, dst_s, perm = group_by_source(x.shape[0], src, vec, dst=dst, row_ptr=row_ptr,
                                                              with_perm=True)
                gx, gw, gv = _eq.eqtp_conv_backward_by_source(vec_s, dst_s, src_ptr, x, weights, g, ctx.lmax,
                                                              path_set=ctx.path_set, need_x=need_x, need_w=need_w,
                                                              need_vec=need_vec, perm=perm,
                                                              weight_mode=ctx.weight_mode, r_cut=ctx.r_cut)
        elif walk:
            if need_vec or need_x or need_w:
                gx, gw, gv = _eq.eqtp_conv_backward(vec, src, x, weights, g, ctx.lmax, row_ptr=row_ptr, dst=dst,
                                                    path_set=ctx.path_set, need_x=need_x, need_w=need_w,
                                                    need_vec=need_vec, weight_mode=ctx.weight_mode,
                                                    r_cut=ctx.r_cut)
        elif ctx.grad_x_mode == "edge":
            if need_vec or need_x or need_w:
                gx, gw, gv = _eq.eqtp_conv_backward(vec, src, x, weights, g, ctx.lmax, row_ptr=row_ptr, dst=dst,
                                                    path_set=ctx.path_set, need_x=need_x, need_w=need_w,
                                                    need_vec=need_vec)
        else:
            if need_x or need_w:
                src_ptr, vec_s, dst_s = group_by_source(x.shape[0], src, vec, dst=dst, row_ptr=row_ptr)
                gx, gw, _ = _eq.eqtp_conv_backward_by_source(vec_s, dst_s, src_ptr, x, weights, g, ctx.lmax,
                                                          path_set=ctx.path_set, need_x=need_x, need_w=need_w)
            if need_vec:
                _, _, gv = _eq.eqtp_conv_backward(vec, src, x, weights, g, ctx.lmax, row_ptr=row_ptr, dst=dst,
                                                  path_set=ctx.path_set, need_x=False, need_w=False, need_vec=True)
        return gv, gx, gw, None, None, None, None, None, None, None, None


def equivariant_conv(vec, x, weights, src, lmax: int, row_ptr=None, dst=None, path_set: int = _eq.EQTP_PATHS_PARITY,
                     grad_x_mode: str = "by_source", weight_mode: int = _eq.EQTP_W_FIXED, r_cut: float = 0.0):
    """Differentiable fused convolution (see eqtp_conv_fused for the layouts).
    grad_x_mode: "by_source" (default) or "edge" (see the module docstring).
    weight_mode=EQTP_W_RADIAL: weights [8, P*C] applied through the radial basis of cut-off r_cut."""
    if grad_x_mode not in ("by_source", "edge"):
        raise ValueError("grad_x_mode must be 'by_source' or 'edge'")
    return EquivariantConvFunction.apply(vec, x, weights, src, row_ptr, dst, lmax, path_set, grad_x_mode,
                                         weight_mode, r_cut)
