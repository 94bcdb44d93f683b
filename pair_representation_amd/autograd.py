"""The whole layer as a torch.autograd.Function on one GPU.

Page 1 (section "Pra quem e") expects the triangle multiplicative update to be
trained through custom autograd functions.  ``TriMul`` composes the library's
entry points (argument marshalling and call order only; every step runs in the
HIP kernels):

  forward   tile_operands (K1) -> tile with FIRST | LAST (K2, K3)
  backward  epilogue_backward (dL/dx, the gate's dL/dz, the epilogue's
            parameters) -> tile_backward (dL/da, dL/db) -> tile_operands_backward
            (the projections' dL/dz and parameters, added to the above)

over the whole N x N grid as one tile and one k-chunk.  The forward keeps the
operands a, b and the contraction result x for the backward (in bf16 mode
2 * 128 * N^2 * 2 bytes plus 128 * N^2 * 4 bytes).
"""
from __future__ import annotations

import torch
from torch.autograd.function import once_differentiable

from . import (BF16, F32, INCOMING, OUTGOING, TILE_FIRST, TILE_LAST, Weights, epilogue_backward, new_xacc, tile,
               tile_backward, tile_operands, tile_operands_backward)

PARAM_NAMES = ("ln_in_w", "ln_in_b", "w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate", "w_out_gate", "ln_out_w",
               "ln_out_b", "w_out_proj")


class TriMul(torch.autograd.Function):
    """out = TriMul.apply(z, mask, direction, eps, *params) with params in
    PARAM_NAMES order.  z is [N, N, 128] bf16 or fp32 (the storage dtype of
    the matrices, which must match it), mask [N, N] uint8; LayerNorm vectors
    fp32.  Returns the fp32 update [N, N, 128]."""

    @staticmethod
    def forward(ctx, z, mask, direction, eps, *params):
        dtype = BF16 if z.dtype == torch.bfloat16 else F32
        w = Weights(dict(zip(PARAM_NAMES, params)), dtype, eps=eps, device=z.device)
        n = z.shape[0]
        kp = (n + 63) // 64 * 64
        a, b = tile_operands(w, direction, z, mask, 0, n, 0, n, 0, n, kp)
        x = new_xacc(n, n, z.device)
        out = tile(w, n, 0, n, 0, n, [(0, n, a, b)], TILE_FIRST | TILE_LAST, x, z, mask)
        ctx.save_for_backward(z, mask, x, a, b, *params)
        ctx.direction, ctx.eps, ctx.dtype = direction, eps, dtype
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, dout):
        z, mask, x, a, b, *params = ctx.saved_tensors
        w = Weights(dict(zip(PARAM_NAMES, params)), ctx.dtype, eps=ctx.eps, device=z.device)
        n = z.shape[0]
        # dx in a buffer of its own: the saved x stays intact for a second
        # backward through the same graph (retain_graph)
        dx, dz, g_epi = epilogue_backward(w, n, 0, n, 0, n, x, z, mask, dout.contiguous().float())
        da, db = tile_backward(w, n, n, [(0, n, a, b)], dx)
        g_proj = {k: torch.zeros(params[PARAM_NAMES.index(k)].shape, dtype=torch.float32, device=z.device)
                  for k in ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate")}
        g_proj["ln_in_w"], g_proj["ln_in_b"] = g_epi["ln_in_w"], g_epi["ln_in_b"]
        tile_operands_backward(w, ctx.direction, z, mask, 0, n, 0, n, 0, n, da=da[0], db=db[0], dz=dz,
                               grads=g_proj, accumulate=True)
        grads = dict(g_epi)
        grads.update(g_proj)
        return (dz.to(z.dtype), None, None, None) + tuple(grads[k].to(p.dtype) for k, p in zip(PARAM_NAMES, params))


def trimul(z, mask, params: dict, direction=OUTGOING, eps=1e-5):
    """Differentiable layer call: ``params`` maps PARAM_NAMES to tensors."""
    return TriMul.apply(z, mask, direction, eps, *[params[k] for k in PARAM_NAMES])


__all__ = ["TriMul", "trimul", "PARAM_NAMES", "OUTGOING", "INCOMING"]
