"""torch.autograd bindings: the forward and backward entry points of the C ABI
as autograd Functions, so the FFN / MoE sub-layer trains inside a PyTorch
graph.  Argument marshalling only: both passes run in the library's kernels.
The backward recomputes the routing from the saved inputs; the gate/up
activations it either recomputes or, with ``keep_activations`` (the
default), takes from the buffer the training forward filled, which holds
them until the backward has run."""
from __future__ import annotations

from typing import Optional

import torch

from . import ops


class _SwiGLUFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, Wg, Wu, Wd, residual, keep):
        ctx.save_for_backward(x, Wg, Wu, Wd)
        ctx.has_residual = residual is not None
        ctx.saved = None
        if keep and any(ctx.needs_input_grad[:4]):
            H, I = x.shape[-1], Wg.shape[0]
            nb = ops.ffn_bwd_workspace_bytes(x.numel() // H, H, I, x.dtype)
            ctx.saved = torch.empty(max(nb, 256), dtype=torch.uint8, device=x.device)
        return ops.ffn_swiglu_fwd(x, Wg, Wu, Wd, residual=residual, saved=ctx.saved)

    @staticmethod
    def backward(ctx, dy):
        x, Wg, Wu, Wd = ctx.saved_tensors
        g = ops.ffn_swiglu_bwd(x, Wg, Wu, Wd, dy.contiguous(), workspace=ctx.saved,
                               from_saved=ctx.saved is not None)
        ctx.saved = None
        return g.dx, g.dWg, g.dWu, g.dWd, (dy if ctx.has_residual else None), None


def swiglu_ffn(x: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor,
               residual: Optional[torch.Tensor] = None, *,
               keep_activations: bool = True) -> torch.Tensor:
    """Differentiable dense SwiGLU FFN: y = residual + Wd (SiLU(Wg x) * Wu x).
    ``keep_activations``: the forward keeps g, u for the backward (one backward
    workspace held from the forward to the backward) instead of the backward
    recomputing them; the results are the same bits either way."""
    keep = keep_activations and torch.is_grad_enabled()  # no backward under no_grad
    return _SwiGLUFunction.apply(x, Wg, Wu, Wd, residual, keep)


class _MoEFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, Wr, Wg, Wu, Wd, residual, k, aux_coef, z_coef, capacity_factor,
                norm_topk_prob, keep):
        ctx.saved = None
        if keep and any(ctx.needs_input_grad[:5]):
            H, (E, I) = x.shape[-1], Wg.shape[:2]
            nb = ops.moe_bwd_workspace_bytes(x.numel() // H, H, I, E, k, x.dtype)
            ctx.saved = torch.empty(max(nb, 256), dtype=torch.uint8, device=x.device)
        out = ops.moe_ffn_fwd(x, Wr, Wg, Wu, Wd, k, aux_coef, residual=residual,
                              norm_topk_prob=norm_topk_prob, z_coef=z_coef,
                              capacity_factor=capacity_factor, return_lists=False,
                              saved=ctx.saved)
        ctx.save_for_backward(x, Wr, Wg, Wu, Wd)
        ctx.cfg = (k, aux_coef, z_coef, capacity_factor, norm_topk_prob, residual is not None)
        z = out.z_loss if out.z_loss is not None else torch.zeros(1, dtype=torch.float32,
                                                                   device=x.device)
        ctx.mark_non_differentiable(out.topk_idx, out.alpha)
        return out.y, out.aux_loss, z, out.topk_idx, out.alpha

    @staticmethod
    def backward(ctx, dy, daux, dz, _didx, _dalpha):
        x, Wr, Wg, Wu, Wd = ctx.saved_tensors
        k, aux_coef, z_coef, capacity_factor, norm, has_res = ctx.cfg
        if dy is None:
            dy = torch.zeros_like(x)
        # the loss terms' upstream gradients stay on the device (the kernel
        # reads them): no host synchronisation in the backward
        f32 = lambda t: t.reshape(-1)[:1].to(torch.float32).contiguous()
        aux_grad = f32(daux) if daux is not None else 0.0
        z_grad = f32(dz) if dz is not None else 0.0
        g = ops.moe_ffn_bwd(x, Wr, Wg, Wu, Wd, dy.contiguous(), k, aux_coef, aux_grad=aux_grad,
                            norm_topk_prob=norm, z_coef=z_coef, z_grad=z_grad,
                            capacity_factor=capacity_factor, workspace=ctx.saved,
                            from_saved=ctx.saved is not None)
        ctx.saved = None
        return (g.dx, g.dWr, g.dWg, g.dWu, g.dWd, (dy if has_res else None),
                None, None, None, None, None, None)


def moe_ffn(x: torch.Tensor, Wr: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor,
            Wd: torch.Tensor, k: int, aux_coef: float, *, residual: Optional[torch.Tensor] = None,
            z_coef: float = 0.0, capacity_factor: float = 0.0, norm_topk_prob: bool = True,
            keep_activations: bool = True):
    """Differentiable top-k MoE FFN.  Returns (y, aux_loss [1], z_loss [1],
    topk_idx, alpha); y, aux_loss and z_loss carry gradients to x and every
    weight (topk_idx and alpha are the router's choices, not differentiable).
    ``keep_activations`` as for swiglu_ffn."""
    keep = keep_activations and torch.is_grad_enabled()  # no backward under no_grad
    return _MoEFunction.apply(x, Wr, Wg, Wu, Wd, residual, k, aux_coef, z_coef, capacity_factor,
                              norm_topk_prob, keep)
