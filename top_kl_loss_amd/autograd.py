"""PyTorch autograd integration of the fused, chunked top-K KL loss.

``topk_kl_loss(H, W, topk_idx, topk_logit, mask, tau, chunk)`` returns the
loss as a 0-dim tensor whose backward produces dL/dH and dL/dW, so the loss
drops into a student training step ("Making Knowledge Distillation Cheap
Enough to Run at Scale", aipuls.nl, section "Summary": the cached teacher
logits are used while the student trains).  Every step runs in the HIP
library; this module only routes tensors.

Two schedules:

* fused (default): the forward calls kd_topk_kl_fwd_bwd, so the three GEMMs
  of loss and gradients run once; the backward scales the stored fp32
  gradients by the upstream gradient and casts them to the inputs' dtype
  (kd_grad_cast).  Holds dH [T,d] and dW [V,d] in fp32 between the passes.
* recompute: the forward calls kd_topk_kl_fwd (logits GEMM only); the
  backward calls kd_topk_kl_bwd, which recomputes the logits: four GEMMs
  in all, nothing [T,d]- or [V,d]-sized held between the passes.
"""
from __future__ import annotations

import torch

from . import (kd_entropy_filter, kd_grad_cast, kd_topk_div_fwd_bwd,
               kd_topk_kl_bwd, kd_topk_kl_fwd, kd_topk_kl_fwd_bwd)

__all__ = ["TopKKLLossFunction", "topk_kl_loss", "TopKKLLoss"]


class TopKKLLossFunction(torch.autograd.Function):
    """forward(H, W, topk_idx, topk_logit, mask, tau, chunk, recompute) ->
    loss (0-dim fp32); gradients flow to H and W."""

    @staticmethod
    def forward(ctx, H, W, topk_idx, topk_logit, mask, tau, chunk, recompute,
                divergence="forward_kl"):
        ctx.recompute = bool(recompute)
        ctx.tau, ctx.chunk = float(tau), chunk
        ctx.dtypes = (H.dtype, W.dtype)
        if divergence != "forward_kl":
            # reverse KL / JSD over the top-K support: one fused call
            if ctx.recompute:
                raise ValueError("recompute applies to the forward KL only")
            loss, _, dH, dW = kd_topk_div_fwd_bwd(divergence, H, W, topk_idx,
                                                  topk_logit, mask, tau,
                                                  row_loss=False)
            ctx.save_for_backward(dH, dW)
        elif ctx.recompute:
            loss, _, _ = kd_topk_kl_fwd(H, W, topk_idx, topk_logit, mask, tau,
                                        chunk, row_loss=False, lse=False)
            ctx.save_for_backward(H, W, topk_idx, topk_logit,
                                  mask if mask is not None else torch.empty(0))
            ctx.has_mask = mask is not None
        else:
            loss, _, dH, dW = kd_topk_kl_fwd_bwd(H, W, topk_idx, topk_logit,
                                                 mask, tau, chunk, row_loss=False)
            ctx.save_for_backward(dH, dW)
        return loss.reshape(())

    @staticmethod
    def backward(ctx, grad):
        g = grad.detach().to(torch.float32).reshape(1).contiguous()
        if ctx.recompute:
            H, W, idx, logit, mask = ctx.saved_tensors
            dH, dW = kd_topk_kl_bwd(H, W, idx, logit,
                                    mask if ctx.has_mask else None, ctx.tau,
                                    ctx.chunk, 0, g)
            scale = None
        else:
            dH, dW = ctx.saved_tensors
            scale = g
        gH = _finish(dH, ctx.dtypes[0], scale) if ctx.needs_input_grad[0] else None
        gW = _finish(dW, ctx.dtypes[1], scale) if ctx.needs_input_grad[1] else None
        return gH, gW, None, None, None, None, None, None, None


def _finish(g32, dtype, scale):
    """The fp32 gradient times scale in the parameter's dtype (a new tensor;
    the saved gradients stay intact for a second backward)."""
    if dtype == torch.float32 and scale is None:
        return g32
    return kd_grad_cast(g32, dtype, scale)


def topk_kl_loss(H, W, topk_idx, topk_logit, mask=None, tau=1.0, chunk=None,
                 recompute=False, entropy_filter=None, divergence="forward_kl"):
    """tau^2 / N * sum_t mask_t KL(q_t || p_t): the teacher's distribution q
    over its K cached logits against the student's softmax p over all V
    logits z = H W^T, both at temperature tau (see include/kd_topk_kl.h).
    H [T,d], W [V,d] bf16 or fp32 CUDA tensors; topk_idx int32 and
    topk_logit fp32 [T,K]; mask [T] or None.  Differentiable in H and W.

    entropy_filter: None, ("above", threshold) or ("top_fraction", fraction):
    the loss then runs only on the tokens kd_entropy_filter keeps (teacher
    entropy above the threshold, or the given fraction of valid tokens with
    the highest entropy), and N counts those tokens.

    divergence: "forward_kl" (the above), or "reverse_kl" / "jsd": the
    divergence between the student restricted to the K cached ids
    (renormalised) and the teacher there (kd_topk_div_fwd_bwd; no chunk).

    When no gradient is wanted (grad mode off, or neither H nor W requires
    one) the forward KL runs kd_topk_kl_fwd alone."""
    if entropy_filter is not None:
        mode, param = entropy_filter
        mask, _ = kd_entropy_filter(topk_logit, mask, tau, mode, param,
                                    entropy=False)
    if divergence == "forward_kl" and not (
            torch.is_grad_enabled() and (H.requires_grad or W.requires_grad)):
        # no gradient wanted (evaluation, torch.no_grad): the forward alone,
        # a third of the work and no gradient buffers; the same loss bits
        loss, _, _ = kd_topk_kl_fwd(H, W, topk_idx, topk_logit, mask, tau,
                                    chunk, row_loss=False, lse=False)
        return loss.reshape(())
    return TopKKLLossFunction.apply(H, W, topk_idx, topk_logit, mask, tau,
                                    chunk, recompute, divergence)


class TopKKLLoss(torch.nn.Module):
    """Module form of topk_kl_loss with fixed tau, chunk and schedule."""

    def __init__(self, tau=1.0, chunk=None, recompute=False, entropy_filter=None,
                 divergence="forward_kl"):
        super().__init__()
        self.tau, self.chunk, self.recompute = float(tau), chunk, bool(recompute)
        self.entropy_filter = entropy_filter
        self.divergence = divergence

    def forward(self, H, W, topk_idx, topk_logit, mask=None):
        return topk_kl_loss(H, W, topk_idx, topk_logit, mask, self.tau,
                            self.chunk, self.recompute, self.entropy_filter,
                            self.divergence)
