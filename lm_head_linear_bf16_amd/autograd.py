"""PyTorch autograd front end of the fused LM-head cross-entropy.

Same structure as page 1 ("fused_linear_diffusion_cross_entropy.py"):
``FusedLinearCrossEntropyFunction`` computes the loss and the gradients of
x, weight and bias in its forward (one ``fldce_fwd_bwd_ex`` call; only those
an input requires, so a frozen weight skips the dW GEMM) and keeps them; its
backward multiplies them by the upstream gradient in place
(``fldce_scale_grads``, skipped on the device when it is 1), as the page's
``fused_linear_cross_entropy_backward`` does.  Because the scaling is in
place, a second backward through the same graph (``retain_graph=True``)
raises instead of scaling the gradients twice.
``FusedLinearDiffusionCrossEntropyLoss`` is the module: it flattens
[B, L, H] inputs, defaults p_mask to ones and applies the end-of-block
weight; without a gradient to compute (evaluation) it runs the forward
alone.  Marshalling only; every step runs in the HIP library.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import fldce


class FusedLinearCrossEntropyFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, target, weight, bias=None, p_mask=None, ignore_index=-100,
                label_smoothing=0.0, logit_scale=1.0, reduction="mean", total=0,
                eob_token_id=None, eob_weight=1.0):
        # only the gradients some input needs (a frozen weight skips the dW GEMM)
        r = fldce.fldce_fwd_bwd_ex(x, weight, target, p_mask, bias, ignore_index=ignore_index,
                                   label_smoothing=label_smoothing, logit_scale=logit_scale,
                                   reduction=reduction, total=total, eob_token_id=eob_token_id,
                                   eob_weight=eob_weight,
                                   want_db=bias is not None and ctx.needs_input_grad[3],
                                   want_dH=ctx.needs_input_grad[0],
                                   want_dW=ctx.needs_input_grad[2])
        ctx.save_for_backward(r["dH"], r["dW"], r["db"])
        ctx.scaled = False
        return r["loss"].view(())

    @staticmethod
    def backward(ctx, do):
        if ctx.scaled:
            raise RuntimeError("a second backward through the fused LM-head loss is not supported: "
                               "its gradients were already scaled in place by the first one; "
                               "recompute the loss instead")
        ctx.scaled = True
        dH, dW, db = ctx.saved_tensors
        g = do.detach().to(torch.float32).reshape(1).contiguous()
        if dH is not None or dW is not None or db is not None:
            fldce.fldce_scale_grads(g, dH, dW, db)
        return dH, None, dW, db, None, None, None, None, None, None, None, None


def fused_linear_cross_entropy_loss(x, target, weight, bias=None, p_mask=None,
                                    ignore_index: int = -100, label_smoothing: float = 0.0,
                                    logit_scale: float = 1.0, reduction: str = "mean",
                                    total: int = 0, eob_token_id: Optional[int] = None,
                                    eob_weight: float = 1.0):
    """x [N, H], target [N] int64, weight [V, H], bias [V] or None, p_mask [N]
    float32 or None.  Returns the scalar loss.  When no gradient is wanted
    (grad mode off, or none of x, weight, bias requires one) only the
    forward runs (fldce_fwd: a third of the flops, same loss bit for bit)."""
    if not (torch.is_grad_enabled()
            and any(t is not None and t.requires_grad for t in (x, weight, bias))):
        r = fldce.fldce_fwd(x, weight, target, p_mask, bias, ignore_index=ignore_index,
                            label_smoothing=label_smoothing, logit_scale=logit_scale,
                            reduction=reduction, total=total, eob_token_id=eob_token_id,
                            eob_weight=eob_weight)
        return r["loss"].view(())
    return FusedLinearCrossEntropyFunction.apply(x, target, weight, bias, p_mask, ignore_index,
                                                 label_smoothing, logit_scale, reduction, total,
                                                 eob_token_id, eob_weight)


class FusedLinearDiffusionCrossEntropyLoss(torch.nn.Module):
    def __init__(self, ignore_index: int = -100, label_smoothing: float = 0.0,
                 logit_scale: float = 1.0, reduction: str = "mean"):
        super().__init__()
        if reduction not in ("mean", "sum"):
            raise ValueError(f"reduction must be 'mean' or 'sum', got {reduction!r}")
        self.ignore_index = ignore_index
        self.label_smoothing = label_smoothing
        self.logit_scale = logit_scale
        self.reduction = reduction

    def forward(self, x, target, weight, bias=None, p_mask=None,
                eob_token_id: Optional[int] = None, eob_weight: float = 1.0, total: int = 0):
        x = x.contiguous().view(-1, x.shape[-1])
        target = target.contiguous().view(-1)
        if p_mask is not None:
            p_mask = p_mask.contiguous().view(-1).to(torch.float32)
        if eob_token_id is not None and eob_weight == 1.0:
            eob_token_id = None
        return fused_linear_cross_entropy_loss(
            x, target, weight.contiguous(), None if bias is None else bias.contiguous(), p_mask,
            self.ignore_index, self.label_smoothing, self.logit_scale, self.reduction, total,
            eob_token_id, eob_weight)
