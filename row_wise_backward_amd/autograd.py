"""torch.autograd.Function wrappers over libvjp: each op is one forward call
and one backward call of the C ABI; PyTorch's autograd engine records the
graph, calls the backward with the upstream gradient and accumulates
parameter gradients across backward passes.

Contract ("Backward in Triton -- autograd.Function and the backward grid",
sections "The mental model: two kernels, one node" and "A complete minimal
example"; "Writing Triton Kernels with Autograd: A Minimal End-to-End
Example", section 5): forward(ctx, *inputs) saves what the backward needs
with ctx.save_for_backward; backward(ctx, grad_out) returns exactly one
gradient per forward input, in order, None for non-tensor inputs and for
inputs that need no gradient.  Inputs are made contiguous before they reach
a kernel.  Parameter gradients are accumulated in fp32 by the kernels and
returned in the parameter's dtype.

What is saved ("Backward in Triton", section "Save vs recompute";
"Backprop for kernel writers", section 07 "Fusion"):
* weighted sum: x and w (full inputs, nothing cheaper to rebuild them from);
* scaled SiLU: x and w; sigmoid(x) is recomputed in the backward kernel;
* softmax: y (save="y"), or x and the row logsumexp (save="lse": one fp32
  per row, y rebuilt on chip);
* LayerNorm / RMSNorm: x, w and the row mean / rstd (one fp32 each per row);
* row gather (embedding lookup): the indices only; the backward is the
  deterministic scatter-add of dy into the table's rows;
* softmax cross-entropy: the logits, the targets and the row logsumexp;
  the backward rebuilds p = exp(z - lse) and reads the upstream gradient
  from device memory (no host synchronisation).

Every computation runs in the libvjp kernels; the only torch operations
here are argument marshalling (contiguous copies, the int64 -> int32 target
cast, reshapes, and the cast of an fp32 gradient to a 16-bit parameter's
dtype).
"""
from __future__ import annotations

import torch

from . import (vjp_gather_rows_bwd, vjp_gather_rows_fwd, vjp_layernorm_bwd, vjp_layernorm_fwd,
               vjp_rmsnorm_bwd, vjp_rmsnorm_fwd,
               vjp_scaled_silu_bwd, vjp_scaled_silu_fwd, vjp_softmax_bwd, vjp_softmax_bwd_lse,
               vjp_softmax_fwd, vjp_softmax_fwd_lse, vjp_softmax_xent_bwd, vjp_softmax_xent_fwd,
               vjp_weighted_sum_bwd, vjp_weighted_sum_fwd)

__all__ = ["WeightedSum", "ScaledSiLU", "Softmax", "SoftmaxCrossEntropy", "LayerNorm", "RMSNorm",
           "GatherRows", "weighted_sum", "scaled_silu", "softmax", "softmax_cross_entropy",
           "layer_norm", "rms_norm", "gather_rows"]


def _param_grad(g32: torch.Tensor, like: torch.Tensor) -> torch.Tensor:
    g = g32.reshape(like.shape)
    return g if like.dtype == torch.float32 else g.to(like.dtype)


class WeightedSum(torch.autograd.Function):
    """y[i] = sum_j x[i, j] w[j]; x [N, D], w [D] -> y [N] in x's dtype."""

    @staticmethod
    def forward(ctx, x, w):
        x = x.contiguous()
        w = w.contiguous()
        y = vjp_weighted_sum_fwd(x, w)
        ctx.save_for_backward(x, w)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        dx, dw = vjp_weighted_sum_bwd(dy.contiguous(), x, w)
        return (dx if ctx.needs_input_grad[0] else None,
                _param_grad(dw, w) if ctx.needs_input_grad[1] else None)


class ScaledSiLU(torch.autograd.Function):
    """y = w x sigmoid(x) elementwise; w is a one-element fp32 tensor."""

    @staticmethod
    def forward(ctx, x, w):
        xc = x.contiguous()
        w32 = w.reshape(1)
        if w32.dtype != torch.float32:
            w32 = w32.float()
        y = vjp_scaled_silu_fwd(xc.reshape(-1), w32).reshape(x.shape)
        ctx.save_for_backward(xc, w32)
        ctx.w_like = (w.shape, w.dtype)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w32 = ctx.saved_tensors
        dx, dw = vjp_scaled_silu_bwd(dy.contiguous().reshape(-1), x.reshape(-1), w32)
        shape, dtype = ctx.w_like
        dw = dw.reshape(shape)
        return (dx.reshape(x.shape) if ctx.needs_input_grad[0] else None,
                (dw if dtype == torch.float32 else dw.to(dtype)) if ctx.needs_input_grad[1] else None)


class Softmax(torch.autograd.Function):
    """Softmax over the last dimension; save = "y" or "lse"."""

    @staticmethod
    def forward(ctx, x, save="y"):
        if save not in ("y", "lse"):
            raise ValueError("save must be 'y' or 'lse'")
        shape = x.shape
        x2 = x.contiguous().reshape(-1, shape[-1])
        ctx.shape = shape
        ctx.save = save
        if save == "y":
            y = vjp_softmax_fwd(x2)
            ctx.save_for_backward(y)
        else:
            y, lse = vjp_softmax_fwd_lse(x2)
            ctx.save_for_backward(x2, lse)
        return y.reshape(shape)

    @staticmethod
    def backward(ctx, dy):
        dy2 = dy.contiguous().reshape(-1, ctx.shape[-1])
        if ctx.save == "y":
            (y,) = ctx.saved_tensors
            dx = vjp_softmax_bwd(dy2, y)
        else:
            x2, lse = ctx.saved_tensors
            dx = vjp_softmax_bwd_lse(dy2, x2, lse)
        return dx.reshape(ctx.shape), None


class SoftmaxCrossEntropy(torch.autograd.Function):
    """Mean cross-entropy of softmax(logits) over rows; targets [R] integer
    class indices (a target outside [0, C) gives a NaN loss)."""

    @staticmethod
    def forward(ctx, logits, targets):
        z = logits.contiguous()
        t = targets.contiguous()
        if t.dtype != torch.int32:
            t = t.to(torch.int32)
        out = vjp_softmax_xent_fwd(z, t, count_invalid=False)
        ctx.save_for_backward(z, t, out["row_lse"])
        return out["loss"].reshape(())

    @staticmethod
    def backward(ctx, dloss):
        z, t, lse = ctx.saved_tensors
        g = dloss.reshape(1)
        if g.dtype != torch.float32:
            g = g.float()
        dz = vjp_softmax_xent_bwd(z, t, lse, g.contiguous())
        return dz, None


class LayerNorm(torch.autograd.Function):
    """LayerNorm over the last dimension with weight w and bias b."""

    @staticmethod
    def forward(ctx, x, w, b, eps=1e-5):
        shape = x.shape
        x2 = x.contiguous().reshape(-1, shape[-1])
        w = w.contiguous()
        y, mean, rstd = vjp_layernorm_fwd(x2, w, b.contiguous(), eps)
        ctx.save_for_backward(x2, w, mean, rstd)
        ctx.shape, ctx.eps, ctx.b_dtype = shape, eps, b.dtype
        return y.reshape(shape)

    @staticmethod
    def backward(ctx, dy):
        x2, w, mean, rstd = ctx.saved_tensors
        dx, dw, db = vjp_layernorm_bwd(dy.contiguous().reshape(x2.shape), x2, w, mean, rstd, ctx.eps)
        return (dx.reshape(ctx.shape) if ctx.needs_input_grad[0] else None,
                _param_grad(dw, w) if ctx.needs_input_grad[1] else None,
                (db if ctx.b_dtype == torch.float32 else db.to(ctx.b_dtype))
                if ctx.needs_input_grad[2] else None,
                None)


class RMSNorm(torch.autograd.Function):
    """RMSNorm over the last dimension with weight w."""

    @staticmethod
    def forward(ctx, x, w, eps=1e-6):
        shape = x.shape
        x2 = x.contiguous().reshape(-1, shape[-1])
        w = w.contiguous()
        y, rstd = vjp_rmsnorm_fwd(x2, w, eps)
        ctx.save_for_backward(x2, w, rstd)
        ctx.shape, ctx.eps = shape, eps
        return y.reshape(shape)

    @staticmethod
    def backward(ctx, dy):
        x2, w, rstd = ctx.saved_tensors
        dx, dw = vjp_rmsnorm_bwd(dy.contiguous().reshape(x2.shape), x2, w, rstd, ctx.eps)
        return (dx.reshape(ctx.shape) if ctx.needs_input_grad[0] else None,
                _param_grad(dw, w) if ctx.needs_input_grad[1] else None,
                None)


class GatherRows(torch.autograd.Function):
    """y[m] = table[idx[m]] (embedding lookup); idx integer indices of any shape."""

    @staticmethod
    def forward(ctx, table, idx):
        t = table.contiguous()
        i = idx.contiguous().reshape(-1)
        if i.dtype != torch.int32:
            i = i.to(torch.int32)
        y = vjp_gather_rows_fwd(t, i)
        ctx.save_for_backward(i)
        ctx.V, ctx.dtype, ctx.out_shape = t.shape[0], t.dtype, (*idx.shape, t.shape[1])
        return y.reshape(ctx.out_shape)

    @staticmethod
    def backward(ctx, dy):
        (i,) = ctx.saved_tensors
        dt, _ = vjp_gather_rows_bwd(dy.contiguous().reshape(i.numel(), -1), i, ctx.V,
                                    count_invalid=False)
        return (dt if ctx.dtype == torch.float32 else dt.to(ctx.dtype)), None


def gather_rows(table, idx):
    return GatherRows.apply(table, idx)


def layer_norm(x, w, b, eps=1e-5):
    return LayerNorm.apply(x, w, b, eps)


def rms_norm(x, w, eps=1e-6):
    return RMSNorm.apply(x, w, eps)


def weighted_sum(x, w):
    return WeightedSum.apply(x, w)


def scaled_silu(x, w):
    return ScaledSiLU.apply(x, w)


def softmax(x, save="y"):
    return Softmax.apply(x, save)


def softmax_cross_entropy(logits, targets):
    return SoftmaxCrossEntropy.apply(logits, targets)
