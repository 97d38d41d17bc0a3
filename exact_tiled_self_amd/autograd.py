"""attn_fwd and attn_bwd as one differentiable torch operation.

The forward keeps only o and the per-row lse beside the inputs; the backward
recomputes the attention weights from q, k and lse instead of storing the
N x N matrix ("Autoatención, kernels CUDA y FlashAttention", section 3,
"Recálculo durante la retropropagación").  Both directions run in the HIP
library; this module only connects them to torch's autograd.  Gradients
need bfloat16 inputs (the backward entry point supports bf16 only).
"""

from __future__ import annotations

import torch

from . import _lib


class ExactAttention(torch.autograd.Function):
    """o = softmax(scale * q k^T [causal mask]) v per head, with grouped K/V
    heads; q [B, Hq, N, d], k and v [B, Hkv, N, d]."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        o, lse = _lib.attn_fwd(q, k, v, scale=scale, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal = scale, causal
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _lib.attn_bwd(q, k, v, o, lse, dout.contiguous(), scale=ctx.scale, causal=ctx.causal)
        return dq, dk, dv, None, None


def attention(q, k, v, scale=None, causal=False):
    """Differentiable exact attention; scale defaults to 1/sqrt(d)."""
    return ExactAttention.apply(q, k, v, scale, causal)
