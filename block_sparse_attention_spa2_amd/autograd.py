"""torch.autograd glue: block-sparse attention as a differentiable op.

The forward runs spa2_fwd and keeps O, LSE and the unrounded O; the backward runs
spa2_bwd with the same mask. The mask itself carries no gradient (the pages' masks are
hard selections made from pooled Q and K; rainbus summary, "方法步骤详情", steps 2-4).
"""
from __future__ import annotations

import torch

from . import BlockMask, bwd, fwd, mask


class _SparseAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, bm, bq, bkv):
        o_f32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o, lse = fwd(q, k, v, bm, bq, bkv, o_f32=o_f32)
        ctx.save_for_backward(q, k, v, o, lse, o_f32)
        ctx.bm, ctx.bq, ctx.bkv = bm, bq, bkv
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, o_f32 = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), ctx.bm, ctx.bq, ctx.bkv, o_f32=o_f32)
        return dq, dk, dv, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bm: BlockMask | None,
              bq: int = 128, bkv: int = 64) -> torch.Tensor:
    """Differentiable attention over the kept blocks of bm (bm = None: dense). q, k, v:
    contiguous [B, H, N, D] on the GPU, float32 or bfloat16."""
    if bm is not None:
        bq, bkv = bm.bq, bm.bkv
    return _SparseAttention.apply(q.contiguous(), k.contiguous(), v.contiguous(), bm, bq, bkv)


def sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_frac: float,
                     p_frac: float, bq: int = 128, bkv: int = 64):
    """The method's layer: hybrid Top-k U Top-p mask from (detached) Q and K, then
    attention over the kept blocks. Returns (O, BlockMask)."""
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    with torch.no_grad():
        bm = mask(q.detach(), k.detach(), k_frac, p_frac, bq, bkv)
    return attention(q, k, v, bm), bm
