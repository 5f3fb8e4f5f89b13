"""Drop-in attention module over the C-ABI (the deployment the SpargeAttention2 pages
describe: every attention layer of the video DiT replaced by the sparse one; mindverse
article, section "Effiziente Kernel-Implementierung und Modellanpassung").

``SparseAttentionFunction`` builds the hybrid Top-k + Top-p mask from Q and K, runs the
sparse forward with the residual output the backward needs, and saves the kept-block lists
so that the backward pass uses the same mask (the mask is held fixed: no gradient flows
through the selection).  ``SpargeAttention`` is the ``nn.Module`` around it.

Tensors are [B, H, N, d] on a ROCm device.  The kernels compute in bf16: other input
dtypes (fp32 master activations, fp16) are rounded to bf16 (nearest even) on the way in,
and so is the incoming output gradient; the output comes back in q's dtype.  The kernels
write the gradients in fp32, or directly in bf16 when every input is bf16; each gradient
is returned in its input's dtype.  Every step runs in the library's kernels; this file only
marshals arguments.
"""
from __future__ import annotations

import torch

from . import build_mask, sparse_attn_bwd, sparse_attn_fwd


class SparseAttentionFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, k_frac: float, p: float, blk_q: int, blk_k: int, scale,
                pooled_scale, mask=None):
        ctx.in_dtypes = (q.dtype, k.dtype, v.dtype)
        ctx.out_dtype = q.dtype
        q, k, v = (t.to(torch.bfloat16).contiguous() for t in (q, k, v))
        if mask is None:
            kv_idx, kv_cnt = build_mask(q, k, blk_q, blk_k, k_frac, p,
                                        pooled_scale=pooled_scale)
        else:  # kept-block lists supplied by the caller (e.g. one mask shared by layers)
            kv_idx, kv_cnt = mask
        o, lse, o_lo = sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, blk_q, blk_k, scale,
                                       with_residual=True)
        ctx.save_for_backward(q, k, v, o, o_lo, lse, kv_idx, kv_cnt)
        ctx.cfg = (blk_q, blk_k, scale)
        return o.to(ctx.out_dtype)

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, o_lo, lse, kv_idx, kv_cnt = ctx.saved_tensors
        blk_q, blk_k, scale = ctx.cfg
        # fp32 gradients cost the kernels nothing extra: bf16 only when every input is bf16
        gdt = (torch.bfloat16 if all(dt == torch.bfloat16 for dt in ctx.in_dtypes)
               else torch.float32)
        dq, dk, dv = sparse_attn_bwd(q, k, v, o, do.contiguous().to(torch.bfloat16), lse,
                                     kv_idx, kv_cnt, blk_q, blk_k, scale, o_lo=o_lo,
                                     grad_dtype=gdt)
        dq, dk, dv = (g.to(dt) for g, dt in zip((dq, dk, dv), ctx.in_dtypes))
        return dq, dk, dv, None, None, None, None, None, None, None


def sparse_attention(q, k, v, k_frac: float = 0.05, p: float = 0.9, blk_q: int = 128,
                     blk_k: int = 64, scale: float | None = None,
                     pooled_scale: float | None = None, mask=None):
    """Hybrid Top-k + Top-p block-sparse attention with autograd support.  ``mask`` may
    supply (kv_idx, kv_cnt) from an earlier build_mask instead of building it here."""
    return SparseAttentionFunction.apply(q, k, v, float(k_frac), float(p), int(blk_q),
                                         int(blk_k), scale, pooled_scale, mask)


class SpargeAttention(torch.nn.Module):
    """Drop-in attention layer: ``forward(q, k, v)`` with [B, H, N, d] tensors.

    With ``keep_mask = True`` the kept-block lists of the last call stay in ``last_mask``
    (for inspection, or to rerun the same mask elsewhere)."""

    def __init__(self, k_frac: float = 0.05, p: float = 0.9, blk_q: int = 128,
                 blk_k: int = 64, scale: float | None = None,
                 pooled_scale: float | None = None):
        super().__init__()
        self.k_frac, self.p = float(k_frac), float(p)
        self.blk_q, self.blk_k = int(blk_q), int(blk_k)
        self.scale, self.pooled_scale = scale, pooled_scale
        self.keep_mask = False
        self.last_mask = None

    def forward(self, q, k, v, mask=None):
        if mask is None and self.keep_mask:
            mask = build_mask(q.detach().to(torch.bfloat16).contiguous(),
                              k.detach().to(torch.bfloat16).contiguous(), self.blk_q,
                              self.blk_k, self.k_frac, self.p, pooled_scale=self.pooled_scale)
        if self.keep_mask:
            self.last_mask = mask
        return sparse_attention(q, k, v, self.k_frac, self.p, self.blk_q, self.blk_k,
                                self.scale, self.pooled_scale, mask)

    def extra_repr(self) -> str:
        return (f"k_frac={self.k_frac}, p={self.p}, blocks={self.blk_q}x{self.blk_k}")
