"""A synthetic, randomly initialised video-DiT-style transformer block around the sparse
attention module, for timing the drop-in replacement in context (no weights, no data).

Block: x + Attn(LN(x)) then x + MLP(LN(x)); Attn projects to per-head Q, K, V
([B, H, N, d]), applies hybrid block-sparse attention, and projects back.  Random weights
give unstructured attention (the hybrid rule then keeps most blocks), so the timing feeds
the block the kept-block lists that the seeded video-like Q and K of the workload produce
(95 % block sparsity at the 1.3B-480p shape), and compares with the same kernels and every
block kept.

Usage:  python -m block_sparse_attention_pooled_amd.dit_block [--workload wan13b_480p]
Prints one JSON object: ms per block forward + backward, sparse and dense-mask.
"""
from __future__ import annotations

import argparse
import json
import sys

import torch

from .module import SpargeAttention


class DiTBlock(torch.nn.Module):
    def __init__(self, dim: int, heads: int, k_frac: float = 0.05, p: float = 0.9,
                 blk_q: int = 128, blk_k: int = 64, mlp_ratio: int = 4):
        super().__init__()
        self.heads, self.dh = heads, dim // heads
        self.norm1 = torch.nn.LayerNorm(dim)
        self.qkv = torch.nn.Linear(dim, 3 * dim)
        self.attn = SpargeAttention(k_frac, p, blk_q, blk_k)
        self.proj = torch.nn.Linear(dim, dim)
        self.norm2 = torch.nn.LayerNorm(dim)
        self.mlp = torch.nn.Sequential(torch.nn.Linear(dim, mlp_ratio * dim),
                                       torch.nn.GELU(approximate="tanh"),
                                       torch.nn.Linear(mlp_ratio * dim, dim))

    def forward(self, x, mask=None):
        B, N, C = x.shape
        qkv = self.qkv(self.norm1(x)).view(B, N, 3, self.heads, self.dh)
        q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3).contiguous() for i in range(3))
        a = self.attn(q, k, v, mask).permute(0, 2, 1, 3).reshape(B, N, C)
        x = x + self.proj(a)
        return x + self.mlp(self.norm2(x))


def main(argv=None):
    ap = argparse.ArgumentParser(prog="block_sparse_attention_pooled_amd.dit_block")
    ap.add_argument("--workload", default="wan13b_480p")
    ap.add_argument("--steps", type=int, default=5)
    a = ap.parse_args(argv)
    from . import synth
    if not torch.cuda.is_available():
        print("the block timing needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    from . import build_mask
    import numpy as np
    w = synth.WORKLOADS[a.workload]
    B, H, N, d = w.shape()
    g = synth.generate(w, with_do=False)
    qs, ks = (torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda()
              for n in ("q", "k"))
    masks = {"sparse": build_mask(qs, ks, w.blk_q, w.blk_k, w.k_frac, w.p),
             "dense_mask": build_mask(qs, ks, w.blk_q, w.blk_k, 1.0, 1.0)}
    del qs, ks, g
    torch.manual_seed(0)
    out = {"workload": w.name, "B": B, "N": N, "heads": H, "head_dim": d, "dim": H * d,
           "density": float(masks["sparse"][1].float().mean()) / w.n_kblk}
    for name in ("sparse", "dense_mask"):
        blk = DiTBlock(H * d, H, w.k_frac, w.p, w.blk_q, w.blk_k).cuda().to(torch.bfloat16)
        x = (torch.randn(B, N, H * d, device="cuda") * 0.5).to(torch.bfloat16)
        x.requires_grad_(True)

        def step():
            y = blk(x, masks[name])
            y.float().pow(2).mean().backward()

        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(a.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_ms_fwd_bwd"] = e0.elapsed_time(e1) / a.steps
        del blk, x
        torch.cuda.empty_cache()
    out["block_speedup"] = out["dense_mask_ms_fwd_bwd"] / out["sparse_ms_fwd_bwd"]
    print(json.dumps(out))


if __name__ == "__main__":
    main()
