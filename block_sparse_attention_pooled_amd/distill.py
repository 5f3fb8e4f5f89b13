"""Velocity-distillation step on a toy, randomly initialised video DiT (SpargeAttention2
pages, mindverse article, section "Velocity Distillation Loss"; the adaptation itself in
"Effiziente Kernel-Implementierung und Modellanpassung").

A frozen teacher with full attention and a student whose attention layers are the hybrid
block-sparse module see the same noisy latent; the student is trained to reproduce the
teacher's velocity prediction instead of a data-driven diffusion target.  Everything here
is synthetic (random weights, smooth random latents): it exercises the step's mechanics
(the loss, the sparse backward through every attention layer, one optimiser update), not
generation quality.

Readings (the pages give no formulas): the noisy input is the flow-matching interpolation
x_t = (1 - t) x_0 + t eps with t ~ U(0, 1) and eps ~ N(0, I); the model maps (x_t, t) to a
velocity of x_t's shape; the loss is the mean squared difference between the student's and
the teacher's velocities.  The teacher's full attention runs through the same kernels with
every block kept (k = p = 1), which is exact full attention.

Usage:  python -m block_sparse_attention_pooled_amd.distill [--grid T H W] [--dim C]
        [--heads H] [--depth L] [--k K] [--p P] [--steps S] [--autocast] [--frac F]
        [--adamw-lr LR]
The defaults are the toy the tests train; a large-shape timing run, e.g. one block at the
1.3B-480p attention shape, is
    --grid 21 30 52 --dim 1536 --heads 12 --depth 1 --k 0.05 --autocast --frac 0
Prints one JSON object: loss per step, mask density, ms per distillation step.
"""
from __future__ import annotations

import argparse
import copy
import json
import math
import sys

import torch

from .dit_block import DiTBlock


def timestep_features(t, dim: int):
    """Sinusoidal features of t (scaled to [0, 1000]), [B] -> [B, dim] fp32."""
    half = dim // 2
    freq = torch.exp(-math.log(10000.0) * torch.arange(half, device=t.device,
                                                       dtype=torch.float32) / half)
    a = (t.float() * 1000.0)[:, None] * freq[None, :]
    return torch.cat([torch.cos(a), torch.sin(a)], dim=1)


def positional_embedding_3d(grid, dim: int):
    """Fixed sinusoidal embedding of (frame, row, column) -> [T*H*W, dim] fp32: each axis
    gets a third of the channels as cos/sin pairs at geometric frequencies (periods from 2
    positions up to 4x the axis length); channels left over stay zero."""
    T, H, W = grid
    per = (dim // 3) // 2
    coords = torch.stack(torch.meshgrid(torch.arange(T), torch.arange(H), torch.arange(W),
                                        indexing="ij"), dim=-1).reshape(-1, 3).float()
    out = torch.zeros(T * H * W, dim)
    for a, n in enumerate((T, H, W)):
        periods = 2.0 * (2.0 * n) ** (torch.arange(per).float() / max(1, per - 1))
        ang = 2.0 * math.pi * coords[:, a:a + 1] / periods[None, :]
        out[:, 2 * per * a:2 * per * a + per] = torch.cos(ang)
        out[:, 2 * per * a + per:2 * per * (a + 1)] = torch.sin(ang)
    return out


class ToyVideoDiT(torch.nn.Module):
    """Latent tokens [B, N, c_in] on a (T, H, W) grid -> velocity [B, N, c_in]: linear patch
    embedding plus a fixed 3-D positional embedding and a timestep embedding, ``depth`` DiT
    blocks with the sparse attention module, and a normalised linear head."""

    def __init__(self, c_in: int, dim: int, heads: int, depth: int, grid, k_frac: float = 0.05,
                 p: float = 0.9, blk_q: int = 128, blk_k: int = 64):
        super().__init__()
        self.dim = dim
        self.register_buffer("pos", positional_embedding_3d(grid, dim), persistent=False)
        self.embed = torch.nn.Linear(c_in, dim)
        self.t_mlp = torch.nn.Sequential(torch.nn.Linear(dim, dim), torch.nn.SiLU(),
                                         torch.nn.Linear(dim, dim))
        self.blocks = torch.nn.ModuleList(DiTBlock(dim, heads, k_frac, p, blk_q, blk_k)
                                          for _ in range(depth))
        self.norm = torch.nn.LayerNorm(dim)
        self.head = torch.nn.Linear(dim, c_in)

    def set_rule(self, k_frac: float, p: float):
        for b in self.blocks:
            b.attn.k_frac, b.attn.p = float(k_frac), float(p)

    def attention_layers(self):
        return [b.attn for b in self.blocks]

    def forward(self, x, t):
        temb = self.t_mlp(timestep_features(t, self.dim).to(self.embed.weight.dtype))
        h = self.embed(x) + self.pos.to(temb.dtype)[None] + temb[:, None, :]
        for b in self.blocks:
            h = b(h)
        return self.head(self.norm(h))


def local_attention_init(model: ToyVideoDiT, qk_gain: float):
    """Give the random model the local attention that trained video DiTs show: the key
    projection starts equal to the query projection (scaled by ``qk_gain``, no biases), so
    a token's logits follow its similarity to other tokens, which the smooth latents and
    the positional embedding make local in (frame, row, column).  With independent random
    projections the attention is unstructured and the hybrid rule keeps ~90 % of blocks."""
    with torch.no_grad():
        for b in model.blocks:
            dim = b.qkv.in_features
            w, bias = b.qkv.weight, b.qkv.bias
            w[:dim] *= qk_gain
            w[dim:2 * dim] = w[:dim]
            bias[:2 * dim] = 0.0


def make_pair(c_in: int, dim: int, heads: int, depth: int, grid, k_frac: float, p: float,
              blk_q: int = 128, blk_k: int = 64, qk_gain: float = 3.0, seed: int = 0,
              device="cuda", dtype=torch.float32):
    """(teacher, student): the teacher keeps every block (full attention) and is frozen; the
    student starts from the teacher's weights with the hybrid rule (k_frac, p).  Weights are
    fp32 masters; the steps below run the forward under bf16 autocast."""
    torch.manual_seed(seed)
    teacher = ToyVideoDiT(c_in, dim, heads, depth, grid, 1.0, 1.0, blk_q, blk_k)
    local_attention_init(teacher, qk_gain)
    teacher = teacher.to(device=device, dtype=dtype).eval()
    for prm in teacher.parameters():
        prm.requires_grad_(False)
    student = copy.deepcopy(teacher).train()
    for prm in student.parameters():
        prm.requires_grad_(True)
    student.set_rule(k_frac, p)
    return teacher, student


def smooth_latents(B: int, grid, c_in: int, seed: int, device="cuda", dtype=torch.float32):
    """Synthetic video latents [B, T*H*W, c_in]: coarse Gaussian noise on a (T/2, H/4, W/4)
    grid, trilinearly upsampled, plus a little white noise (neighbouring tokens alike, as
    in video latents), normalised to unit variance."""
    T, H, W = grid
    g = torch.Generator(device="cpu").manual_seed(seed)
    coarse = torch.randn(B, c_in, max(1, T // 2), max(1, H // 4), max(1, W // 4), generator=g)
    x = torch.nn.functional.interpolate(coarse, size=(T, H, W), mode="trilinear",
                                        align_corners=True)
    x = x + 0.1 * torch.randn(x.shape, generator=g)
    x = (x - x.mean()) / x.std()
    return x.flatten(2).transpose(1, 2).contiguous().to(device=device, dtype=dtype)


def noisy_input(x0, seed: int):
    """(x_t, t) with x_t = (1 - t) x0 + t eps, t ~ U(0, 1) per sample."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    B = x0.shape[0]
    t = torch.rand(B, generator=g)
    eps = torch.randn(x0.shape, generator=g)
    tt = t.view(B, 1, 1)
    xt = (1.0 - tt) * x0.float().cpu() + tt * eps
    return xt.to(device=x0.device, dtype=x0.dtype), t.to(x0.device)


def velocity_distillation_loss(student, teacher, xt, t, autocast: bool = True):
    """Mean squared difference of the student's and the frozen teacher's velocities, in fp32.
    With ``autocast`` the forwards run under bf16 autocast (mixed-precision training);
    without it the projections and MLPs stay fp32 and only the attention kernels compute in
    bf16."""
    with torch.autocast(device_type="cuda", dtype=torch.bfloat16, enabled=autocast):
        with torch.no_grad():
            v_teacher = teacher(xt, t)
        v_student = student(xt, t)
    return torch.mean((v_student.float() - v_teacher.float()) ** 2)


def grad_sq_norm(params) -> float:
    """|g|^2 over the parameters' current gradients."""
    return sum(float(p.grad.float().pow(2).sum()) for p in params if p.grad is not None)


def first_order_lr(loss_value: float, g2: float, frac: float) -> float:
    """Learning rate whose plain gradient step lowers the loss, to first order, by ``frac``
    of its value: lr * |g|^2 = frac * L."""
    return frac * loss_value / max(g2, 1e-30)


def distill_step(student, teacher, xt, t, opt, autocast: bool = True) -> float:
    """One optimiser update of the student on the velocity-distillation loss.  Returns the
    loss before the update."""
    opt.zero_grad(set_to_none=True)
    loss = velocity_distillation_loss(student, teacher, xt, t, autocast)
    loss.backward()
    opt.step()
    return float(loss.detach())


def main(argv=None):
    ap = argparse.ArgumentParser(prog="block_sparse_attention_pooled_amd.distill")
    ap.add_argument("--grid", type=int, nargs=3, default=[4, 16, 32], metavar=("T", "H", "W"))
    ap.add_argument("--c-in", type=int, default=16)
    ap.add_argument("--dim", type=int, default=256)
    ap.add_argument("--heads", type=int, default=4)
    ap.add_argument("--depth", type=int, default=2)
    ap.add_argument("--k", type=float, default=0.10)
    ap.add_argument("--p", type=float, default=0.9)
    ap.add_argument("--adamw-lr", type=float, default=0.0,
                    help="AdamW with this learning rate instead of plain gradient descent")
    ap.add_argument("--frac", type=float, default=0.05,
                    help="gradient descent: first-order loss decrease of the first step "
                         "(0 times the step with a zero learning rate)")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--qk-gain", type=float, default=3.0)
    ap.add_argument("--autocast", action="store_true",
                    help="bf16 autocast for projections and MLPs (default fp32; the attention "
                         "kernels compute in bf16 either way)")
    a = ap.parse_args(argv)
    ac = a.autocast
    if not torch.cuda.is_available():
        print("the distillation step needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    teacher, student = make_pair(a.c_in, a.dim, a.heads, a.depth, a.grid, a.k, a.p,
                                 qk_gain=a.qk_gain)
    x0 = smooth_latents(1, a.grid, a.c_in, seed=1)
    xt, t = noisy_input(x0, seed=2)
    for layer in student.attention_layers():
        layer.keep_mask = True
    loss = velocity_distillation_loss(student, teacher, xt, t, ac)
    loss.backward()
    lr = first_order_lr(float(loss.detach()), grad_sq_norm(student.parameters()), a.frac)
    opt = (torch.optim.AdamW(student.parameters(), lr=a.adamw_lr, weight_decay=0.0)
           if a.adamw_lr > 0 else torch.optim.SGD(student.parameters(), lr=lr))
    losses = [distill_step(student, teacher, xt, t, opt, ac)]
    N = x0.shape[1]
    nkb = (N + 63) // 64
    dens = [float(m[1].float().mean()) / nkb for m in
            (layer.last_mask for layer in student.attention_layers())]
    for layer in student.attention_layers():
        layer.keep_mask = False
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(a.steps):
        losses.append(distill_step(student, teacher, xt, t, opt, ac))
    e1.record()
    torch.cuda.synchronize()
    print(json.dumps({"grid": a.grid, "N": N, "dim": a.dim, "heads": a.heads,
                      "depth": a.depth, "k": a.k, "p": a.p, "autocast_bf16": ac,
                      "optimizer": "adamw" if a.adamw_lr > 0 else "sgd",
                      "density_per_layer": dens,
                      "loss": losses, "ms_per_step": e0.elapsed_time(e1) / a.steps}))


if __name__ == "__main__":
    main()
