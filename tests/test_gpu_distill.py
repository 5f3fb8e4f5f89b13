"""Velocity-distillation step mechanics on a toy random-init video DiT: a frozen teacher
with full attention, a student with the hybrid sparse module in every attention layer.

- With the full rule (k = p = 1) the student computes exactly what the teacher computes:
  loss 0 and zero gradients.
- The student's parameter gradients through the sparse backward match those of the same
  student with each attention layer replaced by a plain fp32 masked softmax over the same
  kept blocks, for the same upstream gradient.
- A few optimiser steps lower the loss, change the student and leave the teacher alone.
"""
import copy
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

GRID = (4, 16, 32)  # N = 2048 tokens: 16 query blocks, 32 key blocks
C_IN, DIM, HEADS, DEPTH = 16, 256, 4, 2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    import block_sparse_attention_pooled_amd as spa
    spa.load_library()
    return torch


def _inputs(torch):
    from block_sparse_attention_pooled_amd import distill as D
    x0 = D.smooth_latents(1, GRID, C_IN, seed=1)
    return D.noisy_input(x0, seed=2)


class MaskedDenseAttention(torch.nn.Module):
    """fp32 softmax(Q K^T / sqrt(d)) V with the kept-block lists expanded to a dense
    boolean mask; output cast back to the input dtype."""

    def __init__(self, mask, blk_q, blk_k, N):
        super().__init__()
        kv_idx, kv_cnt = mask
        B, H, nqb, nkb = kv_idx.shape
        pos = torch.arange(nkb, device=kv_idx.device)
        valid = pos[None, None, None, :] < kv_cnt[..., None]
        idx = torch.where(valid, kv_idx.long(), torch.full_like(kv_idx.long(), nkb))
        blocks = torch.zeros(B, H, nqb, nkb + 1, dtype=torch.bool, device=kv_idx.device)
        blocks.scatter_(3, idx, torch.ones_like(valid))
        blocks = blocks[..., :nkb]
        self.dense = (blocks.repeat_interleave(blk_q, dim=2)[:, :, :N]
                      .repeat_interleave(blk_k, dim=3)[..., :N])

    def forward(self, q, k, v, mask=None):
        with torch.autocast(device_type="cuda", enabled=False):
            qf, kf, vf = q.float(), k.float(), v.float()
            s = torch.matmul(qf, kf.transpose(-1, -2).contiguous()) * q.shape[-1] ** -0.5
            s = s.masked_fill(~self.dense, float("-inf"))
            return torch.matmul(torch.softmax(s, dim=-1), vf).to(q.dtype)


def test_full_rule_student_equals_teacher(torch_gpu):
    torch = torch_gpu
    from block_sparse_attention_pooled_amd import distill as D
    teacher, student = D.make_pair(C_IN, DIM, HEADS, DEPTH, GRID, 1.0, 1.0)
    xt, t = _inputs(torch)
    loss = D.velocity_distillation_loss(student, teacher, xt, t)
    loss.backward()
    torch.cuda.synchronize()
    assert float(loss) == 0.0
    for name, prm in student.named_parameters():
        assert prm.grad is not None and not bool(prm.grad.any()), name
    assert all(prm.grad is None for prm in teacher.parameters())


def test_student_gradients_match_fp32_masked_attention(torch_gpu):
    torch = torch_gpu
    from block_sparse_attention_pooled_amd import distill as D
    teacher, student = D.make_pair(C_IN, DIM, HEADS, DEPTH, GRID, 0.10, 0.9)
    xt, t = _inputs(torch)
    N = xt.shape[1]
    for layer in student.attention_layers():
        layer.keep_mask = True
    with torch.autocast(device_type="cuda", dtype=torch.bfloat16):
        with torch.no_grad():
            v_t = teacher(xt, t).float()
        v_s = student(xt, t)
    # the distillation loss's upstream gradient, fixed from this run for both students
    g = (2.0 * (v_s.detach().float() - v_t) / v_t.numel())
    v_s.float().backward(g)
    masks = [layer.last_mask for layer in student.attention_layers()]
    nkb = (N + 63) // 64
    dens = [float(m[1].float().mean()) / nkb for m in masks]
    log(f"  student mask density per layer {[round(x, 3) for x in dens]}")
    assert all(x < 0.5 for x in dens)

    ref = copy.deepcopy(student)
    for blk, m in zip(ref.blocks, masks):
        blk.attn = MaskedDenseAttention(m, 128, 64, N)
    ref.zero_grad(set_to_none=True)
    with torch.autocast(device_type="cuda", dtype=torch.bfloat16):
        v_r = ref(xt, t)
    v_r.float().backward(g)
    torch.cuda.synchronize()
    out_rel = float((v_s.float() - v_r.float()).norm() / v_r.float().norm())
    log(f"  student output vs fp32-attention student: rel-L2 {out_rel:.2e}")
    assert out_rel < 1e-2
    worst = 0.0
    for (name, a), (_, b) in zip(student.named_parameters(), ref.named_parameters()):
        ga, gb = a.grad.float(), b.grad.float()
        rel = float((ga - gb).norm() / gb.norm().clamp_min(1e-30))
        worst = max(worst, rel)
        assert rel < 2e-2, (name, rel)
    log(f"  worst parameter-gradient rel-L2 {worst:.2e}")


def test_distill_steps_reduce_loss_and_leave_teacher(torch_gpu):
    """Gradient steps sized for a first-order loss decrease of a given fraction of the loss,
    with the projections in fp32 (under bf16 autocast the steps would be quantised by the
    bf16 copies of the weights).  A 1 % step must decrease the loss by about what the
    gradient predicts (the gradient is the loss's own slope; an fp32 CPU emulation with the
    oracle's mask measures 0.97 of the prediction there, 0.83 at 5 % where curvature sets
    in); further steps at the fixed learning rate of a 5 % first step must lower the loss
    every time; the teacher must not move."""
    torch = torch_gpu
    from block_sparse_attention_pooled_amd import distill as D
    teacher, student = D.make_pair(C_IN, DIM, HEADS, DEPTH, GRID, 0.10, 0.9)
    xt, t = _inputs(torch)
    t_before = {n: p.detach().clone() for n, p in teacher.named_parameters()}
    s_before = {n: p.detach().clone() for n, p in student.named_parameters()}
    opt = torch.optim.SGD(student.parameters(), lr=1.0)
    loss = D.velocity_distillation_loss(student, teacher, xt, t, False)
    loss.backward()
    l0, g2 = float(loss), D.grad_sq_norm(student.parameters())
    opt.param_groups[0]["lr"] = D.first_order_lr(l0, g2, 0.01)
    opt.step()
    opt.param_groups[0]["lr"] = D.first_order_lr(l0, g2, 0.05)
    losses = [D.distill_step(student, teacher, xt, t, opt, autocast=False) for _ in range(8)]
    losses.append(float(D.velocity_distillation_loss(student, teacher, xt, t, False)))
    torch.cuda.synchronize()
    ratio = (l0 - losses[0]) / (0.01 * l0)
    log(f"  1 % step: measured / first-order predicted decrease {ratio:.3f}")
    log(f"  losses {[f'{x:.3e}' for x in [l0] + losses]}")
    assert all(torch.isfinite(torch.tensor(losses)))
    assert l0 > 0.0
    assert 0.7 < ratio < 1.3
    assert all(b < a for a, b in zip(losses, losses[1:]))
    assert losses[-1] < 0.9 * losses[0]
    for n, p in teacher.named_parameters():
        assert torch.equal(p, t_before[n]), n
    changed = sum(not torch.equal(p, s_before[n]) for n, p in student.named_parameters())
    assert changed == len(s_before)


class _Recorder(torch.nn.Module):
    """Wraps an attention layer and keeps its inputs and output (with their gradients after
    the backward pass) and the kept-block lists it used."""

    def __init__(self, inner):
        super().__init__()
        self.inner = inner
        self.inner.keep_mask = True
        self.rec = None

    def forward(self, q, k, v, mask=None):
        for t in (q, k, v):
            t.retain_grad()
        o = self.inner(q, k, v, mask)
        o.retain_grad()
        self.rec = dict(q=q, k=k, v=v, o=o, mask=self.inner.last_mask)
        return o


@pytest.mark.parametrize("autocast", [False, True], ids=["fp32", "bf16_autocast"])
def test_student_attention_layers_match_oracle(torch_gpu, autocast):
    """Every sparse attention layer of the student, inside the distillation step: its output
    and the gradients it hands back for its Q, K and V, element by element against the fp64
    oracle on the layer's own inputs and output gradient (rounded to bf16 as the layer
    rounds them), under the layer's own mask.  Without autocast the layer takes fp32
    activations and returns fp32 gradients; under bf16 autocast it takes bf16.  The loss's
    output gradient is ~1e-6, far below the absolute tolerance, and the gradients are linear
    in it, so each gradient is compared after dividing both sides by the reference's
    largest magnitude: the bounds then apply at unit scale and the relative bound always
    applies."""
    torch = torch_gpu
    from block_sparse_attention_pooled_amd import distill as D
    from oracle import spa_oracle as O
    from tests import parity
    teacher, student = D.make_pair(C_IN, DIM, HEADS, DEPTH, GRID, 0.10, 0.9)
    recs = []
    for blk in student.blocks:
        blk.attn = _Recorder(blk.attn)
        recs.append(blk.attn)
    xt, t = _inputs(torch)
    loss = D.velocity_distillation_loss(student, teacher, xt, t, autocast)
    loss.backward()
    torch.cuda.synchronize()

    def bf16_f64(x):
        b = x.detach().cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return O.widen_bf16(b)

    for li, layer in enumerate(recs):
        r = layer.rec
        want_dt = torch.bfloat16 if autocast else torch.float32
        assert r["q"].dtype == want_dt and r["q"].grad.dtype == want_dt
        B, H, N, d = r["q"].shape
        kv_idx, kv_cnt = r["mask"]
        lists = parity.lists_from_gpu(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy())
        f = {n: bf16_f64(r[n]) for n in ("q", "k", "v")}
        f["do"] = bf16_f64(r["o"].grad)
        ro, _ = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, 128, 64)
        rq, rk, rv = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, 128, 64)
        log(f"[distill layer {li} {'bf16' if autocast else 'fp32'}] shape {(B, H, N, d)} "
            f"density {float(kv_cnt.float().mean()) / -(-N // 64):.3f} "
            f"|dO|max {float(np.abs(f['do']).max()):.2e}")
        for name, got, want in (("O", r["o"], ro), ("dQ", r["q"].grad, rq),
                                ("dK", r["k"].grad, rk), ("dV", r["v"].grad, rv)):
            gotn = got.detach().float().cpu().numpy().astype(np.float64)
            s = 1.0 if name == "O" else float(np.abs(want).max())
            assert s > 0.0, (li, name)
            ok, mx, rel, _ = parity.close(gotn / s, want / s, vacuous=0.0)
            log(f"  {name}: max_abs={mx:.3e} (after / {s:.2e}) rel_l2={rel:.3e}")
            assert ok, (li, name, mx, rel)
