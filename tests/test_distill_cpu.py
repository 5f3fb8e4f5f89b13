"""The distillation step's mechanics in fp32 on the CPU, independent of the GPU kernels:
the toy teacher with full softmax attention, the student with attention restricted to the
oracle's hybrid mask (recomputed from each forward's Q and K, as the sparse module does).

Pins for the GPU test of the same step: the student's initial loss, the first-order
accuracy of a gradient step (a 1 % predicted decrease is realised to within a few percent)
and monotone descent at the fixed learning rate of a 5 % first step.
"""
import copy

import pytest
import torch

from block_sparse_attention_pooled_amd import distill as D
from oracle import spa_oracle as O

GRID = (4, 16, 32)
C_IN, DIM, HEADS, DEPTH = 16, 256, 4, 2


class OracleMaskedAttention(torch.nn.Module):
    def __init__(self, k_frac, p):
        super().__init__()
        self.k_frac, self.p = k_frac, p

    def forward(self, q, k, v, mask=None):
        B, H, N, d = q.shape
        s = torch.matmul(q, k.transpose(-1, -2)) * d ** -0.5
        if self.k_frac < 1.0:
            m = O.build_mask(q.detach().double().numpy(), k.detach().double().numpy(), 128, 64,
                             self.k_frac, self.p)
            keep = torch.zeros(B, H, N, N, dtype=torch.bool)
            for (b, h), rows in m["rows"].items():
                for i, r in enumerate(rows):
                    for j in r["keep"]:
                        keep[b, h, i * 128:(i + 1) * 128, j * 64:(j + 1) * 64] = True
            s = s.masked_fill(~keep, float("-inf"))
        return torch.matmul(torch.softmax(s, dim=-1), v)


@pytest.fixture(scope="module")
def pair():
    torch.manual_seed(0)
    teacher = D.ToyVideoDiT(C_IN, DIM, HEADS, DEPTH, GRID, 1.0, 1.0)
    D.local_attention_init(teacher, 3.0)
    for b in teacher.blocks:
        b.attn = OracleMaskedAttention(1.0, 1.0)
    for prm in teacher.parameters():
        prm.requires_grad_(False)
    student = copy.deepcopy(teacher)
    for b in student.blocks:
        b.attn = OracleMaskedAttention(0.10, 0.9)
    for prm in student.parameters():
        prm.requires_grad_(True)
    x0 = D.smooth_latents(1, GRID, C_IN, seed=1, device="cpu")
    xt, t = D.noisy_input(x0, seed=2)
    return teacher, student, xt, t


def _loss(student, teacher, xt, t):
    with torch.no_grad():
        vt = teacher(xt, t)
    return torch.mean((student(xt, t) - vt) ** 2)


def test_full_rule_gives_zero_loss(pair):
    teacher, _, xt, t = pair
    same = copy.deepcopy(teacher)
    assert float(_loss(same, teacher, xt, t)) == 0.0


def test_gradient_step_first_order_and_descent(pair):
    teacher, student, xt, t = pair
    student = copy.deepcopy(student)
    opt = torch.optim.SGD(student.parameters(), lr=1.0)
    loss = _loss(student, teacher, xt, t)
    loss.backward()
    l0, g2 = float(loss.detach()), D.grad_sq_norm(student.parameters())
    assert 1e-5 < l0 < 1e-3
    opt.param_groups[0]["lr"] = D.first_order_lr(l0, g2, 0.01)
    opt.step()
    opt.param_groups[0]["lr"] = D.first_order_lr(l0, g2, 0.05)
    losses = []
    for _ in range(4):
        opt.zero_grad(set_to_none=True)
        loss = _loss(student, teacher, xt, t)
        loss.backward()
        losses.append(float(loss.detach()))
        opt.step()
    ratio = (l0 - losses[0]) / (0.01 * l0)
    assert 0.9 < ratio < 1.1, ratio
    assert all(b < a for a, b in zip(losses, losses[1:])), losses
