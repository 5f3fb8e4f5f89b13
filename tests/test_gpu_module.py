"""The autograd module over the C-ABI: it must give exactly the library's own forward and
backward results (same kernels, same mask), and carry gradients through a synthetic
transformer block (projections, layer norm and MLP around the sparse attention)."""
import sys

import numpy as np
import pytest

import block_sparse_attention_pooled_amd as spa
from block_sparse_attention_pooled_amd import synth

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    spa.load_library()
    return torch


def test_module_matches_direct_calls(torch_gpu):
    torch = torch_gpu
    from block_sparse_attention_pooled_amd.module import SpargeAttention
    w = synth.WORKLOADS["tiny_sparse"]
    g = synth.generate(w)
    dev = {n: torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in g}
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    attn = SpargeAttention(w.k_frac, w.p, w.blk_q, w.blk_k)
    o = attn(q, k, v)
    o.backward(dev["do"])
    torch.cuda.synchronize()
    kv_idx, kv_cnt = spa.build_mask(dev["q"], dev["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
    o2, lse2, o_lo2 = spa.sparse_attn_fwd(dev["q"], dev["k"], dev["v"], kv_idx, kv_cnt, w.blk_q,
                                          w.blk_k, with_residual=True)
    dq2, dk2, dv2 = spa.sparse_attn_bwd(dev["q"], dev["k"], dev["v"], o2, dev["do"], lse2,
                                        kv_idx, kv_cnt, w.blk_q, w.blk_k, o_lo=o_lo2,
                                        grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for got, want, name in ((q.grad, dq2, "dq"), (k.grad, dk2, "dk"), (v.grad, dv2, "dv")):
        assert got.dtype == torch.bfloat16, name
        assert torch.equal(got, want), name


def test_module_in_transformer_block(torch_gpu):
    torch = torch_gpu
    from block_sparse_attention_pooled_amd.dit_block import DiTBlock
    torch.manual_seed(0)
    B, N, H, d = 1, 2048, 4, 64
    blk = DiTBlock(H * d, H, k_frac=0.1, p=0.9).cuda().to(torch.bfloat16)
    x = (torch.randn(B, N, H * d, device="cuda") * 0.5).to(torch.bfloat16).requires_grad_(True)
    y = blk(x)
    loss = y.float().pow(2).mean()
    loss.backward()
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    assert x.grad is not None and torch.isfinite(x.grad.float()).all()
    for name, prm in blk.named_parameters():
        assert prm.grad is not None and torch.isfinite(prm.grad.float()).all(), name
    assert float(blk.qkv.weight.grad.float().abs().sum()) > 0.0
    log(f"  block output rms {float(y.float().pow(2).mean().sqrt()):.4f}")
