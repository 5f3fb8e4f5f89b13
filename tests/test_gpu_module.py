"""The autograd module over the C-ABI: it must give exactly the library's own forward and
backward results (same kernels, same mask), and carry gradients through a synthetic
transformer block (projections, layer norm and MLP around the sparse attention)."""
import sys

import numpy as np
import pytest

import block_sparse_attention_pooled_amd as spa
from block_sparse_attention_pooled_amd import synth
from oracle import spa_oracle as O
from tests import parity

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


def _bf16_of(torch, t):
    """fp64 values of t rounded to bf16 (nearest even) on the CPU, the rounding the module
    applies on the way into the kernels."""
    bits = t.detach().cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return O.widen_bf16(bits)


@pytest.mark.parametrize("dtype_name", ["float32", "float16"])
@pytest.mark.parametrize("wname", ["tiny_sparse", "n1000_d128"])
def test_module_non_bf16_inputs_match_oracle(torch_gpu, dtype_name, wname):
    """fp32 and fp16 inputs through the autograd module: the oracle runs on the inputs and
    the output gradient rounded to bf16, under the module's own mask.  O, dQ, dK and dV
    (returned in the input dtype) must match element by element within max-abs 2e-2 and
    relative L2 1e-2; an fp16 gradient may add its own rounding (half an fp16 ulp of the
    reference value, 2^-11 relative) to the max-abs bound."""
    torch = torch_gpu
    from block_sparse_attention_pooled_amd.module import SpargeAttention
    dtype = getattr(torch, dtype_name)
    w = (synth.WORKLOADS["tiny_sparse"] if wname == "tiny_sparse" else
         synth.Workload("n1000_d128", 1, 2, 1000, 128, 128, 64, 0.1, 0.9, kind="video",
                        grid=(2, 20, 25), alpha=synth.ALPHA_480P, n_sinks=2, seed=5))
    g = synth.generate(w)
    rng = np.random.default_rng(17)
    # values between bf16 grid points, so that the module's rounding is exercised
    x = {n: torch.from_numpy((synth.bf16_bits_to_f32(g[n]).astype(np.float64) *
                              (1.0 + 2.0 ** -9 * rng.uniform(-1, 1, g[n].shape)))
                             .astype(np.float32)).to(dtype).cuda() for n in ("q", "k", "v", "do")}
    q, k, v = (x[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    attn = SpargeAttention(w.k_frac, w.p, w.blk_q, w.blk_k)
    attn.keep_mask = True
    o = attn(q, k, v)
    o.backward(x["do"])
    torch.cuda.synchronize()
    assert o.dtype == dtype and all(t.grad.dtype == dtype for t in (q, k, v))
    kv_idx, kv_cnt = attn.last_mask
    lists = parity.lists_from_gpu(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy())
    f = {n: _bf16_of(torch, x[n]) for n in x}
    log(f"[module {dtype_name} {wname}] density "
        f"{float(kv_cnt.float().mean()) / -(-w.N // w.blk_k):.3f}")
    ro, _ = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, w.blk_q, w.blk_k)
    rq, rk, rv = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, w.blk_q, w.blk_k)
    for name, got, want in (("O", o, ro), ("dQ", q.grad, rq), ("dK", k.grad, rk),
                            ("dV", v.grad, rv)):
        gotn = got.detach().float().cpu().numpy().astype(np.float64)
        ok, mx, rel, _ = parity.close(gotn, want, atol=np.inf)
        lim = parity.ATOL + (2.0 ** -11 * np.abs(want) if dtype == torch.float16 and name != "O"
                             else 0.0)
        over = float(np.max(np.abs(gotn - want) - lim))
        log(f"  {name}: max_abs={mx:.3e} rel_l2={rel:.3e}")
        assert ok and over <= 0.0, (name, mx, rel)
