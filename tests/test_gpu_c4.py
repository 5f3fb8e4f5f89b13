"""GPU parity at the Wan2.1-14B-720p layer shape (B=1, H=40, N=75600, d=128, blocks 128 x 64,
k=5 %, p=0.9), in the launch configuration the benchmark uses.

The oracle runs on sampled heads (mask: every row of the head), sampled query blocks
(O, LSE, dQ) and sampled key blocks (dK, dV); each check widens only the head it needs.
Sampled blocks include the partial last query block (80 rows) and the partial last key
block (16 keys).
"""
import sys

import numpy as np
import pytest

import block_sparse_attention_pooled_amd as spa
from block_sparse_attention_pooled_amd import synth
from oracle import spa_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["wan14b_720p"]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def c4():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    log(f"[c4] generating {W.name} {W.shape()}")
    g = synth.generate(W)
    dev = {n: torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in g}
    log("[c4] GPU run")
    kv_idx, kv_cnt, rl = spa.build_mask(dev["q"], dev["k"], W.blk_q, W.blk_k, W.k_frac, W.p,
                                        rule_len=True)
    o, lse, o_lo = spa.sparse_attn_fwd(dev["q"], dev["k"], dev["v"], kv_idx, kv_cnt, W.blk_q,
                                       W.blk_k, with_residual=True)
    dq, dk, dv = spa.sparse_attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, kv_idx,
                                     kv_cnt, W.blk_q, W.blk_k, o_lo=o_lo)
    torch.cuda.synchronize()
    host = {"kv_idx": kv_idx.cpu().numpy(), "kv_cnt": kv_cnt.cpu().numpy(),
            "rule_len": rl.cpu().numpy(), "lse": lse.cpu().numpy()}
    # only the sampled heads of the large outputs come back to the host
    heads = sorted({h for (_, h, _) in _QBLOCKS} | {h for (_, h, _) in _KBLOCKS})
    for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        host[name] = {h: t[0, h].float().cpu().numpy() for h in heads}
    del dev, o, o_lo, dq, dk, dv
    torch.cuda.empty_cache()
    return dict(g=g, host=host)


def _head(g, name, h):
    """[1, 1, N, d] fp64 view of one head (the oracle's input layout)."""
    return O.widen_bf16(g[name][:, h:h + 1])


_MASK_HEADS = [0, 21, 39]
_QBLOCKS = [(0, 0, 0), (0, 13, 300), (0, 39, W.n_qblk - 1)]
_KBLOCKS = [(0, 5, 0), (0, 30, 600), (0, 39, W.n_kblk - 1)]


def test_c4_mask_sampled_heads(c4):
    h_ = c4["host"]
    dens = h_["kv_cnt"].mean() / W.n_kblk
    log(f"[c4] density {dens:.4f}")
    assert 0.04 < dens < 0.10
    lk = O.topk_count(W.k_frac, W.n_kblk)
    assert np.all(h_["rule_len"][..., 0] == lk)
    for hh in _MASK_HEADS:
        log(f"[c4] oracle mask, head {hh}")
        mask = O.build_mask(_head(c4["g"], "q", hh), _head(c4["g"], "k", hh), W.blk_q, W.blk_k,
                            W.k_frac, W.p)
        n, exempt, fails = parity.compare_mask_rows(h_["kv_idx"][:, hh:hh + 1],
                                                    h_["kv_cnt"][:, hh:hh + 1], mask["rows"], W.p)
        log(f"  {n} rows, {len(exempt)} exempt")
        assert n == W.n_qblk
        assert not fails, fails[:5]


def test_c4_fwd_and_dq_sampled(c4):
    h_, g = c4["host"], c4["g"]
    heads = sorted({hh for (_, hh, _) in _QBLOCKS})
    for (b, hh, i) in _QBLOCKS + parity.worst_qblocks(h_["kv_cnt"], heads):
        log(f"[c4] fwd/dQ q-block (b={b}, h={hh}, i={i}), {h_['kv_cnt'][b, hh, i]} kept")
        lists = parity.lists_from_gpu(h_["kv_idx"][:, hh:hh + 1], h_["kv_cnt"][:, hh:hh + 1])
        f = {n: _head(g, n, hh) for n in ("q", "k", "v", "do")}
        o, lse = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, W.blk_q, W.blk_k,
                                   heads=[(0, 0)], qblocks=[i])
        dq, _, _ = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, W.blk_q, W.blk_k,
                                     heads=[(0, 0)], qblocks=[i])
        s, e = i * W.blk_q, min(W.N, (i + 1) * W.blk_q)
        for name, got, want in (("O", h_["o"][hh][s:e], o[0, 0, s:e]),
                                ("LSE", h_["lse"][b, hh, s:e], lse[0, 0, s:e]),
                                ("dQ", h_["dq"][hh][s:e], dq[0, 0, s:e])):
            ok, mx, rel, _ = parity.close(got, want)
            log(f"  {name}: max_abs={mx:.3e} rel_l2={rel:.3e}")
            assert ok, (name, mx, rel)


def test_c4_dkdv_sampled(c4):
    h_, g = c4["host"], c4["g"]
    heads = sorted({hh for (_, hh, _) in _KBLOCKS})
    for (b, hh, j) in _KBLOCKS + parity.worst_kblocks(h_["kv_idx"], h_["kv_cnt"], heads, W.n_kblk):
        lists = parity.lists_from_gpu(h_["kv_idx"][:, hh:hh + 1], h_["kv_cnt"][:, hh:hh + 1])
        users = [i for i, keep in enumerate(lists[(0, 0)]) if j in set(keep.tolist())]
        log(f"[c4] dK/dV key block (b={b}, h={hh}, j={j}) kept by {len(users)} query blocks")
        f = {n: _head(g, n, hh) for n in ("q", "k", "v", "do")}
        _, dk, dv = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, W.blk_q, W.blk_k,
                                      heads=[(0, 0)], qblocks=users)
        s, e = j * W.blk_k, min(W.N, (j + 1) * W.blk_k)
        for name, got, want in (("dK", h_["dk"][hh][s:e], dk[0, 0, s:e]),
                                ("dV", h_["dv"][hh][s:e], dv[0, 0, s:e])):
            ok, mx, rel, _ = parity.close(got, want)
            log(f"  {name}: max_abs={mx:.3e} rel_l2={rel:.3e}")
            assert ok, (name, mx, rel)
