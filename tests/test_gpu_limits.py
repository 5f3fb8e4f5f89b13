"""GPU parity at the library's size limit and for bf16 gradient output.

- Maximum sequence length: 2048 key blocks of 64 (N = 131072, and a ragged N = 131040
  whose last key block holds 32 keys), d = 64, blocks 128 x 64.  The mask is compared on
  every row of both heads; O, LSE, dQ on the first, a middle and the last query block;
  dK, dV on the first, a middle and the last key block.
- Near-maximal kept lists: unstructured inputs at N = 131035 (last key block 27 keys), where
  the hybrid rule keeps about 1840 of 2048 blocks per row; with 64-row query blocks the
  per-key-block lists of the dK/dV pass near their 2048-entry capacity too.  The mask is
  compared on every row of one head, O, LSE, dQ on the last query block; dK and dV (whose
  oracle would need nearly the dense layer) through invariants that hold at any size.
- bf16 gradients: the backward with ``grad_dtype=bfloat16`` must return exactly the
  round-to-nearest-even bf16 values of its fp32 gradients (same kernels, same arithmetic,
  one rounding at the store).
"""
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


MAX_CASES = [
    ("n131072", synth.Workload("max_video", 1, 2, 131072, 64, 128, 64, 0.05, 0.9,
                               kind="video", grid=(8, 128, 128), alpha=synth.ALPHA_480P,
                               n_sinks=4, seed=11)),
    # ragged: last key block 32 keys, last query block 96 rows
    ("n131040_ragged", synth.Workload("max_ragged", 1, 2, 131040, 64, 128, 64, 0.05, 0.9,
                                      kind="video", grid=(9, 112, 130),
                                      alpha=synth.ALPHA_480P, n_sinks=4, seed=12)),
]


@pytest.mark.parametrize("tag,w", MAX_CASES, ids=[c[0] for c in MAX_CASES])
def test_max_length_sampled(torch_gpu, tag, w):
    torch = torch_gpu
    assert w.n_kblk == 2048
    log(f"[limits {tag}] shape={w.shape()} key blocks={w.n_kblk}")
    g = synth.generate(w)
    dev = {n: torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in g}
    kv_idx, kv_cnt = spa.build_mask(dev["q"], dev["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
    o, lse, o_lo = spa.sparse_attn_fwd(dev["q"], dev["k"], dev["v"], kv_idx, kv_cnt, w.blk_q,
                                       w.blk_k, with_residual=True)
    dq, dk, dv = spa.sparse_attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, kv_idx,
                                     kv_cnt, w.blk_q, w.blk_k, o_lo=o_lo)
    torch.cuda.synchronize()
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    log(f"  mean kept blocks per row {cnt.mean():.1f} of {w.n_kblk}")
    for hh in range(w.H):
        f = {n: O.widen_bf16(g[n][:, hh:hh + 1]) for n in ("q", "k", "v", "do")}
        mask = O.build_mask(f["q"], f["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
        n, exempt, fails = parity.compare_mask_rows(idx[:, hh:hh + 1], cnt[:, hh:hh + 1],
                                                    mask["rows"], w.p)
        log(f"  head {hh}: mask {n} rows, {len(exempt)} exempt")
        assert n == w.n_qblk and not fails, fails[:5]
        lists = parity.lists_from_gpu(idx[:, hh:hh + 1], cnt[:, hh:hh + 1])
        qbs = [0, w.n_qblk // 2, w.n_qblk - 1]
        ro, rl = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, w.blk_q, w.blk_k,
                                   heads=[(0, 0)], qblocks=qbs)
        rdq, _, _ = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, w.blk_q, w.blk_k,
                                      heads=[(0, 0)], qblocks=qbs)
        for i in qbs:
            s, e = i * w.blk_q, min(w.N, (i + 1) * w.blk_q)
            for name, got, want in (("O", o[0, hh, s:e].float().cpu().numpy(), ro[0, 0, s:e]),
                                    ("LSE", lse[0, hh, s:e].cpu().numpy(), rl[0, 0, s:e]),
                                    ("dQ", dq[0, hh, s:e].cpu().numpy(), rdq[0, 0, s:e])):
                ok, mx, rel, _ = parity.close(got, want)
                assert ok, (hh, i, name, mx, rel)
        for j in (0, w.n_kblk // 2, w.n_kblk - 1):
            users = [i for i, keep in enumerate(lists[(0, 0)]) if j in set(keep.tolist())]
            _, rdk, rdv = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, w.blk_q,
                                            w.blk_k, heads=[(0, 0)], qblocks=users)
            s, e = j * w.blk_k, min(w.N, (j + 1) * w.blk_k)
            for name, got, want in (("dK", dk[0, hh, s:e].cpu().numpy(), rdk[0, 0, s:e]),
                                    ("dV", dv[0, hh, s:e].cpu().numpy(), rdv[0, 0, s:e])):
                ok, mx, rel, _ = parity.close(got, want)
                log(f"  head {hh} key block {j} ({len(users)} users) {name}: "
                    f"max_abs={mx:.3e} rel_l2={rel:.3e}")
                assert ok, (hh, j, name, mx, rel)


DENSE_CASES = [
    # query blocks of 128 rows: row lists near 2048 entries
    ("q128", synth.Workload("max_dense", 1, 2, 131072 - 37, 64, 128, 64, 0.05, 0.9,
                            kind="tiny", seed=12)),
    # query blocks of 64 rows: 2048 of them, so the per-key-block lists of the dK/dV pass
    # also approach their 2048-entry capacity
    ("q64", synth.Workload("max_dense_q64", 1, 1, 131072 - 37, 64, 64, 64, 0.05, 0.9,
                           kind="tiny", seed=13)),
]


@pytest.mark.parametrize("tag,w", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_near_maximal_lists(torch_gpu, tag, w):
    torch = torch_gpu
    assert w.n_kblk == 2048 and w.N % 64 == 27
    log(f"[limits dense lists {tag}] shape={w.shape()} query blocks={w.n_qblk}")
    g = synth.generate(w)
    dev = {n: torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in g}
    kv_idx, kv_cnt = spa.build_mask(dev["q"], dev["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
    o, lse, o_lo = spa.sparse_attn_fwd(dev["q"], dev["k"], dev["v"], kv_idx, kv_cnt, w.blk_q,
                                       w.blk_k, with_residual=True)
    dq, dk, dv = spa.sparse_attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, kv_idx,
                                     kv_cnt, w.blk_q, w.blk_k, o_lo=o_lo)
    torch.cuda.synchronize()
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    log(f"  kept blocks per row: mean {cnt.mean():.1f}, max {cnt.max()} of {w.n_kblk}")
    assert cnt.mean() > 1500
    users = np.zeros(w.n_kblk, int)
    for i_ in range(w.n_qblk):
        users[idx[0, 0, i_, :cnt[0, 0, i_]]] += 1
    log(f"  query blocks per key block (head 0): mean {users.mean():.1f}, max {users.max()} "
        f"of {w.n_qblk}")
    f = {n: O.widen_bf16(g[n][:, 0:1]) for n in ("q", "k", "v", "do")}
    mask = O.build_mask(f["q"], f["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
    n, exempt, fails = parity.compare_mask_rows(idx[:, 0:1], cnt[:, 0:1], mask["rows"], w.p)
    log(f"  head 0: mask {n} rows, {len(exempt)} exempt")
    assert n == w.n_qblk and not fails, fails[:5]
    lists = parity.lists_from_gpu(idx[:, 0:1], cnt[:, 0:1])
    i = w.n_qblk - 1
    ro, rl = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, w.blk_q, w.blk_k,
                               heads=[(0, 0)], qblocks=[i])
    rdq, _, _ = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, w.blk_q, w.blk_k,
                                  heads=[(0, 0)], qblocks=[i])
    s, e = i * w.blk_q, w.N
    for name, got, want in (("O", o[0, 0, s:e].float().cpu().numpy(), ro[0, 0, s:e]),
                            ("LSE", lse[0, 0, s:e].cpu().numpy(), rl[0, 0, s:e]),
                            ("dQ", dq[0, 0, s:e].cpu().numpy(), rdq[0, 0, s:e])):
        ok, mx, rel, _ = parity.close(got, want)
        log(f"  last query block {name}: max_abs={mx:.3e} rel_l2={rel:.3e}")
        assert ok, (name, mx, rel)
    for hh in range(w.H):
        dkh, dvh, dqh = (t[0, hh].double().cpu().numpy() for t in (dk, dv, dq))
        qh, kh, doh = (O.widen_bf16(g[n][0, hh]) for n in ("q", "k", "do"))
        # each query row's key gradients sum to zero (softmax shift invariance)
        assert np.abs(dkh.sum(axis=0)).max() <= 1e-3 * np.abs(dkh).sum(axis=0).max()
        # each query row's probabilities sum to one
        np.testing.assert_allclose(dvh.sum(axis=0), doh.sum(axis=0), atol=0.05)
        qdq, kdk = float(np.sum(qh * dqh)), float(np.sum(kh * dkh))
        assert abs(qdq - kdk) <= 1e-3 * (np.abs(qh * dqh).sum() + np.abs(kh * dkh).sum())


@pytest.mark.parametrize("wname", ["tiny_sparse", "wan13b_480p"])
def test_bf16_gradients_are_rounded_fp32_gradients(torch_gpu, wname):
    torch = torch_gpu
    w = synth.WORKLOADS[wname]
    if wname == "wan13b_480p":  # two heads of the full-length layer
        import dataclasses
        w = dataclasses.replace(w, H=2)
    g = synth.generate(w)
    dev = {n: torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in g}
    kv_idx, kv_cnt = spa.build_mask(dev["q"], dev["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
    o, lse, o_lo = spa.sparse_attn_fwd(dev["q"], dev["k"], dev["v"], kv_idx, kv_cnt, w.blk_q,
                                       w.blk_k, with_residual=True)
    args = (dev["q"], dev["k"], dev["v"], o, dev["do"], lse, kv_idx, kv_cnt, w.blk_q, w.blk_k)
    g32 = spa.sparse_attn_bwd(*args, o_lo=o_lo)
    g16 = spa.sparse_attn_bwd(*args, o_lo=o_lo, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), g32, g16):
        assert a.dtype == torch.float32 and b.dtype == torch.bfloat16
        assert torch.equal(a.to(torch.bfloat16), b), name


@pytest.mark.parametrize("blk_q", [128, 64])
def test_mask_d128_at_2048_key_blocks(torch_gpu, blk_q):
    """The mask at d = 128 with 2048 key blocks (N = 131040, ragged: last key block 32 keys),
    where the selection kernel's pooled-logit rows take its whole 160 KiB of LDS: every row
    against the oracle."""
    torch = torch_gpu
    w = synth.Workload("max_d128", 1, 1, 131040, 128, blk_q, 64, 0.05, 0.9, kind="video",
                       grid=(9, 112, 130), alpha=synth.ALPHA_480P, n_sinks=4, seed=13)
    assert w.n_kblk == 2048
    log(f"[limits mask d128 blk_q={blk_q}] shape={w.shape()}")
    g = synth.generate(w, with_do=False)
    q, k = (torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k"))
    kv_idx, kv_cnt, rl = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p, rule_len=True)
    torch.cuda.synchronize()
    idx, cnt, rl = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), rl.cpu().numpy()
    f = {n: O.widen_bf16(g[n]) for n in ("q", "k")}
    mask = O.build_mask(f["q"], f["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
    n, exempt, fails = parity.compare_mask_rows(idx, cnt, mask["rows"], w.p)
    log(f"  {n} rows, {len(exempt)} exempt, mean kept {cnt.mean():.1f} of {w.n_kblk}")
    assert n == w.n_qblk and not fails, fails[:5]
    assert np.all(rl[..., 0] == O.topk_count(w.k_frac, w.n_kblk))
