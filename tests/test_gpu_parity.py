"""GPU parity: the HIP library (through the C ABI) against the fp64 CPU oracle.

Mask: kept lists bit-exact except blocks within 1e-6 of the row threshold (reported).
Attention: O, LSE, dQ, dK, dV computed with the GPU's mask, max-abs <= 2e-2 and
relative L2 <= 1e-2.
"""
import dataclasses
import math
import sys

import numpy as np
import pytest

import block_sparse_attention_pooled_amd as spa
from block_sparse_attention_pooled_amd import synth
from oracle import spa_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    spa.load_library()
    return torch


def to_dev(torch, bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(torch, g, w, k_frac, p, with_bwd=True):
    q, k, v = (to_dev(torch, g[n]) for n in ("q", "k", "v"))
    kv_idx, kv_cnt, rl = spa.build_mask(q, k, w.blk_q, w.blk_k, k_frac, p, rule_len=True)
    o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                       with_residual=True)
    o_plain, lse_plain = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k)
    res = dict(kv_idx=kv_idx.cpu().numpy(), kv_cnt=kv_cnt.cpu().numpy(), rule_len=rl.cpu().numpy(),
               o=o.float().cpu().numpy(), lse=lse.cpu().numpy(),
               o_full=(o.float() + o_lo.float()).cpu().numpy(),
               o_plain=o_plain.float().cpu().numpy(), lse_plain=lse_plain.cpu().numpy())
    if with_bwd:
        do = to_dev(torch, g["do"])
        dq, dk, dv = spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                         o_lo=o_lo)
        res.update(dq=dq.cpu().numpy(), dk=dk.cpu().numpy(), dv=dv.cpu().numpy())
    torch.cuda.synchronize()
    return res


def check_close(name, got, want):
    ok, mx, rel, scaled = parity.close(got, want)
    log(f"  {name}: max_abs={mx:.3e} rel_l2={rel:.3e} max_abs/max(1,|x|inf)={scaled:.3e}")
    assert ok, f"{name}: max_abs={mx:.3e} rel_l2={rel:.3e} scaled={scaled:.3e}"


def small_workload(N, d, bq, grid=None, kind="video", seed=3, B=1, H=2):
    if grid is None:
        kind = "tiny"
    return synth.Workload(f"small_{N}_{d}_{bq}", B, H, N, d, bq, 64, 0.1, 0.9, kind=kind,
                          grid=grid, alpha=synth.ALPHA_480P, n_sinks=2, seed=seed)


SMALL = [
    ("tiny", synth.WORKLOADS["tiny"]),
    ("tiny_sparse", synth.WORKLOADS["tiny_sparse"]),
    ("n1000_d128_q128", small_workload(1000, 128, 128, grid=(2, 20, 25), B=2, H=3)),
    ("n1000_d128_q64", small_workload(1000, 128, 64, grid=(2, 20, 25))),
    ("n1000_d64_q128", small_workload(1000, 64, 128, grid=(2, 20, 25))),
    ("n777_d64_q64", small_workload(777, 64, 64, grid=(3, 7, 37))),
    ("n65_d128_q128", small_workload(65, 128, 128)),
    ("n50_d64_q64", small_workload(50, 64, 64)),
]


def full_check(torch, w, k_frac, p, tag):
    log(f"[case {tag}] shape={w.shape()} blk=({w.blk_q},{w.blk_k}) k={k_frac} p={p}")
    g = synth.generate(w)
    res = run_gpu(torch, g, w, k_frac, p)
    q, k, v, do = (O.widen_bf16(g[n]) for n in ("q", "k", "v", "do"))
    mask = O.build_mask(q, k, w.blk_q, w.blk_k, k_frac, p)
    n, exempt, fails = parity.compare_mask_rows(res["kv_idx"], res["kv_cnt"], mask["rows"], p)
    log(f"  mask: {n} rows, {len(exempt)} exempt near-threshold rows {exempt[:5]}")
    assert not fails, fails[:5]
    for (b, h), rows in mask["rows"].items():
        for i, r in enumerate(rows):
            assert res["rule_len"][b, h, i, 0] == r["Lk"]
            if not exempt:
                assert res["rule_len"][b, h, i, 1] == r["Lp"], (b, h, i)
    lists = parity.lists_from_gpu(res["kv_idx"], res["kv_cnt"])
    o, lse = O.sparse_attn_fwd(q, k, v, lists, w.blk_q, w.blk_k)
    check_close("O", res["o"], o)
    check_close("O without residual", res["o_plain"], o)
    check_close("LSE", res["lse"], lse)
    # the two forward modes round the running maximum differently; LSE agrees to fp32 ulps
    np.testing.assert_allclose(res["lse"], res["lse_plain"], rtol=4e-7, atol=4e-7)
    # o + o_lo carries O to about 12 bits: P enters P*V as one fp16 rounding (relative
    # error at most 2^-11), so |error| <= 2^-11 * max |V|; the residual rounding itself
    # is 2^-17 relative
    vmax = float(np.abs(v).max())
    ok_full, mx_full, rel_full, _ = parity.close(res["o_full"], o, atol=2.0 ** -11 * vmax,
                                                 rtol_l2=2.0 ** -11)
    log(f"  O + o_lo: max_abs={mx_full:.3e} rel_l2={rel_full:.3e} (bound {2.0 ** -11 * vmax:.2e})")
    assert ok_full
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, lists, w.blk_q, w.blk_k)
    check_close("dQ", res["dq"], dq)
    check_close("dK", res["dk"], dk)
    check_close("dV", res["dv"], dv)


@pytest.mark.parametrize("tag,w", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(torch_gpu, tag, w):
    full_check(torch_gpu, w, w.k_frac, w.p, tag)


CALLER_LIST_CASES = [("n1000_d128_q128", small_workload(1000, 128, 128, grid=(2, 20, 25))),
                     ("n777_d64_q64", small_workload(777, 64, 64, grid=(3, 7, 37)))]


@pytest.mark.parametrize("tag,w", CALLER_LIST_CASES, ids=[c[0] for c in CALLER_LIST_CASES])
def test_caller_supplied_lists_parity(torch_gpu, tag, w):
    """Lists passed in by the caller, of kinds the mask never emits: a row keeping only the
    partial last key block (the loop runs no full tile), a row keeping only block 0, a row
    keeping every block, and random ascending subsets.  Forward and backward against the
    oracle on the same lists."""
    torch = torch_gpu
    B, H, N, d = w.shape()
    nqb, nkb = -(-N // w.blk_q), -(-N // w.blk_k)
    rng = np.random.default_rng(11)
    kv_idx = np.zeros((B, H, nqb, nkb), dtype=np.int32)  # entries past the count unused
    kv_cnt = np.zeros((B, H, nqb), dtype=np.int32)
    lists = {}
    for b in range(B):
        for h in range(H):
            rows = []
            for i in range(nqb):
                mode = (i + h) % 4
                if mode == 0:
                    keep = np.array([nkb - 1])
                elif mode == 1:
                    keep = np.array([0])
                elif mode == 2:
                    keep = np.arange(nkb)
                else:
                    keep = np.sort(rng.choice(nkb, size=int(rng.integers(1, nkb + 1)),
                                              replace=False))
                kv_idx[b, h, i, :keep.size] = keep
                kv_cnt[b, h, i] = keep.size
                rows.append(keep.astype(np.int64))
            lists[(b, h)] = rows
    log(f"[case caller lists {tag}] shape={w.shape()} counts={kv_cnt.ravel().tolist()}")
    g = synth.generate(w)
    q, k, v, do = (to_dev(torch, g[n]) for n in ("q", "k", "v", "do"))
    idx_t, cnt_t = torch.from_numpy(kv_idx).cuda(), torch.from_numpy(kv_cnt).cuda()
    o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, idx_t, cnt_t, w.blk_q, w.blk_k,
                                       with_residual=True)
    dq, dk, dv = spa.sparse_attn_bwd(q, k, v, o, do, lse, idx_t, cnt_t, w.blk_q, w.blk_k,
                                     o_lo=o_lo)
    torch.cuda.synchronize()
    qh, kh, vh, doh = (O.widen_bf16(g[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = O.sparse_attn_fwd(qh, kh, vh, lists, w.blk_q, w.blk_k)
    check_close("O", o.float().cpu().numpy(), o_ref)
    check_close("LSE", lse.cpu().numpy(), lse_ref)
    dq_ref, dk_ref, dv_ref = O.sparse_attn_bwd(qh, kh, vh, doh, lists, w.blk_q, w.blk_k)
    check_close("dQ", dq.cpu().numpy(), dq_ref)
    check_close("dK", dk.cpu().numpy(), dk_ref)
    check_close("dV", dv.cpu().numpy(), dv_ref)


RULES = [(0.1, 0.9), (0.0, 0.7), (0.2, 0.0), (1.0, 0.5), (0.05, 1.0), (0.0, 0.0), (0.3, 0.95)]


@pytest.mark.parametrize("k_frac,p", RULES)
def test_rule_variants_parity(torch_gpu, k_frac, p):
    w = small_workload(1000, 128, 128, grid=(2, 20, 25))
    full_check(torch_gpu, w, k_frac, p, f"rules k={k_frac} p={p}")


def test_stress_rows_parity(torch_gpu):
    # near-uniform and sink-dominated heads at reduced length
    w = dataclasses.replace(synth.WORKLOADS["stress"], N=4000, grid=(4, 20, 50), H=4)
    for k_frac, p in ((0.02, 0.7), (0.05, 0.9), (0.1, 0.95)):
        full_check(torch_gpu, w, k_frac, p, f"stress k={k_frac} p={p}")


def test_v_blocks_beyond_fp16_take_the_bf16_path(torch_gpu):
    """Query blocks whose lists hold a key block of V with values that fp16 cannot carry
    (|v| >= 65504) read bf16 V with P as a hi + lo pair; the others go through the fp16
    copy.  With V partly scaled, the error is measured against sum_u P_tu |v_u|."""
    torch = torch_gpu
    w = small_workload(1000, 128, 128, grid=(2, 20, 25))
    g = synth.generate(w)
    vv = synth.bf16_bits_to_f32(g["v"]).astype(np.float64)
    big = slice(3 * 64, 4 * 64)              # key block 3, every head
    vv[:, :, big, :] *= 2.0 ** 17            # |v| up to ~5e5: beyond fp16
    g["v"] = synth.to_bf16_bits(vv)
    q, k, v = (to_dev(torch, g[n]) for n in ("q", "k", "v"))
    kv_idx, kv_cnt = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p)
    o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                       with_residual=True)
    torch.cuda.synchronize()
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    users = sum(int(3 in set(idx[b, h, i, :cnt[b, h, i]].tolist()))
                for (b, h, i), _ in np.ndenumerate(cnt))
    log(f"  rows of query blocks keeping the scaled block: {users} of {cnt.size}")
    assert users > 0
    f = {n: O.widen_bf16(g[n]) for n in ("q", "k", "v")}
    lists = parity.lists_from_gpu(idx, cnt)
    ro, rl = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, w.blk_q, w.blk_k)
    # sum_u P_tu |v_u|: the scale of the rounding error of P in either operand format
    rabs, _ = O.sparse_attn_fwd(f["q"], f["k"], np.abs(f["v"]), lists, w.blk_q, w.blk_k)
    full = o.float().cpu().numpy().astype(np.float64) + o_lo.float().cpu().numpy()
    assert np.all(np.isfinite(full))
    err = float(np.max(np.abs(full - ro) / np.maximum(rabs, 1.0)))
    log(f"  O + o_lo: max |error| / sum P|v| = {err:.3e}")
    assert err <= 2.0 ** -11  # one fp16 rounding of P (the bf16 pair is finer)
    np.testing.assert_allclose(lse.cpu().numpy(), rl, atol=2e-2)


def test_do_and_v_beyond_fp16_take_the_bf16_dv_path(torch_gpu):
    """In dV = P^T dO the backward reads an fp16 copy of dO with P as one fp16 rounding; a
    key block whose query-block list holds a block of dO beyond fp16's range (|dO| >= 65504),
    or whose own V is beyond it, reads bf16 dO with P as a bf16 pair instead.  With dO of
    one query block and V of one key block scaled past fp16, both forms run in one call: dV
    is measured against sum_t P_tu |dO_t| (the scale of P's rounding in either form), dQ on
    the unscaled rows against the usual bound, and dQ, dK elsewhere against their largest
    reference magnitude."""
    torch = torch_gpu
    w = small_workload(1000, 128, 128, grid=(2, 20, 25))
    g = synth.generate(w)
    f = {n: synth.bf16_bits_to_f32(g[n]).astype(np.float64) for n in ("q", "k", "v", "do")}
    big_q = slice(2 * 128, 3 * 128)          # query block 2: dO beyond fp16, every head
    big_k = slice(5 * 64, 6 * 64)            # key block 5: V beyond fp16, every head
    f["do"][:, :, big_q, :] *= 2.0 ** 17
    f["v"][:, :, big_k, :] *= 2.0 ** 17
    for n in ("v", "do"):
        g[n] = synth.to_bf16_bits(f[n])
        f[n] = synth.bf16_bits_to_f32(g[n]).astype(np.float64)
    q, k, v, do = (to_dev(torch, g[n]) for n in ("q", "k", "v", "do"))
    kv_idx, kv_cnt = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p)
    o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                       with_residual=True)
    dq, dk, dv = spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                     o_lo=o_lo)
    torch.cuda.synchronize()
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    lists = parity.lists_from_gpu(idx, cnt)
    nkb = -(-w.N // w.blk_k)
    for (b, h), rows in lists.items():
        users = set(rows[2].tolist()) | {5}   # key blocks that take the bf16 form
        log(f"  head {(b, h)}: {len(users)} of {nkb} key blocks take the bf16 form")
        assert 1 < len(users) < nkb
    rq, rk, rv = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, w.blk_q, w.blk_k)
    _, _, rabs = O.sparse_attn_bwd(f["q"], f["k"], f["v"], np.abs(f["do"]), lists, w.blk_q,
                                   w.blk_k)
    gq, gk, gv = (x.cpu().numpy().astype(np.float64) for x in (dq, dk, dv))
    for name, x in (("dQ", gq), ("dK", gk), ("dV", gv)):
        assert np.all(np.isfinite(x)), name
    err_v = float(np.max(np.abs(gv - rv) / np.maximum(rabs, 1.0)))
    log(f"  dV: max |error| / sum P|dO| = {err_v:.3e}")
    assert err_v <= 2.0 ** -11
    for (b, h), rows in lists.items():  # rows that touch neither scaled block
        plain = [i for i, r in enumerate(rows) if i != 2 and 5 not in set(r.tolist())]
        sel = np.concatenate([np.arange(i * w.blk_q, min(w.N, (i + 1) * w.blk_q))
                              for i in plain])
        check_close(f"dQ {(b, h)} ({len(plain)} unscaled query blocks)", gq[b, h, sel],
                    rq[b, h, sel])
    for name, got, want in (("dQ", gq, rq), ("dK", gk, rk)):
        rel = float(np.abs(got - want).max() / max(1.0, np.abs(want).max()))
        log(f"  {name}: max |error| / max |ref| = {rel:.3e}")
        assert rel <= 1e-3, name


def test_small_v_and_do_keep_relative_precision(torch_gpu):
    """Blocks of small values (all below 2^-9, some below fp16's normal range) do not go
    through the fp16 copies: head 0 has V scaled by 2^-20 and query block 2 has dO scaled
    by 2^-20, so the forward's P V and the backward's dV must keep their precision relative
    to sum_u P_tu |v_u| and sum_t P_tu |dO_t| with no absolute floor (fp16 subnormals would
    lose most of it).  P itself enters dV in fp16 on blocks that do take the copies, which
    keeps an absolute 2^-25 below 2^-14: the dV bound adds 2^-24 sum_t |dO_t| over the rows
    of the query blocks that keep the key, negligible for the scaled block."""
    torch = torch_gpu
    w = small_workload(1000, 128, 128, grid=(2, 20, 25))
    g = synth.generate(w)
    f = {n: synth.bf16_bits_to_f32(g[n]).astype(np.float64) for n in ("q", "k", "v", "do")}
    f["v"][:, 0] *= 2.0 ** -20
    f["do"][:, :, 2 * 128:3 * 128, :] *= 2.0 ** -20
    for n in ("v", "do"):
        g[n] = synth.to_bf16_bits(f[n])
        f[n] = synth.bf16_bits_to_f32(g[n]).astype(np.float64)
    q, k, v, do = (to_dev(torch, g[n]) for n in ("q", "k", "v", "do"))
    kv_idx, kv_cnt = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p)
    o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                       with_residual=True)
    dq, dk, dv = spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                     o_lo=o_lo)
    torch.cuda.synchronize()
    lists = parity.lists_from_gpu(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy())
    ro, _ = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, w.blk_q, w.blk_k)
    rabs, _ = O.sparse_attn_fwd(f["q"], f["k"], np.abs(f["v"]), lists, w.blk_q, w.blk_k)
    full = o.float().cpu().numpy().astype(np.float64) + o_lo.float().cpu().numpy()
    err_o = float(np.max(np.abs(full - ro) / rabs))
    log(f"  O + o_lo: max |error| / sum P|v| = {err_o:.3e}")
    assert err_o <= 2.0 ** -11
    _, _, rv = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, w.blk_q, w.blk_k)
    _, _, rvabs = O.sparse_attn_bwd(f["q"], f["k"], f["v"], np.abs(f["do"]), lists, w.blk_q,
                                    w.blk_k)
    gv = dv.cpu().numpy().astype(np.float64)
    floor = np.zeros_like(gv)  # sum_t |dO_t| over the rows of query blocks keeping the key
    for (b, h), rows in lists.items():
        for i, keep in enumerate(rows):
            s_i = np.abs(f["do"][b, h, i * w.blk_q:(i + 1) * w.blk_q]).sum(axis=0)
            for j in keep.tolist():
                floor[b, h, j * w.blk_k:(j + 1) * w.blk_k] += s_i
    bound = 2.0 ** -11 * rvabs + 2.0 ** -24 * floor
    err_v = float(np.max(np.abs(gv - rv) / np.maximum(bound, 1e-300)))
    log(f"  dV: max |error| / (2^-11 sum P|dO| + 2^-24 sum|dO|) = {err_v:.3e}")
    assert err_v <= 1.0


def test_forward_stages_on_two_streams_match_the_whole_call(torch_gpu):
    """The forward's preparation (the fp16 copy of V) run on a second stream, then the
    attention on the first after a join, equals the unstaged call bit for bit."""
    torch = torch_gpu
    w = small_workload(1000, 128, 128, grid=(2, 20, 25), B=2, H=3)
    g = synth.generate(w)
    q, k, v = (to_dev(torch, g[n]) for n in ("q", "k", "v"))
    kv_idx, kv_cnt = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p)
    o1, l1, r1 = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                     with_residual=True)
    o2, l2, r2 = torch.empty_like(o1), torch.empty_like(l1), torch.empty_like(r1)
    ws = torch.empty(spa.fwd_workspace_bytes(q.shape, w.blk_q, w.blk_k), dtype=torch.uint8,
                     device=q.device)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k, with_residual=True,
                            out=(o2, l2, r2), workspace=ws, stages=spa.FWD_PREP)
    main.wait_stream(side)
    spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k, with_residual=True,
                        out=(o2, l2, r2), workspace=ws, stages=spa.FWD_ATTN)
    torch.cuda.synchronize()
    for a, b in ((o1, o2), (l1, l2), (r1, r2)):
        assert torch.equal(a, b)


def test_column_lists_built_beside_the_forward_match_the_whole_call(torch_gpu):
    """The backward's column lists built on a second stream while the forward runs on the
    first (the two read nothing the other writes), then dQ and dK/dV after a join, equal
    the unstaged backward bit for bit."""
    torch = torch_gpu
    w = small_workload(1000, 128, 128, grid=(2, 20, 25), B=2, H=3)
    g = synth.generate(w)
    q, k, v, do = (to_dev(torch, g[n]) for n in ("q", "k", "v", "do"))
    kv_idx, kv_cnt = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p)
    o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                       with_residual=True)
    want = spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                               o_lo=o_lo)
    o2, l2, r2 = torch.empty_like(o), torch.empty_like(lse), torch.empty_like(o_lo)
    got = tuple(torch.empty_like(x) for x in want)
    bws = torch.empty(spa.bwd_workspace_bytes(q.shape, w.blk_q, w.blk_k), dtype=torch.uint8,
                      device=q.device)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        spa.sparse_attn_bwd(q, k, v, o2, do, l2, kv_idx, kv_cnt, w.blk_q, w.blk_k, o_lo=r2,
                            out=got, workspace=bws, stages=spa.BWD_PREP)
    spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k, with_residual=True,
                        out=(o2, l2, r2))
    main.wait_stream(side)
    for st in (spa.BWD_DQ, spa.BWD_DKDV):
        spa.sparse_attn_bwd(q, k, v, o2, do, l2, kv_idx, kv_cnt, w.blk_q, w.blk_k, o_lo=r2,
                            out=got, workspace=bws, stages=st)
    torch.cuda.synchronize()
    for a, b in zip(want, got):
        assert torch.equal(a, b)


def test_determinism(torch_gpu):
    torch = torch_gpu
    w = small_workload(1000, 128, 128, grid=(2, 20, 25), B=2, H=3)
    g = synth.generate(w)
    a = run_gpu(torch, g, w, 0.1, 0.9)
    b = run_gpu(torch, g, w, 0.1, 0.9)
    assert np.array_equal(a["kv_cnt"], b["kv_cnt"])
    for (bb, hh, i), c in np.ndenumerate(a["kv_cnt"]):  # defined prefix of each list
        assert np.array_equal(a["kv_idx"][bb, hh, i, :c], b["kv_idx"][bb, hh, i, :c])
    for key in a:
        if key != "kv_idx":
            assert np.array_equal(a[key], b[key], equal_nan=True), key


NAN_GUARD_CASES = [("n1000_d128_q128", small_workload(1000, 128, 128, grid=(2, 20, 25))),
                   ("n777_d64_q64", small_workload(777, 64, 64, grid=(3, 7, 37))),
                   ("n1000_d128_q64", small_workload(1000, 128, 64, grid=(2, 20, 25)))]


def _front_of_nan_buffer(torch, bits, pad_rows=128):
    """A contiguous device bf16 tensor holding `bits`, placed at the front of a larger
    allocation whose remaining pad_rows rows hold NaN."""
    shape, d = bits.shape, bits.shape[-1]
    buf = torch.full((bits.size + pad_rows * d,), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    buf[:bits.size].copy_(to_dev(torch, bits).reshape(-1))
    return buf[:bits.size].view(shape)


@pytest.mark.parametrize("tag,w", NAN_GUARD_CASES, ids=[c[0] for c in NAN_GUARD_CASES])
def test_rows_beyond_n_are_never_read(torch_gpu, tag, w):
    """Partial last blocks stage rows at or beyond N as zeros through the buffer range
    check, never from the memory after the tensor: Q, K, V and dO are views at the front of
    NaN-filled allocations (so rows past the last head's end are NaN), the workspaces are
    filled with NaN bit patterns, and every output must be finite and match the oracle."""
    torch = torch_gpu
    log(f"[case nan guard {tag}] shape={w.shape()} blk=({w.blk_q},{w.blk_k})")
    g = synth.generate(w)
    q, k, v, do = (_front_of_nan_buffer(torch, g[n]) for n in ("q", "k", "v", "do"))
    kv_idx, kv_cnt = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p)
    fws = torch.full((spa.fwd_workspace_bytes(q.shape, w.blk_q, w.blk_k),), 255,
                     dtype=torch.uint8, device=q.device)
    bws = torch.full((spa.bwd_workspace_bytes(q.shape, w.blk_q, w.blk_k),), 255,
                     dtype=torch.uint8, device=q.device)
    o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                       with_residual=True, workspace=fws)
    o_plain, _ = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k)
    dq, dk, dv = spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                     o_lo=o_lo, workspace=bws)
    torch.cuda.synchronize()
    got = {"O": o, "O without residual": o_plain, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv}
    for name, t in got.items():
        assert bool(torch.isfinite(t.float()).all()), f"{name} has non-finite values"
    f = {n: O.widen_bf16(g[n]) for n in ("q", "k", "v", "do")}
    lists = parity.lists_from_gpu(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy())
    ro, rl = O.sparse_attn_fwd(f["q"], f["k"], f["v"], lists, w.blk_q, w.blk_k)
    rq, rk, rv = O.sparse_attn_bwd(f["q"], f["k"], f["v"], f["do"], lists, w.blk_q, w.blk_k)
    for name, want in (("O", ro), ("O without residual", ro), ("LSE", rl), ("dQ", rq),
                       ("dK", rk), ("dV", rv)):
        check_close(name, got[name].float().cpu().numpy(), want)
