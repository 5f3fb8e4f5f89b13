"""Pins for the CPU oracle: each check ties the oracle to something other than itself
(closed forms, brute force, library routines, hand-worked fixtures, finite differences).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import spa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ input widening
def test_widen_bf16_matches_torch_on_every_bit_pattern():
    # all 65536 bf16 patterns: normals, subnormals, both zeros, both infinities, NaNs
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127  # exponent all ones with a nonzero 7-bit fraction, two signs
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 stays -0


def test_widen_bf16_closed_forms():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x0001 = 2^-133 (smallest subnormal), 0x7F7F = largest
    # finite (2 - 2^-7) 2^127, 0x7F80 = +inf, 0x8000 = -0
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x7F80, 0x8000], dtype=np.uint16)
    got = O.widen_bf16(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133
    assert got[3] == (2.0 - 2.0 ** -7) * 2.0 ** 127 and got[4] == np.inf
    assert got[5] == 0.0 and np.signbit(got[5])


# ------------------------------------------------------------------ pooling (O1, O2)
def test_pool_closed_form_with_partial_tail():
    # Q[t] = t * ones: the block mean is the block centre; the tail block [96, 100)
    # averages its 4 valid rows only (worked by hand: 15.5, 47.5, 79.5, 97.5).
    x = np.repeat(np.arange(100, dtype=np.float64)[:, None], 3, axis=1)
    got = O.pool_blocks(x, 32)
    assert got.shape == (4, 3)
    np.testing.assert_array_equal(got[:, 0], [15.5, 47.5, 79.5, 97.5])
    assert O.block_ranges(100, 32) == [(0, 32), (32, 64), (64, 96), (96, 100)]


def test_pool_matches_torch_avg_pool_on_full_blocks():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((256, 16))
    ref = torch.nn.functional.avg_pool1d(torch.from_numpy(x.T[None]), 64).numpy()[0].T
    np.testing.assert_allclose(O.pool_blocks(x, 64), ref, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ pooled softmax (O3)
def test_pooled_softmax_matches_library_softmax():
    from scipy.special import softmax
    rng = np.random.default_rng(1)
    qb, kb = rng.standard_normal((5, 8)), rng.standard_normal((11, 8))
    P = O.pooled_probs(qb, kb, 0.3)
    ref = softmax(0.3 * (qb @ kb.T), axis=1)
    np.testing.assert_allclose(P, ref, rtol=1e-14, atol=0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-15)


def test_pooled_softmax_shift_invariant():
    rng = np.random.default_rng(2)
    z = rng.standard_normal(40) * 5
    np.testing.assert_allclose(O.softmax_row(z), O.softmax_row(z + 123.25), rtol=1e-12)


# ------------------------------------------------------------------ Top-k (O5)
@pytest.mark.parametrize("k,n,want", [(0.05, 512, 26), (0.05, 1182, 60), (0.10, 16, 2),
                                      (0.05, 100, 5), (1.0, 7, 7), (0.0, 9, 1),
                                      (0.02, 512, 11), (0.10, 512, 52), (0.25, 512, 128)])
def test_topk_count_closed_form(k, n, want):
    assert O.topk_count(k, n) == want


def test_topk_equals_full_sort_on_distinct_values():
    rng = np.random.default_rng(3)
    for _ in range(20):
        row = rng.dirichlet(np.ones(37))
        lk = O.topk_count(0.2, 37)
        ref = np.sort(np.argsort(-row, kind="stable")[:lk])
        np.testing.assert_array_equal(O.topk_set(row, 0.2), ref)


def test_topk_tie_row_keeps_lowest_indices():
    row = np.full(10, 0.1)
    np.testing.assert_array_equal(O.topk_set(row, 0.3), [0, 1, 2])


# ------------------------------------------------------------------ Top-p (O6) by brute force
def _brute_topp(row, p):
    n = row.shape[0]
    for size in range(1, n + 1):
        best = max(sum(row[list(c)]) for c in itertools.combinations(range(n), size))
        if best >= p:
            return size, best
    return n, row.sum()


@pytest.mark.parametrize("n", [4, 7, 10, 12])
def test_topp_brute_force_minimal_and_max_mass(n):
    rng = np.random.default_rng(10 + n)
    for trial in range(6):
        row = rng.dirichlet(np.ones(n) * (0.3 + trial))
        for p in (0.3, 0.5, 0.8, 0.9, 0.95):
            size, best = _brute_topp(row, p)
            r = O.select_row(row, 0.0, p)
            assert r["Lp"] == size
            # the prefix of the descending order attains the maximal mass at that size
            assert abs(r["cum"][r["Lp"] - 1] - best) <= 1e-15
            # C_{Lp-2} < p <= C_{Lp-1}
            assert r["cum"][r["Lp"] - 1] >= p
            if r["Lp"] >= 2:
                assert r["cum"][r["Lp"] - 2] < p


def test_topp_p_one_keeps_all_even_under_rounding():
    row = np.full(10, 0.1)  # sums to 0.9999999999999999 in sequential fp64
    assert np.cumsum(row)[-1] < 1.0
    assert O.select_row(row, 0.0, 1.0)["Lp"] == 10


# ------------------------------------------------------------------ failure cases + union (O7)
def _fixture_rows(case, n):
    if case["name"] == "uniform":
        return np.full(n, 1.0 / n)
    row = np.full(n, 0.06 / 14)
    row[0], row[1] = 0.91, 0.03
    return row


def test_failure_cases_and_union_repair_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "failure_rows.json")))
    n, k, p = fx["n"], fx["k_frac"], fx["p"]
    for case in fx["cases"]:
        row = _fixture_rows(case, n)
        r = O.select_row(row, k, p)
        assert r["Lk"] == case["Lk"] and r["Lp"] == case["Lp"], case["name"]
        np.testing.assert_array_equal(O.topk_set(row, k), case["topk_keep"])
        np.testing.assert_array_equal(O.topp_set(row, p), case["topp_keep"])
        np.testing.assert_array_equal(r["keep"], case["union_keep"])
        if "topk_mass" in case:
            assert row[case["topk_keep"]].sum() == pytest.approx(case["topk_mass"], abs=1e-15)
            assert row[case["topp_keep"]].sum() == pytest.approx(case["topp_mass"], abs=1e-15)


def test_union_invariants_random_rows():
    rng = np.random.default_rng(4)
    for trial in range(200):
        n = int(rng.integers(1, 80))
        row = rng.dirichlet(np.ones(n) * rng.uniform(0.05, 3))
        k, p = float(rng.uniform(0, 1)), float(rng.uniform(0, 1))
        r = O.select_row(row, k, p)
        keep = set(r["keep"].tolist())
        assert keep >= set(O.topk_set(row, k).tolist()) | set(O.topp_set(row, p).tolist())
        assert len(keep) == max(r["Lk"], r["Lp"]) >= 1
        assert r["mass"] >= p - 1e-15 or len(keep) == n or r["Lk"] >= r["Lp"]
        assert np.all(np.diff(r["keep"]) > 0) and r["keep"].max() < n
        # no dropped block beats the weakest kept block (ties resolved by index)
        dropped = [j for j in range(n) if j not in keep]
        for j in dropped:
            assert (row[j], -j) < (r["tau"], -r["order"][r["L"] - 1])


def test_k_zero_is_topp_and_p_zero_is_topk():
    rng = np.random.default_rng(5)
    row = rng.dirichlet(np.ones(30) * 0.5)
    np.testing.assert_array_equal(O.select_row(row, 0.0, 0.8)["keep"], O.topp_set(row, 0.8))
    np.testing.assert_array_equal(O.select_row(row, 0.2, 0.0)["keep"], O.topk_set(row, 0.2))


# ------------------------------------------------------------------ masked attention (O8)
def _rand_qkv(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)) for _ in range(4))


def test_dense_attn_matches_torch_sdpa():
    q, k, v, _ = _rand_qkv(1, 1, 70, 8, 6)
    o, lse = O.dense_attn(q[0, 0], k[0, 0], v[0, 0], 0.35)
    tq, tk, tv = (torch.from_numpy(x[0, 0]) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], scale=0.35)[0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    ref_lse = torch.logsumexp(0.35 * tq @ tk.T, dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-13)


@pytest.mark.parametrize("k_frac,p", [(1.0, 0.5), (0.1, 1.0)])
def test_full_keep_reproduces_dense(k_frac, p):
    B, H, N, d = 1, 2, 100, 8
    q, k, v, _ = _rand_qkv(B, H, N, d, 7)
    mask = O.build_mask(q, k, 32, 16, k_frac, p)
    lists = O.lists_from_mask(mask)
    for bh in lists:
        assert all(len(x) == 7 for x in lists[bh])
    o, lse = O.sparse_attn_fwd(q, k, v, lists, 32, 16)
    for b in range(B):
        for h in range(H):
            od, ld = O.dense_attn(q[b, h], k[b, h], v[b, h], 1 / math.sqrt(d))
            np.testing.assert_allclose(o[b, h], od, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[b, h], ld, atol=1e-12, rtol=0)


def test_sparse_attn_matches_torch_sdpa_with_block_mask():
    B, H, N, d, bq, bk = 1, 2, 100, 8, 32, 16
    q, k, v, _ = _rand_qkv(B, H, N, d, 8)
    mask = O.build_mask(q, k, bq, bk, 0.2, 0.5)
    lists = O.lists_from_mask(mask)
    o, lse = O.sparse_attn_fwd(q, k, v, lists, bq, bk)
    for (b, h), rows in lists.items():
        allowed = torch.zeros(N, N, dtype=torch.bool)
        for i, keep in enumerate(rows):
            for j in keep:
                allowed[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk] = True
        tq, tk, tv = (torch.from_numpy(x[b, h]) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq[None], tk[None], tv[None], attn_mask=allowed[None], scale=1 / math.sqrt(d))[0]
        np.testing.assert_allclose(o[b, h], ref.numpy(), atol=1e-13, rtol=0)


def test_attention_special_values():
    B, H, N, d, bq, bk = 1, 1, 100, 8, 32, 16
    q, k, _, _ = _rand_qkv(B, H, N, d, 9)
    lists = O.lists_from_mask(O.build_mask(q, k, bq, bk, 0.3, 0.6))
    ones = np.ones((B, H, N, d))
    o, lse = O.sparse_attn_fwd(q, k, ones, lists, bq, bk)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)
    # one-hot value columns reveal the attention weights: V[u, c] = [u == c]
    vv = np.zeros((B, H, N, N))
    vv[0, 0] = np.eye(N)
    qq = np.concatenate([q, np.zeros((B, H, N, N - d))], axis=3)
    kk = np.concatenate([k, np.zeros((B, H, N, N - d))], axis=3)
    a_rows, lse2 = O.sparse_attn_fwd(qq, kk, vv, lists, bq, bk, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(a_rows[0, 0].sum(axis=1), 1.0, atol=1e-14)
    for i, keep in enumerate(lists[(0, 0)]):
        allowed = O.kept_keys(keep, bk, N)
        row = a_rows[0, 0, i * bq]
        outside = np.setdiff1d(np.arange(N), allowed)
        assert np.all(row[outside] == 0)
        z = (q[0, 0, i * bq] @ k[0, 0, allowed].T) / math.sqrt(d)
        np.testing.assert_allclose(row[allowed], np.exp(z - lse2[0, 0, i * bq]), atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


def test_single_kept_block_reduces_to_small_softmax():
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 1, 64, 4)) for _ in range(3))
    lists = {(0, 0): [np.array([2]), np.array([0])]}
    o, lse = O.sparse_attn_fwd(q, k, v, lists, 32, 16)
    z = q[0, 0, 5] @ k[0, 0, 32:48].T / 2.0
    w = np.exp(z - z.max())
    np.testing.assert_allclose(o[0, 0, 5], (w / w.sum()) @ v[0, 0, 32:48], atol=1e-14)


# ------------------------------------------------------------------ gradients (O9)
def _loss(q, k, v, do, lists, bq, bk):
    o, _ = O.sparse_attn_fwd(q, k, v, lists, bq, bk)
    return float(np.sum(o * do))


def test_gradients_exhaustive_finite_differences_micro():
    # B=1 H=1 N=100 d=8, blocks 32 x 16: both query and key tails are partial.
    B, H, N, d, bq, bk = 1, 1, 100, 8, 32, 16
    q, k, v, do = _rand_qkv(B, H, N, d, 12)
    lists = O.lists_from_mask(O.build_mask(q, k, bq, bk, 0.3, 0.7))
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, lists, bq, bk)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, lists, bq, bk)
            x[idx] = old - h
            lm = _loss(q, k, v, do, lists, bq, bk)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-7, (name, err)


def test_gradients_match_torch_autograd_fp64():
    B, H, N, d, bq, bk = 1, 2, 130, 16, 64, 32
    q, k, v, do = _rand_qkv(B, H, N, d, 13)
    lists = O.lists_from_mask(O.build_mask(q, k, bq, bk, 0.25, 0.6))
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, lists, bq, bk)
    for (b, h), rows in lists.items():
        allowed = torch.zeros(N, N, dtype=torch.bool)
        for i, keep in enumerate(rows):
            for j in keep:
                allowed[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk] = True
        tq, tk, tv = (torch.from_numpy(x[b, h].copy()).requires_grad_() for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq[None], tk[None], tv[None], attn_mask=allowed[None], scale=1 / math.sqrt(d))[0]
        (o * torch.from_numpy(do[b, h])).sum().backward()
        np.testing.assert_allclose(dq[b, h], tq.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dk[b, h], tk.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dv[b, h], tv.grad.numpy(), atol=1e-12)


def test_gradient_invariants():
    B, H, N, d, bq, bk = 1, 1, 200, 8, 64, 32
    q, k, v, do = _rand_qkv(B, H, N, d, 14)
    lists = O.lists_from_mask(O.build_mask(q, k, bq, bk, 0.3, 0.5))
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, lists, bq, bk)
    # shift invariance of the softmax: keys summed over all rows have zero gradient sum
    np.testing.assert_allclose(dk[0, 0].sum(axis=0), 0.0, atol=1e-12)
    # each query distributes dO_t over its keys with weights summing to 1
    np.testing.assert_allclose(dv[0, 0].sum(axis=0), do[0, 0].sum(axis=0), atol=1e-12)
    # Q -> cQ, K -> K/c leaves the logits unchanged
    assert abs(np.sum(q * dq) - np.sum(k * dk)) < 1e-11


def test_sampled_bwd_restriction_consistent():
    B, H, N, d, bq, bk = 1, 1, 256, 8, 64, 32
    q, k, v, do = _rand_qkv(B, H, N, d, 15)
    lists = O.lists_from_mask(O.build_mask(q, k, bq, bk, 0.3, 0.5))
    full = O.sparse_attn_bwd(q, k, v, do, lists, bq, bk)
    parts = [O.sparse_attn_bwd(q, k, v, do, lists, bq, bk, qblocks=[i]) for i in range(4)]
    for t in range(3):
        np.testing.assert_allclose(sum(p[t] for p in parts), full[t], atol=1e-13)


# ------------------------------------------------------------------ failure modes at attention level
def _attention_failure_case(kind):
    """One query block over 16 key blocks of 8 tokens, pooled rows shaped like the fixture rows.

    Every token of key block j equals c_j * e1 and every query equals e1, so the token
    logits equal the pooled logits and the attention weights are P[j] / 8 per token.
    """
    nkb, bk, d = 16, 8, 4
    if kind == "uniform":
        probs = np.full(nkb, 1.0 / nkb)
    else:
        probs = np.full(nkb, 0.06 / 14)
        probs[0], probs[1] = 0.91, 0.03
    scale = 0.5
    logits = np.log(probs)
    c = logits / scale
    N = nkb * bk
    q = np.zeros((1, 1, bk * 2, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d))
    for j in range(nkb):
        k[0, 0, j * bk:(j + 1) * bk, 0] = c[j]
    rng = np.random.default_rng(21)
    v = rng.standard_normal((1, 1, N, d)) * 0.1
    v[0, 0, :bk, 0] += 1.0          # the sink block (column 0 only)
    v[0, 0, bk:2 * bk, 1] += 10.0   # the informative block
    # pad queries to N tokens (only the first query block is inspected)
    qq = np.zeros((1, 1, N, d))
    qq[0, 0, :bk * 2] = q[0, 0]
    return qq, k, v, bk, scale, probs


@pytest.mark.parametrize("kind", ["uniform", "sink"])
def test_failure_modes_at_attention_level(kind):
    q, k, v, bk, scale, probs = _attention_failure_case(kind)
    bq = 2 * bk
    mask = O.build_mask(q, k, bq, bk, 0.10, 0.9, pooled_scale=scale)
    np.testing.assert_allclose(mask["probs"][(0, 0)][0], probs, atol=1e-12)
    N = q.shape[2]
    od, _ = O.dense_attn(q[0, 0], k[0, 0], v[0, 0], scale)
    row = mask["probs"][(0, 0)][0]
    errs, info = {}, {}
    for rule, keep in (("topk", O.topk_set(row, 0.10)), ("topp", O.topp_set(row, 0.9)),
                       ("union", mask["rows"][(0, 0)][0]["keep"])):
        lists = {(0, 0): [keep] * (N // bq)}
        o, _ = O.sparse_attn_fwd(q, k, v, lists, bq, bk, scale=scale)
        errs[rule] = np.linalg.norm(o[0, 0, :bq] - od[:bq]) / np.linalg.norm(od[:bq])
        # relative error on column 1, which only the informative block 1 drives
        info[rule] = np.abs(o[0, 0, :bq, 1] - od[:bq, 1]).max() / np.abs(od[:bq, 1]).max()
    if kind == "uniform":
        assert errs["topk"] > 0.5 and errs["union"] < 0.1, errs
        assert errs["union"] <= min(errs["topk"], errs["topp"]) + 1e-12
    else:
        # Top-p alone drops block 1 (weight 0.03, +10 in column 1); the union keeps it
        assert info["topp"] > 0.8 and info["union"] < 0.1, info
        assert errs["union"] < errs["topp"], errs
