"""CPU oracle for hybrid Top-k + Top-p block-sparse attention (test infrastructure only).

This is the plain, slow, fp64 statement of what the HIP library computes.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
library never calls it and shares no code with it.

Sources (the pages describe the method in prose only; no formula is printed):
  [P4] "Optimierung der Effizienz von Video-Diffusionsmodellen durch SpargeAttention2"
       (mindverse news article), sections "Grundlagen der dünnbesetzten Aufmerksamkeit",
       "Block-dünnbesetzte Aufmerksamkeit", "Maskierungsstrategien: Top-k und Top-p",
       "Einschränkungen traditioneller Methoden", "Hybride Top-k+Top-p Maskierung",
       "Effiziente Kernel-Implementierung und Modellanpassung".
  [P2] "SpargeAttention2: Trainable Sparse Attention via Hybrid Top-k+Top-p Masking and
       Distillation Fine-Tuning" (chatpaper abstract page), English abstract,
       contributions (i) and (ii).
  [P1] "SpargeAttention2" news item (knowai.space), the "hybrid masking" paragraph.

Readings taken where the pages are silent (each is repeated in the design notes):
  R1 pooling is the block mean of Q and of K;
  R2 the pooled softmax uses the attention scale 1/sqrt(d) unless given;
  R3 a partial tail block is pooled over its valid rows only and competes in the
     pooled softmax like any other block; keys >= N never enter the attention;
  R4 the Top-k count is ceil(k * Nkb) clamped to [1, Nkb] (a 1e-9 guard absorbs
     decimal k such as 0.05 * 100);
  R5 Top-p keeps the smallest prefix of the descending order whose cumulative pooled
     probability is >= p; p >= 1 keeps every block;
  R6 among minimal sets the prefix of the descending order is taken;
  R7 the two rules are combined by union, which is the prefix of length max(Lk, Lp);
  R8 ties are broken by the lower block index;
  R9 every row keeps at least one block;
  R11 one mask per (batch, head, query block);
  R12 the mask is held fixed for the gradients;
  R13 the log-sum-exp is in natural log.

Every function works on fp64 numpy arrays.  Inputs given as bf16 bit patterns are
widened exactly.
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------------
# input widening
# ----------------------------------------------------------------------------------
def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------
# O1: blocks
# ----------------------------------------------------------------------------------
def block_ranges(n_tokens: int, blk: int):
    """Token ranges [start, stop) of each block; the last block may be partial (R3)."""
    return [(s, min(n_tokens, s + blk)) for s in range(0, n_tokens, blk)]


# ----------------------------------------------------------------------------------
# O2: block-mean pooling  ([P4] "Maskierungsstrategien": block-pooled attention map; R1, R3)
# ----------------------------------------------------------------------------------
def pool_blocks(x: np.ndarray, blk: int) -> np.ndarray:
    """x [N, d] -> [nblk, d]: mean over the valid rows of each block."""
    rows = []
    for s, e in block_ranges(x.shape[0], blk):
        rows.append(x[s:e].sum(axis=0) / (e - s))
    return np.stack(rows)


# ----------------------------------------------------------------------------------
# O3: pooled softmax ([P4] "Grundlagen": row-wise softmax; "Maskierungsstrategien")
# ----------------------------------------------------------------------------------
def softmax_row(z: np.ndarray) -> np.ndarray:
    m = np.max(z)
    e = np.exp(z - m)
    return e / np.sum(e)


def pooled_probs(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """P[i, j] = softmax_j(scale * <qbar_i, kbar_j>)  (one row per query block)."""
    logits = scale * (qbar @ kbar.T)
    return np.stack([softmax_row(logits[i]) for i in range(logits.shape[0])])


# ----------------------------------------------------------------------------------
# O4-O7: row order, Top-k, Top-p, union ([P4] "Maskierungsstrategien",
# "Hybride Top-k+Top-p Maskierung"; [P2] contribution (i); [P1])
# ----------------------------------------------------------------------------------
def row_order(prob_row: np.ndarray) -> np.ndarray:
    """Block indices sorted by probability descending, ties by lower index (R8)."""
    j = np.arange(prob_row.shape[0])
    return np.lexsort((j, -prob_row))


def topk_count(k_frac: float, n_blocks: int) -> int:
    """Lk: the k % largest positions of a row, as a count (R4)."""
    return int(min(n_blocks, max(1, math.ceil(k_frac * n_blocks - 1e-9))))


def topp_count(sorted_probs: np.ndarray, p: float) -> int:
    """Lp: length of the shortest descending prefix whose cumulative probability reaches p (R5, R6)."""
    n = sorted_probs.shape[0]
    if p >= 1.0:
        return n
    c = 0.0
    for r in range(n):
        c += float(sorted_probs[r])
        if c >= p:
            return r + 1
    return n  # rounding left the total below p


def select_row(prob_row: np.ndarray, k_frac: float, p: float) -> dict:
    """Hybrid rule on one pooled row: the union of the Top-k and Top-p sets (R7).

    Both sets are prefixes of the same order, so the union is the prefix of length
    max(Lk, Lp).  Returns the kept blocks (ascending) and diagnostics.
    """
    n = prob_row.shape[0]
    order = row_order(prob_row)
    sp = prob_row[order]
    lk = topk_count(k_frac, n)
    lp = topp_count(sp, p)
    L = max(lk, lp)
    keep = np.sort(order[:L])
    cum = np.cumsum(sp)  # sequential fp64 sums in order
    return {
        "keep": keep, "Lk": lk, "Lp": lp, "L": L,
        "mass": float(cum[L - 1]), "tau": float(sp[L - 1]),
        "order": order, "sorted": sp, "cum": cum,
    }


def topk_set(prob_row: np.ndarray, k_frac: float) -> np.ndarray:
    order = row_order(prob_row)
    return np.sort(order[:topk_count(k_frac, prob_row.shape[0])])


def topp_set(prob_row: np.ndarray, p: float) -> np.ndarray:
    order = row_order(prob_row)
    return np.sort(order[:topp_count(prob_row[order], p)])


# ----------------------------------------------------------------------------------
# whole mask
# ----------------------------------------------------------------------------------
def build_mask(q: np.ndarray, k: np.ndarray, blk_q: int, blk_k: int, k_frac: float,
               p: float, pooled_scale: float | None = None, heads=None) -> dict:
    """q, k [B, H, N, d] fp64.  Returns per-(b,h) lists of kept blocks per query block.

    result["rows"][(b, h)] is a list (one entry per query block) of select_row dicts;
    result["probs"][(b, h)] is the pooled probability map [Nqb, Nkb].
    """
    B, H, N, d = q.shape
    scale = (1.0 / math.sqrt(d)) if (pooled_scale is None or pooled_scale <= 0) else pooled_scale
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    out = {"rows": {}, "probs": {}}
    for (b, h) in heads:
        qbar = pool_blocks(q[b, h], blk_q)
        kbar = pool_blocks(k[b, h], blk_k)
        P = pooled_probs(qbar, kbar, scale)
        out["probs"][(b, h)] = P
        out["rows"][(b, h)] = [select_row(P[i], k_frac, p) for i in range(P.shape[0])]
    return out


# ----------------------------------------------------------------------------------
# O8: masked softmax attention over kept tiles ([P4] "Block-dünnbesetzte Aufmerksamkeit":
# a tile is either kept whole or dropped; "Effiziente Kernel-Implementierung": dropped
# tiles' matmuls and softmax are skipped)
# ----------------------------------------------------------------------------------
def kept_keys(keep_blocks, blk_k: int, n_tokens: int) -> np.ndarray:
    """Token indices of the kept key blocks (keys >= N excluded, R3)."""
    parts = [np.arange(j * blk_k, min(n_tokens, (j + 1) * blk_k)) for j in keep_blocks]
    return np.concatenate(parts)


def attn_qblock(qi: np.ndarray, k: np.ndarray, v: np.ndarray, keys: np.ndarray, scale: float):
    """Softmax attention of query rows qi over the listed keys.  Returns O, LSE, A."""
    z = scale * (qi @ k[keys].T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    a = e / s
    o = a @ v[keys]
    lse = (m + np.log(s))[:, 0]
    return o, lse, a


def sparse_attn_fwd(q, k, v, kv_lists, blk_q: int, blk_k: int, scale: float | None = None,
                    heads=None, qblocks=None):
    """O, LSE for every (b, h) in heads; kv_lists[(b,h)][i] = kept key blocks of query block i.

    Rows outside the requested query blocks are left as NaN.
    """
    B, H, N, d = q.shape
    scale = (1.0 / math.sqrt(d)) if (scale is None or scale <= 0) else scale
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    o = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    qr = block_ranges(N, blk_q)
    for (b, h) in heads:
        for i in (qblocks if qblocks is not None else range(len(qr))):
            s, e = qr[i]
            keys = kept_keys(kv_lists[(b, h)][i], blk_k, N)
            oi, li, _ = attn_qblock(q[b, h, s:e], k[b, h], v[b, h], keys, scale)
            o[b, h, s:e] = oi
            lse[b, h, s:e] = li
    return o, lse


# ----------------------------------------------------------------------------------
# O9: analytic gradients with the mask fixed (R12); loss = sum_t <O_t, dO_t>
# ----------------------------------------------------------------------------------
def sparse_attn_bwd(q, k, v, do, kv_lists, blk_q: int, blk_k: int, scale: float | None = None,
                    heads=None, qblocks=None):
    """dQ, dK, dV (fp64).  With qblocks given, only those query blocks contribute (their
    dQ rows are exact; dK, dV hold only their contributions)."""
    B, H, N, d = q.shape
    scale = (1.0 / math.sqrt(d)) if (scale is None or scale <= 0) else scale
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    qr = block_ranges(N, blk_q)
    for (b, h) in heads:
        for i in (qblocks if qblocks is not None else range(len(qr))):
            s, e = qr[i]
            keys = kept_keys(kv_lists[(b, h)][i], blk_k, N)
            qi, doi = q[b, h, s:e], do[b, h, s:e]
            _, _, a = attn_qblock(qi, k[b, h], v[b, h], keys, scale)
            dpa = doi @ v[b, h][keys].T                      # <dO_t, v_u>
            dsum = np.sum(a * dpa, axis=1, keepdims=True)    # D_t
            ds = a * (dpa - dsum)                            # dS_tu
            dq[b, h, s:e] = scale * (ds @ k[b, h][keys])
            dk[b, h][keys] += scale * (ds.T @ qi)
            dv[b, h][keys] += a.T @ doi
    return dq, dk, dv


# ----------------------------------------------------------------------------------
# textbook dense attention (for the self-checks: k = 100 % or p = 1 must match it)
# ----------------------------------------------------------------------------------
def dense_attn(q2: np.ndarray, k2: np.ndarray, v2: np.ndarray, scale: float):
    """Full N x N softmax attention of one head: O, LSE."""
    z = scale * (q2 @ k2.T)
    o = np.zeros_like(q2)
    lse = np.zeros(q2.shape[0])
    for t in range(q2.shape[0]):
        w = np.exp(z[t] - z[t].max())
        o[t] = (w / w.sum()) @ v2
        lse[t] = z[t].max() + math.log(w.sum())
    return o, lse


def lists_from_mask(mask: dict):
    """{(b,h): [keep_i ...]} from build_mask's result."""
    return {bh: [r["keep"] for r in rows] for bh, rows in mask["rows"].items()}
