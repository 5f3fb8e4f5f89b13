"""Comparison helpers for GPU-vs-oracle parity (test infrastructure)."""
from __future__ import annotations

import numpy as np

MASK_BAND = 1e-6       # blocks whose pooled probability is within this of the threshold
ATOL = 2e-2            # attention outputs / gradients: max-abs
RTOL_L2 = 1e-2         # and relative L2
VACUOUS = 1e-6         # a reference slice whose every |value| is at most this is zero in effect

# (max |reference|, rel-L2) of every compared slice that passed only through the vacuity
# rule; the test session prints them at its end
VACUOUS_HITS = []


def compare_mask_rows(gpu_idx: np.ndarray, gpu_cnt: np.ndarray, oracle_rows: dict, p: float,
                      band: float = MASK_BAND):
    """Compare GPU kept lists with the oracle's, row by row.

    gpu_idx [B,H,Nqb,Nkb], gpu_cnt [B,H,Nqb]; oracle_rows {(b,h): [select_row dicts]}.
    A differing block is exempt if its oracle probability lies within `band` of the row
    threshold tau, or if the row's Top-p length is decided within `band` of p (then the
    blocks at ranks Lp-1 and Lp are exempt).  Returns (n_rows, exempt_report, failures).
    """
    failures, exempt = [], []
    n = 0
    for (b, h), rows in oracle_rows.items():
        for i, r in enumerate(rows):
            n += 1
            cnt = int(gpu_cnt[b, h, i])
            lst = gpu_idx[b, h, i, :cnt]
            nk = r["order"].shape[0]
            if cnt < 1 or cnt > nk or np.any(lst < 0) or np.any(lst >= nk) or \
                    np.any(np.diff(lst) <= 0):
                failures.append(((b, h, i), "malformed list", lst.tolist()))
                continue
            g, o = set(lst.tolist()), set(r["keep"].tolist())
            if g == o:
                continue
            probs = r["sorted"]
            order = r["order"]
            ex = set()
            for rank in range(nk):
                if abs(probs[rank] - r["tau"]) <= band:
                    ex.add(int(order[rank]))
            lp = r["Lp"]
            if lp >= r["Lk"] and p < 1.0:
                cum = r["cum"]
                near = abs(cum[lp - 1] - p) <= band or (lp >= 2 and abs(cum[lp - 2] - p) <= band)
                if near:
                    ex.update(int(order[x]) for x in (lp - 2, lp - 1, lp) if 0 <= x < nk)
            diff = g ^ o
            if diff <= ex:
                exempt.append(((b, h, i), sorted(diff), r["tau"]))
            else:
                failures.append(((b, h, i), "kept sets differ", sorted(diff - ex)))
    return n, exempt, failures


def close(got: np.ndarray, want: np.ndarray, atol: float = ATOL, rtol_l2: float = RTOL_L2,
          vacuous: float = VACUOUS):
    """Max-abs and relative-L2 check; returns (ok, max_abs, rel_l2, max_abs_rel_to_inf_norm).

    Both bounds apply unless every reference value of the compared slice is at most
    `vacuous` in magnitude (a gradient that is zero in effect, e.g. dQ of a query whose
    attention sits entirely on one key, ~1e-22): the relative error then has no meaningful
    denominator and the max-abs bound alone decides.  A slice of measurable size always
    needs both, so an output that is zero where the reference is not fails."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = got - want
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-300))
    ref_inf = float(np.abs(want).max()) if want.size else 0.0
    scaled = max_abs / max(1.0, ref_inf)
    rel_ok = rel <= rtol_l2 or ref_inf <= vacuous
    if rel > rtol_l2 and ref_inf <= vacuous:
        VACUOUS_HITS.append((ref_inf, rel, got.shape))
    return bool(max_abs <= atol and rel_ok and np.all(np.isfinite(got))), max_abs, rel, scaled


def lists_from_gpu(kv_idx: np.ndarray, kv_cnt: np.ndarray):
    B, H, nqb, _ = kv_idx.shape
    return {(b, h): [kv_idx[b, h, i, :kv_cnt[b, h, i]].astype(np.int64) for i in range(nqb)]
            for b in range(B) for h in range(H)}


def worst_qblocks(kv_cnt, heads):
    """Per head, the query block with the longest kept list (lowest index on ties)."""
    return [(0, hh, int(np.argmax(kv_cnt[0, hh]))) for hh in heads]


def worst_kblocks(kv_idx, kv_cnt, heads, nkb):
    """Per head, the key block kept by the most query blocks (lowest index on ties)."""
    out = []
    for hh in heads:
        uses = np.zeros(nkb, dtype=np.int64)
        for i, c in enumerate(kv_cnt[0, hh]):
            uses[kv_idx[0, hh, i, :c]] += 1
        out.append((0, hh, int(np.argmax(uses))))
    return out
