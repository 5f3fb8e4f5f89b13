"""Mask-rule stress sweep: per (k, p) the mask kernel's rate, the kept-block counts of each
rule and the attention time, on the stress layer (B=1, H=12, N=32760, d=128, blocks 128 x 64;
heads 0-5 near-uniform, heads 6-11 sink-dominated).

The sweep spans the two failure regimes the SpargeAttention2 pages name (mindverse article,
sections "Einschränkungen traditioneller Methoden" and "Hybride Top-k+Top-p Maskierung"): on
near-uniform rows Top-k's fixed count keeps little mass and Top-p decides; on sink-dominated
rows Top-p stops at the sink block and Top-k decides.  Per (k, p) in {2, 5, 10} % x {0.7, 0.9,
0.95} it reports:

- mask: pool + select time with Q and K read from HBM (the 256 MB last-level cache flushed
  before each call) and the rate on the mask's algorithmic bytes (read Q and K once, write
  the lists and counts), as a fraction of the 8 TB/s peak; also the warm-cache time;
- per head kind, histograms of the kept-block counts per query-block row for Top-k alone
  (Lk), Top-p alone (Lp) and the union (L = max(Lk, Lp), the list the kernels run);
- the attention time of the layer (forward with residual + backward) on the union lists,
  HIP events around the kernels on the launch stream.

Usage:  python -m block_sparse_attention_pooled_amd.stress_sweep [--steps S]
Prints one JSON object.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

SWEEP = [(k, p) for k in (0.02, 0.05, 0.10) for p in (0.7, 0.9, 0.95)]
# histogram bin edges over the kept-block count of a row (1 .. Nkb = 512 at this shape)
EDGES = [1, 2, 4, 8, 16, 32, 64, 128, 256, 384, 512, 513]
PEAK_HBM_GBS = 8000.0


def histogram(counts: np.ndarray) -> dict:
    h, _ = np.histogram(counts, bins=EDGES)
    return {f"[{a},{b})": int(n) for a, b, n in zip(EDGES[:-1], EDGES[1:], h)}


def main(argv=None):
    ap = argparse.ArgumentParser(prog="block_sparse_attention_pooled_amd.stress_sweep")
    ap.add_argument("--workload", default="stress")
    ap.add_argument("--steps", type=int, default=5)
    a = ap.parse_args(argv)

    import torch
    import block_sparse_attention_pooled_amd as spa
    from block_sparse_attention_pooled_amd import synth

    if not torch.cuda.is_available():
        print("the stress sweep needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    w = synth.WORKLOADS[a.workload]
    B, H, N, d = w.shape()
    print(f"[stress_sweep] generating {w.name} {w.shape()}", file=sys.stderr, flush=True)
    g = synth.generate(w)
    dev = {n: torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in g}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    nqb, nkb = w.n_qblk, w.n_kblk
    i32 = dict(dtype=torch.int32, device=q.device)
    kv_idx = torch.empty((B, H, nqb, nkb), **i32)
    kv_cnt = torch.empty((B, H, nqb), **i32)
    rl = torch.empty((B, H, nqb, 2), **i32)
    mws = torch.empty(spa.mask_workspace_bytes(q.shape, w.blk_q, w.blk_k), dtype=torch.uint8,
                      device=q.device)
    flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=q.device)
    kinds = {"uniform heads": slice(0, H // 2), "sink heads": slice(H // 2, H)}
    if w.kind != "stress":
        kinds = {"all heads": slice(0, H)}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def mask_ms(kf, p, cold):
        ts = []
        for _ in range(a.steps):
            if cold:
                float(flush.sum())
                torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record()
            spa.build_mask(q, k, w.blk_q, w.blk_k, kf, p, out=(kv_idx, kv_cnt, None),
                           workspace=mws)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.mean(ts))

    def attn_ms():
        def run():
            o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                               with_residual=True)
            spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                o_lo=o_lo)
        run()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(a.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    out = {"workload": w.name, "shape": [B, H, N, d], "blocks": [w.blk_q, w.blk_k],
           "histogram_bins": EDGES, "sweep": []}
    for kf, p in SWEEP:
        spa.build_mask(q, k, w.blk_q, w.blk_k, kf, p, rule_len=True, out=(kv_idx, kv_cnt, rl),
                       workspace=mws)
        torch.cuda.synchronize()
        cnt, rlh = kv_cnt.cpu().numpy(), rl.cpu().numpy()
        mbytes = 2.0 * B * H * N * d * 2 + 4.0 * (cnt.sum() + B * H * nqb)
        cold, warm = mask_ms(kf, p, True), mask_ms(kf, p, False)
        row = {"k": kf, "p": p,
               "mask_ms": cold, "mask_gbs": mbytes / (cold * 1e-3) / 1e9,
               "mask_hbm_frac": mbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "mask_ms_warm_cache": warm,
               "attn_fwd_bwd_ms": attn_ms(), "kinds": {}}
        for kind, hs in kinds.items():
            lk, lp, L = rlh[:, hs, :, 0], rlh[:, hs, :, 1], cnt[:, hs]
            row["kinds"][kind] = {
                "density": float(L.mean()) / nkb,
                "rows_topp_bound": float((lp > lk).mean()),
                "hist_topk": histogram(lk), "hist_topp": histogram(lp),
                "hist_union": histogram(L),
                "mean_topk": float(lk.mean()), "mean_topp": float(lp.mean()),
                "mean_union": float(L.mean()),
            }
        print(f"[stress_sweep] k={kf} p={p}: mask {cold:.3f} ms "
              f"({row['mask_hbm_frac'] * 100:.1f} % of HBM), attention {row['attn_fwd_bwd_ms']:.2f} ms",
              file=sys.stderr, flush=True)
        out["sweep"].append(row)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
