"""Rule ablation on the mask-rule stress layer: Top-k alone, Top-p alone and the hybrid
union, each through the same kernels, against the dense-mask run.

The three rules are the ones the SpargeAttention2 pages compare in their failure analysis
(mindverse article, sections "Maskierungsstrategien: Top-k und Top-p", "Einschränkungen"
and "Hybride Top-k+Top-p Maskierung"): a fixed count keeps little attention mass on
near-uniform rows, a mass target stops at the sink block on sink-dominated rows, and the
union repairs both.  Per rule and head kind this reports:

- kept attention mass per query row, exp(LSE_rule - LSE_dense) (the exact share of the
  row's softmax mass on the kept keys);
- the output error against dense attention (max-abs and relative L2 of O);
- the union density and the forward + backward time of the layer.

Usage:  python -m block_sparse_attention_pooled_amd.ablation [--workload stress]
Prints one JSON object.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def main(argv=None):
    ap = argparse.ArgumentParser(prog="block_sparse_attention_pooled_amd.ablation")
    ap.add_argument("--workload", default="stress")
    ap.add_argument("--k", type=float, default=0.05)
    ap.add_argument("--p", type=float, default=0.9)
    ap.add_argument("--steps", type=int, default=5)
    a = ap.parse_args(argv)

    import torch
    import block_sparse_attention_pooled_amd as spa
    from block_sparse_attention_pooled_amd import synth

    if not torch.cuda.is_available():
        print("the ablation needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    w = synth.WORKLOADS[a.workload]
    g = synth.generate(w)
    dev = {n: torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).cuda() for n in g}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]

    def layer(k_frac, p):
        kv_idx, kv_cnt = spa.build_mask(q, k, w.blk_q, w.blk_k, k_frac, p)
        o, lse, o_lo = spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                           with_residual=True)
        grads = spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k,
                                    o_lo=o_lo)
        return kv_cnt, o, lse, grads

    def timed(k_frac, p):
        layer(k_frac, p)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(a.steps):
            layer(k_frac, p)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    _, o_d, lse_d, _ = layer(1.0, 1.0)
    o_d, lse_d = o_d.float(), lse_d.clone()
    kinds = {"all": slice(0, w.H)}
    if w.kind == "stress":
        kinds = {"uniform heads": slice(0, w.H // 2), "sink heads": slice(w.H // 2, w.H)}
    rules = {"top-k only": (a.k, 0.0), "top-p only": (0.0, a.p), "hybrid": (a.k, a.p),
             "dense": (1.0, 1.0)}
    out = {"workload": w.name, "shape": list(w.shape()), "k": a.k, "p": a.p, "rules": {}}
    for name, (kf, pp) in rules.items():
        cnt, o, lse, _ = layer(kf, pp)
        torch.cuda.synchronize()
        row = {"k_frac": kf, "p": pp, "ms_fwd_bwd_with_mask": timed(kf, pp)}
        for kind, hs in kinds.items():
            mass = torch.exp(lse[:, hs] - lse_d[:, hs])
            diff = o[:, hs].float() - o_d[:, hs]
            row[kind] = {
                "density": float(cnt[:, hs].float().mean()) / w.n_kblk,
                "kept_mass_mean": float(mass.mean()),
                "kept_mass_min": float(mass.min()),
                "o_max_abs_vs_dense": float(diff.abs().max()),
                "o_rel_l2_vs_dense": float(diff.norm() / o_d[:, hs].norm()),
            }
        out["rules"][name] = row
    print(json.dumps(out))


if __name__ == "__main__":
    main()
