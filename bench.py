"""Benchmark of the hybrid Top-k + Top-p block-sparse attention layer on one MI355X.

One step = the whole hot path on one synthetic layer with inputs resident in HBM:
build_mask (pool + select) -> sparse forward (with the O residual) -> sparse backward
(column lists, dQ with D, dK/dV).  Default workload: the Wan2.1-1.3B-480p-shaped layer
(B=1, H=12, N=32760 on a 21x30x52 grid, d=128, blocks 128x64, k=5 %, p=0.9).

Two preparations run on a second stream: the forward's fp16 copy of V (it reads V only)
during the mask selection, and the backward's column lists (they read the mask only)
during the forward.  Each consumer waits for its preparation.

Prints one JSON line with the step time (ms/layer), the per-stage times measured with
HIP events on the stream each stage runs on, the
roofline of the dominant kernel, a dense-mask run of the same kernels and the CPU
oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd ms/layer & MFMA util at 95% block sparsity, N=32760 H=12 d=128"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PRECISION = ("bf16 Q/K/V/dO; fp32 accumulation, softmax and gradients; S and dP as bf16 "
             "products; P*V and dV = P^T dO as fp16 products of P (one rounding) against "
             "range-checked fp16 copies of V and dO (a bf16 hi+lo pair of P where a block is "
             "not eligible); dS as a bf16 hi+lo pair (two products); mask in fp64")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kept_pairs_weight(kv_idx, kv_cnt, N, bq, bk):
    """sum over kept (i, j) of n_i * m_j (valid rows times valid keys)."""
    B, H, nqb, nkb = kv_idx.shape
    n_i = np.minimum(bq, N - np.arange(nqb) * bq).astype(np.int64)
    m_j = np.minimum(bk, N - np.arange(nkb) * bk).astype(np.int64)
    total = 0
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                c = int(kv_cnt[b, h, i])
                total += int(n_i[i]) * int(m_j[kv_idx[b, h, i, :c]].sum())
    return total


def host_cpu_info():
    """CPU model and counts of the host this process runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count(), "usable_cpus": usable}


def cpu_oracle_baseline(g, w, lists, budget_s: float, single_budget_s: float):
    """Time the CPU oracle on a bounded sample of the layer and scale to ms/layer.

    The mask is computed for every head; forward + backward run query block by query
    block (all heads, a fixed interleaved order) until the time budget is spent, and the
    per-block time is scaled to the whole layer.  Then the same on one head with the BLAS
    thread pool limited to one thread (query blocks of head 0 until `single_budget_s` is
    spent, scaled to the head).
    """
    from oracle import spa_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((x.get("num_threads", 1) for x in threadpool_info()), default=1)
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count()
    f = {n: O.widen_bf16(g[n]) for n in ("q", "k", "v", "do")}
    t0 = time.perf_counter()
    O.build_mask(f["q"], f["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
    t_mask = time.perf_counter() - t0
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    order = [(heads[x % len(heads)], (x * 37) % w.n_qblk)
             for x in range(len(heads) * w.n_qblk)]

    def run_units(units, budget):
        done = 0
        t0 = time.perf_counter()
        for ((b, h), i) in units:
            one = {n: f[n][b:b + 1, h:h + 1] for n in f}   # this head only
            l1 = {(0, 0): lists[(b, h)]}
            O.sparse_attn_fwd(one["q"], one["k"], one["v"], l1, w.blk_q, w.blk_k, qblocks=[i])
            O.sparse_attn_bwd(one["q"], one["k"], one["v"], one["do"], l1, w.blk_q, w.blk_k,
                              qblocks=[i])
            done += 1
            if time.perf_counter() - t0 > budget:
                break
        return done, time.perf_counter() - t0

    done, t_attn = run_units(order, budget_s)
    per_layer = t_mask + t_attn / done * len(order)
    out = {
        "value": per_layer * 1e3, "unit": "ms/layer", "cores": int(threads), "kind": "oracle",
        "sample": (f"fp64 numpy oracle on {threads} BLAS threads: mask of all {len(heads)} heads "
                   f"({t_mask:.2f} s) and fwd+bwd of {done} of {len(order)} (head, query block) "
                   f"units ({t_attn:.2f} s), scaled linearly to the whole layer"),
    }
    out.update(host_cpu_info())
    if threadpool_limits is not None and single_budget_s > 0:
        with threadpool_limits(limits=1):
            h0 = {n: f[n][:1, :1] for n in f}
            t0 = time.perf_counter()
            O.build_mask(h0["q"], h0["k"], w.blk_q, w.blk_k, w.k_frac, w.p)
            t_mask1 = time.perf_counter() - t0
            units = [((0, 0), (x * 37) % w.n_qblk) for x in range(w.n_qblk)]
            done1, t1 = run_units(units, single_budget_s)
        out["single_thread_one_head_ms"] = (t_mask1 + t1 / done1 * w.n_qblk) * 1e3
        out["single_thread_sample"] = (f"head 0 with one BLAS thread: mask ({t_mask1:.2f} s) and "
                                       f"fwd+bwd of {done1} of {w.n_qblk} query blocks "
                                       f"({t1:.2f} s), scaled to the head")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan13b_480p")
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU oracle work to time for the baseline")
    ap.add_argument("--cpu-single-budget", type=float, default=6.0,
                    help="seconds of single-thread oracle work on one head")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps timed with the 256 MB last-level cache flushed before "
                         "each (a secondary, cold-cache figure)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run a plain device copy of this size (the "
                         "scale reference for memory-traffic counter passes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer shards by "
              "(batch, head) with no exchange, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_pooled_amd as spa
    from block_sparse_attention_pooled_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    spa.load_library()
    w = synth.WORKLOADS[args.workload]
    B, H, N, d = w.shape()
    log(f"[bench] generating {w.name} {w.shape()}")
    g = synth.generate(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).to(dev)
                   for n in ("q", "k", "v", "do"))
    nqb, nkb = w.n_qblk, w.n_kblk
    i32 = dict(dtype=torch.int32, device=dev)
    kv_idx = torch.empty((B, H, nqb, nkb), **i32)
    kv_cnt = torch.empty((B, H, nqb), **i32)
    o, o_lo = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))
    mws = torch.empty(spa.mask_workspace_bytes(q.shape, w.blk_q, w.blk_k), dtype=torch.uint8,
                      device=dev)
    fws = torch.empty(spa.fwd_workspace_bytes(q.shape, w.blk_q, w.blk_k), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty(spa.bwd_workspace_bytes(q.shape, w.blk_q, w.blk_k), dtype=torch.uint8,
                      device=dev)
    stream = torch.cuda.current_stream(dev)
    # Two preparation stages run on a second stream (default priority) beside the launch
    # stream: the forward's fp16 copy of V reads V only and runs during the mask selection;
    # the backward's column lists read the mask only and are built during the forward.
    side = torch.cuda.Stream(dev)
    ev_fork, ev_join = torch.cuda.Event(), torch.cuda.Event()
    ev_fork2, ev_join2 = torch.cuda.Event(), torch.cuda.Event()
    stage_names = ["mask_pool", "mask_select", "fwd", "bwd_dq", "bwd_dkdv"]
    # events 0-5 bound the launch stream's stages; 6-7 and 8-9 bound the two preparations
    side_stages = {"fwd_prep_overlapped": 6, "bwd_prep_overlapped": 8}
    n_ev = 10

    def step(events=None, k_frac=w.k_frac, p=w.p):
        def mark(idx, st=stream):
            if events is not None:
                events[idx].record(st)
        mark(0)
        spa.build_mask(q, k, w.blk_q, w.blk_k, k_frac, p, out=(kv_idx, kv_cnt, None),
                       workspace=mws, stages=spa.MASK_POOL)
        mark(1)
        # forked after the pooling (which, like the conversion, streams from HBM), so that
        # the conversion overlaps the selection, whose time is the latency of its rows
        ev_fork.record(stream)
        side.wait_event(ev_fork)
        with torch.cuda.stream(side):
            mark(6, side)
            spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k, with_residual=True,
                                out=(o, lse, o_lo), workspace=fws, stages=spa.FWD_PREP)
            mark(7, side)
        ev_join.record(side)
        spa.build_mask(q, k, w.blk_q, w.blk_k, k_frac, p, out=(kv_idx, kv_cnt, None),
                       workspace=mws, stages=spa.MASK_SELECT)
        mark(2)
        ev_fork2.record(stream)
        side.wait_event(ev_fork2)
        with torch.cuda.stream(side):
            mark(8, side)
            spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k, o_lo=o_lo,
                                out=(dq, dk, dv), workspace=bws, stages=spa.BWD_PREP)
            mark(9, side)
        ev_join2.record(side)
        stream.wait_event(ev_join)
        spa.sparse_attn_fwd(q, k, v, kv_idx, kv_cnt, w.blk_q, w.blk_k, with_residual=True,
                            out=(o, lse, o_lo), workspace=fws, stages=spa.FWD_ATTN)
        mark(3)
        stream.wait_event(ev_join2)
        for st, idx in ((spa.BWD_DQ, 4), (spa.BWD_DKDV, 5)):
            spa.sparse_attn_bwd(q, k, v, o, do, lse, kv_idx, kv_cnt, w.blk_q, w.blk_k, o_lo=o_lo,
                                out=(dq, dk, dv), workspace=bws, stages=st)
            mark(idx)

    # ---- warmup + timed steps -------------------------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    stage_ms = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1])
                                     for s in range(args.steps)]))
                for i, name in enumerate(stage_names)}
    for name, i in side_stages.items():
        stage_ms[name] = float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1])
                                        for s in range(args.steps)]))
    event_step_ms = float(np.mean([ev[s][0].elapsed_time(ev[s][5]) for s in range(args.steps)]))
    log(f"[bench] {ms_per_step:.3f} ms/step (events {event_step_ms:.3f}); stages {stage_ms}")

    # ---- algorithmic work ---------------------------------------------------------------
    idx_h, cnt_h = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    nm = kept_pairs_weight(idx_h, cnt_h, N, w.blk_q, w.blk_k)
    density = float(cnt_h.mean() / nkb)
    fl_fwd, fl_dkdv, fl_dq = 4.0 * d * nm, 8.0 * d * nm, 2.0 * d * nm
    fl_total = fl_fwd + fl_dkdv + fl_dq
    mask_bytes = 2.0 * B * H * N * d * 2 + 4.0 * (cnt_h.sum() + B * H * nqb)
    pool_bytes = 2.0 * B * H * N * d * 2
    work = {
        "mask_pool": ("hbm", pool_bytes / 1e9, "GB/s", PEAK_HBM_GBS),
        "fwd": ("mfma", fl_fwd / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "bwd_dkdv": ("mfma", fl_dkdv / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
        "bwd_dq": ("mfma", fl_dq / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS),
    }
    dom = max(work, key=lambda n: stage_ms[n])
    bound, units_per_launch, unit, peak = work[dom]
    achieved = units_per_launch / (stage_ms[dom] * 1e-3)
    from block_sparse_attention_pooled_amd import traffic as traffic_rec
    roofline = {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic_rec.load(dom, w.name)}
    # the attention kernels' own times, the overlapped preparation included (the step time
    # shows what the overlap saves)
    attn_ms = (stage_ms["fwd"] + stage_ms["fwd_prep_overlapped"] + stage_ms["bwd_prep_overlapped"]
               + stage_ms["bwd_dkdv"] + stage_ms["bwd_dq"])
    mask_in_step_ms = stage_ms["mask_pool"] + stage_ms["mask_select"]
    # the mask kernels alone (pool + select back to back, nothing on the second stream):
    # inside a step the selection shares the GPU with the forward's preparation.  The
    # headline figure reads Q and K from HBM: reading 512 MB before each timed call evicts
    # them from the 256 MB last-level cache (which holds both at this shape); the warm
    # figure (back-to-back calls, Q and K largely cache-resident) is reported beside it.
    def time_mask(flush_buf):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for s_ in range(args.steps):
            if flush_buf is not None:
                float(flush_buf.sum())
                torch.cuda.synchronize()
            evs[s_][0].record(stream)
            spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p, out=(kv_idx, kv_cnt, None),
                           workspace=mws)
            evs[s_][1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))

    mask_ms_warm = time_mask(None)
    flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    mask_ms = time_mask(flush)
    del flush

    # ---- cold-cache steps: reading 512 MB evicts the 256 MB last-level cache before each
    # step (a read, so that no dirty lines are written back during the step) -------------
    cold = None
    if args.cold_steps > 0:
        flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
               for _ in range(args.cold_steps)]
        for s_ in range(args.cold_steps):
            float(flush.sum())
            torch.cuda.synchronize()
            step(cev[s_])
            torch.cuda.synchronize()
        cold_stage = {name: float(np.mean([cev[s_][i].elapsed_time(cev[s_][i + 1])
                                           for s_ in range(args.cold_steps)]))
                      for i, name in enumerate(stage_names)}
        for name, i in side_stages.items():
            cold_stage[name] = float(np.mean([cev[s_][i].elapsed_time(cev[s_][i + 1])
                                              for s_ in range(args.cold_steps)]))
        # the mask's rate here is its time inside the step (beside the copy of V)
        cold = {"ms_per_step": float(np.mean([cev[s_][0].elapsed_time(cev[s_][5])
                                              for s_ in range(args.cold_steps)])),
                "stage_ms": cold_stage,
                "mask_hbm_frac": mask_bytes / ((cold_stage["mask_pool"] + cold_stage["mask_select"])
                                               * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del flush
        log(f"[bench] cold-cache step {cold['ms_per_step']:.3f} ms")

    # ---- rule statistics of the measured mask -------------------------------------------
    _, _, rl = spa.build_mask(q, k, w.blk_q, w.blk_k, w.k_frac, w.p, rule_len=True)
    rl_h = rl.cpu().numpy()
    lk_h, lp_h = rl_h[..., 0], rl_h[..., 1]
    rules = {"Lk": int(lk_h.flat[0]), "mean_Lp": float(lp_h.mean()),
             "mean_L": float(cnt_h.mean()), "rows_topp_bound": float((lp_h > lk_h).mean()),
             "L_percentiles_50_90_99_100": [float(x) for x in
                                            np.percentile(cnt_h, [50, 90, 99, 100])]}

    if args.calib_copy_mib > 0:  # scale reference for the traffic counters
        n = args.calib_copy_mib << 20
        src_buf = torch.ones(n, dtype=torch.uint8, device=dev)
        dst_buf = torch.empty_like(src_buf)
        for _ in range(3):
            dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf

    # ---- dense-mask run on the same kernels ---------------------------------------------
    dense = None
    if args.dense_steps > 0:
        step(k_frac=1.0, p=1.0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.dense_steps):
            step(k_frac=1.0, p=1.0)
        torch.cuda.synchronize()
        dense_ms = (time.perf_counter() - t0) * 1e3 / args.dense_steps
        nm_dense = kept_pairs_weight(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), N, w.blk_q,
                                     w.blk_k)
        dense = {"ms_per_step": dense_ms, "sparse_over_dense_speedup": dense_ms / ms_per_step,
                 "credited_tflops": 14.0 * d * nm_dense / (dense_ms * 1e-3) / 1e12}
        log(f"[bench] dense mask: {dense_ms:.3f} ms/step")
        step()  # restore the sparse lists
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a sample")
        lists = {(b, h): [idx_h[b, h, i, :cnt_h[b, h, i]].astype(np.int64) for i in range(nqb)]
                 for b in range(B) for h in range(H)}
        cpu = cpu_oracle_baseline(g, w, lists, args.cpu_budget, args.cpu_single_budget)
        log(f"[bench] cpu oracle: {cpu['value']:.1f} ms/layer on {cpu['cores']} threads")
    out = {
        "metric": METRIC, "value": ms_per_step, "unit": "ms/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded video-grid Q/K/V/dO, bf16)",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "blk_q": w.blk_q,
                   "blk_k": w.blk_k, "k_frac": w.k_frac, "p": w.p, "alpha": w.alpha,
                   "grid": list(w.grid) if w.grid else None, "density": density,
                   "grad_dtype": "fp32", "precision": PRECISION},
        "stage_ms": stage_ms, "mask_ms": mask_ms, "mask_in_step_ms": mask_in_step_ms,
        "attn_fwd_bwd_ms": attn_ms,
        "credited_tflops_fwd_bwd": fl_total / (attn_ms * 1e-3) / 1e12,
        "mfma_util_credited": fl_total / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "mask_hbm_frac": mask_bytes / (mask_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "mask_ms_warm": mask_ms_warm,
        "mask_hbm_frac_warm_cache": mask_bytes / (mask_ms_warm * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "rules": rules, "cold_cache": cold,
        "roofline": roofline, "dense": dense, "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
