"""Measured HBM traffic per kernel launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE passes.

The counters report kilobytes moved between L2 and memory per dispatch.  Their scale is
calibrated against a plain device-to-device copy of known size recorded in the same run
(the copy reads and writes exactly its size), and every figure carries a fingerprint of
the kernel sources it was measured with: once those sources change, the figure is stale
and ``load`` returns None.

Also summarises an executed-MFMA counter pass (``summarize-mfma``), a kernel trace
(``summarize-trace``) and a breakdown of SIMD cycles (``summarize-stalls``).

Command line (writes the markdown summary to stdout):

    python -m block_sparse_attention_pooled_amd.traffic summarize \
        --fetch FETCH.csv --write WRITE.csv --copy-mib 512 --workload wan13b_480p \
        --command-fetch "..." --command-write "..."
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# bench stage -> (kernel-name prefix in the trace, sources the kernel is built from)
STAGES = {
    "mask_pool": ("spa::k_pool", ["mask.hip", "spa_common.h"]),
    "mask_select": ("spa::k_select", ["mask.hip", "spa_common.h"]),
    "fwd": ("spa::k_fwd", ["attn_fwd.hip", "attn_tiles.h", "spa_common.h"]),
    "bwd_dkdv": ("spa::k_dkdv", ["attn_bwd.hip", "attn_tiles.h", "spa_common.h"]),
    "bwd_dq": ("spa::k_dq", ["attn_bwd.hip", "attn_tiles.h", "spa_common.h"]),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def fingerprint(stage: str) -> str:
    h = hashlib.sha256()
    for name in STAGES[stage][1]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _per_kernel(path: str, counter: str) -> dict:
    """Average counter value per dispatch, by kernel name (argument lists stripped).  For
    the copy kernel only the largest dispatches count (the calibration copy; smaller ones
    are host transfers of the run)."""
    vals = defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
            vals[name].append(float(r["Counter_Value"]))
    out = {}
    for k, v in vals.items():
        if k.startswith(COPY_KERNEL):
            v = [x for x in v if x >= 0.9 * max(v)]
        out[k] = sum(v) / len(v)
    return out


def _match(table: dict, prefix: str) -> tuple:
    hits = [(k, v) for k, v in table.items() if k.startswith(prefix)]
    if not hits:
        return None, None
    # the largest value (for fwd: the instantiation with the residual output)
    return max(hits, key=lambda kv: kv[1])


def summarize(fetch_csv, write_csv, copy_mib, workload, cmd_fetch, cmd_write) -> str:
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    _, cf = _match(fetch, COPY_KERNEL)
    _, cw = _match(write, COPY_KERNEL)
    if not cf or not cw:
        raise SystemExit("the calibration copy is missing from the counter files")
    kf, kw = copy_kib / cf, copy_kib / cw
    out = [f"# Measured memory traffic per launch: {workload}", "",
           "Counter passes (from the repository root on one MI355X):", "", "```",
           cmd_fetch, cmd_write, "```", "",
           f"Calibration: a {copy_mib} MiB device copy (`{COPY_KERNEL}`) read {cf:.0f} KiB "
           f"(FETCH_SIZE) and wrote {cw:.0f} KiB (WRITE_SIZE); scale factors "
           f"fetch {kf:.4f}, write {kw:.4f}.", "",
           "| stage | kernel | fetch KiB (raw) | write KiB (raw) | traffic bytes (scaled) "
           "| fetch factor | write factor | source fingerprint |",
           "|---|---|---|---|---|---|---|---|"]
    for stage, (prefix, _) in STAGES.items():
        name, f_raw = _match(fetch, prefix)
        _, w_raw = _match(write, prefix)
        if name is None or w_raw is None:
            continue
        traffic = (f_raw * kf + w_raw * kw) * 1024.0
        out.append(f"| {stage} | `{name}` | {f_raw:.0f} | {w_raw:.0f} | {traffic:.4e} | "
                   f"{kf:.4f} | {kw:.4f} | {fingerprint(stage)} |")
    return "\n".join(out) + "\n"


def load(stage: str, workload: str):
    """Scaled traffic in bytes per launch for `stage`, or None (no record, or stale)."""
    path = os.path.join(PROFILES, f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    row = re.compile(r"^\| (\S+) \| `[^`]*` \| [\d.]+ \| [\d.]+ \| ([\d.e+]+) \| [\d.]+ \| "
                     r"[\d.]+ \| ([0-9a-f]+) \|$")
    with open(path) as f:
        for line in f:
            m = row.match(line.strip())
            if m and m.group(1) == stage:
                return float(m.group(2)) if m.group(3) == fingerprint(stage) else None
    return None


def summarize_trace(trace_csv, title, command) -> str:
    """Per-kernel call count, total and average duration from a rocprofv3 kernel-trace CSV
    (``--kernel-trace``), with each kernel's launch shape."""
    durs = defaultdict(list)
    shape = {}
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
            durs[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            if name not in shape:
                g = lambda k: r.get(k, "?")
                shape[name] = (f"({g('Grid_Size_X')}, {g('Grid_Size_Y')})", g("Workgroup_Size_X"),
                               r.get("Arch_VGPR_Count", r.get("VGPR_Count", "?")),
                               g("Accum_VGPR_Count"),
                               r.get("LDS_Block_Size", r.get("Group_Segment_Size", "?")))
    total = sum(sum(v) for v in durs.values())
    out = [f"# Kernel trace: {title}", "", "Command (from the repository root on one MI355X):",
           "", "```", command, "```", "",
           "| kernel | calls | total (us) | average (us) | share |", "|---|---|---|---|---|"]
    order = sorted(durs, key=lambda n: -sum(durs[n]))
    for n in order:
        t = sum(durs[n])
        out.append(f"| `{n}` | {len(durs[n])} | {t:.1f} | {t / len(durs[n]):.1f} | "
                   f"{100.0 * t / total:.1f} % |")
    out += ["", "Launch shapes:", "",
            "| kernel | grid (x, y) | workgroup | arch VGPR | acc VGPR | LDS bytes |",
            "|---|---|---|---|---|---|"]
    for n in order:
        out.append(f"| `{n}` | " + " | ".join(shape[n]) + " |")
    out += ["", "The VGPR columns are rocprofv3's `Arch_VGPR_Count` / `Accum_VGPR_Count` fields as "
            "recorded. On this part they read half of the allocation that the compiler reports "
            "(`-Rpass-analysis=kernel-resource-usage`): 128 for a kernel built with 256 vector "
            "registers."]
    return "\n".join(out) + "\n"


STALL_KERNELS = ("spa::k_dkdv", "spa::k_dq", "spa::k_fwd", "spa::k_select", "spa::k_pool")


def _counters(path):
    per = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(dict)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
            per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[name][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    avg = {n: {k: sum(v) / len(v) for k, v in c.items()} for n, c in per.items()}
    d_us = {n: sum(v.values()) / len(v) / 1e3 for n, v in dur.items()}
    return avg, d_us


def summarize_stalls(csv_a, csv_b, workload, cmd_a, cmd_b, simds=1024, xcds=8) -> str:
    """Where the SIMDs' cycles go, per kernel, from two counter passes: MFMA-pipe busy
    cycles, VALU issue (4 cycles per non-MFMA VALU instruction of a 64-wide wavefront),
    their overlap, and the wavefront states.  The clock is GRBM_GUI_ACTIVE over the
    dispatch (summed over the XCDs); SIMD cycles = SIMDs x duration x clock."""
    a, da = _counters(csv_a)
    b, db = _counters(csv_b)
    out = [f"# Where the SIMD cycles go: {workload}", "",
           "Counter passes (from the repository root on one MI355X):", "", "```", cmd_a,
           cmd_b, "```", "",
           "Per kernel, as fractions of SIMD cycles (1024 SIMDs x duration x the clock from "
           "GRBM_GUI_ACTIVE): MFMA = SQ_VALU_MFMA_BUSY_CYCLES; VALU = 4 x (SQ_INSTS_VALU - "
           "SQ_INSTS_MFMA), the issue cycles of the other vector instructions; both = "
           "SQ_VALU_MFMA_COEXEC_CYCLES.  Wavefront states are fractions of SQ_WAVE_CYCLES.", "",
           "| kernel | us | GHz | MFMA only | VALU only | both | neither | waiting (SQ_WAIT_ANY) "
           "| ready, not issued (SQ_WAIT_INST_ANY) | issuing (SQ_ACTIVE_INST_ANY) | "
           "exp / transcendental instr | LDS instr |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for pre in STALL_KERNELS:
        na = max((n for n in a if n.startswith(pre)), key=lambda n: da[n], default=None)
        nb = max((n for n in b if n.startswith(pre)), key=lambda n: db[n], default=None)
        if na is None or nb is None:
            continue
        ca, cb = a[na], b[nb]
        clk = ca.get("GRBM_GUI_ACTIVE", 0.0) / xcds / (da[na] * 1e-6)
        cyc = simds * da[na] * 1e-6 * clk
        if cyc <= 0:
            continue
        mf = ca.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / cyc
        va = 4.0 * (cb.get("SQ_INSTS_VALU", 0.0) - cb.get("SQ_INSTS_MFMA", 0.0)) / cyc
        bo = ca.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / cyc
        wc = ca.get("SQ_WAVE_CYCLES", 0.0) or float("nan")
        out.append(
            f"| `{na}` | {da[na]:.0f} | {clk / 1e9:.2f} | {100 * (mf - bo):.0f} % | "
            f"{100 * (va - bo):.0f} % | {100 * bo:.0f} % | {100 * (1 - mf - va + bo):.0f} % | "
            f"{100 * ca.get('SQ_WAIT_ANY', 0) / wc:.0f} % | "
            f"{100 * ca.get('SQ_WAIT_INST_ANY', 0) / wc:.0f} % | "
            f"{100 * ca.get('SQ_ACTIVE_INST_ANY', 0) / wc:.0f} % | "
            f"{cb.get('SQ_INSTS_VALU_TRANS_F32', 0):.3g} | {cb.get('SQ_INSTS_LDS', 0):.3g} |")
    return "\n".join(out) + "\n"


def summarize_mfma(csv_path, workload, command) -> str:
    """Executed MFMA work per dispatch from SQ_INSTS_MFMA (every MFMA here is a
    32x32x16 bf16 or fp16 instruction: 32768 FLOP per wavefront instruction) over the dispatch's
    duration, with the MFMA-busy and GPU-busy cycle counters as recorded."""
    per = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(dict)
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
            per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[name][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = [f"# Executed MFMA work per launch: {workload}", "",
           "Counter pass (from the repository root on one MI355X):", "", "```", command, "```",
           "",
           "Executed FLOP = SQ_INSTS_MFMA x 32768 (all MFMAs are v_mfma_f32_32x32x16_bf16 or "
           "_f16); "
           "the rate divides by the dispatch's own duration in this run.  Credited (kept-tile "
           "algorithmic) FLOP are lower: the precision splits and the recomputation in the "
           "backward are executed but not credited.", "",
           "| kernel | dispatches | MFMA instr / dispatch | executed TFLOP / dispatch | "
           "duration us | executed TFLOP/s | SQ_VALU_MFMA_BUSY_CYCLES | SQ_BUSY_CYCLES | "
           "GRBM_GUI_ACTIVE |", "|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(per, key=lambda n: -sum(dur[n].values())):
        c = per[name]
        mf = c.get("SQ_INSTS_MFMA")
        if not mf or max(mf) == 0:
            continue
        avg = lambda k: sum(c[k]) / len(c[k]) if c.get(k) else float("nan")
        d_us = sum(dur[name].values()) / len(dur[name]) / 1e3
        tf = avg("SQ_INSTS_MFMA") * 32768 / 1e12
        out.append(f"| `{name}` | {len(dur[name])} | {avg('SQ_INSTS_MFMA'):.4g} | {tf:.4f} | "
                   f"{d_us:.1f} | {tf / (d_us * 1e-6):.0f} | {avg('SQ_VALU_MFMA_BUSY_CYCLES'):.4g} | "
                   f"{avg('SQ_BUSY_CYCLES'):.4g} | {avg('GRBM_GUI_ACTIVE'):.4g} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(prog="block_sparse_attention_pooled_amd.traffic")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-mib", type=float, required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--command-fetch", required=True)
    s.add_argument("--command-write", required=True)
    t = sub.add_parser("summarize-trace")
    t.add_argument("--trace", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    st = sub.add_parser("summarize-stalls")
    st.add_argument("--csv-a", required=True)
    st.add_argument("--csv-b", required=True)
    st.add_argument("--workload", required=True)
    st.add_argument("--command-a", required=True)
    st.add_argument("--command-b", required=True)
    m = sub.add_parser("summarize-mfma")
    m.add_argument("--csv", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "summarize":
        sys.stdout.write(summarize(a.fetch, a.write, a.copy_mib, a.workload, a.command_fetch,
                                   a.command_write))
    elif a.cmd == "summarize-stalls":
        sys.stdout.write(summarize_stalls(a.csv_a, a.csv_b, a.workload, a.command_a,
                                          a.command_b))
    elif a.cmd == "summarize-trace":
        sys.stdout.write(summarize_trace(a.trace, a.title, a.command))
    else:
        sys.stdout.write(summarize_mfma(a.csv, a.workload, a.command))


if __name__ == "__main__":
    main()
