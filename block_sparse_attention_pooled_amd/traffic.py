"""Measured HBM traffic per kernel launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE passes.

The counters report kilobytes moved between L2 and memory per dispatch.  Their scale is
calibrated against a plain device-to-device copy of known size recorded in the same run
(the copy reads and writes exactly its size), and every figure carries a fingerprint of
the kernel sources it was measured with: once those sources change, the figure is stale
and ``load`` returns None.

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
    a = ap.parse_args(argv)
    sys.stdout.write(summarize(a.fetch, a.write, a.copy_mib, a.workload, a.command_fetch,
                               a.command_write))


if __name__ == "__main__":
    main()
