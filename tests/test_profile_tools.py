"""Host-side checks of the rocprofv3 summarisers (no GPU): kernel-trace statistics, the
memory-traffic scaling against a copy of known size, and the SIMD-cycle breakdown, on
small hand-made CSV files whose expected figures follow from their definitions."""
import csv

import pytest

from block_sparse_attention_pooled_amd import traffic

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
              "LDS_Block_Size", "VGPR_Count", "Accum_VGPR_Count", "Workgroup_Size_X",
              "Grid_Size_X", "Grid_Size_Y"]
CTR_COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]


def write_csv(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_trace_summary_totals_and_shares(tmp_path):
    rows = []
    for i, (name, dur_ns) in enumerate([("void spa::k_a<1>(int)", 3000), ("void spa::k_a<1>(int)", 1000),
                                         ("void spa::k_b(float*)", 4000)]):
        rows.append(dict(Kind="KERNEL_DISPATCH", Agent_Id=1, Queue_Id=1, Kernel_Name=name,
                         Start_Timestamp=10_000 * i, End_Timestamp=10_000 * i + dur_ns,
                         LDS_Block_Size=512, VGPR_Count=8, Accum_VGPR_Count=0,
                         Workgroup_Size_X=256, Grid_Size_X=1024, Grid_Size_Y=1))
    p = tmp_path / "trace.csv"
    write_csv(p, TRACE_COLS, rows)
    md = traffic.summarize_trace(str(p), "t", "cmd")
    # k_a: 2 calls, 4.0 us in all, 2.0 us average, half of the 8 us total
    assert "| `spa::k_a<1>` | 2 | 4.0 | 2.0 | 50.0 % |" in md
    assert "| `spa::k_b` | 1 | 4.0 | 4.0 | 50.0 % |" in md
    assert "| `spa::k_b` | (1024, 1) | 256 | 8 | 0 | 512 |" in md


def test_traffic_scaled_by_the_copy(tmp_path):
    # the copy of 1 MiB reads 512 KiB on FETCH_SIZE (factor 2) and writes 1024 KiB (factor 1)
    fetch = [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name="FETCH_SIZE",
                  Counter_Value=512, Start_Timestamp=0, End_Timestamp=1),
             dict(Dispatch_Id=2, Kernel_Name="void spa::k_dkdv<128, 128>(int)",
                  Counter_Name="FETCH_SIZE", Counter_Value=100, Start_Timestamp=0,
                  End_Timestamp=1)]
    write = [dict(r, Counter_Name="WRITE_SIZE",
                  Counter_Value=1024 if "copy" in r["Kernel_Name"] else 50) for r in fetch]
    pf, pw = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(pf, CTR_COLS, fetch)
    write_csv(pw, CTR_COLS, write)
    md = traffic.summarize(str(pf), str(pw), 1.0, "wl", "cf", "cw")
    # (100 KiB x 2 + 50 KiB x 1) x 1024 bytes
    assert f"| bwd_dkdv | `spa::k_dkdv<128, 128>` | 100 | 50 | {250 * 1024:.4e} |" in md


def test_stall_breakdown_fractions(tmp_path):
    dur_ns, clk = 1000, 2.0e9          # 1 us at 2 GHz: 2000 cycles per SIMD
    cyc = 1024 * 2000                  # SIMD cycles of the dispatch
    name = "void spa::k_dkdv<128, 128>(int)"
    base = dict(Dispatch_Id=1, Kernel_Name=name, Start_Timestamp=0, End_Timestamp=dur_ns)
    grbm = 8 * clk * dur_ns * 1e-9     # summed over the 8 XCDs
    a = {"SQ_VALU_MFMA_BUSY_CYCLES": 0.30 * cyc, "SQ_VALU_MFMA_COEXEC_CYCLES": 0.10 * cyc,
         "SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 400.0, "SQ_WAIT_INST_ANY": 250.0,
         "SQ_ACTIVE_INST_ANY": 350.0, "GRBM_GUI_ACTIVE": grbm}
    # VALU issue 20 % of the SIMD cycles: 4 cycles per non-MFMA instruction
    b = {"SQ_INSTS_VALU": 0.20 * cyc / 4 + 1000.0, "SQ_INSTS_MFMA": 1000.0,
         "SQ_INSTS_LDS": 5.0, "SQ_INSTS_VALU_TRANS_F32": 7.0, "GRBM_GUI_ACTIVE": grbm}
    pa, pb = tmp_path / "a.csv", tmp_path / "b.csv"
    write_csv(pa, CTR_COLS, [dict(base, Counter_Name=k, Counter_Value=v) for k, v in a.items()])
    write_csv(pb, CTR_COLS, [dict(base, Counter_Name=k, Counter_Value=v) for k, v in b.items()])
    md = traffic.summarize_stalls(str(pa), str(pb), "wl", "ca", "cb")
    row = [ln for ln in md.splitlines() if ln.startswith("| `spa::k_dkdv")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    # MFMA only 20 %, VALU only 10 %, both 10 %, neither 60 %; waits 40 / 25 / 35 %
    assert cells[1:11] == ["1", "2.00", "20 %", "10 %", "10 %", "60 %", "40 %", "25 %", "35 %",
                           "7"]


@pytest.mark.parametrize("stage", list(traffic.STAGES))
def test_fingerprints_follow_the_sources(stage):
    f = traffic.fingerprint(stage)
    assert len(f) == 16 and f == traffic.fingerprint(stage)
