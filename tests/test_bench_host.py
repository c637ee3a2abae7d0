"""CPU checks of bench.py's host-side summaries (no GPU): the counter arithmetic behind the
roofline traffic and the MFMA-busy fractions, on small synthetic rocprofv3 CSV files, and the
recorded-traffic lookup keyed to the kernel code."""
import csv
import io
import os
import re
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (disp, name, grid, counter, value, ns) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": disp, "Agent_Id": "Agent 1", "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid, "Kernel_Id": 1, "Kernel_Name": name,
                        "Workgroup_Size": 256, "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 0,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 0, "Counter_Name": counter, "Counter_Value": value,
                        "Start_Timestamp": 1000, "End_Timestamp": 1000 + ns})


def run(fn, *args):
    buf = io.StringIO()
    with redirect_stdout(buf):
        fn(*args)
    return buf.getvalue()


def test_pmc_summary_scales_by_the_copy_probe(tmp_path):
    dense = "void safe::(anonymous namespace)::attn_fwd_kernel<96, false, false, 0, 2>(safe::AttnParams)"
    srsu = "void safe::(anonymous namespace)::attn_fwd_kernel<96, true, false, 0, 2>(safe::AttnParams)"
    copy = "void at::native::vectorized_elementwise_kernel<4, AddFunctor>(...)"
    gib_kib = float(1 << 20)   # counters are KiB per dispatch
    # FETCH reads half the copy's bytes (factor 2), WRITE the full (factor 1)
    write_csv(tmp_path / "fc.csv", [(1, copy, 1, "FETCH_SIZE", gib_kib / 2, 10)])
    write_csv(tmp_path / "wc.csv", [(1, copy, 1, "WRITE_SIZE", gib_kib, 10)])
    write_csv(tmp_path / "f.csv", [(1, dense, 1, "FETCH_SIZE", 1000.0, 10), (2, dense, 1, "FETCH_SIZE", 3000.0, 10),
                                   (3, srsu, 1, "FETCH_SIZE", 500.0, 10)])
    write_csv(tmp_path / "w.csv", [(1, dense, 1, "WRITE_SIZE", 100.0, 10), (2, dense, 1, "WRITE_SIZE", 300.0, 10),
                                   (3, srsu, 1, "WRITE_SIZE", 50.0, 10)])
    out = run(bench.pmc_summary, str(tmp_path / "f.csv"), str(tmp_path / "fc.csv"), str(tmp_path / "w.csv"),
              str(tmp_path / "wc.csv"))
    lines = dict((m.group(1), (int(m.group(2)), int(m.group(3)), int(m.group(4))))
                 for m in re.finditer(r"^traffic (\w+) bytes=(\d+) fetch=(\d+) write=(\d+)", out, flags=re.M))
    # dense: mean fetch 2000 KiB x 1024 x 2, mean write 200 KiB x 1024 x 1
    assert lines["dense"] == (2000 * 1024 * 2 + 200 * 1024, 2000 * 1024 * 2, 200 * 1024)
    assert lines["srsu"] == (500 * 1024 * 2 + 50 * 1024, 500 * 1024 * 2, 50 * 1024)
    assert "scale factors fetch 2.0000, write 1.0000" in out


def test_mfma_busy_summary_fraction_and_clock(tmp_path):
    name = "void safe::(anonymous namespace)::attn_fwd_kernel<96, false, false, 0, 2>(safe::AttnParams)"
    ns = 1_000_000                      # 1 ms launches
    cycles = 1_800_000                  # per XCD -> 1800 MHz
    rows = []
    for disp in (1, 2):
        rows += [(disp, name, 1024, "GRBM_GUI_ACTIVE", cycles * 8, ns),
                 (disp, name, 1024, "SQ_INSTS_MFMA", 30_000_000, ns),
                 (disp, name, 1024, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cycles * 1024, ns)]
    write_csv(tmp_path / "m.csv", rows)
    out = run(bench.mfma_busy_summary, str(tmp_path / "m.csv"))
    row = [ln for ln in out.splitlines() if "attn_fwd_kernel" in ln]
    assert len(row) == 1, out
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "1024" and cells[2] == "2"          # grid, launches
    assert cells[6] == "1800"                               # clock MHz
    assert cells[8] == "0.500"                              # busy fraction
    assert cells[7] == "983"                                # 3e7 x 32768 FLOP / 1 ms, in TFLOP/s


def test_mfma_flops_per_instruction_follows_the_kernel_shape():
    assert bench.mfma_flops_per_instruction("safe::attn_fwd_kernel<96, true, false, 0, 2, false>") == 32768
    assert bench.mfma_flops_per_instruction("safe::pcsp_accum_kernel<96>") == 32768
    assert bench.mfma_flops_per_instruction("safe::linear_ring_kernel<safe::LinCfg<4, 2, 2, 4> >") == 16384
    assert bench.mfma_flops_per_instruction("safe::linear_kernel<safe::LinCfg<2, 2, 2, 2> >") == 16384


def test_recorded_traffic_ignores_comment_edits(tmp_path, monkeypatch):
    src = tmp_path / "k.h"
    src.write_text("int f() {\n  return 1;  // one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "ATTN_SOURCES", ("k.h",))
    h0 = bench.attn_source_hash()
    src.write_text("// a new comment\nint f() {\n  return 1;  /* other */\n\n}\n")
    assert bench.attn_source_hash() == h0
    src.write_text("int f() {\n  return 2;\n}\n")
    assert bench.attn_source_hash() != h0


def test_stage_rooflines_bytes_and_fractions():
    """Per-stage roofline entries: algorithmic bytes of the HBM-bound stages from the shapes,
    achieved rates from the stage times, fractions of the MI355X peaks."""
    B, N, H, d, M, k = 2, 1000, 4, 64, 100, 250
    mask_bytes, kv_bytes = B * N * N * 2, 4 * B * N * H * d * 2
    fl_s, fl_c, fl_d = 4.0 * B * H * k * N * d, 4.0 * H * d * k * 150, 4.0 * B * H * N * N * d
    ms = {"classify": 0.5, "pcsp_accum": 0.1, "pcsp_select": 0.05, "kv_assemble": 0.2, "srsu_self": 1.0,
          "srsu_cross": 0.02, "dense": 4.0}
    r = bench.stage_rooflines(ms, B, N, H, d, M, k, mask_bytes, kv_bytes, fl_s, fl_c, fl_d)
    assert r["classify"]["bytes"] == mask_bytes and r["classify"]["bound"] == "hbm"
    assert r["pcsp_accum"]["bytes"] == B * N * H * d * 2 + B * M * H * d * 2 + B * M * 4 + 2 * B * N * 4
    assert r["srsu_cross"]["bytes"] == 2 * B * k * H * d * 2 + 2 * B * M * H * d * 2
    gbs = kv_bytes / 0.2e-3 / 1e9
    assert abs(r["kv_assemble"]["achieved"] - gbs) < 0.1 and abs(r["kv_assemble"]["frac"] - gbs / 8000.0) < 1e-4
    t = fl_d / 4.0e-3 / 1e12
    assert r["dense"]["bound"] == "mfma" and abs(r["dense"]["frac"] - t / 2500.0) < 1e-4
    assert r["pcsp_select"] == {"bound": "latency", "ms": 0.05}
    assert "mfma_tflops" not in r["pcsp_accum"]
    fl_p = 2.0 * N * H * d * 150
    r = bench.stage_rooflines(ms, B, N, H, d, M, k, mask_bytes, kv_bytes, fl_s, fl_c, fl_d, fl_p)
    assert r["pcsp_accum"]["flops"] == fl_p and abs(r["pcsp_accum"]["mfma_tflops"] - fl_p / 0.1e-3 / 1e12) < 0.01
