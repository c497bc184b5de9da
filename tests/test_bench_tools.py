"""CPU tests of bench.py's profile tools (host logic, no GPU): kernel labels
of rocprofv3 names, the clock table of a counter run, and the timed-step
window of the kernel-trace summary, on small synthetic CSV files."""
import csv
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))
import bench  # noqa: E402

COLUMN_MANGLED = ("_ZN5tpmlp12_GLOBAL__N_116gemm_ring_kernelINS0_7TileCfgILi256ELi192ELi8ELi2ELi1ELi1EEE"
                  "Lb1ELb0ELNS_3EpiE2EDF16bEEvNS_8GemmArgsEiii")


def test_kernel_label_demangles_and_names_tiles():
    assert bench.kernel_label(COLUMN_MANGLED) == \
        "gemm_ring_kernel<256x192, true, false, (Epi)2, bf16>"
    split = COLUMN_MANGLED.replace("ILi256ELi192ELi8ELi2ELi1ELi1EEE", "ILi128ELi96ELi4ELi2ELi1ELi2EEE")
    assert bench.kernel_label(split) == "gemm_ring_kernel<128x96 K-split, true, false, (Epi)2, bf16>"
    assert bench.kernel_label("void tpmlp::(anonymous namespace)::column_final_kernel(float const*, "
                              "float*, long, long)") == "column_final_kernel"
    # the profiler's own demangler reads two bf16 template arguments as "bool _Accum"
    assert bench.kernel_label("void tpmlp::(anonymous namespace)::shard_sum_kernel<bool _Accum, 8>"
                              "(bool _Accum const*, 8*, long, long, int)") == \
        "shard_sum_kernel<bf16, bf16, 8>"
    long_name = "x" * 300
    assert len(bench.kernel_label(long_name)) == 110


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size",
                                          "Start_Timestamp", "End_Timestamp", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_ingest_clock_groups_by_workgroups(tmp_path, capsys):
    rows = []
    did = 0
    # 256 workgroups: 100 us, 1.9e5 active cycles per XCD (1.9 GHz), busy 0.65 of all SIMDs
    # 128 workgroups: 80 us, 1.96e5 cycles per XCD (2.45 GHz), busy 0.33 of all SIMDs
    for wgs, ns, act, busy in ((256, 100_000, 190_000, 0.65), (128, 80_000, 196_000, 0.33)):
        for _ in range(8):
            did += 1
            base = dict(Dispatch_Id=did, Kernel_Name=COLUMN_MANGLED, Grid_Size=wgs * 512,
                        Workgroup_Size=512, Start_Timestamp=0, End_Timestamp=ns)
            rows.append({**base, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": act * 8})
            rows.append({**base, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                         "Counter_Value": busy * act * 1024})
    _write_counters(tmp_path / "c_counter_collection.csv", rows)
    bench.ingest_clock(str(tmp_path))
    out = capsys.readouterr().out.splitlines()
    by = {int(l.split("|")[1]): [c.strip() for c in l.strip("|").split("|")] for l in out[2:]}
    assert by[256][2:] == ["100.0", "1.90", "65.0%", "65.0%"]
    assert by[128][2:] == ["80.0", "2.45", "33.0%", "66.0%"]
    assert by[256][1] == "6"   # the first quarter of the dispatches is dropped


def test_trace_summary_counts_the_timed_steps(tmp_path, capsys):
    # 4 steps of (column GEMM 100 us, other kernel 50 us), 1 ms apart; warm-up 1, timed 2:
    # the window opens at the column GEMM of step 1 and closes 3 ms after that of step 2
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    with open(tmp_path / "b_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i in range(4):
            t0 = i * 10_000_000
            w.writerow({"Kernel_Name": COLUMN_MANGLED, "Start_Timestamp": t0,
                        "End_Timestamp": t0 + 100_000})
            w.writerow({"Kernel_Name": "void tpmlp::(anonymous namespace)::transpose16_kernel(int)",
                        "Start_Timestamp": t0 + 200_000, "End_Timestamp": t0 + 250_000})
    bench.trace_summary(str(tmp_path), 1, 2)
    out = capsys.readouterr().out.splitlines()
    blank = out.index("")
    rows = {l.split("`")[1]: [c.strip() for c in l.split("`")[2].strip().strip("|").split("|")]
            for l in out[2:blank]}
    col = rows["gemm_ring_kernel<256x192, true, false, (Epi)2, bf16>"]
    assert col[:2] == ["4", "100.0"] and col[4:] == ["2", "100.0"]
    tr = rows["transpose16_kernel"]
    assert tr[0] == "4" and tr[4] == "2"
    # then the launches by place in the step: two per step, not the bench step's eight
    places = out[blank + 3:]
    assert [p.split("|")[1].strip() for p in places[:2]] == ["1", "2"]
    assert places[0].split("|")[3].strip() == "-" and places[1].split("|")[4].strip() == "50.0"


def test_trace_summary_needs_exactly_one_column_kernel(tmp_path):
    with open(tmp_path / "b_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerow({"Kernel_Name": "other", "Start_Timestamp": 0, "End_Timestamp": 1})
    with pytest.raises(SystemExit):
        bench.trace_summary(str(tmp_path), 0, 1)


def test_code_text_drops_comments_and_layout():
    src = "int a; // one\n/* two\n three */  int   b;\n"
    assert bench.code_text(src) == "int a; int b;"
    # the same code with other comments and line breaks reads the same
    assert bench.code_text("int a;\n\n// x\nint b; /* y */") == bench.code_text(src)
    assert bench.code_text("int a; int c;") != bench.code_text(src)


def test_stored_counters_match_the_kernel_code():
    with open(bench.COUNTERS_FILE) as f:
        stored = json.load(f)
    assert stored["kernel_source_digest"] == bench.kernel_source_digest()
    assert bench.stored_traffic() == int(round(stored["hbm_bytes_per_launch"]))


def test_step_launch_table_names_launches_by_place():
    col = "gemm_ring_kernel_column"
    names = [col, "row", "dy", "tr", "dw2", "tr", "dw1", "dx"]
    runs = {}
    t = 0
    for step in range(3):
        for i, name in enumerate(names):
            runs.setdefault(name, []).append((t, 10.0 * (i + 1) + step))
            t += 1000
    starts = sorted(runs[col])
    lines = bench.step_launch_table(runs, starts)
    assert len(lines) == 2 + len(names) + 1
    # place 5 is dW2 (the second "tr" launch is place 6), means over the 3 steps
    assert "| 5 | `dw2` | " + bench.STEP_LAUNCHES[4] + " | 51.0 |" in lines[2 + 4]
    assert lines[-1].endswith("| " + f"{sum(10.0 * (i + 1) + 1 for i in range(8)):.1f}" + " | |")


def test_step_launch_table_flags_uneven_steps():
    runs = {"col": [(0, 5.0), (100, 5.0)], "x": [(50, 1.0)]}
    lines = bench.step_launch_table(runs, sorted(runs["col"]))
    assert lines == ["(steps hold different launch counts: [1, 2])"]


def test_stored_counters_record_their_commands():
    with open(bench.COUNTERS_FILE) as f:
        stored = json.load(f)
    assert "FETCH_SIZE" in stored["commands"] and "WRITE_SIZE" in stored["commands"]
    assert "--ingest-counters" in stored["commands"]
