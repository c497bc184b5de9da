"""Throughput of one tensor-parallel rank's MLP shard, forward + backward,
on one MI355X.

Workload: the GPT-3-shaped shard (h = 12288, ffn = 49152, t = 8, rank 0,
2048 tokens, bf16, seeded synthetic inputs).  One step is the whole path:
  column GEMM + bias + GeLU (pre-activation saved)      tp_column_linear
  row GEMM, fp32 partial output                        tp_row_linear
  backward: dY (GeLU' epilogue), dW2, dW1, dX, db1     tp_mlp_shard_bwd
The first two calls are exactly what tp_mlp_shard_fwd issues; calling them
separately lets HIP events on the launch stream time the column GEMM alone.
The shard-sum stand-in for the all-reduce is timed on its own workload (the
8 fp32 partial outputs of the h = 8192 full-layer emulation).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "TFLOP/s per TP-shard MLP fwd+bwd (bf16) and % of MI355X MFMA peak"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters_column_gemm_gpt3.json")
# How the stored HBM counters are taken (recorded with them unless given
# otherwise): two passes over a short bench run, two over a plain copy.
COUNTER_COMMANDS = (
    "B='python3 bench.py --steps 2 --warmup 1 --warmup-ms 0 --cpu-seconds 0 --no-reduce "
    "--no-vendor --no-attention --no-sp --no-full-layer --no-small'; "
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o c -- $B; "
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o c -- $B; "
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_cfetch -o c -- "
    "python3 bench.py --copy-calibration 3; "
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_cwrite -o c -- "
    "python3 bench.py --copy-calibration 3; "
    "python3 bench.py --ingest-counters gpurun_out/pmc_fetch gpurun_out/pmc_write "
    "gpurun_out/pmc_cfetch gpurun_out/pmc_cwrite")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C++ source without its comments and with runs of blank space folded to
    one space: what a compiler sees of it (the sources hold no string
    literal with a comment marker in it)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_digest() -> str:
    """Digest of the GEMM kernel sources' code (comments and layout left
    out); stored HBM counters are used only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_transformer_layer_columnparallel_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("gemm") or name in ("common.h", "epilogue.h"):
            with open(os.path.join(csrc, name)) as f:
                h.update((name + "\n" + code_text(f.read())).encode())
    return h.hexdigest()[:16]


def stored_traffic():
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_digest") != kernel_source_digest():
        return None
    b = c.get("hbm_bytes_per_launch")
    return None if b is None else int(round(b))


# The column GEMM: the 256 x 192-tile instance with the bias + GeLU epilogue
# and bf16 results, as rocprofv3 names it (mangled, or demangled; every part
# of a key must match).
COLUMN_KERNEL_KEYS = (("gemm_ring_kernel",
                       "TileCfgILi256ELi192ELi8ELi2ELi1ELi1EEELb1ELb0ELNS_3EpiE2EDF16b"),
                      ("gemm_ring_kernel<", "TileCfg<256, 192, 8, 2, 1, 1>, true, false, "
                                            "(tpmlp::Epi)2, __bf16>"))
COPY_KERNEL_KEYS = (("shard_concat_kernel",),)


def _counter_per_dispatch(csv_dir: str, counter: str, keys) -> float:
    """Mean over dispatches of `counter` (summed over its instances) for the
    kernels whose name contains one of `keys`, from a rocprofv3 --pmc CSV."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                if not any(all(k in row["Kernel_Name"] for k in key) for key in keys):
                    continue
                per[row["Dispatch_Id"]] = per.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} samples for {keys} under {csv_dir}")
    return sum(per.values()) / len(per)


def ingest_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands):
    """Turns four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the bench
    and of the calibration copy) into HBM bytes per launch of the column GEMM.
    The counters report KiB; each is scaled by the ratio of the copy's known
    byte count to what the same counter reads for the copy."""
    copy_bytes = COPY_ROWS * COPY_COLS * 4
    f_col = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", COLUMN_KERNEL_KEYS)
    w_col = _counter_per_dispatch(write_dir, "WRITE_SIZE", COLUMN_KERNEL_KEYS)
    f_cp = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", COPY_KERNEL_KEYS)
    w_cp = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", COPY_KERNEL_KEYS)
    f_scale = copy_bytes / (f_cp * 1024)
    w_scale = copy_bytes / (w_cp * 1024)
    read_b = f_col * 1024 * f_scale
    write_b = w_col * 1024 * w_scale
    out = {"kernel": "gemm_ring_kernel: NN, bias + GeLU epilogue, bf16 output", "kernel_source_digest": kernel_source_digest(),
           "fetch_kib_raw": f_col, "write_kib_raw": w_col,
           "copy_bytes": copy_bytes, "copy_fetch_kib_raw": f_cp, "copy_write_kib_raw": w_cp,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": write_b,
           "hbm_bytes_per_launch": read_b + write_b, "commands": commands}
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


TILE_NAMES = {"TileCfg<256, 192, 8, 2, 1, 1>": "256x192", "TileCfg<256, 192, 8, 4, 1, 1>": "256x192tn",
              "TileCfg<128, 96, 4, 2, 2, 1>": "128x96", "TileCfg<128, 96, 4, 2, 1, 2>": "128x96 K-split"}


def kernel_label(name: str) -> str:
    """A short readable label for a kernel name from a rocprofv3 table:
    demangled (c++filt) when it is mangled, without namespaces, `void` and
    the parameter list, tile configurations by their tile size."""
    import subprocess
    if name.startswith("_Z"):
        try:
            # c++filt does not know the bf16 builtin's code; spell it as a
            # vendor type of the same name
            name = subprocess.run(["c++filt", name.replace("DF16b", "u6__bf16")],
                                  capture_output=True, text=True,
                                  timeout=10).stdout.strip() or name
        except (OSError, subprocess.SubprocessError):
            pass
    name = name.replace("tpmlp::(anonymous namespace)::", "").replace("tpmlp::", "")
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    if name.endswith(")") and "(" in name:          # drop the parameter list
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    for cfg, short in TILE_NAMES.items():
        name = name.replace(cfg, short)
    # the profiler's own demangler reads two bf16 template arguments as this
    name = name.replace("bool _Accum", "bf16, bf16")
    name = name.replace("__bf16", "bf16").replace("unsigned short", "u16")
    return name if len(name) <= 110 else name[:107] + "..."


COPY_ROWS, COPY_COLS = 8192, 8192

MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE", "GRBM_COUNT")


def ingest_mfma(pmc_dir: str, simds: int = 1024, xcds: int = 8):
    """Markdown table from one rocprofv3 --pmc run of MFMA_COUNTERS: per GEMM
    kernel instance, the mean per dispatch of the bf16 MFMA work (the
    counter counts multiply and add operations / 512), the MFMA unit's busy
    fraction (busy cycles summed over the SIMDs / (GPU-active cycles of one
    XCD x SIMDs)), the GPU-active cycles of one XCD and the engine clock they
    imply over the dispatch's duration.  rocprofv3 reports each counter as
    one value per dispatch, summed over its instances; GRBM_GUI_ACTIVE is
    summed over the XCDs, hence divided by their count."""
    import csv
    import glob
    disp = {}
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if "gemm" not in row["Kernel_Name"]:
                    continue
                d = disp.setdefault(row["Dispatch_Id"], {
                    "name": row["Kernel_Name"],
                    "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
                c, v = row["Counter_Name"], float(row["Counter_Value"])
                d[c] = d.get(c, 0.0) + v
    if not disp:
        raise SystemExit(f"no GEMM dispatches under {pmc_dir}")
    per = {}
    for d in disp.values():
        per.setdefault(d["name"], []).append(d)
    print("| kernel | dispatches | bf16 MFMA GFLOP per dispatch | MFMA busy | GPU-active cycles per XCD | clock GHz | duration us |")
    print("|---|---|---|---|---|---|---|")
    for name, ds in sorted(per.items(), key=lambda kv: -len(kv[1])):
        mean = lambda k: sum(d.get(k, 0.0) for d in ds) / len(ds)
        act, ns = mean("GRBM_GUI_ACTIVE") / xcds, mean("ns")
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (act * simds) if act else float("nan")
        short = kernel_label(name)
        print(f"| `{short}` | {len(ds)} | {mean('SQ_INSTS_VALU_MFMA_MOPS_BF16') * 512 / 1e9:.1f} | "
              f"{100 * busy:.1f}% | {act:.0f} | {act / ns:.2f} | {ns / 1e3:.1f} |")



def ingest_pmc(pmc_dir: str, xcds: int = 8, cus: int = 256):
    """Markdown table from one rocprofv3 --pmc run: per GEMM kernel instance
    (and the activation transpose), the mean per dispatch of every counter
    collected (rocprofv3 sums a counter over its hardware instances), and
    each one divided by the GPU-active cycles of all CUs (GRBM_GUI_ACTIVE,
    summed over the XCDs, / XCDs x CUs) when that counter was collected: for
    a counter of cycles per CU or per SQ that is the fraction of the
    kernel's active time it covers."""
    import csv
    import glob
    disp = {}
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                k = row["Kernel_Name"]
                if "gemm" not in k and "transpose" not in k:
                    continue
                d = disp.setdefault(row["Dispatch_Id"], {
                    "name": k, "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
                c, v = row["Counter_Name"], float(row["Counter_Value"])
                d[c] = d.get(c, 0.0) + v
    if not disp:
        raise SystemExit(f"no GEMM dispatches under {pmc_dir}")
    per = {}
    for d in disp.values():
        per.setdefault(d["name"], []).append(d)
    names = sorted({c for d in disp.values() for c in d if c not in ("name", "ns")})
    print("| kernel | dispatches | duration us | " + " | ".join(names) + " |")
    print("|---|---|---|" + "---|" * len(names))
    for name, ds in sorted(per.items(), key=lambda kv: -len(kv[1])):
        mean = lambda k: sum(d.get(k, 0.0) for d in ds) / len(ds)
        act = mean("GRBM_GUI_ACTIVE") / xcds
        cells = []
        for c in names:
            v = mean(c)
            frac = f" ({v / (act * cus):.3f})" if act and c != "GRBM_GUI_ACTIVE" else ""
            cells.append(f"{v:.4g}{frac}")
        short = kernel_label(name)
        print(f"| `{short}` | {len(ds)} | {mean('ns') / 1e3:.1f} | " + " | ".join(cells) + " |")


def copy_calibration(reps: int):
    """A plain device copy of known size (8192 x 8192 fp32 = 256 MiB read and
    written), issued through the library's concatenation with t = 1."""
    import torch
    from tensor_transformer_layer_columnparallel_amd import binding as B
    src = torch.randn(1, COPY_ROWS, COPY_COLS, device="cuda")
    dst = torch.empty(COPY_ROWS, COPY_COLS, device="cuda")
    for _ in range(reps):
        B.tp_shard_reduce(src, dst, COPY_ROWS, COPY_COLS, 1, B.TP_REDUCE_CONCAT, torch.float32,
                          torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(src[0], dst)
    log(f"copy calibration: {reps} copies of {COPY_ROWS * COPY_COLS * 4} bytes")


def warm(fn, ms: float = 80.0) -> int:
    """Calls fn back to back for about `ms` milliseconds of device time, so
    that the measurement after it starts at the sustained engine clock.
    Returns the number of calls."""
    import torch
    t0, calls = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        calls += 4
        torch.cuda.synchronize()
    return calls


def trace_summary(trace_dir: str, warmup: int, steps: int):
    """Markdown table of kernel durations (microseconds) from the
    *kernel_trace.csv that rocprofv3 --kernel-trace writes under trace_dir
    for a bench run with `warmup` warm-up and `steps` timed steps: calls,
    mean, min and max over all dispatches of each kernel, and calls and mean
    inside the timed steps.  The step loop runs first, one column GEMM per
    step, so the timed steps are the window from the start of the column
    GEMM's dispatch number `warmup` (from 0) to 3 ms after the start of
    number `warmup + steps - 1` (the rest of that step)."""
    import csv
    import glob
    runs = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                t0, t1 = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
                runs.setdefault(row["Kernel_Name"], []).append((t0, (t1 - t0) / 1e3))
    if not runs:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    col = [v for k, v in runs.items()
           if any(all(x in k for x in key) for key in COLUMN_KERNEL_KEYS)]
    if len(col) != 1:
        raise SystemExit("the column GEMM kernel is not in the trace exactly once")
    col = sorted(col[0])
    if len(col) < warmup + steps:
        raise SystemExit("fewer column GEMM dispatches than warm-up + timed steps")
    w0, w1 = col[warmup][0], col[warmup + steps - 1][0] + 3_000_000
    rows = []
    for name, v in runs.items():
        ds = [d for _, d in v]
        tw = [d for t, d in v if w0 <= t <= w1]
        rows.append((sum(ds), name, len(ds), sum(ds) / len(ds), min(ds), max(ds), len(tw),
                     sum(tw) / len(tw) if tw else float("nan")))
    rows.sort(reverse=True)
    print(f"| kernel | calls | mean us | min us | max us | calls in the timed steps | mean us in the timed steps |")
    print("|---|---|---|---|---|---|---|")
    for _, name, c, mean, mn, mx, nt, tmean in rows:
        short = kernel_label(name)
        print(f"| `{short}` | {c} | {mean:.1f} | {mn:.1f} | {mx:.1f} | {nt} | {tmean:.1f} |")
    print()
    for line in step_launch_table(runs, col[warmup:warmup + steps]):
        print(line)


# The launches of one bench step in issue order: tp_column_linear, then
# tp_row_linear, then tp_mlp_shard_bwd (transposed-operand weight gradients).
STEP_LAUNCHES = ("column GEMM + bias + GeLU, Y saved (a1+a2)", "row GEMM, fp32 partial (a3)",
                 "dY with GeLU' and db1's row-block partials (a5)",
                 "H_i transpose, with db1's last pass in extra blocks",
                 "dW2_i = (H_i^T) dZ (a6)", "dY_i transpose",
                 "dW1_i^T = (dY_i^T) X, stored transposed (a7)", "dX_i = dY_i W1_i^T (a8)")


def step_launch_table(runs, col_starts):
    """Markdown lines: the mean duration of each launch of the timed steps by
    its place in the step.  A step runs from the start of one column-GEMM
    dispatch (`col_starts`, (start, duration) pairs) to the next or, for the
    last, 3 ms on.  Launches are named after STEP_LAUNCHES when every step
    has that many."""
    launches = sorted((t, d, name) for name, v in runs.items() for t, d in v)
    starts = [t for t, _ in col_starts]
    ends = starts[1:] + [starts[-1] + 3_000_000]
    steps = [[(d, name) for t, d, name in launches if a <= t < b] for a, b in zip(starts, ends)]
    counts = {len(s) for s in steps}
    if len(counts) != 1:
        return [f"(steps hold different launch counts: {sorted(counts)})"]
    n = counts.pop()
    named = n == len(STEP_LAUNCHES)
    lines = ["| place in the step | kernel | product | mean us in the timed steps | share of the step |",
             "|---|---|---|---|---|"]
    means = [sum(s[i][0] for s in steps) / len(steps) for i in range(n)]
    total = sum(means)
    for i in range(n):
        lines.append(f"| {i + 1} | `{kernel_label(steps[0][i][1])}` | "
                     f"{STEP_LAUNCHES[i] if named else '-'} | {means[i]:.1f} | "
                     f"{100 * means[i] / total:.1f}% |")
    lines.append(f"| | | sum of the kernel durations | {total:.1f} | |")
    return lines


def max_engine_clock_mhz():
    """The GPU agent's maximum engine clock as rocminfo reports it (None if
    rocminfo is unavailable)."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    clock, is_gpu = None, False
    for line in txt.splitlines():
        line = line.strip()
        if line.startswith("Device Type:"):
            is_gpu = "GPU" in line
        elif is_gpu and line.startswith("Max Clock Freq. (MHz):"):
            clock = int(line.split(":")[1].split()[0])
            break
    return clock


def vendor_matmul_context(T, h, n, reps=10):
    """For context only (not the product path): torch.matmul (the vendor BLAS)
    on the step's six products with bf16 outputs and no epilogue."""
    import torch
    bf, dev = torch.bfloat16, "cuda"
    g = torch.Generator(device=dev).manual_seed(1)
    r = lambda *sh: torch.randn(*sh, device=dev, generator=g).to(bf)
    X, W1, H, W2, dZ, dY = r(T, h), r(h, n), r(T, n), r(n, h), r(T, h), r(T, n)
    prods = [lambda: X @ W1, lambda: H @ W2, lambda: dZ @ W2.t(), lambda: H.t() @ dZ,
             lambda: X.t() @ dY, lambda: dY @ W1.t()]
    warm(lambda: [f() for f in prods])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for f in prods:
            f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"what": "torch.matmul (vendor BLAS), same six products, bf16 out, no epilogue",
            "ms_per_step": round(ms, 4), "tflops": round(12.0 * T * h * n / (ms * 1e-3) / 1e12, 2)}


def attention_shard(B, aw, stream, sptr, reps=10):
    """The attention block's two projections of one rank (QKV column-parallel
    on head boundaries, output projection row-parallel with an fp32 partial)
    at the GPT-3 shape, timed with HIP events on the launch stream."""
    import torch
    from tensor_transformer_layer_columnparallel_amd import synth
    r = aw.ranks[0]
    d = synth.make_attn_inputs(aw)
    s = synth.attn_shard(aw, d, r)
    dev = "cuda"
    X, Wqkv, bqkv = d["X"].to(dev), s["Wqkv"].to(dev), s["bqkv"].to(dev)
    O, Wo = s["O"].to(dev), s["Wo"].to(dev)
    bf = torch.bfloat16
    Y = torch.empty(aw.T, aw.qkv_width, dtype=bf, device=dev)
    Z = torch.empty(aw.T, aw.h, dtype=torch.float32, device=dev)
    qkv = lambda: B.tp_column_linear(X, Wqkv, bqkv, Y, None, aw.T, aw.h, 3 * aw.h, aw.t, r, bf,
                                     bf, B.TP_ACT_NONE, stream=sptr)
    proj = lambda: B.tp_row_linear(O, Wo, Z, aw.T, aw.h, aw.h, aw.t, r, bf, torch.float32,
                                   stream=sptr)
    # backward of both projections (dX, dW, and db for QKV), from drawn
    # output gradients
    g = synth.make_attn_grads(aw)
    dQ = g["dQKV"][:, synth.qkv_columns(aw, r)].contiguous().to(dev)
    dZ = g["dZ"].to(dev)
    f32 = torch.float32
    dX = torch.empty(aw.T, aw.h, dtype=f32, device=dev)
    dWq = torch.empty(aw.h, aw.qkv_width, dtype=f32, device=dev)
    dbq = torch.empty(aw.qkv_width, dtype=f32, device=dev)
    dO = torch.empty(aw.T, aw.w, dtype=f32, device=dev)
    dWo = torch.empty(aw.w, aw.h, dtype=f32, device=dev)
    qkv_bwd = lambda: B.tp_linear_bwd(X, Wqkv, dQ, dX, dWq, dbq, aw.T, aw.h, aw.qkv_width, bf,
                                      stream=sptr)
    proj_bwd = lambda: B.tp_linear_bwd(O, Wo, dZ, dO, dWo, None, aw.T, aw.w, aw.h, bf,
                                       stream=sptr)
    times = []
    for f in (qkv, proj, qkv_bwd, proj_bwd):
        warm(f)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    fl = aw.qkv_flops() + aw.out_flops()
    return {"workload": f"gpt3-shaped attention projections, rank {r} of t={aw.t}: "
                        f"QKV [{aw.T},{aw.h}]x[{aw.h},{aw.qkv_width}] + bias (head-boundary "
                        f"shard), out-proj [{aw.T},{aw.w}]x[{aw.w},{aw.h}] -> fp32",
            "qkv_ms": round(times[0], 4), "out_proj_ms": round(times[1], 4),
            "qkv_tflops": round(aw.qkv_flops() / (times[0] * 1e-3) / 1e12, 2),
            "out_proj_tflops": round(aw.out_flops() / (times[1] * 1e-3) / 1e12, 2),
            "tflops": round(fl / ((times[0] + times[1]) * 1e-3) / 1e12, 2),
            "backward": {"what": "tp_linear_bwd of both projections: dX, dW (and db for QKV), "
                                 "two products each",
                         "qkv_ms": round(times[2], 4), "out_proj_ms": round(times[3], 4),
                         "tflops": round(2 * fl / ((times[2] + times[3]) * 1e-3) / 1e12, 2)}}


def sequence_parallel(B, stream, sptr, reps=50):
    """The sequence-parallel stand-ins at the GPT-3 shape (t = 8, 2048
    tokens, h = 12288), each HBM-bound and reported in GB/s: ReduceScatter of
    the eight fp32 row-layer partials to one rank's 256 tokens, layer norm of
    that shard (fp32 in, bf16 out), and the token AllGather of eight bf16
    shards."""
    import torch
    T, h, t = 2048, 12288, 8
    Tr = T // t
    bf, f32 = torch.bfloat16, torch.float32
    # Each repetition works on data no earlier repetition touched, so that
    # the 256 MB last-level cache does not serve it: the reduce-scatter walks
    # the ranks (8 blocks of 100 MB), the layer norm and the concatenation
    # rotate through copies of their buffers (600 and 800 MB).
    parts = torch.randn(t, T, h, device="cuda")
    rs = torch.empty(Tr, h, device="cuda")
    n_ln, n_cat = 32, 8
    ln_in = [torch.randn(Tr, h, device="cuda") for _ in range(n_ln)]
    ln_out = [torch.empty(Tr, h, dtype=bf, device="cuda") for _ in range(n_ln)]
    gam = torch.ones(h, dtype=bf, device="cuda")
    bet = torch.zeros(h, dtype=bf, device="cuda")
    shards = [torch.randn(t, Tr, h, device="cuda").to(bf) for _ in range(n_cat)]
    full = [torch.empty(T, h, dtype=bf, device="cuda") for _ in range(n_cat)]
    k = [0]

    def nxt(n):
        k[0] += 1
        return k[0] % n

    # The calls pass plain device addresses (the binding's unchecked form):
    # checking torch tensors costs about 7 us of host time per call, as long
    # as the layer norm itself, which would then time the host, not the GPU.
    a = lambda x: x.data_ptr()
    a_parts, a_rs, a_gam, a_bet = a(parts), a(rs), a(gam), a(bet)
    a_in, a_out = [a(x) for x in ln_in], [a(x) for x in ln_out]
    a_sh, a_full = [a(x) for x in shards], [a(x) for x in full]
    ops = {
        "reduce_scatter": (lambda: B.tp_shard_reduce_scatter(a_parts, a_rs, T, h, t, nxt(t), f32,
                                                             f32, stream=sptr),
                           (t * Tr * h + Tr * h) * 4),
        "layernorm": (lambda: (lambda i: B.tp_layernorm(a_in[i], a_gam, a_bet, a_out[i], Tr, h,
                                                        1e-5, f32, bf, stream=sptr))(nxt(n_ln)),
                      Tr * h * 4 + Tr * h * 2 + 2 * h * 2),
        "concat_tokens": (lambda: (lambda i: B.tp_shard_reduce(a_sh[i], a_full[i], Tr, h, t,
                                                               B.TP_REDUCE_CONCAT_TOKENS, bf,
                                                               bf, stream=sptr))(nxt(n_cat)),
                          2 * T * h * 2),
        # the first two in one pass: the rank's rows summed as they are loaded
        # and normalised without writing the fp32 sum
        "reduce_scatter_layernorm": (lambda: B.tp_shard_reduce_scatter_layernorm(
            a_parts, a_gam, a_bet, a_out[nxt(n_ln)], T, h, t, nxt(t), 1e-5, f32, bf,
            stream=sptr),
            (t * Tr * h) * 4 + Tr * h * 2 + 2 * h * 2),
        # context, not the product path: torch's fp32 -> bf16 copy of the same
        # rows (no reduction), the floor of any one pass over the layer norm's
        # bytes timed this way
        "context_cast": (lambda: (lambda i: ln_out[i].copy_(ln_in[i]))(nxt(n_ln)),
                         Tr * h * 4 + Tr * h * 2),
    }
    out = {"workload": f"t={t}, {T} tokens, h={h}: ReduceScatter of {t} fp32 partials to "
                       f"{Tr} tokens; layer norm of the shard (fp32 -> bf16); token "
                       f"AllGather of {t} bf16 shards; ReduceScatter and layer norm fused "
                       f"(bf16 out); every repetition on data not in the last-level cache; "
                       f"context_cast: torch's fp32 -> bf16 copy of the shard, for scale",
           "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    for name, (f, nbytes) in ops.items():
        warm(f)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "bytes": nbytes,
                     "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    return out


def full_layer(B, stream, sptr, reps=5):
    """The full-layer emulation (h = 8192, ffn = 28672, t = 8, 4096 tokens,
    no bias): every rank's shard forward, then the fp32 shard sum, once with
    one tp_mlp_shard_fwd call per rank in rank order and once with all
    shards batched into two launches (tp_mlp_layer_fwd).  Seeded random
    inputs drawn on the device (same distributions as the parity cases)."""
    import torch
    from tensor_transformer_layer_columnparallel_amd import configs
    w = configs.FULL_LAYER_8
    T, h, n, t = w.T, w.h, w.n, w.t
    bf, f32 = torch.bfloat16, torch.float32
    g = torch.Generator(device="cuda").manual_seed(0)
    X = torch.randn(T, h, device="cuda", generator=g).to(bf)
    W1 = (torch.randn(t, h, n, device="cuda", generator=g) * w.std_w).to(bf)
    W2 = (torch.randn(t, n, h, device="cuda", generator=g) * w.std_w).to(bf)
    H = torch.empty(t, T, n, dtype=bf, device="cuda")
    parts = torch.empty(t, T, h, dtype=f32, device="cuda")
    Z = torch.empty(T, h, dtype=f32, device="cuda")

    def seq():
        for r in range(t):
            B.tp_mlp_shard_fwd(X, W1[r], None, W2[r], H[r], None, parts[r], T, h, w.ffn, t, r,
                               bf, stream=sptr)
        B.tp_shard_reduce(parts, Z, T, h, t, B.TP_REDUCE_SUM, f32, f32, stream=sptr)

    def batched():
        B.tp_mlp_layer_fwd(X, W1, None, W2, H, None, parts, T, h, w.ffn, t, bf, stream=sptr)
        B.tp_shard_reduce(parts, Z, T, h, t, B.TP_REDUCE_SUM, f32, f32, stream=sptr)

    out = {"workload": f"full-layer emulation, h={h}, ffn={w.ffn}, t={t}, {T} tokens, no bias: "
                       f"every shard's forward, then the fp32 shard sum",
           "flops": w.fwd_flops()}
    for name, f in (("sequential", seq), ("batched", batched)):
        warm(f)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "tflops": round(w.fwd_flops() / (ms * 1e-3) / 1e12, 2)}
    out["sequential"]["what"] = "tp_mlp_shard_fwd per rank in rank order, then tp_shard_reduce"
    out["batched"]["what"] = "tp_mlp_layer_fwd (all shards in two launches), then tp_shard_reduce"
    return out


def small_configs(B, stream, reps=50):
    """The two small workloads, each timed after 80 ms of warm-up calls with
    HIP events on the launch stream, both as `reps` eager calls and as the
    same calls captured once in a HIP graph and replayed (the graph removes
    the host's launch gaps, which dominate at these sizes):
      tiny fp32 MLP, t = 2: both shards' forward (tp_mlp_shard_fwd per shard,
        and both at once with tp_mlp_layer_fwd) and the fp32 shard sum
        (tp_shard_reduce) of the two partials;
      column-parallel linear 768 -> 3072, t = 4, rank 0, bf16: one
        tp_column_linear call, X [4096, 768] x W_0 [768, 768], bf16 output."""
    import torch
    from tensor_transformer_layer_columnparallel_amd import configs, synth
    f32, bf = torch.float32, torch.bfloat16
    dev = "cuda"

    w1 = configs.TINY_F32
    d = synth.make_inputs(w1)
    X = d["X"].to(dev)
    W1 = [d["W1"][r].to(dev) for r in w1.ranks]
    b1 = [d["b1"][r].to(dev) for r in w1.ranks]
    W2 = [d["W2"][r].to(dev) for r in w1.ranks]
    H = [torch.empty(w1.T, w1.n, device=dev) for _ in w1.ranks]
    parts = torch.empty(w1.t, w1.T, w1.h, device=dev)
    Z = torch.empty(w1.T, w1.h, device=dev)

    def c1(st):
        for r in w1.ranks:
            B.tp_mlp_shard_fwd(X, W1[r], b1[r], W2[r], H[r], None, parts[r], w1.T, w1.h, w1.ffn,
                               w1.t, r, f32, stream=st.cuda_stream)
        B.tp_shard_reduce(parts, Z, w1.T, w1.h, w1.t, B.TP_REDUCE_SUM, f32, f32,
                          stream=st.cuda_stream)

    W1s, b1s, W2s = torch.stack(W1), torch.stack(b1), torch.stack(W2)
    Hs = torch.empty(w1.t, w1.T, w1.n, device=dev)

    def c1_batched(st):
        B.tp_mlp_layer_fwd(X, W1s, b1s, W2s, Hs, None, parts, w1.T, w1.h, w1.ffn, w1.t, f32,
                           stream=st.cuda_stream)
        B.tp_shard_reduce(parts, Z, w1.T, w1.h, w1.t, B.TP_REDUCE_SUM, f32, f32,
                          stream=st.cuda_stream)

    w2 = configs.COLUMN_768
    d2 = synth.make_inputs(w2)
    X2, Wc, bc = d2["X"].to(dev), d2["W1"][0].to(dev), d2["b1"][0].to(dev)
    Y2 = torch.empty(w2.T, w2.n, dtype=bf, device=dev)

    # plain device addresses: the tensor checks' host time (about 7 us a
    # call) would otherwise come close to the kernel's own
    c2_args = (X2.data_ptr(), Wc.data_ptr(), bc.data_ptr(), Y2.data_ptr())

    def c2(st):
        B.tp_column_linear(*c2_args, None, w2.T, w2.h, w2.ffn, w2.t, 0, bf, bf,
                           B.TP_ACT_NONE, stream=st.cuda_stream)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm(lambda: fn(stream))
        e0.record(stream)
        for _ in range(reps):
            fn(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) / reps * 1e3
        # The same calls captured in a HIP graph on a side stream, replayed on
        # the launch stream.
        g, cap = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap):
            for _ in range(reps):
                fn(cap)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            warm(g.replay)
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return eager_us, e0.elapsed_time(e1) / reps * 1e3

    out = {}
    for name, f, flops, what in (
            ("tiny_mlp_f32_t2", c1, w1.fwd_flops(),
             f"tiny fp32 MLP, t={w1.t}, both shards: X[{w1.T},{w1.h}], W1_r[{w1.h},{w1.n}], "
             f"W2_r[{w1.n},{w1.h}]; two tp_mlp_shard_fwd + tp_shard_reduce SUM (5 kernels)"),
            ("tiny_mlp_f32_t2_batched", c1_batched, w1.fwd_flops(),
             f"the same, both shards in one tp_mlp_layer_fwd + tp_shard_reduce SUM (3 kernels)"),
            ("column_linear_768", c2, w2.fwd_flops(),
             f"column-parallel linear 768->3072, t={w2.t}, rank 0: X[{w2.T},{w2.h}] x "
             f"W_0[{w2.h},{w2.n}], bf16 out, no activation; one tp_column_linear")):
        eager_us, graph_us = timed(f)
        tf = flops / (graph_us * 1e-6) / 1e12
        tf_eager = flops / (eager_us * 1e-6) / 1e12
        out[name] = {"workload": what, "flops": flops, "eager_us": round(eager_us, 2),
                     "graph_us": round(graph_us, 2), "tflops_eager": round(tf_eager, 3),
                     "pct_peak_eager": round(100 * tf_eager / PEAK_BF16_TFLOPS, 2),
                     "tflops_graph": round(tf, 3),
                     "pct_peak_graph": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    out["reps"] = reps
    return out


def cpu_baseline(w, d_h, seconds: float):
    """Times the fp64 oracle on a bounded sample: chunks of 32 token rows of
    the same workload, each chunk a full forward + backward (6 products) of
    those rows, until `seconds` have passed."""
    import numpy as np
    import torch

    import oracle
    oracle.build(force=False)
    f64 = lambda x: np.ascontiguousarray(x.to(torch.float64).numpy())
    X, dZ = f64(d_h["X"]), f64(d_h["dZ"])
    W1, b1, W2 = f64(d_h["W1"][0]), f64(d_h["b1"][0]), f64(d_h["W2"][0])
    chunk, done, flops = 32, 0, 0.0
    t0 = time.perf_counter()
    while done + chunk <= w.T:
        rows = slice(done, done + chunk)
        oracle.mlp_shard_bwd(X[rows], W1, b1, W2, dZ[rows])
        done += chunk
        flops += 6 * 2.0 * chunk * w.h * w.n
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 forward+backward of token rows 0..{done - 1} of {w.T} "
                      f"({done // chunk} chunks of {chunk}), {el:.1f} s wall"}


BUSY_CU_SHAPES = ((2048, 12288, 6144), (1536, 12288, 6144), (1024, 12288, 6144), (2048, 12288, 4608))


def busy_cus_sweep(rounds: int = 2, reps: int = 40):
    """The column product (bias + GeLU, pre-activation saved, K = 12288) with
    256, 192 and 128 tiles of 256 x 192 (T = 2048, 1536, 1024 at n = 6144)
    and the QKV shard's shape (192 tiles): median time per launch over `reps`
    event-timed launches after 150 ms of warm-up calls.  Under rocprofv3
    --pmc the dispatches are told apart by their workgroup counts."""
    import torch
    from tensor_transformer_layer_columnparallel_amd import binding as B
    dev, bf = "cuda", torch.bfloat16
    out = []
    for rnd in range(rounds):
        for T, h, n in BUSY_CU_SHAPES:
            g = torch.Generator(device=dev).manual_seed(3)
            X = torch.randn(T, h, device=dev, generator=g).to(bf)
            W = (0.02 * torch.randn(h, n, device=dev, generator=g)).to(bf)
            b = (0.02 * torch.randn(n, device=dev, generator=g)).to(bf)
            H = torch.empty(T, n, device=dev, dtype=bf)
            Y = torch.empty(T, n, device=dev, dtype=bf)
            f = lambda: B.tp_column_linear(X, W, b, H, Y, T, h, n, 1, 0, bf, bf,
                                           B.TP_ACT_GELU_TANH)
            warm(f, 150.0)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for e0, e1 in ev:
                e0.record()
                f()
                e1.record()
            torch.cuda.synchronize()
            ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
            us = ts[len(ts) // 2]
            tiles = ((T + 255) // 256) * ((n + 191) // 192)
            r = {"round": rnd, "T": T, "h": h, "n": n, "tiles": tiles, "median_us": round(us, 1),
                 "tflops": round(2 * T * h * n / us / 1e6, 1)}
            out.append(r)
            print(json.dumps(r), flush=True)
    return out


def column_load(T: int, seconds: float):
    """The column product (bias + GeLU, saved pre-activation, K = 12288,
    n = 6144) on T tokens back to back for `seconds`, its launch rate
    printed twice a second: a steady load beside which power and clock are
    read (amd-smi)."""
    import torch
    from tensor_transformer_layer_columnparallel_amd import binding as B
    h, n, dev, bf = 12288, 6144, "cuda", torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(3)
    X = torch.randn(T, h, device=dev, generator=g).to(bf)
    W = (0.02 * torch.randn(h, n, device=dev, generator=g)).to(bf)
    b = (0.02 * torch.randn(n, device=dev, generator=g)).to(bf)
    H = torch.empty(T, n, device=dev, dtype=bf)
    Y = torch.empty(T, n, device=dev, dtype=bf)
    t0 = last = time.perf_counter()
    calls = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            B.tp_column_linear(X, W, b, H, Y, T, h, n, 1, 0, bf, bf, B.TP_ACT_GELU_TANH)
        torch.cuda.synchronize()
        calls += 20
        now = time.perf_counter()
        if now - last > 0.5:
            print(f"column load T={T}: {now - t0:.1f} s, {calls} launches, "
                  f"{1e6 * (now - t0) / calls:.1f} us per launch", flush=True)
            last = now


def ingest_clock(pmc_dir: str, xcds: int = 8, simds: int = 1024, cus: int = 256):
    """Markdown table from a rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE over --busy-cus-sweep: per workgroup count (one
    workgroup per CU), the median over the dispatches after the first
    quarter of the kernel's duration, its engine clock (GPU-active cycles of
    one XCD over the duration) and the MFMA busy fraction of all SIMDs and
    of the SIMDs in use."""
    import csv
    import glob
    import statistics
    disp = {}
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if "gemm_ring" not in row["Kernel_Name"]:
                    continue
                d = disp.setdefault(row["Dispatch_Id"], {
                    "wgs": int(row["Grid_Size"]) // int(row["Workgroup_Size"]),
                    "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"])})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    if not disp:
        raise SystemExit(f"no GEMM dispatches under {pmc_dir}")
    per = {}
    for k in sorted(disp, key=int):
        per.setdefault(disp[k]["wgs"], []).append(disp[k])
    print("| workgroups (CUs busy) | dispatches | duration us | clock GHz | MFMA busy, all SIMDs | "
          "MFMA busy, SIMDs in use |")
    print("|---|---|---|---|---|---|")
    for wgs, ds in sorted(per.items()):
        ds = ds[len(ds) // 4:]
        med = lambda f: statistics.median(f(d) for d in ds)
        act = lambda d: d["GRBM_GUI_ACTIVE"] / xcds
        busy = med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (act(d) * simds))
        print(f"| {wgs} | {len(ds)} | {med(lambda d: d['ns']) / 1e3:.1f} | "
              f"{med(lambda d: act(d) / d['ns']):.2f} | {100 * busy:.1f}% | "
              f"{100 * busy * cus / min(wgs, cus):.1f}% |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The engine clock needs about 25 ms of sustained load to settle: the
    # first launches run at a boost clock, the next ones dip well below the
    # sustained clock while the power control catches up.  40 warm-up steps
    # (about 70 ms) put the timed steps in the sustained state.
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="after the warm-up steps, keep calling the step for at least this "
                         "long (device time), whatever --warmup is")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle baseline (0 disables it)")
    ap.add_argument("--no-reduce", action="store_true", help="skip the shard-sum measurement")
    ap.add_argument("--no-sp", action="store_true",
                    help="skip the sequence-parallel stand-ins")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the tiny fp32 MLP and the 768 -> 3072 column layer")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the attention-projection measurement")
    ap.add_argument("--no-full-layer", action="store_true",
                    help="skip the full-layer emulation (h = 8192, 8 shards + shard sum)")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the vendor-BLAS context timing (torch.matmul)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="REPS",
                    help="only run the HBM-counter calibration copy REPS times")
    ap.add_argument("--ingest-counters", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc CSV output into the stored traffic figure")
    ap.add_argument("--counter-commands", default=COUNTER_COMMANDS,
                    help="commands recorded with the counters (default: the standard recipe)")
    ap.add_argument("--trace-summary", nargs=3, metavar=("TRACE_DIR", "WARMUP", "STEPS"),
                    help="per-kernel durations from a rocprofv3 --kernel-trace CSV of a bench "
                         "run with these warm-up and timed step counts: over all dispatches "
                         "and inside the timed steps")
    ap.add_argument("--ingest-pmc", metavar="PMC_DIR",
                    help="every counter of a rocprofv3 --pmc run per GEMM kernel, and its "
                         "ratio to the CUs' GPU-active cycles")
    ap.add_argument("--ingest-mfma", metavar="PMC_DIR",
                    help="MFMA work, busy fraction and clock per GEMM from a rocprofv3 --pmc run "
                         "of " + " ".join(MFMA_COUNTERS))
    ap.add_argument("--busy-cus-sweep", action="store_true",
                    help="only time the column product on 256, 192 and 128 tiles (and the QKV "
                         "shard's shape), for the clock and MFMA counters per busy CU count")
    ap.add_argument("--ingest-clock", metavar="PMC_DIR",
                    help="clock and MFMA busy fraction per workgroup count from a rocprofv3 --pmc "
                         "run of SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE over --busy-cus-sweep")
    ap.add_argument("--column-load", nargs=2, type=float, metavar=("TOKENS", "SECONDS"),
                    help="only run the column product on TOKENS tokens back to back for SECONDS "
                         "(a steady load for power and clock readings)")
    args = ap.parse_args()
    if args.column_load:
        column_load(int(args.column_load[0]), args.column_load[1])
        return
    if args.ingest_clock:
        ingest_clock(args.ingest_clock)
        return
    if args.busy_cus_sweep:
        busy_cus_sweep()
        return
    if args.ingest_mfma:
        ingest_mfma(args.ingest_mfma)
        return
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary[0], int(args.trace_summary[1]),
                      int(args.trace_summary[2]))
        return
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, commands=args.counter_commands)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library computes one tensor-parallel rank's "
              "shard per GPU and has no exchange between GPUs; run with --gpus 1.", flush=True)
        sys.exit(2)

    import torch

    from tensor_transformer_layer_columnparallel_amd import binding as B
    from tensor_transformer_layer_columnparallel_amd import configs, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    clock_mhz = max_engine_clock_mhz()
    log(f"device: {props.name}, {props.multi_processor_count} CUs, "
        f"{props.total_memory / 2**30:.0f} GiB, max engine clock {clock_mhz} MHz")

    w = configs.GPT3_SHARD
    T, h, ffn, t, n = w.T, w.h, w.ffn, w.t, w.n
    log(f"workload {w.name}: T={T} h={h} ffn={ffn} t={t} n={n}; generating inputs")
    d_h = synth.make_inputs(w)
    bf = torch.bfloat16
    X, W1, b1, W2, dZ = (d_h["X"].to(dev), d_h["W1"][0].to(dev), d_h["b1"][0].to(dev),
                         d_h["W2"][0].to(dev), d_h["dZ"].to(dev))
    H = torch.empty(T, n, dtype=bf, device=dev)
    Y = torch.empty(T, n, dtype=bf, device=dev)
    Z = torch.empty(T, h, dtype=torch.float32, device=dev)
    dY = torch.empty(T, n, dtype=bf, device=dev)
    dW2 = torch.empty(n, h, dtype=torch.float32, device=dev)
    dW1 = torch.empty(h, n, dtype=torch.float32, device=dev)
    dX = torch.empty(T, h, dtype=torch.float32, device=dev)
    db1 = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.tp_column_linear(X, W1, b1, H, Y, T, h, ffn, t, 0, bf, bf, B.TP_ACT_GELU_TANH,
                           stream=sptr)
        if ev is not None:
            ev[1].record(stream)
        B.tp_row_linear(H, W2, Z, T, ffn, h, t, 0, bf, torch.float32, stream=sptr)
        if ev is not None:
            ev[2].record(stream)
        B.tp_mlp_shard_bwd(X, W1, W2, Y, H, dZ, dY, dW2, dW1, dX, db1, T, h, ffn, t, 0, bf,
                           stream=sptr)
        if ev is not None:
            ev[3].record(stream)

    log(f"warmup {args.warmup} steps, then at least {args.warmup_ms:.0f} ms of steps")
    wall0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warmup_steps = args.warmup
    if args.warmup_ms > 0:
        warmup_steps += warm(step, args.warmup_ms)
    warmup_ms = (time.perf_counter() - wall0) * 1e3
    log(f"warm-up: {warmup_steps} steps in {warmup_ms:.0f} ms")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    col_list = sorted(e[0].elapsed_time(e[1]) for e in evs)
    step_list = sorted(e[0].elapsed_time(e[3]) for e in evs)
    col_med, step_med = col_list[len(col_list) // 2], step_list[len(step_list) // 2]
    col_ms = sum(col_list) / args.steps
    row_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    bwd_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}); "
        f"column {col_ms:.3f} ms, row {row_ms:.3f} ms, backward {bwd_ms:.3f} ms")

    gemm = 2.0 * T * h * n
    fwd_flops, bwd_flops = 2 * gemm, 4 * gemm
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    col_tflops = gemm / (col_ms * 1e-3) / 1e12
    traffic = stored_traffic()
    roofline = {"bound": "mfma", "achieved": round(col_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(col_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic,
                "kernel": "column GEMM + bias + GeLU epilogue (tp_column_linear), "
                          f"{gemm / 1e9:.1f} GFLOP per launch"}

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warmup_steps,
           "warmup_ms": round(warmup_ms, 1),
           "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
           "config": {"workload": "gpt3-shaped MLP shard fwd+bwd, rank 0 of t=8",
                      "tokens": T, "h": h, "ffn": ffn, "t": t, "n": n,
                      "parallelism": "one tp8 shard on 1 GPU"},
           "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
           "fwd_tflops": round(fwd_flops / ((col_ms + row_ms) * 1e-3) / 1e12, 2),
           "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
           "roofline": roofline,
           "median": {"ms_per_step": round(step_med, 4), "column_gemm_ms": round(col_med, 4),
                      "column_gemm_tflops": round(gemm / (col_med * 1e-3) / 1e12, 2)},
           "device": {"name": props.name, "cus": props.multi_processor_count,
                      "max_engine_clock_mhz": clock_mhz}}
    del H, Y, Z, dY, dW2, dW1, dX, db1

    if not args.no_small:
        out["small_configs"] = small_configs(B, stream)
        sc = out["small_configs"]
        log("small configs: " + ", ".join(f"{k} {v['eager_us']:.1f} us eager, "
                                         f"{v['graph_us']:.1f} us graph"
                                         for k, v in sc.items() if isinstance(v, dict)))

    if not args.no_attention:
        out["attention_shard"] = attention_shard(B, configs.ATTN_GPT3, stream, sptr)
        a = out["attention_shard"]
        log(f"attention shard: QKV {a['qkv_ms']:.4f} ms, out-proj {a['out_proj_ms']:.4f} ms, "
            f"{a['tflops']:.1f} TFLOP/s")

    if not args.no_sp:
        out["sequence_parallel"] = sequence_parallel(B, stream, sptr)
        sp = out["sequence_parallel"]
        log("sequence parallel: " + ", ".join(f"{k} {sp[k]['ms']:.4f} ms {sp[k]['achieved']:.0f} GB/s"
                                              for k in ("reduce_scatter", "layernorm",
                                                        "concat_tokens",
                                                        "reduce_scatter_layernorm",
                                                        "context_cast")))

    if not args.no_full_layer:
        out["full_layer"] = full_layer(B, stream, sptr)
        fl = out["full_layer"]
        log(f"full layer: sequential {fl['sequential']['ms']:.3f} ms, batched "
            f"{fl['batched']['ms']:.3f} ms ({fl['batched']['tflops']:.0f} TFLOP/s)")

    if not args.no_vendor:
        out["context_vendor_matmul"] = vendor_matmul_context(T, h, n)
        log(f"vendor BLAS context: {out['context_vendor_matmul']['ms_per_step']:.3f} ms for "
            f"the six products")

    if not args.no_reduce:
        wr = configs.FULL_LAYER_8
        count = wr.T * wr.h
        Zs = torch.empty(wr.T, wr.h, device=dev)

        def time_sum(parts):
            def call():
                B.tp_shard_reduce(parts, Zs, wr.T, wr.h, wr.t, B.TP_REDUCE_SUM, parts.dtype,
                                  torch.float32, stream=sptr)
            warm(call)
            reps = 10
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            nbytes = wr.t * count * parts.element_size() + count * 4
            return ms, nbytes, nbytes / (ms * 1e-3) / 1e9

        parts = torch.randn(wr.t, wr.T, wr.h, device=dev)
        ms, nbytes, gbs = time_sum(parts)
        # The same exchange with bf16 partials (half the bytes on the wire),
        # summed in fp32.
        ms16, nbytes16, gbs16 = time_sum(parts.to(torch.bfloat16))
        out["shard_reduce"] = {"workload": "sum of 8 fp32 partials [4096, 8192]",
                               "ms": round(ms, 4), "achieved": round(gbs, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM_GBS, 4),
                               "bytes_per_launch": nbytes,
                               "bf16_partials": {"ms": round(ms16, 4), "achieved": round(gbs16, 1),
                                                 "frac": round(gbs16 / PEAK_HBM_GBS, 4),
                                                 "bytes_per_launch": nbytes16}}
        log(f"shard reduce: {ms:.4f} ms, {gbs:.0f} GB/s; bf16 partials {ms16:.4f} ms, "
            f"{gbs16:.0f} GB/s")
        del parts, Zs

    if args.cpu_seconds > 0:
        log(f"cpu baseline: oracle for about {args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(w, d_h, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
