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
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "TFLOP/s per TP-shard MLP fwd+bwd (bf16) and % of MI355X MFMA peak"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters_column_gemm_gpt3.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """Digest of the GEMM kernel sources; stored HBM counters are used only
    while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_transformer_layer_columnparallel_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("gemm") or name in ("common.h", "epilogue.h"):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_digest") != kernel_source_digest():
        return None
    return c.get("hbm_bytes_per_launch")


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle baseline (0 disables it)")
    ap.add_argument("--no-reduce", action="store_true", help="skip the shard-sum measurement")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs one tensor-parallel rank's "
              "shard per GPU and has no multi-GPU exchange; run with --gpus 1.", flush=True)
        sys.exit(2)

    import torch

    from tensor_transformer_layer_columnparallel_amd import binding as B
    from tensor_transformer_layer_columnparallel_amd import configs, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name}, {props.multi_processor_count} CUs, "
        f"{props.total_memory / 2**30:.0f} GiB")

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

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

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
    col_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
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
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
           "config": {"workload": "gpt3-shaped MLP shard fwd+bwd, rank 0 of t=8",
                      "tokens": T, "h": h, "ffn": ffn, "t": t, "n": n,
                      "parallelism": "one tp8 shard on 1 GPU"},
           "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
           "fwd_tflops": round(fwd_flops / ((col_ms + row_ms) * 1e-3) / 1e12, 2),
           "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
           "roofline": roofline}
    del H, Y, Z, dY, dW2, dW1, dX, db1

    if not args.no_reduce:
        wr = configs.FULL_LAYER_8
        count = wr.T * wr.h
        parts = torch.randn(wr.t, wr.T, wr.h, device=dev)
        Zs = torch.empty(wr.T, wr.h, device=dev)
        for _ in range(2):
            B.tp_shard_reduce(parts, Zs, wr.T, wr.h, wr.t, B.TP_REDUCE_SUM, torch.float32,
                              torch.float32, stream=sptr)
        reps = 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            B.tp_shard_reduce(parts, Zs, wr.T, wr.h, wr.t, B.TP_REDUCE_SUM, torch.float32,
                              torch.float32, stream=sptr)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = (wr.t + 1) * count * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["shard_reduce"] = {"workload": "sum of 8 fp32 partials [4096, 8192]",
                               "ms": round(ms, 4), "achieved": round(gbs, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM_GBS, 4),
                               "bytes_per_launch": nbytes}
        log(f"shard reduce: {ms:.4f} ms, {gbs:.0f} GB/s")
        del parts, Zs

    if args.cpu_seconds > 0:
        log(f"cpu baseline: oracle for about {args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(w, d_h, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
