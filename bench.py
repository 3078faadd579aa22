"""Benchmark: the 8B-shaped ternary linear stack on one MI355X.

A step is one decode-and-verify pair over the whole stack of 252 ternary
linears (36 layers x 7; hidden 4,096, FFN 12,288): one persistent
``tern_linear_stack`` launch at M = 1 token and one at M = 8 tokens (seven
drafted tokens plus the verified one).  Weights are synthetic, seeded, with
the pages' shapes and zero shares, packed on the device before timing.

``value`` is the effective HBM bandwidth of the whole step: algorithmic bytes
(packed weights + 8 B of row metadata per row + int8 activations + 8 B per
token + fp32 outputs, per linear) divided by wall time between two device
synchronisations around exactly ``--steps`` steps.  The ``roofline`` object
is for the launch that takes longer, timed with HIP events on the stream the
kernels run on; ``cpu_baseline`` is the CPU oracle on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "packed_bit_gemv_tern_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    rec = t.get("kernels", {}).get(kernel)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def cpu_baseline(seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload:
    layer 0's seven linears at M = 1 and at M = 8, repeated until `seconds`
    of CPU time have passed."""
    import numpy as np
    import oracle
    from packed_bit_gemv_tern_amd import synth

    lib = oracle.load()
    cases = []
    for (layer, idx, name, N, K, p0) in synth.stack_specs("8b", 1):
        w, s_row = synth.make_weights(0, layer, idx, N, K, p0)
        packed, rowsum, _ = oracle.pack(w, lib=lib)
        for M in (1, 8):
            q, s_act, z = synth.make_activations(0, layer, idx, K, M)
            nbytes = N * packed.shape[1] + 8 * N + M * K + 8 * M + 4 * M * N
            cases.append((packed, s_row, rowsum, K, q, s_act, z, nbytes))
    done_bytes, t = 0, 0.0
    reps = 0
    while t < seconds:
        for (packed, s_row, rowsum, K, q, s_act, z, nbytes) in cases:
            t0 = time.perf_counter()
            oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
            t += time.perf_counter() - t0
            done_bytes += nbytes
        reps += 1
    return {
        "value": round(done_bytes / t / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": "layer 0 of the 8B-shaped stack (7 linears, 48.7 MB packed + metadata) at "
                  "M=1 and M=8, %d repetitions, %.1f s" % (reps, t),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=None, help="fewer layers (testing only)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["m1", "m8"], default=None,
                    help="launch a single pass per step (for profiling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; the stack is the one-GPU share "
              "at its real shape (--gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from packed_bit_gemv_tern_amd import tern
    from packed_bit_gemv_tern_amd.stack import DeviceStack

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    t0 = time.time()
    st = DeviceStack("8b", layers=args.layers, seed=0, threads=16)
    log("packed %d linears, %d weights in %.1f s" % (len(st.linears), st.weights, time.time() - t0))
    passes = []
    if args.only != "m8":
        passes.append(("m1", st.bind(1)))
    if args.only != "m1":
        passes.append(("m8", st.bind(8)))
    stream = torch.cuda.current_stream()

    def step(events=None):
        for i, (_, b) in enumerate(passes):
            if events is not None:
                events[i][0].record(stream)
            b.run(stream)
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in passes] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log("timed %d steps in %.3f s" % (args.steps, elapsed))

    step_bytes = sum(b.bytes for _, b in passes)
    value = step_bytes * args.steps / elapsed / 1e9
    per_pass = {}
    for i, (name, b) in enumerate(passes):
        ms = [ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)]
        ms.sort()
        avg = sum(ms) / len(ms)
        kname = "valu_stack_kernel<1>" if b.plan.kernel == 0 else (
            "mfma_stack_kernel<1>" if b.M <= 16 else "mfma_stack_kernel<4>")
        if b.plan.kernel in (1, 2, 3):
            kname = "valu_stack_kernel<%d>" % {1: 2, 2: 4, 3: 8}[b.plan.kernel]
        per_pass[name] = {
            "M": b.M, "kernel": kname, "bytes": b.bytes, "avg_us": round(avg * 1e3, 3),
            "p10_us": round(ms[len(ms) // 10] * 1e3, 3), "p90_us": round(ms[(9 * len(ms)) // 10] * 1e3, 3),
            "GBps": round(b.bytes / (avg * 1e-3) / 1e9, 1),
            "frac_of_peak": round(b.bytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "grid": b.plan.grid, "waves": b.plan.workers, "segments": b.plan.segments,
        }
    dom = max(per_pass, key=lambda n: per_pass[n]["avg_us"])
    d = per_pass[dom]
    traffic = load_traffic(d["kernel"])
    roofline = {"bound": "hbm", "achieved": d["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(d["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": d["kernel"], "M": d["M"]}

    out = {
        "metric": "effective HBM GB/s (% of peak) for 8B ternary linear stack at M=1 and M=8",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "8B-shaped ternary linear stack: %d linears (%d layers x 7, hidden 4096, "
                        "FFN 12288), %d weights, one M=1 pass + one M=8 pass per step"
                        % (len(st.linears), len(st.linears) // 7, st.weights),
            "bytes_per_step": step_bytes,
            "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "passes": per_pass,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
