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


_VALU_SETS = {0: "80u", 1: "14u", 2: "255u", 3: "511u"}


def kernel_name(plan) -> str:
    """Name of the HIP kernel a prepared stack launches (as the profiler shows it)."""
    k = plan.kernel
    if k in _VALU_SETS:
        return "valu_stack_kernel<1, %s>" % _VALU_SETS[k]
    if k in (4, 5, 6):
        return "valu_stack_kernel<%d, 0u>" % {4: 2, 5: 4, 6: 8}[k]
    v = k - 8
    if v == 8:
        return "mfma_win_stack_kernel"
    ragged = "true" if v & 2 else "false"
    if v & 1:
        return "mfma_stack_kernel<4, %s>" % ragged
    return "mfma_wg_stack_kernel<%d, %s>" % (16 if v & 4 else 8, ragged)


def read_probe(nbytes: int, reps: int = 5):
    """Best plain-read rate over a few launch shapes (the achievable ceiling)."""
    import torch
    from packed_bit_gemv_tern_amd import tern
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    results = []
    for bpc in (2, 4, 8):
        for unroll in (8, 16):
            for nt in (1, 0):
                tern.tern_read_probe(buf, nbytes, sink, bpc, unroll, nt)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(reps):
                    tern.tern_read_probe(buf, nbytes, sink, bpc, unroll, nt)
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                results.append({"blocks_per_cu": bpc, "unroll": unroll, "nontemporal": nt,
                                "avg_us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1)})
    del buf
    best = max(results, key=lambda r: r["GBps"])
    return {"bytes": nbytes, "best_GBps": best["GBps"], "best": best, "all": results}


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
    ap.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth probe")
    ap.add_argument("--only", choices=["m1", "m8"], default=None,
                    help="launch a single pass per step (for profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times "
                         "(reference for the HBM byte counters) and exit")
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
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return
    # Each pass gets its own copy of the stack (different seeds): the two
    # passes never share weights, so neither can hit lines the other left in
    # the caches (as in drafted decoding, where they are different models).
    t0 = time.time()
    passes, stacks = [], []
    for name, M, seed in (("m1", 1, 0), ("m8", 8, 1)):
        if args.only not in (None, name):
            continue
        st = DeviceStack("8b", layers=args.layers, seed=seed, threads=16)
        stacks.append(st)
        passes.append((name, st.bind(M)))
    st = stacks[0]
    log("packed %d x %d linears, %d weights each, in %.1f s"
        % (len(stacks), len(st.linears), st.weights, time.time() - t0))
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
        kname = kernel_name(b.plan)
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
                        "FFN 12288), %d weights; per step one M=1 pass and one M=8 pass, each "
                        "over its own resident copy of the stack"
                        % (len(st.linears), len(st.linears) // 7, st.weights),
            "bytes_per_step": step_bytes,
            "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "passes": per_pass,
        "roofline": roofline,
    }
    if not args.no_probe:
        probe = read_probe(max(b.bytes for _, b in passes) // 16 * 16)
        out["read_probe"] = probe
        for name in per_pass:
            per_pass[name]["frac_of_probe"] = round(per_pass[name]["GBps"] / probe["best_GBps"], 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
