"""Benchmark: the 8B-shaped ternary linear stack on one MI355X.

A step is one decode-and-verify pair over the whole stack of 252 ternary
linears (36 layers x 7; hidden 4,096, FFN 12,288): one
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

``--suite`` instead measures the other workloads of the method, one JSON line
each: the single 256 x 512 GEMV; one 8B layer at M = 1 per linear and per
layer (eight rotating copies, 390 MB, more than the 256 MB Infinity Cache);
the 0.6B stack as seven M = 1 passes per step (three rotating copies, and
warm); the prefill sweep M = 1 .. 512 on one 8B layer (eight copies), that
layer's gated feed-forward as two launches (gate and up, then down reading
silu(g) * u through its fused quantiser) at M = 1 and 8, and
M = 16, 64, 512 on four layers; the int8 output head (151,936 x 4,096) at
M = 1 and 8; block-wise scales on the 8B's stacked gate projections; the
same gate projections in 2-bit and in 1.6-bit rows; the weight quantiser;
one decode step (quantiser, stack, head) eager and replayed from a HIP
graph, with the quantiser fused into the stack launch (two launches) and as
a launch of its own (three); the whole 8B stack at M = 16; q/k/v and gate/up
sharing inputs; block-wise scales inside the stack; and the activation
quantiser.  Most lines carry the oracle timed on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
# vector ALU lane-operations per second: 256 CUs x 64 lanes per clock (four
# SIMD16 units) x 2.4 GHz; the fp32 vector peak of 157.3 TFLOP/s is this
# times 2 (FMA) times 2 (packed fp32)
VALU_LANE_OPS_PER_S = 256 * 64 * 2.4e9


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources that define the stack kernels' device code and schedule, and
# the compile flags: the committed HBM counters hold only while none of them
# has changed.
STACK_KERNEL_SOURCES = ("csrc/tern_api.hip", "csrc/tern_device.h", "csrc/tern_gemm.hip",
                        "csrc/tern_internal.h", "csrc/tern_mfma.hip", "csrc/tern_prologue.h",
                        "csrc/tern_valu.hip", "build.py")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in STACK_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "packed_bit_gemv_tern_amd", name), "rb") as f:
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


def _counter_means(path: str):
    """Mean counter value per kernel name over its dispatches (rocprofv3 csv)."""
    import csv
    sums, counts = {}, {}
    with open(path) as f:
        for row in csv.DictReader(f):
            k = row["Kernel_Name"]
            sums[k] = sums.get(k, 0.0) + float(row["Counter_Value"])
            counts[k] = counts.get(k, 0) + 1
    return {k: (sums[k] / counts[k], counts[k]) for k in sums}


def write_traffic(d: str):
    """profiles/traffic.json from FETCH_SIZE / WRITE_SIZE runs of the m1 and
    m8 passes and of a 1 GiB device copy (the calibration: the copy reads and
    writes 1 GiB, so scale = 2^20 KiB / its counter reading)."""
    def means(c, w):
        return _counter_means(os.path.join(d, "pmc_%s_%s" % (c, w), "run_counter_collection.csv"))
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = [v for k, v in means(c, "copy").items() if "copyBuffer" in k]
        kib = max(v[0] for v in cp)  # the 1 GiB copies (other copies are small)
        scale[c] = float(1 << 20) / kib
    from packed_bit_gemv_tern_amd import synth, tern

    def algo_bytes(M):  # the stack planner's count for one pass (plan.bytes)
        return sum(N * tern.tern_row_bytes(K) + 8 * N + M * K + 8 * M + 4 * M * N
                   for (_, _, _, N, K, _) in synth.stack_specs("8b"))
    algo = {"m1": algo_bytes(1), "m8": algo_bytes(8)}
    out = {"source_hash": kernel_source_hash(), "fetch_scale": scale["FETCH_SIZE"],
           "write_scale": scale["WRITE_SIZE"], "kernels": {}}
    for w, M in (("m1", 1), ("m8", 8)):
        f = {k: v for k, v in means("FETCH_SIZE", w).items() if "stack_kernel" in k}
        wr = {k: v for k, v in means("WRITE_SIZE", w).items() if "stack_kernel" in k}
        (k, (fk, _)), = f.items()
        wk = wr[k][0]
        # the profiler's name without return type, namespaces and arguments,
        # as kernel_name() gives it (the defaulted template argument dropped)
        name = k.split("(")[0].replace("void ", "").replace("tern::", "").replace("(anonymous namespace)::", "")
        name = {"mfma_win_stack_kernel<false, false>": "mfma_win_stack_kernel<false>"}.get(name, name)
        hbm = fk * 1024 * scale["FETCH_SIZE"] + wk * 1024 * scale["WRITE_SIZE"]
        out["kernels"][name] = {"M": M, "fetch_kib": fk, "write_kib": wk, "hbm_bytes_per_launch": int(round(hbm)),
                                "algorithmic_bytes": algo[w], "ratio": round(hbm / algo[w], 4)}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def kernel_name(plan) -> str:
    """Name of the HIP kernel a prepared stack launches (as the profiler shows it)."""
    k = plan.kernel
    if k in _VALU_SETS:
        return "valu_stack_kernel<1, %s>" % _VALU_SETS[k]
    if k in (4, 5, 6):
        return "valu_stack_kernel<%d, 0u>" % {4: 2, 5: 4, 6: 8}[k]
    if 8 <= k < 12:
        return "valu_stack_blk_kernel<%s>" % _VALU_SETS[k - 8]
    if 12 <= k < 16:
        return "valu_stack_tok_kernel<%s>" % _VALU_SETS[k - 12]
    v = k - 16
    if v == 8:
        return "mfma_win_stack_kernel<%s>" % ("true" if getattr(plan, "splits", 0) else "false")
    if v == 12:
        return "mfma_win_stack_kernel<false, true>"
    if v == 13:
        return "mfma_win16_stack_kernel<false, true>"
    if v in (9, 10, 14):
        return {9: "gemm_stack_kernel<64, 128>", 10: "gemm_stack_kernel<128, 512>", 14: "gemm_stack_kernel<128, 256>"}[v]
    if v == 11:
        return "mfma_win16_stack_kernel<false>"
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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload:
    layer 0's seven linears at M = 1 and at M = 8, repeated until `seconds`
    of CPU time have passed, on every host core and then on one."""
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

    def timed(limit):
        done_bytes, t, reps = 0, 0.0, 0
        while t < limit:
            for (packed, s_row, rowsum, K, q, s_act, z, nbytes) in cases:
                t0 = time.perf_counter()
                oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
                t += time.perf_counter() - t0
                done_bytes += nbytes
            reps += 1
        return done_bytes / t / 1e9, reps, t

    all_cores = oracle.threads()
    gbs, reps, t = timed(seconds * 2 / 3)
    oracle.set_threads(1)
    gbs1, reps1, t1 = timed(seconds / 3)
    oracle.set_threads(all_cores)
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": all_cores,
        "kind": "oracle",
        "sample": "layer 0 of the 8B-shaped stack (7 linears, 48.7 MB packed + metadata) at "
                  "M=1 and M=8, %d repetitions, %.1f s" % (reps, t),
        "single_thread": {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1,
                          "sample": "the same, %d repetitions, %.1f s" % (reps1, t1)},
        "host": {"nproc": os.cpu_count(), "cpu_model": _cpu_model(),
                 "oracle_build": "gcc " + " ".join(oracle.CFLAGS[:-2])},
    }


INT8_DENSE_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, published peak


def _event_times(fn, calls: int, warm: int = 3, warm_s: float = 0.2):
    """Per-call HIP-event durations (us, sorted) of fn(i), i = 0..calls-1,
    after at least `warm` untimed calls and `warm_s` seconds of them (the
    first launches after a change of workload run several percent slow),
    on the current stream."""
    import torch
    stream = torch.cuda.current_stream()
    t_end = time.perf_counter() + warm_s
    i = 0
    while i < warm or time.perf_counter() < t_end:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    torch.cuda.synchronize()
    for i in range(calls):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e3 for a, b in ev)


def _stats(us, nbytes=None):
    n = len(us)
    med = us[n // 2]
    out = {"median_us": round(med, 3), "p10_us": round(us[n // 10], 3),
           "p90_us": round(us[(9 * n) // 10], 3), "calls": n}
    if nbytes is not None:
        out["bytes"] = int(nbytes)
        out["GBps"] = round(nbytes / med / 1e3, 1)
        out["frac_of_peak"] = round(nbytes / med / 1e3 / HBM_PEAK_GBS, 4)
    return out


def _oracle_rate(cases, seconds: float):
    """The oracle on `cases` [(packed, s_row, rowsum, K, q, s_act, z, nbytes)],
    repeated until `seconds` have passed: (GB/s of algorithmic bytes, us per
    pass over the cases, repetitions)."""
    import oracle
    lib = oracle.load()
    t, done, reps = 0.0, 0, 0
    while t < seconds or reps == 0:
        for (packed, s_row, rowsum, K, q, s_act, z, nbytes) in cases:
            t0 = time.perf_counter()
            oracle.linear(packed, s_row, rowsum, K, q, s_act, z, lib=lib)
            t += time.perf_counter() - t0
            done += nbytes
        reps += 1
    return done / t / 1e9, t / reps * 1e6, reps


def suite(args):
    """The measurement suite (one JSON line per workload)."""
    import numpy as np
    import torch
    import oracle
    from packed_bit_gemv_tern_amd import synth, tern
    from packed_bit_gemv_tern_amd.stack import DeviceStack

    dev = "cuda:0"
    olib = oracle.load()
    cores = oracle.threads()

    def emit(d):
        print(json.dumps(d), flush=True)

    def linear_bytes(N, K, M):
        return N * tern.tern_row_bytes(K) + 8 * N + M * K + 8 * M + 4 * M * N

    # --- single GEMV, 256 x 512 (cache-resident, launch-bound: microseconds only)
    lin = synth.single_gemv_case()
    N, K = lin.w.shape
    wd = torch.from_numpy(lin.w).to(dev)
    packed = torch.empty((N, tern.tern_row_bytes(K)), dtype=torch.uint8, device=dev)
    rowsum = torch.empty(N, dtype=torch.int32, device=dev)
    tern.tern_pack(wd, N, K, K, packed, rowsum)
    s_row = torch.from_numpy(lin.s_row).to(dev)
    q = torch.from_numpy(lin.q.reshape(-1)).to(dev)
    s_act = torch.from_numpy(lin.s_act).to(dev)
    z = torch.from_numpy(lin.z).to(dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)
    us = _event_times(lambda i: tern.tern_gemv(packed, s_row, rowsum, N, K, q, s_act, z, y), 200)
    opk, ors, _ = oracle.pack(lin.w, lib=olib)
    ogb, ous, oreps = _oracle_rate([(opk, lin.s_row, ors, K, lin.q, lin.s_act, lin.z,
                                     linear_bytes(N, K, 1))], 2.0)
    emit({"suite": "single_gemv", "workload": "one 256 x 512 ternary GEMV (seed 0), M = 1",
          "kernel": "valu_linear_kernel", **_stats(us, linear_bytes(N, K, 1)),
          "note": "cache-resident and launch-bound: microseconds, no roofline claim",
          "cpu_oracle": {"us": round(ous, 2), "cores": cores, "reps": oreps}})

    # --- one 8B layer at M = 1: per linear and per layer, eight rotating copies
    copies = [DeviceStack("8b", layers=1, seed=c, threads=16) for c in range(8)]
    specs = copies[0].specs
    b1 = [st.bind(1) for st in copies]
    for idx, (layer, _, name, N, K, p0) in enumerate(specs):
        def call(i, idx=idx):
            c = i % 8
            pl, b = copies[c].linears[idx], b1[c]
            tern.tern_gemv(pl.packed, pl.s_row, pl.rowsum, pl.N, pl.K, b.q[idx].view(-1),
                           b.s_act[idx], b.z[idx], b.y[idx].view(-1))
        us = _event_times(call, 64)
        emit({"suite": "layer8b_linear", "workload": "8B layer 0 %s (%d x %d), M = 1, 8 rotating "
              "copies" % (name, N, K), "linear": name, "N": N, "K": K,
              "kernel": "valu_linear_kernel", **_stats(us, linear_bytes(N, K, 1))})
    us = _event_times(lambda i: b1[i % 8].run(), 64)
    lb = b1[0].bytes
    # oracle: layer 0 at M = 1
    cases = []
    for (layer, idx, name, N, K, p0) in specs:
        w, sr = synth.make_weights(0, layer, idx, N, K, p0)
        pk, rs, _ = oracle.pack(w, lib=olib)
        qq, sa, zz = synth.make_activations(0, layer, idx, K, 1)
        cases.append((pk, sr, rs, K, qq, sa, zz, linear_bytes(N, K, 1)))
    ogb, ous, oreps = _oracle_rate(cases, 5.0)
    emit({"suite": "layer8b", "workload": "one 8B layer (7 linears), M = 1, one stack launch, "
          "8 rotating copies (390 MB)", "kernel": kernel_name(b1[0].plan), **_stats(us, lb),
          "cpu_oracle": {"GBps": round(ogb, 4), "us": round(ous, 1), "cores": cores,
                         "reps": oreps}})
    del b1, cases

    # --- prefill sweep on one 8B layer, eight rotating copies
    for M in (1, 2, 4, 8, 16, 64, 512):
        bm = [st.bind(M) for st in copies]
        us = _event_times(lambda i: bm[i % 8].run(), 48)
        st = _stats(us, bm[0].bytes)
        dense_ops = 2 * M * sum(N * K for (_, _, _, N, K, _) in specs)
        st["dense_TOPS"] = round(dense_ops / st["median_us"] / 1e6, 2)
        st["frac_of_int8_peak"] = round(st["dense_TOPS"] / INT8_DENSE_PEAK_TOPS, 4)
        rec = {"suite": "prefill_sweep", "workload": "one 8B layer (7 linears), M = %d, one "
               "stack launch, 8 rotating copies" % M, "M": M, "kernel": kernel_name(bm[0].plan),
               **st}
        if M == 512:
            # oracle on a row sample: 32 rows of each linear at M = 512
            cases = []
            for (layer, idx, name, N, K, p0) in specs:
                w, sr = synth.make_weights(0, layer, idx, N, K, p0)
                rows = np.arange(0, N, N // 32)[:32]
                pk, rs, _ = oracle.pack(w[rows], lib=olib)
                qq, sa, zz = synth.make_activations(0, layer, idx, K, M)
                cases.append((pk, sr[rows], rs, K, qq, sa, zz, 2 * M * 32 * K))
            ogb, ous, oreps = _oracle_rate(cases, 5.0)
            rec["cpu_oracle"] = {"dense_GOPS": round(ogb, 3), "cores": cores, "reps": oreps,
                                 "sample": "32 rows of each of the 7 linears at M = 512"}
        emit(rec)
        del bm

    # --- one 8B layer's gated feed-forward chained over two launches, eight
    # rotating copies: launch 1 quantises the fp32 hidden state and runs gate
    # and up; launch 2 quantises silu(g) * u (from launch 1's outputs) inside
    # its own prologue and runs down
    for M in (1, 8):
        chain = []
        for st in copies:
            gate, up, down = st.linears[4], st.linears[5], st.linears[6]
            H, F = gate.K, gate.N
            x = torch.from_numpy(synth.make_hidden(0, 0, 4, H, M)).to(dev)
            b = {"x": x}
            for key, n in (("q1", H), ("q2", F)):
                b[key] = torch.zeros((M, n), dtype=torch.int8, device=dev)
            for key in ("s1", "s2"):
                b[key] = torch.empty(M, dtype=torch.float32, device=dev)
            for key in ("z1", "z2"):
                b[key] = torch.empty(M, dtype=torch.int32, device=dev)
            b["g"] = torch.empty((M, F), dtype=torch.float32, device=dev)
            b["u"] = torch.empty((M, F), dtype=torch.float32, device=dev)
            b["y"] = torch.empty((M, H), dtype=torch.float32, device=dev)
            d1 = [tern.make_desc(pl.packed, pl.s_row, pl.rowsum, pl.N, pl.K, b["q1"], H, b["s1"], b["z1"], yy, F,
                                 x=x, ldx=H) for pl, yy in ((gate, b["g"]), (up, b["u"]))]
            d2 = [tern.make_desc(down.packed, down.s_row, down.rowsum, down.N, down.K, b["q2"], F, b["s2"],
                                 b["z2"], b["y"], H, x=b["g"], ldx=F, x_up=b["u"])]
            b["ws1"] = torch.empty(tern.tern_linear_stack_workspace_bytes(2, M), dtype=torch.uint8, device=dev)
            b["ws2"] = torch.empty(tern.tern_linear_stack_workspace_bytes(1, M), dtype=torch.uint8, device=dev)
            b["p1"] = tern.tern_linear_stack_prepare(d1, M, b["ws1"])
            b["p2"] = tern.tern_linear_stack_prepare(d2, M, b["ws2"])
            chain.append(b)

        def ffn(i):
            tern.tern_linear_stack(chain[i % 8]["p1"])
            tern.tern_linear_stack(chain[i % 8]["p2"])
        us = _event_times(ffn, 40)
        nb = int(chain[0]["p1"].bytes + chain[0]["p2"].bytes)
        emit({"suite": "ffn_chain", "workload": "one 8B layer's gated feed-forward (gate, up 12,288 x 4,096; "
              "down 4,096 x 12,288), M = %d: two launches, the fp32 hidden state and silu(g) * u quantised "
              "inside them, 8 rotating copies" % M, "M": M,
              "kernels": [kernel_name(chain[0]["p1"]), kernel_name(chain[0]["p2"])],
              "note": "bytes: packed weights, metadata, int8 activations and outputs of the three linears "
                      "(the fp32 inputs the launches quantise are not counted)", **_stats(us, nb)})
        del chain
    del copies

    # --- prefill over four 8B layers (28 linears, 195 MB): enough tiles to
    # fill the chip, so the rate is the kernel's rather than one layer's
    # longest tile chain (the K = 12,288 down projection)
    st4 = DeviceStack("8b", layers=4, seed=3, threads=16)
    specs4 = synth.stack_specs("8b", 4)
    for M in (16, 64, 512):
        b4 = st4.bind(M)
        us = _event_times(lambda i: b4.run(), 24)
        st = _stats(us, b4.bytes)
        dense_ops = 2 * M * sum(N * K for (_, _, _, N, K, _) in specs4)
        st["dense_TOPS"] = round(dense_ops / st["median_us"] / 1e6, 2)
        st["frac_of_int8_peak"] = round(st["dense_TOPS"] / INT8_DENSE_PEAK_TOPS, 4)
        emit({"suite": "prefill_4layers", "workload": "four 8B layers (28 linears), M = %d, one stack "
              "launch" % M, "M": M, "kernel": kernel_name(b4.plan), **st})
        del b4
    del st4

    # --- 0.6B stack, M = 1, seven passes per step: 3 rotating copies, and warm
    st06 = [DeviceStack("0.6b", seed=c, threads=16) for c in range(3)]
    b06 = [st.bind(1) for st in st06]
    pb = b06[0].bytes
    us = _event_times(lambda i: b06[i % 3].run(), 63)
    rot = _stats(us, pb)
    us = _event_times(lambda i: b06[0].run(), 63)
    warm = _stats(us, pb)
    warm.pop("frac_of_peak")
    cases = []
    for (layer, idx, name, N, K, p0) in synth.stack_specs("0.6b"):
        w, sr = synth.make_weights(0, layer, idx, N, K, p0)
        pk, rs, _ = oracle.pack(w, lib=olib)
        qq, sa, zz = synth.make_activations(0, layer, idx, K, 1)
        cases.append((pk, sr, rs, K, qq, sa, zz, linear_bytes(N, K, 1)))
    ogb, ous, oreps = _oracle_rate(cases, 5.0)
    emit({"suite": "stack06b", "workload": "0.6B-shaped stack (196 linears), M = 1; a step is "
          "seven passes (one per drafted token)", "kernel": kernel_name(b06[0].plan),
          "pass_rotating_3_copies": rot, "step_us_rotating": round(7 * rot["median_us"], 2),
          "pass_warm_same_copy": warm,
          "note": "warm passes re-read a stack that fits the 256 MB Infinity Cache: no HBM "
                  "fraction is claimed for them",
          "cpu_oracle": {"GBps": round(ogb, 4), "us_per_pass": round(ous, 1), "cores": cores,
                         "reps": oreps}})
    del b06, st06
    torch.cuda.empty_cache()

    def oracle_time(fn, seconds):
        t, reps = 0.0, 0
        while t < seconds:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            reps += 1
        return t / reps, reps

    # --- the int8 output head (151,936 x 4,096), M = 1 and 8
    W, s_row_h = synth.make_head(0)
    N, K = W.shape
    Wd = torch.from_numpy(W).to(dev)
    srh = torch.from_numpy(s_row_h).to(dev)
    rsh = torch.empty(N, dtype=torch.int32, device=dev)
    tern.tern_head_rowsum(Wd, N, K, K, rsh)
    rows = np.arange(0, N, N // 256)[:256]
    Ws = np.ascontiguousarray(W[rows])
    ors = oracle.head_rowsum(Ws, lib=olib)
    for M in (1, 8):
        qq, sa, zz = synth.make_activations(0, 36, 7, K, M)
        qd, sad, zd = (torch.from_numpy(a).to(dev) for a in (qq, sa, zz))
        yd = torch.empty((M, N), dtype=torch.float32, device=dev)
        us = _event_times(lambda i: tern.tern_head_gemv(Wd, srh, rsh, N, K, K, M, qd, K, sad, zd, yd, N), 48)
        hb = N * K + 8 * N + M * K + 8 * M + 4 * M * N
        ot, oreps = oracle_time(lambda: oracle.head(Ws, s_row_h[rows], ors, qq, sa, zz, lib=olib), 2.0)
        sb = len(rows) * K + 8 * len(rows) + M * K + 8 * M + 4 * M * len(rows)
        emit({"suite": "head8b", "workload": "int8 output head 151,936 x 4,096 (one scale per row), "
              "M = %d" % M, "M": M, "kernel": "head_kernel<%d>" % (1 if M == 1 else 8),
              **_stats(us, hb),
              "cpu_oracle": {"GBps": round(sb / ot / 1e9, 4), "cores": cores, "reps": oreps,
                             "sample": "256 rows"}})
    del Wd, srh, rsh, W
    torch.cuda.empty_cache()

    # --- block-wise scales: the 8B's 36 gate projections stacked (442,368 x 4,096)
    specs8 = [s_ for s_ in synth.stack_specs("8b") if s_[2] == "gate"]
    K = specs8[0][4]
    N = sum(s_[3] for s_ in specs8)
    ld = tern.tern_row_bytes(K)
    packed = torch.empty((N, ld), dtype=torch.uint8, device=dev)
    r0 = 0
    for (layer, idx, name, n_, k_, p0) in specs8:
        w, _ = synth.make_weights(0, layer, idx, n_, k_, p0)
        rs_ = torch.empty(n_, dtype=torch.int32, device=dev)
        tern.tern_pack(torch.from_numpy(w).to(dev), n_, k_, k_, packed[r0:r0 + n_], rs_)
        r0 += n_
    qq, sa, zz = synth.make_activations(0, 0, 4, K, 1)
    qd, sad, zd = (torch.from_numpy(a).to(dev) for a in (qq.reshape(-1), sa, zz))
    yd = torch.empty(N, dtype=torch.float32, device=dev)
    w0, _ = synth.make_weights(0, 0, 4, 256, K, specs8[0][5])
    opk, _, _ = oracle.pack(w0, lib=olib)
    for B in (128, 1024):
        nb = K // B
        sbd = torch.from_numpy(np.random.default_rng([B, 1]).uniform(0.01, 0.1, (N, nb))
                               .astype(np.float32)).to(dev)
        rbd = torch.empty((N, nb), dtype=torch.int32, device=dev)
        tern.tern_block_rowsum(packed, N, K, B, rbd)
        us = _event_times(lambda i: tern.tern_gemv_blocked(packed, sbd, rbd, N, K, B, qd, sad, zd, yd), 48)
        bb = N * ld + 8 * N * nb + K + 8 + 4 * N
        s_o = sbd[:256].cpu().numpy()
        r_o = oracle.block_rowsum(w0, B, lib=olib)
        ot, oreps = oracle_time(lambda: oracle.linear_blocked(opk, s_o, r_o, K, B, qq, sa, zz, lib=olib), 2.0)
        emit({"suite": "blocked", "workload": "8B gate projections stacked (442,368 x 4,096), "
              "block scales every %d columns, M = 1" % B, "B": B, "kernel": "blocked_gemv_kernel<1>",
              **_stats(us, bb),
              "cpu_oracle": {"GBps": round((256 * ld + 8 * 256 * nb + K + 4 * 256) / ot / 1e9, 4),
                             "cores": cores, "reps": oreps, "sample": "256 rows of layer 0's gate"}})
        del sbd, rbd
    del packed
    torch.cuda.empty_cache()

    # --- 1.6-bit rows against 2-bit rows: the same 36 stacked 8B gate
    # projections (442,368 x 4,096), one M = 1 call each
    N5 = sum(s_[3] for s_ in specs8)
    ld2, ld5 = tern.tern_row_bytes(K), tern.tern_row_bytes5(K)
    p2 = torch.empty((N5, ld2), dtype=torch.uint8, device=dev)
    p5 = torch.empty((N5, ld5), dtype=torch.uint8, device=dev)
    rs5 = torch.empty(N5, dtype=torch.int32, device=dev)
    sr5 = torch.empty(N5, dtype=torch.float32, device=dev)
    r0 = 0
    for (layer, idx, name, n_, k_, p0) in specs8:
        w, sr_ = synth.make_weights(0, layer, idx, n_, k_, p0)
        wd = torch.from_numpy(w).to(dev)
        tern.tern_pack(wd, n_, k_, k_, p2[r0:r0 + n_], rs5[r0:r0 + n_])
        tern.tern_pack5(wd, n_, k_, k_, p5[r0:r0 + n_], rs5[r0:r0 + n_])
        sr5[r0:r0 + n_] = torch.from_numpy(sr_).to(dev)
        r0 += n_
    qq, sa, zz = synth.make_activations(0, 0, 4, K, 1)
    qd, sad, zd = (torch.from_numpy(a).to(dev) for a in (qq.reshape(-1), sa, zz))
    yd = torch.empty(N5, dtype=torch.float32, device=dev)
    w0, s0 = synth.make_weights(0, 0, 4, 256, K, specs8[0][5])
    weights = N5 * K
    for label, ld_, fn, kern, ops in (
            ("2-bit", ld2, lambda i: tern.tern_gemv(p2, sr5, rs5, N5, K, qd, sad, zd, yd),
             "valu_linear_kernel", 0.5),
            ("1.6-bit", ld5, lambda i: tern.tern_gemv5(p5, sr5, rs5, N5, K, qd, sad, zd, yd),
             "gemv5_kernel<8, 2>", 26 / 20)):
        us = _event_times(fn, 48)
        st_ = _stats(us, N5 * ld_ + 8 * N5 + K + 8 + 4 * N5)
        wps = weights / (st_["median_us"] * 1e-6)
        if label == "2-bit":
            o_pk, o_rs, _ = oracle.pack(w0, lib=olib)
            ofn = lambda: oracle.linear(o_pk, s0, o_rs, K, qq, sa, zz, lib=olib)
        else:
            o_pk, o_rs, _ = oracle.pack5(w0, lib=olib)
            ofn = lambda: oracle.linear5(o_pk, s0, o_rs, K, qq, sa, zz, lib=olib)
        ot, oreps = oracle_time(ofn, 2.0)
        emit({"suite": "packed5", "workload": "8B gate projections stacked (442,368 x 4,096) in "
              "%s rows, M = 1" % label, "layout": label, "kernel": kern, **st_,
              "weights_per_s": float("%.4g" % wps),
              "valu_ops_per_weight": ops,
              "frac_of_valu_peak": round(ops * wps / VALU_LANE_OPS_PER_S, 4),
              "cpu_oracle": {"weights_per_s": float("%.4g" % (256 * K / ot)), "cores": cores,
                             "reps": oreps, "sample": "256 rows of layer 0's gate"}})
    del p2, p5, rs5, sr5, yd
    torch.cuda.empty_cache()

    # --- weight quantiser (load time): one 8B gate projection, fp32 12,288 x 4,096
    Nw, Kw, Bw = 12288, 4096, 128
    Wf = (np.random.default_rng([1, 4, 7]).standard_normal((Nw, Kw)) * 0.02).astype(np.float32)
    Wd = torch.from_numpy(Wf).to(dev)
    td = torch.empty((Nw, Kw), dtype=torch.int8, device=dev)
    sd = torch.empty((Nw, Kw // Bw), dtype=torch.float32, device=dev)
    us = _event_times(lambda i: tern.tern_quantize_weights(Wd, Nw, Kw, Kw, Bw, td, Kw, sd), 20)
    ot, oreps = oracle_time(lambda: oracle.quantize_weights(Wf[:256], Bw, lib=olib), 1.0)
    emit({"suite": "quantize_weights", "workload": "ternarise one 8B gate projection (fp32 12,288 x 4,096), "
          "block scales every %d columns (load time)" % Bw, "B": Bw, "kernel": "wquant_kernel",
          **_stats(us, 5 * Nw * Kw + 4 * Nw * (Kw // Bw)),
          "cpu_oracle": {"GBps": round((5 * 256 * Kw + 4 * 256 * (Kw // Bw)) / ot / 1e9, 4), "cores": cores,
                         "reps": oreps, "sample": "256 rows"}})
    del Wd, td, sd, Wf
    torch.cuda.empty_cache()

    # --- one decode step's linears, eager and replayed from a HIP graph:
    # the token's fp32 hidden state quantised, the 252-linear 8B stack (layer
    # 0's q/k/v read that token; each layer's q/k/v and gate/up share one
    # input), the int8 head reading the same quantised token.  Fused: the
    # stack launch quantises its fp32 input itself (two launches); separate:
    # the quantiser is a launch of its own (three).
    st = DeviceStack("8b", seed=5, threads=16)
    Wh, srh_ = synth.make_head(0)
    Nh, Kh = Wh.shape
    Whd, srhd = torch.from_numpy(Wh).to(dev), torch.from_numpy(srh_).to(dev)
    del Wh
    rshd = torch.empty(Nh, dtype=torch.int32, device=dev)
    tern.tern_head_rowsum(Whd, Nh, Kh, Kh, rshd)
    for M in (1, 8):
        rec = {"suite": "decode_step", "workload": "one decode step's linears at M = %d: quantise the fp32 "
               "token(s), the 252-linear 8B stack (one launch; q/k/v and gate/up share inputs), the int8 head "
               "151,936 x 4,096 reading the quantised token(s)" % M, "M": M}
        head_bytes = Nh * Kh + 8 * Nh + M * Kh + 8 * M + 4 * M * Nh
        for mode in ("fused", "separate"):
            b = st.bind(M, share_inputs=True, quantise="first" if mode == "fused" else "none")
            ldq = b.q[0].shape[1]
            xd = b.x[0] if mode == "fused" else torch.from_numpy(
                synth.make_hidden(5, 0, 0, Kh, M)).to(dev)
            logits = torch.empty((M, Nh), dtype=torch.float32, device=dev)

            def dstep(i=0, b=b, xd=xd, logits=logits, M=M, ldq=ldq, mode=mode):
                if mode == "separate":
                    tern.tern_quantize_act(xd, M, Kh, Kh, b.q[0], ldq, b.s_act[0], b.z[0])
                b.run()
                tern.tern_head_gemv(Whd, srhd, rshd, Nh, Kh, Kh, M, b.q[0], ldq, b.s_act[0], b.z[0], logits, Nh)
            eager = _event_times(dstep, 20)
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                dstep()
            torch.cuda.synchronize()
            replay = _event_times(lambda i: g.replay(), 20)
            # (fused: the stack's bytes include its input's 5*M*K + 8*M)
            db = b.bytes + head_bytes + (5 * M * Kh + 8 * M if mode == "separate" else 0)
            rec[mode] = {"launches": 2 if mode == "fused" else 3, "eager": _stats(eager, db),
                         "graph_replay": _stats(replay, db)}
            if mode == "fused":
                tern.tern_linear_stack_status(b.plan)
            del b, g, xd, logits
        rec["note"] = "the other linears take independent synthetic activations (one per shared group)"
        emit(rec)
    # --- the same 252-linear stack at 16 tokens (a longer verify pass), one launch
    b16 = st.bind(16)
    us = _event_times(lambda i: b16.run(), 20)
    emit({"suite": "stack8b_m16", "workload": "full 8B-shaped stack (252 linears) at M = 16, one stack launch",
          "M": 16, "kernel": kernel_name(b16.plan), **_stats(us, b16.bytes)})
    del b16

    # --- per-layer input sharing: q/k/v read one activation buffer, gate/up
    # another (a real layer's call layout), beside independent activations
    for M in (1, 8):
        rec = {"suite": "stack8b_shared_inputs", "workload": "full 8B-shaped stack (252 linears), M = %d: "
               "q/k/v and gate/up sharing one input per layer, against independent inputs" % M, "M": M}
        for share in (False, True):
            b = st.bind(M, share_inputs=share)
            us = _event_times(lambda i: b.run(), 40)
            # algorithmic bytes: a shared input is read once per group
            nb_ = b.bytes - (108 * (M * 4096 + 8 * M) if share else 0)  # 3 reads saved per layer
            rec["shared" if share else "independent"] = {"kernel": kernel_name(b.plan),
                                                         "restages_per_pass": int(b.plan.restages),
                                                         **_stats(us, nb_)}
            del b
        emit(rec)
    del st, Whd, srhd, rshd
    torch.cuda.empty_cache()

    # --- block-wise scales inside the stack launch: the full 8B-shaped stack
    # with one fp32 scale and int32 row sum per block of B columns (8 bytes
    # of metadata per row and block counted in the bytes)
    # (at M = 8 blocks of 128 columns run token by token on the vector ALU)
    for B in (128, 512):
        stb = DeviceStack("8b", seed=6, threads=16, block=B)
        for M in (1, 8):
            b = stb.bind(M)
            us = _event_times(lambda i: b.run(), 20)
            emit({"suite": "stack8b_blocked", "workload": "full 8B-shaped stack (252 linears), block scales "
                  "every %d columns, M = %d, one stack launch" % (B, M), "B": B, "M": M,
                  "kernel": kernel_name(b.plan), **_stats(us, b.bytes)})
            del b
        del stb
        torch.cuda.empty_cache()

    # --- activation quantiser (launch-bound at decode sizes)
    for M in (1, 8, 512):
        x = np.random.default_rng([M, 5]).normal(0, 1, (M, 4096)).astype(np.float32)
        xd = torch.from_numpy(x).to(dev)
        qd = torch.empty((M, 4096), dtype=torch.int8, device=dev)
        sd = torch.empty(M, dtype=torch.float32, device=dev)
        zd = torch.empty(M, dtype=torch.int32, device=dev)
        us = _event_times(lambda i: tern.tern_quantize_act(xd, M, 4096, 4096, qd, 4096, sd, zd), 100)
        ot, oreps = oracle_time(lambda: oracle.quantize_act(x, lib=olib), 1.0)
        st_ = _stats(us, 5 * M * 4096 + 8 * M)
        if M < 512:
            st_.pop("frac_of_peak")
        emit({"suite": "quantize", "workload": "per-token int8 quantisation of M x 4,096 fp32 "
              "activations, M = %d" % M, "M": M, "kernel": "quant_kernel", **st_,
              "cpu_oracle": {"us": round(ot * 1e6, 2), "cores": cores, "reps": oreps}})


def prefill_case(args, M: int):
    """Four 8B layers at M tokens, --steps launches after the warm-up (a
    profiling workload for the prefill GEMM); prints one JSON line."""
    import torch
    from packed_bit_gemv_tern_amd import synth
    from packed_bit_gemv_tern_amd.stack import DeviceStack
    st4 = DeviceStack("8b", layers=4, seed=3, threads=16)
    b4 = st4.bind(M)
    us = _event_times(lambda i: b4.run(), args.steps, warm=args.warmup, warm_s=args.warmup_seconds)
    st = _stats(us, b4.bytes)
    dense_ops = 2 * M * sum(N * K for (_, _, _, N, K, _) in synth.stack_specs("8b", 4))
    st["dense_TOPS"] = round(dense_ops / st["median_us"] / 1e6, 2)
    st["frac_of_int8_peak"] = round(st["dense_TOPS"] / INT8_DENSE_PEAK_TOPS, 4)
    print(json.dumps({"case": "prefill_4layers", "M": M, "kernel": kernel_name(b4.plan), **st}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="untimed warm-up lasts at least this long (and --warmup steps)")
    ap.add_argument("--layers", type=int, default=None, help="fewer layers (testing only)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth probe")
    ap.add_argument("--only", choices=["m1", "m8", "prefill64", "prefill512"], default=None,
                    help="launch a single pass per step (for profiling); prefill64 / prefill512: "
                         "four 8B layers (28 linears) at M = 64 / 512 instead of the headline")
    ap.add_argument("--suite", action="store_true",
                    help="measure the single GEMV, one 8B layer, the prefill sweeps, the 0.6B "
                         "stack, the int8 head, block scales, 1.6-bit rows, the quantisers and a "
                         "graph-captured decode step instead (one JSON line each)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times "
                         "(reference for the HBM byte counters) and exit")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="no GPU: read the rocprofv3 counter runs under DIR (pmc_<C>_<m1|m8|copy>/"
                         "run_counter_collection.csv for C = FETCH_SIZE, WRITE_SIZE) and write "
                         "profiles/traffic.json for the current sources")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return

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
    if args.suite:
        suite(args)
        return
    if args.only in ("prefill64", "prefill512"):
        prefill_case(args, 64 if args.only == "prefill64" else 512)
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

    # untimed warm-up: at least --warmup steps and --warmup-seconds of them
    # (the first launches after the stacks are built run up to ~8 % slow)
    t_w = time.perf_counter()
    warm_steps = 0
    while warm_steps < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        step()
        warm_steps += 1
        if warm_steps % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w
    log("warmup done: %d steps, %.2f s" % (warm_steps, warm_s))

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
            "median_us": round(ms[len(ms) // 2] * 1e3, 3),
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
        "warmup_steps_run": warm_steps,
        "warmup_s": round(warm_s, 3),
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
