#!/usr/bin/env python3
"""Benchmark of the exact-integer block-quantized projection on one MI355X.

Metric: bit-exact int GEMM -- weight GB/s at T=1 and useful TOPS at T=512,
each as a fraction of its roofline, on a 14336x4096 Q8 matrix (a 7B-class
dense projection; synthetic seeded codes, Q24 scales and Q16 activations).

One step = one decode pass (a T=1 projection over each of `--copies` distinct
resident copies of the weights, so the 256 MB Infinity Cache cannot serve
them), one T=512 prefill projection, the 24-layer Qwen2.5-0.5B-shaped FFN
chain (T=30) and the OLMoE-shaped routed FFN (64 experts, 512 tokens, top-8).
Each part is recorded once as a HIP graph and replayed; HIP events on the
launch stream time every part of every step.  After timing, every output is
checked bit-exactly against the CPU oracle: whole-output digests (all 14336
T=1 outputs of every copy, all 512 x 14336 prefill outputs, the chain's final
activations, all 4096 x 2048 routed outputs), and the prefill element by
element against the oracle run of the CPU baseline.

Prints ONE JSON line.  `value` is the decode weight bandwidth (GB/s); the
prefill rate, the chain and routed FFN rates, their roofline fractions, and
the oracle timed on the host cores (`cpu_baseline`) ride along in the same
line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "bit-exact int GEMM: weight GB/s (T=1) + useful TOPS (T=512), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, published
N, K = 14336, 4096
LIMBS = 3                      # Q16 activations with |x| <= 2^22 need 3 balanced base-256 limbs
W_BYTES = N * K + N * (K // 32) * 4          # canonical Q8: 1 B/code + 4 B/32-block scale
GEMV_KERNEL = "gemv_kernel"
GEMM_KERNEL = "gemm_tiled_qreg_kernel"   # the T=512 kernel for narrow scales (the synthetic Q24 ones)
# the source file each timed kernel is built from: a stored HBM-traffic figure
# is used only while that file is unchanged
KERNEL_SOURCES = {GEMV_KERNEL: "gemv.hip", GEMM_KERNEL: "gemm_tiled.hip"}
# the template instance each timed kernel runs as in the bench step (the routed
# FFN in the same step runs other instances of the same templates)
KERNEL_MATCH = {GEMV_KERNEL: "gemv_kernel<3, 1, long, 8, 2, false>",
                GEMM_KERNEL: "gemm_tiled_qreg_kernel<false, false, true, 1>"}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
GOLDEN = os.path.join(ROOT, "tests", "golden", "oracle_digests.json")


def kernel_source_hash(kernel: str) -> str:
    p = os.path.join(ROOT, "exact_integer_amd", "csrc", KERNEL_SOURCES[kernel])
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    rec = json.load(open(TRAFFIC_JSON)).get(kernel)
    if not rec or rec.get("source_sha") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def summarize_counters(fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str) -> int:
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, each on
    `bench.py --profile` and on `bench.py --copy-calibration`) into HBM bytes per
    launch of the timed kernels, scaled by what the same counters read for the
    256 MiB copy, and write profiles/traffic.json."""
    import csv
    import statistics

    def per_kernel(d):
        out = {}
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    def copy_kib(d):
        vals = [v for k, vs in per_kernel(d).items() if "copyBuffer" in k for v in vs]
        return statistics.median(vals)

    true_kib = (256 << 20) / 1024
    f_fac, w_fac = true_kib / copy_kib(copy_fetch_dir), true_kib / copy_kib(copy_write_dir)
    fetch, write = per_kernel(fetch_dir), per_kernel(write_dir)
    out = {"_calibration": {"copy_bytes": 256 << 20, "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4)}}
    for kern in (GEMV_KERNEL, GEMM_KERNEL):
        fk = [v for k, vs in fetch.items() if KERNEL_MATCH[kern] in k for v in vs]
        wk = [v for k, vs in write.items() if KERNEL_MATCH[kern] in k for v in vs]
        if not fk or not wk:
            continue
        f_b, w_b = statistics.median(fk) * 1024 * f_fac, statistics.median(wk) * 1024 * w_fac
        out[kern] = {"bytes_per_launch": int(f_b + w_b), "fetch_bytes": int(f_b), "write_bytes": int(w_b),
                     "launches_sampled": len(fk), "source_sha": kernel_source_hash(kern)}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out))
    return 0


SQ_JSON = os.path.join(ROOT, "profiles", "sq_counters.json")
XCDS, SIMDS = 8, 1024   # MI355X: GRBM_GUI_ACTIVE is summed over 8 XCDs; 256 CUs x 4 SIMDs


def summarize_sq(pass1: str, pass2: str) -> int:
    """Two rocprofv3 --pmc runs of `bench.py --profile` (SQ instruction and
    busy counters) -> per-kernel medians, VALU / MFMA busy fractions, the
    engine clock under load and the VALU ceiling (the launch's VALU
    instructions at one per 4 cycles on each of the 1024 SIMDs), written to
    profiles/sq_counters.json."""
    import csv
    import statistics

    vals = {}
    for d in (pass1, pass2):
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            for kern in (GEMM_KERNEL,):
                if KERNEL_MATCH[kern] in r["Kernel_Name"]:
                    v = vals.setdefault(kern, {})
                    v.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    v.setdefault("_ns", []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for kern, v in vals.items():
        m = {k: statistics.median(x) for k, x in v.items()}
        us = m["_ns"] / 1e3
        cyc = m["GRBM_GUI_ACTIVE"] / XCDS
        clock = cyc / (us * 1e-6) / 1e9
        valu_ceiling_us = m["SQ_INSTS_VALU"] * 4 / SIMDS / (clock * 1e9) * 1e6
        out[kern] = {
            "duration_us": round(us, 2), "clock_ghz": round(clock, 3),
            "valu_insts": int(m["SQ_INSTS_VALU"]), "valu_int64_insts": int(m.get("SQ_INSTS_VALU_INT64", 0)),
            "mfma_insts": int(m["SQ_INSTS_MFMA"]), "lds_insts": int(m["SQ_INSTS_LDS"]),
            "valu_busy": round(m["SQ_ACTIVE_INST_VALU"] * 4 / SIMDS / cyc, 4),
            "mfma_busy": round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / cyc, 4),
            "valu_ceiling_us": round(valu_ceiling_us, 2),
            "lds_bank_conflicts": int(m.get("SQ_LDS_BANK_CONFLICT", 0)),
            "source_sha": kernel_source_hash(kern)}
    with open(SQ_JSON, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out))
    return 0


def stored_sq(kernel: str):
    """The committed SQ counter summary of `kernel`, if taken on the current source."""
    if not os.path.exists(SQ_JSON):
        return None
    rec = json.load(open(SQ_JSON)).get(kernel)
    return rec if rec and rec.get("source_sha") == kernel_source_hash(kernel) else None


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform string."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_threads() -> int:
    """Threads for the multi-threaded oracle leg: the CPUs this process may run
    on, capped at OMP_NUM_THREADS when that is set (a shared host gives each
    GPU's jobs a share of its cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap))) if cap and cap.isdigit() else n


def cpu_baseline(q, s, x1, x512, runs: int = 3, t1_seconds: float = 1.0, t512_rows_1thread: int = 256):
    """The CPU oracle, as it stands, on the host cores, on the same input
    bytes; median of `runs` runs of each leg (GEMM loops only):
      * T=1 over the whole matrix, repeated for about `t1_seconds` per run,
        with one thread and with cpu_threads() threads (disjoint output rows);
      * T=512 over all rows with cpu_threads() threads (its output is kept for
        the full-output parity check), and over the first `t512_rows_1thread`
        rows with one thread.
    Returns (record, y at T=1, y at T=512)."""
    import statistics
    import oracle
    nt = cpu_threads()

    def t1(threads):
        times = []
        for _ in range(runs):
            reps, t0 = 0, time.perf_counter()
            while True:
                y = oracle.q8(q, s, x1, threads=threads)
                reps += 1
                if time.perf_counter() - t0 >= t1_seconds:
                    break
            times.append((time.perf_counter() - t0) / reps)
        return statistics.median(times), y

    def t512(threads, rows):
        times = []
        for _ in range(runs):
            t0 = time.perf_counter()
            y = oracle.q8(q[:rows], s[:rows], x512, threads=threads)
            times.append(time.perf_counter() - t0)
        return statistics.median(times), y

    d1_n, y1 = t1(nt)
    d1_1, _ = t1(1)
    p_n, y512 = t512(nt, N)
    p_1, _ = t512(1, t512_rows_1thread)
    use_n = LIMBS * 2.0 * 512 * N * K
    use_1 = LIMBS * 2.0 * 512 * t512_rows_1thread * K
    return {
        "value": W_BYTES / d1_n / 1e9, "unit": "GB/s", "cores": nt, "kind": "oracle",
        "sample": f"median of {runs} runs per leg. T=1: all {N} rows, passes repeated for ~{t1_seconds:g} s per run, "
                  f"{nt} threads and 1 thread; T=512: all {N} rows with {nt} threads, rows 0..{t512_rows_1thread - 1} "
                  f"with 1 thread",
        "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
        "threads_note": "threads = the CPUs this process may use, capped at OMP_NUM_THREADS (the host's share of CPUs per GPU)",
        "t1_ms": d1_n * 1e3, "t1_ms_1thread": d1_1 * 1e3, "value_1thread": W_BYTES / d1_1 / 1e9,
        "t512_s": p_n, "t512_useful_tops": use_n / p_n / 1e12, "t512_logical_tops": use_n / LIMBS / p_n / 1e12,
        "t512_1thread_s_per_row_sample": p_1, "t512_useful_tops_1thread": use_1 / p_1 / 1e12,
        "t512_logical_tops_1thread": use_1 / LIMBS / p_1 / 1e12,
    }, y1, y512


def copy_calibration(torch, dev) -> int:
    """A plain copy of known size: each launch reads and writes 256 MiB.  The
    HBM byte counters of this copy give the scale factor for the counters
    read on the projection kernels."""
    nbytes = 256 << 20
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5,
                      "ms_per_copy": round(ms, 4), "copy_gbs_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}))
    return 0


def _time_graph(torch, fn, steps: int, warmup: int, reps: int = 1):
    """Record fn (reps times in a row) as a HIP graph, replay it warmup + steps
    times; median ms per call of fn from HIP events on the capturing stream.
    Work of a few microseconds needs reps > 1: a replay's events also see the
    host's submission of the graph when the device finishes first."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(); g.replay(); b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) / reps for a, b in ev)
    return ms[len(ms) // 2], wall / steps * 1e3


def bench_q4_table(args, torch, np, ei, synth, dev) -> int:
    """The 4-bit projections of the d512 workload (512x512, 2048x512,
    512x2048; T=1 and T=64) by the table-read derivation and by the MFMA/GEMV
    path, each timed as one graph of all six projections; parity: the two agree
    and match the stored oracle digests."""
    import json as _json
    gold = _json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))["q4_d512"]
    cases = []
    for name, (n, k) in synth.Q4_SHAPES.items():
        nib, sme = synth.q4_d512_matrix(name)
        nd, sd = torch.from_numpy(nib).to(dev), torch.from_numpy(sme).to(dev)
        w = ei.pack_q4(nd, sd)
        for t in (1, 64):
            x = torch.from_numpy(synth.q4_d512_x(k, t)).to(dev)
            cases.append((f"{name}_t{t}", n, k, t, nd, sd, w, x, torch.empty((t, n), dtype=torch.int64, device=dev),
                          torch.empty((t, n), dtype=torch.int64, device=dev),
                          torch.empty(max(ei.workspace_bytes(w, t), 1), dtype=torch.uint8, device=dev),
                          torch.empty(max(ei.q4_table_workspace_bytes(n, k, t), 1), dtype=torch.uint8, device=dev)))
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step_table():
        for _, n, k, t, nd, sd, w, x, yt, ym, ws, wt in cases:
            ei.gemm_q4_table(nd, sd, x, out=yt, workspace=wt, status=status)

    def step_mfma(limbs):
        def f():
            for _, n, k, t, nd, sd, w, x, yt, ym, ws, wt in cases:
                ei.gemm_q4(w, x, limbs, out=ym, workspace=ws, status=status)
        return f

    ms_t, wall_t = _time_graph(torch, step_table, args.steps, args.warmup, reps=10)
    ok = True
    ms_m = {}
    for limbs in (3, 2):   # the two-limb form (x - 128 split, row offsets added back) last
        ms_m[limbs], _ = _time_graph(torch, step_mfma(limbs), args.steps, args.warmup, reps=10)
        ok = ok and all(ei.digest(ym) == gold[name] for name, n, k, t, nd, sd, w, x, yt, ym, ws, wt in cases)
    ok = ok and int(status.item()) == 0 and all(ei.digest(yt) == gold[name]
                                                for name, n, k, t, nd, sd, w, x, yt, ym, ws, wt in cases)
    logical = sum(2.0 * t * n * k for _, n, k, t, *rest in cases)
    tops = logical / (ms_t * 1e-3) / 1e12
    # int32 VALU peak in lane-ops/s: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz = 39.3 T (a wave64
    # instruction issues over 4 clocks; the 157.3 TFLOP/s fp32 figure counts an FMA as 2 and packed fp32 as 2
    # more, neither of which an int32 add or shift has).  `achieved` counts logical ops 2*T*N*K, while a
    # table read spends at least one table read and one add per logical multiply-add.
    alu_peak = 256 * 4 * 16 * 2.4e9 / 1e12
    print(json.dumps({
        "metric": "4-bit projection by table reads: logical int TOPS", "value": round(tops, 3), "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_t, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32 x 4-bit by table reads",
        "data": "synthetic (seeded 4-bit codes and m*2^e scale bytes, int32 activations)",
        "config": {"workload": "q4_d512_table_read", "shapes": list(synth.Q4_SHAPES.values()), "tokens": [1, 64],
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "alu", "achieved": round(tops, 3), "peak": round(alu_peak, 2), "unit": "TOP/s",
                     "frac": round(tops / alu_peak, 4), "traffic": None, "step_ms": round(ms_t, 4)},
        "mfma_path_step_ms": round(ms_m[2], 4), "mfma_path_3_limbs_step_ms": round(ms_m[3], 4),
        "parity": {"table_read_and_mfma_digests_equal_oracle": ok}}))
    return 0 if ok else 1


def bench_schedule_gate(args, torch, np, ei, synth, dev) -> int:
    """The two small workloads, timed per schedule: the single 896x896 Q8
    projection at T=1, and the schedule gate's Q (896x896), K and V (128x896)
    projections of a 4-token prefix (also as one batched launch of the three).
    Both are cache-resident and launch-bound, so they are reported in
    microseconds.  Parity: every schedule's digest equals the oracle's; the
    float32 shadow of Q/K/V is run in the five orders for contrast and its
    distinct digests are counted (the integer ones must be one per matrix)."""
    import json as _json
    gold = _json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    scheds = ("canonical", "reversed", "tiled_shuffled", "split_k", "tree_walk")

    def prepare(c, sc, x):
        w = ei.pack_q8(torch.from_numpy(c).to(dev), torch.from_numpy(sc).to(dev))
        t = x.shape[0]
        return {"w": w, "y": torch.empty((t, w.n), dtype=torch.int64, device=dev),
                "ws": {sd: torch.empty(max(ei.workspace_bytes(w, t, 3, sd), 1), dtype=torch.uint8, device=dev)
                       for sd in ("default",) + scheds}}

    (c0, s0), x0 = synth.q8_896_inputs()
    x0d = torch.from_numpy(x0).to(dev)
    m0 = prepare(c0, s0, x0)
    mats, xq = synth.qkv_inputs()
    xqd = torch.from_numpy(xq).to(dev)
    mq = {name: prepare(c, sc, xq) for name, (c, sc) in mats.items()}
    out, ok = {"q8_896x896_t1": {}, "qkv_t4": {}}, True
    for sd in ("default",) + scheds:
        def one():
            ei.gemm_q8(m0["w"], x0d, 3, sd, 0xE1, out=m0["y"], workspace=m0["ws"][sd], status=status)

        def qkv():
            for m in mq.values():
                ei.gemm_q8(m["w"], xqd, 3, sd, 0xE1, out=m["y"], workspace=m["ws"][sd], status=status)

        ms, _ = _time_graph(torch, one, args.steps, args.warmup, reps=20)
        out["q8_896x896_t1"][sd] = round(ms * 1e3, 2)
        ok = ok and ei.digest(m0["y"]) == gold["q8_896x896"]["y"]
        ms, _ = _time_graph(torch, qkv, args.steps, args.warmup, reps=20)
        out["qkv_t4"][sd] = round(ms * 1e3, 2)
        ok = ok and all(ei.digest(m["y"]) == gold["qkv_gate"][name] for name, m in mq.items())
    outs = [m["y"] for m in mq.values()]

    def qkv_batched():
        ei.gemm_q8_multi([m["w"] for m in mq.values()], xqd, 3, outs=outs, status=status)

    ms_b, _ = _time_graph(torch, qkv_batched, args.steps, args.warmup, reps=20)
    ok = ok and all(ei.digest(m["y"]) == gold["qkv_gate"][name] for name, m in mq.items())
    shadow = {}
    for name, (c, sc) in mats.items():
        cd, scd = torch.from_numpy(c).to(dev), torch.from_numpy(sc).to(dev)
        shadow[name] = len({ei.digest(ei.fp32_shadow(cd, scd, xqd, sd, seed=0xE1)) for sd in scheds})
    ok = ok and int(status.item()) == 0
    wbytes = 896 * 896 * (1 + 4 / 32)
    us = out["q8_896x896_t1"]["default"]
    print(json.dumps({
        "metric": "896x896 Q8 projection at T=1 (default schedule): microseconds per launch", "value": us,
        "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 codes, Q24 block scales, Q16 activations)",
        "config": {"workload": "q8_896x896_t1_and_qkv_schedule_gate", "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(wbytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "note": "0.9 MB of weights: cache-resident and launch-bound, so the fraction is not its bound"},
        "us_per_schedule": out, "qkv_t4_batched_us": round(ms_b * 1e3, 2),
        "fp32_shadow_distinct_digests_of_5": shadow,
        "parity": {"every_schedule_digest_equals_oracle": ok}}))
    return 0 if ok else 1


def bench_wide(args, torch, np, ei, synth, dev) -> int:
    """The wide-code hot kernel: 12-trit codes 896x896 against 4096 rows of
    int32 activations, exact int64 output; i8-MFMA bound (12 digit products
    per tile and block, no per-block epilogue)."""
    c, a = synth.wide_inputs()
    w = ei.pack_wide(torch.from_numpy(c).to(dev))
    xd = torch.from_numpy(a).to(dev)
    T, N, K = a.shape[0], c.shape[0], c.shape[1]
    y = torch.empty((T, N), dtype=torch.int64, device=dev)
    ws = torch.empty(int(ei.lib().ei_wide_workspace_bytes(ctypes.byref(w.desc), T)), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        ei.gemm_wide(w, xd, out=y, workspace=ws, status=status)

    ms, wall_ms = _time_graph(torch, step, args.steps, args.warmup)
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))["wide_896x896_t4096"]["y"]
    ok = int(status.item()) == 0 and ei.digest(y) == gold
    logical = 2.0 * T * N * K
    digit_ops = 12 * logical
    tops = digit_ops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "wide-code exact GEMM: i8 digit TOPS", "value": round(tops, 1), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32 digits, int64 result",
        "data": "synthetic (12-trit codes, activations quantized per tensor to 2^28)",
        "config": {"workload": "wide_896x896_t4096", "rows": T, "n": N, "k": K, "weight_digits": 3,
                   "act_digits": 4, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(tops / I8_PEAK_TOPS, 4), "traffic": None, "step_ms": round(ms, 4),
                     "note": "i8 ops = 12 digit products x 2*T*N*K; the step includes the activation digit split"},
        "logical_tops": round(logical / (ms * 1e-3) / 1e12, 2),
        "parity": {"digest_equals_oracle": ok}}))
    return 0 if ok else 1


def bench_olmoe_router(args, torch, np, ei, synth, dev) -> int:
    """The OLMoE-shaped routed FFN behind an integer router: the router's Q8
    projection (64 x 2048) of the 512 tokens, integer top-8, then the routed
    FFN on that route, all inside the timed step."""
    E, H, I, T, TOPK = synth.OLMOE_E, synth.OLMOE_H, synth.OLMOE_I, synth.OLMOE_T, synth.OLMOE_TOPK
    mats = [synth.olmoe_expert(e) for e in range(E)]

    def stack(m, k):
        return torch.from_numpy(np.ascontiguousarray(np.stack([mm[m][k] for mm in mats]))).to(dev)
    wg, wu, wd = (ei.pack_q8_stacked(stack(m, 0), stack(m, 1)) for m in range(3))
    del mats
    rc, rs = synth.olmoe_router()
    wr = ei.pack_q8(torch.from_numpy(rc).to(dev), torch.from_numpy(rs).to(dev))
    xd = torch.from_numpy(synth.olmoe_x()).to(dev)
    scores = torch.empty((T, E), dtype=torch.int64, device=dev)
    route = torch.empty((T, TOPK), dtype=torch.int32, device=dev)
    out = torch.empty((T * TOPK, H), dtype=torch.int64, device=dev)
    ws_r = torch.empty(max(ei.workspace_bytes(wr, T), 1), dtype=torch.uint8, device=dev)
    ws = torch.empty(ei.moe_ffn_workspace_bytes(wg, wd, T, TOPK), dtype=torch.uint8, device=dev)
    lut = ei.silu_lut(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        ei.gemm_q8(wr, xd, out=scores, workspace=ws_r, status=status)
        ei.topk_route(scores, TOPK, out=route)
        ei.moe_ffn_q8(wg, wu, wd, xd, route, lut, out=out, workspace=ws, status=status)

    ms, wall_ms = _time_graph(torch, step, args.steps, args.warmup)
    gold = json.load(open(GOLDEN))["olmoe_router"]
    route_ok = int(status.item()) == 0 and ei.digest(route) == gold["route"]
    ok = route_ok and ei.digest(out) == gold["y"]
    wbytes = 3 * E * I * H * (1 + 4 / 32) + E * H * (1 + 4 / 32)
    gbs = wbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "routed expert FFN with integer router: weight GB/s", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 experts and router, Q16 activations; route from the integer router)",
        "config": {"workload": "olmoe_router_ffn", "experts": E, "hidden": H, "intermediate": I, "tokens": T,
                   "top_k": TOPK, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "step_ms": round(ms, 4),
                     "weight_bytes": int(wbytes)},
        "parity": {"route_digest_equals_oracle": route_ok, "full_output_digest_equals_oracle": ok}}))
    return 0 if ok else 1


def setup_olmoe(torch, np, ei, synth, dev):
    """The OLMoE-shaped routed FFN: 64 experts (gate/up 1024x2048, down
    2048x1024, Q8), 512 tokens, top-8: grouped gate and up projections in one
    pass with the SiLU-gated product, then the grouped down projection, in one
    int_moe_ffn_q8 call.  HBM-bound: every expert's weights are read once per
    step.  Returns the step, its parity check (the whole output's digest
    against the oracle's) and the byte / op counts."""
    E, H, I, T, TOPK = synth.OLMOE_E, synth.OLMOE_H, synth.OLMOE_I, synth.OLMOE_T, synth.OLMOE_TOPK
    mats = [synth.olmoe_expert(e) for e in range(E)]

    def stack(m, k):
        return torch.from_numpy(np.ascontiguousarray(np.stack([mm[m][k] for mm in mats]))).to(dev)
    wg, wu, wd = (ei.pack_q8_stacked(stack(m, 0), stack(m, 1)) for m in range(3))
    del mats
    xd, rd = torch.from_numpy(synth.olmoe_x()).to(dev), torch.from_numpy(synth.olmoe_route()).to(dev)
    P = T * TOPK
    out = torch.empty((P, H), dtype=torch.int64, device=dev)
    ws = torch.empty(ei.moe_ffn_workspace_bytes(wg, wd, T, TOPK), dtype=torch.uint8, device=dev)
    lut = ei.silu_lut(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    gold = json.load(open(GOLDEN))["olmoe_step"]["y"]

    def step():
        ei.moe_ffn_q8(wg, wu, wd, xd, rd, lut, out=out, workspace=ws, status=status)

    def check() -> bool:
        return int(status.item()) == 0 and ei.digest(out) == gold

    return {"step": step, "check": check, "wbytes": 3 * E * I * H * (1 + 4 / 32),
            "useful": LIMBS * 2.0 * P * 3 * I * H, "config": {"experts": E, "hidden": H, "intermediate": I,
                                                              "tokens": T, "top_k": TOPK}}


def bench_olmoe(args, torch, np, ei, synth, dev) -> int:
    """The routed FFN alone (see setup_olmoe)."""
    o = setup_olmoe(torch, np, ei, synth, dev)
    ms, wall_ms = _time_graph(torch, o["step"], args.steps, args.warmup)
    ok = o["check"]()
    gbs = o["wbytes"] / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "routed expert FFN: weight GB/s", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 experts, Q16 activations, uniform top-8 routing)",
        "config": {"workload": "olmoe_grouped_ffn", **o["config"], "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "step_ms": round(ms, 4),
                     "weight_bytes": int(o["wbytes"])},
        "useful_tops": round(o["useful"] / (ms * 1e-3) / 1e12, 2),
        "parity": {"full_output_digest_equals_oracle": ok}}))
    return 0 if ok else 1


def setup_qwen(torch, ei, synth, dev, prenorm: bool = False):
    """The Qwen2.5-0.5B-shaped FFN chain: 24 layers of gate and up (4864x896)
    and down (896x4864) Q8 projections at T=30 with the SiLU-gated product and
    the residual add (pre-norm: an integer RMSNorm in front of every layer),
    fresh weights per layer (353 MB, read once per step), run as one chain
    call.  Parity: the final layer's output digest against the oracle's."""
    layers = []
    for layer in range(synth.QWEN_LAYERS):
        (gc, gs), (uc, us), (dc, ds) = synth.qwen_ffn_layer(layer)
        t = [torch.from_numpy(a).to(dev) for a in (gc, gs, uc, us, dc, ds)]
        layers.append((ei.pack_q8(t[0], t[1]), ei.pack_q8(t[2], t[3]), ei.pack_q8(t[4], t[5])))
    x0 = torch.from_numpy(synth.qwen_ffn_x0()).to(dev)
    T, D, F = synth.QWEN_T, synth.QWEN_D, synth.QWEN_F
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]
    ws = torch.empty(max(ei.ffn_workspace_bytes(layers[0][0], layers[0][2], T),
                         ei.ffn_chain_workspace_bytes(layers[0][0], layers[0][2], T), 1), dtype=torch.uint8, device=dev)
    lut = ei.silu_lut(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    norms = [torch.from_numpy(synth.qwen_norm_weight(i)).to(dev) for i in range(synth.QWEN_LAYERS)]
    final = bufs[(synth.QWEN_LAYERS - 1) % 2]
    gold = json.load(open(GOLDEN))["qwen05b_ffn_prenorm" if prenorm else "qwen05b_ffn"]["layers"][-1]["x_next"]

    def step():   # the whole stack in one call
        if prenorm:
            ei.ffn_q8_prenorm_chain(layers, norms, synth.QWEN_RMS_EPS_Q32, x0, lut, out=final, workspace=ws,
                                    status=status)
        else:
            ei.ffn_q8_chain(layers, x0, lut, out=final, workspace=ws, status=status)

    def step_layers():   # the pre-norm stack as 24 layer calls: layer l reads x_l and writes x_{l+1}
        src = x0
        for i, (wg, wu, wd) in enumerate(layers):
            dst = bufs[i % 2]
            ei.ffn_q8_prenorm(wg, wu, wd, norms[i], synth.QWEN_RMS_EPS_Q32, src, lut, out=dst, workspace=ws,
                              status=status)
            src = dst

    def check() -> bool:
        ok = int(status.item()) == 0 and ei.digest(final) == gold
        final.zero_()
        return ok

    return {"step": step, "step_layers": step_layers, "check": check,
            "wbytes": synth.QWEN_LAYERS * 3 * F * D * (1 + 4 / 32),
            "useful": LIMBS * 2.0 * T * 3 * F * D * synth.QWEN_LAYERS,
            "config": {"tokens": T, "hidden": D, "intermediate": F, "layers": synth.QWEN_LAYERS}}


def bench_qwen_ffn(args, torch, np, ei, synth, dev, prenorm: bool = False) -> int:
    """The FFN chain alone (see setup_qwen); with prenorm, also as 24 layer calls."""
    qw = setup_qwen(torch, ei, synth, dev, prenorm)
    layer_calls_ms, ok_layers = None, True
    if prenorm:
        layer_calls_ms, _ = _time_graph(torch, qw["step_layers"], args.steps, args.warmup)
        ok_layers = qw["check"]()
    ms, wall_ms = _time_graph(torch, qw["step"], args.steps, args.warmup)
    ok = qw["check"]() and ok_layers
    gbs = qw["wbytes"] / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": ("24-layer pre-norm Q8 FFN chain" if prenorm else "24-layer Q8 FFN chain") + ": weight GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 layers, Q16 activations)",
        "config": {"workload": "qwen05b_ffn_24_layers" + ("_prenorm" if prenorm else ""), **qw["config"],
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "step_ms": round(ms, 4),
                     "weight_bytes": int(qw["wbytes"])},
        **({"layer_calls_step_ms": round(layer_calls_ms, 4)} if prenorm else {}),
        "parity": {"final_digest_equals_oracle": ok}}))
    return 0 if ok else 1


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=12, help="distinct resident weight copies for the T=1 pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true", help="short run for rocprofv3 (no baseline, few steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 256 MiB, 5 times (the reference for HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output directories -> profiles/traffic.json (no GPU needed)")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PASS1", "PASS2"),
                    help="two rocprofv3 --pmc output directories of SQ counters -> profiles/sq_counters.json")
    ap.add_argument("--workload", choices=("dense", "olmoe", "olmoe_router", "qwen_ffn", "qwen_ffn_prenorm", "wide",
                                           "q4_table", "schedule_gate"),
                    default="dense",
                    help="dense: the 14336x4096 decode + prefill step (default); olmoe / qwen_ffn: the routed "
                         "expert FFN or the 24-layer FFN chain, timed the same way; olmoe_router: the routed "
                         "FFN behind the integer router; qwen_ffn_prenorm: the chain with an integer RMSNorm "
                         "in front of every layer; wide: the 12-trit wide-code GEMM (896x896, 4096 rows); q4_table: the "
                         "4-bit projections by table reads against the MFMA path; schedule_gate: the 896x896 projection at T=1 "
                         "and the Q/K/V schedule gate, per schedule")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.summarize_sq:
        return summarize_sq(*args.summarize_sq)
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the projection would shard by rows across GPUs)", file=sys.stderr)
        return 2
    if args.profile:
        args.steps, args.warmup, args.no_cpu_baseline = 5, 2, True

    import numpy as np
    import torch
    import exact_integer_amd as ei
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no HIP device", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        return copy_calibration(torch, dev)
    if args.workload == "olmoe":
        return bench_olmoe(args, torch, np, ei, synth, dev)
    if args.workload == "q4_table":
        return bench_q4_table(args, torch, np, ei, synth, dev)
    if args.workload == "schedule_gate":
        return bench_schedule_gate(args, torch, np, ei, synth, dev)
    if args.workload == "wide":
        return bench_wide(args, torch, np, ei, synth, dev)
    if args.workload == "olmoe_router":
        return bench_olmoe_router(args, torch, np, ei, synth, dev)
    if args.workload in ("qwen_ffn", "qwen_ffn_prenorm"):
        return bench_qwen_ffn(args, torch, np, ei, synth, dev, prenorm=args.workload == "qwen_ffn_prenorm")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    gold = json.load(open(GOLDEN))
    q, s = synth.dense_w()
    x1, x512 = synth.dense_x(1), synth.dense_x(512)
    w0 = ei.pack_q8(to_dev(q), to_dev(s))
    copies = [w0]
    for _ in range(args.copies - 1):
        buf = w0.buf.clone()
        d = ei.Weights.from_buffer_copy(w0.desc)
        d.packed = buf.data_ptr()
        copies.append(ei.PackedWeights(buf, d))
    x1d, x512d = to_dev(x1), to_dev(x512)
    y1 = torch.empty((args.copies, 1, N), dtype=torch.int64, device=dev)
    y512 = torch.empty((512, N), dtype=torch.int64, device=dev)
    ws = torch.empty(max(ei.workspace_bytes(w0, 512, LIMBS), 1), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    qw = setup_qwen(torch, ei, synth, dev)
    om = setup_olmoe(torch, np, ei, synth, dev)
    torch.cuda.synchronize()

    def decode():
        for c, w in enumerate(copies):
            ei.gemm_q8(w, x1d, LIMBS, out=y1[c], status=status)

    def prefill():
        ei.gemm_q8(w0, x512d, LIMBS, out=y512, workspace=ws, status=status)

    # One step: the T=1 decode pass over the copies, the T=512 prefill, the
    # 24-layer Qwen-shaped FFN chain (SiLU epilogue, residual) and the
    # OLMoE-shaped routed FFN (grouping, grouped projections): every part of
    # the path.  Each part is a HIP graph; events on the launch stream
    # bracket each part of each step.
    parts = [("decode", decode), ("prefill", prefill), ("qwen", qw["step"]), ("olmoe", om["step"])]
    graphs = []
    for _, fn in parts:   # eager run first (also the graph's warm-up)
        fn()
    torch.cuda.synchronize()
    for _, fn in parts:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs.append(g)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        for i, g in enumerate(graphs):
            g.replay()
            e[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    med = {}
    for i, (name, _) in enumerate(parts):
        ms = sorted(e[i].elapsed_time(e[i + 1]) for e in ev)
        med[name] = ms[len(ms) // 2]
    dec_med, pre_med = med["decode"], med["prefill"]
    if int(status.item()) != 0:
        print(f"bench.py: device status {int(status.item())}", file=sys.stderr)
        return 1

    # ---- the same decode pass as batched launches (int_gemm_q8_multi, up to
    # 16 matrices sharing x per launch): reported beside `value`, not in it
    yb = [torch.empty((1, N), dtype=torch.int64, device=dev) for _ in copies]
    batched, batched_ok = {}, True
    for group in (2, 16):   # 2: gate and up of one FFN layer; 16: the largest batch
        def decode_batched():
            for i in range(0, len(copies), group):
                ei.gemm_q8_multi(copies[i:i + group], x1d, LIMBS, outs=yb[i:i + group], status=status)

        batched[group], _ = _time_graph(torch, decode_batched, args.steps, args.warmup)
        batched_ok = batched_ok and {ei.digest(y) for y in yb} == {gold["dense_14336x4096"]["t1_y"]}
        yb = [torch.empty((1, N), dtype=torch.int64, device=dev) for _ in copies]

    # ---- the oracle on the host cores (it also yields every T=512 row)
    base = y512_ref = None
    if not args.no_cpu_baseline:
        base, _, y512_ref = cpu_baseline(q, s, x1, x512)

    # ---- parity of what was timed: whole outputs against the oracle
    dig = {ei.digest(y1[c]) for c in range(args.copies)}
    y512h = y512.cpu().numpy()
    parity = {
        "t1_digest_equals_oracle": dig == {gold["dense_14336x4096"]["t1_y"]},
        "t512_full_digest_equals_oracle": oracle_digest(y512h) == gold["dense_14336x4096"]["t512_y"],
        "t512_rows_checked_elementwise": 0,
        "t1_batched_digests_equal_oracle": batched_ok,
        "qwen_ffn_final_digest_equals_oracle": qw["check"](),
        "olmoe_full_output_digest_equals_oracle": om["check"](),
    }
    if y512_ref is not None:
        ok = bool((y512h == y512_ref).all())
        parity["t512_rows_checked_elementwise"] = N if ok else -1
    if not all(v for k, v in parity.items() if k != "t512_rows_checked_elementwise") or \
            parity["t512_rows_checked_elementwise"] < 0:
        print(json.dumps({"error": "parity failure", "parity": parity}))
        return 1

    # ---- rates
    per_gemv_ms = dec_med / args.copies
    algo_bytes = W_BYTES + K * 8 + N * 8                 # weights + x + y, one T=1 launch
    dec_gbs = W_BYTES * args.copies / (dec_med * 1e-3) / 1e9
    ach_gbs = algo_bytes / (per_gemv_ms * 1e-3) / 1e9
    useful = LIMBS * 2.0 * 512 * N * K
    pre_tops = useful / (pre_med * 1e-3) / 1e12
    tr_dec, tr_pre = stored_traffic(GEMV_KERNEL), stored_traffic(GEMM_KERNEL)

    def valu_ceiling(step_ms):
        # the prefill kernel is bound by its per-block VALU epilogue (exact
        # int64 scale multiply-adds): its VALU instructions at one per 4 cycles
        # on every SIMD, at the clock measured under load, give its ceiling
        sq = stored_sq(GEMM_KERNEL)
        if sq is None:
            return None
        return {"bound": "valu", "ceiling_us": sq["valu_ceiling_us"], "kernel_us_profiled": sq["duration_us"],
                "frac": round(sq["valu_ceiling_us"] / sq["duration_us"], 4),
                "valu_busy": sq["valu_busy"], "mfma_busy": sq["mfma_busy"], "clock_ghz": sq["clock_ghz"],
                "valu_insts_per_launch": sq["valu_insts"],
                "valu_insts_per_wave_block": round(sq["valu_insts"] / (512 // 32 * N // 32 * (K // 32)), 1),
                "step_us_this_run": round(step_ms * 1e3, 1),
                "source": "profiles/sq_counters.json (rocprofv3 --pmc of bench.py --profile)"}

    # a plain device copy: the measured HBM ceiling beside the datasheet's
    csrc_t = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cdst_t = torch.empty_like(csrc_t)
    cdst_t.copy_(csrc_t)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        cdst_t.copy_(csrc_t)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (256 << 20) * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc_t, cdst_t

    def hbm_part(name, rec):
        ms = med[name]
        gbs = rec["wbytes"] / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), **rec["config"],
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                             "weight_bytes": int(rec["wbytes"])},
                "useful_tops": round(rec["useful"] / (ms * 1e-3) / 1e12, 2)}

    out = {
        "metric": METRIC, "value": round(dec_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 codes, Q24 block scales, Q16 activations; no checkpoint)",
        "config": {"workload": "dense_14336x4096_q8", "t_decode": 1, "t_prefill": 512, "weight_copies": args.copies,
                   "act_limbs": LIMBS, "step_also_runs": ["qwen05b_ffn_24_layers", "olmoe_grouped_ffn"],
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(ach_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach_gbs / HBM_PEAK_GBS, 4), "traffic": tr_dec, "kernel": GEMV_KERNEL,
                     "launch_us": round(per_gemv_ms * 1e3, 3), "algorithmic_bytes": algo_bytes},
        "decode_batched": {
            f"{g}_per_launch": {
                "launches": (args.copies + g - 1) // g, "us_per_matrix": round(ms * 1e3 / args.copies, 3),
                "weight_gbs": round(W_BYTES * args.copies / (ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(W_BYTES * args.copies / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            for g, ms in batched.items()} | {
            "note": "the same T=1 projections in launches of up to 2 (gate and up of a layer) or 16 matrices "
                    "sharing x (int_gemm_q8_multi); `value` times one launch per matrix"},
        "prefill_t512": {
            "ms": round(pre_med, 4), "useful_tops": round(pre_tops, 2),
            "logical_tops": round(pre_tops / LIMBS, 2),
            "roofline": {"bound": "mfma", "achieved": round(pre_tops, 2), "peak": I8_PEAK_TOPS, "unit": "TOPS",
                         "frac": round(pre_tops / I8_PEAK_TOPS, 4), "traffic": tr_pre, "kernel": GEMM_KERNEL,
                         "note": "useful i8 ops = 3 limbs x 2*T*N*K; the event span covers the limb split and the MFMA kernel"},
            "valu_ceiling": valu_ceiling(pre_med),
        },
        "measured_ceilings": {"hbm_copy_gbs_read_plus_write": round(copy_gbs, 1),
                              "note": "a 256 MiB device copy timed in this run (bytes read + written per second)"},
        "qwen05b_ffn_24_layers": hbm_part("qwen", qw),
        "olmoe_grouped_ffn": hbm_part("olmoe", om),
        "parity": parity,
    }
    if base is not None:
        out["cpu_baseline"] = base
    print(json.dumps(out))
    return 0


def oracle_digest(a) -> str:
    """SHA-256 of an array's little-endian bytes (the oracle's digest layout)."""
    import numpy as np
    a = np.ascontiguousarray(a)
    return hashlib.sha256(a.astype(a.dtype.newbyteorder("<"), copy=False).tobytes()).hexdigest()


if __name__ == "__main__":
    sys.exit(main())
