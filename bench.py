#!/usr/bin/env python3
"""Benchmark of the exact-integer block-quantized projection on one MI355X.

Metric: bit-exact int GEMM -- weight GB/s at T=1 and useful TOPS at T=512,
each as a fraction of its roofline, on a 14336x4096 Q8 matrix (a 7B-class
dense projection; synthetic seeded codes, Q24 scales and Q16 activations).

One step = one decode pass (a T=1 projection over each of `--copies` distinct
resident copies of the weights, so the 256 MB Infinity Cache cannot serve
them) followed by one T=512 prefill projection.  Both are recorded once as
HIP graphs and replayed; HIP events on the launch stream time every replay.
After timing, the outputs are checked bit-exactly against the CPU oracle
(full digest at T=1, sampled rows at T=512).

Prints ONE JSON line.  `value` is the decode weight bandwidth (GB/s); the
prefill rate, both roofline fractions, and the oracle timed on the host cores
(`cpu_baseline`) ride along in the same line.
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
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


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
        fk = [v for k, vs in fetch.items() if kern in k for v in vs]
        wk = [v for k, vs in write.items() if kern in k for v in vs]
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


def cpu_baseline(q, s, x1, x512, rows: int, decode_seconds: float = 8.0):
    """The CPU oracle, as it stands, on the host cores: T=1 passes over the whole
    matrix repeated for about `decode_seconds`, and one T=512 pass over the
    first `rows` rows.  Threads own disjoint output rows."""
    import oracle
    cores = min(os.cpu_count() or 1, 16)
    reps, t0 = 0, time.perf_counter()
    while True:
        y1 = oracle.q8(q, s, x1, threads=cores)
        reps += 1
        if time.perf_counter() - t0 >= decode_seconds:
            break
    t_dec = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    oracle.q8(q[:rows], s[:rows], x512, threads=cores)
    t_pre = time.perf_counter() - t0
    useful = LIMBS * 2.0 * 512 * rows * K
    return {
        "value": W_BYTES / t_dec / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"T=1: all {N} rows x {reps} passes ({reps * t_dec:.1f} s); "
                  f"T=512: rows 0..{rows - 1} of {N}, one pass ({t_pre:.1f} s)",
        "t1_ms": t_dec * 1e3, "t512_useful_tops": useful / t_pre / 1e12,
        "t512_logical_tops": useful / LIMBS / t_pre / 1e12, "t512_sample_s": t_pre,
    }, y1


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


def _time_graph(torch, fn, steps: int, warmup: int):
    """Record fn once as a HIP graph, replay it warmup + steps times; median ms
    per replay from HIP events on the capturing stream."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
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
    ms = sorted(a.elapsed_time(b) for a, b in ev)
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

    def step_mfma():
        for _, n, k, t, nd, sd, w, x, yt, ym, ws, wt in cases:
            ei.gemm_q4(w, x, out=ym, workspace=ws, status=status)

    ms_t, wall_t = _time_graph(torch, step_table, args.steps, args.warmup)
    ms_m, _ = _time_graph(torch, step_mfma, args.steps, args.warmup)
    ok = int(status.item()) == 0 and all(ei.digest(yt) == gold[name] and ei.digest(ym) == gold[name]
                                         for name, n, k, t, nd, sd, w, x, yt, ym, ws, wt in cases)
    logical = sum(2.0 * t * n * k for _, n, k, t, *rest in cases)
    tops = logical / (ms_t * 1e-3) / 1e12
    alu_peak = 78.6   # int32 VALU lane-ops/s: 256 CUs x 4 SIMDs x 32 lanes x 2 issue x 2.4 GHz (fp32 157.3 TFLOP/s / 2)
    print(json.dumps({
        "metric": "4-bit projection by table reads: logical int TOPS", "value": round(tops, 3), "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_t, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32 x 4-bit by table reads",
        "data": "synthetic (seeded 4-bit codes and m*2^e scale bytes, int32 activations)",
        "config": {"workload": "q4_d512_table_read", "shapes": list(synth.Q4_SHAPES.values()), "tokens": [1, 64],
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "alu", "achieved": round(tops, 3), "peak": alu_peak, "unit": "TOP/s",
                     "frac": round(tops / alu_peak, 4), "traffic": None, "step_ms": round(ms_t, 4)},
        "mfma_path_step_ms": round(ms_m, 4),
        "parity": {"table_read_and_mfma_digests_equal_oracle": ok}}))
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
    import oracle
    E, H, I, T, TOPK = synth.OLMOE_E, synth.OLMOE_H, synth.OLMOE_I, synth.OLMOE_T, synth.OLMOE_TOPK
    mats = [synth.olmoe_expert(e) for e in range(E)]

    def stack(m, k):
        return torch.from_numpy(np.ascontiguousarray(np.stack([mm[m][k] for mm in mats]))).to(dev)
    wg, wu, wd = (ei.pack_q8_stacked(stack(m, 0), stack(m, 1)) for m in range(3))
    rc, rs = synth.olmoe_router()
    wr = ei.pack_q8(torch.from_numpy(rc).to(dev), torch.from_numpy(rs).to(dev))
    x = synth.olmoe_x()
    xd = torch.from_numpy(x).to(dev)
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
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))["olmoe_router"]
    route_ok = int(status.item()) == 0 and ei.digest(route) == gold["route"]
    rs_ = np.random.default_rng(6)
    pairs = [(int(t), int(k)) for t, k in zip(rs_.integers(0, T, 6), rs_.integers(0, TOPK, 6))]
    ref = oracle.moe_pairs(x, route.cpu().numpy(), lambda e: mats[e], oracle.silu_lut(), pairs=pairs,
                           threads=min(os.cpu_count() or 1, 16))
    got = out.cpu().numpy()
    ok = route_ok and all((got[t * TOPK + k] == r).all() for (t, k), r in zip(pairs, ref))
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
        "parity": {"route_digest_equals_oracle": route_ok, "sampled_pairs_equal_oracle": ok,
                   "pairs_checked": len(pairs)}}))
    return 0 if ok else 1


def bench_olmoe(args, torch, np, ei, synth, dev) -> int:
    """The OLMoE-shaped routed FFN: 64 experts (gate/up 1024x2048, down
    2048x1024, Q8), 512 tokens, top-8: grouped gate and up projections, the
    SiLU-gated product, grouped down projection.  HBM-bound: every expert's
    weights are read once per step."""
    import oracle
    E, H, I, T, TOPK = synth.OLMOE_E, synth.OLMOE_H, synth.OLMOE_I, synth.OLMOE_T, synth.OLMOE_TOPK
    mats = [synth.olmoe_expert(e) for e in range(E)]

    def stack(m, k):
        return torch.from_numpy(np.ascontiguousarray(np.stack([mm[m][k] for mm in mats]))).to(dev)
    wg, wu, wd = (ei.pack_q8_stacked(stack(m, 0), stack(m, 1)) for m in range(3))
    x, route = synth.olmoe_x(), synth.olmoe_route()
    xd, rd = torch.from_numpy(x).to(dev), torch.from_numpy(route).to(dev)
    P = T * TOPK
    out = torch.empty((P, H), dtype=torch.int64, device=dev)
    ws = torch.empty(ei.moe_ffn_workspace_bytes(wg, wd, T, TOPK), dtype=torch.uint8, device=dev)
    lut = ei.silu_lut(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        ei.moe_ffn_q8(wg, wu, wd, xd, rd, lut, out=out, workspace=ws, status=status)

    ms, wall_ms = _time_graph(torch, step, args.steps, args.warmup)
    if int(status.item()) != 0:
        print(f"bench.py: device status {int(status.item())}", file=sys.stderr)
        return 1
    rs = np.random.default_rng(5)
    pairs = [(int(t), int(k)) for t, k in zip(rs.integers(0, T, 6), rs.integers(0, TOPK, 6))]
    ref = oracle.moe_pairs(x, route, lambda e: mats[e], oracle.silu_lut(), pairs=pairs,
                           threads=min(os.cpu_count() or 1, 16))
    got = out.cpu().numpy()
    ok = all((got[t * TOPK + k] == r).all() for (t, k), r in zip(pairs, ref))
    wbytes = 3 * E * I * H * (1 + 4 / 32)
    useful = LIMBS * 2.0 * P * 3 * I * H
    gbs = wbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "routed expert FFN: weight GB/s", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 experts, Q16 activations, uniform top-8 routing)",
        "config": {"workload": "olmoe_grouped_ffn", "experts": E, "hidden": H, "intermediate": I, "tokens": T,
                   "top_k": TOPK, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "step_ms": round(ms, 4),
                     "weight_bytes": int(wbytes)},
        "useful_tops": round(useful / (ms * 1e-3) / 1e12, 2),
        "parity": {"sampled_pairs_equal_oracle": ok, "pairs_checked": len(pairs)}}))
    return 0 if ok else 1


def bench_qwen_ffn(args, torch, np, ei, synth, dev, prenorm: bool = False) -> int:
    """The Qwen2.5-0.5B-shaped FFN chain: 24 layers of gate and up (4864x896)
    and down (896x4864) Q8 projections at T=30 with the SiLU-gated product and
    the residual add, fresh weights per layer (353 MB, read once per step)."""
    import json as _json
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

    gold = _json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))[
        "qwen05b_ffn_prenorm" if prenorm else "qwen05b_ffn"]["layers"]
    layer_calls_ms = None
    if prenorm:
        layer_calls_ms, _ = _time_graph(torch, step_layers, args.steps, args.warmup)
        ok_layers = int(status.item()) == 0 and ei.digest(final) == gold[-1]["x_next"]
        final.zero_()
    ms, wall_ms = _time_graph(torch, step, args.steps, args.warmup)
    ok = int(status.item()) == 0 and ei.digest(final) == gold[-1]["x_next"]
    if prenorm:
        ok = ok and ok_layers
    wbytes = synth.QWEN_LAYERS * 3 * F * D * (1 + 4 / 32)
    gbs = wbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": ("24-layer pre-norm Q8 FFN chain" if prenorm else "24-layer Q8 FFN chain") + ": weight GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 layers, Q16 activations)",
        "config": {"workload": "qwen05b_ffn_24_layers" + ("_prenorm" if prenorm else ""), "tokens": T,
                   "hidden": D, "intermediate": F,
                   "layers": synth.QWEN_LAYERS, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "step_ms": round(ms, 4),
                     "weight_bytes": int(wbytes)},
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
    ap.add_argument("--cpu-rows", type=int, default=N, help="rows of the T=512 oracle sample")
    ap.add_argument("--profile", action="store_true", help="short run for rocprofv3 (no baseline, few steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 256 MiB, 5 times (the reference for HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output directories -> profiles/traffic.json (no GPU needed)")
    ap.add_argument("--workload", choices=("dense", "olmoe", "olmoe_router", "qwen_ffn", "qwen_ffn_prenorm", "wide",
                                           "q4_table"),
                    default="dense",
                    help="dense: the 14336x4096 decode + prefill step (default); olmoe / qwen_ffn: the routed "
                         "expert FFN or the 24-layer FFN chain, timed the same way; olmoe_router: the routed "
                         "FFN behind the integer router; qwen_ffn_prenorm: the chain with an integer RMSNorm "
                         "in front of every layer; wide: the 12-trit wide-code GEMM (896x896, 4096 rows); q4_table: the "
                         "4-bit projections by table reads against the MFMA path")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the projection would shard by rows across GPUs, see the design notes)", file=sys.stderr)
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
    if args.workload == "wide":
        return bench_wide(args, torch, np, ei, synth, dev)
    if args.workload == "olmoe_router":
        return bench_olmoe_router(args, torch, np, ei, synth, dev)
    if args.workload in ("qwen_ffn", "qwen_ffn_prenorm"):
        return bench_qwen_ffn(args, torch, np, ei, synth, dev, prenorm=args.workload == "qwen_ffn_prenorm")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

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
    torch.cuda.synchronize()

    def decode():
        for c, w in enumerate(copies):
            ei.gemm_q8(w, x1d, LIMBS, out=y1[c], status=status)

    def prefill():
        ei.gemm_q8(w0, x512d, LIMBS, out=y512, workspace=ws, status=status)

    # eager run first (also the graph's warm-up)
    decode(); prefill()
    torch.cuda.synchronize()
    g_dec, g_pre = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dec):
        decode()
    with torch.cuda.graph(g_pre):
        prefill()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for _ in range(args.warmup):
        g_dec.replay(); g_pre.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(); g_dec.replay(); e1.record(); g_pre.replay(); e2.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = sorted(a.elapsed_time(b) for a, b, _ in ev)
    pre_ms = sorted(b.elapsed_time(c) for _, b, c in ev)
    dec_med, pre_med = dec_ms[len(dec_ms) // 2], pre_ms[len(pre_ms) // 2]
    if int(status.item()) != 0:
        print(f"bench.py: device status {int(status.item())}", file=sys.stderr)
        return 1

    # ---- the same decode pass as batched launches (int_gemm_q8_multi, up to
    # 16 matrices sharing x per launch): reported beside `value`, not in it
    yb = [torch.empty((1, N), dtype=torch.int64, device=dev) for _ in copies]
    batched = {}
    for group in (2, 16):   # 2: gate and up of one FFN layer; 16: the largest batch
        def decode_batched():
            for i in range(0, len(copies), group):
                ei.gemm_q8_multi(copies[i:i + group], x1d, LIMBS, outs=yb[i:i + group], status=status)

        batched[group], _ = _time_graph(torch, decode_batched, args.steps, args.warmup)
        if {ei.digest(y) for y in yb} != {json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))[
                "dense_14336x4096"]["t1_y"]}:
            print(json.dumps({"error": "parity failure (batched decode)", "group": group}))
            return 1
        yb = [torch.empty((1, N), dtype=torch.int64, device=dev) for _ in copies]

    # ---- parity of what was timed
    import oracle
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "oracle_digests.json")))["dense_14336x4096"]["t1_y"]
    dig = {ei.digest(y1[c]) for c in range(args.copies)}
    rows = np.concatenate([np.random.default_rng(11).choice(N, 24, replace=False), [0, N - 1]])
    ref = oracle.q8(q[rows], s[rows], x512, threads=min(os.cpu_count() or 1, 16))
    ok512 = bool((y512.cpu().numpy()[:, rows] == ref).all())
    parity = {"t1_digest_equals_oracle": dig == {gold}, "t512_sampled_rows_equal_oracle": ok512,
              "t512_rows_checked": int(rows.size), "t1_batched_digests_equal_oracle": True}
    if not (parity["t1_digest_equals_oracle"] and ok512):
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
    out = {
        "metric": METRIC, "value": round(dec_gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32, int64 accumulate",
        "data": "synthetic (seeded Q8 codes, Q24 block scales, Q16 activations; no checkpoint)",
        "config": {"workload": "dense_14336x4096_q8", "t_decode": 1, "t_prefill": 512, "weight_copies": args.copies,
                   "act_limbs": LIMBS, "parallelism": "single-gpu"},
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
        },
        "parity": parity,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"], _ = cpu_baseline(q, s, x1, x512, args.cpu_rows)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
