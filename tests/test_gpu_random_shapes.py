"""GPU parity on seeded random shapes: projections, FFN layers and routed FFNs.

Each case draws its shape, limb count, schedule and scale range from one
seeded generator and compares the whole output with the oracle.  The draws
reach combinations the hand-picked shapes do not: every limb count on every
path, wide scales on the skinny and generic kernels, K splits of every count,
FFN layers on and off the fused path, routed FFNs with 1-23 experts.  One
fixed case, a one-limb projection whose skinny pass splits K over eight
workgroups, once wrote its (h, r) partials past a workspace sized one int64
per output; it runs first.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

SCH = ["default", "canonical", "reversed", "tiled_shuffled", "split_k", "tree_walk"]
LIMB = {1: (-128, 127), 2: (-32896, 32639), 3: (-8421504, 8355711), 4: (-2155905152, 2139062143)}
CASES = 400


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


@pytest.fixture(scope="module")
def ei():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import exact_integer_amd
    return exact_integer_amd


def _q8(ei, r, n, k, t, L, sched, wide):
    q = synth.q8_codes(r, n, k)
    if wide:
        s = r.integers(-(2**31), 2**31, size=(n, k // 32), dtype=np.int64).astype(np.int32)
    else:
        s = synth.q8_scales(r, n, k)
    lo, hi = LIMB[L]
    x = r.integers(lo, hi + 1, size=(t, k)).astype(np.int64)
    seed = int(r.integers(0, 2**32))
    print("q8", n, k, t, L, sched, "wide" if wide else "", flush=True)
    y = host(ei.gemm_q8(ei.pack_q8(dev(q), dev(s)), dev(x), L, sched, seed))
    assert (y == oracle.q8(q, s, x, threads=8)).all(), (n, k, t, L, sched, wide)


def test_one_limb_skinny_split_partials(ei):
    _q8(ei, np.random.default_rng(30), 45, 4224, 32, 1, "canonical", False)


def test_random_shapes(ei, lut):
    r = np.random.default_rng(20261203)
    lut_d = ei.silu_lut()

    def pick_t():
        c = r.integers(0, 3)
        return int(r.integers(1, 5)) if c == 0 else int(r.integers(5, 64)) if c == 1 else int(r.integers(64, 320))

    for _ in range(CASES):
        kind = str(r.choice(["q8", "q4", "ffn", "moe"], p=[0.45, 0.25, 0.15, 0.15]))
        if kind in ("q8", "q4"):
            t = pick_t()
            k = 32 * int(r.integers(1, 160))
            n = int(r.integers(1, max(2, min(3000, 3e8 // (k * t)))))
            sched = str(r.choice(SCH))
            if kind == "q8":
                _q8(ei, r, n, k, t, int(r.choice([1, 2, 3, 3, 3, 4])), sched, bool(r.random() < 0.2))
            else:
                L = int(r.choice([2, 3]))
                nib, sme, x = synth.q4_codes_packed(r, n, k), synth.q4_scale_bytes(r, n, k), synth.i32_acts(r, t, k)
                print("q4", n, k, t, L, sched, flush=True)
                y = host(ei.gemm_q4(ei.pack_q4(dev(nib), dev(sme)), dev(x), L, sched))
                assert (y == oracle.q4(nib, sme, x, threads=8)).all(), (n, k, t, L, sched)
        elif kind == "ffn":
            D, F, T = 32 * int(r.integers(1, 40)), 32 * int(r.integers(1, 160)), int(r.integers(1, 80))
            mats = [(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                    (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                    (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))]
            x = synth.q16_acts(r, T, D)
            print("ffn", D, F, T, flush=True)
            _, _, h, _, xn = oracle.ffn_layer(x, mats[0], mats[1], mats[2], lut, threads=8)
            wg, wu, wd = (ei.pack_q8(dev(c), dev(sc)) for c, sc in mats)
            lo, hi = LIMB[3]
            if h.min() < lo or h.max() > hi:   # the down projection's input leaves its 3-limb range
                with pytest.raises(ei.EIError):
                    ei.ffn_q8(wg, wu, wd, dev(x), lut_d)
            else:
                assert (host(ei.ffn_q8(wg, wu, wd, dev(x), lut_d)) == xn).all(), (D, F, T)
        else:
            E = int(r.integers(1, 24))
            topk = int(r.integers(1, min(E, 8) + 1))
            rows, D, F = int(r.integers(1, 200)), 32 * int(r.integers(1, 24)), 32 * int(r.integers(1, 24))
            mats = [[(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                     (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                     (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))] for _ in range(E)]
            x = synth.q16_acts(r, rows, D)
            route = r.integers(0, E, (rows, topk)).astype(np.int32)
            print("moe", E, topk, rows, D, F, flush=True)

            def stack(m):
                return (dev(np.stack([mm[m][0] for mm in mats])), dev(np.stack([mm[m][1] for mm in mats])))
            wg, wu, wd = (ei.pack_q8_stacked(*stack(m)) for m in range(3))
            y = host(ei.moe_ffn_q8(wg, wu, wd, dev(x), dev(route), lut_d))
            assert (y == oracle.moe_pairs(x, route, lambda e: mats[e], lut, threads=8)).all(), (E, topk, rows, D, F)


def test_random_shapes_other_entry_points(ei, lut):
    # the batched GEMV (1-16 matrices, 1-4 limbs), the routed projection
    # (ragged rows, repeated experts), FFN chains plain and pre-norm (1-5
    # layers, fused and unfused paths), the allocation-free projection and
    # projections large enough for the tiled kernels (narrow, wide and 4-bit)
    r = np.random.default_rng(20261204)
    lut_d = ei.silu_lut()
    lo3, hi3 = LIMB[3]
    for _ in range(120):
        kind = str(r.choice(["multi", "grouped", "chain", "prenorm", "noalloc", "tiled"]))
        if kind == "multi":
            L, t, k = int(r.choice([1, 2, 3, 4])), int(r.integers(1, 5)), 32 * int(r.integers(1, 200))
            mats = [(synth.q8_codes(r, n, k), synth.q8_scales(r, n, k))
                    for n in [int(r.integers(1, 3000)) for _ in range(int(r.integers(1, 17)))]]
            lo, hi = LIMB[L]
            x = r.integers(lo, hi + 1, size=(t, k)).astype(np.int64)
            print("multi", L, t, k, [q.shape[0] for q, _ in mats], flush=True)
            ys = ei.gemm_q8_multi([ei.pack_q8(dev(q), dev(s)) for q, s in mats], dev(x), L)
            for (q, s), y in zip(mats, ys):
                assert (host(y) == oracle.q8(q, s, x, threads=8)).all()
        elif kind == "grouped":
            E = int(r.integers(1, 40))
            topk, rows = int(r.integers(1, min(E, 8) + 1)), int(r.integers(1, 300))
            n = 32 * int(r.integers(1, 40)) if r.random() < 0.5 else int(r.integers(1, 1200))
            k = 32 * int(r.integers(1, 40))
            mats = [(synth.q8_codes(r, n, k), synth.q8_scales(r, n, k)) for _ in range(E)]
            x = synth.q16_acts(r, rows, k)
            route = r.integers(0, E, (rows, topk)).astype(np.int32)
            print("grouped", E, topk, rows, n, k, flush=True)
            w = ei.pack_q8_stacked(dev(np.stack([m[0] for m in mats])), dev(np.stack([m[1] for m in mats])))
            y = host(ei.gemm_q8_grouped(w, dev(x), dev(route)))
            for e in range(E):
                pr = [(i, s) for i in range(rows) for s in range(topk) if route[i, s] == e]
                if pr:
                    ye = oracle.q8(mats[e][0], mats[e][1], x[[i for i, _ in pr]], threads=8)
                    assert all((y[i * topk + s] == ye[j]).all() for j, (i, s) in enumerate(pr)), (E, e)
        elif kind in ("chain", "prenorm"):
            D, F, T, nl = 32 * int(r.integers(1, 33)), 32 * int(r.integers(1, 130)), int(r.integers(1, 80)), \
                int(r.integers(1, 6))
            layers = [[(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                       (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                       (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))] for _ in range(nl)]
            x = synth.q16_acts(r, T, D)
            gns = [np.rint(r.normal(1.0, 0.2, D) * 2**16).astype(np.int32) for _ in range(nl)]
            eps = int(r.integers(1, 2**20))
            print(kind, D, F, T, nl, flush=True)
            xi, in_range = x, True
            for li, m in enumerate(layers):
                if kind == "prenorm":   # the normalized input, the gated product and x + d
                    src, _, xn = oracle.ffn_layer_prenorm(xi, gns[li], eps, *m, lut, threads=8)
                    h = oracle.ffn_layer(src, *m, lut, threads=8)[2]
                else:
                    src = xi
                    _, _, h, _, xn = oracle.ffn_layer(xi, *m, lut, threads=8)
                # what the library splits into limbs: each layer's input (or its norm) and h
                in_range = in_range and lo3 <= src.min() and src.max() <= hi3 and lo3 <= h.min() and h.max() <= hi3
                xi = xn
            x_next = xi
            pk = [tuple(ei.pack_q8(dev(c), dev(s)) for c, s in m) for m in layers]
            run = (lambda: ei.ffn_q8_prenorm_chain(pk, [dev(g) for g in gns], eps, dev(x), lut_d)) \
                if kind == "prenorm" else (lambda: ei.ffn_q8_chain(pk, dev(x), lut_d))
            if in_range:
                assert (host(run()) == x_next).all(), (kind, D, F, T, nl)
            else:
                with pytest.raises(ei.EIError):
                    run()
        elif kind == "noalloc":
            t, k = int(r.integers(1, 320)), 32 * int(r.integers(1, 160))
            n = int(r.integers(1, max(2, min(4000, 3e8 // (k * t)))))
            q, s, x = synth.q8_codes(r, n, k), synth.q8_scales(r, n, k), synth.q16_acts(r, t, k)
            print("noalloc", n, k, t, flush=True)
            w = ei.pack_q8(dev(q), dev(s))
            if ei.workspace_bytes(w, t) > 32 << 20:
                with pytest.raises(ei.EIError):
                    ei.gemm_q8_noalloc(w, dev(x))
            else:
                assert (host(ei.gemm_q8_noalloc(w, dev(x))) == oracle.q8(q, s, x, threads=8)).all()
        else:
            fmt, t, k = str(r.choice(["q8", "q8", "q4"])), int(r.integers(64, 700)), 32 * int(r.integers(1, 24))
            need = (128 * 128 * 32) // ((t + 31) // 32 * 32)
            n = int(r.integers(min(max(1, need - 200), 5999), 6000))
            print("tiled", fmt, n, k, t, flush=True)
            if fmt == "q8":
                q = synth.q8_codes(r, n, k)
                s = (r.integers(-(2**31), 2**31, size=(n, k // 32), dtype=np.int64).astype(np.int32)
                     if r.random() < 0.3 else synth.q8_scales(r, n, k))
                x = synth.q16_acts(r, t, k)
                assert (host(ei.gemm_q8(ei.pack_q8(dev(q), dev(s)), dev(x), 3)) == oracle.q8(q, s, x, threads=8)).all()
            else:
                nib, sme, x = synth.q4_codes_packed(r, n, k), synth.q4_scale_bytes(r, n, k), synth.i32_acts(r, t, k)
                y = host(ei.gemm_q4(ei.pack_q4(dev(nib), dev(sme)), dev(x), 3))
                assert (y == oracle.q4(nib, sme, x, threads=8)).all()


def test_random_shapes_wide_scales_and_large_routes(ei, lut):
    # FFN layers, chains and routed FFNs with block scales past the narrow
    # bound (|S| up to 2^17: the per-limb gate/up and down forms), routed FFNs
    # with up to 319 experts (the radix grouping) and 2,048 rows, and 4-bit
    # and Q8 projections of up to 1,024 tokens; an h or input outside the
    # 3-limb range must be flagged
    r = np.random.default_rng(20261205)
    lut_d = ei.silu_lut()
    lo3, hi3 = LIMB[3]

    def scales(n, k, wide):
        if not wide:
            return synth.q8_scales(r, n, k)
        lim = int(r.choice([2**15, 2**16, 2**17]))
        return r.integers(-lim, lim + 1, size=(n, k // 32), dtype=np.int64).astype(np.int32)

    def mats_for(F, D, wide):
        return [(synth.q8_codes(r, F, D), scales(F, D, wide)), (synth.q8_codes(r, F, D), scales(F, D, wide)),
                (synth.q8_codes(r, D, F), scales(D, F, wide))]

    for _ in range(60):
        kind = str(r.choice(["chain", "moe", "big"]))
        if kind == "chain":
            D, F, T, nl = 32 * int(r.integers(1, 33)), 32 * int(r.integers(1, 130)), int(r.integers(1, 80)), \
                int(r.integers(1, 5))
            layers = [mats_for(F, D, bool(r.random() < 0.6)) for _ in range(nl)]
            x = synth.q16_acts(r, T, D)
            print("chain", D, F, T, nl, flush=True)
            xi, in_range = x, True
            for m in layers:
                _, _, h, _, xn = oracle.ffn_layer(xi, *m, lut, threads=8)
                in_range = in_range and lo3 <= xi.min() and xi.max() <= hi3 and lo3 <= h.min() and h.max() <= hi3
                xi = xn
            pk = [tuple(ei.pack_q8(dev(c), dev(s)) for c, s in m) for m in layers]
            if in_range:
                assert (host(ei.ffn_q8_chain(pk, dev(x), lut_d)) == xi).all(), (D, F, T, nl)
            else:
                with pytest.raises(ei.EIError):
                    ei.ffn_q8_chain(pk, dev(x), lut_d)
        elif kind == "moe":
            E = int(r.integers(1, 64)) if r.random() < 0.5 else int(r.integers(200, 320))
            topk = int(r.integers(1, min(E, 8) + 1))
            rows, D, F = int(r.integers(1, 2049)), 32 * int(r.integers(1, 12)), 32 * int(r.integers(1, 12))
            wide = bool(r.random() < 0.5)
            mats = [mats_for(F, D, wide) for _ in range(E)]
            x = synth.q16_acts(r, rows, D)
            route = r.integers(0, E, (rows, topk)).astype(np.int32)
            print("moe", E, topk, rows, D, F, wide, flush=True)
            in_range = True
            for e in range(E):
                idx = np.nonzero((route == e).any(axis=1))[0]
                if len(idx):
                    h = oracle.ffn_layer(x[idx], *mats[e], lut, threads=8)[2]
                    in_range = in_range and lo3 <= h.min() and h.max() <= hi3

            def stack(i):
                return (dev(np.stack([mm[i][0] for mm in mats])), dev(np.stack([mm[i][1] for mm in mats])))
            wg, wu, wd = (ei.pack_q8_stacked(*stack(i)) for i in range(3))
            if in_range:
                y = host(ei.moe_ffn_q8(wg, wu, wd, dev(x), dev(route), lut_d))
                assert (y == oracle.moe_pairs(x, route, lambda e: mats[e], lut, threads=8)).all(), (E, topk, rows)
            else:
                with pytest.raises(ei.EIError):
                    ei.moe_ffn_q8(wg, wu, wd, dev(x), dev(route), lut_d)
        else:
            t, k, n = int(r.integers(64, 1025)), 32 * int(r.integers(1, 16)), int(r.integers(1, 8000))
            print("big", n, k, t, flush=True)
            if r.random() < 0.5:
                q, s, x = synth.q8_codes(r, n, k), scales(n, k, bool(r.random() < 0.3)), synth.q16_acts(r, t, k)
                assert (host(ei.gemm_q8(ei.pack_q8(dev(q), dev(s)), dev(x), 3)) == oracle.q8(q, s, x, threads=8)).all()
            else:
                L = int(r.choice([2, 3]))
                nib, sme, x = synth.q4_codes_packed(r, n, k), synth.q4_scale_bytes(r, n, k), synth.i32_acts(r, t, k)
                y = host(ei.gemm_q4(ei.pack_q4(dev(nib), dev(sme)), dev(x), L))
                assert (y == oracle.q4(nib, sme, x, threads=8)).all(), (n, k, t, L)
