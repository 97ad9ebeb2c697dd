"""GPU parity: the HIP path against the CPU oracle, bit-exact (integer work).

Every comparison is element by element (and by SHA-256 of the output bytes)
on the same seeded inputs.  Small ragged shapes span several 32x32 tiles and
a ragged tail in rows and tokens; the workloads run at their full sizes.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "oracle_digests.json")))
SCHEDS = ["default", "canonical", "reversed", "tiled_shuffled", "split_k", "tree_walk"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ei():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import exact_integer_amd
    return exact_integer_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# -------------------------------------------------------------- building blocks

def test_limb_split_matches_oracle(ei):
    r = np.random.default_rng(1)
    x = np.concatenate([r.integers(-(2**22), 2**22 + 1, 100000),
                        [8355711, -8421504, 0, 1, -1, 127, 128, -128, -129]]).astype(np.int64)
    for L in (1, 2, 3, 4):
        say("limb_split L", L)
        d, st = ei.limb_split(dev(x), L)
        do, ok = oracle.limb_split(x, L)
        assert (host(d) == do).all()
        assert (int(st.item()) == 0) == ok


def test_silu_lut_matches_oracle(ei):
    say("silu lut")
    assert (host(ei.silu_lut()) == oracle.silu_lut()).all()


def test_silu_mul_matches_oracle(ei, lut):
    r = np.random.default_rng(2)
    g = np.concatenate([r.integers(-(2**21), 2**21, 50000), r.integers(-(2**40), 2**40, 1000),
                        [-(2**63), 2**63 - 1, -16, -17, 15, 16, 31, 32, 33]]).astype(np.int64)
    u = r.integers(-(2**40), 2**40, g.size).astype(np.int64)
    say("silu_mul")
    h = ei.silu_mul(dev(g), dev(u), dev(lut))
    assert (host(h) == oracle.silu_mul(g, u, lut)).all()


# --------------------------------------------------------------- projections

SMALL = [(37, 96, 1), (37, 96, 2), (100, 320, 3), (33, 64, 4), (100, 320, 5), (130, 1024, 33),
         (64, 288, 64), (7, 32, 40), (257, 2048, 70)]


@pytest.mark.parametrize("shape", SMALL)
def test_q8_small_all_schedules(ei, shape):
    N, K, T = shape
    r = np.random.default_rng(N * 7 + K + T)
    q, s, x = synth.q8_codes(r, N, K), synth.q8_scales(r, N, K), synth.q16_acts(r, T, K)
    ref = oracle.q8(q, s, x)
    w = ei.pack_q8(dev(q), dev(s))
    xd = dev(x)
    for sched in SCHEDS:
        say("q8", shape, sched)
        y = host(ei.gemm_q8(w, xd, 3, sched, seed=0xE1 + N))
        assert (y == ref).all(), sched


@pytest.mark.parametrize("shape", [(37, 96, 1), (70, 160, 3), (40, 128, 9)])
def test_q8_extremes_bit_exact(ei, shape):
    # codes at -128/127, scales at the int32 ends, activations at the 3-limb
    # range ends: the largest magnitudes the formats allow.
    N, K, T = shape
    r = np.random.default_rng(5)
    q = r.choice(np.array([-128, 127, -127, 1, 0], np.int8), size=(N, K))
    s = r.choice(np.array([-(2**31), 2**31 - 1, 1, -1, 0], np.int64), size=(N, K // 32)).astype(np.int32)
    x = r.choice(np.array([8355711, -8421504, 0, 1, -1, 2**22], np.int64), size=(T, K))
    ref = oracle.q8(q, s, x)
    w = ei.pack_q8(dev(q), dev(s))
    for sched in SCHEDS:
        say("q8 extremes", shape, sched)
        assert (host(ei.gemm_q8(w, dev(x), 3, sched)) == ref).all(), sched


@pytest.mark.parametrize("sign", [-1, 1])
def test_q8_max_k_extreme_accumulators(ei, sign):
    # K = 262144 (8192 blocks, the largest the library accepts) with every
    # term at its extreme: codes -128, scales -2^31, activations at one end of
    # the 3-limb range.  With sign -1 every limb's sum is exactly -2^63, the
    # int64 end; every path (GEMV, skinny with its splits, tiled) and, at T=5,
    # every schedule must still give the oracle's bits.
    N, K = 40, 262144
    q = np.full((N, K), -128, np.int8)
    s = np.full((N, K // 32), -(2**31), np.int32)
    w = ei.pack_q8(dev(q), dev(s))
    xv = -8421504 if sign < 0 else 8355711
    for T in (1, 5, 64):
        x = np.full((T, K), xv, np.int64)
        ref = oracle.q8(q, s, x, threads=8)
        scheds = SCHEDS if T == 5 else ["default"]
        for sched in scheds:
            say("q8 max K", sign, T, sched)
            assert (host(ei.gemm_q8(w, dev(x), 3, sched)) == ref).all(), (T, sched)


def test_q8_four_limbs_wide_activations(ei):
    r = np.random.default_rng(6)
    N, K = 64, 256
    q, s = synth.q8_codes(r, N, K), synth.q8_scales(r, N, K)
    for T in (2, 40):
        x = r.integers(-(2**30), 2**30, size=(T, K)).astype(np.int64)
        say("q8 L=4", T)
        assert (host(ei.gemm_q8(ei.pack_q8(dev(q), dev(s)), dev(x), 4)) == oracle.q8(q, s, x)).all()


def _limb_bounds(L):
    # balanced base-256: L digits in [-128, 127] reach [-128 (256^L - 1)/255, 127 (256^L - 1)/255]
    m = (256 ** L - 1) // 255
    return -128 * m, 127 * m


@pytest.mark.parametrize("shape", [(40, 8192, 30, 3), (70, 4096, 17, 2), (33, 2048, 64, 4), (64, 1024, 5, 1),
                                   (96, 2560, 48, 3), (7, 160, 63, 3)])
def test_q8_skinny_split_k(ei, shape):
    # few row tiles and a long K: the workgroups split the blocks and write
    # per-limb partials that a second kernel combines; limbs 1 to 4, activations
    # spanning each limb count's whole range
    N, K, T, L = shape
    r = np.random.default_rng(N + K + T + L)
    q, s = synth.q8_codes(r, N, K), synth.q8_scales(r, N, K)
    lo, hi = _limb_bounds(L)
    x = r.integers(lo, hi + 1, size=(T, K)).astype(np.int64)
    x[0, :4] = [lo, hi, 0, -1]
    w = ei.pack_q8(dev(q), dev(s))
    say("q8 skinny", shape, "workspace", ei.workspace_bytes(w, T, L))
    assert (host(ei.gemm_q8(w, dev(x), L)) == oracle.q8(q, s, x)).all()


def test_q4_skinny_split_k(ei):
    N, K, T = 50, 4096, 12
    r = np.random.default_rng(12)
    nib, sme, x = synth.q4_codes_packed(r, N, K), synth.q4_scale_bytes(r, N, K), synth.i32_acts(r, T, K)
    w = ei.pack_q4(dev(nib), dev(sme))
    say("q4 skinny", (N, K, T))
    assert (host(ei.gemm_q4(w, dev(x), 3)) == oracle.q4(nib, sme, x)).all()


def test_q8_limb_range_is_flagged(ei):
    r = np.random.default_rng(7)
    q, s = synth.q8_codes(r, 32, 64), synth.q8_scales(r, 32, 64)
    w = ei.pack_q8(dev(q), dev(s))
    for T in (1, 8):
        x = np.zeros((T, 64), np.int64)
        x[0, 5] = 8355712      # one past the 3-limb range
        say("range flag", T)
        with pytest.raises(ei.EIError):
            ei.gemm_q8(w, dev(x), 3)
        ei.gemm_q8(w, dev(x), 4)   # four limbs hold it


def test_q8_multi_limb_range_is_flagged(ei):
    # the batched GEMV splits x into limbs once per row group of every
    # matrix: an activation past the 3-limb range is flagged there too
    r = np.random.default_rng(8)
    mats = [(synth.q8_codes(r, n, 64), synth.q8_scales(r, n, 64)) for n in (32, 40)]
    ws = [ei.pack_q8(dev(q), dev(s)) for q, s in mats]
    for T in (1, 4):
        x = np.zeros((T, 64), np.int64)
        x[T - 1, 63] = -8421505      # one past the 3-limb range, below
        say("multi range flag", T)
        with pytest.raises(ei.EIError):
            ei.gemm_q8_multi(ws, dev(x), 3)
        ys = [host(y) for y in ei.gemm_q8_multi(ws, dev(x), 4)]
        for (q, s), y in zip(mats, ys):
            assert (y == oracle.q8(q, s, x)).all()


@pytest.mark.parametrize("shape", [(37, 96, 1), (100, 320, 4), (64, 288, 64), (33, 512, 7)])
def test_q4_small_all_schedules(ei, shape):
    N, K, T = shape
    r = np.random.default_rng(N + 3 * K + T)
    nib, sme, x = synth.q4_codes_packed(r, N, K), synth.q4_scale_bytes(r, N, K), synth.i32_acts(r, T, K)
    ref = oracle.q4(nib, sme, x)
    w = ei.pack_q4(dev(nib), dev(sme))
    for sched in SCHEDS:
        say("q4", shape, sched)
        assert (host(ei.gemm_q4(w, dev(x), 3, sched)) == ref).all(), sched


@pytest.mark.parametrize("shape", [(37, 96, 1), (100, 320, 4), (64, 288, 64), (33, 512, 7), (50, 4096, 12),
                                   (300, 1024, 100)])
def test_q4_two_limbs_all_schedules(ei, shape):
    # the two-limb form: x - 128 split into two digits, R_i added back as
    # each row is finished (GEMV, skinny with and without K splits, the
    # generic MFMA kernel and every schedule's reducer); activations at both
    # ends of [-2^15, 2^15)
    N, K, T = shape
    r = np.random.default_rng(N + 5 * K + T)
    nib, sme, x = synth.q4_codes_packed(r, N, K), synth.q4_scale_bytes(r, N, K), synth.i32_acts(r, T, K)
    x[0, :4] = [-(2**15), 2**15 - 1, 128, 127]
    x[T - 1, K - 2:] = [2**15 - 1, -(2**15)]
    ref = oracle.q4(nib, sme, x)
    w = ei.pack_q4(dev(nib), dev(sme))
    for sched in SCHEDS:
        say("q4 two limbs", shape, sched)
        assert (host(ei.gemm_q4(w, dev(x), 2, sched)) == ref).all(), sched


@pytest.mark.parametrize("shape", [(1, 32, 1), (1, 32, 5), (1, 32, 64), (3, 32, 100), (1, 64, 4)])
def test_single_row_single_block(ei, shape):
    # the degenerate sizes: one output row (31 padded rows in its tile), one or
    # two blocks along K (most waves, K splits and split-K partials empty),
    # every schedule, Q8 at three limbs and the two-limb 4-bit form
    N, K, T = shape
    r = np.random.default_rng(N * 1000 + K + T)
    q, s, x = synth.q8_codes(r, N, K), synth.q8_scales(r, N, K), synth.q16_acts(r, T, K)
    nib, sme, x4 = synth.q4_codes_packed(r, N, K), synth.q4_scale_bytes(r, N, K), synth.i32_acts(r, T, K)
    w8, w4 = ei.pack_q8(dev(q), dev(s)), ei.pack_q4(dev(nib), dev(sme))
    ref8, ref4 = oracle.q8(q, s, x), oracle.q4(nib, sme, x4)
    for sched in SCHEDS:
        say("single row/block", shape, sched)
        assert (host(ei.gemm_q8(w8, dev(x), 3, sched)) == ref8).all(), sched
        assert (host(ei.gemm_q4(w4, dev(x4), 2, sched)) == ref4).all(), sched


def test_q4_row_offsets_in_the_image(ei):
    # the packed 4-bit image carries R_i = 128 * row weight sum after the scales
    N, K = 70, 160
    r = np.random.default_rng(70)
    nib, sme = synth.q4_codes_packed(r, N, K), synth.q4_scale_bytes(r, N, K)
    w = ei.pack_q4(dev(nib), dev(sme))
    n_pad = (N + 31) // 32 * 32
    at = 256 + n_pad * K + n_pad * (K // 32) * 4
    roff = host(w.buf[at:at + 8 * n_pad].view(torch.int64))
    assert (roff[:N] == oracle.q4_row_offsets(nib, sme)).all()
    assert (roff[N:] == 0).all()


def test_q4_two_limb_range_is_flagged(ei):
    r = np.random.default_rng(9)
    nib, sme = synth.q4_codes_packed(r, 32, 64), synth.q4_scale_bytes(r, 32, 64)
    w = ei.pack_q4(dev(nib), dev(sme))
    for T in (1, 8):
        for v in (2**15, -(2**15) - 1):   # one past [-2^15, 2^15) either side
            x = np.zeros((T, 64), np.int32)
            x[T - 1, 7] = v
            say("q4 two-limb range flag", T, v)
            with pytest.raises(ei.EIError):
                ei.gemm_q4(w, dev(x), 2)
            assert (host(ei.gemm_q4(w, dev(x), 3)) == oracle.q4(nib, sme, x)).all()


# ------------------------------------------------------------------ workloads

def test_q8_896x896_gemv(ei):
    # the single 896x896 GEMV under every schedule ([Handshake] Schedule gate)
    (q, s), x = synth.q8_896_inputs()
    w = ei.pack_q8(dev(q), dev(s))
    assert GOLDEN["q8_896x896"]["y"] == oracle.digest(oracle.q8(q, s, x))
    xd = dev(x)
    for sched in SCHEDS:
        say("q8 896x896 T=1", sched)
        assert ei.digest(ei.gemm_q8(w, xd, 3, sched)) == GOLDEN["q8_896x896"]["y"], sched


def test_qkv_schedule_gate(ei):
    mats, x = synth.qkv_inputs()
    xd = dev(x)
    for name, (c, sc) in mats.items():
        w = ei.pack_q8(dev(c), dev(sc))
        digests = set()
        for sched in SCHEDS:
            say("qkv gate", name, sched)
            digests.add(ei.digest(ei.gemm_q8(w, xd, 3, sched, seed=0xE1)))
        assert digests == {GOLDEN["qkv_gate"][name]}, name


def test_q4_d512(ei):
    for name, (n, k) in synth.Q4_SHAPES.items():
        nib, sme = synth.q4_d512_matrix(name)
        w = ei.pack_q4(dev(nib), dev(sme))
        for t in (1, 64):
            xd = dev(synth.q4_d512_x(k, t))
            for limbs in (2, 3):
                for sched in SCHEDS:
                    say("q4 d512", name, t, limbs, sched)
                    y = ei.gemm_q4(w, xd, limbs, sched)
                    assert ei.digest(y) == GOLDEN["q4_d512"][f"{name}_t{t}"], (limbs, sched)


def test_qwen_ffn_24_layers(ei):
    lut = ei.silu_lut()
    x = dev(synth.qwen_ffn_x0())
    for layer in range(synth.QWEN_LAYERS):
        (gc, gs), (uc, us), (dc, ds) = synth.qwen_ffn_layer(layer)
        wg, wu, wd = ei.pack_q8(dev(gc), dev(gs)), ei.pack_q8(dev(uc), dev(us)), ei.pack_q8(dev(dc), dev(ds))
        say("ffn layer", layer)
        g = ei.gemm_q8(wg, x)
        u = ei.gemm_q8(wu, x)
        h = ei.silu_mul(g, u, lut)
        d = ei.gemm_q8(wd, h)
        x = x + d
        exp = GOLDEN["qwen05b_ffn"]["layers"][layer]
        assert ei.digest(d) == exp["d"], layer
        assert ei.digest(x) == exp["x_next"], layer


def test_qwen_ffn_schedule_gate(ei):
    # every projection of the 24 Qwen-shaped layers (gate, up 4864x896; down
    # 896x4864; T=30) under the five schedules: g, u, h and d digests equal
    # the oracle's, layer by layer ([Handshake] Schedule gate)
    lut = ei.silu_lut()
    x = dev(synth.qwen_ffn_x0())
    for layer in range(synth.QWEN_LAYERS):
        (gc, gs), (uc, us), (dc, ds) = synth.qwen_ffn_layer(layer)
        wg, wu, wd = ei.pack_q8(dev(gc), dev(gs)), ei.pack_q8(dev(uc), dev(us)), ei.pack_q8(dev(dc), dev(ds))
        exp = GOLDEN["qwen05b_ffn"]["layers"][layer]
        for sched in SCHEDS:
            say("qwen schedule gate, layer", layer, sched)
            g = ei.gemm_q8(wg, x, 3, sched)
            u = ei.gemm_q8(wu, x, 3, sched)
            h = ei.silu_mul(g, u, lut)
            d = ei.gemm_q8(wd, h, 3, sched)
            assert (ei.digest(g), ei.digest(u), ei.digest(h), ei.digest(d)) == \
                (exp["g"], exp["u"], exp["h"], exp["d"]), (layer, sched)
        x = x + d
        assert ei.digest(x) == exp["x_next"], layer


@pytest.mark.parametrize("shape", [(96, 64, 1), (96, 64, 3), (160, 96, 30), (128, 64, 40), (64, 4096, 30),
                                   (4096, 64, 30), (96, 160, 70), (32, 320, 5), (4096, 1024, 30), (4096, 1056, 30),
                                   (1056, 64, 17), (5120, 96, 16), (800, 64, 40), (5152, 64, 30)])
def test_ffn_q8_matches_the_separate_steps(ei, lut, shape):
    # one layer through int_ffn_q8 against the oracle's gate, up, SiLU
    # product, down projection and residual: the fused gate/up pass (5..63
    # tokens with one workgroup split), the GEMV path, the tiled path, the
    # unfused path, and split-K partials (with the residual) on the down
    # projection; K = 1024 is the largest the fused pass stages in LDS
    # (152 KB with its exchange buffers), K = 1056 the smallest it does not.
    # The one-launch down projection on 16 x 16 tiles takes 16..160 blocks:
    # 33 (ragged over its 16 waves), 160 (the most), 25 (a token half of 8),
    # and 161 blocks falls back to split-K
    F, D, T = shape
    r = np.random.default_rng(F + D + T)
    mats = [(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)), (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
            (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))]
    x = synth.q16_acts(r, T, D)
    wg, wu, wd = (ei.pack_q8(dev(c), dev(sc)) for c, sc in mats)
    say("ffn", shape, "workspace", ei.ffn_workspace_bytes(wg, wd, T))
    y = host(ei.ffn_q8(wg, wu, wd, dev(x), dev(lut)))
    *_, xn = oracle.ffn_layer(x, mats[0], mats[1], mats[2], lut)
    assert (y == xn).all()


@pytest.mark.parametrize("shape", [(96, 64, 1), (160, 96, 30), (128, 64, 40), (64, 4096, 30), (4096, 64, 30),
                                   (96, 160, 70)])
def test_ffn_q8_prenorm_matches_oracle(ei, lut, shape):
    # the RMSNorm in front of the layer: fused into the gate/up limb tiles (5..63
    # tokens), or as its own pass ahead of the GEMV, tiled and unfused paths
    F, D, T = shape
    r = np.random.default_rng(F * 3 + D + T)
    mats = [(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)), (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
            (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))]
    x = synth.q16_acts(r, T, D)
    gn = np.rint(r.normal(1.0, 0.2, D) * 2**16).astype(np.int32)
    eps = int(r.integers(1, 2**20))
    wg, wu, wd = (ei.pack_q8(dev(c), dev(sc)) for c, sc in mats)
    say("ffn prenorm", shape)
    y = host(ei.ffn_q8_prenorm(wg, wu, wd, dev(gn), eps, dev(x), dev(lut)))
    _, _, xn = oracle.ffn_layer_prenorm(x, gn, eps, mats[0], mats[1], mats[2], lut)
    assert (y == xn).all()


@pytest.mark.parametrize("shape", [(96, 64, 3), (160, 96, 30), (64, 4096, 30), (4096, 64, 30), (4096, 64, 50),
                                   (2048, 96, 33), (96, 160, 70)])
def test_ffn_q8_chain_matches_oracle(ei, lut, shape):
    # three layers in one call: the fused path hands limb tiles from each
    # layer's combiner to the next (K-split down projections: 4096 x 64 with
    # one and two token tiles, 2048 x 96 with a one-token second tile); other
    # token counts take the plain path
    F, D, T = shape
    r = np.random.default_rng(F * 7 + D + T)
    layers = [[(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)), (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
               (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))] for _ in range(3)]
    x = synth.q16_acts(r, T, D)
    packed = [tuple(ei.pack_q8(dev(c), dev(sc)) for c, sc in layer) for layer in layers]
    say("ffn chain", shape)
    y = host(ei.ffn_q8_chain(packed, dev(x), dev(lut)))
    ref = x
    for wg, wu, wd in layers:
        *_, ref = oracle.ffn_layer(ref, wg, wu, wd, lut)
    assert (y == ref).all()


def test_qwen_ffn_24_layers_chain(ei):
    lut = ei.silu_lut()
    packed = []
    for layer in range(synth.QWEN_LAYERS):
        (gc, gs), (uc, us), (dc, ds) = synth.qwen_ffn_layer(layer)
        packed.append((ei.pack_q8(dev(gc), dev(gs)), ei.pack_q8(dev(uc), dev(us)), ei.pack_q8(dev(dc), dev(ds))))
    say("ffn chain 24 layers")
    y = ei.ffn_q8_chain(packed, dev(synth.qwen_ffn_x0()), lut)
    assert ei.digest(y) == GOLDEN["qwen05b_ffn"]["layers"][-1]["x_next"]


@pytest.mark.parametrize("shape", [(96, 64, 3), (160, 96, 30), (4096, 64, 30), (4096, 64, 50), (2048, 96, 33),
                                   (96, 160, 70)])
def test_ffn_q8_prenorm_chain_matches_oracle(ei, lut, shape):
    # three pre-norm layers in one call: with a K-split down projection each
    # layer's output and the next layer's normalized limb tiles come from one
    # kernel per token; other shapes take the per-layer paths
    F, D, T = shape
    r = np.random.default_rng(F * 3 + D + T)
    layers = [[(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)), (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
               (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))] for _ in range(3)]
    norms = [r.integers(1 << 14, 1 << 17, D).astype(np.int32) for _ in range(3)]
    eps = 1 << 20
    x = synth.q16_acts(r, T, D)
    packed = [tuple(ei.pack_q8(dev(c), dev(sc)) for c, sc in layer) for layer in layers]
    say("ffn prenorm chain", shape)
    y = host(ei.ffn_q8_prenorm_chain(packed, [dev(g) for g in norms], eps, dev(x), dev(lut)))
    ref = x
    for (wg, wu, wd), gn in zip(layers, norms):
        *_, ref = oracle.ffn_layer_prenorm(ref, gn, eps, wg, wu, wd, lut)
    assert (y == ref).all()


def test_qwen_ffn_24_layers_prenorm_chain(ei):
    lut = ei.silu_lut()
    gold = GOLDEN["qwen05b_ffn_prenorm"]
    packed, norms = [], []
    for layer in range(synth.QWEN_LAYERS):
        (gc, gs), (uc, us), (dc, ds) = synth.qwen_ffn_layer(layer)
        packed.append((ei.pack_q8(dev(gc), dev(gs)), ei.pack_q8(dev(uc), dev(us)), ei.pack_q8(dev(dc), dev(ds))))
        norms.append(dev(synth.qwen_norm_weight(layer)))
    say("prenorm ffn chain 24 layers")
    y = ei.ffn_q8_prenorm_chain(packed, norms, gold["eps_q32"], dev(synth.qwen_ffn_x0()), lut)
    assert ei.digest(y) == gold["layers"][-1]["x_next"]


def test_qwen_ffn_24_layers_prenorm(ei):
    lut = ei.silu_lut()
    x = dev(synth.qwen_ffn_x0())
    y = torch.empty_like(x)
    gold = GOLDEN["qwen05b_ffn_prenorm"]
    for layer in range(synth.QWEN_LAYERS):
        (gc, gs), (uc, us), (dc, ds) = synth.qwen_ffn_layer(layer)
        wg, wu, wd = ei.pack_q8(dev(gc), dev(gs)), ei.pack_q8(dev(uc), dev(us)), ei.pack_q8(dev(dc), dev(ds))
        say("prenorm ffn layer", layer)
        ei.ffn_q8_prenorm(wg, wu, wd, dev(synth.qwen_norm_weight(layer)), gold["eps_q32"], x, lut, out=y)
        x, y = y, x
        assert ei.digest(x) == gold["layers"][layer]["x_next"], layer


def test_qwen_ffn_24_layers_fused(ei):
    lut = ei.silu_lut()
    x = dev(synth.qwen_ffn_x0())
    y = torch.empty_like(x)
    for layer in range(synth.QWEN_LAYERS):
        (gc, gs), (uc, us), (dc, ds) = synth.qwen_ffn_layer(layer)
        wg, wu, wd = ei.pack_q8(dev(gc), dev(gs)), ei.pack_q8(dev(uc), dev(us)), ei.pack_q8(dev(dc), dev(ds))
        say("fused ffn layer", layer)
        ei.ffn_q8(wg, wu, wd, x, lut, out=y)
        x, y = y, x
        assert ei.digest(x) == GOLDEN["qwen05b_ffn"]["layers"][layer]["x_next"], layer


@pytest.mark.parametrize("shape", [(5, 37, 3, 64, 96), (9, 12, 4, 32, 288), (100, 600, 2, 32, 64), (7, 50, 2, 160, 64)])
def test_moe_ffn_q8_small(ei, lut, shape):
    E, rows, topk, F, D = shape
    r = np.random.default_rng(E * 7 + rows)
    mats = [[(synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)), (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
             (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))] for _ in range(E)]
    x = synth.q16_acts(r, rows, D)
    route = (r.integers(0, E, (rows, topk)) ** 2 % E).astype(np.int32)
    if E == 9:   # one gate scale of 2^15 sends the fused gate/up pass to its per-limb accumulators
        mats[0][0][1][0, 0] = 32768

    def stack(m):
        return (dev(np.stack([mm[m][0] for mm in mats])), dev(np.stack([mm[m][1] for mm in mats])))
    wg, wu, wd = (ei.pack_q8_stacked(*stack(m)) for m in range(3))
    say("moe ffn", shape)
    y = host(ei.moe_ffn_q8(wg, wu, wd, dev(x), dev(route), dev(lut)))
    ref = oracle.moe_pairs(x, route, lambda e: mats[e], lut)
    assert (y == ref).all()


@pytest.mark.parametrize("t", [1, 2, 3, 4])
def test_q8_multi_qkv_and_ragged(ei, t):
    # one batched GEMV launch over Q, K, V of the Qwen layer-0 shapes plus
    # ragged row counts; every output equal to the oracle's and to the
    # separate projections
    r = np.random.default_rng(40 + t)
    K = 896
    ns = [896, 128, 128, 1000, 33, 32]
    mats = [(synth.q8_codes(r, n, K), synth.q8_scales(r, n, K)) for n in ns]
    mats[4] = (r.choice(np.array([-128, 127], np.int8), size=(33, K)),
               r.choice(np.array([-(2**31), 2**31 - 1], np.int64), size=(33, K // 32)).astype(np.int32))
    x = synth.q16_acts(r, t, K)
    x[0, :5] = [8355711, -8421504, 8355711, -8421504, 0]
    ws = [ei.pack_q8(dev(q), dev(s)) for q, s in mats]
    xd = dev(x)
    say("q8 multi", t)
    ys = [host(y) for y in ei.gemm_q8_multi(ws, xd)]
    for (q, s), w, y in zip(mats, ws, ys):
        assert (y == oracle.q8(q, s, x)).all()
        assert (y == host(ei.gemm_q8(w, xd))).all()


def test_q8_multi_sixteen_matrices(ei):
    # the largest batch, each matrix a different row count
    r = np.random.default_rng(77)
    K = 256
    mats = [(synth.q8_codes(r, 32 * (m + 1) - m, K), synth.q8_scales(r, 32 * (m + 1) - m, K)) for m in range(16)]
    x = synth.q16_acts(r, 1, K)
    ws = [ei.pack_q8(dev(q), dev(s)) for q, s in mats]
    say("q8 multi 16")
    ys = [host(y) for y in ei.gemm_q8_multi(ws, dev(x))]
    for (q, s), y in zip(mats, ys):
        assert (y == oracle.q8(q, s, x)).all()


@pytest.fixture(scope="module")
def dense(ei):
    q, s = synth.dense_w()
    return q, s, ei.pack_q8(dev(q), dev(s))


def test_dense_t1(ei, dense):
    # the whole T=1 output against the oracle's digest, under every schedule
    q, s, w = dense
    xd = dev(synth.dense_x(1))
    for sched in SCHEDS:
        say("dense T=1", sched)
        assert ei.digest(ei.gemm_q8(w, xd, 3, sched)) == GOLDEN["dense_14336x4096"]["t1_y"], sched


def test_dense_t512_full_output_all_schedules(ei, dense):
    # all 512 x 14336 outputs against the oracle's digest ([Handshake]
    # Falsifier 3: a single mismatched cell at any scale), under every
    # schedule including the pairwise tree (22.5 GB of per-block terms)
    q, s, w = dense
    x = synth.dense_x(512)
    xd = dev(x)
    say("dense T=512 default")
    y = host(ei.gemm_q8(w, xd))
    assert oracle.digest(y) == GOLDEN["dense_14336x4096"]["t512_y"]
    rows = np.array([0, 31, 32, 14335])
    assert (y[:, rows] == oracle.q8(q[rows], s[rows], x, threads=8)).all()
    del y
    for sched in SCHEDS[1:]:
        say("dense T=512", sched)
        assert ei.digest(ei.gemm_q8(w, xd, 3, sched)) == GOLDEN["dense_14336x4096"]["t512_y"], sched
        torch.cuda.empty_cache()


def test_repeat_runs_identical(ei, dense):
    q, s, w = dense
    for t in (1, 64):
        xd = dev(synth.dense_x(t))
        say("repeat", t)
        assert len({ei.digest(ei.gemm_q8(w, xd)) for _ in range(3)}) == 1


# ------------------------------------------------- tiled kernel accumulators

def test_q8_tiled_per_limb_accumulators_extreme_scales(ei):
    # scales at the int32 ends through the tiled kernel (8 x 17 workgroups,
    # ragged in rows and tokens): its per-limb int64 accumulators stay exact
    N, K, T = 1000, 256, 520
    r = np.random.default_rng(12)
    q = r.choice(np.array([-128, 127, -127, 3, 0], np.int8), size=(N, K))
    s = r.choice(np.array([-(2**31), 2**31 - 1, 1, -1, 40000], np.int64), size=(N, K // 32)).astype(np.int32)
    x = r.choice(np.array([8355711, -8421504, 0, 1, -1, 2**22], np.int64), size=(T, K))
    say("tiled per-limb accumulators")
    w = ei.pack_q8(dev(q), dev(s))
    assert (host(ei.gemm_q8(w, dev(x))) == oracle.q8(q, s, x)).all()


@pytest.mark.parametrize("N", [1000, 1100])
def test_q8_tiled_narrow_scales_at_the_edge(ei, N):
    # max|S| = 2^15 - 1: the tiled kernel's two-chain accumulation (S (P_0 +
    # 2^8 P_1) and 2^16 S P_2), with codes and activations at their ends;
    # 8 x 17 = 136 workgroups take the XCD-contiguous order, 9 x 17 = 153 the
    # launch order
    K, T = 256, 520
    r = np.random.default_rng(13 + N)
    q = r.choice(np.array([-128, 127, -127, 3, 0], np.int8), size=(N, K))
    s = r.choice(np.array([-32767, 32767, 1, -1, 0, 12345], np.int64), size=(N, K // 32)).astype(np.int32)
    x = r.choice(np.array([8355711, -8421504, 0, 1, -1, 2**22], np.int64), size=(T, K))
    say("tiled narrow scales")
    w = ei.pack_q8(dev(q), dev(s))
    assert w.desc.smax == 32767
    assert (host(ei.gemm_q8(w, dev(x))) == oracle.q8(q, s, x)).all()


# Wide scales (|S| >= 2^15) send the tiled kernels to their per-limb form,
# which addresses a whole matrix's code tiles through one buffer resource.
# At n_pad * k = 2^27 (16384 x 8192) that size must not wrap: a wrapped size
# reads every code as zero.
WRAP_N, WRAP_K = 16384, 8192


def _wide_scale_matrix(r, n, k):
    q = synth.q8_codes(r, n, k)
    s = r.integers(-(2**16), 2**16 + 1, (n, k // 32)).astype(np.int32)
    s[0, 0] = 2**16   # never narrow
    return q, s


def test_q8_tiled_wide_scales_at_the_code_size_wrap(ei):
    r = np.random.default_rng(31)
    q, s = _wide_scale_matrix(r, WRAP_N, WRAP_K)
    x = synth.q16_acts(r, 64, WRAP_K)
    say("tiled wide scales at n_pad*k = 2^27")
    w = ei.pack_q8(dev(q), dev(s))
    assert w.desc.smax == 2**16
    y = host(ei.gemm_q8(w, dev(x)))
    rows = np.concatenate([r.choice(WRAP_N, 12, replace=False), [0, 31, WRAP_N - 32, WRAP_N - 1]])
    assert (y[:, rows] == oracle.q8(q[rows], s[rows], x, threads=8)).all()
    assert (y[:, rows] != 0).any()


def test_grouped_wide_scales_at_the_code_size_wrap(ei, lut):
    # two experts of 16384 x 8192 (gate, up) and 8192 x 16384 (down): the
    # routed projection and the fused gate/up pass in their per-limb form
    r = np.random.default_rng(32)
    E, rows, topk = 2, 48, 2
    F, D = WRAP_N, WRAP_K
    mats = [[_wide_scale_matrix(r, F, D), _wide_scale_matrix(r, F, D), _wide_scale_matrix(r, D, F)]
            for _ in range(E)]
    x = r.integers(-(2**12), 2**12 + 1, (rows, D)).astype(np.int64)
    route = np.stack([r.permutation(E)[:topk] for _ in range(rows)]).astype(np.int32)

    def stack(m):
        return (dev(np.stack([mm[m][0] for mm in mats])), dev(np.stack([mm[m][1] for mm in mats])))
    say("grouped wide scales: pack")
    wg, wu, wd = (ei.pack_q8_stacked(*stack(m)) for m in range(3))
    assert wg.desc.smax == 2**16
    xd, rd = dev(x), dev(route)
    say("grouped wide scales: gate projection")
    g = host(ei.gemm_q8_grouped(wg, xd, rd))
    pick = [(0, 0), (0, 1), (17, 0), (rows - 1, 1)]
    for (t, k) in pick:
        e = int(route[t, k])
        want = oracle.q8(mats[e][0][0], mats[e][0][1], x[t:t + 1], threads=8)[0]
        assert (g[t * topk + k] == want).all(), (t, k)
    say("grouped wide scales: routed FFN")
    y = host(ei.moe_ffn_q8(wg, wu, wd, xd, rd, dev(lut)))
    down_rows = [0, 1, 4095, D - 1]
    ref = oracle.moe_pairs(x, route, lambda e: mats[e], lut, pairs=pick, down_rows=down_rows, threads=8)
    for (t, k), want in zip(pick, ref):
        assert (y[t * topk + k][down_rows] == want).all(), (t, k)
    assert (y != 0).any()


@pytest.mark.parametrize("emax", [14, 15])
def test_q4_tiled_exact_output(ei, emax):
    # the tiled prefill path (128 workgroups of 128 rows x 32 tokens) with the
    # exact, unrounded output of the 4-bit format: scales 2^e with e <= 14 take
    # the register-fed narrow kernel, one e = 15 (max|S| = 2^15) the per-limb one
    N, K, T = 2048, 128, 256
    r = np.random.default_rng(31 + emax)
    nib = synth.q4_codes_packed(r, N, K)
    m = r.integers(1, 16, (N, K // 32))
    e = r.integers(0, emax + 1, (N, K // 32))
    e[5, 1] = emax
    sme = (m | (e << 4)).astype(np.uint8)
    x = r.integers(-(2**15), 2**15, (T, K), dtype=np.int64).astype(np.int32)
    x[3] = -(2**15)
    say("q4 tiled exact", emax)
    w = ei.pack_q4(dev(nib), dev(sme))
    assert w.desc.smax == 2**emax
    assert (host(ei.gemm_q4(w, dev(x))) == oracle.q4(nib, sme, x)).all()


@pytest.mark.parametrize("shape", [(200, 512, 40), (70, 131072, 8), (96, 1024, 63)])
@pytest.mark.parametrize("scale", [32767, -32768])
def test_q8_skinny_accumulators_at_the_narrow_bound(ei, shape, scale):
    # the skinny kernel (5 <= T < 64, K split over workgroups) with every term
    # at its extreme: |S| = 2^15 - 1 takes the two-chain accumulation (at
    # K = 131072 its sums reach about 2^62), |S| = 2^15 the per-limb one
    N, K, T = shape
    r = np.random.default_rng(N + K + T)
    q = r.choice(np.array([-128, 127], np.int8), size=(N, K))
    s = np.full((N, K // 32), scale, np.int32)
    s[::5] = -scale
    x = r.choice(np.array([8355711, -8421504], np.int64), size=(T, K))
    x[0] = -8421504
    q[0] = -128
    say("skinny narrow bound", shape, scale)
    w = ei.pack_q8(dev(q), dev(s))
    assert (host(ei.gemm_q8(w, dev(x))) == oracle.q8(q, s, x)).all()


@pytest.mark.parametrize("scale", [-32767, -32768])
def test_q8_grouped_accumulators_at_the_narrow_bound(ei, scale):
    # K = 131072 (4096 blocks) with every term at its extreme: at |S| = 2^15 - 1
    # the two-chain accumulation reaches nb * max|S| = 2^27 - 4096, its bound
    # (sums near 2^62); at |S| = 2^15 the per-limb accumulators take over
    E, rows, topk, N, K = 2, 40, 1, 32, 131072
    codes = np.full((E, N, K), -128, np.int8)
    codes[1, ::3] = 127
    scales = np.full((E, N, K // 32), scale, np.int32)
    x = np.full((rows, K), -8421504, np.int64)
    x[::4] = 8355711
    route = (np.arange(rows) % E).astype(np.int32)[:, None]
    say("grouped narrow bound", scale)
    w = ei.pack_q8_stacked(dev(codes), dev(scales))
    y = host(ei.gemm_q8_grouped(w, dev(x), dev(route)))
    assert (y == _grouped_reference(codes, scales, x, route)).all()


# ------------------------------------------------------------- routed (MoE)

def _grouped_reference(codes, scales, x, route):
    """Oracle rows y[r*topk + s] = Q8(expert route[r][s], x[r]), one oracle
    call per expert on the rows routed to it."""
    rows, topk = route.shape
    y = np.zeros((rows * topk, codes.shape[1]), np.int64)
    for e in np.unique(route):
        rr, ss = np.nonzero(route == e)
        y[rr * topk + ss] = oracle.q8(codes[e], scales[e], x[rr])
    return y


@pytest.mark.parametrize("shape", [(5, 37, 3, 70, 96), (3, 50, 2, 33, 64), (9, 12, 4, 130, 288)])
def test_q8_grouped_small(ei, shape):
    E, rows, topk, N, K = shape
    r = np.random.default_rng(E * 100 + rows)
    codes = np.stack([synth.q8_codes(r, N, K) for _ in range(E)])
    scales = np.stack([synth.q8_scales(r, N, K) for _ in range(E)])
    x = synth.q16_acts(r, rows, K)
    route = np.stack([np.sort(r.choice(E, topk, replace=False)) for _ in range(rows)]).astype(np.int32)
    say("grouped", shape)
    w = ei.pack_q8_stacked(dev(codes), dev(scales))
    y = host(ei.gemm_q8_grouped(w, dev(x), dev(route)))
    assert (y == _grouped_reference(codes, scales, x, route)).all()


def test_q8_grouped_skewed_and_extreme(ei):
    # one expert takes most pairs (several token tiles), one takes none, and
    # the scales force the per-limb accumulators
    E, rows, topk, N, K = 4, 80, 2, 64, 128
    r = np.random.default_rng(21)
    codes = np.stack([r.integers(-128, 128, (N, K), dtype=np.int16).astype(np.int8) for _ in range(E)])
    scales = np.stack([r.integers(-(2**31), 2**31, (N, K // 32), dtype=np.int64).astype(np.int32)
                       for _ in range(E)])
    x = r.integers(-8421504, 8355712, (rows, K), dtype=np.int64)
    route = np.zeros((rows, topk), np.int32)
    route[:, 0] = 0
    route[:, 1] = np.where(np.arange(rows) % 5 == 0, 3, 1)
    say("grouped skewed")
    w = ei.pack_q8_stacked(dev(codes), dev(scales))
    y = host(ei.gemm_q8_grouped(w, dev(x), dev(route)))
    assert (y == _grouped_reference(codes, scales, x, route)).all()


@pytest.mark.parametrize("shape", [(100, 1500, 2, 32, 64), (1, 70, 3, 40, 32), (7, 8192, 2, 32, 32),
                                   (300, 200, 2, 32, 32)])
def test_q8_grouped_sort_sizes(ei, shape):
    # pair counts that leave ragged per-thread runs in the grouping sort, up to
    # the 2^14-pair maximum; a single expert; 100 experts (a non-power-of-two
    # expert field); 300 experts (more buckets than the counting sort has: the
    # radix sort); unsorted routes that may repeat an expert within a row
    E, rows, topk, N, K = shape
    r = np.random.default_rng(E + rows)
    codes = np.stack([synth.q8_codes(r, N, K) for _ in range(E)])
    scales = np.stack([synth.q8_scales(r, N, K) for _ in range(E)])
    x = synth.q16_acts(r, rows, K)
    route = (r.integers(0, E, (rows, topk)) ** 2 % E).astype(np.int32)   # skewed toward some experts
    say("grouped sort sizes", shape)
    w = ei.pack_q8_stacked(dev(codes), dev(scales))
    y = host(ei.gemm_q8_grouped(w, dev(x), dev(route)))
    assert (y == _grouped_reference(codes, scales, x, route)).all()


@pytest.mark.parametrize("E", [3, 300])   # the counting sort and the radix sort
def test_q8_grouped_bad_expert_is_flagged(ei, E):
    rows, topk, N, K = 8, 2, 32, 64
    r = np.random.default_rng(22)
    codes = np.stack([synth.q8_codes(r, N, K) for _ in range(E)])
    scales = np.stack([synth.q8_scales(r, N, K) for _ in range(E)])
    route = np.tile(np.array([[0, 1]], np.int32), (rows, 1))
    route[3, 1] = E
    say("grouped bad expert", E)
    w = ei.pack_q8_stacked(dev(codes), dev(scales))
    with pytest.raises(ei.EIError):
        ei.gemm_q8_grouped(w, dev(synth.q16_acts(r, rows, K)), dev(route))


@pytest.fixture(scope="module")
def olmoe(ei):
    # 64 experts (gate/up 1024x2048, down 2048x1024), 512 tokens, top-8
    E = synth.OLMOE_E
    mats = [synth.olmoe_expert(e) for e in range(E)]

    def stacked(m):
        return ei.pack_q8_stacked(dev(np.stack([mm[m][0] for mm in mats])), dev(np.stack([mm[m][1] for mm in mats])))
    say("olmoe pack")
    return mats, stacked(0), stacked(1), stacked(2), synth.olmoe_x(), synth.olmoe_route()


def test_olmoe_grouped_ffn_full_output(ei, lut, olmoe):
    # the full routed FFN on the GPU: all 4096 x 2048 outputs against the
    # oracle's digest, by three grouped calls and by the one-call routed FFN
    mats, wg, wu, wd, x, route = olmoe
    xd, rd = dev(x), dev(route)
    say("olmoe grouped ffn")
    g = ei.gemm_q8_grouped(wg, xd, rd)
    u = ei.gemm_q8_grouped(wu, xd, rd)
    h = ei.silu_mul(g, u, ei.silu_lut())
    out = ei.gemm_q8_grouped(wd, h, rd.reshape(-1, 1))
    assert tuple(out.shape) == (synth.OLMOE_T * synth.OLMOE_TOPK, synth.OLMOE_H)
    assert ei.digest(out) == GOLDEN["olmoe_step"]["y"]
    pairs = [(0, 0), (511, 7), (200, 3)]
    ref = oracle.moe_pairs(x, route, lambda e: mats[e], lut, pairs=pairs, threads=8)
    outh = host(out)
    for (t, k), want in zip(pairs, ref):
        assert (outh[t * 8 + k] == want).all(), (t, k)
    say("olmoe routed ffn, one call")
    assert ei.digest(ei.moe_ffn_q8(wg, wu, wd, xd, rd, dev(lut))) == GOLDEN["olmoe_step"]["y"]


def test_olmoe_expert_schedule_gate(ei, olmoe):
    # each expert's three projections on the rows routed to it, run as plain
    # projections under the five schedules, equal the grouped outputs row for
    # row (whose whole digest equals the oracle's above)
    mats, wg, wu, wd, x, route = olmoe
    xd, rd = dev(x), dev(route)
    g = ei.gemm_q8_grouped(wg, xd, rd)
    u = ei.gemm_q8_grouped(wu, xd, rd)
    h = ei.silu_mul(g, u, ei.silu_lut())
    out = ei.gemm_q8_grouped(wd, h, rd.reshape(-1, 1))
    for e in range(synth.OLMOE_E):
        tt, kk = np.nonzero(route == e)
        pr = torch.from_numpy(tt * synth.OLMOE_TOPK + kk).cuda()
        (gc, gs), (uc, us), (dc, ds) = mats[e]
        pg, pu, pd = ei.pack_q8(dev(gc), dev(gs)), ei.pack_q8(dev(uc), dev(us)), ei.pack_q8(dev(dc), dev(ds))
        xe, he = xd[torch.from_numpy(tt).cuda()].contiguous(), h[pr].contiguous()
        for sched in SCHEDS:
            say("olmoe expert", e, "rows", len(tt), sched)
            assert torch.equal(ei.gemm_q8(pg, xe, 3, sched), g[pr]), (e, sched, "gate")
            assert torch.equal(ei.gemm_q8(pu, xe, 3, sched), u[pr]), (e, sched, "up")
            assert torch.equal(ei.gemm_q8(pd, he, 3, sched), out[pr]), (e, sched, "down")


# ------------------------------------- second derivations (table reads)

@pytest.mark.parametrize("shape", [(37, 96, 1), (100, 320, 4), (64, 288, 64), (1030, 512, 3), (33, 2048, 7)])
def test_q4_table_read_equals_mfma_path_and_oracle(ei, shape):
    N, K, T = shape
    r = np.random.default_rng(N * 5 + K + T)
    nib, sme, x = synth.q4_codes_packed(r, N, K), synth.q4_scale_bytes(r, N, K), synth.i32_acts(r, T, K)
    say("q4 table read", shape)
    yt = host(ei.gemm_q4_table(dev(nib), dev(sme), dev(x)))
    assert (yt == oracle.q4(nib, sme, x)).all()
    assert (yt == host(ei.gemm_q4(ei.pack_q4(dev(nib), dev(sme)), dev(x)))).all()


def test_q4_table_read_full_ranges(ei):
    # every nibble and scale byte value (m = 0 and code -8 included), int32 ends
    N, K, T = 64, 512, 5
    r = np.random.default_rng(81)
    nib = r.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sme = r.integers(0, 256, (N, K // 32)).astype(np.uint8)
    x = r.choice(np.array([2**31 - 1, -(2**31), 0, 1, -1, 12345], np.int64), size=(T, K)).astype(np.int32)
    say("q4 table read ranges")
    assert (host(ei.gemm_q4_table(dev(nib), dev(sme), dev(x))) == oracle.q4(nib, sme, x)).all()


def test_q4_table_read_overflow_is_flagged(ei):
    # codes -8, m = 15, e = 15, x = -2^31: every group of 32 adds
    # 15 * 2^15 * 32 * 2^34 = 15 * 2^54, so 64 groups (eight chunks of 256
    # columns) reach 15 * 2^60 > 2^63; the int128 sums of the chunks meet in
    # the combiner, which flags the result
    N, K, T = 40, 2048, 2
    nib = np.full((N, K // 2), 0x88, np.uint8)
    sme = np.full((N, K // 32), 0xFF, np.uint8)
    x = np.full((T, K), -(2**31), np.int32)
    say("q4 table read overflow")
    with pytest.raises(ei.EIError):
        ei.gemm_q4_table(dev(nib), dev(sme), dev(x))
    # 16 groups left (15 * 2^58): the sum fits again
    x[:, K // 2:] = 0
    x[:, : K // 4] = 0
    assert (host(ei.gemm_q4_table(dev(nib), dev(sme), dev(x))) == oracle.q4(nib, sme, x)).all()


def test_silu_mul_radix16_equals_silu_mul(ei, lut):
    r = np.random.default_rng(82)
    g = np.concatenate([r.integers(-(2**21), 2**21, 50000), r.integers(-(2**40), 2**40, 1000),
                        [-(2**63), 2**63 - 1, -16, -17, 15, 16, 31, 32, 33]]).astype(np.int64)
    u = np.concatenate([r.integers(-(2**40), 2**40, g.size - 4), [-(2**63), 2**63 - 1, 0, -1]]).astype(np.int64)
    say("silu_mul radix16")
    h = host(ei.silu_mul_radix16(dev(g), dev(u), dev(lut)))
    assert (h == oracle.silu_mul(g, u, lut)).all()
    assert (h == host(ei.silu_mul(dev(g), dev(u), dev(lut)))).all()


# ------------------------------------------------------- wide-code GEMM

WIDE_ACT_MAX = 127 * (256**4 - 1) // 255   # 2,139,062,143: four balanced digits reach no higher

@pytest.mark.parametrize("shape", [(32, 32, 1), (37, 64, 5), (100, 96, 70), (64, 1024, 33), (130, 320, 200)])
def test_wide_gemm_matches_oracle(ei, shape):
    N, K, T = shape
    r = np.random.default_rng(N * K + T)
    c = synth.wide_codes_from_trits(synth.wide_trits(r, N, K))
    a = r.integers(-(2**31), WIDE_ACT_MAX + 1, (T, K)).astype(np.int32)   # all four-digit int32 values
    say("wide", shape)
    w = ei.pack_wide(dev(c))
    assert (host(ei.gemm_wide(w, dev(a))) == oracle.wide_gemm(c, a)).all()


def test_wide_gemm_digit_range_ends_and_max_k(ei):
    r = np.random.default_rng(71)
    # codes at the three-digit ends, activations at the int32 ends
    N, K, T = 40, 96, 9
    c = r.choice(np.array([8355711, -8421504, 0, 1, -1], np.int32), size=(N, K))
    a = r.choice(np.array([WIDE_ACT_MAX, -(2**31), 0, 1, -1], np.int64), size=(T, K)).astype(np.int32)
    say("wide ends")
    assert (host(ei.gemm_wide(ei.pack_wide(dev(c)), dev(a))) == oracle.wide_gemm(c, a)).all()
    # K = 32768, the largest the int32 accumulators allow
    N, K, T = 32, 32768, 40
    c = synth.wide_codes_from_trits(synth.wide_trits(r, N, K))
    a = synth.wide_acts(r, T, K)
    say("wide max K")
    assert (host(ei.gemm_wide(ei.pack_wide(dev(c)), dev(a))) == oracle.wide_gemm(c, a)).all()
    # a code outside the three-digit range is refused at pack time
    c[3, 7] = 8355712
    with pytest.raises(ei.EIError):
        ei.pack_wide(dev(c))
    # an activation above the four-digit range is flagged
    a[0, 0] = WIDE_ACT_MAX + 1
    with pytest.raises(ei.EIError):
        ei.gemm_wide(ei.pack_wide(dev(synth.wide_codes_from_trits(synth.wide_trits(r, 32, K)))), dev(a))


def test_wide_hot_kernel_digest(ei):
    c, a = synth.wide_inputs()
    say("wide hot kernel 896x896, 4096 rows")
    y = ei.gemm_wide(ei.pack_wide(dev(c)), dev(a))
    assert ei.digest(y) == GOLDEN["wide_896x896_t4096"]["y"]


# ------------------------------------------- requantization and RMSNorm

def test_requant_matches_oracle(ei):
    r = np.random.default_rng(51)
    c = np.concatenate([r.integers(-(2**62), 2**62, 4000), np.arange(-9, 10),
                        [np.iinfo(np.int64).min + 1, np.iinfo(np.int64).max]]).astype(np.int64)
    for m, k in ((1, 0), (1, 1), (3, 2), (2**31 - 7, 31), (-(2**40) + 3, 60), (2**63 - 1, 126), (-(2**63), 126)):
        say("requant", m, k)
        assert (host(ei.requant(dev(c), m, k)) == oracle.requant(c, m, k)).all(), (m, k)


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 7, 42950), (16, 896, 42950), (4, 2048, 2**32),
                                   (2, 65536, 429497)])
def test_rmsnorm_q16_matches_oracle(ei, shape):
    T, D, eps = shape
    r = np.random.default_rng(T * D)
    x = synth.q16_acts(r, T, D)
    g = r.integers(2**15, 2**17, D).astype(np.int32)
    say("rmsnorm", shape)
    assert (host(ei.rmsnorm_q16(dev(x), dev(g), eps)) == oracle.rmsnorm_q16(x, g, eps)).all()


def test_rmsnorm_q16_extremes_and_range_flag(ei):
    D = 4096
    x = np.full((3, D), 2**23, np.int64)
    x[1] = -(2**23)
    x[2, ::2] = 0
    g = np.full(D, 2**31 - 1, np.int32)
    g[::3] = -(2**31)
    say("rmsnorm extremes")
    assert (host(ei.rmsnorm_q16(dev(x), dev(g), 1)) == oracle.rmsnorm_q16(x, g, 1)).all()
    x[0, 5] = 2**23 + 1
    with pytest.raises(ei.EIError):
        ei.rmsnorm_q16(dev(x), dev(g), 1)


# ---------------------------------------------------------- top-k routing

@pytest.mark.parametrize("shape", [(1, 1, 1), (37, 5, 3), (100, 64, 8), (50, 100, 7), (20, 300, 20),
                                   (9, 2048, 64), (3, 130, 130)])
def test_topk_route_matches_oracle(ei, shape):
    # scores from a small range, so ties are everywhere: the lower index wins
    T, E, k = shape
    r = np.random.default_rng(T + E + k)
    sc = r.integers(-3, 4, (T, E)).astype(np.int64)
    say("topk", shape)
    assert (host(ei.topk_route(dev(sc), k)) == oracle.topk_route(sc, k)).all()


def test_topk_route_int64_ends(ei):
    lo, hi = np.iinfo(np.int64).min, np.iinfo(np.int64).max
    sc = np.array([[lo, hi, 0, hi, -1, lo, 1], [lo] * 7, [hi] * 7], np.int64)
    for k in (1, 4, 7):
        say("topk ends", k)
        assert (host(ei.topk_route(dev(sc), k)) == oracle.topk_route(sc, k)).all()


def test_olmoe_integer_router(ei):
    # the router as a Q8 projection (64 experts x 2048) of the OLMoE
    # activations, then integer top-8: scores and route digests = oracle's
    (rc, rs), x = synth.olmoe_router(), synth.olmoe_x()
    say("olmoe router")
    scores = ei.gemm_q8(ei.pack_q8(dev(rc), dev(rs)), dev(x))
    route = ei.topk_route(scores, synth.OLMOE_TOPK)
    assert ei.digest(scores) == GOLDEN["olmoe_router"]["scores"]
    assert ei.digest(route) == GOLDEN["olmoe_router"]["route"]


def test_olmoe_step_with_integer_router(ei, lut, olmoe):
    # the routed FFN behind the integer router: the whole output = oracle's
    _, wg, wu, wd, x, _ = olmoe
    (rc, rs) = synth.olmoe_router()
    xd = dev(x)
    say("olmoe step with the integer router")
    route = ei.topk_route(ei.gemm_q8(ei.pack_q8(dev(rc), dev(rs)), xd), synth.OLMOE_TOPK)
    assert ei.digest(ei.moe_ffn_q8(wg, wu, wd, xd, route, dev(lut))) == GOLDEN["olmoe_router"]["y"]


# ------------------------------------------------------------- FP32 shadow

def test_fp32_shadow_matches_oracle_orders_and_splinters(ei):
    # the float negative control of the schedule gate: each schedule's float32
    # sum matches the oracle's float32 sum in that order bit for bit, and the
    # five schedules do not all agree (the integer digests do)
    mats, x = synth.qkv_inputs()
    xd = dev(x)
    for name, (c, sc) in mats.items():
        cd, sd = dev(c), dev(sc)
        digests = set()
        for order in oracle.SCHEDULES:
            say("fp32 shadow", name, order)
            dg = ei.digest(ei.fp32_shadow(cd, sd, xd, order, seed=0xE1))
            assert dg == GOLDEN["qkv_gate"][name + "_fp32"][order], (name, order)
            digests.add(dg)
        assert len(digests) >= 2, name


@pytest.mark.parametrize("shape", [(37, 96, 3), (5, 3200, 2), (64, 4096, 1)])
def test_fp32_shadow_small_all_orders(ei, shape):
    N, K, T = shape
    r = np.random.default_rng(N + K + T)
    q, s, x = synth.q8_codes(r, N, K), synth.q8_scales(r, N, K), synth.q16_acts(r, T, K)
    for order in oracle.SCHEDULES:
        say("fp32 shadow small", shape, order)
        y = host(ei.fp32_shadow(dev(q), dev(s), dev(x), order, seed=0x77))
        assert (y.view(np.uint32) == oracle.q8_fp32(q, s, x, order, seed=0x77).view(np.uint32)).all(), order


def test_gemv_repeated_calls_and_flagged_call(ei):
    # back-to-back GEMV calls of different T with one shared workspace; a
    # call whose activations are out of range is flagged, not fatal, and the
    # calls after it are still exact
    N, K = 1000, 2048
    r = np.random.default_rng(31)
    q, s = synth.q8_codes(r, N, K), synth.q8_scales(r, N, K)
    w = ei.pack_q8(dev(q), dev(s))
    ws = torch.zeros(max(ei.workspace_bytes(w, 4), 1), dtype=torch.uint8, device="cuda")
    for t in (1, 3, 4, 1, 2):
        x = synth.q16_acts(r, t, K)
        say("gemv reuse", t)
        assert (host(ei.gemm_q8(w, dev(x), workspace=ws)) == oracle.q8(q, s, x)).all(), t
    bad = synth.q16_acts(r, 1, K)
    bad[0, 7] = 2**40
    with pytest.raises(ei.EIError):
        ei.gemm_q8(w, dev(bad), workspace=ws)
    x = synth.q16_acts(r, 2, K)
    assert (host(ei.gemm_q8(w, dev(x), workspace=ws)) == oracle.q8(q, s, x)).all()
