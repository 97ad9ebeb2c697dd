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


def test_q8_four_limbs_wide_activations(ei):
    r = np.random.default_rng(6)
    N, K = 64, 256
    q, s = synth.q8_codes(r, N, K), synth.q8_scales(r, N, K)
    for T in (2, 40):
        x = r.integers(-(2**30), 2**30, size=(T, K)).astype(np.int64)
        say("q8 L=4", T)
        assert (host(ei.gemm_q8(ei.pack_q8(dev(q), dev(s)), dev(x), 4)) == oracle.q8(q, s, x)).all()


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


# ------------------------------------------------------------------ workloads

def test_q8_896x896_gemv(ei):
    (q, s), x = synth.q8_896_inputs()
    w = ei.pack_q8(dev(q), dev(s))
    say("q8 896x896 T=1")
    y = ei.gemm_q8(w, dev(x))
    assert ei.digest(y) == GOLDEN["q8_896x896"]["y"] == oracle.digest(oracle.q8(q, s, x))


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
            say("q4 d512", name, t)
            y = ei.gemm_q4(w, dev(synth.q4_d512_x(k, t)))
            assert ei.digest(y) == GOLDEN["q4_d512"][f"{name}_t{t}"]


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


def test_dense_t1(ei):
    q, s = synth.dense_w()
    w = ei.pack_q8(dev(q), dev(s))
    say("dense T=1")
    y = ei.gemm_q8(w, dev(synth.dense_x(1)))
    assert ei.digest(y) == GOLDEN["dense_14336x4096"]["t1_y"]


def test_dense_t512_sampled_rows_and_schedules(ei):
    q, s = synth.dense_w()
    x = synth.dense_x(512)
    w = ei.pack_q8(dev(q), dev(s))
    xd = dev(x)
    say("dense T=512 default")
    y = host(ei.gemm_q8(w, xd))
    rows = np.random.default_rng(9).choice(q.shape[0], 48, replace=False)
    rows = np.concatenate([rows, [0, 31, 32, 14335]])
    ref = oracle.q8(q[rows], s[rows], x, threads=8)
    assert (y[:, rows] == ref).all()
    # properties that hold at any size: every schedule gives the same bytes
    d0 = oracle.digest(y)
    for sched in ("reversed", "split_k", "tiled_shuffled"):
        say("dense T=512", sched)
        assert ei.digest(ei.gemm_q8(w, xd, 3, sched)) == d0, sched


def test_repeat_runs_identical(ei):
    q, s = synth.dense_w()
    w = ei.pack_q8(dev(q), dev(s))
    for t in (1, 64):
        xd = dev(synth.dense_x(t))
        say("repeat", t)
        assert len({ei.digest(ei.gemm_q8(w, xd)) for _ in range(3)}) == 1
