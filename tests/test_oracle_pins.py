"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against what the pages or the mathematics fix:
values printed on the pages (tests/golden/), closed forms, special cases
that reduce to a library routine (numpy integer matmul), invariants the
pages state (schedule invariance, row-order = column-stream), and brute
force with Python's arbitrary-precision integers on tiny inputs.
"""
import itertools
import zlib
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import bigint

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(tag):
    return np.random.default_rng(zlib.crc32(repr(tag).encode()))


def _rand_q8(r, N, K, T, extreme=False):
    if extreme:
        q = r.integers(-128, 128, size=(N, K), dtype=np.int16).astype(np.int8)
        s = r.integers(-(2**31), 2**31, size=(N, K // 32), dtype=np.int64).astype(np.int32)
        x = r.integers(-(2**40), 2**40, size=(T, K), dtype=np.int64)
    else:
        q = synth.q8_codes(r, N, K)
        s = synth.q8_scales(r, N, K)
        x = synth.q16_acts(r, T, K)
    return q, s, x


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("shape", [(1, 32, 1), (3, 64, 2), (5, 96, 3), (7, 128, 1)])
@pytest.mark.parametrize("extreme", [False, True])
def test_q8_matches_bigint(shape, extreme):
    N, K, T = shape
    r = np.random.default_rng(N * 1000 + K + T + int(extreme))
    q, s, x = _rand_q8(r, N, K, T, extreme)
    y = oracle.q8(q, s, x)
    yb = np.array(bigint.q8(q.tolist(), s.tolist(), x.tolist()), dtype=object)
    assert (y.astype(object) == yb).all()


def test_q8_extreme_corners_bigint():
    # every code at -128 or 127, every scale at the int32 ends, activations at
    # the ends of the 3-limb range: the largest magnitudes the int32/int8
    # formats allow (the spirit of Falsifier 7: exactness at the extremes).
    K = 64
    q = np.array([[-128] * K, [127] * K, [-128, 127] * (K // 2)], dtype=np.int8)
    s = np.array([[-(2**31), 2**31 - 1], [2**31 - 1, 2**31 - 1], [-(2**31), -(2**31)]], dtype=np.int32)
    x = np.array([[-8421504] * K, [8355711] * K, [8355711, -8421504] * (K // 2)], dtype=np.int64)
    y = oracle.q8(q, s, x)
    yb = np.array(bigint.q8(q.tolist(), s.tolist(), x.tolist()), dtype=object)
    assert (y.astype(object) == yb).all()


def test_q8_int64_overflow_reported():
    q = np.full((1, 32), 127, np.int8)
    s = np.full((1, 1), 2**31 - 1, np.int32)
    x = np.full((1, 32), 2**62, np.int64)
    with pytest.raises(oracle.OracleError):
        oracle.q8(q, s, x)


# ---------------------------------------------- reductions to library calls

def test_q8_reduces_to_integer_matmul():
    # With S = 2^24 and x = 2^16 X: acc = 2^40 (Q X), so y = 2^16 (Q X) exactly.
    r = _rng("matmul")
    N, K, T = 37, 160, 11
    Q = r.integers(-127, 128, size=(N, K)).astype(np.int8)
    X = r.integers(-1000, 1001, size=(T, K)).astype(np.int64)
    S = np.full((N, K // 32), 2**24, np.int32)
    y = oracle.q8(Q, S, X * 2**16)
    assert (y == (X @ Q.astype(np.int64).T) * 2**16).all()


def test_q8_scale_one_matches_floor_division():
    # With S = 1 the sum is (Q X); y = floor((QX + 2^23) / 2^24), via numpy.
    r = _rng("s1")
    N, K, T = 9, 96, 4
    Q = r.integers(-127, 128, size=(N, K)).astype(np.int8)
    X = r.integers(-(2**30), 2**30, size=(T, K)).astype(np.int64)
    S = np.ones((N, K // 32), np.int32)
    acc = X @ Q.astype(np.int64).T
    assert (oracle.q8(Q, S, X) == np.floor_divide(acc + 2**23, 2**24)).all()


@pytest.mark.parametrize("k", list(range(-6, 6)))
def test_q8_rounding_ties(k):
    # acc = (2k+1) 2^23 is exactly half-way: add-half-then-floor gives k+1;
    # one below gives k (round half up, for negative k too).
    q = np.zeros((1, 32), np.int8); q[0, 0] = 1
    s = np.ones((1, 1), np.int32)
    x = np.zeros((1, 32), np.int64)
    x[0, 0] = (2 * k + 1) * 2**23
    assert oracle.q8(q, s, x)[0, 0] == k + 1
    x[0, 0] -= 1
    assert oracle.q8(q, s, x)[0, 0] == k


def test_q8_hand_example():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "q8_hand_example.txt")) if l.strip() and not l.startswith("#")]
    rec = {l[0]: l[1:] for l in lines}
    q = np.zeros((1, 64), np.int8)
    x = np.zeros((1, 64), np.int64)
    for item in rec["codes"]:
        j, v = item.split(":"); q[0, int(j)] = int(v)
    for item in rec["x"]:
        j, v = item.split(":"); x[0, int(j)] = int(v)
    s = np.array([[int(v) for v in rec["scales"]]], np.int32)
    assert oracle.q8(q, s, x)[0, 0] == int(rec["y"][0])
    assert bigint.q8(q.tolist(), s.tolist(), x.tolist())[0][0] == int(rec["y"][0])


# ----------------------------------------------------------- invariants

@pytest.mark.parametrize("shape", [(37, 96, 19), (64, 288, 33), (5, 32, 1), (130, 1024, 3)])
def test_q8_all_orders_agree(shape):
    # Handshake C2 (row-order = column-stream) and C3 (five schedules, one
    # digest), on ragged shapes: N, T not multiples of the 16x16 tiles, nb
    # not a multiple of the 8 split-K ranges or of the 4-block K tiles.
    N, K, T = shape
    r = _rng(("orders",) + shape)
    q, s, x = _rand_q8(r, N, K, T, extreme=(N == 5))
    ref = oracle.q8(q, s, x)
    for order in oracle.ORDERS:
        for seed in (0xE1, 7):
            assert (oracle.q8(q, s, x, order=order, seed=seed) == ref).all(), order
    assert (oracle.q8(q, s, x, threads=4) == ref).all()
    assert (oracle.q8(q, s, x, order="row_order", threads=3) == ref).all()


def test_q8_radix16_products_agree():
    r = _rng("radix")
    q, s, x = _rand_q8(r, 11, 128, 3, extreme=True)
    ref = oracle.q8(q, s, x)
    for order in ("canonical", "column_stream", "tree_walk"):
        assert (oracle.q8(q, s, x, order=order, mul="radix16") == ref).all()


def test_radix16_product_identity():
    # UORLUT01 "Products of two runtime values": ab = sum_k 16^k T_a[d_k(b)].
    r = np.random.default_rng(5)
    vals = [0, 1, 15, 16, 255, 2**32 - 1, 2**63, 2**64 - 1, 2**64, 2**127, 2**128 - 1]
    vals += [int(v) for v in r.integers(0, 2**63, size=20, dtype=np.uint64)]
    vals += [(int(a) << 64) | int(b) for a, b in zip(r.integers(0, 2**63, 10, dtype=np.uint64),
                                                    r.integers(0, 2**63, 10, dtype=np.uint64))]
    for a in vals:
        for b in vals[::3]:
            assert oracle.mul128_radix16(a, b) == (a * b) % 2**128
            if a < 2**64 and b < 2**64:
                assert bigint.radix16_mul(a, b) == a * b


# ---------------------------------------------------------------- Q4 path

def _decode_q4(nib):
    lo = (nib & 0xF).astype(np.int16)
    hi = (nib >> 4).astype(np.int16)
    c = np.empty((nib.shape[0], nib.shape[1] * 2), np.int16)
    c[:, 0::2] = lo
    c[:, 1::2] = hi
    return np.where(c >= 8, c - 16, c).astype(np.int64)


def test_q4_reduces_to_integer_matmul():
    # m = 1, e = 0: y = Q X, computed with numpy int64.
    r = _rng("q4mm")
    N, K, T = 33, 256, 7
    nib = synth.q4_codes_packed(r, N, K)
    sme = np.ones((N, K // 32), np.uint8)
    x = synth.i32_acts(r, T, K)
    y = oracle.q4(nib, sme, x)
    assert (y == x.astype(np.int64) @ _decode_q4(nib).T).all()


def test_q4_power_of_two_scale_matches_matmul():
    # a single scale byte m=1, e=k everywhere: y = 2^k Q X.
    r = _rng("q4e")
    N, K, T = 8, 64, 3
    nib = synth.q4_codes_packed(r, N, K)
    x = synth.i32_acts(r, T, K)
    for e in (0, 5, 15):
        sme = np.full((N, K // 32), 1 | (e << 4), np.uint8)
        assert (oracle.q4(nib, sme, x) == (x.astype(np.int64) @ _decode_q4(nib).T) * 2**e).all()


@pytest.mark.parametrize("shape", [(1, 32, 1), (6, 64, 2), (9, 96, 3)])
def test_q4_matches_bigint(shape):
    N, K, T = shape
    r = _rng(("q4b",) + shape)
    nib = synth.q4_codes_packed(r, N, K)
    sme = synth.q4_scale_bytes(r, N, K)
    x = r.integers(-(2**31), 2**31, size=(T, K), dtype=np.int64).astype(np.int32)
    y = oracle.q4(nib, sme, x)
    assert (y.astype(object) == np.array(bigint.q4(nib.tolist(), sme.tolist(), x.tolist()), dtype=object)).all()


@pytest.mark.parametrize("shape", [(512, 512, 4), (13, 2048, 2), (7, 96, 5)])
def test_q4_table_read_equals_definition(shape):
    # UORLUT01's engine mechanism (tables by addition, 4-row blocking, scale by
    # shifts and adds) is a second derivation of the same projection.
    N, K, T = shape
    r = _rng(("q4t",) + shape)
    nib = synth.q4_codes_packed(r, N, K)
    sme = synth.q4_scale_bytes(r, N, K)
    x = synth.i32_acts(r, T, K)
    assert (oracle.q4(nib, sme, x, "table_read") == oracle.q4(nib, sme, x, "definition")).all()


# ------------------------------------------------------------ SiLU table

def test_silu_lut_closed_forms(lut):
    assert lut.shape == (65537,) and lut.dtype == np.int32
    assert lut[32768] == 0                          # silu(0) = 0
    assert lut[65536] == 1048576                    # 16 sigmoid(16) 2^16 = 1048575.88
    assert lut[0] == 0                              # silu(-16) 2^16 = -0.118
    assert lut[32768 + 2048] == round(math.e / (math.e + 1) * 65536)   # silu(1) = e/(e+1)
    assert lut[32768 - 2048] == round(-1 / (math.e + 1) * 65536)      # silu(-1) = -1/(e+1)


def test_silu_lut_within_half_of_float64(lut):
    k = np.arange(-32768, 32769, dtype=np.float64)
    z = k / 2048.0
    v = z / (1.0 + np.exp(-z)) * 65536.0
    assert np.max(np.abs(lut - v)) <= 0.5 + 1e-9
    # no entry near a tie, so the rounding rule never decides an entry
    frac = np.abs((v - np.floor(v)) - 0.5)
    assert np.min(frac) > 1e-6


def test_silu_lut_digest(lut):
    with open(os.path.join(GOLDEN, "silu_lut.sha256")) as f:
        assert oracle.digest(lut) == f.read().split()[0]


def test_silu_clip_matches_page_figures(lut):
    # Handshake C4: errors of the clipped table are x - 16 for x > 16, and the
    # worst activation's error is printed to 9 decimals.  With u = 1.0 (2^16)
    # the epilogue returns the table value itself.
    for line in open(os.path.join(GOLDEN, "silu_clip_page.txt")):
        if line.startswith("#") or not line.strip():
            continue
        act, err, dec = line.split()
        g = np.array([round(float(act) * 65536)], np.int64)
        h = oracle.silu_mul(g, np.array([65536], np.int64), lut)
        real = float(g[0]) / 65536
        silu_f64 = real / (1 + math.exp(-real))
        assert round(silu_f64 - h[0] / 65536, int(dec)) == pytest.approx(float(err), abs=10 ** -int(dec))
    # negative side: silu(-16) reads the first entry, 0 (|silu(-16)| ~ 1.8e-6)
    h = oracle.silu_mul(np.array([-16 * 65536, -40 * 65536], np.int64), np.array([65536, 65536], np.int64), lut)
    assert (h == 0).all()


def test_silu_mul_matches_bigint(lut):
    r = _rng("silu")
    n = 4000
    g = np.concatenate([r.integers(-(2**21), 2**21, n), r.integers(-(2**40), 2**40, 100),
                        np.array([-(2**63), 2**63 - 1 - 16, -16, -17, 15, 16, 17, 31, 32, 33, -1048576 - 1, 1048575])])
    u = r.integers(-(2**40), 2**40, g.size)
    g = g.astype(np.int64); u = u.astype(np.int64)
    h = oracle.silu_mul(g, u, lut)
    assert h.tolist() == bigint.silu_mul(g.tolist(), u.tolist(), lut.tolist())


def test_silu_index_is_add_half_shift(lut):
    # Q16 -> Q11: idx = floor((g + 16) / 32): g = 32k - 16 rounds up to k,
    # g = 32k - 17 rounds down to k - 1.
    u = np.array([65536], np.int64)
    for kk in (-5, 0, 1, 100, 2047, -2048):
        hi = oracle.silu_mul(np.array([32 * kk - 16], np.int64), u, lut)[0]
        lo = oracle.silu_mul(np.array([32 * kk - 17], np.int64), u, lut)[0]
        assert hi == lut[kk + 32768] and lo == lut[kk - 1 + 32768]


# -------------------------------------------------------- limb definition

def test_limb_split_exhaustive_3_limbs():
    x = np.arange(-(2**22), 2**22 + 1, dtype=np.int64)
    d, ok = oracle.limb_split(x, 3)
    assert ok
    rec = d[0].astype(np.int64) + 256 * d[1].astype(np.int64) + 65536 * d[2].astype(np.int64)
    assert (rec == x).all()


def test_limb_split_range_edges():
    for L in (1, 2, 3, 4, 8):
        hi = sum(127 * 256**l for l in range(L))
        lo = -sum(128 * 256**l for l in range(L))
        for v, good in ((hi, True), (lo, True), (hi + 1, False), (lo - 1, False)):
            if abs(v) >= 2**63:
                continue
            d, ok = oracle.limb_split(np.array([v], np.int64), L)
            assert ok == good
            if good:
                assert sum(int(d[l, 0]) * 256**l for l in range(L)) == v
            assert bigint.limbs(v, L)[1] == good


def test_limb_split_matches_bigint_random():
    r = _rng("limbs")
    x = r.integers(-(2**62), 2**62, 2000, dtype=np.int64)
    d, ok = oracle.limb_split(x, 8)
    assert ok
    for e in range(0, 2000, 37):
        assert d[:, e].tolist() == bigint.limbs(int(x[e]), 8)[0]


def test_limb_split_offset_covers_int16():
    # two digits of x - 128 cover exactly the int16 range [-2^15, 2^15)
    x = np.arange(-(2**15), 2**15, dtype=np.int64)
    d, ok = oracle.limb_split(x, 2, offset=oracle.Q4_OFFSET)
    assert ok
    rec = d[0].astype(np.int64) + 256 * d[1].astype(np.int64) + 128
    assert (rec == x).all()
    for v in (2**15, -(2**15) - 1):
        assert not oracle.limb_split(np.array([v], np.int64), 2, offset=oracle.Q4_OFFSET)[1]
    # without the offset two digits stop short of the top of the range
    assert not oracle.limb_split(np.array([2**15 - 1], np.int64), 2)[1]


def _rand_q4(r, N, K):
    nib = r.integers(0, 256, size=(N, K // 2), dtype=np.int64).astype(np.uint8)
    sme = (r.integers(0, 16, size=(N, K // 32)) | (r.integers(0, 16, size=(N, K // 32)) << 4)).astype(np.uint8)
    return nib, sme


@pytest.mark.parametrize("N,K", [(1, 32), (7, 64), (33, 160)])
def test_q4_row_offsets_equal_q4_at_the_offset(N, K):
    # with every activation equal to the offset, y = R exactly
    nib, sme = _rand_q4(_rng(("roff", N, K)), N, K)
    x = np.full((1, K), oracle.Q4_OFFSET, dtype=np.int32)
    assert (oracle.q4(nib, sme, x)[0] == oracle.q4_row_offsets(nib, sme)).all()


@pytest.mark.parametrize("N,K,T", [(5, 32, 3), (40, 96, 4), (17, 320, 2)])
def test_q4_row_offsets_two_limb_form_equals_q4(N, K, T):
    # y = q4(d_0) + 256 q4(d_1) + R with d the digits of x - 128: the two-limb form
    r = _rng(("two-limb", N, K, T))
    nib, sme = _rand_q4(r, N, K)
    x = r.integers(-(2**15), 2**15, size=(T, K)).astype(np.int32)
    x[0, :4] = [-(2**15), 2**15 - 1, 0, 128]
    d, ok = oracle.limb_split(x.astype(np.int64), 2, offset=oracle.Q4_OFFSET)
    assert ok
    d0 = d[0].reshape(T, K).astype(np.int32)
    d1 = d[1].reshape(T, K).astype(np.int32)
    y = oracle.q4(nib, sme, d0) + 256 * oracle.q4(nib, sme, d1) + oracle.q4_row_offsets(nib, sme)[None, :]
    assert (y == oracle.q4(nib, sme, x)).all()


# ------------------------------------------------------------ Q16 reading

def test_q16_semantics_page_values():
    for line in open(os.path.join(GOLDEN, "q16_semantics.txt")):
        if line.startswith("#") or not line.strip():
            continue
        q, real, dec = line.split()
        assert round(int(q) / 2**16, int(dec)) == float(real)


# -------------------------------------------------- FP32 negative control

def _shadow_operands(q, s, x):
    w = ((s.astype(np.int64).repeat(32, axis=1) * q.astype(np.int64)).astype(np.float64) * 2.0**-24).astype(np.float32)
    xf = (x.astype(np.float64) * 2.0**-16).astype(np.float32)
    return w, xf


def test_fp32_shadow_canonical_is_sequential_float32():
    r = _rng("fp32")
    q, s, x = _rand_q8(r, 6, 256, 3)
    w, xf = _shadow_operands(q, s, x)
    y = oracle.q8_fp32(q, s, x, "canonical")
    yr = oracle.q8_fp32(q, s, x, "reversed")
    for t in range(3):
        for i in range(6):
            prods = (w[i] * xf[t]).astype(np.float32)          # IEEE single products
            assert np.cumsum(prods, dtype=np.float32)[-1] == y[t, i]
            assert np.cumsum(prods[::-1], dtype=np.float32)[-1] == yr[t, i]


def test_fp32_shadow_tree_walk_is_pairwise_float32():
    r = _rng("fp32t")
    q, s, x = _rand_q8(r, 4, 224, 2)     # 7 blocks: an odd element passes up
    w, xf = _shadow_operands(q, s, x)
    y = oracle.q8_fp32(q, s, x, "tree_walk")
    for t in range(2):
        for i in range(4):
            prods = (w[i] * xf[t]).astype(np.float32)
            terms = [np.cumsum(prods[32 * b:32 * b + 32], dtype=np.float32)[-1] for b in range(7)]
            while len(terms) > 1:
                nxt = [np.float32(terms[m] + terms[m + 1]) for m in range(0, len(terms) - 1, 2)]
                if len(terms) % 2:
                    nxt.append(terms[-1])
                terms = nxt
            assert terms[0] == y[t, i]


def test_fp32_shadow_splinters_on_qkv_workload():
    # Handshake C3: the float shadow of the same GEMM splinters across the
    # five schedules while the integer result does not.
    q, s = synth.q8_matrix("qkv_gate", 0, "q", 896, 896)
    x = synth.q16_acts(synth.rng_for("qkv_gate", 0, "x"), 4, 896)
    fp = {o: oracle.digest(oracle.q8_fp32(q, s, x, o)) for o in oracle.SCHEDULES}
    ints = {o: oracle.digest(oracle.q8(q, s, x, o)) for o in oracle.SCHEDULES}
    assert len(set(ints.values())) == 1
    assert len(set(fp.values())) >= 2


# ------------------------------------------------------------ FFN chain

def test_ffn_layer_matches_bigint(lut):
    r = _rng("ffn")
    D, F, T = 64, 96, 2
    wg = (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D))
    wu = (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D))
    wd = (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))
    x = synth.q16_acts(r, T, D)
    g, u, h, d, xn = oracle.ffn_layer(x, wg, wu, wd, lut)
    gb = bigint.q8(wg[0].tolist(), wg[1].tolist(), x.tolist())
    ub = bigint.q8(wu[0].tolist(), wu[1].tolist(), x.tolist())
    hb = [bigint.silu_mul(gb[t], ub[t], lut.tolist()) for t in range(T)]
    db = bigint.q8(wd[0].tolist(), wd[1].tolist(), hb)
    assert g.tolist() == gb and u.tolist() == ub and h.tolist() == hb and d.tolist() == db
    assert xn.tolist() == [[x[t, j] + db[t][j] for j in range(D)] for t in range(T)]


# ------------------------------------------------------------- top-k routing

def _topk_brute(scores, k):
    # the unique permutation p with, for every i < j, p[i] ahead of p[j]:
    # a higher score, or an equal score and a lower index; its first k
    E = len(scores)
    for p in itertools.permutations(range(E)):
        if all(scores[p[i]] > scores[p[j]] or (scores[p[i]] == scores[p[j]] and p[i] < p[j])
               for i in range(E) for j in range(i + 1, E)):
            return list(p[:k])
    raise AssertionError("no order found")


def test_topk_route_brute_force_with_ties():
    r = np.random.default_rng(31)
    for _ in range(200):
        E = int(r.integers(1, 7))
        k = int(r.integers(1, E + 1))
        sc = r.integers(-2, 3, (1, E)).astype(np.int64)   # a tiny range: many ties
        assert oracle.topk_route(sc, k)[0].tolist() == _topk_brute(sc[0].tolist(), k)


def test_topk_route_special_cases():
    r = np.random.default_rng(32)
    sc = r.integers(-1000, 1000, (50, 64)).astype(np.int64)
    # k = 1 is the first maximum (numpy's argmax returns the first one)
    assert (oracle.topk_route(sc, 1)[:, 0] == np.argmax(sc, axis=1)).all()
    # k = E is a stable sort by descending score
    assert (oracle.topk_route(sc, 64) == np.argsort(-sc, axis=1, kind="stable")).all()
    # the int64 ends, all equal scores, and a constant row
    ext = np.array([[np.iinfo(np.int64).min, np.iinfo(np.int64).max, 0, np.iinfo(np.int64).max, -1]], np.int64)
    assert oracle.topk_route(ext, 5)[0].tolist() == [1, 3, 2, 4, 0]
    assert oracle.topk_route(np.zeros((1, 9), np.int64), 4)[0].tolist() == [0, 1, 2, 3]


# -------------------------------------------- requantization and RMSNorm

def _half_away(fr):
    """Round a Fraction half away from zero (exact)."""
    from fractions import Fraction
    a = abs(fr)
    n = int(a + Fraction(1, 2))   # floor(|v| + 1/2)
    return n if fr >= 0 else -n


def test_requant_exact_halves_and_fractions():
    from fractions import Fraction
    # exact halves go away from zero; quarters to the nearer integer
    assert [oracle.requant(v, 1, 1) for v in (3, -3, 1, -1, 2, -2)] == [2, -2, 1, -1, 1, -1]
    assert [oracle.requant(v, 1, 2) for v in (5, -5, 6, -6, 7, -7)] == [1, -1, 2, -2, 2, -2]
    r = np.random.default_rng(41)
    for _ in range(2000):
        c = int(r.integers(-(2**62), 2**62))
        m = int(r.integers(1, 2**63 - 1))
        k = int(r.integers(64, 126))
        want = _half_away(Fraction(c * m, 2**k))
        if -(2**63) <= want < 2**63:
            assert oracle.requant(c, m, k) == want


def test_rms_inverse_against_decimal_sqrt_and_float64():
    from decimal import Decimal, getcontext
    getcontext().prec = 80
    r = np.random.default_rng(42)
    worst = 0.0
    for _ in range(3000):
        d = int(r.integers(1, 5000))
        ss = int(r.integers(0, d * 2**46))
        eps = int(r.integers(1, 2**32))
        inv = oracle.rms_inverse(ss, d, eps)
        exact = (Decimal(2**104) * d / (ss + d * eps)).sqrt()
        assert inv == int(exact)                       # the floor of the exact root
        ref = 2.0**52 / math.sqrt(ss / d + eps)       # float64 1/sqrt, the pages' twin
        worst = max(worst, abs(inv - ref) / ref)
    assert worst < 2e-9                                # [tritify] Table 1: below 2e-9


def test_rmsnorm_q16_against_exact_real_rounding():
    from decimal import Decimal, getcontext
    getcontext().prec = 80
    r = np.random.default_rng(43)
    for d in (1, 7, 64, 896):
        x = np.clip(np.rint(r.normal(0, 1, (3, d)) * 2**16), -(2**22), 2**22).astype(np.int64)
        g = r.integers(2**15, 2**17, d).astype(np.int32)
        eps = 42950   # 1e-5 in Q32
        y = oracle.rmsnorm_q16(x, g, eps)
        for t in range(3):
            ms = Decimal(sum(int(v) ** 2 for v in x[t])) / d + eps
            rs = ms.sqrt()
            for i in range(d):
                v = Decimal(int(x[t, i])) * int(g[i]) / rs
                want = int(v + Decimal("0.5")) if v >= 0 else -int(-v + Decimal("0.5"))
                assert abs(int(y[t, i]) - want) <= 1


def test_rmsnorm_q16_closed_form():
    # X = 3 and eps = 16 in code units: mean square + eps = 25, rms = 5; with
    # G = 5 * 2^16 every output is X * G / 5 = 3 * 2^16 after rounding
    x = np.full((2, 9), 3, np.int64)
    x[1] = -3
    g = np.full(9, 5 * 2**16, np.int32)
    y = oracle.rmsnorm_q16(x, g, 16)
    assert (y[0] == 3 * 2**16).all() and (y[1] == -3 * 2**16).all()


# ------------------------------------------------------- wide-code GEMM

def test_wide_gemm_brute_force():
    r = np.random.default_rng(61)
    for n, k, t in ((1, 1, 1), (3, 5, 2), (7, 33, 4)):
        c = synth.wide_codes_from_trits(synth.wide_trits(r, n, k))
        a = r.integers(-(2**31), 2**31, (t, k)).astype(np.int32)
        y = oracle.wide_gemm(c, a)
        for tt in range(t):
            for i in range(n):
                assert int(y[tt, i]) == sum(int(c[i, j]) * int(a[tt, j]) for j in range(k))


def test_wide_gemm_trit_planes_and_one_hot():
    r = np.random.default_rng(62)
    trits = synth.wide_trits(r, 40, 96)
    c = synth.wide_codes_from_trits(trits)
    assert int(np.abs(c).max()) <= oracle.WIDE_CODE_MAX
    a = synth.wide_acts(r, 6, 96)
    # a second derivation: one integer matmul per trit plane, weighted by 3^i
    planes = sum((3 ** i) * (a.astype(np.int64) @ trits[i].astype(np.int64).T) for i in range(12))
    assert (oracle.wide_gemm(c, a) == planes).all()
    # one-hot activations pick columns of the codes
    e = np.zeros((3, 96), np.int32)
    e[0, 5], e[1, 0], e[2, 95] = 1, -1, 7
    y = oracle.wide_gemm(c, e)
    assert (y[0] == c[:, 5]).all() and (y[1] == -c[:, 0]).all() and (y[2] == 7 * c[:, 95].astype(np.int64)).all()


def test_wide_gemm_beyond_the_int64_fast_path():
    # |c| |a| K above 2^63 takes the Python-integer path; one large activation
    # and alternating +-1 elsewhere keep the exact sums in int64 with a plain
    # closed form
    K = 1025
    c = np.full((2, K), 8355711, np.int32)
    c[1] = -8355711
    a = np.ones((1, K), np.int64)
    a[0, 2::2] = -1
    a[0, 0] = 2**31 - 1
    y = oracle.wide_gemm(c, a.astype(np.int32))
    assert y[0, 0] == 8355711 * (2**31 - 1) and y[0, 1] == -8355711 * (2**31 - 1)
