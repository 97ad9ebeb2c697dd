"""Pins of the oracle's composed functions (CPU only).

moe_pairs and ffn_layer_prenorm are built from pieces that are pinned on
their own (q8, silu_mul, rmsnorm_q16); what can still go wrong is the
composition: which activation row a pair reads, which expert a slot names,
which operand is the gate, where the residual comes from.  Each is checked
here against a per-pair / per-row brute force with Python integers, and a
planted mistake of each kind, made in a copy of the oracle function's source,
must fail the same check.  The float32 shadow's split_k and tiled_shuffled
orders are pinned against numpy float32 sequences, the shuffled order drawn
with a splitmix64 / Fisher-Yates written here from the published definition.

Sources: [tritify] 3.2 "Mixture-of-Experts" and "Normalization";
[Handshake] C3 (the float negative control of the schedule gate).
"""
import inspect
import zlib
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import bigint


def _rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def _mutant(fn, old, new):
    """A copy of oracle function `fn` with `old` replaced by `new` in its
    source, compiled in the oracle module's namespace."""
    src = inspect.getsource(fn)
    assert old in src, (fn.__name__, old)
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


# ------------------------------------------------------------ routed experts

E, D, F, T, TOPK = 5, 64, 96, 4, 3
# unsorted slots, an expert repeated within a token, one token on one expert
ROUTE = np.array([[3, 1, 3], [0, 4, 2], [2, 2, 2], [4, 0, 1]], np.int32)


def _experts():
    r = _rng("moe-experts")
    mats = []
    for _ in range(E):
        mats.append(((synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                     (synth.q8_codes(r, F, D), synth.q8_scales(r, F, D)),
                     (synth.q8_codes(r, D, F), synth.q8_scales(r, D, F))))
    return mats


def _moe_brute(x, route, mats, lut, pairs, down_rows=None):
    out = []
    lutl = lut.tolist()
    for t, k in pairs:
        (gc, gs), (uc, us), (dc, ds) = mats[int(route[t][k])]
        xt = [x[t].tolist()]
        g = bigint.q8(gc.tolist(), gs.tolist(), xt)[0]
        u = bigint.q8(uc.tolist(), us.tolist(), xt)[0]
        h = bigint.silu_mul(g, u, lutl)
        if down_rows is not None:
            dc, ds = dc[down_rows], ds[down_rows]
        out.append(bigint.q8(dc.tolist(), ds.tolist(), [h])[0])
    return out


def _moe_checks(moe_pairs, lut, mats, x) -> bool:
    every = [(t, k) for t in range(T) for k in range(TOPK)]
    if moe_pairs(x, ROUTE, lambda e: mats[e], lut).tolist() != _moe_brute(x, ROUTE, mats, lut, every):
        return False
    # a subset of pairs in a scrambled order, and a subset of down rows
    pairs = [(3, 2), (0, 0), (2, 1), (0, 2), (1, 1)]
    rows = [0, 5, 63, 17]
    got = moe_pairs(x, ROUTE, lambda e: mats[e], lut, pairs=pairs, down_rows=rows)
    return got.tolist() == _moe_brute(x, ROUTE, mats, lut, pairs, rows)


@pytest.fixture(scope="module")
def moe_case():
    mats = _experts()
    x = synth.q16_acts(_rng("moe-x"), T, D)
    return mats, x


def test_moe_pairs_matches_per_pair_brute_force(lut, moe_case):
    mats, x = moe_case
    assert _moe_checks(oracle.moe_pairs, lut, mats, x)


MOE_MUTANTS = {
    "slot_for_token": ("xe = x[[pairs[p][0] for p in idx]]", "xe = x[[pairs[p][1] for p in idx]]"),
    "shifted_slot": ("by_expert.setdefault(int(route[t, k]), [])",
                     "by_expert.setdefault(int(route[t, (k + 1) % topk]), [])"),
    "transposed_route": ("by_expert.setdefault(int(route[t, k]), [])",
                         "by_expert.setdefault(int(route.ravel()[k * T + t]), [])"),
    "gate_and_up_swapped": ("h = silu_mul(g, u, lut)", "h = silu_mul(u, g, lut)"),
    "down_on_gate": ("d = q8(dc, ds, h, threads=threads)", "d = q8(dc, ds, g, threads=threads)"),
}


@pytest.mark.parametrize("name", sorted(MOE_MUTANTS))
def test_moe_pairs_mutant_is_caught(lut, moe_case, name):
    mats, x = moe_case
    old, new = MOE_MUTANTS[name]
    bad = _mutant(oracle.moe_pairs, old, new)
    try:
        ok = _moe_checks(bad, lut, mats, x)
    except (IndexError, oracle.OracleError, ValueError):
        ok = False
    assert not ok, name


# --------------------------------------------------- pre-norm residual block

def _rmsnorm_rational(x, g, eps_q32):
    """RMSNorm of Q16 rows with exact rationals: inv = floor of the real
    sqrt(2^104 d / (sum X^2 + d eps)) (Decimal square root, its floor checked
    by squaring), Y = X G inv / 2^52 rounded half away from zero (Fraction)."""
    getcontext().prec = 100
    out = []
    d = len(g)
    for row in x.tolist():
        den = sum(v * v for v in row) + d * eps_q32
        inv = int((Decimal(2**104) * d / den).sqrt())
        while inv * inv * den > 2**104 * d:
            inv -= 1
        while (inv + 1) ** 2 * den <= 2**104 * d:
            inv += 1
        ys = []
        for xi, gi in zip(row, g.tolist()):
            v = Fraction(xi * gi * inv, 2**52)
            a = int(abs(v) + Fraction(1, 2))
            ys.append(a if v >= 0 else -a)
        out.append(ys)
    return out


def _prenorm_brute(x, g_norm, eps, wg, wu, wd, lut):
    n = _rmsnorm_rational(x, g_norm, eps)
    gb = bigint.q8(wg[0].tolist(), wg[1].tolist(), n)
    ub = bigint.q8(wu[0].tolist(), wu[1].tolist(), n)
    hb = [bigint.silu_mul(gr, ur, lut.tolist()) for gr, ur in zip(gb, ub)]
    db = bigint.q8(wd[0].tolist(), wd[1].tolist(), hb)
    xn = [[xv + dv for xv, dv in zip(xr, dr)] for xr, dr in zip(x.tolist(), db)]
    return n, db, xn


@pytest.fixture(scope="module")
def prenorm_case():
    r = _rng("prenorm")
    d, f, t = 64, 96, 3
    wg = (synth.q8_codes(r, f, d), synth.q8_scales(r, f, d))
    wu = (synth.q8_codes(r, f, d), synth.q8_scales(r, f, d))
    wd = (synth.q8_codes(r, d, f), synth.q8_scales(r, d, f))
    x = synth.q16_acts(r, t, d)
    g = np.rint(r.normal(1.0, 0.1, d) * 2**16).astype(np.int32)
    return x, g, 4295, wg, wu, wd


def _prenorm_checks(fn, lut, case) -> bool:
    x, g, eps, wg, wu, wd = case
    n, d, xn = fn(x, g, eps, wg, wu, wd, lut)
    nb, db, xnb = _prenorm_brute(x, g, eps, wg, wu, wd, lut)
    return n.tolist() == nb and d.tolist() == db and xn.tolist() == xnb


def test_ffn_layer_prenorm_matches_rational_norm_and_brute_force(lut, prenorm_case):
    assert _prenorm_checks(oracle.ffn_layer_prenorm, lut, prenorm_case)


PRENORM_MUTANTS = {
    "residual_from_norm": ("return n, d, add_i64(x, d)", "return n, d, add_i64(n, d)"),
    "norm_skipped": ("ffn_layer(n, wg, wu, wd, lut, threads=threads)",
                     "ffn_layer(x, wg, wu, wd, lut, threads=threads)"),
    "norm_weight_reversed": ("n = rmsnorm_q16(x, g_norm, eps_q32)", "n = rmsnorm_q16(x, g_norm[::-1], eps_q32)"),
}


@pytest.mark.parametrize("name", sorted(PRENORM_MUTANTS))
def test_ffn_layer_prenorm_mutant_is_caught(lut, prenorm_case, name):
    old, new = PRENORM_MUTANTS[name]
    assert not _prenorm_checks(_mutant(oracle.ffn_layer_prenorm, old, new), lut, prenorm_case), name


def test_residual_add_overflow_is_an_error():
    a = np.array([2**62, -(2**62), 5], np.int64)
    assert oracle.add_i64(a, np.array([2**62 - 1, -(2**62), -7], np.int64)).tolist() == \
        [2**63 - 1, -(2**63), -2]
    with pytest.raises(oracle.OracleError):
        oracle.add_i64(a, np.array([2**62, 0, 0], np.int64))
    with pytest.raises(oracle.OracleError):
        oracle.add_i64(a, np.array([0, -(2**62) - 1, 0], np.int64))


# ------------------------------------------------ float32 shadow, all orders

def _shadow_operands(q, s, x):
    w = ((s.astype(np.int64).repeat(32, axis=1) * q.astype(np.int64)).astype(np.float64) * 2.0**-24) \
        .astype(np.float32)
    xf = (x.astype(np.float64) * 2.0**-16).astype(np.float32)
    return w, xf


def _seq32(v):
    """Left-to-right float32 sum starting from 0 (numpy's cumsum is sequential)."""
    return np.float32(np.cumsum(np.concatenate([[np.float32(0)], v]).astype(np.float32), dtype=np.float32)[-1])


M64 = (1 << 64) - 1


def _splitmix64(state):
    """splitmix64 (Steele, Lea and Flood, 2014): returns (new state, output)."""
    state = (state + 0x9E3779B97F4A7C15) & M64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return state, z ^ (z >> 31)


def _fisher_yates(n, seed):
    v = list(range(n))
    st = seed
    for i in range(n - 1, 0, -1):
        st, r = _splitmix64(st)
        j = r % (i + 1)
        v[i], v[j] = v[j], v[i]
    return v


def test_splitmix64_published_values():
    # the first outputs for seed 0 given with the generator's published
    # reference implementation
    st, outs = 0, []
    for _ in range(3):
        st, o = _splitmix64(st)
        outs.append(o)
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


@pytest.mark.parametrize("shape", [(5, 352, 2), (3, 1024, 1), (2, 96, 3)])
def test_fp32_shadow_split_k_is_eight_float32_partials(shape):
    N, K, Tn = shape
    q, s = synth.q8_codes(_rng("sk" + str(K)), N, K), synth.q8_scales(_rng("sks" + str(K)), N, K)
    x = synth.q16_acts(_rng("skx" + str(K)), Tn, K)
    w, xf = _shadow_operands(q, s, x)
    y = oracle.q8_fp32(q, s, x, "split_k")
    nb = K // 32
    for t in range(Tn):
        for i in range(N):
            prods = (w[i] * xf[t]).astype(np.float32)
            parts = [_seq32(prods[(p * nb // 8) * 32:((p + 1) * nb // 8) * 32]) for p in range(8)]
            a = np.float32(0)
            for p in range(7, -1, -1):
                a = np.float32(a + parts[p])
            assert a == y[t, i]


@pytest.mark.parametrize("shape,seed", [((4, 352, 2), 0xE1), ((3, 1280, 1), 12345), ((2, 64, 2), 7)])
def test_fp32_shadow_tiled_shuffled_is_a_seeded_tile_order(shape, seed):
    N, K, Tn = shape
    q, s = synth.q8_codes(_rng("ts" + str(K)), N, K), synth.q8_scales(_rng("tss" + str(K)), N, K)
    x = synth.q16_acts(_rng("tsx" + str(K)), Tn, K)
    w, xf = _shadow_operands(q, s, x)
    y = oracle.q8_fp32(q, s, x, "tiled_shuffled", seed=seed)
    order = _fisher_yates((K + 127) // 128, seed)
    cols = [j for v in order for j in range(128 * v, min(128 * v + 128, K))]
    assert sorted(cols) == list(range(K))
    for t in range(Tn):
        for i in range(N):
            prods = (w[i] * xf[t]).astype(np.float32)
            assert _seq32(prods[cols]) == y[t, i]
