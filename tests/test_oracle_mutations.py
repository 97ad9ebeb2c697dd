"""Planted mistakes in a temporary copy of the oracle must fail its pins (CPU).

Each mutation is a plausible slip (a dropped term, a wrong sign, index or
constant, a transposed operand).  The mutated copy is compiled to a
temporary library and checked against the arbitrary-precision referee and
the oracle's own cross-derivations; every mutant must be caught.  The
committed oracle is never modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import bigint

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "round_half_constant": ("floor_div_pow2(acc[e] + ((i128)1 << 23), 24)", "floor_div_pow2(acc[e] + ((i128)1 << 22), 24)"),
    "round_shift": ("floor_div_pow2(acc[e] + ((i128)1 << 23), 24)", "floor_div_pow2(acc[e] + ((i128)1 << 23), 23)"),
    "floor_as_trunc": ("if (a % d != 0 && a < 0) q -= 1;", ""),
    "dropped_column": ("for (int jj = 0; jj < 32; ++jj) {", "for (int jj = 0; jj < 31; ++jj) {"),
    "block_stride": ("const int8_t* qi = jb->q + i * jb->K + b * 32;", "const int8_t* qi = jb->q + i * jb->K + b * 16;"),
    "scale_index": ("return mul((i128)jb->s[i * jb->nb + b], block_dot", "return mul((i128)jb->s[(i * jb->nb + b + 1) % (jb->N * jb->nb)], block_dot"),
    "column_swap": ("m += mul((i128)jb->x[t * jb->K + j], (i128)jb->q[i * jb->K + j], jb->mul_mode);",
                    "m += mul((i128)jb->x[t * jb->K + (j ^ 1)], (i128)jb->q[i * jb->K + j], jb->mul_mode);"),
    "split_k_dropped_partial": ("for (int p = 7; p >= 0; --p) a += part[p];", "for (int p = 7; p >= 1; --p) a += part[p];"),
    "tree_odd_lost": ("if (n & 1) terms[m++] = terms[n - 1];", "if (n & 1) m++;"),
    "radix16_digit": ("r += table[(int)(b & 15)] << (4 * k);", "r += table[(int)(b & 15)] << (3 * k);"),
    "q4_nibble_order": ("int c = (nib[i * (K / 2) + j / 2] >> (4 * (j & 1))) & 0xF;",
                        "int c = (nib[i * (K / 2) + j / 2] >> (4 * ((j + 1) & 1))) & 0xF;"),
    "q4_sign": ("return c >= 8 ? c - 16 : c;", "return c > 8 ? c - 16 : c;"),
    "q4_exponent": ("i128 sc = (i128)q4_mant(jb->sme, jb->ng, i, g) * ((i128)1 << q4_expo(jb->sme, jb->ng, i, g));",
                    "i128 sc = (i128)q4_mant(jb->sme, jb->ng, i, g) * ((i128)1 << q4_mant(jb->sme, jb->ng, i, g));"),
    "q4_table_sign": ("for (int v = 7; v >= 0; --v) tab[v] = tab[v + 1] - xj;", "for (int v = 7; v >= 0; --v) tab[v] = tab[v + 1] + xj;"),
    "silu_index_half": ("i128 idx = floor_div_pow2((i128)g[e] + 16, 5);", "i128 idx = floor_div_pow2((i128)g[e] + 15, 5);"),
    "silu_clamp": ("if (idx > 32768) idx = 32768;", "if (idx > 32767) idx = 32767;"),
    "silu_out_shift": ("i128 v = floor_div_pow2((i128)lut[(int64_t)idx + 32768] * (i128)u[e], 16);",
                       "i128 v = floor_div_pow2((i128)lut[(int64_t)idx + 32768] * (i128)u[e], 15);"),
    "limb_digit": ("i128 m = (r + 128) % 256;", "i128 m = (r + 127) % 256;"),
}


def _compile(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-pthread", str(src), "-o", str(lib)], check=True)
    L = ctypes.CDLL(str(lib))
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.orc_q8.argtypes = [P, P, P, P, P, I64, I64, I64, I, ctypes.c_uint64, I, I]
    L.orc_q4.argtypes = [P, P, P, P, I64, I64, I64, I, I]
    L.orc_silu_mul.argtypes = [P, P, P, P, I64]
    L.orc_limb_split.argtypes = [P, P, I64, I]
    return L


def _pins_hold(L, lut) -> bool:
    """A compact run of the oracle's pins against library L; False on any miss."""
    r = np.random.default_rng(11)
    N, K, T = 5, 320, 3          # 10 blocks: every one of the 8 split-K ranges is non-empty
    q = r.integers(-128, 128, size=(N, K)).astype(np.int8)
    s = r.integers(-(2**20), 2**20, size=(N, K // 32)).astype(np.int32)
    x = r.integers(-(2**30), 2**30, size=(T, K)).astype(np.int64)
    yb = np.array(bigint.q8(q.tolist(), s.tolist(), x.tolist()), dtype=np.int64)
    for order in range(7):
        for mul in (0, 1):
            y = np.zeros((T, N), np.int64)
            st = L.orc_q8(q.ctypes.data, s.ctypes.data, x.ctypes.data, y.ctypes.data, None, N, K, T, order, 0xE1, mul, 1)
            if st != 0 or not (y == yb).all():
                return False
    # rounding ties
    for k in (-3, 0, 2):
        qq = np.zeros((1, 32), np.int8); qq[0, 0] = 1
        ss = np.ones((1, 1), np.int32)
        xx = np.zeros((1, 32), np.int64); xx[0, 0] = (2 * k + 1) * 2**23
        y = np.zeros((1, 1), np.int64)
        L.orc_q8(qq.ctypes.data, ss.ctypes.data, xx.ctypes.data, y.ctypes.data, None, 1, 32, 1, 0, 0, 0, 1)
        if y[0, 0] != k + 1:
            return False
    # Q4: both derivations against the referee
    nib = r.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    sme = r.integers(0, 256, size=(N, K // 32)).astype(np.uint8)
    x4 = r.integers(-(2**31), 2**31, size=(T, K)).astype(np.int32)
    y4b = np.array(bigint.q4(nib.tolist(), sme.tolist(), x4.tolist()), dtype=np.int64)
    for der in (0, 1):
        y4 = np.zeros((T, N), np.int64)
        if L.orc_q4(nib.ctypes.data, sme.ctypes.data, x4.ctypes.data, y4.ctypes.data, N, K, T, der, 1) != 0 or not (y4 == y4b).all():
            return False
    # SiLU epilogue, including both clip sides
    g = np.concatenate([r.integers(-(2**21), 2**21, 300), [2**22, -(2**22), 16, -17]]).astype(np.int64)
    u = r.integers(-(2**30), 2**30, g.size).astype(np.int64)
    h = np.zeros(g.size, np.int64)
    L.orc_silu_mul(g.ctypes.data, u.ctypes.data, lut.ctypes.data, h.ctypes.data, g.size)
    if h.tolist() != bigint.silu_mul(g.tolist(), u.tolist(), lut.tolist()):
        return False
    # limbs
    xs = np.concatenate([r.integers(-(2**22), 2**22, 500), [8355711, -8421504]]).astype(np.int64)
    d = np.zeros((3, xs.size), np.int8)
    if L.orc_limb_split(xs.ctypes.data, d.ctypes.data, xs.size, 3) != 0:
        return False
    rec = d[0].astype(np.int64) + 256 * d[1].astype(np.int64) + 65536 * d[2].astype(np.int64)
    return bool((rec == xs).all())


def test_unmutated_copy_passes(tmp_path, lut):
    assert _pins_hold(_compile(tmp_path, "orig", open(SRC).read()), lut)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(tmp_path, lut, name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    assert not _pins_hold(_compile(tmp_path, name, text.replace(old, new)), lut)


# --------------------------------------------- top-k routing (Python oracle)

def _topk_checks(topk) -> bool:
    """The routing pins, applied to a candidate implementation."""
    import itertools
    r = np.random.default_rng(33)
    for _ in range(60):
        E = int(r.integers(1, 6))
        k = int(r.integers(1, E + 1))
        sc = r.integers(-2, 3, (1, E)).astype(np.int64)
        row = sc[0].tolist()
        want = next(list(p[:k]) for p in itertools.permutations(range(E))
                    if all(row[p[i]] > row[p[j]] or (row[p[i]] == row[p[j]] and p[i] < p[j])
                           for i in range(E) for j in range(i + 1, E)))
        if topk(sc, k)[0].tolist() != want:
            return False
    return True


def _topk_mutant(key):
    def f(scores, k):
        out = np.empty((scores.shape[0], k), np.int32)
        for t in range(scores.shape[0]):
            row = [int(v) for v in scores[t]]
            out[t] = sorted(range(len(row)), key=lambda e: key(row, e))[:k]
        return out
    return f


@pytest.mark.parametrize("name,key", [
    ("ties_to_higher_index", lambda row, e: (-row[e], -e)),
    ("ascending_scores", lambda row, e: (row[e], e)),
    ("index_only", lambda row, e: e),
])
def test_topk_mutants_are_caught(name, key):
    assert _topk_checks(oracle.topk_route)
    assert not _topk_checks(_topk_mutant(key)), name


# ------------------------------------ requantization and RMSNorm (Python oracle)

def _rms_checks(requant, rms_inverse) -> bool:
    """The requant / inverse-RMS pins, applied to candidate implementations."""
    from decimal import Decimal, getcontext
    from fractions import Fraction
    import math
    getcontext().prec = 80
    r = np.random.default_rng(44)
    for v in (1, 3, 5, 7, -1, -3, -5, -7):   # exact halves
        if requant(v, 1, 1) != (abs(v) + 1) // 2 * (1 if v > 0 else -1):
            return False
    for _ in range(300):
        c, m, k = int(r.integers(-(2**40), 2**40)), int(r.integers(1, 2**40)), int(r.integers(24, 60))
        fr = Fraction(c * m, 2**k)
        want = int(abs(fr) + Fraction(1, 2)) * (1 if fr >= 0 else -1)
        if requant(c, m, k) != want:
            return False
    for _ in range(300):
        d, eps = int(r.integers(1, 3000)), int(r.integers(1, 2**32))
        ss = int(r.integers(0, d * 2**44))
        if rms_inverse(ss, d, eps) != int((Decimal(2**104) * d / (ss + d * eps)).sqrt()):
            return False
    return True


def _requant_half_even(c, m, k):
    from fractions import Fraction
    return round(Fraction(int(c) * int(m), 2**k))     # Python rounds half to even


def _requant_floor(c, m, k):
    return (int(c) * int(m)) >> k


def _rms_no_d(ss, d, eps):
    import math
    return math.isqrt((1 << 104) // (ss + d * eps))


def _rms_eps_unscaled(ss, d, eps):
    import math
    return math.isqrt(((1 << 104) * d) // (ss + eps))


@pytest.mark.parametrize("name", ["half_even", "floor", "no_d", "eps_unscaled"])
def test_rms_mutants_are_caught(name):
    assert _rms_checks(oracle.requant, oracle.rms_inverse)
    rq = {"half_even": _requant_half_even, "floor": _requant_floor}.get(name, oracle.requant)
    ri = {"no_d": _rms_no_d, "eps_unscaled": _rms_eps_unscaled}.get(name, oracle.rms_inverse)
    assert not _rms_checks(rq, ri), name


# ------------------------------------------- 4-bit row offsets (Python oracle)

def _q4_offset_checks(row_offsets) -> bool:
    """The row-offset pins, applied to a candidate implementation."""
    r = np.random.default_rng(45)
    for N, K in ((3, 32), (9, 96)):
        nib = r.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
        sme = (r.integers(0, 16, size=(N, K // 32)) | (r.integers(0, 16, size=(N, K // 32)) << 4)).astype(np.uint8)
        if not (oracle.q4(nib, sme, np.full((1, K), 128, np.int32))[0] == row_offsets(nib, sme)).all():
            return False
    return True


def _roff_mutant(kind):
    def f(nib, sme):
        N, K = nib.shape[0], nib.shape[1] * 2
        q = np.empty((N, K), dtype=np.int64)
        q[:, 0::2], q[:, 1::2] = nib & 15, nib >> 4
        q = np.where(q > 8 if kind == "sign" else q >= 8, q - 16, q)
        sm = np.roll(sme, 1, axis=1) if kind == "scale_group" else sme
        m = (sm & 15).astype(np.int64)
        e = (sm >> 4).astype(np.int64)
        g = q.reshape(N, K // 32, 32).sum(axis=2)
        if kind == "exponent":
            return 128 * (m * g).sum(axis=1)
        return (127 if kind == "offset" else 128) * ((m * g) << e).sum(axis=1)
    return f


@pytest.mark.parametrize("kind", ["scale_group", "sign", "exponent", "offset"])
def test_q4_offset_mutants_are_caught(kind):
    assert _q4_offset_checks(oracle.q4_row_offsets)
    assert not _q4_offset_checks(_roff_mutant(kind)), kind
