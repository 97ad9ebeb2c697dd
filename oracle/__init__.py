"""CPU oracle for the exact-integer block-quantized projection.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The product library
never loads it, and it shares no code with the GPU path: the C part
(``oracle.c``) and the Python parts here are written from the pages'
definitions alone.

Sources, cited by page title and section:
  [UORLUT01]  "D11 integer table serving (UORLUT01)", "How it works".
  [Handshake] "Vendor-Invariant Integer Inference for MindChain: Handshake v0",
              Claims C1-C4, "Construction".
  [tritify]   "Deterministic, Reproducible Inference in Exact Integer
              Arithmetic, and Verifiable Distributed Inference as Its
              Consequence" (arXiv 2611.13730), sections 3.1, 3.2, 3.4, 4.

Parity status of each function and the test that pins it:
  q8          brute force with Python integers, reductions to numpy integer
              matmul, crafted rounding ties, schedule invariance
              (test_oracle_pins.py, test_oracle_mutations.py);
  q4          brute force, m = 1 / e = 0 reductions, the table-read
              derivation;
  silu_lut, silu_mul   closed forms, float64 and page clip figures, brute force;
  limb_split  exhaustive over the 3-limb range, and with the 4-bit offset
              over the whole int16 range;
  q4_row_offsets       equal to q4 at x = 128 everywhere, and the two-limb
              form (q4 of each digit vector, weighted, plus the offsets)
              equal to q4, with planted mistakes caught
              (test_q4_row_offsets_*, test_q4_offset_mutants_are_caught);
  ffn_layer   composed from brute-force q8 and silu_mul (test_ffn_layer_*);
  ffn_layer_prenorm    composed from a Fraction/Decimal RMSNorm and brute-force
              q8 and silu_mul, with planted mistakes (residual from the norm,
              skipped norm, misindexed norm weight) caught
              (test_ffn_layer_prenorm_*);
  moe_pairs   per-pair brute force on tiny shapes with unsorted and repeated
              experts, with planted mistakes (slot for token, shifted slot,
              transposed route, swapped gate and up) caught (test_moe_pairs_*);
  topk_route  brute force with ties; requant, rms_inverse, rmsnorm_q16
              exact rationals and decimal square roots; wide_gemm brute force;
  q8_fp32     (the float negative control) every order against numpy float32
              sequences, the shuffled order with a splitmix64 / Fisher-Yates
              of the test's own (test_fp32_shadow_*).
"""
from __future__ import annotations

import ctypes
import hashlib
import math
import os
import subprocess
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORDERS = {
    "canonical": 0, "reversed": 1, "tiled_shuffled": 2, "split_k": 3,
    "tree_walk": 4, "row_order": 5, "column_stream": 6,
}
SCHEDULES = ("canonical", "reversed", "tiled_shuffled", "split_k", "tree_walk")
MULS = {"native": 0, "radix16": 1}
ORC_OK, ORC_EINVAL, ORC_ERANGE, ORC_ENOMEM = 0, 1, 2, 3


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (plain scalar C, no vectorizer)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=c11", "-O2", "-fno-tree-vectorize", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


@lru_cache(maxsize=1)
def _lib() -> ctypes.CDLL:
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.orc_q8.argtypes = [P, P, P, P, P, I64, I64, I64, I, ctypes.c_uint64, I, I]
    lib.orc_q4.argtypes = [P, P, P, P, I64, I64, I64, I, I]
    lib.orc_silu_mul.argtypes = [P, P, P, P, I64]
    lib.orc_limb_split.argtypes = [P, P, I64, I]
    lib.orc_q8_fp32.argtypes = [P, P, P, P, I64, I64, I64, I, ctypes.c_uint64]
    lib.orc_mul128_radix16.argtypes = [ctypes.c_uint64] * 4 + [P]
    lib.orc_mul128_radix16.restype = None
    for f in ("orc_q8", "orc_q4", "orc_silu_mul", "orc_limb_split", "orc_q8_fp32"):
        getattr(lib, f).restype = I
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _check(st: int, what: str) -> None:
    if st == ORC_ERANGE:
        raise OracleError(f"{what}: result outside int64 (ERANGE)")
    if st != ORC_OK:
        raise OracleError(f"{what}: status {st}")


def q8(codes: np.ndarray, scales: np.ndarray, x: np.ndarray, order: str = "canonical",
       seed: int = 0xE1, mul: str = "native", threads: int = 1) -> np.ndarray:
    """y[t][i] = floor((sum_b S[i][b] sum_{j in b} q[i][j] x[t][j] + 2^23) / 2^24).

    codes int8 [N][K], scales int32 [N][K/32], x int64 [T][K] -> int64 [T][N].
    [UORLUT01] "One projection (definition)"; [Handshake] C1 / "The frozen
    profile" (Q24 block scales, Q16 int64 activations, exact accumulation).
    """
    codes, scales, x = _c(codes, np.int8), _c(scales, np.int32), _c(x, np.int64)
    N, K = codes.shape
    T = x.shape[0]
    assert x.shape == (T, K) and scales.shape == (N, K // 32)
    y = np.zeros((T, N), dtype=np.int64)
    st = _lib().orc_q8(codes.ctypes.data, scales.ctypes.data, x.ctypes.data, y.ctypes.data, None,
                       N, K, T, ORDERS[order], seed, MULS[mul], threads)
    _check(st, "q8")
    return y


def q4(nib: np.ndarray, sme: np.ndarray, x: np.ndarray, derivation: str = "definition",
       threads: int = 1) -> np.ndarray:
    """y[t][i] = sum_g m 2^e sum_{j in g} q[i][j] x[t][j], exact, no rounding.

    nib uint8 [N][K/2], sme uint8 [N][K/32], x int32 [T][K] -> int64 [T][N].
    derivation "definition" or "table_read" ([UORLUT01] "One projection").
    """
    nib, sme, x = _c(nib, np.uint8), _c(sme, np.uint8), _c(x, np.int32)
    N = nib.shape[0]
    K = nib.shape[1] * 2
    T = x.shape[0]
    assert x.shape == (T, K) and sme.shape == (N, K // 32)
    y = np.zeros((T, N), dtype=np.int64)
    st = _lib().orc_q4(nib.ctypes.data, sme.ctypes.data, x.ctypes.data, y.ctypes.data,
                       N, K, T, {"definition": 0, "table_read": 1}[derivation], threads)
    _check(st, "q4")
    return y


Q4_OFFSET = 128


def q4_row_offsets(nib: np.ndarray, sme: np.ndarray, offset: int = Q4_OFFSET) -> np.ndarray:
    """R[i] = offset * sum_j m 2^e q[i][j], the row's weight sum times offset.

    The 4-bit projection ([UORLUT01] "One projection (definition)") is linear
    in x, so with x' = x - offset every output is y = sum_j w x' + R[i].  For
    int32 activations in [-2^15, 2^15), x - 128 lies in [-32896, 32639], the
    exact range of two balanced base-256 digits, which is what lets the 4-bit
    projection run on two activation limbs instead of three.
    nib uint8 [N][K/2], sme uint8 [N][K/32] -> int64 [N].  Group sums of q are
    at most 256 in magnitude, a group term m 2^e sum q below 2^27, the row sum
    below 2^40 for K <= 262144, so int64 holds every step.
    """
    nib, sme = _c(nib, np.uint8), _c(sme, np.uint8)
    N, K = nib.shape[0], nib.shape[1] * 2
    assert sme.shape == (N, K // 32) and abs(offset) <= 128
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = nib & 15          # element 2j: low nibble of byte j
    q[:, 1::2] = nib >> 4
    q = np.where(q >= 8, q - 16, q)   # two's-complement nibbles
    m = (sme & 15).astype(np.int64)
    e = (sme >> 4).astype(np.int64)
    groups = q.reshape(N, K // 32, 32).sum(axis=2)
    return np.int64(offset) * ((m * groups) << e).sum(axis=1)


def silu_mul(g: np.ndarray, u: np.ndarray, lut: np.ndarray) -> np.ndarray:
    """h = floor(LUT[clamp(floor((g+16)/32), +-32768) + 32768] * u / 2^16)."""
    g, u, lut = _c(g, np.int64), _c(u, np.int64), _c(lut, np.int32)
    assert g.shape == u.shape and lut.shape == (65537,)
    h = np.zeros(g.shape, dtype=np.int64)
    _check(_lib().orc_silu_mul(g.ctypes.data, u.ctypes.data, lut.ctypes.data, h.ctypes.data, g.size), "silu_mul")
    return h


def limb_split(x: np.ndarray, L: int, offset: int = 0) -> tuple[np.ndarray, bool]:
    """Balanced base-256 digits d [L][n] in [-128, 127], x - offset = sum 256^l d_l.

    offset 0 is the plain split; the two-limb form of the 4-bit projection
    splits x - Q4_OFFSET (see q4_row_offsets).  Returns (digits, in_range)."""
    x = _c(x.reshape(-1), np.int64)
    if offset:
        lo, hi = -(2**63) + max(offset, 0), 2**63 - 1 + min(offset, 0)
        if x.size and (int(x.min()) < lo or int(x.max()) > hi):
            raise OracleError("limb_split: x - offset leaves int64")
        x = x - np.int64(offset)
    d = np.zeros((L, x.size), dtype=np.int8)
    st = _lib().orc_limb_split(x.ctypes.data, d.ctypes.data, x.size, L)
    if st not in (ORC_OK, ORC_ERANGE):
        raise OracleError(f"limb_split: status {st}")
    return d, st == ORC_OK


def q8_fp32(codes: np.ndarray, scales: np.ndarray, x: np.ndarray, order: str = "canonical",
            seed: int = 0xE1) -> np.ndarray:
    """The float32 shadow of the Q8 sum in one schedule's order ([Handshake] C3)."""
    codes, scales, x = _c(codes, np.int8), _c(scales, np.int32), _c(x, np.int64)
    N, K = codes.shape
    T = x.shape[0]
    y = np.zeros((T, N), dtype=np.float32)
    _check(_lib().orc_q8_fp32(codes.ctypes.data, scales.ctypes.data, x.ctypes.data, y.ctypes.data,
                              N, K, T, ORDERS[order], seed), "q8_fp32")
    return y


def mul128_radix16(a: int, b: int) -> int:
    """The C oracle's radix-16 multiples-table product of two unsigned 128-bit
    values, mod 2^128 ([UORLUT01] "Products of two runtime values")."""
    m = (1 << 64) - 1
    out = (ctypes.c_uint64 * 2)()
    _lib().orc_mul128_radix16(a & m, (a >> 64) & m, b & m, (b >> 64) & m, out)
    return out[0] | (out[1] << 64)


@lru_cache(maxsize=1)
def silu_lut() -> np.ndarray:
    """The 65537-entry SiLU table: LUT[k + 32768] = round(silu(k / 2^11) * 2^16).

    [Handshake] C1 and C4: a table committed in decimal, Q11 input over +-16,
    Q16 output.  silu(z) = z / (1 + e^-z), evaluated here with 50-digit
    decimal arithmetic and rounded to the nearest integer; the only exact
    half-way case would need silu(z) 2^16 to be a half-integer, which does
    not occur (checked by the tests), so the tie rule never acts.
    """
    from decimal import Decimal, getcontext, ROUND_HALF_EVEN
    getcontext().prec = 50
    out = np.empty(65537, dtype=np.int32)
    scale = Decimal(65536)
    for k in range(-32768, 32769):
        z = Decimal(k) / Decimal(2048)
        v = z / (Decimal(1) + (-z).exp()) * scale
        out[k + 32768] = int(v.to_integral_value(rounding=ROUND_HALF_EVEN))
    out.setflags(write=False)
    return out


def digest(a: np.ndarray) -> str:
    """SHA-256 of the array's raw little-endian bytes, row-major, no header."""
    a = np.ascontiguousarray(a)
    return hashlib.sha256(a.astype(a.dtype.newbyteorder("<"), copy=False).tobytes()).hexdigest()


def ffn_layer(x: np.ndarray, wg, wu, wd, lut: np.ndarray, threads: int = 1):
    """One Q8 FFN layer: g = Q8(Wg, x), u = Q8(Wu, x), h = silu(g)*u >> 16,
    d = Q8(Wd, h), x_next = x + d (a residual stream; the pages' per-layer
    digests come from a residual transformer, [Handshake] C2).

    wg, wu, wd are (codes, scales) pairs.  Returns (g, u, h, d, x_next)."""
    g = q8(wg[0], wg[1], x, threads=threads)
    u = q8(wu[0], wu[1], x, threads=threads)
    h = silu_mul(g, u, lut)
    d = q8(wd[0], wd[1], h, threads=threads)
    xn = add_i64(x, d)
    return g, u, h, d, xn


def add_i64(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a + b elementwise for int64 arrays, raising OracleError if a sum leaves
    int64 (numpy's own add would wrap without a word)."""
    a, b = np.asarray(a, np.int64), np.asarray(b, np.int64)
    s = a + b   # wraps on overflow; detected below
    over = ((a >= 0) == (b >= 0)) & ((s >= 0) != (a >= 0))
    if over.any():
        raise OracleError("add_i64: sum outside int64")
    return s


def requant(c, m: int, k: int):
    """Fixed-point requantization round(c * m / 2^k), rounding half away from
    zero ([tritify] 3.1, arithmetic specification: a 128-bit product, then a
    round-half-away-from-zero arithmetic shift).  c: int array or int; Python
    integers throughout (the exact product).  Returns int64 values; raises if
    one does not fit."""
    def one(v: int) -> int:
        p = int(v) * int(m)
        if k == 0:
            r = p
        else:
            a = (abs(p) + (1 << (k - 1))) >> k
            r = a if p >= 0 else -a
        if not -(1 << 63) <= r < (1 << 63):
            raise OracleError("requant: result outside int64")
        return r
    if np.ndim(c) == 0:
        return one(c)
    return np.array([one(v) for v in np.asarray(c).ravel()], np.int64).reshape(np.shape(c))


RMS_SHIFT = 52   # inverse-RMS fixed point: 2^52 / rms, at least 2^29 for |x| <= 2^23


def rms_inverse(ss: int, d: int, eps_q32: int) -> int:
    """The integer inverse-RMS of a row ([tritify] 3.2 Normalization: an exact
    integer sum of squares and an integer inverse square root folded into a
    scale).  Reading: for Q16 codes X with ss = sum X^2, the real mean square
    plus eps is (ss / d + eps_q32) / 2^32, and the scale is
    inv = floor(sqrt(2^(2*52) * d / (ss + d * eps_q32))), i.e. 2^52 / rms in the
    codes' units, by math.isqrt of the exact floor of the rational."""
    return math.isqrt(((1 << (2 * RMS_SHIFT)) * d) // (ss + d * eps_q32))


def rmsnorm_q16(x: np.ndarray, g: np.ndarray, eps_q32: int) -> np.ndarray:
    """Integer RMSNorm of Q16 rows: Y_i = round_half_away(X_i * G_i * inv / 2^52)
    with G the Q16 norm weight and inv = rms_inverse(sum X^2, d, eps), i.e.
    Y = X * G / sqrt(mean(X^2) + eps * 2^32) in Q16, the scale applied by one
    requantization ([tritify] 3.1, 3.2).  x int64 [T][d], g int32 [d],
    eps_q32 >= 1.  Returns int64 [T][d]."""
    T, d = x.shape
    out = np.empty((T, d), np.int64)
    gi = [int(v) for v in g]
    for t in range(T):
        row = [int(v) for v in x[t]]
        inv = rms_inverse(sum(v * v for v in row), d, int(eps_q32))
        out[t] = [requant(row[i] * gi[i], inv, RMS_SHIFT) for i in range(d)]
    return out


WIDE_TRITS = 12
WIDE_CODE_MAX = (3 ** WIDE_TRITS - 1) // 2   # 265,720


def wide_gemm(codes: np.ndarray, acts: np.ndarray) -> np.ndarray:
    """The wide-code linear kernel ([tritify] 3.1 and 3.2 Matmul: weights are
    integer codes of b = 12 balanced trits, activations int32 codes, the
    products i32 x i32 accumulated exactly; no rounding):
        y[t][i] = sum_j codes[i][j] * acts[t][j]
    codes int32 [N][K], acts int32 [T][K]; returns int64 [T][N].  numpy's
    int64 matmul is exact when sum_j |c| |a| < 2^63, which is checked first;
    otherwise Python integers are used (and the result must fit int64)."""
    c = np.asarray(codes, np.int64)
    a = np.asarray(acts, np.int64)
    bound = int(np.abs(c).max(initial=0)) * int(np.abs(a).max(initial=0)) * c.shape[1]
    if bound < (1 << 63):
        return a @ c.T
    out = np.empty((a.shape[0], c.shape[0]), np.int64)
    cl, al = c.tolist(), a.tolist()
    for t in range(a.shape[0]):
        for i in range(c.shape[0]):
            v = sum(x * y for x, y in zip(cl[i], al[t]))
            if not -(1 << 63) <= v < (1 << 63):
                raise OracleError("wide_gemm: result outside int64")
            out[t, i] = v
    return out


def topk_route(scores: np.ndarray, k: int) -> np.ndarray:
    """Integer top-k routing ([tritify] 3.2 "Mixture-of-Experts": the router
    scores the experts in integer, the top-k selection compares integers and
    breaks ties by index).  Reading: slot s of token t holds the expert of rank
    s in the order (score descending, expert index ascending).

    scores: int64 [T][E]; returns int32 [T][k].  Python integers throughout,
    so the int64 ends compare without overflow."""
    T, E = scores.shape
    if not 1 <= k <= E:
        raise OracleError(f"topk_route: need 1 <= k <= E, got k={k}, E={E}")
    out = np.empty((T, k), np.int32)
    for t in range(T):
        row = [int(v) for v in scores[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        out[t] = order[:k]
    return out


def ffn_layer_prenorm(x: np.ndarray, g_norm: np.ndarray, eps_q32: int, wg, wu, wd, lut: np.ndarray,
                      threads: int = 1):
    """The pre-norm residual block: n = rmsnorm_q16(x, g_norm, eps), then
    ffn_layer's gate, up, SiLU product and down projection on n, and
    x_next = x + d (the residual from the un-normalized x).  Returns
    (n, d, x_next)."""
    n = rmsnorm_q16(x, g_norm, eps_q32)
    _, _, _, d, _ = ffn_layer(n, wg, wu, wd, lut, threads=threads)
    return n, d, add_i64(x, d)


def moe_pairs(x: np.ndarray, route: np.ndarray, experts, lut: np.ndarray, pairs=None,
              down_rows=None, threads: int = 1) -> np.ndarray:
    """Routed expert FFNs: out[p] = Wd_e (silu(Wg_e x_t) * (Wu_e x_t) >> 16)
    for pair p = (t, k) and e = route[t][k] ([tritify] 3.2 "Mixture-of-Experts":
    each selected expert is an exact-integer MLP).  No combine: the router
    weights are not part of this workload.

    experts(e) -> ((gc, gs), (uc, us), (dc, ds)).  pairs: optional list of
    (t, k) to compute (default: every pair, t-major); down_rows: optional
    subset of output rows.  Returns an int64 array [len(pairs)][n_rows].

    The pairs of one expert go through q8 together, one activation row per
    pair: every output of q8 depends on its own row alone, so this is the
    per-pair definition evaluated a batch at a time."""
    T, topk = route.shape
    if pairs is None:
        pairs = [(t, k) for t in range(T) for k in range(topk)]
    by_expert = {}
    for p, (t, k) in enumerate(pairs):
        by_expert.setdefault(int(route[t, k]), []).append(p)
    out = None
    for e in sorted(by_expert):
        idx = by_expert[e]
        (gc, gs), (uc, us), (dc, ds) = experts(e)
        if down_rows is not None:
            dc, ds = dc[down_rows], ds[down_rows]
        xe = x[[pairs[p][0] for p in idx]]
        g = q8(gc, gs, xe, threads=threads)
        u = q8(uc, us, xe, threads=threads)
        h = silu_mul(g, u, lut)
        d = q8(dc, ds, h, threads=threads)
        if out is None:
            out = np.zeros((len(pairs), d.shape[1]), np.int64)
        out[idx] = d
    return out if out is not None else np.zeros((0, 0), np.int64)
