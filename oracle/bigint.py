"""Arbitrary-precision referee for tiny inputs (pure Python integers).

TEST INFRASTRUCTURE ONLY.  These functions restate the same definitions as
``oracle.c`` with Python's unbounded integers and loops, so that the C
oracle's 128-bit arithmetic, indexing and rounding can be checked by brute
force on small shapes.  Sources as in ``oracle/__init__.py``.
"""
from __future__ import annotations


def q8(codes, scales, x):
    """[UORLUT01] "One projection (definition)" with [Handshake] C1's Q24
    scales and Q16 activations; rounding: add 2^23, floor-divide by 2^24.
    Python's >> on negative integers is a floor shift."""
    N, K = len(codes), len(codes[0])
    T = len(x)
    y = [[0] * N for _ in range(T)]
    for t in range(T):
        for i in range(N):
            acc = 0
            for b in range(K // 32):
                p = sum(int(codes[i][j]) * int(x[t][j]) for j in range(32 * b, 32 * b + 32))
                acc += int(scales[i][b]) * p
            y[t][i] = (acc + (1 << 23)) >> 24
    return y


def q4(nib, sme, x):
    """[UORLUT01] "One projection (definition)", 4-bit codes in groups of 32,
    scale m * 2^e; exact, not rounded."""
    N = len(nib)
    K = 2 * len(nib[0])
    T = len(x)

    def code(i, j):
        c = (int(nib[i][j // 2]) >> (4 * (j & 1))) & 0xF
        return c - 16 if c >= 8 else c

    y = [[0] * N for _ in range(T)]
    for t in range(T):
        for i in range(N):
            acc = 0
            for g in range(K // 32):
                m, e = int(sme[i][g]) & 0xF, int(sme[i][g]) >> 4
                acc += m * 2**e * sum(code(i, j) * int(x[t][j]) for j in range(32 * g, 32 * g + 32))
            y[t][i] = acc
    return y


def silu_mul(g, u, lut):
    """h = floor(LUT[clamp(floor((g+16)/32), -32768, 32768) + 32768] * u / 2^16)."""
    out = []
    for gv, uv in zip(g, u):
        idx = (int(gv) + 16) >> 5
        idx = max(-32768, min(32768, idx))
        out.append((int(lut[idx + 32768]) * int(uv)) >> 16)
    return out


def radix16_mul(a: int, b: int) -> int:
    """[UORLUT01] "Products of two runtime values": the sixteen multiples of a
    by repeated addition, read at each base-16 digit of b, summed with shifts."""
    assert a >= 0 and b >= 0
    table = [0]
    for _ in range(15):
        table.append(table[-1] + a)
    r, k = 0, 0
    while b:
        r += table[b & 15] << (4 * k)
        b >>= 4
        k += 1
    return r


def limbs(x: int, L: int):
    """Balanced base-256 digits in [-128, 127]: x = sum_l 256^l d_l."""
    d = []
    for _ in range(L):
        m = (x + 128) % 256          # Python % is non-negative for positive modulus
        dl = m - 128
        d.append(dl)
        x = (x - dl) // 256
    return d, x == 0
