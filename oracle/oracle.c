/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the exact-integer
 * block-quantized projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the
 * GPU library: it is written from the definitions on the pages alone.
 *
 * Sources (cited by page title and section):
 *   [UORLUT01]  "D11 integer table serving (UORLUT01)", section "How it works"
 *               (paragraphs "Export", "One projection (definition)",
 *               "Products of two runtime values").
 *   [Handshake] "Vendor-Invariant Integer Inference for MindChain: Handshake
 *               v0", Claims C1-C4, section "Construction" (the frozen
 *               profile; probe 2; schedule gate; probe 1), Falsifiers 3, 7.
 *   [tritify]   "Deterministic, Reproducible Inference in Exact Integer
 *               Arithmetic, and Verifiable Distributed Inference as Its
 *               Consequence" (arXiv 2611.13730), section 3.1 "Arithmetic
 *               specification", 3.2 "Matmul", 3.4 "Multithreading".
 *
 * Everything is accumulated in __int128 (the i128 reference accumulator of
 * [tritify] 3.1) so that no intermediate can overflow for the sizes used;
 * results are checked to fit int64 before they are stored.
 *
 * Build: gcc -O2 -fno-tree-vectorize -ffp-contract=off -fPIC -shared -pthread
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

typedef __int128 i128;
typedef unsigned __int128 u128;

enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_ERANGE = 2, ORC_ENOMEM = 3 };

/* Evaluation orders.  The first five are the adversarial schedules named in
 * [Handshake] "Construction", schedule gate (canonical, reversed,
 * tiled_shuffled, split_k, tree_walk); the pages name them only, the
 * readings used here are:
 *   canonical      blocks ascending, columns ascending within a block;
 *   reversed       blocks descending, columns descending;
 *   tiled_shuffled 16x16 (token,row) output tiles and 4-block K tiles, both
 *                  visited in a seeded random permutation;
 *   split_k        8 contiguous block ranges summed as independent partials,
 *                  the partials then added from the 8th down to the 1st;
 *   tree_walk      the per-block terms added in a pairwise binary tree.
 * The last two are the two GEMM derivations of [Handshake] claim C2:
 *   row_order      row chunks outer, per-block partials, then explicit
 *                  per-block scalar accumulation;
 *   column_stream  column blocks outer, one (T,32)x(32,rows) exact product
 *                  per block accumulated into the output. */
enum {
  ORD_CANONICAL = 0, ORD_REVERSED = 1, ORD_TILED_SHUFFLED = 2, ORD_SPLIT_K = 3,
  ORD_TREE_WALK = 4, ORD_ROW_ORDER = 5, ORD_COLUMN_STREAM = 6, ORD_COUNT = 7
};

/* Products: MUL_NATIVE uses the compiler's 128-bit multiply; MUL_RADIX16 uses
 * the multiples-table product of [UORLUT01] "Products of two runtime
 * values": build the sixteen multiples of one operand by repeated addition,
 * read them at each base-16 digit of the other and sum the reads with
 * shifts, ab = sum_k 16^k T_a[d_k(b)].  Both must give the same bits. */
enum { MUL_NATIVE = 0, MUL_RADIX16 = 1 };

/* ---------------------------------------------------------------- helpers */

/* floor(a / 2^s) for 0 < s < 127, written with truncating division. */
static i128 floor_div_pow2(i128 a, int s) {
  i128 d = (i128)1 << s;
  i128 q = a / d;
  if (a % d != 0 && a < 0) q -= 1;
  return q;
}

static int fits_i64(i128 v) { return v >= (i128)INT64_MIN && v <= (i128)INT64_MAX; }

u128 orc_mul_u128_radix16(u128 a, u128 b) {
  u128 table[16];
  table[0] = 0;
  for (int d = 1; d < 16; ++d) table[d] = table[d - 1] + a;   /* d*a by additions */
  u128 r = 0;
  for (int k = 0; b != 0; ++k, b >>= 4) r += table[(int)(b & 15)] << (4 * k);
  return r;
}

/* 128-bit operands passed as (lo, hi) halves; out = a*b mod 2^128 as (lo, hi). */
void orc_mul128_radix16(uint64_t a_lo, uint64_t a_hi, uint64_t b_lo, uint64_t b_hi, uint64_t* out) {
  u128 a = ((u128)a_hi << 64) | a_lo, b = ((u128)b_hi << 64) | b_lo;
  u128 r = orc_mul_u128_radix16(a, b);
  out[0] = (uint64_t)r;
  out[1] = (uint64_t)(r >> 64);
}

/* Signed product by magnitudes; callers keep |a*b| < 2^127. */
static i128 mul_radix16(i128 a, i128 b) {
  int neg = (a < 0) != (b < 0);
  u128 ua = a < 0 ? (u128)0 - (u128)a : (u128)a;
  u128 ub = b < 0 ? (u128)0 - (u128)b : (u128)b;
  u128 r = orc_mul_u128_radix16(ua, ub);
  return neg ? (i128)((u128)0 - r) : (i128)r;
}

static i128 mul(i128 a, i128 b, int mode) { return mode == MUL_RADIX16 ? mul_radix16(a, b) : a * b; }

/* splitmix64 (Steele, Lea, Flood 2014): a published counter-based generator,
 * used only to draw the tiled_shuffled visiting order. */
static uint64_t splitmix64(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ULL);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static void shuffle(int64_t* v, int64_t n, uint64_t* state) { /* Fisher-Yates */
  for (int64_t i = n - 1; i > 0; --i) {
    int64_t j = (int64_t)(splitmix64(state) % (uint64_t)(i + 1));
    int64_t t = v[i]; v[i] = v[j]; v[j] = t;
  }
}

/* ------------------------------------------------------ Q8 projection core */

typedef struct {
  const int8_t* q;      /* [N][K] codes                                   */
  const int32_t* s;     /* [N][K/32] block scales                         */
  const int64_t* x;     /* [T][K] activations                             */
  i128* acc;            /* [T][N] exact sums, before rounding             */
  int64_t N, K, T, nb;
  int order, mul_mode;
  uint64_t seed;
  int64_t i0, i1;       /* this worker's rows [i0, i1)                   */
  int status;
} q8_job;

/* Sum over one block of q[i][j]*x[t][j], columns ascending or descending. */
static i128 block_dot(const q8_job* jb, int64_t t, int64_t i, int64_t b, int descending) {
  const int8_t* qi = jb->q + i * jb->K + b * 32;
  const int64_t* xt = jb->x + t * jb->K + b * 32;
  i128 p = 0;
  for (int jj = 0; jj < 32; ++jj) {
    int j = descending ? 31 - jj : jj;
    p += mul((i128)qi[j], (i128)xt[j], jb->mul_mode);
  }
  return p;
}

/* The per-block term S[i][b] * sum_{j in b} q[i][j] x[t][j]. */
static i128 block_term(const q8_job* jb, int64_t t, int64_t i, int64_t b, int descending) {
  return mul((i128)jb->s[i * jb->nb + b], block_dot(jb, t, i, b, descending), jb->mul_mode);
}

static void q8_canonical(q8_job* jb, int descending) {
  for (int64_t t = 0; t < jb->T; ++t)
    for (int64_t i = jb->i0; i < jb->i1; ++i) {
      i128 a = 0;
      for (int64_t bb = 0; bb < jb->nb; ++bb) {
        int64_t b = descending ? jb->nb - 1 - bb : bb;
        a += block_term(jb, t, i, b, descending);
      }
      jb->acc[t * jb->N + i] = a;
    }
}

static void q8_tiled_shuffled(q8_job* jb) {
  const int64_t TT = 16, TI = 16, KB = 4;   /* output tile 16x16, K tile 4 blocks */
  int64_t rows = jb->i1 - jb->i0;
  int64_t nt = (jb->T + TT - 1) / TT, ni = (rows + TI - 1) / TI, nk = (jb->nb + KB - 1) / KB;
  int64_t* otiles = malloc(sizeof(int64_t) * (size_t)(nt * ni > 0 ? nt * ni : 1));
  int64_t* ktiles = malloc(sizeof(int64_t) * (size_t)(nk > 0 ? nk : 1));
  if (!otiles || !ktiles) { free(otiles); free(ktiles); jb->status = ORC_ENOMEM; return; }
  uint64_t st = jb->seed ^ (uint64_t)jb->i0;
  for (int64_t v = 0; v < nt * ni; ++v) otiles[v] = v;
  for (int64_t v = 0; v < nk; ++v) ktiles[v] = v;
  shuffle(otiles, nt * ni, &st);
  shuffle(ktiles, nk, &st);
  for (int64_t t = 0; t < jb->T; ++t)
    for (int64_t i = jb->i0; i < jb->i1; ++i) jb->acc[t * jb->N + i] = 0;
  for (int64_t o = 0; o < nt * ni; ++o) {
    int64_t tt = otiles[o] / ni, ti = otiles[o] % ni;
    for (int64_t kk = 0; kk < nk; ++kk) {
      int64_t kt = ktiles[kk];
      for (int64_t t = tt * TT; t < tt * TT + TT && t < jb->T; ++t)
        for (int64_t i = jb->i0 + ti * TI; i < jb->i0 + ti * TI + TI && i < jb->i1; ++i)
          for (int64_t b = kt * KB; b < kt * KB + KB && b < jb->nb; ++b)
            jb->acc[t * jb->N + i] += block_term(jb, t, i, b, 0);
    }
  }
  free(otiles); free(ktiles);
}

static void q8_split_k(q8_job* jb) {
  for (int64_t t = 0; t < jb->T; ++t)
    for (int64_t i = jb->i0; i < jb->i1; ++i) {
      i128 part[8];
      for (int p = 0; p < 8; ++p) {
        int64_t b0 = p * jb->nb / 8, b1 = (p + 1) * jb->nb / 8;
        part[p] = 0;
        for (int64_t b = b0; b < b1; ++b) part[p] += block_term(jb, t, i, b, 0);
      }
      i128 a = 0;
      for (int p = 7; p >= 0; --p) a += part[p];
      jb->acc[t * jb->N + i] = a;
    }
}

static void q8_tree_walk(q8_job* jb) {
  i128* terms = malloc(sizeof(i128) * (size_t)(jb->nb > 0 ? jb->nb : 1));
  if (!terms) { jb->status = ORC_ENOMEM; return; }
  for (int64_t t = 0; t < jb->T; ++t)
    for (int64_t i = jb->i0; i < jb->i1; ++i) {
      int64_t n = jb->nb;
      for (int64_t b = 0; b < n; ++b) terms[b] = block_term(jb, t, i, b, 0);
      while (n > 1) {                      /* pairs (0,1),(2,3),...; an odd last one passes up */
        int64_t m = 0;
        for (; 2 * m + 1 < n; ++m) terms[m] = terms[2 * m] + terms[2 * m + 1];
        if (n & 1) terms[m++] = terms[n - 1];
        n = m;
      }
      jb->acc[t * jb->N + i] = jb->nb > 0 ? terms[0] : 0;
    }
  free(terms);
}

static void q8_row_order(q8_job* jb) {
  const int64_t CH = 64;                   /* row chunk */
  i128* part = malloc(sizeof(i128) * (size_t)(jb->T * CH * (jb->nb > 0 ? jb->nb : 1)));
  if (!part) { jb->status = ORC_ENOMEM; return; }
  for (int64_t c0 = jb->i0; c0 < jb->i1; c0 += CH) {
    int64_t c1 = c0 + CH < jb->i1 ? c0 + CH : jb->i1;
    /* per-block partials P[t][i][b] for the chunk */
    for (int64_t t = 0; t < jb->T; ++t)
      for (int64_t i = c0; i < c1; ++i)
        for (int64_t b = 0; b < jb->nb; ++b)
          part[(t * CH + (i - c0)) * jb->nb + b] = block_dot(jb, t, i, b, 0);
    /* explicit per-block scalar accumulation */
    for (int64_t t = 0; t < jb->T; ++t)
      for (int64_t i = c0; i < c1; ++i) {
        i128 a = 0;
        for (int64_t b = 0; b < jb->nb; ++b)
          a += mul((i128)jb->s[i * jb->nb + b], part[(t * CH + (i - c0)) * jb->nb + b], jb->mul_mode);
        jb->acc[t * jb->N + i] = a;
      }
  }
  free(part);
}

static void q8_column_stream(q8_job* jb) {
  for (int64_t t = 0; t < jb->T; ++t)
    for (int64_t i = jb->i0; i < jb->i1; ++i) jb->acc[t * jb->N + i] = 0;
  for (int64_t b = 0; b < jb->nb; ++b)          /* column blocks outer */
    for (int64_t t = 0; t < jb->T; ++t)         /* (T,32) x (32,rows) */
      for (int64_t i = jb->i0; i < jb->i1; ++i) {
        i128 m = 0;
        for (int64_t j = b * 32; j < b * 32 + 32; ++j)
          m += mul((i128)jb->x[t * jb->K + j], (i128)jb->q[i * jb->K + j], jb->mul_mode);
        jb->acc[t * jb->N + i] += mul(m, (i128)jb->s[i * jb->nb + b], jb->mul_mode);
      }
}

static void* q8_worker(void* arg) {
  q8_job* jb = arg;
  switch (jb->order) {
    case ORD_CANONICAL: q8_canonical(jb, 0); break;
    case ORD_REVERSED: q8_canonical(jb, 1); break;
    case ORD_TILED_SHUFFLED: q8_tiled_shuffled(jb); break;
    case ORD_SPLIT_K: q8_split_k(jb); break;
    case ORD_TREE_WALK: q8_tree_walk(jb); break;
    case ORD_ROW_ORDER: q8_row_order(jb); break;
    case ORD_COLUMN_STREAM: q8_column_stream(jb); break;
    default: jb->status = ORC_EINVAL;
  }
  return NULL;
}

/* Workers own disjoint output rows, so the thread count changes nothing but
 * speed ([tritify] 3.4, "Multithreading"). */
static int run_q8(q8_job* proto, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > proto->N) nthreads = (int)(proto->N > 0 ? proto->N : 1);
  q8_job jobs[256];
  pthread_t th[256];
  for (int w = 0; w < nthreads; ++w) {
    jobs[w] = *proto;
    jobs[w].i0 = proto->N * w / nthreads;
    jobs[w].i1 = proto->N * (w + 1) / nthreads;
    jobs[w].status = ORC_OK;
  }
  if (nthreads == 1) { q8_worker(&jobs[0]); return jobs[0].status; }
  for (int w = 0; w < nthreads; ++w) pthread_create(&th[w], NULL, q8_worker, &jobs[w]);
  int st = ORC_OK;
  for (int w = 0; w < nthreads; ++w) { pthread_join(th[w], NULL); if (jobs[w].status) st = jobs[w].status; }
  return st;
}

/*
 * Q8 projection.  [UORLUT01] "One projection (definition)": y_i = sum_j w_ij
 * x_j with each weight a block scale times a code; [Handshake] C1 and "The
 * frozen profile": 8-bit codes in blocks of 32 with frozen Q24 integer
 * scales, Q16 int64 activations, exact accumulation with no saturation.
 * The rounding back to Q16 adds 2^23 and takes the floor of the division by
 * 2^24 (an arithmetic right shift of the exact sum).
 *
 *   acc[t][i] = sum_b S[i][b] * sum_{j in b} q[i][j] * x[t][j]
 *   y[t][i]   = floor((acc[t][i] + 2^23) / 2^24)
 *
 * acc_out, if not NULL, receives the exact sums as int128 (before
 * rounding).  Returns ORC_ERANGE if some y does not fit int64.
 */
int orc_q8(const int8_t* q, const int32_t* s, const int64_t* x, int64_t* y, i128* acc_out,
           int64_t N, int64_t K, int64_t T, int order, uint64_t seed, int mul_mode, int nthreads) {
  if (N < 0 || K < 0 || T < 0 || K % 32 != 0 || order < 0 || order >= ORD_COUNT) return ORC_EINVAL;
  if (N == 0 || T == 0) return ORC_OK;
  i128* acc = acc_out ? acc_out : malloc(sizeof(i128) * (size_t)(T * N));
  if (!acc) return ORC_ENOMEM;
  q8_job proto = {q, s, x, acc, N, K, T, K / 32, order, mul_mode, seed, 0, N, ORC_OK};
  int st = run_q8(&proto, nthreads);
  if (st == ORC_OK)
    for (int64_t e = 0; e < T * N; ++e) {
      i128 v = floor_div_pow2(acc[e] + ((i128)1 << 23), 24);
      if (!fits_i64(v)) { st = ORC_ERANGE; y[e] = 0; } else y[e] = (int64_t)v;
    }
  if (!acc_out) free(acc);
  return st;
}

/* ------------------------------------------------------ Q4 projection core */

/* Code j of row i: a two's-complement nibble, element 2k in the low nibble
 * of byte k (reading of [UORLUT01] "Export": 4-bit codes in groups of 32). */
static int q4_code(const uint8_t* nib, int64_t K, int64_t i, int64_t j) {
  int c = (nib[i * (K / 2) + j / 2] >> (4 * (j & 1))) & 0xF;
  return c >= 8 ? c - 16 : c;
}

/* One scale byte per group: mantissa m in the low nibble, exponent e in the
 * high nibble, s = m * 2^e ([UORLUT01] "Export"). */
static int q4_mant(const uint8_t* sme, int64_t ng, int64_t i, int64_t g) { return sme[i * ng + g] & 0xF; }
static int q4_expo(const uint8_t* sme, int64_t ng, int64_t i, int64_t g) { return sme[i * ng + g] >> 4; }

typedef struct {
  const uint8_t* nib; const uint8_t* sme; const int32_t* x; i128* acc;
  int64_t N, K, T, ng;
  int derivation;
  int64_t i0, i1;
} q4_job;

/* Definition ([UORLUT01] "One projection (definition)"):
 *   y[t][i] = sum_g m[i][g] 2^e[i][g] * sum_{j in g} q[i][j] x[t][j]  (exact) */
static void q4_definition(q4_job* jb) {
  for (int64_t t = 0; t < jb->T; ++t)
    for (int64_t i = jb->i0; i < jb->i1; ++i) {
      i128 a = 0;
      for (int64_t g = 0; g < jb->ng; ++g) {
        i128 p = 0;
        for (int64_t j = g * 32; j < g * 32 + 32; ++j) p += (i128)q4_code(jb->nib, jb->K, i, j) * jb->x[t * jb->K + j];
        i128 sc = (i128)q4_mant(jb->sme, jb->ng, i, g) * ((i128)1 << q4_expo(jb->sme, jb->ng, i, g));
        a += sc * p;
      }
      jb->acc[t * jb->N + i] = a;
    }
}

/* The engine's table read ([UORLUT01] "One projection (definition)"): for
 * each activation build the 16-entry table T_j[q] = q x_j by additions, read
 * T_j[q_ij] for each weight, block four output rows to reuse the table, and
 * apply s = m 2^e by shifts and adds.  No multiply is used. */
static void q4_table_read(q4_job* jb) {
  for (int64_t t = 0; t < jb->T; ++t)
    for (int64_t i4 = jb->i0; i4 < jb->i1; i4 += 4) {
      int64_t nr = jb->i1 - i4 < 4 ? jb->i1 - i4 : 4;
      i128 acc[4] = {0, 0, 0, 0};
      for (int64_t g = 0; g < jb->ng; ++g) {
        i128 part[4] = {0, 0, 0, 0};
        for (int64_t j = g * 32; j < g * 32 + 32; ++j) {
          i128 tab[16];                     /* tab[q + 8] = q * x_j, q in [-8, 7] */
          i128 xj = jb->x[t * jb->K + j];
          tab[8] = 0;
          for (int v = 9; v < 16; ++v) tab[v] = tab[v - 1] + xj;
          for (int v = 7; v >= 0; --v) tab[v] = tab[v + 1] - xj;
          for (int64_t r = 0; r < nr; ++r) part[r] += tab[q4_code(jb->nib, jb->K, i4 + r, j) + 8];
        }
        for (int64_t r = 0; r < nr; ++r) {
          int m = q4_mant(jb->sme, jb->ng, i4 + r, g), e = q4_expo(jb->sme, jb->ng, i4 + r, g);
          for (int bit = 0; bit < 4; ++bit)
            if (m & (1 << bit)) {
              /* shift of a possibly negative value: shift the magnitude */
              i128 v = part[r];
              if (v < 0) acc[r] -= (i128)((u128)(-v) << (e + bit));
              else acc[r] += (i128)((u128)v << (e + bit));
            }
        }
      }
      for (int64_t r = 0; r < nr; ++r) jb->acc[t * jb->N + i4 + r] = acc[r];
    }
}

static void* q4_worker(void* arg) {
  q4_job* jb = arg;
  if (jb->derivation == 1) q4_table_read(jb); else q4_definition(jb);
  return NULL;
}

/* Q4 projection; derivation 0 = definition, 1 = table read.  The result is
 * exact and not rounded; ORC_ERANGE if it does not fit int64. */
int orc_q4(const uint8_t* nib, const uint8_t* sme, const int32_t* x, int64_t* y,
           int64_t N, int64_t K, int64_t T, int derivation, int nthreads) {
  if (N < 0 || K < 0 || T < 0 || K % 32 != 0 || derivation < 0 || derivation > 1) return ORC_EINVAL;
  if (N == 0 || T == 0) return ORC_OK;
  i128* acc = malloc(sizeof(i128) * (size_t)(T * N));
  if (!acc) return ORC_ENOMEM;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > N) nthreads = (int)N;
  q4_job jobs[256];
  pthread_t th[256];
  for (int w = 0; w < nthreads; ++w) {
    q4_job jb = {nib, sme, x, acc, N, K, T, K / 32, derivation, N * w / nthreads, N * (w + 1) / nthreads};
    jobs[w] = jb;
  }
  if (nthreads == 1) q4_worker(&jobs[0]);
  else {
    for (int w = 0; w < nthreads; ++w) pthread_create(&th[w], NULL, q4_worker, &jobs[w]);
    for (int w = 0; w < nthreads; ++w) pthread_join(th[w], NULL);
  }
  int st = ORC_OK;
  for (int64_t e = 0; e < T * N; ++e) {
    if (!fits_i64(acc[e])) { st = ORC_ERANGE; y[e] = 0; } else y[e] = (int64_t)acc[e];
  }
  free(acc);
  return st;
}

/* --------------------------------------------------------- SiLU epilogue */

/*
 * h = (silu(g) * u) >> 16 with silu read from the frozen table.
 * [Handshake] C1 and C4: SiLU is evaluated through a committed 65537-entry
 * table, Q11 input clamped at +-16, Q16 output; C4's clip behaviour (inputs
 * above +16 read the end entry, error growing as x - 16) fixes that the
 * index is clamped, not extrapolated.  Readings: the Q16 gate is brought to
 * Q11 by an add-half shift (as the same page's harness rescales Q16 to Q4),
 * idx = floor((g + 16) / 32) clamped to [-32768, 32768]; the product of the
 * Q16 table value and the Q16 up value is brought back to Q16 by a floor
 * shift of 16 bits.
 */
int orc_silu_mul(const int64_t* g, const int64_t* u, const int32_t* lut, int64_t* h, int64_t n) {
  int st = ORC_OK;
  for (int64_t e = 0; e < n; ++e) {
    i128 idx = floor_div_pow2((i128)g[e] + 16, 5);
    if (idx < -32768) idx = -32768;
    if (idx > 32768) idx = 32768;
    i128 v = floor_div_pow2((i128)lut[(int64_t)idx + 32768] * (i128)u[e], 16);
    if (!fits_i64(v)) { st = ORC_ERANGE; h[e] = 0; } else h[e] = (int64_t)v;
  }
  return st;
}

/* ------------------------------------------------------- limb definition */

/*
 * Balanced base-256 digits: d_l in [-128, 127] with x = sum_l 256^l d_l.
 * The digit set is a complete residue system mod 256, so the digits are
 * unique.  d is [L][n].  Returns ORC_ERANGE (digits still written) if x
 * needs more than L digits.
 */
int orc_limb_split(const int64_t* x, int8_t* d, int64_t n, int L) {
  if (L < 1 || L > 8) return ORC_EINVAL;
  int st = ORC_OK;
  for (int64_t e = 0; e < n; ++e) {
    i128 r = x[e];
    for (int l = 0; l < L; ++l) {
      i128 m = (r + 128) % 256;
      if (m < 0) m += 256;
      int dl = (int)m - 128;
      d[(int64_t)l * n + e] = (int8_t)dl;
      r = (r - dl) / 256;                 /* exact */
    }
    if (r != 0) st = ORC_ERANGE;
  }
  return st;
}

/* ---------------------------------------------------------- FP32 shadow */

/*
 * The same Q8 sum in float32, the negative control of [Handshake] C3 and
 * "Construction", schedule gate: w = fl32(S q 2^-24), x = fl32(X 2^-16),
 * products fl32(w x) and sums fl32(a + b) taken one at a time in the
 * schedule's order, with no fused multiply-add.  Orders:
 *   canonical      columns ascending over all of K;
 *   reversed       columns descending;
 *   tiled_shuffled 128-column K tiles in a seeded permutation, ascending
 *                  within a tile, one running sum;
 *   split_k        8 partials over contiguous block ranges (ascending), then
 *                  0 + p7 + p6 + ... + p0;
 *   tree_walk      per-block sums (ascending), then a pairwise tree.
 * The pages print float values only for their checkpoint, not for synthetic
 * inputs; each order is pinned instead against float32 sequences formed
 * independently in the tests.
 */
static float shadow_w(const int8_t* q, const int32_t* s, int64_t K, int64_t i, int64_t j) {
  return (float)((double)((int64_t)s[i * (K / 32) + j / 32] * q[i * K + j]) * (1.0 / 16777216.0));
}
static float shadow_x(const int64_t* x, int64_t K, int64_t t, int64_t j) {
  return (float)((double)x[t * K + j] * (1.0 / 65536.0));
}

int orc_q8_fp32(const int8_t* q, const int32_t* s, const int64_t* x, float* y,
                int64_t N, int64_t K, int64_t T, int order, uint64_t seed) {
  if (K % 32 != 0 || order < 0 || order > ORD_TREE_WALK) return ORC_EINVAL;
  int64_t nb = K / 32, nkt = (K + 127) / 128;
  int64_t* kt = malloc(sizeof(int64_t) * (size_t)(nkt > 0 ? nkt : 1));
  float* bs = malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
  if (!kt || !bs) { free(kt); free(bs); return ORC_ENOMEM; }
  uint64_t st = seed;
  for (int64_t v = 0; v < nkt; ++v) kt[v] = v;
  shuffle(kt, nkt, &st);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t i = 0; i < N; ++i) {
      float a = 0.0f;
      if (order == ORD_CANONICAL) {
        for (int64_t j = 0; j < K; ++j) a = a + shadow_w(q, s, K, i, j) * shadow_x(x, K, t, j);
      } else if (order == ORD_REVERSED) {
        for (int64_t j = K - 1; j >= 0; --j) a = a + shadow_w(q, s, K, i, j) * shadow_x(x, K, t, j);
      } else if (order == ORD_TILED_SHUFFLED) {
        for (int64_t v = 0; v < nkt; ++v)
          for (int64_t j = kt[v] * 128; j < kt[v] * 128 + 128 && j < K; ++j)
            a = a + shadow_w(q, s, K, i, j) * shadow_x(x, K, t, j);
      } else if (order == ORD_SPLIT_K) {
        float part[8];
        for (int p = 0; p < 8; ++p) {
          part[p] = 0.0f;
          for (int64_t j = (p * nb / 8) * 32; j < ((p + 1) * nb / 8) * 32; ++j)
            part[p] = part[p] + shadow_w(q, s, K, i, j) * shadow_x(x, K, t, j);
        }
        for (int p = 7; p >= 0; --p) a = a + part[p];
      } else {
        int64_t n = nb;
        for (int64_t b = 0; b < nb; ++b) {
          float c = 0.0f;
          for (int64_t j = b * 32; j < b * 32 + 32; ++j) c = c + shadow_w(q, s, K, i, j) * shadow_x(x, K, t, j);
          bs[b] = c;
        }
        while (n > 1) {
          int64_t m = 0;
          for (; 2 * m + 1 < n; ++m) bs[m] = bs[2 * m] + bs[2 * m + 1];
          if (n & 1) bs[m++] = bs[n - 1];
          n = m;
        }
        a = nb > 0 ? bs[0] : 0.0f;
      }
      y[t * N + i] = a;
    }
  free(kt); free(bs);
  return ORC_OK;
}
