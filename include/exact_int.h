/*
 * exact_int.h -- C ABI of the exact-integer block-quantized projection
 * library for AMD Instinct MI355X (gfx950).
 *
 * The library computes the projection stated on the pages
 *
 *     y_i = rnd( sum_b S_ib * sum_{j in b} q_ij * x_j )
 *
 * exactly, so that its output bits do not depend on loop order, tiling or
 * split-K.  Sources (cited by page title and section):
 *   [UORLUT01]  "D11 integer table serving (UORLUT01)", "How it works":
 *               "Export" (4-bit codes in groups of 32, one-byte scale with
 *               a 4-bit mantissa and a 4-bit exponent) and "One projection
 *               (definition)" (y_i = sum_j w_ij x_j, w_ij = s_g q_ij,
 *               s_g = m 2^e).
 *   [Handshake] "Vendor-Invariant Integer Inference for MindChain:
 *               Handshake v0", claim C1 and "Construction / The frozen
 *               profile" (Q8_0 codes in blocks of 32, FP16 block scales
 *               frozen into Q24 integers, Q16 activations in int64, exact
 *               accumulation with no saturation, a SiLU table committed
 *               in decimal); C3 and "Schedule gate" (five adversarial
 *               schedules); C4 (the SiLU table's clip behaviour).
 *   [tritify]   "Deterministic, Reproducible Inference in Exact Integer
 *               Arithmetic, and Verifiable Distributed Inference as Its
 *               Consequence" (arXiv 2611.13730), 3.1 "Arithmetic
 *               specification" (i128 reference accumulator, i64 hot path
 *               with a proven bound on the range), 3.2 "Mixture-of-Experts",
 *               4 (SHA-256 of the integer output).
 *
 * Conventions (all entry points):
 *   - Pointers are DEVICE pointers owned by the caller unless a comment says
 *     "host".  The library never frees caller memory.  Arrays are dense,
 *     row-major, little-endian, and 16-byte aligned unless stated.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous on `stream` unless a comment says "synchronous".
 *   - The return value reports errors the host can see at once (EI_EINVAL,
 *     EI_ERANGE, EI_ENOSPACE, EI_EDEVICE); nothing is launched when it is
 *     not EI_OK.  Errors only the device can see (an activation outside the
 *     declared limb range, a result outside int64) are OR-ed into the
 *     device word `d_status` (may be NULL to skip), which the caller reads
 *     after synchronising; the outputs are then unspecified.
 *   - No entry point allocates device memory except where a comment says
 *     so; scratch space is the caller's `workspace` of at least the size
 *     the matching *_workspace_bytes() returns.
 *   - The library holds no mutable global state apart from the scratch
 *     array of int_gemm_q8_noalloc; calls on different streams may run
 *     concurrently.  Calls that share a workspace must be ordered.
 *   - Weight matrices have K (the reduction dimension) a multiple of 32:
 *     the block structure of the formats.  N and T may be anything >= 1.
 */
#ifndef EXACT_INT_H
#define EXACT_INT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* ei_stream;   /* a hipStream_t */

/* Return codes. */
enum {
  EI_OK = 0,
  EI_EINVAL = 1,    /* null pointer, bad size or enum, K % 32 != 0, misaligned */
  EI_ERANGE = 2,    /* request outside the proven-exact envelope (see below)  */
  EI_EDEVICE = 3,   /* a HIP runtime call failed                               */
  EI_ENOSPACE = 4   /* workspace or output buffer too small                    */
};

/* Bits OR-ed into *d_status by the device. */
enum {
  EI_DEV_LIMB_RANGE = 1,    /* an activation does not fit the declared limbs */
  EI_DEV_OUT_RANGE = 2,     /* a result does not fit int64                   */
  EI_DEV_ROUTE = 4          /* a routed pair names an expert outside [0, E)  */
};

/* Accumulation schedules ([Handshake] "Schedule gate": canonical, reversed,
 * tiled_shuffled, split_k, tree_walk).  Every schedule returns identical
 * bits; EI_SCHED_DEFAULT is the fastest kernel for the shape. */
enum {
  EI_SCHED_DEFAULT = 0,
  EI_SCHED_CANONICAL = 1,       /* blocks ascending                               */
  EI_SCHED_REVERSED = 2,        /* blocks descending                              */
  EI_SCHED_TILED_SHUFFLED = 3,  /* output tiles and K blocks in a seeded order    */
  EI_SCHED_SPLIT_K = 4,         /* 8 K-ranges as separate partials, then summed   */
  EI_SCHED_TREE = 5             /* per-block terms summed in a pairwise tree      */
};

enum { EI_FORMAT_Q8 = 1, EI_FORMAT_Q4 = 2, EI_FORMAT_WIDE = 3 };

/* Host-side descriptor of a packed weight matrix, filled by ei_q8_pack or
 * ei_q4_pack.  `packed` points into the caller's device buffer.  The fields
 * are read as the pack call wrote them; in particular `smax` selects the
 * accumulation form of the MFMA kernels (two int64 chains per output when
 * smax < 2^15 and nb * smax <= 2^27, else one per activation limb), so a
 * descriptor whose smax understates the packed scales voids exactness. */
typedef struct ei_weights {
  const void* packed;   /* device: packed tiles, see ei_q8_pack            */
  int64_t n;            /* output rows                                     */
  int64_t k;            /* reduction length, a multiple of 32              */
  int64_t n_pad;        /* n rounded up to a multiple of 32                */
  int64_t nb;           /* k / 32 blocks                                   */
  uint32_t smax;        /* max |scale| over all blocks (Q4: max 2^e)       */
  int32_t format;       /* EI_FORMAT_Q8, EI_FORMAT_Q4 or EI_FORMAT_WIDE    */
  int64_t experts;      /* matrices stacked in the buffer (1 unless packed */
                        /* with ei_q8_pack_stacked)                         */
  int64_t expert_stride;/* bytes from one stacked matrix to the next       */
} ei_weights;

/* ------------------------------------------------------------ weights */

/* Bytes of device memory ei_q8_pack / ei_q4_pack need for an n x k matrix
 * (one layout for both formats; see ei_q8_pack). */
size_t ei_packed_bytes(int64_t n, int64_t k);

/*
 * Repack a Q8 matrix ([Handshake] C1: 8-bit codes, one Q24 int32 scale per
 * 32-wide block along K) into the kernels' layout, once, at load time.
 *   codes   device int8 [n][k]
 *   scales  device int32 [n][k/32]
 *   packed  device buffer of >= ei_packed_bytes(n, k) bytes, 256-B aligned;
 *           after the call it holds a 256-byte header, then the code tiles
 *           [n_pad/32][k/32][64 lanes][16 B] (lane l holds row l%32 and
 *           columns 16*(l/32) .. +15 of the block), then the scales
 *           [n_pad/32][k/32][32] int32, then a row-offset area [n_pad]
 *           int64 (used by 4-bit images, zero here); rows >= n are zero.
 *   out     host: the descriptor to pass to the GEMM entry points.
 * Synchronous (it reads back the largest scale).  Errors: EI_EINVAL for a
 * null pointer, n < 1, k < 32 or k % 32 != 0; EI_ENOSPACE if packed_bytes is
 * too small; EI_EDEVICE on a HIP failure.
 */
int ei_q8_pack(const int8_t* codes, const int32_t* scales, int64_t n, int64_t k,
               void* packed, size_t packed_bytes, ei_weights* out, ei_stream stream);

/*
 * Repack a UORLUT01-style 4-bit matrix ([UORLUT01] "Export": 4-bit codes in
 * groups of 32 with a one-byte scale, mantissa m and exponent e, s = m 2^e).
 *   nib     device uint8 [n][k/2]: two's-complement nibbles, element 2j in
 *           the low nibble of byte j
 *   sme     device uint8 [n][k/32]: m in the low nibble, e in the high nibble
 * The mantissa is folded into the codes (m q lies in [-120, 105], an int8)
 * and the scale kept as 2^e, so sum_g m 2^e sum_j q x is computed exactly
 * as sum_g 2^e sum_j (m q) x.  The row-offset area holds R_i = 128 sum_j
 * m 2^e q[i][j] (|R_i| < 2^47), which the two-limb form of int_gemm_q4 adds
 * back.  Layout, sync and errors as ei_q8_pack.
 */
int ei_q4_pack(const uint8_t* nib, const uint8_t* sme, int64_t n, int64_t k,
               void* packed, size_t packed_bytes, ei_weights* out, ei_stream stream);

/* Bytes for `experts` stacked n x k matrices (ei_q8_pack_stacked). */
size_t ei_packed_bytes_stacked(int64_t experts, int64_t n, int64_t k);

/*
 * Repack E same-shape Q8 matrices, the experts of a Mixture-of-Experts layer
 * ([tritify] 3.2 "Mixture-of-Experts": every selected expert is an exact-
 * integer MLP), into one buffer: matrix e is packed exactly as ei_q8_pack
 * would, at byte offset e * expert_stride (expert_stride = ei_packed_bytes(n,
 * k) rounded up to 256).
 *   codes   device int8 [E][n][k]
 *   scales  device int32 [E][n][k/32]
 *   packed  device buffer of >= ei_packed_bytes_stacked(E, n, k) bytes,
 *           256-B aligned
 *   out     host: descriptor with experts = E; smax is the largest scale of
 *           all experts
 * Synchronous.  Errors as ei_q8_pack; EI_EINVAL for E < 1.
 */
int ei_q8_pack_stacked(const int8_t* codes, const int32_t* scales, int64_t experts, int64_t n, int64_t k,
                       void* packed, size_t packed_bytes, ei_weights* out, ei_stream stream);

/* ------------------------------------------------------ activations */

/*
 * Balanced base-256 limb split, the activation quantiser: digits d_l in
 * [-128, 127] with x = sum_{l<L} 256^l d_l (unique).  Q16 activations with
 * |x| <= 2^22 need L = 3 (range [-8421504, 8355711]).
 *   x       device int64 [n]
 *   d       device int8 [L][n]
 * An x outside the L-limb range sets EI_DEV_LIMB_RANGE.  L in 1..8.
 */
int ei_limb_split(const int64_t* x, int8_t* d, int64_t n, int limbs,
                  int32_t* d_status, ei_stream stream);

/* ------------------------------------------------------ projections */

/* Workspace bytes int_gemm_q8 / int_gemm_q4 need for T tokens. */
size_t ei_gemm_workspace_bytes(const ei_weights* w, int64_t t, int limbs, int schedule);

/*
 * Q8 projection ([UORLUT01] "One projection (definition)"; [Handshake] C1,
 * "The frozen profile"):
 *     acc[t][i] = sum_b S[i][b] * sum_{j in b} q[i][j] * x[t][j]   (exact)
 *     y[t][i]   = (acc[t][i] + 2^23) >> 24   (arithmetic shift: floor)
 *   w        host: descriptor from ei_q8_pack (format EI_FORMAT_Q8)
 *   x        device int64 [t][k], Q16 activations
 *   y        device int64 [t][n]
 *   limbs    activation limbs L in 1..8; every x must satisfy the L-limb
 *            range (3 limbs: [-8421504, 8355711], which holds |x| <= 2^22)
 *   schedule EI_SCHED_*; shuffle_seed seeds EI_SCHED_TILED_SHUFFLED
 * Exactness: per-limb partial sums are carried in int64 and are exact for
 * any int32 scales while k <= 262144 (each term |S P| < 2^31 2^19 = 2^50);
 * the limbs are combined in int128 and rounded once.  With 3 limbs and
 * narrow scales (w->smax < 2^15 and nb * smax <= 2^27) the MFMA kernels
 * carry S (P_0 + 2^8 P_1) and 2^16 S P_2 instead, both below 2^62.01: the
 * same exact sum.  EI_ERANGE if k > 262144 or t > 65535 * 32.  A y outside
 * int64 sets EI_DEV_OUT_RANGE.
 */
int int_gemm_q8(const ei_weights* w, const int64_t* x, int64_t* y, int64_t t, int limbs,
                int schedule, uint64_t shuffle_seed, void* workspace, size_t workspace_bytes,
                int32_t* d_status, ei_stream stream);

/*
 * 4-bit projection ([UORLUT01] "One projection (definition)"), exact, not
 * rounded:  y[t][i] = sum_g m[i][g] 2^e[i][g] sum_{j in g} q[i][j] x[t][j]
 *   w        descriptor from ei_q4_pack (format EI_FORMAT_Q4)
 *   x        device int32 [t][k]
 *   limbs    2: the two-limb form for x in [-2^15, 2^15): the split takes the
 *            digits of x - 128 (two balanced base-256 digits hold exactly
 *            [-32896, 32639]) and row i gets R_i = 128 sum_j w[i][j] from
 *            the packed image back, which is exact because the projection
 *            is linear in x; an x outside [-2^15, 2^15) sets
 *            EI_DEV_LIMB_RANGE.  Any other L in 1..4 splits x itself, as
 *            int_gemm_q8 does (3 covers |x| < 2^23).
 *   y        device int64 [t][n]
 * Other arguments and errors as int_gemm_q8.
 */
int int_gemm_q4(const ei_weights* w, const int32_t* x, int64_t* y, int64_t t, int limbs,
                int schedule, uint64_t shuffle_seed, void* workspace, size_t workspace_bytes,
                int32_t* d_status, ei_stream stream);

/*
 * int_gemm_q8 under EI_SCHED_DEFAULT for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same definition and the same bits, with no workspace
 * argument.  The scratch space it needs (activation limb tiles, workgroup
 * partials) is a fixed 32 MiB array inside the library's code object, one per
 * device, held until the process ends; the device current at the call is the
 * one used.  Nothing is allocated or freed by the call.
 *   w, x, y, t, limbs, d_status, stream   as int_gemm_q8
 * EI_ENOSPACE if ei_gemm_workspace_bytes(w, t, limbs, EI_SCHED_DEFAULT)
 * exceeds 32 MiB (e.g. k = 4096 with more than about 2,700 tokens); other
 * errors as int_gemm_q8.  All calls on one device share the array: calls
 * that overlap in time on one device (different streams, or threads) race
 * and must be ordered by the caller.  Every call writes all the scratch it
 * reads, so no clearing between calls is needed.
 */
int int_gemm_q8_noalloc(const ei_weights* w, const int64_t* x, int64_t* y, int64_t t, int limbs,
                        int32_t* d_status, ei_stream stream);

/*
 * Several Q8 projections of the same activations in one launch, for decode
 * sizes (the Q, K and V projections of a layer, or gate and up, share x;
 * [Handshake] C1 profile): for m < count,
 *     y[m] = int_gemm_q8(w[m], x)   (the same definition, the same bits)
 * One GEMV launch streams all the matrices, so no matrix waits for the
 * previous launch to drain.
 *   w        host array of count descriptors from ei_q8_pack, all with the
 *            same k
 *   count    1 .. 16
 *   x        device int64 [t][k], Q16 activations
 *   y        host array of count device pointers; y[m] int64 [t][w[m]->n]
 *   t        1 .. 4 tokens;  limbs 1 .. 4 (3 for |x| <= 2^22)
 * No workspace.  EI_EINVAL for a null pointer, count or t out of range,
 * differing k or a bad descriptor; EI_ERANGE for limbs 5 .. 8 or k >
 * 262144.  Device flags as int_gemm_q8.
 */
int int_gemm_q8_multi(const ei_weights* const* w, int count, const int64_t* x, int64_t* const* y, int64_t t,
                      int limbs, int32_t* d_status, ei_stream stream);

/* Workspace bytes int_gemm_q8_grouped needs for `rows` activation rows routed
 * to `topk` experts each. */
size_t ei_grouped_workspace_bytes(const ei_weights* w, int64_t rows, int topk, int limbs);

/*
 * Routed (grouped) Q8 projection, the expert GEMM of a Mixture-of-Experts
 * layer ([tritify] 3.2 "Mixture-of-Experts"; the Q8 profile of [Handshake]
 * C1): for every activation row r and slot s, with e = route[r][s],
 *     y[r * topk + s][i] = (sum_b S_e[i][b] sum_{j in b} q_e[i][j] x[r][j]
 *                           + 2^23) >> 24
 * exactly, i.e. int_gemm_q8 of expert e on row r.  The pairs (r, s) are
 * grouped by expert on the device (a stable sort, ties by pair index), each
 * group runs as MFMA token tiles against its expert's tiles, and every result
 * lands in its pair's own output row, so y does not depend on the grouping.
 *   w        descriptor from ei_q8_pack_stacked (experts = E)
 *   x        device int64 [rows][k], Q16 activations
 *   route    device int32 [rows][topk], expert ids in [0, E)
 *   y        device int64 [rows * topk][n]
 *   limbs    3 (Q16 activations with |x| <= 2^22)
 * rows * topk <= 16384 and E <= 2^17, else EI_ERANGE; other host errors as
 * int_gemm_q8.  An expert id outside [0, E) sets EI_DEV_ROUTE (that pair's
 * output row is left unwritten).
 */
int int_gemm_q8_grouped(const ei_weights* w, const int64_t* x, const int32_t* route, int64_t rows, int topk,
                        int64_t* y, int limbs, void* workspace, size_t workspace_bytes, int32_t* d_status,
                        ei_stream stream);

/* ------------------------------------------------------- epilogues */

/*
 * Build the 65537-entry SiLU table ([Handshake] C1, C4: Q11 input over
 * +-16, Q16 output): lut[k + 32768] = round(silu(k / 2^11) * 2^16),
 * silu(z) = z / (1 + e^-z), k in [-32768, 32768].
 *   lut     device int32 [65537]
 */
int ei_silu_lut_build(int32_t* lut, ei_stream stream);

/*
 * SiLU-gated product ([Handshake] C1, C4), elementwise over n values:
 *     idx  = clamp(floor((g + 16) / 32), -32768, 32768)   (Q16 -> Q11, add-half)
 *     h    = floor(lut[idx + 32768] * u / 2^16)            (Q16)
 *   gate, up, h  device int64 [n];  lut device int32 [65537]
 * An h outside int64 sets EI_DEV_OUT_RANGE.
 */
int silu_lut_epilogue(const int64_t* gate, const int64_t* up, const int32_t* lut, int64_t* h,
                      int64_t n, int32_t* d_status, ei_stream stream);

/* ------------------------------------- second derivations (table reads) */

/*
 * The 4-bit projection by the table read of [UORLUT01] "One projection
 * (definition)": per activation a 16-entry table T_j[q] = q x_j filled by
 * additions, one read per weight, four output rows per table, and the group
 * scale m 2^e applied by shifts and adds.  Reads the export format directly
 * and gives the same integers as int_gemm_q4 (a second implementation for
 * the two to be compared bit for bit; not the fast path).  K is cut into
 * chunks of 256 columns, one workgroup each; their exact sums meet in the
 * workspace.
 *   nib      device uint8 [n][k/2] (element 2j in the low nibble of byte j)
 *   sme      device uint8 [n][k/32] (m low nibble, e high nibble)
 *   x        device int32 [t][k];  y device int64 [t][n]
 *   workspace device scratch of ei_q4_table_workspace_bytes(n, k, t) bytes,
 *            16-byte aligned (none, and may be NULL, for k <= 256); owned by
 *            the caller, not kept after the call's work completes on the stream
 * EI_EINVAL for null pointers, n < 1, t < 1, k % 32 != 0, a misaligned
 * workspace; EI_ERANGE for
 * t > 65535 or k > 262,144; EI_ENOSPACE for a missing or short workspace; a
 * sum outside int64 sets EI_DEV_OUT_RANGE.
 */
size_t ei_q4_table_workspace_bytes(int64_t n, int64_t k, int64_t t);
int int_gemm_q4_table(const uint8_t* nib, const uint8_t* sme, const int32_t* x, int64_t* y, int64_t n, int64_t k,
                      int64_t t, void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream);

/*
 * silu_lut_epilogue with its runtime product lut[idx] * u formed as
 * [UORLUT01] "Products of two runtime values" does: the sixteen multiples of
 * the table value by repeated addition, read at each base-16 digit of |u|
 * and summed with shifts.  Same arguments and results as silu_lut_epilogue.
 */
int silu_lut_epilogue_radix16(const int64_t* gate, const int64_t* up, const int32_t* lut, int64_t* h, int64_t n,
                              int32_t* d_status, ei_stream stream);

/* ------------------------------------------------ wide-code GEMM */

/*
 * Wide integer codes ([tritify] 3.1: weights of 12 balanced trits,
 * |c| <= 265,720; activations int32 codes; 3.2 Matmul: the products are
 * accumulated exactly).  The repack splits every code into three balanced
 * base-256 digits (|c| <= 8,355,711 fits) in MFMA tile order.
 *   codes    device int32 [n][k], 16-byte aligned; k % 32 == 0
 *   packed   device, 256-byte aligned, ei_wide_packed_bytes(n, k) bytes
 * Synchronous (reads the header back).  EI_ERANGE if a code is outside the
 * three-digit range or n_pad * k * 3 >= 2^32.
 */
size_t ei_wide_packed_bytes(int64_t n, int64_t k);
int ei_wide_pack(const int32_t* codes, int64_t n, int64_t k, void* packed, size_t packed_bytes, ei_weights* out,
                 ei_stream stream);

/*
 * y[t][i] = sum_j c[i][j] * x[t][j], exact, int64 (no scale, no rounding):
 * activations split into 4 balanced digits, 12 digit products per 32x32
 * tile accumulated across K in the matrix cores' int32 accumulators, one
 * combination per output.
 *   w        descriptor from ei_wide_pack
 *   x        device int32 [t][k] in [-2^31, 2,139,062,143] (four balanced
 *            digits; larger values set EI_DEV_LIMB_RANGE)
 *   y        device int64 [t][n]
 * Workspace: ei_wide_workspace_bytes(w, t).  EI_ERANGE for k > 32768 (the
 * int32 accumulators' bound) or 4 * t_pad * k >= 2^32; a sum outside int64
 * sets EI_DEV_OUT_RANGE.
 */
size_t ei_wide_workspace_bytes(const ei_weights* w, int64_t t);
int int_gemm_wide(const ei_weights* w, const int32_t* x, int64_t* y, int64_t t, void* workspace,
                  size_t workspace_bytes, int32_t* d_status, ei_stream stream);

/* ------------------------------------------ requantization and norms */

/*
 * Fixed-point requantization ([tritify] 3.1, arithmetic specification: a
 * scale is an integer mantissa and a shift; scaling is a 128-bit product and
 * a round-half-away-from-zero arithmetic shift):
 *   y[e] = round_half_away(c[e] * m / 2^k),   0 <= k <= 126.
 *   c, y     device int64 [n] (may be the same buffer)
 * EI_EINVAL for null pointers with n > 0, n < 0 or k outside [0, 126]; a
 * result outside int64 is written as 0 and sets EI_DEV_OUT_RANGE.
 */
int ei_requant(const int64_t* c, int64_t m, int k, int64_t* y, int64_t n, int32_t* d_status, ei_stream stream);

/*
 * Integer RMSNorm of Q16 rows ([tritify] 3.2 Normalization: an exact integer
 * sum of squares, the inverse-RMS by an integer inverse square root, folded
 * into an integer scale and applied by one requantization):
 *   inv = floor(sqrt(2^104 d / (sum_i X_i^2 + d eps_q32)))     (2^52 / rms)
 *   Y_i = round_half_away(X_i * G_i * inv / 2^52)
 * i.e. Y = X G / sqrt(mean(X^2) + eps) in Q16 with the float-free scale; inv
 * is within 2^-29 of 2^52 / rms (relative).
 *   x        device int64 [t][d], Q16 codes with |X| <= 2^23
 *   g        device int32 [d], the norm weight in Q16
 *   eps_q32  eps * 2^32, in [1, 2^32]
 *   y        device int64 [t][d]
 * EI_EINVAL for null pointers, t < 1 or d < 1; EI_ERANGE for d > 65536 or
 * eps_q32 outside [1, 2^32]; |X| > 2^23 sets EI_DEV_LIMB_RANGE (that row's
 * output is not meaningful).
 */
int ei_rmsnorm_q16(const int64_t* x, const int32_t* g, int64_t eps_q32, int64_t* y, int64_t t, int64_t d,
                   int32_t* d_status, ei_stream stream);

/* ------------------------------------------------------- routing */

/*
 * Integer top-k routing ([tritify] 3.2 "Mixture-of-Experts": integer router
 * scores, the top-k selection an integer comparison with ties broken by
 * index).  route[t][s] = the expert of rank s of token t in the order (score
 * descending, expert index ascending).  The scores are typically a Q8
 * projection of the activations with the router's weights (int_gemm_q8 with
 * n = E); the result is the route int_gemm_q8_grouped / int_moe_ffn_q8 take.
 *   scores   device int64 [t][e]
 *   route    device int32 [t][k]
 * EI_EINVAL for null pointers, t < 1, e < 1, k < 1 or k > e; EI_ERANGE for
 * e > 2048.  Asynchronous on stream; no workspace.
 */
int ei_topk_route(const int64_t* scores, int64_t t, int64_t e, int k, int32_t* route, ei_stream stream);

/* ------------------------------------------------------- FFN layers */

/*
 * One feed-forward layer of Q8 projections with the SiLU gate ([Handshake]
 * C1 and C4: the committed SiLU table applied to the gate projection, the
 * gated product, the down projection, the residual stream):
 *   g = Q8(wg, x), u = Q8(wu, x), h = silu_lut_epilogue(g, u),
 *   y = x + Q8(wd, h).
 * Every value equals that sequence of int_gemm_q8 / silu_lut_epilogue calls
 * and an int64 add; for 5 to 63 tokens the gate and up projections share one
 * pass (the SiLU product in its epilogue, g and u never stored).
 *   wg, wu   descriptors [f][d] from ei_q8_pack (the same shape)
 *   wd       descriptor [d][f]
 *   x        device int64 [t][d], Q16 activations with |x| <= 2^22
 *   lut      device int32 [65537] from ei_silu_lut_build
 *   y        device int64 [t][d]; must not overlap x
 * Workspace: ei_ffn_workspace_bytes(wg, wd, t) bytes (EI_ENOSPACE if
 * smaller).  EI_EINVAL for null pointers, t < 1 or mismatched shapes; a sum
 * that leaves int64 sets EI_DEV_OUT_RANGE, an activation outside three limbs
 * EI_DEV_LIMB_RANGE.
 */
size_t ei_ffn_workspace_bytes(const ei_weights* wg, const ei_weights* wd, int64_t t);
int int_ffn_q8(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd, const int64_t* x,
               const int32_t* lut, int64_t* y, int64_t t, void* workspace, size_t workspace_bytes,
               int32_t* d_status, ei_stream stream);

/*
 * A stack of such layers in one call: x_{l+1} = int_ffn_q8(layer l, x_l) for
 * l = 0 .. n_layers - 1, y = x_{n_layers}.  Where the fused gate/up pass and
 * a split-K down projection apply, each layer's partial combiner also writes
 * the next layer's activation limb tiles, so no layer after the first splits
 * its input again.  Results equal n_layers calls of int_ffn_q8.
 *   layers   host array of 3 * n_layers descriptors: gate, up, down of each
 *            layer, all layers of one shape ([f][d], [f][d], [d][f])
 *   x, y     device int64 [t][d]; y must not overlap x
 * Workspace: ei_ffn_chain_workspace_bytes(gate, down, t) (any layer's).
 */
size_t ei_ffn_chain_workspace_bytes(const ei_weights* wg, const ei_weights* wd, int64_t t);
int int_ffn_q8_chain(const ei_weights* const* layers, int n_layers, const int64_t* x, const int32_t* lut, int64_t* y,
                     int64_t t, void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream);

/*
 * The same layer behind an integer RMSNorm ([tritify] 3.2 Normalization; the
 * pre-norm residual block): y = x + FFN(ei_rmsnorm_q16(x, g_norm, eps_q32)),
 * with FFN as int_ffn_q8 and the residual taken from x itself.  On the fused
 * path the normalized rows go straight into the gate/up limb tiles.
 *   g_norm   device int32 [d], Q16;  eps_q32 in [1, 2^32];  d <= 65536
 * Workspace: ei_ffn_workspace_bytes(wg, wd, t).  Errors as int_ffn_q8 and
 * ei_rmsnorm_q16.
 */
int int_ffn_q8_prenorm(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd, const int32_t* g_norm,
                       int64_t eps_q32, const int64_t* x, const int32_t* lut, int64_t* y, int64_t t,
                       void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream);

/*
 * A stack of pre-norm layers in one call: x_{l+1} = int_ffn_q8_prenorm(layer
 * l, g_norms[l], x_l) for l = 0 .. n_layers - 1, y = x_{n_layers}; results
 * equal n_layers calls of int_ffn_q8_prenorm.  Where the fused gate/up pass
 * and a split-K down projection apply, one kernel per token forms each
 * layer's output (residual plus the combined partials) and writes the next
 * layer's RMSNorm of it as that layer's activation limb tiles.
 *   layers   host array of 3 * n_layers descriptors as int_ffn_q8_chain
 *   g_norms  host array of n_layers device pointers, each int32 [d], Q16
 *   eps_q32  in [1, 2^32];  d <= 65536
 *   x, y     device int64 [t][d]; y must not overlap x
 * Workspace: ei_ffn_chain_workspace_bytes(gate, down, t).  Errors as
 * int_ffn_q8_chain and int_ffn_q8_prenorm.
 */
int int_ffn_q8_prenorm_chain(const ei_weights* const* layers, int n_layers, const int32_t* const* g_norms,
                             int64_t eps_q32, const int64_t* x, const int32_t* lut, int64_t* y, int64_t t,
                             void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream);

/*
 * The routed (mixture-of-experts) feed-forward layer ([tritify] 3.2
 * "Mixture-of-Experts": each selected expert is an exact-integer MLP; the
 * gate as in [Handshake] C1 and C4): for every pair (r, s), with
 * e = route[r][s],
 *   y[r * topk + s] = Q8(wd_e, silu_lut_epilogue(Q8(wg_e, x[r]), Q8(wu_e, x[r]))),
 * no residual and no combination over s (the router's weights are not part
 * of the layer).  The pairs are grouped by expert once for all three
 * projections.
 *   wg, wu   stacked descriptors [E][f][d] from ei_q8_pack_stacked
 *   wd       stacked descriptor [E][d][f]
 *   x        device int64 [rows][d]; route device int32 [rows][topk]
 *   y        device int64 [rows * topk][d]
 * Limits as int_gemm_q8_grouped; workspace ei_moe_ffn_workspace_bytes(wg,
 * wd, rows, topk).  An expert id outside [0, E) sets EI_DEV_ROUTE.
 */
size_t ei_moe_ffn_workspace_bytes(const ei_weights* wg, const ei_weights* wd, int64_t rows, int topk);
int int_moe_ffn_q8(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd, const int64_t* x,
                   const int32_t* route, int64_t rows, int topk, const int32_t* lut, int64_t* y, void* workspace,
                   size_t workspace_bytes, int32_t* d_status, ei_stream stream);

/*
 * FP32 shadow of the Q8 projection, the negative control of the schedule gate
 * ([Handshake] C3 and "Construction / Schedule gate": the same GEMM in float
 * under the five schedules splinters into several bit patterns).  Contrast
 * only: nothing on the exact path uses it.
 *     y[t][i] = the float32 sum of fl32(fl32(S[i][b] q[i][j] 2^-24) *
 *               fl32(x[t][j] 2^-16)) over j, one float32 rounding per product
 *               and per addition, in the schedule's order (EI_SCHED_DEFAULT
 *               and CANONICAL: j ascending; REVERSED: j descending;
 *               TILED_SHUFFLED: 128-column tiles in the splitmix64/Fisher-
 *               Yates permutation drawn from shuffle_seed; SPLIT_K: 8
 *               block-range partials added last to first; TREE: per-block sums
 *               in a pairwise tree)
 *   codes   device int8 [n][k] (canonical, not packed); scales device int32
 *           [n][k/32]; x device int64 [t][k]; y device float32 [t][n]
 * Errors: EI_EINVAL for null pointers, bad sizes or schedule.
 */
int ei_q8_fp32_shadow(const int8_t* codes, const int32_t* scales, const int64_t* x, float* y, int64_t n, int64_t k,
                      int64_t t, int schedule, uint64_t shuffle_seed, ei_stream stream);

/* -------------------------------------------------------- digests */

/*
 * SHA-256 of the raw bytes of a device buffer ([tritify] 4: the integer
 * output carries a reproducing SHA-256).  Synchronous: waits for `stream`,
 * copies the bytes to host memory (allocated and freed inside the call)
 * and hashes them.
 *   out     host uint8 [32]
 */
int output_digest(const void* dptr, size_t nbytes, uint8_t* out, ei_stream stream);

/* SHA-256 (FIPS 180-4) of a host buffer; host-only, no device work. */
void ei_sha256_host(const void* data, size_t nbytes, uint8_t* out);

/* Human-readable name of a return code. */
const char* ei_status_string(int code);

/* Library ABI version (major * 100 + minor). */
int ei_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_INT_H */
