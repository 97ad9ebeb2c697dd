// Internal declarations shared by the library's translation units.
// Not installed; the public interface is include/exact_int.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "exact_int.h"

namespace ei {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr uint32_t kMagic = 0x31514945u;   // "EIQ1"
constexpr int kHeaderBytes = 256;
constexpr int kTile = 32;                   // rows per row group, tokens per token group, columns per block
constexpr int kTileBytes = 1024;            // one 32x32 int8 tile in MFMA lane order
constexpr int64_t kMaxK = 262144;           // per-limb int64 sums exact up to here (2^13 blocks x 2^50)
constexpr int kMaxLimbs = 4;                // the largest limb count the kernels are instantiated for

// The packed weight buffer starts with this header (device memory).
struct PackedHeader {
  uint32_t magic;
  int32_t format;
  int64_t n, k, n_pad, nb;
  uint32_t smax;     // max |scale| (written by the pack pass with atomicMax)
  uint32_t pad0;
  int64_t codes_off, scales_off;
  int64_t roff_off;  // row offsets, int64 [n_pad] (4-bit images; zero in Q8 images)
};
static_assert(sizeof(PackedHeader) <= kHeaderBytes, "header too large");

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Three-limb accumulation in two int64 chains per output instead of one per
// limb: S (P_0 + 2^8 P_1) and (2^16 S) P_2, each multiply-add on 32-bit
// operands.  With |P_l| <= 32 * 128 * 128 = 2^19 a block adds at most
// |S| (2^27 + 2^19) to the first chain and |S| 2^35 to the second, so both
// chains and their sum stay below 2^62.01 (and 2^16 S fits int32) whenever
// max|S| < 2^15 and nb * max|S| <= 2^27.
inline bool narrow_scales(uint32_t smax, int64_t nb) {
  return smax < 32768u && (uint64_t)smax * (uint64_t)nb <= ((uint64_t)1 << 27);
}

// Bytes of the code tiles of an n_pad x k packed matrix: (n_pad / 32) row
// groups of nb 1 KB tiles, i.e. one byte per code.  Kernels size the buffer
// resource over a whole matrix's codes with this (host checks keep it below
// 2^32).
__host__ __device__ inline int64_t code_bytes(int64_t n_pad, int64_t nb) { return n_pad * nb * 32; }

// header, code tiles, scales [n_pad/32][nb][32] int32, row offsets [n_pad] int64
__host__ __device__ inline size_t row_offsets_at(int64_t n_pad, int64_t k) {
  return (size_t)kHeaderBytes + (size_t)n_pad * (size_t)k + (size_t)n_pad * (size_t)(k / 32) * 4u;
}
inline size_t packed_bytes(int64_t n, int64_t k) {
  const int64_t n_pad = round_up(n, kTile);
  return row_offsets_at(n_pad, k) + (size_t)n_pad * 8u;
}

// The 4-bit projection's two-limb form: activations are split as x - kQ4Offset
// (two balanced base-256 digits hold exactly [-2^15, 2^15) then), and row i's
// output gets R_i = kQ4Offset * (row i's weight sum) added back, since the
// projection is linear in x.
constexpr int64_t kQ4Offset = 128;

// Output modes of the projection kernels.
enum OutMode : int {
  OUT_ROUND_Q24 = 0,   // y = floor((acc + 2^23) / 2^24)       (Q8)
  OUT_EXACT = 1,       // y = acc, checked to fit int64          (Q4)
  OUT_PARTIAL = 2,     // partial sums to workspace: per limb [part][L][T][N] (the skinny kernel
                       // writes (h, r) pairs [part][2][T][N] for up to three limbs)
  OUT_TERMS = 3        // per-limb int64 per-block terms to workspace [b][L][T][N]
};

// Block visiting orders inside a kernel.
enum BlockOrder : int { ORDER_ASC = 0, ORDER_DESC = 1, ORDER_PERM = 2 };

// Everything a projection kernel launch needs.
struct GemmArgs {
  const int8_t* codes;       // packed code tiles
  const int32_t* scales;     // packed scales
  const void* x;             // int64 (Q8) or int32 (Q4) activations [T][K]
  int x_is_i32;
  const int8_t* limb_tiles;  // [L][t_pad/32][nb][1 KB] (MFMA path)
  int64_t* y;                // [T][N]
  int64_t* part;             // OUT_PARTIAL / OUT_TERMS destination
  const int32_t* kperm;      // ORDER_PERM: block order [nb]
  const int32_t* tperm;      // tile order for the shuffled schedule (or null)
  int32_t* status;           // device status word (or null)
  int64_t n, k, t, n_pad, t_pad, nb;
  int64_t b0, b1;            // block range [b0, b1)
  int part_index;            // OUT_PARTIAL: which partial this launch writes
  int out_mode, order;
  int chunk;                 // GEMV: blocks per wave per LDS limb chunk (a multiple of its prefetch depth)
  // grouped (expert) launches: token tile j holds sorted pairs
  // tile_row0[j] .. + tile_rows[j] - 1 of expert tile_expert[j]; sorted pair
  // i is original pair sorted_pair[i], whose output row it is
  const int32_t* tile_expert;
  const int32_t* tile_row0;
  const int32_t* tile_rows;
  const int32_t* sorted_pair;
  const int32_t* ntiles;     // device: tiles in use (<= tiles_max)
  int64_t tiles_max;
  int64_t expert_stride;     // bytes between the packed images of two experts
  // fused FFN launches: a second weight matrix of the same shape (the up
  // projection) whose result meets the first's in the SiLU-gated product,
  // and a residual added to the final output (y = resid + result)
  const int8_t* codes2;
  const int32_t* scales2;
  const int32_t* lut;
  const int64_t* resid;
  int8_t* limb_out;          // fused gate/up: h as limb tiles [3][t_pad/32][n/32][1 KB]
  // two-limb 4-bit form: x_off is subtracted from every (int32) activation
  // before its split, row_off[i] added to output row i as it is finished
  int64_t x_off;
  const int64_t* row_off;
};

// Matrices of one batched GEMV launch (same k, same activations): matrix m
// owns the launch's row groups rg0[m] .. rg0[m + 1] - 1.
constexpr int kMultiMax = 16;
struct GemvMulti {
  const int8_t* codes[kMultiMax];
  const int32_t* scales[kMultiMax];
  int64_t* y[kMultiMax];
  int64_t n[kMultiMax], n_pad[kMultiMax];
  int64_t rg0[kMultiMax + 1];
  int count;
};

// Work item of a grouped (routed) launch over a grid of rbs x tiles_max
// workgroups: the rbs * ntiles items in use go token tile by token tile
// (w = tb * rbs + rb, row blocks fastest), so the workgroups that read one
// token tile's activation limb tiles, and then the token tiles of one expert,
// which read the same weight rows, run together.  Workgroup blk runs on XCD
// blk % 8: each XCD takes a contiguous run of an eighth of the items in use,
// so the unused tail of the grid is shared out evenly too.  False: no item.
__device__ inline bool grouped_item(int64_t blk, int64_t grid, int64_t rbs, int64_t ntiles, int64_t* rb,
                                    int64_t* tb) {
  const int64_t active = rbs * ntiles;
  int64_t w = blk;
  if (grid % 8 == 0) {
    const int64_t x = blk % 8, l = blk / 8;
    const int64_t s0 = x * active / 8, s1 = (x + 1) * active / 8;
    if (l >= s1 - s0) return false;
    w = s0 + l;
  } else if (blk >= active) {
    return false;
  }
  *tb = w / rbs;
  *rb = w % rbs;
  return true;
}

// pos-th block visited by a kernel in the block range [b0, b1) of `a`.
__device__ inline int64_t block_at(const GemmArgs& a, int64_t pos) {
  if (a.order == ORDER_DESC) return a.b1 - 1 - pos;
  if (a.order == ORDER_PERM) return a.kperm[a.b0 + pos];
  return a.b0 + pos;
}

// Launchers (each defined in the translation unit that holds its kernel).
hipError_t launch_pack_q8(const int8_t* codes, const int32_t* scales, int64_t n, int64_t k,
                          void* packed, hipStream_t s);
hipError_t launch_pack_q4(const uint8_t* nib, const uint8_t* sme, int64_t n, int64_t k,
                          void* packed, hipStream_t s);
hipError_t launch_limb_split_flat(const int64_t* x, int8_t* d, int64_t n, int limbs,
                                  int32_t* status, hipStream_t s);
// x_off: subtracted from every activation before its split (int32 x only)
hipError_t launch_limb_tiles(const void* x, int x_is_i32, int64_t t, int64_t k, int limbs,
                             int8_t* tiles, int64_t t_pad, int32_t* status, hipStream_t s, int64_t x_off = 0);
hipError_t launch_gemv(const GemmArgs& a, int limbs, hipStream_t s);
// a carries k, t, x, the block range and status; mm the matrices and outputs
hipError_t launch_gemv_multi(const GemmArgs& a, const GemvMulti& mm, int limbs, hipStream_t s);
hipError_t launch_gemm_mfma(const GemmArgs& a, int limbs, hipStream_t s);
// narrow: the scales allow two int64 accumulators per output (narrow_scales);
// otherwise one per limb
hipError_t launch_gemm_tiled(const GemmArgs& a, bool narrow, hipStream_t s);    // 3 limbs, see tiled_ok()
hipError_t launch_gemm_grouped(const GemmArgs& a, bool narrow, hipStream_t s);  // 3 limbs
// narrow scales only (the register-fed tiled kernel), dense or grouped
hipError_t launch_gemm_tiled_qreg(const GemmArgs& a, bool grouped, hipStream_t s);
// grouped gate (a.codes, a.scales) and up (a.codes2, a.scales2, same shape and
// expert stride) projections in one pass; writes h = SiLU-gated product as
// limb tiles [3][tiles_max][n/32][1 KB] (a.limb_out); n % 32 == 0
hipError_t launch_gemm_grouped_gateup(const GemmArgs& a, bool narrow, hipStream_t s);
int skinny_splits(int64_t n_pad, int64_t t_pad, int64_t nb);       // workgroup K splits of the skinny kernel
// a.part when splits > 1: (h, r) partials [splits][2][t][n] for up to three
// limbs, per-limb partials [splits][limbs][t][n] for four
hipError_t launch_gemm_skinny(const GemmArgs& a, int limbs, int splits, bool narrow, hipStream_t s);   // narrow: 3 limbs
hipError_t launch_moe_sort(const int32_t* route, int64_t pairs, int64_t experts, int32_t* sorted_pair,
                           int32_t* offsets, int32_t* tile_expert, int32_t* tile_row0, int32_t* tile_rows,
                           int32_t* ntiles, int32_t* status, hipStream_t s);
hipError_t launch_grouped_limb_tiles(const int64_t* x, int64_t k, int topk, const int32_t* sorted_pair,
                                     const int32_t* tile_row0, const int32_t* tile_rows, const int32_t* ntiles,
                                     int64_t tiles_max, int8_t* tiles, int32_t* status, hipStream_t s);
// row_off (exact outputs only): row_off[i] is added to output row i
hipError_t launch_combine_partials(const int64_t* part, int nparts, int64_t* y, int64_t t, int64_t n,
                                   int limbs, int out_mode, const int64_t* resid, int32_t* status, hipStream_t s,
                                   const int64_t* row_off = nullptr);
hipError_t launch_combine_hr(const int64_t* part, int nparts, int64_t* y, int64_t t, int64_t n, int out_mode,
                             const int64_t* resid, int32_t* status, hipStream_t s,
                             const int64_t* row_off = nullptr);   // (h, r) partials
hipError_t launch_combine_hr_tiles(const int64_t* part, int nparts, int64_t* y, int64_t t, int64_t n,
                                   const int64_t* resid, int8_t* tiles, int64_t t_pad, int32_t* status,
                                   hipStream_t s);   // Q8 rounding; n % 32 == 0
hipError_t launch_add_residual(int64_t* y, const int64_t* resid, int64_t n, int32_t* status, hipStream_t s);
hipError_t launch_gemm_skinny_gateup(const GemmArgs& a, bool narrow, hipStream_t s);   // 3 limbs, one split
// A projection with narrow scales at t <= 64 in one launch on 16 x 16 tiles:
// y = resid + Q8-rounded result, and, if a.limb_out is set, y's limb tiles
// [3][t_pad/32][n/32][1 KB] (n % 32 == 0).  skinny16_finish_fits: the shapes
// it takes.
bool skinny16_finish_fits(int64_t n, int64_t nb, int64_t t);
hipError_t launch_skinny16_finish(const GemmArgs& a, hipStream_t s);
hipError_t launch_tree_terms(int64_t* terms, int64_t nb, int64_t* y, int64_t t, int64_t n,
                             int limbs, int out_mode, int32_t* status, hipStream_t s,
                             const int64_t* row_off = nullptr);
hipError_t launch_make_perm(int32_t* perm, int64_t n, uint64_t seed, hipStream_t s);
hipError_t launch_silu_lut(int32_t* lut, hipStream_t s);
hipError_t launch_wide_pack(const int32_t* codes, int64_t n, int64_t k, int64_t n_pad, int8_t* tiles, uint32_t* bad,
                            hipStream_t s);
hipError_t launch_wide_gemm(const int8_t* wtiles, const int8_t* atiles, int64_t* y, int64_t n, int64_t t,
                            int64_t n_pad, int64_t t_pad, int64_t nb, int32_t* status, hipStream_t s);
// workspace: q4_table_workspace_bytes(n, k, t) bytes (int128 chunk sums), or none for k <= 256
size_t q4_table_workspace_bytes(int64_t n, int64_t k, int64_t t);
hipError_t launch_q4_table(const uint8_t* nib, const uint8_t* sme, const int32_t* x, int64_t* y, int64_t n,
                           int64_t k, int64_t t, void* workspace, int32_t* status, hipStream_t s);
hipError_t launch_silu_mul_radix16(const int64_t* g, const int64_t* u, const int32_t* lut, int64_t* h, int64_t n,
                                   int32_t* status, hipStream_t s);
hipError_t launch_topk(const int64_t* scores, int64_t t, int64_t e, int k, int32_t* route, hipStream_t s);
hipError_t launch_rmsnorm_q16(const int64_t* x, const int32_t* g, int64_t eps, int64_t* y, int64_t t, int64_t d,
                              int32_t* status, hipStream_t s);
hipError_t launch_rmsnorm_limb_tiles(const int64_t* x, const int32_t* g, int64_t eps, int8_t* tiles, int64_t t,
                                     int64_t t_pad, int64_t d, int32_t* status, hipStream_t s);   // d % 32 == 0
// y = resid + combined (h, r) partials [nparts][2][t][d]; tiles = limb tiles of rmsnorm(y, g, eps); d % 32 == 0
hipError_t launch_combine_rmsnorm_tiles(const int64_t* part, int nparts, const int64_t* resid, int64_t* y,
                                        const int32_t* g, int64_t eps, int8_t* tiles, int64_t t, int64_t t_pad,
                                        int64_t d, int32_t* status, hipStream_t s);
hipError_t launch_requant(const int64_t* c, int64_t m, int k, int64_t* y, int64_t n, int32_t* status,
                          hipStream_t s);
hipError_t launch_shadow(const int8_t* q, const int32_t* s, const int64_t* x, float* y, int64_t n, int64_t k,
                         int64_t t, int schedule, uint64_t seed, hipStream_t st);
hipError_t launch_silu_mul(const int64_t* g, const int64_t* u, const int32_t* lut, int64_t* h,
                           int64_t n, int32_t* status, hipStream_t s);

void sha256(const void* data, size_t n, uint8_t out[32]);

// ---------------------------------------------------------------- device
// v as int64, or false if it does not fit.
__device__ inline bool fit_i64(__int128 v, int64_t* out) {
  const __int128 lo = -((__int128)1 << 63), hi = ((__int128)1 << 63) - 1;
  if (v < lo || v > hi) { *out = 0; return false; }
  *out = (int64_t)v;
  return true;
}

// Combine per-limb int64 sums A_l into sum_l 2^(8l) A_l (int128) and apply
// the output rounding.  Returns false if the result does not fit int64.
__device__ inline bool finish_output(__int128 acc, int mode, int64_t* out) {
  __int128 v = acc;
  if (mode == OUT_ROUND_Q24) v = (acc + ((__int128)1 << 23)) >> 24;   // arithmetic: floor
  const __int128 lo = -((__int128)1 << 63), hi = ((__int128)1 << 63) - 1;
  if (v < lo || v > hi) { *out = 0; return false; }
  *out = (int64_t)v;
  return true;
}

// acc = a0 + 2^8 a1 + 2^16 a2 (any int64 a_l) as acc = 2^24 h + r without
// 128-bit arithmetic: with a_l = h_l 2^(24-8l) + r_l, 0 <= r_l < 2^(24-8l)
// (arithmetic shifts and masks), h = h_0 + h_1 + h_2 and r = r_0 + 2^8 r_1 +
// 2^16 r_2 in [0, 3 * 2^24).  |h_l| < 2^39, 2^47, 2^55, so nothing overflows.
// The pair is additive: sums of (h, r) over disjoint block ranges give the
// (h, r) of the whole sum, with r below 2^24 times the number of terms.
__device__ inline void split_hr(int64_t a0, int64_t a1, int64_t a2, int64_t* h, int64_t* r) {
  *h = (a0 >> 24) + (a1 >> 16) + (a2 >> 8);
  *r = (a0 & 0xFFFFFF) + ((a1 & 0xFFFF) << 8) + ((a2 & 0xFF) << 16);
}

// y from acc = 2^24 h + r (r >= 0): Q8 rounding floor((acc + 2^23) / 2^24) =
// h + floor((r + 2^23) / 2^24), which cannot overflow for |h| < 2^62 and
// r < 2^62; or the exact acc, checked to fit int64.
__device__ inline bool finish_hr(int64_t h, int64_t r, int mode, int64_t* out) {
  if (mode == OUT_ROUND_Q24) {
    *out = h + ((r + ((int64_t)1 << 23)) >> 24);
    return true;
  }
  return fit_i64((__int128)h * ((__int128)1 << 24) + r, out);
}

__device__ inline int64_t round_q24_3(int64_t a0, int64_t a1, int64_t a2) {
  int64_t h, r;
  split_hr(a0, a1, a2, &h, &r);
  return h + ((r + ((int64_t)1 << 23)) >> 24);
}

// Balanced base-256 digits d_l in [-128, 127] with v = sum_{l<L} 256^l d_l
// (unique: the digit set is a complete residue system mod 256), for four
// values at once, packed per limb: byte p of w[l] is d_l of v[p].  With u = v + 128 * (1 + 256 + ... + 256^(L-1)), the
// ordinary base-256 digits of u are d_l + 128, and v fits L digits exactly
// when 0 <= u < 2^(8L); d_l + 128 -> d_l as a byte is an XOR with 0x80.
// The bytes are gathered with v_perm_b32 (selector byte k picks byte k of
// the pair {S1 = bytes 0-3, S0 = bytes 4-7}; 0x0c gives zero).  L <= 4.
template <int L>
__device__ inline bool limb_words(const int64_t (&v)[4], uint32_t (&w)[L]) {
  static_assert(L >= 1 && L <= 4, "limb_words handles 1..4 limbs");
  constexpr uint64_t kBias = 0x8080808080808080ull >> (64 - 8 * L);
  uint32_t lo[4];
  uint64_t bad = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint64_t u = (uint64_t)v[p] + kBias;
    bad |= u >> (8 * L);
    lo[p] = (uint32_t)u ^ 0x80808080u;
  }
#pragma unroll
  for (int l = 0; l < L; ++l) {
    const uint32_t sel = 0x0c0c0000u | ((uint32_t)(4 + l) << 8) | (uint32_t)l;   // [byte l of S1, byte l of S0, 0, 0]
    const uint32_t a = __builtin_amdgcn_perm(lo[1], lo[0], sel);
    const uint32_t b = __builtin_amdgcn_perm(lo[3], lo[2], sel);
    w[l] = __builtin_amdgcn_perm(b, a, 0x05040100u);                             // [a0, a1, b0, b1]
  }
  return bad == 0;
}

// Buffer resource (V#) over `bytes` bytes at `base`, for raw buffer loads:
// a scalar base and a per-load scalar offset leave only the lane offset in a
// VGPR.  Word 3 is the gfx9 raw-buffer configuration (32-bit data format).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct-to-LDS copy of 16 bytes per lane from buffer r at voffset +
// soffset; lane i writes LDS bytes dst + 16 i .. +15.  (A device function of
// its own: the host pass of a kernel must not see the LDS address space.)
__device__ inline void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voffset, soffset, 0, 0);
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding, as an instruction the compiler's own wait insertion takes into
// account (it cannot see into inline asm, and would otherwise add a wait of
// its own, down to zero, before the first use of a register loaded N
// requests back).  s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; the last two are left at their maxima (no wait).
template <int N>
__device__ inline void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier once at most N of this wave's vector-memory operations
// (direct-to-LDS copies of later blocks) are outstanding and its LDS reads
// are done.  __syncthreads would wait for every copy in flight.
template <int N>
__device__ inline void barrier_after_vmcnt() {
  vmcnt_wait<N>();
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ inline void flag(int32_t* status, int bits) {
  if (status) atomicOr(status, bits);
}

// SiLU-gated product: h = floor(lut[clamp(floor((g + 16) / 32), -32768,
// 32768) + 32768] * u / 2^16); false if h does not fit int64.
__device__ inline bool silu_gate(int64_t g, int64_t u, const int32_t* __restrict__ lut, int64_t* h) {
  // floor((g + 16) / 32) without overflowing at the int64 ends
  int64_t idx = (g >> 5) + ((g & 31) >= 16 ? 1 : 0);
  idx = idx < -32768 ? -32768 : (idx > 32768 ? 32768 : idx);
  const __int128 p = (__int128)lut[idx + 32768] * (__int128)u;
  return fit_i64(p >> 16, h);   // arithmetic shift: floor
}

}  // namespace ei
