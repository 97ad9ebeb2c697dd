// Tiled exact projection for many tokens: the prefill GEMM.
//
// Computes, for three activation limbs d_0, d_1, d_2 (x = d_0 + 2^8 d_1 +
// 2^16 d_2) and every (token t, row i), the per-limb sums
//     A_l[t][i] = sum_b S[i][b] * P_l[t][i][b],
//     P_l[t][i][b] = sum_{j in b} q[i][j] * d_l[t][j]          (int32, exact)
// in int64 (|S P_l| < 2^31 * 2^19 = 2^50, so any partial sum over up to 2^13
// blocks is exact for any int32 scale), then acc = A_0 + 2^8 A_1 + 2^16 A_2
// in int128 and y = floor((acc + 2^23) / 2^24) (or acc).  Every step is exact
// integer arithmetic, so the result is the same bits as any other
// evaluation order.
// When the matrix's scales are narrow (max|S| < 2^15 and nb max|S| <= 2^27,
// checked on the host from the packed header) the register-fed kernel keeps
// two chains per output instead: S (P_0 + 2^8 P_1) and (2^16 S) P_2, both
// below 2^62.01 -- two multiply-adds per element instead of three.  (One
// shared chain would save registers, but the compiler then re-associates the
// two dependent multiply-adds into three operations.)
//
// Work split.  A workgroup of 4 waves owns a tile of 32 RT WR rows x
// 32 TT (4 / WR) tokens; each wave owns RT x TT 32x32 MFMA tiles.  Per
// 32-wide block the workgroup needs its code tiles, 3 limb tiles per token
// tile (1 KB each, already in MFMA lane order in global memory) and the
// scales of its rows; they are copied global -> LDS with direct-to-LDS
// buffer loads (no VGPR round trip, scalar block offsets) into a ring of
// NBUF one-block buffers, NBUF - 1 blocks ahead of use.  Per block a wave
// issues 3 RT TT v_mfma_i32_32x32x32_i8 and, per output element, three
// v_mad_i64_i32 (narrow: two and a shift-add): this VALU epilogue, which the
// matrix cores only partly overlap, is the critical resource.
#include "ei_internal.h"

namespace ei {

// Shape of a tiled launch: each of the 4 waves owns RT x TT MFMA tiles; the
// waves are arranged WR x (4 / WR) over rows x tokens.
template <int RT, int TT, int WR>
struct TiledShape {
  static constexpr int WT = 4 / WR;
  static constexpr int kRowTiles = RT * WR, kTokTiles = TT * WT;        // per workgroup
  static constexpr int kRows = 32 * kRowTiles, kToks = 32 * kTokTiles;
  static constexpr int kCodeOff = 0, kLimbOff = kRowTiles * 1024;
  static constexpr int kScaleOff = kLimbOff + 3 * kTokTiles * 1024;
  static constexpr int kCopies = kRowTiles + 3 * kTokTiles;            // 1 KB tiles per block
  static constexpr int kPerWave = (kCopies + 3) / 4;
  static constexpr int kPad = kPerWave * 4 - kCopies;                  // dummy copies
  static constexpr int kBlockBytes = kScaleOff + kRowTiles * 128 + kPad * 1024;
};

// kGrouped: each token tile belongs to one expert, whose packed image and
// output rows it looks up.  PIPE: the epilogue of block b runs after the
// MFMAs of block b + 1 are issued.  XMAP: XCD-contiguous tile order.
template <int RT, int TT, int WR, int NBUF, bool kExact, bool kGrouped, bool PIPE, bool XMAP>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmArgs a) {
  using Sh = TiledShape<RT, TT, WR>;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave % WR, wt = wave / WR;

  // ---- tile of this workgroup
  const int64_t tbs = kGrouped ? a.tiles_max : (a.t_pad + Sh::kToks - 1) / Sh::kToks;
  // XMAP: workgroup g runs on XCD g % 8; give each XCD a contiguous run of
  // tiles (token tiles fastest), so a row block's code tiles are fetched into
  // one XCD's L2 and reused there by the token tiles that follow
  const int64_t rbs = (a.n_pad + Sh::kRows - 1) / Sh::kRows, ntiles = rbs * tbs;
  int64_t g = blockIdx.x;
  if (XMAP && ntiles % 8 == 0) g = (g % 8) * (ntiles / 8) + g / 8;
  const int64_t rb = g / tbs, tb = g % tbs;
  const int64_t rgs = a.n_pad / kTile, tgs = kGrouped ? a.tiles_max : a.t_pad / kTile;
  const int8_t* codes = a.codes;
  const int32_t* scales = a.scales;
  if (kGrouped) {
    static_assert(!kGrouped || (TT == 1 && WR == 4), "grouped launches use one token tile per workgroup");
    if (tb >= *a.ntiles) return;   // the whole workgroup: no tile here
    const int64_t e = a.tile_expert[tb];
    codes += e * a.expert_stride;
    scales = reinterpret_cast<const int32_t*>(reinterpret_cast<const int8_t*>(scales) + e * a.expert_stride);
  }

  // ---- copies of one block: every wave issues kPerWave tile copies
  // (j = wave + 4 i; j < kRowTiles: code tile j, then the limb tiles, then
  // dummy copies into a pad area) and one copy of the scales of its own row
  // tiles, so that every wave has the same number of loads per block.  Row
  // and token groups past the matrix re-read the last one (results unused).
  // Scalar offsets of tile j at block 0; block b adds b * 1 KB.
  const __amdgpu_buffer_rsrc_t rcode = make_rsrc(codes, (uint32_t)code_bytes(a.n_pad, a.nb));
  const __amdgpu_buffer_rsrc_t rlimb = make_rsrc(a.limb_tiles, (uint32_t)(3 * tgs * a.nb * 1024));
  const __amdgpu_buffer_rsrc_t rscal = make_rsrc(scales, (uint32_t)(a.n_pad * a.nb * 4));
  uint32_t soff[Sh::kPerWave];
  bool is_code[Sh::kPerWave];
  int dst_off[Sh::kPerWave];
#pragma unroll
  for (int i = 0; i < Sh::kPerWave; ++i) {
    const int j = wave + 4 * i;
    is_code[i] = true;
    if (j < Sh::kRowTiles) {
      int64_t rg = Sh::kRowTiles * rb + j;
      rg = rg < rgs ? rg : rgs - 1;
      soff[i] = (uint32_t)(rg * a.nb * 1024);
      dst_off[i] = Sh::kCodeOff + j * 1024;
    } else if (j < Sh::kCopies) {
      const int jj = j - Sh::kRowTiles;
      const int l = jj / Sh::kTokTiles, tt = jj % Sh::kTokTiles;
      int64_t tg = Sh::kTokTiles * tb + tt;
      tg = tg < tgs ? tg : tgs - 1;
      is_code[i] = false;
      soff[i] = (uint32_t)(((int64_t)l * tgs + tg) * a.nb * 1024);
      dst_off[i] = Sh::kLimbOff + (l * Sh::kTokTiles + tt) * 1024;
    } else {   // dummy: re-read this workgroup's first code tile into the pad area
      int64_t rg = Sh::kRowTiles * rb;
      rg = rg < rgs ? rg : rgs - 1;
      soff[i] = (uint32_t)(rg * a.nb * 1024);
      dst_off[i] = Sh::kScaleOff + Sh::kRowTiles * 128 + (j - Sh::kCopies) * 1024;
    }
  }
  // scales: lane i < 8 RT copies 16 B of the wave's row tile RT wr + i / 8
  // (the row group's offset rides in the lane offset, the block's in the
  // scalar one); the direct-to-LDS copy puts lane i at sdst + 16 i
  uint32_t svoff;
  {
    const int jr = RT * wr + (lane >> 3) % RT;
    int64_t rg = Sh::kRowTiles * rb + jr;
    rg = rg < rgs ? rg : rgs - 1;
    svoff = (uint32_t)(rg * a.nb * 128) + (lane & 7) * 16;
  }
  const int sdst = Sh::kScaleOff + RT * wr * 128;
  auto issue = [&](int64_t b) {
    uint8_t* blk = lds + (int)(b % NBUF) * Sh::kBlockBytes;
#pragma unroll
    for (int i = 0; i < Sh::kPerWave; ++i)
      copy16_to_lds(is_code[i] ? rcode : rlimb, blk + dst_off[i], lane * 16, soff[i] + (uint32_t)b * 1024u);
    if (lane < 8 * RT)   // one load instruction per wave either way: the per-wave count stays uniform
      copy16_to_lds(rscal, blk + sdst, svoff, (uint32_t)b * 128u);
  };

  int64_t acc[3][RT][TT][16];
#pragma unroll
  for (int c = 0; c < 3; ++c)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][rt][tt][r] = 0;
  const v16i zero = {};

  const int64_t nb = a.nb;
  // Block b: wait for its copies (all waves), start the copy of block
  // b + NBUF - 1 into the buffer block b - 1 used, read the operands and
  // scales into registers, issue the MFMAs.  The epilogue of a block needs
  // only registers, so with PIPE it runs one block later, while the matrix
  // cores work on the next block; two named register sets (A, B) keep the
  // loop free of copies.
  using Dset = v16i[RT][TT][3];
  auto step = [&](int64_t b, Dset& D, int32_t (&S)[RT]) {
    // (__syncthreads would also wait for the copies still in flight)
    if (b + NBUF - 2 < nb)
      barrier_after_vmcnt<(NBUF - 2) * (Sh::kPerWave + 1)>();
    else
      barrier_after_vmcnt<0>();
    if (b + NBUF - 1 < nb) issue(b + NBUF - 1);
    const uint8_t* blk = lds + (int)(b % NBUF) * Sh::kBlockBytes;
    v4i q[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int jr = RT * wr + rt;
      q[rt] = *reinterpret_cast<const v4i*>(blk + Sh::kCodeOff + jr * 1024 + lane * 16);
      S[rt] = *reinterpret_cast<const int32_t*>(blk + Sh::kScaleOff + (jr * 32 + (lane & 31)) * 4);
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int jt = TT * wt + tt;
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        const v4i d = *reinterpret_cast<const v4i*>(blk + Sh::kLimbOff + (l * Sh::kTokTiles + jt) * 1024 + lane * 16);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) D[rt][tt][l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(d, q[rt], zero, 0, 0, 0);
      }
    }
  };
  auto epilogue = [&](const Dset& D, const int32_t (&S)[RT]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int l = 0; l < 3; ++l) acc[l][rt][tt][r] += (int64_t)S[rt] * D[rt][tt][l][r];
  };

  for (int64_t b = 0; b < NBUF - 1 && b < nb; ++b) issue(b);
  Dset DA, DB;
  int32_t SA[RT], SB[RT];
  if (PIPE) {
    step(0, DA, SA);
    for (int64_t b = 0; b < nb; b += 2) {
      if (b + 1 < nb) step(b + 1, DB, SB);
      epilogue(DA, SA);
      if (b + 1 < nb) {
        if (b + 2 < nb) step(b + 2, DA, SA);
        epilogue(DB, SB);
      }
    }
  } else {
    for (int64_t b = 0; b < nb; ++b) {
      step(b, DA, SA);
      epilogue(DA, SA);
    }
  }

  // ---- store: lane holds row 32 jr + lane % 32 and tokens 32 jt + 8 (r / 4)
  // + 4 (lane / 32) + r % 4 of the workgroup tile
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t row = rb * Sh::kRows + (RT * wr + rt) * 32 + (lane & 31);
    if (row >= a.n) continue;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tloc = (TT * wt + tt) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        int64_t orow;   // output row of this token (grouped: the original pair)
        if (kGrouped) {
          if (tloc >= a.tile_rows[tb]) continue;
          orow = a.sorted_pair[a.tile_row0[tb] + tloc];
        } else {
          orow = tb * Sh::kToks + tloc;
          if (orow >= a.t) continue;
        }
        const __int128 v = (__int128)acc[0][rt][tt][r] + ((__int128)acc[1][rt][tt][r] << 8) +
                           ((__int128)acc[2][rt][tt][r] << 16);
        int64_t out;
        if (!finish_output(v, kExact ? OUT_EXACT : OUT_ROUND_Q24, &out)) flag(a.status, EI_DEV_OUT_RANGE);
        a.y[orow * a.n + row] = out;
      }
  }
}

template <int RT, int TT, int WR, int NBUF, bool kGrouped = false, bool PIPE = false, bool XMAP = false>
hipError_t launch_tiled_shape(const GemmArgs& a, hipStream_t s) {
  using Sh = TiledShape<RT, TT, WR>;
  const int64_t rbs = (a.n_pad + Sh::kRows - 1) / Sh::kRows;
  const int64_t tbs = kGrouped ? a.tiles_max : (a.t_pad + Sh::kToks - 1) / Sh::kToks;
  const dim3 grid((unsigned)(rbs * tbs)), block(256);
  const size_t lds = (size_t)NBUF * Sh::kBlockBytes;
  if (a.out_mode == OUT_EXACT)
    hipLaunchKernelGGL((gemm_tiled_kernel<RT, TT, WR, NBUF, true, kGrouped, PIPE, XMAP>), grid, block, lds, s,
                       a);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<RT, TT, WR, NBUF, false, kGrouped, PIPE, XMAP>), grid, block, lds,
                       s, a);
  return hipGetLastError();
}

// ================================================================ register-fed form
// The narrow-scale tiled projection: the same 128-row x 32-token workgroup
// tiles (XCD-contiguous order), one 32x32 tile per wave, but each wave's code
// tile and scales are loaded straight into its registers (a wave is the only
// reader of its row tile), so only the three activation limb tiles of a
// block, which all four waves read, pass through LDS (measured 7 % faster
// than staging the code tiles in LDS too).  P_0 + 2^8 P_1 comes out of the
// matrix core: the limb-1 result, shifted left by 8 bits, is the accumulator
// input of the limb-0 product (every partial sum stays below 2^28 in
// magnitude).  Then two int64 chains per output, S (P_0 + 2^8 P_1) and
// (2^16 S) P_2, exact for narrow scales (narrow_scales).
// XB (dense): each XCD takes a block of a quarter of the row blocks by half the
// token tiles (token tiles fastest), so its share of the activation limb tiles
// stays in its L2 while the code tiles stream; a code tile is fetched by two
// XCDs.  Measured on the dense 14336 x 4096, T = 512 projection: 184.7 us mean
// against 190.2 us for contiguous runs of row blocks with all their token tiles.
// PF: blocks of operands in flight ahead of the one consumed (an LDS ring of
// PF + 1 one-block buffers, PF + 1 register sets).
template <bool kExact, bool kGrouped, bool XB = true, int PF = 1>
__global__ __launch_bounds__(256) void gemm_tiled_qreg_kernel(GemmArgs a) {
  constexpr int kBuf = 4 * 1024;   // per block: 3 limb tiles + 1 KB for the fourth wave's dummy copy
  constexpr int kRing = PF + 1;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- tile of this workgroup: 128 rows x 32 tokens in an XCD-aware order
  // (dense: XB blocks, else row blocks in runs, token tiles fastest; grouped:
  // grouped_item)
  const int64_t tbs = kGrouped ? a.tiles_max : a.t_pad / kTile;
  const int64_t rbs = (a.n_pad + 127) / 128, ntiles = rbs * tbs;
  int64_t rb, tb;
  if (kGrouped) {
    const int64_t used = *a.ntiles < a.tiles_max ? *a.ntiles : a.tiles_max;
    if (!grouped_item(blockIdx.x, ntiles, rbs, used, &rb, &tb)) return;   // the whole workgroup: no tile
  } else if (XB && rbs % 4 == 0 && tbs % 2 == 0) {
    // XCD x: row blocks of quarter x / 2, token tiles of half x % 2, token tiles fastest
    const int64_t x = blockIdx.x % 8, l = blockIdx.x / 8, th = tbs / 2;
    rb = (x / 2) * (rbs / 4) + l / th;
    tb = (x % 2) * th + l % th;
  } else {
    int64_t g = blockIdx.x;
    if (ntiles % 8 == 0) g = (g % 8) * (ntiles / 8) + g / 8;
    rb = g / tbs;
    tb = g % tbs;
  }
  const int64_t rgs = a.n_pad / kTile, tgs = kGrouped ? a.tiles_max : a.t_pad / kTile;
  const int8_t* codes = a.codes;
  const int32_t* scales = a.scales;
  int trows = kTile;   // pairs in this token tile
  if (kGrouped) {
    const int64_t e = a.tile_expert[tb];
    codes += e * a.expert_stride;
    scales = reinterpret_cast<const int32_t*>(reinterpret_cast<const int8_t*>(scales) + e * a.expert_stride);
    // the output rows of the tile's tokens, copied now into this wave's 256 B
    // after the ring (lanes 32-63 repeat lanes 0-31) and read at the end: no
    // dependent load in the epilogue, and no register held through the loop
    trows = a.tile_rows[tb];
    const int l = lane & 31;
    const __amdgpu_buffer_rsrc_t rpair = make_rsrc(a.sorted_pair, (uint32_t)(a.t * 4));   // a.t: the pairs
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rpair, (lds_ptr)(lds + kRing * kBuf + wave * 256), 4,
                                             (uint32_t)(a.tile_row0[tb] + (l < trows ? l : trows - 1)) * 4u, 0, 0, 0);
  }
  int64_t rg = 4 * rb + wave;     // this wave's row tile (past the matrix: the last one, results unused)
  rg = rg < rgs ? rg : rgs - 1;
  const __amdgpu_buffer_rsrc_t rcode = make_rsrc(codes + rg * a.nb * 1024, (uint32_t)(a.nb * 1024));
  const __amdgpu_buffer_rsrc_t rscal = make_rsrc(scales + rg * a.nb * 32, (uint32_t)(a.nb * 128));
  const __amdgpu_buffer_rsrc_t rlimb = make_rsrc(a.limb_tiles, (uint32_t)(3 * tgs * a.nb * 1024));
  // limb copy of this wave: waves 0-2 limb tile `wave`, wave 3 limb tile 0
  // again into the spare kilobyte (every wave issues one copy per block)
  const int64_t tg = tb < tgs ? tb : tgs - 1;
  const uint32_t lsoff = (uint32_t)(((int64_t)(wave < 3 ? wave : 0) * tgs + tg) * a.nb * 1024);
  const int ldst = wave * 1024;
  const int64_t nb = a.nb;
  // block b's operands (b < nb): its limb tiles into LDS slot `slot` (every
  // wave one copy), its code tile and scales into a register set: 3 requests
  auto fetch = [&](int slot, int64_t b, v4i& q, int32_t& S) {
    copy16_to_lds(rlimb, lds + slot * kBuf + ldst, lane * 16, lsoff + (uint32_t)b * 1024u);
    q = __builtin_amdgcn_raw_buffer_load_b128(rcode, lane * 16, (int)b * 1024, 0);
    S = __builtin_amdgcn_raw_buffer_load_b32(rscal, (lane & 31) * 4, (int)b * 128, 0);
  };

  int64_t acc0[16], acc1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0;
  const v16i zero = {};
  auto consume = [&](int slot, const v4i& q, int32_t S) {
    const uint8_t* blk = lds + slot * kBuf;
    const int32_t S16 = (int32_t)((uint32_t)S << 16);
    const v4i d2 = *reinterpret_cast<const v4i*>(blk + 2 * 1024 + lane * 16);
    if constexpr (kGrouped) {
      // (2^16 S) P_2 first, then S (P_0 + 2^8 P_1): one product tile live at
      // a time, which leaves room for the grouped launch's ring depth (117
      // VGPRs against 130, 4 waves per SIMD instead of 3); the dense loop is
      // as fast either way and keeps the other order
      const v16i P2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d2, q, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc1[r] += (int64_t)S16 * P2[r];
      __builtin_amdgcn_sched_barrier(0);
      const v4i d0 = *reinterpret_cast<const v4i*>(blk + 0 * 1024 + lane * 16);
      const v4i d1 = *reinterpret_cast<const v4i*>(blk + 1 * 1024 + lane * 16);
      v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(d1, q, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = (int)((uint32_t)c[r] << 8);
      const v16i P01 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d0, q, c, 0, 0, 0);   // P_0 + 2^8 P_1
#pragma unroll
      for (int r = 0; r < 16; ++r) acc0[r] += (int64_t)S * P01[r];
    } else {
      const v4i d0 = *reinterpret_cast<const v4i*>(blk + 0 * 1024 + lane * 16);
      const v4i d1 = *reinterpret_cast<const v4i*>(blk + 1 * 1024 + lane * 16);
      v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(d1, q, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = (int)((uint32_t)c[r] << 8);
      const v16i P01 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d0, q, c, 0, 0, 0);   // P_0 + 2^8 P_1
      const v16i P2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d2, q, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc0[r] += (int64_t)S * P01[r];
        acc1[r] += (int64_t)S16 * P2[r];
      }
    }
  };
  if constexpr (PF == 1) {
    // one block ahead: the loop the dense prefill was tuned with (block b's
    // copies waited for, block b + 1 requested, block b consumed)
    v4i qn = {};
    int32_t Sn = 0;
    if (nb > 0) fetch(0, 0, qn, Sn);
    for (int64_t b = 0; b < nb; ++b) {
      barrier_after_vmcnt<0>();   // block b: limb tiles in LDS (every wave), code tile and scales in registers
      const v4i q = qn;
      const int32_t S = Sn;
      if (b + 1 < nb) fetch((int)((b + 1) % kRing), b + 1, qn, Sn);   // into the buffer block b - 1 used: every wave is past it
      consume((int)(b % kRing), q, S);
    }
  } else {
  // Ring turns: iteration b waits until only the PF - 1 newer fetches are
  // out, so block b has landed for every wave, fetches block b + PF into the
  // slot block b - 1 used (every wave is past it) and consumes block b.  No
  // fetch sits under a branch -- one the compiler cannot rule out would make
  // it drain every load before the first use of a register set -- so the
  // loop runs whole turns of the ring: fetches past the last block re-read
  // it, and blocks past the last are consumed with scale 0 (adding nothing).
  v4i qs[kRing];
  int32_t Ss[kRing];
  // (scheduling barriers keep each fetch in its place: requests in block
  // order, and no load moved across the multiply-adds it would keep
  // registers live through)
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    fetch(j, j < nb ? j : nb - 1, qs[j], Ss[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int64_t turns = (nb + kRing - 1) / kRing;
  for (int64_t t = 0; t < turns; ++t) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int64_t b = t * kRing + j;
      barrier_after_vmcnt<(PF - 1) * 3>();
      fetch((j + PF) % kRing, b + PF < nb ? b + PF : nb - 1, qs[(j + PF) % kRing], Ss[(j + PF) % kRing]);
      __builtin_amdgcn_sched_barrier(0);
      consume(j, qs[j], b < nb ? Ss[j] : 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  vmcnt_wait<0>();   // the re-reads past the end have landed before the wave ends
  }

  // ---- store: lane holds row 32 (4 rb + wave) + lane % 32 and tokens
  // 8 (r / 4) + 4 (lane / 32) + r % 4 of the token tile
  const int64_t row = (4 * rb + wave) * 32 + (lane & 31);
  if (row >= a.n) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tloc = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    int64_t orow;
    if (kGrouped) {
      if (tloc >= trows) continue;
      orow = reinterpret_cast<const int32_t*>(lds + kRing * kBuf + wave * 256)[tloc];
    } else {
      orow = tb * kTile + tloc;
      if (orow >= a.t) continue;
    }
    const int64_t v = acc0[r] + acc1[r];   // |v| < 2^62.01: the rounding add cannot overflow
    // non-temporal: the outputs are not read again here, the code tiles are
    // (prefill step 199 us against 203 us, medians of two rounds)
    __builtin_nontemporal_store(kExact ? v : (v + ((int64_t)1 << 23)) >> 24, a.y + orow * a.n + row);
  }
}

// Prefetch depth: the dense prefill's code tiles are mostly L2 hits (each is
// read by the token tiles that share its XCD), one block ahead suffices; a
// routed projection's expert weights serve only a few token tiles and stream
// from HBM, so its loads go further ahead.
constexpr int kDensePF = 1, kGroupedPF = 3;

hipError_t launch_gemm_tiled_qreg(const GemmArgs& a, bool grouped, hipStream_t s) {
  const int64_t rbs = (a.n_pad + 127) / 128;
  const int64_t tbs = grouped ? a.tiles_max : a.t_pad / kTile;
  const dim3 grid((unsigned)(rbs * tbs)), block(256);
  const bool exact = a.out_mode == OUT_EXACT;
  // the ring; grouped: and 256 B per wave for the tile's output rows
  const size_t lds = (size_t)((grouped ? kGroupedPF : kDensePF) + 1) * 4 * 1024 + (grouped ? 4 * 256 : 0);
  if (grouped && exact)
    hipLaunchKernelGGL((gemm_tiled_qreg_kernel<true, true, true, kGroupedPF>), grid, block, lds, s, a);
  else if (grouped)
    hipLaunchKernelGGL((gemm_tiled_qreg_kernel<false, true, true, kGroupedPF>), grid, block, lds, s, a);
  else if (exact)
    hipLaunchKernelGGL((gemm_tiled_qreg_kernel<true, false, true, kDensePF>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((gemm_tiled_qreg_kernel<false, false, true, kDensePF>), grid, block, lds, s, a);
  return hipGetLastError();
}

// Launch shape of the per-limb form: one 32x32 tile per wave, 128 rows x 32
// tokens per workgroup, copies one block ahead, no software pipelining (the
// fastest of the variants measured on MI355X; larger wave tiles, deeper rings
// and a pipelined epilogue were all slower).  Narrow scales take the
// register-fed kernel above.
hipError_t launch_gemm_tiled(const GemmArgs& a, bool narrow, hipStream_t s) {
  return narrow ? launch_gemm_tiled_qreg(a, false, s) : launch_tiled_shape<1, 1, 4, 2>(a, s);
}

// Grouped: XCD-contiguous order, so that the token tiles of one expert
// share an XCD's L2 (see the gate/up kernel).
hipError_t launch_gemm_grouped(const GemmArgs& a, bool narrow, hipStream_t s) {
  return narrow ? launch_gemm_tiled_qreg(a, true, s) : launch_tiled_shape<1, 1, 4, 2, true, false, true>(a, s);
}

// ================================================================ routed FFN gate + up
// The gate and up projections of a routed FFN in one pass over each token
// tile's activation limbs.  A workgroup of 8 waves owns 128 rows of both
// matrices for one token tile (one expert): waves 0-3 the four row tiles of
// the gate matrix, waves 4-7 the same row tiles of the up matrix, all reading
// the tile's three limb tiles from one LDS ring (per block: 8 code tiles, 3
// limb tiles, 8 x 128 B of scales; every wave copies its own row tile's
// scales).  The accumulation is the tiled kernel's (per-limb int64, exact for
// any int32 scale).  At the end the up waves put their rounded results u in
// LDS; each gate wave forms h = SiLU-gated product of its own g and the u of
// the same elements in place, and writes its 32 x 32 tile of h (rows of the
// tile x pairs) out as limb tile (block 4 rb + wave, token tile tb) of the
// down projection's input, zero for pairs past the tile.  g and u never reach
// HBM.
constexpr int kGuWaves = 8;
constexpr int kGuLimbOff = 8 * 1024;               // after the 8 code tiles
constexpr int kGuScaleOff = kGuLimbOff + 3 * 1024;
constexpr int kGuBlockBytes = kGuScaleOff + 8 * 128;
constexpr int kGuNbuf = 2;
constexpr int kGuTileBytes = 32 * 33 * 8;          // one wave's 32 x 32 int64 exchange tile (padded rows)
constexpr int kGateUpPF = 3;                        // narrow form: blocks of operands in flight ahead (ring of 4 x 3 KB)

// NARROW: two int64 accumulators per output, as in the register-fed tiled kernel.
template <bool NARROW>
__global__ __launch_bounds__(kGuWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void gemm_grouped_gateup_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 3;              // row tile within the workgroup's 128 rows
  const bool is_up = wave >= 4;
  const int64_t tgs = a.tiles_max, rgs = a.n_pad / kTile;
  // token tiles in turn, row blocks fastest, an eighth of the tiles in use
  // per XCD (grouped_item): the row blocks of a token tile share its limb
  // tiles, and the token tiles of one expert its weight rows, in one XCD's L2
  const int64_t rbs = (a.n_pad + 4 * kTile - 1) / (4 * kTile);
  int64_t rb, tb;
  const int64_t used = *a.ntiles < tgs ? *a.ntiles : tgs;
  if (!grouped_item(blockIdx.x, rbs * tgs, rbs, used, &rb, &tb)) return;   // the whole workgroup: no tile
  const int64_t ex = a.tile_expert[tb];
  const int8_t* codes[2] = {a.codes + ex * a.expert_stride, a.codes2 + ex * a.expert_stride};
  const int32_t* scales[2] = {
      reinterpret_cast<const int32_t*>(reinterpret_cast<const int8_t*>(a.scales) + ex * a.expert_stride),
      reinterpret_cast<const int32_t*>(reinterpret_cast<const int8_t*>(a.scales2) + ex * a.expert_stride)};
  const int64_t nb = a.nb;
  const __amdgpu_buffer_rsrc_t rlimb = make_rsrc(a.limb_tiles, (uint32_t)(3 * tgs * nb * 1024));
  // copies j = wave and j = wave + 8 (< 11): j < 8 code tile (matrix j / 4,
  // row tile j % 4), else limb tile j - 8.  Row tiles past the matrix re-read
  // the last one (results unused).
  constexpr int kCopies = 11;
  __amdgpu_buffer_rsrc_t rsrc[2];
  uint32_t soff[2];
  int dst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave + kGuWaves * i;
    if (j < 8) {
      int64_t rg = 4 * rb + (j & 3);
      rg = rg < rgs ? rg : rgs - 1;
      rsrc[i] = make_rsrc(codes[j >> 2], (uint32_t)code_bytes(a.n_pad, nb));
      soff[i] = (uint32_t)(rg * nb * 1024);
      dst[i] = j * 1024;
    } else {   // j < kCopies is checked where the copy is issued
      rsrc[i] = rlimb;
      soff[i] = (uint32_t)(((int64_t)(j - 8) * tgs + tb) * nb * 1024);
      dst[i] = kGuLimbOff + (j - 8) * 1024;
    }
  }
  const __amdgpu_buffer_rsrc_t rscal = make_rsrc(scales[is_up ? 1 : 0], (uint32_t)(a.n_pad * nb * 4));
  uint32_t svoff;
  {
    int64_t rg = 4 * rb + wr;
    rg = rg < rgs ? rg : rgs - 1;
    svoff = (uint32_t)(rg * nb * 128) + (lane & 7) * 16;
  }
  const bool second = wave + kGuWaves < kCopies;   // waves 0-2 copy a limb tile too
  auto issue = [&](int64_t b) {
    uint8_t* blk = lds + (int)(b % kGuNbuf) * kGuBlockBytes;
    copy16_to_lds(rsrc[0], blk + dst[0], lane * 16, soff[0] + (uint32_t)b * 1024u);
    if (second) copy16_to_lds(rsrc[1], blk + dst[1], lane * 16, soff[1] + (uint32_t)b * 1024u);
    if (lane < 8) copy16_to_lds(rscal, blk + kGuScaleOff + wave * 128, svoff, (uint32_t)b * 128u);
  };

  constexpr int NACC = NARROW ? 2 : 3;
  int64_t acc[NACC][16];
#pragma unroll
  for (int l = 0; l < NACC; ++l)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[l][r] = 0;
  const v16i zero = {};
  if constexpr (NARROW) {
    // register-fed, as in gemm_tiled_qreg_kernel: each wave loads its own
    // code tile and scales into registers one block ahead; only the three
    // limb tiles (copied by waves 0-2) pass through LDS
    int64_t rg = 4 * rb + wr;
    rg = rg < rgs ? rg : rgs - 1;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes[is_up ? 1 : 0] + rg * nb * 1024, (uint32_t)(nb * 1024));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales[is_up ? 1 : 0] + rg * nb * 32, (uint32_t)(nb * 128));
    const uint32_t lsoff = (uint32_t)(((int64_t)(wave < 3 ? wave : 0) * tgs + tb) * nb * 1024);
    // block b (b < nb): limb tiles into LDS slot `slot` (waves 0-2 copy one
    // each; the others issue the same copy against an empty buffer range,
    // which reads nothing, into a spare kilobyte, so that every wave issues
    // the same three requests per block on one path, and the compiler's wait
    // tracking follows that count), code tile and scales into a register
    // set, kGateUpPF blocks ahead
    constexpr int PF = kGateUpPF, kRing = PF + 1;
    constexpr int kSlot = 4 * 1024;
    static_assert(kRing * kSlot <= 4 * kGuTileBytes, "the ring fits the allocation of the exchange tiles");
    const __amdgpu_buffer_rsrc_t rcopy = wave < 3 ? rlimb : make_rsrc(a.limb_tiles, 0u);
    const int cdst = (wave < 3 ? wave : 3) * 1024;
    auto fetch = [&](int slot, int64_t b, v4i& q, int32_t& S) {
      copy16_to_lds(rcopy, lds + slot * kSlot + cdst, lane * 16, lsoff + (uint32_t)b * 1024u);
      q = __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16, (int)b * 1024, 0);
      S = __builtin_amdgcn_raw_buffer_load_b32(rs, (lane & 31) * 4, (int)b * 128, 0);
    };
    auto consume = [&](int slot, const v4i& q, int32_t S) {
      const uint8_t* blk = lds + slot * kSlot;
      const v4i d0 = *reinterpret_cast<const v4i*>(blk + lane * 16);
      const v4i d1 = *reinterpret_cast<const v4i*>(blk + 1024 + lane * 16);
      const v4i d2 = *reinterpret_cast<const v4i*>(blk + 2048 + lane * 16);
      v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(d1, q, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = (int)((uint32_t)c[r] << 8);
      const v16i P01 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d0, q, c, 0, 0, 0);   // P_0 + 2^8 P_1
      const v16i P2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d2, q, zero, 0, 0, 0);
      const int32_t S16 = (int32_t)((uint32_t)S << 16);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[0][r] += (int64_t)S * P01[r];
        acc[NACC - 1][r] += (int64_t)S16 * P2[r];
      }
    };
    // Ring turns as in the register-fed kernel: iteration b waits until only
    // the PF - 1 newer fetches are out (block b has landed for every wave),
    // fetches block b + PF into the slot block b - 1 used (every wave is past
    // it) and consumes block b.  No fetch sits under a branch (one the
    // compiler cannot rule out would make it drain every load before a first
    // use); fetches past the last block re-read it.
    v4i qs[kRing];
    int32_t Ss[kRing];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      fetch(j, j < nb ? j : nb - 1, qs[j], Ss[j]);
      __builtin_amdgcn_sched_barrier(0);   // requests in block order
    }
    const int64_t turns = (nb + kRing - 1) / kRing;
    for (int64_t t = 0; t < turns; ++t) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        const int64_t b = t * kRing + j;
        if (b >= nb) break;
        barrier_after_vmcnt<(PF - 1) * 3>();
        fetch((j + PF) % kRing, b + PF < nb ? b + PF : nb - 1, qs[(j + PF) % kRing], Ss[(j + PF) % kRing]);
        __builtin_amdgcn_sched_barrier(0);
        consume(j, qs[j], Ss[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    barrier_after_vmcnt<0>();   // no LDS copy in flight when the exchange below reuses this memory
  } else {
    if (nb > 0) issue(0);
    for (int64_t b = 0; b < nb; ++b) {
      barrier_after_vmcnt<0>();   // block b has landed for every wave; block b - 1's buffer is free
      if (b + 1 < nb) issue(b + 1);
      const uint8_t* blk = lds + (int)(b % kGuNbuf) * kGuBlockBytes;
      const v4i q = *reinterpret_cast<const v4i*>(blk + wave * 1024 + lane * 16);
      const int32_t S = *reinterpret_cast<const int32_t*>(blk + kGuScaleOff + (wave * 32 + (lane & 31)) * 4);
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        const v4i d = *reinterpret_cast<const v4i*>(blk + kGuLimbOff + l * 1024 + lane * 16);
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(d, q, zero, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[l][r] += (int64_t)S * D[r];
      }
    }
  }
  // the output before rounding, from the accumulators of element r
  auto total = [&](int r) -> __int128 {
    if constexpr (NARROW) return (__int128)(acc[0][r] + acc[1][r]);   // |sum| < 2^62.01
    else return (__int128)acc[0][r] + ((__int128)acc[NACC - 2][r] << 8) + ((__int128)acc[NACC - 1][r] << 16);
  };

  // ---- u through LDS, h in place, h out as limb tiles
  __syncthreads();   // every wave is done with the ring
  int64_t(*xt)[33] = reinterpret_cast<int64_t(*)[33]>(lds + wr * kGuTileBytes);   // [pair][row]
  const int64_t rtile = rb * 4 + wr, row = rtile * kTile + (lane & 31);
  const int rows = a.tile_rows[tb];
  bool good = true;
  if (is_up) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tloc = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      int64_t u = 0;
      if (row < a.n && tloc < rows) {
        const __int128 v = total(r);
        good = finish_output(v, OUT_ROUND_Q24, &u) && good;
      }
      xt[tloc][lane & 31] = u;
    }
  }
  __syncthreads();   // u is in place for the gate waves
  if (is_up) {
    if (!good) flag(a.status, EI_DEV_OUT_RANGE);
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tloc = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    int64_t h = 0;
    if (row < a.n && tloc < rows) {
      const __int128 v = total(r);
      int64_t g;
      good = finish_output(v, OUT_ROUND_Q24, &g) && good;
      good = silu_gate(g, xt[tloc][lane & 31], a.lut, &h) && good;
    }
    xt[tloc][lane & 31] = h;   // the element this lane read: no other lane touches it
  }
  if (!good) flag(a.status, EI_DEV_OUT_RANGE);
  __builtin_amdgcn_wave_barrier();   // this wave's LDS writes land before its reads
  if (rtile >= a.n / kTile) return;
  const int64_t* src = &xt[lane & 31][16 * (lane >> 5)];   // pair lane % 32, rows 16 (lane / 32) .. + 15
  uint32_t words[3][4];
  bool ok = true;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int64_t v4[4] = {src[4 * q4], src[4 * q4 + 1], src[4 * q4 + 2], src[4 * q4 + 3]};
    uint32_t w[3];
    ok = limb_words<3>(v4, w) && ok;
#pragma unroll
    for (int l = 0; l < 3; ++l) words[l][q4] = w[l];
  }
  if (!ok) flag(a.status, EI_DEV_LIMB_RANGE);
  const int64_t nb_out = a.n / kTile;
#pragma unroll
  for (int l = 0; l < 3; ++l) {
    const v4i v = {(int)words[l][0], (int)words[l][1], (int)words[l][2], (int)words[l][3]};
    reinterpret_cast<v4i*>(a.limb_out)[((l * tgs + tb) * nb_out + rtile) * 64 + lane] = v;
  }
}

hipError_t launch_gemm_grouped_gateup(const GemmArgs& a, bool narrow, hipStream_t s) {
  const int64_t rbs = (a.n_pad + 4 * kTile - 1) / (4 * kTile);
  const size_t ring = (size_t)kGuNbuf * kGuBlockBytes, xch = (size_t)4 * kGuTileBytes;
  const dim3 grid((unsigned)(rbs * a.tiles_max)), block(kGuWaves * 64);
  if (narrow)
    hipLaunchKernelGGL(gemm_grouped_gateup_kernel<true>, grid, block, ring > xch ? ring : xch, s, a);
  else
    hipLaunchKernelGGL(gemm_grouped_gateup_kernel<false>, grid, block, ring > xch ? ring : xch, s, a);
  return hipGetLastError();
}

}  // namespace ei
