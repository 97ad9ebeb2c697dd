// extern "C" entry points of libexact_int.so (declared in include/exact_int.h).
// Host-side validation, workspace layout and schedule dispatch; all
// arithmetic runs in the kernels of the other translation units.
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ei_internal.h"

using namespace ei;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
constexpr int kSmallT = 4;   // token counts up to this use the GEMV kernel
constexpr int kSplitParts = 8;

// The tiled prefill kernel: 3 limbs, default/canonical schedule, T >= 64,
// 32-bit buffer offsets, and enough 128-row x 32-token workgroups to occupy the
// chip (fewer go to the skinny kernel, which also splits K).
constexpr int64_t kTiledMinT = 64, kTiledMinWorkgroups = 128;
constexpr int64_t kMaxQ4TableK = kMaxK;   // the table-read projection: at most 1,024 chunks of 256 columns
bool tiled_ok(const ei_weights* w, int64_t t, int limbs, int schedule) {
  if (limbs != 3 || t < kTiledMinT) return false;
  if (schedule != EI_SCHED_DEFAULT && schedule != EI_SCHED_CANONICAL) return false;
  const int64_t t_pad = round_up(t, kTile);
  if ((w->n_pad + 127) / 128 * (t_pad / kTile) < kTiledMinWorkgroups) return false;
  return w->n_pad * w->k < ((int64_t)1 << 32) && 3 * t_pad * w->k < ((int64_t)1 << 32);
}

// Which kernel runs a projection: the GEMV for T <= 4; for larger T under the
// default/canonical schedule the tiled kernel where it applies, else the
// skinny split-K kernel; the other schedules use the generic MFMA kernel,
// which visits the blocks in the schedule's order.
enum GemmPath { PATH_GEMV, PATH_TILED, PATH_SKINNY, PATH_MFMA };

struct WsLayout {
  size_t limb_off = 0, perm_off = 0, part_off = 0, total = 0;
  bool mfma = false;
  GemmPath path = PATH_GEMV;
  int splits = 1;   // skinny: workgroup-level K splits (partials when > 1)
  int64_t t_pad = 0, ntiles = 0;
};

WsLayout layout_for(const ei_weights* w, int64_t t, int limbs, int schedule) {
  WsLayout L;
  L.mfma = t > kSmallT;
  L.t_pad = round_up(t, kTile);
  const bool plain = schedule == EI_SCHED_DEFAULT || schedule == EI_SCHED_CANONICAL;
  if (!L.mfma)
    L.path = PATH_GEMV;
  else if (tiled_ok(w, t, limbs, schedule))
    L.path = PATH_TILED;
  else
    L.path = plain ? PATH_SKINNY : PATH_MFMA;
  size_t off = 0;
  if (L.mfma) {
    L.limb_off = off;
    off = align_up(off + (size_t)limbs * (size_t)L.t_pad * (size_t)w->k);
    L.ntiles = ((w->n_pad / kTile + 1) / 2) * ((L.t_pad / kTile + 1) / 2);
  } else {
    L.ntiles = w->n_pad / kTile;
  }
  if (L.path == PATH_SKINNY) {
    L.splits = skinny_splits(w->n_pad, L.t_pad, w->nb);
    if (L.splits > 1) {
      // the workgroups' partials: an (h, r) pair per output for up to three
      // limbs (two int64 even for one limb), one int64 per limb for four
      const size_t slots = limbs <= 3 ? 2 : (size_t)limbs;
      L.part_off = off;
      off = align_up(off + sizeof(int64_t) * (size_t)L.splits * slots * (size_t)t * (size_t)w->n);
    }
  }
  if (schedule == EI_SCHED_TILED_SHUFFLED) {
    L.perm_off = off;
    off = align_up(off + sizeof(int32_t) * (size_t)(L.ntiles + w->nb));
  }
  if (schedule == EI_SCHED_SPLIT_K) {
    L.part_off = off;
    off = align_up(off + sizeof(int64_t) * (size_t)kSplitParts * limbs * (size_t)t * (size_t)w->n);
  }
  if (schedule == EI_SCHED_TREE) {
    L.part_off = off;
    off = align_up(off + sizeof(int64_t) * (size_t)w->nb * limbs * (size_t)t * (size_t)w->n);
  }
  L.total = off;
  return L;
}

int check_weights(const ei_weights* w, int format) {
  if (!w || !w->packed || w->format != format) return EI_EINVAL;
  if (w->n < 1 || w->k < 32 || w->k % 32 != 0 || w->nb != w->k / 32 || w->n_pad != round_up(w->n, kTile))
    return EI_EINVAL;
  if (w->k > kMaxK) return EI_ERANGE;
  return EI_OK;
}

// y = projection of x (+ resid when resid is not null: the skinny kernel and
// the partial combiner add it as they write y, other paths in a pass of
// their own).
// With pre_limbs (T > 4 only), x is already split: its limb tiles
// [limbs][t_pad/32][nb][1 KB] are read from there.
// With row_off (exact outputs), x_off is subtracted from every activation
// before its split and row_off[i] added to output row i (the two-limb 4-bit
// form).
int run_gemm(const ei_weights* w, const void* x, int x_is_i32, int64_t* y, int64_t t, int limbs, int schedule,
             uint64_t seed, void* ws, size_t ws_bytes, int32_t* status, hipStream_t s, int out_mode,
             const int64_t* resid = nullptr, const int8_t* pre_limbs = nullptr, const int64_t* row_off = nullptr,
             int64_t x_off = 0) {
  if ((!x && !pre_limbs) || !y || t < 1) return EI_EINVAL;
  if (limbs < 1 || limbs > 8) return EI_EINVAL;
  if (limbs > kMaxLimbs) return EI_ERANGE;
  if (schedule < EI_SCHED_DEFAULT || schedule > EI_SCHED_TREE) return EI_EINVAL;
  if (round_up(t, kTile) / kTile > 65535) return EI_ERANGE;   // token tiles index a grid dimension
  const WsLayout lay = layout_for(w, t, limbs, schedule);
  if (lay.total > 0 && (!ws || ws_bytes < lay.total)) return EI_ENOSPACE;
  uint8_t* wsb = static_cast<uint8_t*>(ws);

  GemmArgs a;
  std::memset(&a, 0, sizeof a);
  const uint8_t* base = static_cast<const uint8_t*>(w->packed);
  a.codes = reinterpret_cast<const int8_t*>(base + kHeaderBytes);
  a.scales = reinterpret_cast<const int32_t*>(base + kHeaderBytes + w->n_pad * w->k);
  a.x = x;
  a.x_is_i32 = x_is_i32;
  a.y = y;
  a.status = status;
  a.n = w->n;
  a.k = w->k;
  a.t = t;
  a.n_pad = w->n_pad;
  a.t_pad = lay.t_pad;
  a.nb = w->nb;
  a.b0 = 0;
  a.b1 = w->nb;
  a.out_mode = out_mode;
  a.order = ORDER_ASC;
  a.row_off = row_off;
  a.x_off = x_off;

  hipError_t e = hipSuccess;
  if (lay.mfma && pre_limbs) {
    a.limb_tiles = pre_limbs;
  } else if (lay.mfma) {
    a.limb_tiles = reinterpret_cast<const int8_t*>(wsb + lay.limb_off);
    e = launch_limb_tiles(x, x_is_i32, t, w->k, limbs, reinterpret_cast<int8_t*>(wsb + lay.limb_off), lay.t_pad,
                          status, s, x_off);
    if (e != hipSuccess) return EI_EDEVICE;
  } else if (pre_limbs) {
    return EI_EINVAL;
  }
  auto launch = [&](const GemmArgs& args) {
    if (lay.path == PATH_TILED) return launch_gemm_tiled(args, narrow_scales(w->smax, w->nb), s);
    return lay.mfma ? launch_gemm_mfma(args, limbs, s) : launch_gemv(args, limbs, s);
  };

  switch (schedule) {
    case EI_SCHED_DEFAULT:
    case EI_SCHED_CANONICAL:
      if (lay.path == PATH_SKINNY) {
        if (lay.splits > 1) {
          int64_t* part = reinterpret_cast<int64_t*>(wsb + lay.part_off);
          a.part = part;
          a.out_mode = OUT_PARTIAL;
          e = launch_gemm_skinny(a, limbs, lay.splits, limbs == 3 && narrow_scales(w->smax, w->nb), s);
          if (e == hipSuccess)
            e = limbs <= 3
                    ? launch_combine_hr(part, lay.splits, y, t, w->n, out_mode, resid, status, s, row_off)
                    : launch_combine_partials(part, lay.splits, y, t, w->n, limbs, out_mode, resid, status, s,
                                              row_off);
        } else {
          a.resid = resid;
          e = launch_gemm_skinny(a, limbs, 1, limbs == 3 && narrow_scales(w->smax, w->nb), s);
        }
        return e == hipSuccess ? EI_OK : EI_EDEVICE;
      }
      e = launch(a);
      break;
    case EI_SCHED_REVERSED:
      a.order = ORDER_DESC;
      e = launch(a);
      break;
    case EI_SCHED_TILED_SHUFFLED: {
      int32_t* tperm = reinterpret_cast<int32_t*>(wsb + lay.perm_off);
      int32_t* kperm = tperm + lay.ntiles;
      e = launch_make_perm(tperm, lay.ntiles, seed, s);
      if (e == hipSuccess) e = launch_make_perm(kperm, w->nb, seed ^ 0x5851F42D4C957F2Dull, s);
      a.tperm = tperm;
      a.kperm = kperm;
      a.order = ORDER_PERM;
      if (e == hipSuccess) e = launch(a);
      break;
    }
    case EI_SCHED_SPLIT_K: {
      int64_t* part = reinterpret_cast<int64_t*>(wsb + lay.part_off);
      a.part = part;
      a.out_mode = OUT_PARTIAL;
      for (int p = 0; p < kSplitParts && e == hipSuccess; ++p) {
        a.b0 = p * w->nb / kSplitParts;
        a.b1 = (p + 1) * w->nb / kSplitParts;
        a.part_index = p;
        e = launch(a);
      }
      if (e == hipSuccess)
        e = launch_combine_partials(part, kSplitParts, y, t, w->n, limbs, out_mode, resid, status, s, row_off);
      return e == hipSuccess ? EI_OK : EI_EDEVICE;
    }
    case EI_SCHED_TREE: {
      int64_t* terms = reinterpret_cast<int64_t*>(wsb + lay.part_off);
      a.part = terms;
      a.out_mode = OUT_TERMS;
      e = launch(a);
      if (e == hipSuccess) e = launch_tree_terms(terms, w->nb, y, t, w->n, limbs, out_mode, status, s, row_off);
      break;
    }
  }
  if (e == hipSuccess && resid) e = launch_add_residual(y, resid, t * w->n, status, s);
  return e == hipSuccess ? EI_OK : EI_EDEVICE;
}

int do_pack(int format, const void* codes, const void* scales, int64_t n, int64_t k, void* packed,
            size_t packed_bytes_, ei_weights* out, hipStream_t s) {
  if (!codes || !scales || !packed || !out) return EI_EINVAL;
  if (n < 1 || k < 32 || k % 32 != 0) return EI_EINVAL;
  if (!aligned(packed, 256) || (format == EI_FORMAT_Q8 && !aligned(codes, 16))) return EI_EINVAL;
  if (packed_bytes_ < ei::packed_bytes(n, k)) return EI_ENOSPACE;
  hipError_t e = format == EI_FORMAT_Q8
                     ? launch_pack_q8(static_cast<const int8_t*>(codes), static_cast<const int32_t*>(scales), n, k,
                                      packed, s)
                     : launch_pack_q4(static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales), n, k,
                                      packed, s);
  if (e != hipSuccess) return EI_EDEVICE;
  PackedHeader h;
  if (hipMemcpyAsync(&h, packed, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess) return EI_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return EI_EDEVICE;
  if (h.magic != kMagic || h.n != n || h.k != k) return EI_EDEVICE;
  out->packed = packed;
  out->n = n;
  out->k = k;
  out->n_pad = h.n_pad;
  out->nb = h.nb;
  out->smax = h.smax;
  out->format = format;
  out->experts = 1;
  out->expert_stride = (int64_t)align_up(ei::packed_bytes(n, k));
  return EI_OK;
}

// Grouped (expert) workspace: sorted pairs, segment offsets, the token-tile
// table, the tile count and the gathered limb tiles.
struct GroupedLayout {
  size_t sorted_off, offsets_off, texp_off, trow0_off, trows_off, ntiles_off, limb_off, total;
  int64_t pairs, tiles_max;
};

GroupedLayout grouped_layout(const ei_weights* w, int64_t rows, int topk, int limbs) {
  GroupedLayout g;
  g.pairs = rows * topk;
  g.tiles_max = (g.pairs + kTile - 1) / kTile + (w->experts < g.pairs ? w->experts : g.pairs);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  g.sorted_off = take(sizeof(int32_t) * (size_t)g.pairs);
  g.offsets_off = take(sizeof(int32_t) * (size_t)(w->experts + 1));
  g.texp_off = take(sizeof(int32_t) * (size_t)g.tiles_max);
  g.trow0_off = take(sizeof(int32_t) * (size_t)g.tiles_max);
  g.trows_off = take(sizeof(int32_t) * (size_t)g.tiles_max);
  g.ntiles_off = take(sizeof(int32_t));
  g.limb_off = take((size_t)limbs * (size_t)g.tiles_max * (size_t)w->k * kTile);
  g.total = off;
  return g;
}

int grouped_check(const ei_weights* w, int64_t rows, int topk, int limbs) {
  const int c = check_weights(w, EI_FORMAT_Q8);
  if (c != EI_OK) return c;
  if (rows < 1 || topk < 1 || w->experts < 1) return EI_EINVAL;
  if (limbs != 3) return limbs < 1 || limbs > 8 ? EI_EINVAL : EI_ERANGE;
  if (rows * topk > ((int64_t)1 << 14) || w->experts > ((int64_t)1 << 17)) return EI_ERANGE;
  if (w->n_pad * w->k >= ((int64_t)1 << 32)) return EI_ERANGE;
  const int64_t tiles_max = grouped_layout(w, rows, topk, limbs).tiles_max;
  if (3 * tiles_max * w->k * kTile >= ((int64_t)1 << 32)) return EI_ERANGE;
  return EI_OK;
}

// Pointers into a grouped workspace laid out by grouped_layout.
struct Grouping {
  int32_t *sorted, *offs, *texp, *trow0, *trows, *ntiles;
  int8_t* limb;
};

Grouping grouping_at(void* workspace, const GroupedLayout& g) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Grouping p;
  p.sorted = reinterpret_cast<int32_t*>(ws + g.sorted_off);
  p.offs = reinterpret_cast<int32_t*>(ws + g.offsets_off);
  p.texp = reinterpret_cast<int32_t*>(ws + g.texp_off);
  p.trow0 = reinterpret_cast<int32_t*>(ws + g.trow0_off);
  p.trows = reinterpret_cast<int32_t*>(ws + g.trows_off);
  p.ntiles = reinterpret_cast<int32_t*>(ws + g.ntiles_off);
  p.limb = reinterpret_cast<int8_t*>(ws + g.limb_off);
  return p;
}

// The grouped projection of w over the limb tiles in p (already gathered for
// the sorted pairs): y[pair][n].  With up, lut and h_limbs: w is the gate
// matrix of a routed FFN and one pass computes gate and up and writes
// h = silu(g, u) as limb tiles to h_limbs.
hipError_t launch_grouped_projection(const ei_weights* w, const GroupedLayout& g, const Grouping& p, int64_t* y,
                                     int32_t* status, hipStream_t s, const ei_weights* up = nullptr,
                                     const int32_t* lut = nullptr, int8_t* h_limbs = nullptr,
                                     const int8_t* limbs = nullptr) {
  GemmArgs a;
  std::memset(&a, 0, sizeof a);
  const uint8_t* base = static_cast<const uint8_t*>(w->packed);
  a.codes = reinterpret_cast<const int8_t*>(base + kHeaderBytes);
  a.scales = reinterpret_cast<const int32_t*>(base + kHeaderBytes + w->n_pad * w->k);
  a.limb_tiles = p.limb;
  a.y = y;
  a.status = status;
  a.n = w->n;
  a.k = w->k;
  a.t = g.pairs;
  a.n_pad = w->n_pad;
  a.t_pad = g.tiles_max * kTile;
  a.nb = w->nb;
  a.b0 = 0;
  a.b1 = w->nb;
  a.out_mode = OUT_ROUND_Q24;
  a.order = ORDER_ASC;
  a.tile_expert = p.texp;
  a.tile_row0 = p.trow0;
  a.tile_rows = p.trows;
  a.sorted_pair = p.sorted;
  a.ntiles = p.ntiles;
  a.tiles_max = g.tiles_max;
  a.expert_stride = w->expert_stride;
  if (limbs) a.limb_tiles = limbs;
  if (up) {
    const uint8_t* ubase = static_cast<const uint8_t*>(up->packed);
    a.codes2 = reinterpret_cast<const int8_t*>(ubase + kHeaderBytes);
    a.scales2 = reinterpret_cast<const int32_t*>(ubase + kHeaderBytes + up->n_pad * up->k);
    a.lut = lut;
    a.limb_out = h_limbs;
    return launch_gemm_grouped_gateup(a, narrow_scales(w->smax, w->nb) && narrow_scales(up->smax, up->nb), s);
  }
  return launch_gemm_grouped(a, narrow_scales(w->smax, w->nb), s);
}

// FFN workspace: fused gate/up, h as the down projection's limb tiles
// [3][t_pad/32][f/32][1 KB]; otherwise h, g and u [t][f]; then the
// projections' own workspace.
struct FfnLayout {
  bool fused;
  size_t h_off, g_off, u_off, n_off, gemm_off, total;
};

FfnLayout ffn_layout(const ei_weights* wg, const ei_weights* wd, int64_t t) {
  FfnLayout f;
  const WsLayout lg = layout_for(wg, t, 3, EI_SCHED_DEFAULT), ld = layout_for(wd, t, 3, EI_SCHED_DEFAULT);
  f.fused = lg.path == PATH_SKINNY && lg.splits == 1 && ld.mfma;
  f.h_off = 0;
  size_t off;
  if (f.fused) {
    off = align_up((size_t)3 * (size_t)lg.t_pad * (size_t)wg->n);
    f.g_off = f.u_off = off;
  } else {
    const size_t hb = align_up(sizeof(int64_t) * (size_t)t * (size_t)wg->n);
    f.g_off = hb;
    f.u_off = 2 * hb;
    off = 3 * hb;
  }
  // the normalized input (prenorm form, unfused path)
  f.n_off = off;
  if (!f.fused) off += align_up(sizeof(int64_t) * (size_t)t * (size_t)wg->k);
  f.gemm_off = off;
  f.total = off + (lg.total > ld.total ? lg.total : ld.total);
  return f;
}

int ffn_check(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd) {
  int c = check_weights(wg, EI_FORMAT_Q8);
  if (c == EI_OK) c = check_weights(wu, EI_FORMAT_Q8);
  if (c == EI_OK) c = check_weights(wd, EI_FORMAT_Q8);
  if (c != EI_OK) return c;
  if (wu->n != wg->n || wu->k != wg->k || wd->k != wg->n || wd->n != wg->k) return EI_EINVAL;
  return EI_OK;
}

// Routed FFN workspace: one grouping (its limb area holds x's limb tiles),
// then h as the down projection's limb tiles [3][tiles_max][f/32][1 KB].
struct MoeLayout {
  GroupedLayout g;
  size_t hl_off, total;
};

MoeLayout moe_layout(const ei_weights* wg, const ei_weights* wd, int64_t rows, int topk) {
  MoeLayout m;
  (void)wd;
  m.g = grouped_layout(wg, rows, topk, 3);
  m.hl_off = m.g.total;
  m.total = m.hl_off + align_up((size_t)3 * (size_t)m.g.tiles_max * (size_t)wg->n * kTile);
  return m;
}

}  // namespace

extern "C" {

size_t ei_packed_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 32 || k % 32 != 0) return 0;
  return ei::packed_bytes(n, k);
}

int ei_q8_pack(const int8_t* codes, const int32_t* scales, int64_t n, int64_t k, void* packed, size_t packed_bytes,
               ei_weights* out, ei_stream stream) {
  return do_pack(EI_FORMAT_Q8, codes, scales, n, k, packed, packed_bytes, out, static_cast<hipStream_t>(stream));
}

int ei_q4_pack(const uint8_t* nib, const uint8_t* sme, int64_t n, int64_t k, void* packed, size_t packed_bytes,
               ei_weights* out, ei_stream stream) {
  return do_pack(EI_FORMAT_Q4, nib, sme, n, k, packed, packed_bytes, out, static_cast<hipStream_t>(stream));
}

size_t ei_packed_bytes_stacked(int64_t experts, int64_t n, int64_t k) {
  if (experts < 1 || n < 1 || k < 32 || k % 32 != 0) return 0;
  return (size_t)experts * align_up(ei::packed_bytes(n, k));
}

int ei_q8_pack_stacked(const int8_t* codes, const int32_t* scales, int64_t experts, int64_t n, int64_t k,
                       void* packed, size_t packed_bytes, ei_weights* out, ei_stream stream) {
  if (!codes || !scales || !packed || !out || experts < 1) return EI_EINVAL;
  if (n < 1 || k < 32 || k % 32 != 0) return EI_EINVAL;
  if (packed_bytes < ei_packed_bytes_stacked(experts, n, k)) return EI_ENOSPACE;
  const size_t stride = align_up(ei::packed_bytes(n, k));
  ei_weights one;
  uint32_t smax = 0;
  for (int64_t e = 0; e < experts; ++e) {
    const int c = do_pack(EI_FORMAT_Q8, codes + e * n * k, scales + e * n * (k / 32), n, k,
                          static_cast<uint8_t*>(packed) + e * stride, stride, &one, static_cast<hipStream_t>(stream));
    if (c != EI_OK) return c;
    smax = one.smax > smax ? one.smax : smax;
  }
  *out = one;
  out->packed = packed;
  out->smax = smax;
  out->experts = experts;
  out->expert_stride = (int64_t)stride;
  return EI_OK;
}

size_t ei_grouped_workspace_bytes(const ei_weights* w, int64_t rows, int topk, int limbs) {
  if (!w || rows < 1 || topk < 1 || limbs < 1) return 0;
  return grouped_layout(w, rows, topk, limbs).total;
}

int int_gemm_q8_grouped(const ei_weights* w, const int64_t* x, const int32_t* route, int64_t rows, int topk,
                        int64_t* y, int limbs, void* workspace, size_t workspace_bytes, int32_t* d_status,
                        ei_stream stream) {
  if (!x || !route || !y) return EI_EINVAL;
  const int c = grouped_check(w, rows, topk, limbs);
  if (c != EI_OK) return c;
  const GroupedLayout g = grouped_layout(w, rows, topk, limbs);
  if (!workspace || workspace_bytes < g.total) return EI_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Grouping p = grouping_at(workspace, g);
  hipError_t e = launch_moe_sort(route, g.pairs, w->experts, p.sorted, p.offs, p.texp, p.trow0, p.trows, p.ntiles,
                                 d_status, s);
  if (e == hipSuccess)
    e = launch_grouped_limb_tiles(x, w->k, topk, p.sorted, p.trow0, p.trows, p.ntiles, g.tiles_max, p.limb, d_status,
                                  s);
  if (e == hipSuccess) e = launch_grouped_projection(w, g, p, y, d_status, s);
  return e == hipSuccess ? EI_OK : EI_EDEVICE;
}

size_t ei_ffn_workspace_bytes(const ei_weights* wg, const ei_weights* wd, int64_t t) {
  if (!wg || !wd || t < 1) return 0;
  return ffn_layout(wg, wd, t).total;
}

}  // extern "C"

namespace {

// y = x + FFN(x), or y = x + FFN(rmsnorm(x)) when gnorm is given.
// in_limbs (fused path only): x's limb tiles are already there; out_limbs:
// y's limb tiles for the next layer's gate/up pass are written there too
// (of rmsnorm(y, next_gnorm, eps_q32) when next_gnorm is given).
int ffn_run(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd, const int64_t* x,
            const int32_t* gnorm, int64_t eps_q32, const int32_t* lut, int64_t* y, int64_t t, void* workspace,
            size_t workspace_bytes, int32_t* d_status, hipStream_t s, const int8_t* in_limbs = nullptr,
            int8_t* out_limbs = nullptr, const int32_t* next_gnorm = nullptr) {
  if (!x || !lut || !y || t < 1) return EI_EINVAL;
  const int c = ffn_check(wg, wu, wd);
  if (c != EI_OK) return c;
  if (gnorm && (wg->k > 65536 || eps_q32 < 1 || eps_q32 > ((int64_t)1 << 32))) return EI_ERANGE;
  const FfnLayout f = ffn_layout(wg, wd, t);
  if (!workspace || workspace_bytes < f.total) return EI_ENOSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void* gws = ws + f.gemm_off;
  const size_t gws_bytes = workspace_bytes - f.gemm_off;
  if (f.fused) {
    // gate and up in one pass, the SiLU-gated product in its epilogue; the
    // (normalized) input goes straight into limb tiles
    const WsLayout lay = layout_for(wg, t, 3, EI_SCHED_DEFAULT);
    const int8_t* limb = in_limbs;
    if (!limb) {
      int8_t* own = static_cast<int8_t*>(gws) + lay.limb_off;
      const hipError_t e = gnorm ? launch_rmsnorm_limb_tiles(x, gnorm, eps_q32, own, t, lay.t_pad, wg->k, d_status, s)
                                 : launch_limb_tiles(x, 0, t, wg->k, 3, own, lay.t_pad, d_status, s);
      if (e != hipSuccess) return EI_EDEVICE;
      limb = own;
    }
    GemmArgs a;
    std::memset(&a, 0, sizeof a);
    const uint8_t* bg = static_cast<const uint8_t*>(wg->packed);
    const uint8_t* bu = static_cast<const uint8_t*>(wu->packed);
    a.codes = reinterpret_cast<const int8_t*>(bg + kHeaderBytes);
    a.scales = reinterpret_cast<const int32_t*>(bg + kHeaderBytes + wg->n_pad * wg->k);
    a.codes2 = reinterpret_cast<const int8_t*>(bu + kHeaderBytes);
    a.scales2 = reinterpret_cast<const int32_t*>(bu + kHeaderBytes + wu->n_pad * wu->k);
    a.lut = lut;
    a.limb_tiles = limb;
    a.limb_out = reinterpret_cast<int8_t*>(ws + f.h_off);
    a.status = d_status;
    a.n = wg->n;
    a.k = wg->k;
    a.t = t;
    a.n_pad = wg->n_pad;
    a.t_pad = lay.t_pad;
    a.nb = wg->nb;
    a.b0 = 0;
    a.b1 = wg->nb;
    a.out_mode = OUT_ROUND_Q24;
    if (launch_gemm_skinny_gateup(a, narrow_scales(wg->smax, wg->nb) && narrow_scales(wu->smax, wu->nb), s) !=
        hipSuccess)
      return EI_EDEVICE;
    const int8_t* h_limbs = reinterpret_cast<const int8_t*>(ws + f.h_off);
    const WsLayout ld = layout_for(wd, t, 3, EI_SCHED_DEFAULT);
    if (!next_gnorm && narrow_scales(wd->smax, wd->nb) && skinny16_finish_fits(wd->n, wd->nb, t)) {
      // the down projection in one launch on 16 x 16 tiles: y = x + result,
      // and the next layer's input limb tiles, with no split-K combiner
      GemmArgs b;
      std::memset(&b, 0, sizeof b);
      const uint8_t* bd = static_cast<const uint8_t*>(wd->packed);
      b.codes = reinterpret_cast<const int8_t*>(bd + kHeaderBytes);
      b.scales = reinterpret_cast<const int32_t*>(bd + kHeaderBytes + wd->n_pad * wd->k);
      b.limb_tiles = h_limbs;
      b.resid = x;
      b.y = y;
      b.limb_out = out_limbs;
      b.status = d_status;
      b.n = wd->n;
      b.k = wd->k;
      b.t = t;
      b.n_pad = wd->n_pad;
      b.t_pad = lay.t_pad;
      b.nb = wd->nb;
      b.b0 = 0;
      b.b1 = wd->nb;
      b.out_mode = OUT_ROUND_Q24;
      return launch_skinny16_finish(b, s) == hipSuccess ? EI_OK : EI_EDEVICE;
    }
    if (out_limbs && ld.path == PATH_SKINNY && ld.splits > 1) {
      // split-K down projection whose combiner also writes the next input's limb tiles
      GemmArgs b;
      std::memset(&b, 0, sizeof b);
      const uint8_t* bd = static_cast<const uint8_t*>(wd->packed);
      b.codes = reinterpret_cast<const int8_t*>(bd + kHeaderBytes);
      b.scales = reinterpret_cast<const int32_t*>(bd + kHeaderBytes + wd->n_pad * wd->k);
      b.limb_tiles = h_limbs;
      int64_t* part = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(gws) + ld.part_off);
      b.part = part;
      b.status = d_status;
      b.n = wd->n;
      b.k = wd->k;
      b.t = t;
      b.n_pad = wd->n_pad;
      b.t_pad = ld.t_pad;
      b.nb = wd->nb;
      b.b0 = 0;
      b.b1 = wd->nb;
      b.out_mode = OUT_PARTIAL;
      if (launch_gemm_skinny(b, 3, ld.splits, narrow_scales(wd->smax, wd->nb), s) != hipSuccess) return EI_EDEVICE;
      const hipError_t e =
          next_gnorm ? launch_combine_rmsnorm_tiles(part, ld.splits, x, y, next_gnorm, eps_q32, out_limbs, t,
                                                    ld.t_pad, wd->n, d_status, s)
                     : launch_combine_hr_tiles(part, ld.splits, y, t, wd->n, x, out_limbs, ld.t_pad, d_status, s);
      return e == hipSuccess ? EI_OK : EI_EDEVICE;
    }
    const int r = run_gemm(wd, nullptr, 0, y, t, 3, EI_SCHED_DEFAULT, 0, gws, gws_bytes, d_status, s, OUT_ROUND_Q24,
                           x, h_limbs);
    if (r != EI_OK || !out_limbs) return r;
    const hipError_t e = next_gnorm
                             ? launch_rmsnorm_limb_tiles(y, next_gnorm, eps_q32, out_limbs, t, ld.t_pad, wd->n,
                                                         d_status, s)
                             : launch_limb_tiles(y, 0, t, wd->n, 3, out_limbs, ld.t_pad, d_status, s);
    return e == hipSuccess ? EI_OK : EI_EDEVICE;
  }
  const int64_t* xin = x;
  if (gnorm) {
    int64_t* n = reinterpret_cast<int64_t*>(ws + f.n_off);
    if (launch_rmsnorm_q16(x, gnorm, eps_q32, n, t, wg->k, d_status, s) != hipSuccess) return EI_EDEVICE;
    xin = n;
  }
  int64_t* h = reinterpret_cast<int64_t*>(ws + f.h_off);
  int64_t* g = reinterpret_cast<int64_t*>(ws + f.g_off);
  int64_t* u = reinterpret_cast<int64_t*>(ws + f.u_off);
  int r = EI_OK;
  if (t <= kSmallT) {   // decode sizes: gate and up share x, one batched GEMV launch
    const ei_weights* pair[2] = {wg, wu};
    int64_t* outs[2] = {g, u};
    r = int_gemm_q8_multi(pair, 2, xin, outs, t, 3, d_status, s);
  } else {
    r = run_gemm(wg, xin, 0, g, t, 3, EI_SCHED_DEFAULT, 0, gws, gws_bytes, d_status, s, OUT_ROUND_Q24);
    if (r == EI_OK) r = run_gemm(wu, xin, 0, u, t, 3, EI_SCHED_DEFAULT, 0, gws, gws_bytes, d_status, s, OUT_ROUND_Q24);
  }
  if (r != EI_OK) return r;
  if (launch_silu_mul(g, u, lut, h, t * wg->n, d_status, s) != hipSuccess) return EI_EDEVICE;
  return run_gemm(wd, h, 0, y, t, 3, EI_SCHED_DEFAULT, 0, gws, gws_bytes, d_status, s, OUT_ROUND_Q24, x);
}

}  // namespace

extern "C" {

int int_ffn_q8(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd, const int64_t* x,
               const int32_t* lut, int64_t* y, int64_t t, void* workspace, size_t workspace_bytes,
               int32_t* d_status, ei_stream stream) {
  return ffn_run(wg, wu, wd, x, nullptr, 0, lut, y, t, workspace, workspace_bytes, d_status,
                 static_cast<hipStream_t>(stream));
}

size_t ei_ffn_chain_workspace_bytes(const ei_weights* wg, const ei_weights* wd, int64_t t) {
  if (!wg || !wd || t < 1) return 0;
  return ffn_layout(wg, wd, t).total + align_up(sizeof(int64_t) * (size_t)t * (size_t)wg->k) +
         align_up((size_t)3 * (size_t)round_up(t, kTile) * (size_t)wg->k);
}

int int_ffn_q8_chain(const ei_weights* const* layers, int n_layers, const int64_t* x, const int32_t* lut, int64_t* y,
                     int64_t t, void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  if (!layers || n_layers < 1 || !x || !lut || !y || t < 1) return EI_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    const ei_weights *wg = layers[3 * l], *wu = layers[3 * l + 1], *wd = layers[3 * l + 2];
    const int c = ffn_check(wg, wu, wd);
    if (c != EI_OK) return c;
    if (wg->n != layers[0]->n || wg->k != layers[0]->k) return EI_EINVAL;   // one shape for the whole chain
  }
  const ei_weights *g0 = layers[0], *d0 = layers[2];
  const FfnLayout f = ffn_layout(g0, d0, t);
  if (!workspace || workspace_bytes < ei_ffn_chain_workspace_bytes(g0, d0, t)) return EI_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int64_t* xbuf = reinterpret_cast<int64_t*>(ws + f.total);
  int8_t* limbs = reinterpret_cast<int8_t*>(ws + f.total + align_up(sizeof(int64_t) * (size_t)t * (size_t)g0->k));
  const int64_t t_pad = round_up(t, kTile);
  // layer l writes y when n_layers - 1 - l is even, else xbuf, so the last
  // layer lands in y; on the fused path each layer's combiner leaves the next
  // layer's input limbs in `limbs` (the first layer's are split here)
  if (f.fused && launch_limb_tiles(x, 0, t, g0->k, 3, limbs, t_pad, d_status, s) != hipSuccess) return EI_EDEVICE;
  const int64_t* in = x;
  for (int l = 0; l < n_layers; ++l) {
    int64_t* out = ((n_layers - 1 - l) % 2 == 0) ? y : xbuf;
    const bool last = l == n_layers - 1;
    const int r = ffn_run(layers[3 * l], layers[3 * l + 1], layers[3 * l + 2], in, nullptr, 0, lut, out, t, workspace,
                          f.total, d_status, s, f.fused ? limbs : nullptr, f.fused && !last ? limbs : nullptr);
    if (r != EI_OK) return r;
    in = out;
  }
  return EI_OK;
}

int int_ffn_q8_prenorm(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd, const int32_t* g_norm,
                       int64_t eps_q32, const int64_t* x, const int32_t* lut, int64_t* y, int64_t t,
                       void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  if (!g_norm) return EI_EINVAL;
  return ffn_run(wg, wu, wd, x, g_norm, eps_q32, lut, y, t, workspace, workspace_bytes, d_status,
                 static_cast<hipStream_t>(stream));
}

int int_ffn_q8_prenorm_chain(const ei_weights* const* layers, int n_layers, const int32_t* const* g_norms,
                             int64_t eps_q32, const int64_t* x, const int32_t* lut, int64_t* y, int64_t t,
                             void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  if (!layers || n_layers < 1 || !g_norms || !x || !lut || !y || t < 1) return EI_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    const ei_weights *wg = layers[3 * l], *wu = layers[3 * l + 1], *wd = layers[3 * l + 2];
    const int c = ffn_check(wg, wu, wd);
    if (c != EI_OK) return c;
    if (wg->n != layers[0]->n || wg->k != layers[0]->k) return EI_EINVAL;   // one shape for the whole chain
    if (!g_norms[l]) return EI_EINVAL;
  }
  const ei_weights *g0 = layers[0], *d0 = layers[2];
  if (g0->k > 65536 || eps_q32 < 1 || eps_q32 > ((int64_t)1 << 32)) return EI_ERANGE;
  const FfnLayout f = ffn_layout(g0, d0, t);
  if (!workspace || workspace_bytes < ei_ffn_chain_workspace_bytes(g0, d0, t)) return EI_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int64_t* xbuf = reinterpret_cast<int64_t*>(ws + f.total);
  int8_t* limbs = reinterpret_cast<int8_t*>(ws + f.total + align_up(sizeof(int64_t) * (size_t)t * (size_t)g0->k));
  const int64_t t_pad = round_up(t, kTile);
  // as int_ffn_q8_chain; on the fused path the first layer's normalized input
  // goes into `limbs` here and every later layer's as its predecessor's
  // residual stream is formed
  if (f.fused && launch_rmsnorm_limb_tiles(x, g_norms[0], eps_q32, limbs, t, t_pad, g0->k, d_status, s) != hipSuccess)
    return EI_EDEVICE;
  const int64_t* in = x;
  for (int l = 0; l < n_layers; ++l) {
    int64_t* out = ((n_layers - 1 - l) % 2 == 0) ? y : xbuf;
    const bool last = l == n_layers - 1;
    const int r = ffn_run(layers[3 * l], layers[3 * l + 1], layers[3 * l + 2], in, g_norms[l], eps_q32, lut, out, t,
                          workspace, f.total, d_status, s, f.fused ? limbs : nullptr,
                          f.fused && !last ? limbs : nullptr, f.fused && !last ? g_norms[l + 1] : nullptr);
    if (r != EI_OK) return r;
    in = out;
  }
  return EI_OK;
}

size_t ei_moe_ffn_workspace_bytes(const ei_weights* wg, const ei_weights* wd, int64_t rows, int topk) {
  if (!wg || !wd || rows < 1 || topk < 1) return 0;
  return moe_layout(wg, wd, rows, topk).total;
}

int int_moe_ffn_q8(const ei_weights* wg, const ei_weights* wu, const ei_weights* wd, const int64_t* x,
                   const int32_t* route, int64_t rows, int topk, const int32_t* lut, int64_t* y, void* workspace,
                   size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  if (!x || !route || !lut || !y) return EI_EINVAL;
  int c = ffn_check(wg, wu, wd);
  if (c == EI_OK) c = grouped_check(wg, rows, topk, 3);
  if (c == EI_OK) c = grouped_check(wd, rows * topk, 1, 3);
  if (c != EI_OK) return c;
  if (wu->experts != wg->experts || wd->experts != wg->experts || wu->expert_stride != wg->expert_stride)
    return EI_EINVAL;
  const MoeLayout m = moe_layout(wg, wd, rows, topk);
  if (!workspace || workspace_bytes < m.total) return EI_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const Grouping p = grouping_at(workspace, m.g);
  int8_t* hl = reinterpret_cast<int8_t*>(ws + m.hl_off);
  const int64_t pairs = m.g.pairs;
  // one grouping serves all three projections: pair p of the down projection
  // is row p of h, in the same sorted order, so the gate/up pass writes h
  // straight into the down projection's limb tiles
  hipError_t e = launch_moe_sort(route, pairs, wg->experts, p.sorted, p.offs, p.texp, p.trow0, p.trows, p.ntiles,
                                 d_status, s);
  if (e == hipSuccess)
    e = launch_grouped_limb_tiles(x, wg->k, topk, p.sorted, p.trow0, p.trows, p.ntiles, m.g.tiles_max, p.limb,
                                  d_status, s);
  if (e == hipSuccess) e = launch_grouped_projection(wg, m.g, p, nullptr, d_status, s, wu, lut, hl);
  if (e == hipSuccess) {
    GroupedLayout gd = m.g;   // the down projection: same pairs and tiles, its own k
    e = launch_grouped_projection(wd, gd, p, y, d_status, s, nullptr, nullptr, nullptr, hl);
  }
  return e == hipSuccess ? EI_OK : EI_EDEVICE;
}

int ei_limb_split(const int64_t* x, int8_t* d, int64_t n, int limbs, int32_t* d_status, ei_stream stream) {
  if (!x || !d || n < 0) return EI_EINVAL;
  if (limbs < 1 || limbs > 8) return EI_EINVAL;
  return launch_limb_split_flat(x, d, n, limbs, d_status, static_cast<hipStream_t>(stream)) == hipSuccess
             ? EI_OK
             : EI_EDEVICE;
}

size_t ei_gemm_workspace_bytes(const ei_weights* w, int64_t t, int limbs, int schedule) {
  if (!w || t < 1 || limbs < 1) return 0;
  return layout_for(w, t, limbs, schedule).total;
}

int int_gemm_q8(const ei_weights* w, const int64_t* x, int64_t* y, int64_t t, int limbs, int schedule,
                uint64_t shuffle_seed, void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  const int c = check_weights(w, EI_FORMAT_Q8);
  if (c != EI_OK) return c;
  return run_gemm(w, x, 0, y, t, limbs, schedule, shuffle_seed, workspace, workspace_bytes, d_status,
                  static_cast<hipStream_t>(stream), OUT_ROUND_Q24);
}

// ------------------------------------------------ allocation-free projection
// Scratch memory of int_gemm_q8_noalloc: one array per device, in the code
// object, held until the process ends.  Host code never uses the symbol's
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device, and is cached below.
}  // extern "C"

namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;   // 32 MiB
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, looked up on the first call made
// with that device current.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EI_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EI_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EI_OK;
}
}  // namespace

extern "C" {

int int_gemm_q8_noalloc(const ei_weights* w, const int64_t* x, int64_t* y, int64_t t, int limbs,
                        int32_t* d_status, ei_stream stream) {
  const int c = check_weights(w, EI_FORMAT_Q8);
  if (c != EI_OK) return c;
  if (!x || !y || t < 1 || limbs < 1 || limbs > 8) return EI_EINVAL;
  if (limbs > kMaxLimbs) return EI_ERANGE;
  const size_t need = layout_for(w, t, limbs, EI_SCHED_DEFAULT).total;
  if (need > kNoAllocScratchBytes) return EI_ENOSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int sc = scratch_of_current_device(&ws);
    if (sc != EI_OK) return sc;
  }
  return run_gemm(w, x, 0, y, t, limbs, EI_SCHED_DEFAULT, 0, ws, need, d_status, static_cast<hipStream_t>(stream),
                  OUT_ROUND_Q24);
}

int int_gemm_q8_multi(const ei_weights* const* w, int count, const int64_t* x, int64_t* const* y, int64_t t,
                      int limbs, int32_t* d_status, ei_stream stream) {
  if (!w || !y || !x || count < 1 || count > kMultiMax) return EI_EINVAL;
  if (t < 1 || t > kSmallT || limbs < 1 || limbs > 8) return EI_EINVAL;
  if (limbs > kMaxLimbs) return EI_ERANGE;
  GemvMulti mm;
  std::memset(&mm, 0, sizeof mm);
  mm.count = count;
  for (int m = 0; m < count; ++m) {
    const int c = check_weights(w[m], EI_FORMAT_Q8);
    if (c != EI_OK) return c;
    if (w[m]->k != w[0]->k || !y[m]) return EI_EINVAL;
    const uint8_t* base = static_cast<const uint8_t*>(w[m]->packed);
    mm.codes[m] = reinterpret_cast<const int8_t*>(base + kHeaderBytes);
    mm.scales[m] = reinterpret_cast<const int32_t*>(base + kHeaderBytes + w[m]->n_pad * w[m]->k);
    mm.y[m] = y[m];
    mm.n[m] = w[m]->n;
    mm.n_pad[m] = w[m]->n_pad;
    mm.rg0[m + 1] = mm.rg0[m] + w[m]->n_pad / kTile;
  }
  if (mm.rg0[count] > 0x7FFFFFFF) return EI_ERANGE;   // one grid dimension
  GemmArgs a;
  std::memset(&a, 0, sizeof a);
  a.x = x;
  a.status = d_status;
  a.k = w[0]->k;
  a.t = t;
  a.nb = w[0]->nb;
  a.b0 = 0;
  a.b1 = w[0]->nb;
  a.out_mode = OUT_ROUND_Q24;
  a.order = ORDER_ASC;
  return launch_gemv_multi(a, mm, limbs, static_cast<hipStream_t>(stream)) == hipSuccess ? EI_OK : EI_EDEVICE;
}

int int_gemm_q4(const ei_weights* w, const int32_t* x, int64_t* y, int64_t t, int limbs, int schedule,
                uint64_t shuffle_seed, void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  const int c = check_weights(w, EI_FORMAT_Q4);
  if (c != EI_OK) return c;
  // two limbs: the split takes x - 128 and every row gets its R_i back
  const int64_t* roff =
      limbs == 2 ? reinterpret_cast<const int64_t*>(static_cast<const uint8_t*>(w->packed) + row_offsets_at(w->n_pad, w->k))
                 : nullptr;
  return run_gemm(w, x, 1, y, t, limbs, schedule, shuffle_seed, workspace, workspace_bytes, d_status,
                  static_cast<hipStream_t>(stream), OUT_EXACT, nullptr, nullptr, roff, roff ? kQ4Offset : 0);
}

int ei_topk_route(const int64_t* scores, int64_t t, int64_t e, int k, int32_t* route, ei_stream stream) {
  if (!scores || !route || t < 1 || e < 1 || k < 1 || k > e) return EI_EINVAL;
  if (e > 2048) return EI_ERANGE;
  return launch_topk(scores, t, e, k, route, static_cast<hipStream_t>(stream)) == hipSuccess ? EI_OK : EI_EDEVICE;
}

size_t ei_wide_packed_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 32 || k % 32 != 0) return 0;
  return (size_t)kHeaderBytes + (size_t)round_up(n, kTile) * (size_t)k * 3u;
}

int ei_wide_pack(const int32_t* codes, int64_t n, int64_t k, void* packed, size_t packed_bytes, ei_weights* out,
                 ei_stream stream) {
  if (!codes || !packed || !out || n < 1 || k < 32 || k % 32 != 0) return EI_EINVAL;
  if (!aligned(packed, 256) || !aligned(codes, 16)) return EI_EINVAL;
  if (packed_bytes < ei_wide_packed_bytes(n, k)) return EI_ENOSPACE;
  const int64_t n_pad = round_up(n, kTile);
  if (n_pad * k * 3 >= ((int64_t)1 << 32)) return EI_ERANGE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PackedHeader h;
  std::memset(&h, 0, sizeof h);
  h.magic = kMagic;
  h.format = EI_FORMAT_WIDE;
  h.n = n;
  h.k = k;
  h.n_pad = n_pad;
  h.nb = k / 32;
  h.codes_off = kHeaderBytes;
  h.scales_off = 0;
  PackedHeader* dh = static_cast<PackedHeader*>(packed);
  if (hipMemcpyAsync(dh, &h, sizeof h, hipMemcpyHostToDevice, s) != hipSuccess) return EI_EDEVICE;
  // pad0 of the device header collects the range flag of the digit split
  if (launch_wide_pack(codes, n, k, n_pad, static_cast<int8_t*>(packed) + kHeaderBytes, &dh->pad0, s) != hipSuccess)
    return EI_EDEVICE;
  if (hipMemcpyAsync(&h, dh, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess) return EI_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return EI_EDEVICE;
  if (h.magic != kMagic || h.n != n || h.k != k) return EI_EDEVICE;
  if (h.pad0 != 0) return EI_ERANGE;
  out->packed = packed;
  out->n = n;
  out->k = k;
  out->n_pad = n_pad;
  out->nb = k / 32;
  out->smax = 0;
  out->format = EI_FORMAT_WIDE;
  out->experts = 1;
  out->expert_stride = (int64_t)align_up(ei_wide_packed_bytes(n, k));
  return EI_OK;
}

size_t ei_wide_workspace_bytes(const ei_weights* w, int64_t t) {
  if (!w || t < 1) return 0;
  return (size_t)4 * (size_t)round_up(t, kTile) * (size_t)w->k;
}

int int_gemm_wide(const ei_weights* w, const int32_t* x, int64_t* y, int64_t t, void* workspace,
                  size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  if (!w || !w->packed || w->format != EI_FORMAT_WIDE || !x || !y || t < 1) return EI_EINVAL;
  if (w->k < 32 || w->k % 32 != 0 || w->nb != w->k / 32 || w->n_pad != round_up(w->n, kTile)) return EI_EINVAL;
  const int64_t t_pad = round_up(t, kTile);
  if (w->k > 32768 || 4 * t_pad * w->k >= ((int64_t)1 << 32)) return EI_ERANGE;
  if (!workspace || workspace_bytes < ei_wide_workspace_bytes(w, t)) return EI_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int8_t* atiles = static_cast<int8_t*>(workspace);
  if (launch_limb_tiles(x, 1, t, w->k, 4, atiles, t_pad, d_status, s) != hipSuccess) return EI_EDEVICE;
  const int8_t* wtiles = static_cast<const int8_t*>(w->packed) + kHeaderBytes;
  return launch_wide_gemm(wtiles, atiles, y, w->n, t, w->n_pad, t_pad, w->nb, d_status, s) == hipSuccess
             ? EI_OK
             : EI_EDEVICE;
}

int ei_requant(const int64_t* c, int64_t m, int k, int64_t* y, int64_t n, int32_t* d_status, ei_stream stream) {
  if (n < 0 || (n > 0 && (!c || !y)) || k < 0 || k > 126) return EI_EINVAL;
  return launch_requant(c, m, k, y, n, d_status, static_cast<hipStream_t>(stream)) == hipSuccess ? EI_OK
                                                                                                 : EI_EDEVICE;
}

int ei_rmsnorm_q16(const int64_t* x, const int32_t* g, int64_t eps_q32, int64_t* y, int64_t t, int64_t d,
                   int32_t* d_status, ei_stream stream) {
  if (!x || !g || !y || t < 1 || d < 1) return EI_EINVAL;
  if (d > 65536 || eps_q32 < 1 || eps_q32 > ((int64_t)1 << 32)) return EI_ERANGE;
  return launch_rmsnorm_q16(x, g, eps_q32, y, t, d, d_status, static_cast<hipStream_t>(stream)) == hipSuccess
             ? EI_OK
             : EI_EDEVICE;
}

size_t ei_q4_table_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  if (n < 1 || t < 1 || k < 32 || k % 32 != 0 || t > 65535 || k > kMaxQ4TableK) return 0;
  return q4_table_workspace_bytes(n, k, t);
}

int int_gemm_q4_table(const uint8_t* nib, const uint8_t* sme, const int32_t* x, int64_t* y, int64_t n, int64_t k,
                      int64_t t, void* workspace, size_t workspace_bytes, int32_t* d_status, ei_stream stream) {
  if (!nib || !sme || !x || !y || n < 1 || t < 1 || k < 32 || k % 32 != 0) return EI_EINVAL;
  if (t > 65535 || k > kMaxQ4TableK) return EI_ERANGE;
  const size_t need = q4_table_workspace_bytes(n, k, t);
  if (need > 0 && (!workspace || workspace_bytes < need)) return EI_ENOSPACE;
  if (need > 0 && !aligned(workspace, 16)) return EI_EINVAL;   // int128 sums
  return launch_q4_table(nib, sme, x, y, n, k, t, workspace, d_status, static_cast<hipStream_t>(stream)) == hipSuccess
             ? EI_OK
             : EI_EDEVICE;
}

int silu_lut_epilogue_radix16(const int64_t* gate, const int64_t* up, const int32_t* lut, int64_t* h, int64_t n,
                              int32_t* d_status, ei_stream stream) {
  if (!gate || !up || !lut || !h || n < 0) return EI_EINVAL;
  return launch_silu_mul_radix16(gate, up, lut, h, n, d_status, static_cast<hipStream_t>(stream)) == hipSuccess
             ? EI_OK
             : EI_EDEVICE;
}

int ei_silu_lut_build(int32_t* lut, ei_stream stream) {
  if (!lut) return EI_EINVAL;
  return launch_silu_lut(lut, static_cast<hipStream_t>(stream)) == hipSuccess ? EI_OK : EI_EDEVICE;
}

int silu_lut_epilogue(const int64_t* gate, const int64_t* up, const int32_t* lut, int64_t* h, int64_t n,
                      int32_t* d_status, ei_stream stream) {
  if (!gate || !up || !lut || !h || n < 0) return EI_EINVAL;
  return launch_silu_mul(gate, up, lut, h, n, d_status, static_cast<hipStream_t>(stream)) == hipSuccess
             ? EI_OK
             : EI_EDEVICE;
}

int ei_q8_fp32_shadow(const int8_t* codes, const int32_t* scales, const int64_t* x, float* y, int64_t n, int64_t k,
                      int64_t t, int schedule, uint64_t shuffle_seed, ei_stream stream) {
  if (!codes || !scales || !x || !y || n < 1 || t < 1 || k < 32 || k % 32 != 0) return EI_EINVAL;
  if (schedule < EI_SCHED_DEFAULT || schedule > EI_SCHED_TREE) return EI_EINVAL;
  if ((k + 127) / 128 > 16384) return EI_ERANGE;   // the tile permutation lives in LDS
  return launch_shadow(codes, scales, x, y, n, k, t, schedule, shuffle_seed, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? EI_OK
             : EI_EDEVICE;
}

int output_digest(const void* dptr, size_t nbytes, uint8_t* out, ei_stream stream) {
  if (!out || (!dptr && nbytes)) return EI_EINVAL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return EI_EDEVICE;
  void* host = std::malloc(nbytes ? nbytes : 1);
  if (!host) return EI_ENOSPACE;
  if (nbytes && hipMemcpy(host, dptr, nbytes, hipMemcpyDeviceToHost) != hipSuccess) {
    std::free(host);
    return EI_EDEVICE;
  }
  ei::sha256(host, nbytes, out);
  std::free(host);
  return EI_OK;
}

void ei_sha256_host(const void* data, size_t nbytes, uint8_t* out) { ei::sha256(data, nbytes, out); }

const char* ei_status_string(int code) {
  switch (code) {
    case EI_OK: return "ok";
    case EI_EINVAL: return "invalid argument";
    case EI_ERANGE: return "outside the exactness envelope";
    case EI_EDEVICE: return "HIP runtime error";
    case EI_ENOSPACE: return "workspace or buffer too small";
    default: return "unknown status";
  }
}

int ei_version(void) { return 109; }

}  // extern "C"
