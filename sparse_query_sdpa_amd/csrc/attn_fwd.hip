// Attention forward: launch planning and the mask-free instances ("SAFE-DiT" Eq. 2
// with m empty, Eq. 16-18).  The kernels themselves are in attn_kernel.h; the masked
// instances are compiled in attn_masked.hip.
#include "attn_kernel.h"

namespace safe {
namespace {

template <int D>
hipError_t dispatch_flags(const AttnParams& p, bool gather, bool kvlen, hipStream_t s) {
  if (gather) return kvlen ? launch<D, true, true, kMaskNone, 1>(p, s) : launch<D, true, false, kMaskNone, 1>(p, s);
  return kvlen ? launch<D, false, true, kMaskNone, 1>(p, s) : launch<D, false, false, kMaskNone, 1>(p, s);
}
template <int D>
hipError_t dispatch_two_blocks(const AttnParams& p, bool gather, hipStream_t s) {
  return gather ? launch<D, true, false, kMaskNone, 2>(p, s) : launch<D, false, false, kMaskNone, 2>(p, s);
}

// Fused global K/V (a per-token source map, Eq. 14/16 without the assembly pass): no key
// lengths, no mask; one row block per wave, or two where the mask-free kernel has them.
template <int D, int RB>
hipError_t dispatch_map(const AttnParams& p, bool gather, hipStream_t s) {
  return gather ? launch<D, true, false, kMaskNone, RB, true>(p, s) : launch<D, false, false, kMaskNone, RB, true>(p, s);
}
template <int D, int RB>
int resident_map_d(bool gather) {
  return gather ? resident_workgroups<D, true, false, kMaskNone, RB, true>()
                : resident_workgroups<D, false, false, kMaskNone, RB, true>();
}
int resident_map(int d, bool gather, int rb) {
  switch (d) {
    case 32: return resident_map_d<32, 1>(gather);
    case 64: return resident_map_d<64, 1>(gather);
    case 72: return rb == 2 ? resident_map_d<72, 2>(gather) : resident_map_d<72, 1>(gather);
    case 96: return rb == 2 ? resident_map_d<96, 2>(gather) : resident_map_d<96, 1>(gather);
    case 128: return resident_map_d<128, 1>(gather);
    default: return 0;
  }
}

// Two row blocks per wave are compiled for the head dimensions of the workloads (96) and of
// the paper's tax measurement (72), without key lengths (the text cross-attention keeps one).
bool two_blocks_available(int d) { return d == 96 || d == 72; }

template <int D, int RB>
int resident_rb(bool gather) {
  return gather ? resident_workgroups<D, true, false, kMaskNone, RB>() : resident_workgroups<D, false, false, kMaskNone, RB>();
}

int resident_for(int d, bool gather, int rb) {
  switch (d) {
    case 32: return resident_rb<32, 1>(gather);
    case 64: return resident_rb<64, 1>(gather);
    case 72: return rb == 2 ? resident_rb<72, 2>(gather) : resident_rb<72, 1>(gather);
    case 96: return rb == 2 ? resident_rb<96, 2>(gather) : resident_rb<96, 1>(gather);
    case 128: return resident_rb<128, 1>(gather);
    default: return 0;
  }
}

// Mask element type of a call (kMaskNone without a mask).
int mask_kind(const safe_attn_args* a) {
  if (a->mask == nullptr || a->Nq == 0) return kMaskNone;   // Nq == 0: no row can read the mask
  switch (a->mask_dtype) {
    case SAFE_DT_BOOL: return kMaskBool;
    case SAFE_DT_BF16: return kMaskBf16;
    case SAFE_DT_F16: return kMaskF16;
    default: return kMaskF32;
  }
}

// Time model of a launch (seconds), for the split and row-block choices below: the
// one-row-block kernel runs ~1.1e15 FLOP/s on the whole chip, two row blocks 6% faster
// (both measured at d = 96), and the merge of split partials moves their bytes at ~2.5e12
// B/s (read, plus the rows written).  Rounds of S resident workgroups take equal time.
constexpr double kRate = 1.1e15;
constexpr double kTwoBlockSpeed = 1.06;
constexpr double kMergeBw = 2.5e12;

// Tail split plan.  With S workgroups resident, T whole tiles run in rounds of S; the
// last round holds tail = T mod S tiles (all of them when T < S).  Those tiles are split
// along the keys into nsplit ranges (at least kMinSplitTiles key tiles each, at most
// kMaxSplit ranges); the dispatcher hands the range workgroups to slots as they free up,
// so tail * nsplit may exceed S: the tail then takes ceil(tail * nsplit / S) / nsplit of a
// round.  nsplit minimises that time plus the merge of the partials.
struct SplitPlan {
  int n_full = 0, nsplit = 1, split_tiles = 0, tail = 0;
  int64_t bytes = 0;
};
constexpr int kMinSplitTiles = 4;
constexpr int kMaxSplit = 16;

SplitPlan plan_split(const safe_attn_args* a, int64_t total_tiles, int S, int rows, double round_s) {
  SplitPlan pl;
  pl.n_full = (int)total_tiles;
  if (a->kv_len != nullptr || total_tiles <= 0 || a->Nk <= 0 || S <= 0) return pl;
  const int64_t tail = total_tiles % S;
  if (tail == 0) return pl;
  const int nk_tiles = (a->Nk + BN - 1) / BN;
  const double piece_bytes = (double)tail * rows * ((double)a->d * 4 + 8);
  int best = 1;
  double best_t = round_s;   // unsplit: the tail takes a whole round
  for (int n = 2; n <= kMaxSplit && nk_tiles / n >= kMinSplitTiles; ++n) {
    const double t = (double)((tail * n + S - 1) / S) / n * round_s + n * piece_bytes / kMergeBw;
    if (t < best_t) {
      best_t = t;
      best = n;
    }
  }
  if (best < 2) return pl;
  pl.split_tiles = (nk_tiles + best - 1) / best;
  pl.nsplit = (nk_tiles + pl.split_tiles - 1) / pl.split_tiles;   // every range non-empty
  if (pl.nsplit < 2) return SplitPlan{(int)total_tiles};
  pl.tail = (int)tail;
  pl.n_full = (int)(total_tiles - tail);
  pl.bytes = (int64_t)pl.tail * pl.nsplit * rows * ((int64_t)a->d * 4 + 8);
  return pl;
}

// Row blocks per wave and the split plan of a call.  Two row blocks do the same work 6%
// faster (half the LDS fragment reads and copies per MFMA, and the chip clocks higher for
// it) but hold two workgroups per CU instead of three and make tiles twice as tall; the
// time model picks the faster of the two.
struct Choice {
  int rb = 1, rows = 0;
  int64_t tiles = 0;
  SplitPlan split;
};
Choice choose(const safe_attn_args* a, bool allow_split) {
  const int mt = mask_kind(a);
  const bool gather = a->q_rows != nullptr;
  const double row_flops = 4.0 * a->Nk * a->d;
  Choice best;
  double best_t = 0.0;
  const bool map = a->kv_src != nullptr;
  const int max_rb = (mt == kMaskNone && a->kv_len == nullptr && two_blocks_available(a->d)) ? 2 : 1;
  for (int rb = 1; rb <= max_rb; ++rb) {
    Choice c;
    c.rb = rb;
    c.rows = tile_rows(rb);
    c.tiles = (int64_t)((a->n_rows + c.rows - 1) / c.rows) * a->H * a->B;
    const int S = map ? resident_map(a->d, gather, rb)
                      : (mt == kMaskNone ? resident_for(a->d, gather, rb) : attn_masked_resident(a->d, gather, mt));
    if (rb > 1 && S <= 0) break;
    const double round_s = S > 0 ? (double)S * c.rows * row_flops / (kRate * (rb > 1 ? kTwoBlockSpeed : 1.0)) : 0.0;
    c.split = SplitPlan{(int)std::min<int64_t>(c.tiles, 0x7fffffff)};
    if (allow_split && c.tiles <= 0x7fffffff) c.split = plan_split(a, c.tiles, S, c.rows, round_s);
    double t = 0.0;
    if (S > 0) {
      const int64_t full = c.tiles / S, tail = c.tiles % S;
      const SplitPlan& pl = c.split;
      double rounds = (double)full;
      if (tail > 0) rounds += pl.tail > 0 ? (double)((pl.tail * pl.nsplit + S - 1) / S) / pl.nsplit : 1.0;
      t = rounds * round_s + (pl.tail > 0 ? (double)pl.bytes / kMergeBw : 0.0);
    }
    if (rb == 1 || t < best_t) {
      best = c;
      best_t = t;
    }
  }
  return best;
}

}  // namespace

// The schedule of a call: the split needs a workspace of at least its bytes, else the
// best unsplit schedule runs.
static Choice call_plan(const safe_attn_args* a) {
  Choice c = choose(a, a->workspace != nullptr && a->workspace_bytes > 0);
  if (c.split.tail > 0 && a->workspace_bytes < c.split.bytes) c = choose(a, false);
  return c;
}

int attn_plan(const safe_attn_args* a, safe_attn_plan_info* out) {
  *out = safe_attn_plan_info{};
  if (a->n_rows == 0 || (int64_t)a->H * a->B == 0) return SAFE_OK;
  const Choice c = call_plan(a);
  if (c.tiles > 0x7fffffff) return SAFE_ERR_SHAPE;
  out->rows_per_tile = c.rows;
  out->row_tiles = (int32_t)c.tiles;
  out->split_tiles = c.split.tail;
  out->key_ranges = c.split.tail > 0 ? c.split.nsplit : 1;
  out->keys_per_range = c.split.tail > 0 ? c.split.split_tiles * BN : a->Nk;
  out->workspace_bytes = c.split.tail > 0 ? c.split.bytes : 0;
  return SAFE_OK;
}

int64_t attn_workspace_bytes(const safe_attn_args* a) {
  if (a->n_rows == 0 || (int64_t)a->H * a->B == 0) return 0;
  const Choice c = choose(a, true);
  if (c.tiles > 0x7fffffff) return 0;
  return c.split.tail > 0 ? c.split.bytes : 0;
}

// Enqueue the attention kernel (and the merge of split tiles).  Arguments were validated
// by the caller.
int attn_fwd_launch(const safe_attn_args* a, float scale, hipStream_t stream) {
  if (a->n_rows == 0) return SAFE_OK;
  AttnParams p;
  p.q = static_cast<const u16*>(a->q);
  p.k = static_cast<const u16*>(a->k);
  p.v = static_cast<const u16*>(a->v);
  p.o = static_cast<u16*>(a->o);
  p.qs0 = a->q_stride[0]; p.qs1 = a->q_stride[1]; p.qs2 = a->q_stride[2];
  p.ks0 = a->k_stride[0]; p.ks1 = a->k_stride[1]; p.ks2 = a->k_stride[2];
  p.vs0 = a->v_stride[0]; p.vs1 = a->v_stride[1]; p.vs2 = a->v_stride[2];
  p.os0 = a->o_stride[0]; p.os1 = a->o_stride[1]; p.os2 = a->o_stride[2];
  p.q_rows = a->q_rows;
  p.qr_bs = a->q_rows_bstride;
  p.kv_len = a->kv_len;
  p.lse = a->lse;
  p.B = a->B; p.H = a->H; p.Nq = a->Nq; p.Nk = a->Nk; p.n_rows = a->n_rows;
  const int mt = mask_kind(a);
  const Choice c = call_plan(a);
  p.n_row_tiles = (a->n_rows + c.rows - 1) / c.rows;
  const int64_t total = (int64_t)p.n_row_tiles * a->H * a->B;
  if (total > 0x7fffffff) return SAFE_ERR_SHAPE;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.scatter = (a->flags & SAFE_ATTN_SCATTER_OUT) ? 1 : 0;
  p.mask = static_cast<const char*>(mt == kMaskNone ? nullptr : a->mask);
  p.ms0 = a->mask_stride[0]; p.ms1 = a->mask_stride[1]; p.ms2 = a->mask_stride[2];
  p.inv_scale = 1.0f / scale;
  p.kv_src = a->kv_src;
  p.src_bs = a->kv_src_bstride;
  p.nsel = a->n_fresh;
  p.kf = static_cast<const u16*>(a->k_fresh);
  p.vf = static_cast<const u16*>(a->v_fresh);
  p.fs0 = a->fresh_stride[0]; p.fs1 = a->fresh_stride[1]; p.fs2 = a->fresh_stride[2];
  const SplitPlan& pl = c.split;
  p.n_full = pl.n_full;
  p.nsplit = pl.nsplit;
  p.split_tiles = pl.split_tiles;
  p.n_slots = pl.tail * pl.nsplit;
  p.part = pl.tail > 0 ? static_cast<float*>(a->workspace) : nullptr;
  p.total_wg = pl.n_full + p.n_slots;
  // a per-query-row mask shared by the heads: tiles of four (two) heads of one row tile side
  // by side (a key mask, broadcast over the rows too, is small and keeps the K/V order)
  p.head_group = 1;
  if (mt != kMaskNone && a->mask_stride[1] == 0 && a->mask_stride[2] != 0)
    p.head_group = a->H % 4 == 0 ? 4 : (a->H % 2 == 0 ? 2 : 1);
  const bool gather = a->q_rows != nullptr;
  const bool kvlen = a->kv_len != nullptr;
  hipError_t e;
  if (p.kv_src != nullptr) {
    switch (a->d) {
      case 32: e = dispatch_map<32, 1>(p, gather, stream); break;
      case 64: e = dispatch_map<64, 1>(p, gather, stream); break;
      case 72: e = c.rb == 2 ? dispatch_map<72, 2>(p, gather, stream) : dispatch_map<72, 1>(p, gather, stream); break;
      case 96: e = c.rb == 2 ? dispatch_map<96, 2>(p, gather, stream) : dispatch_map<96, 1>(p, gather, stream); break;
      case 128: e = dispatch_map<128, 1>(p, gather, stream); break;
      default: return SAFE_ERR_UNSUPPORTED;
    }
  } else if (mt != kMaskNone) {
    e = attn_masked_dispatch(p, a->d, gather, mt, stream);
  } else if (attn_short_applies(a)) {
    e = attn_short_launch(p, a->d, stream);
  } else {
    switch (a->d) {
      case 32: e = dispatch_flags<32>(p, gather, kvlen, stream); break;
      case 64: e = dispatch_flags<64>(p, gather, kvlen, stream); break;
      case 72: e = c.rb == 2 ? dispatch_two_blocks<72>(p, gather, stream) : dispatch_flags<72>(p, gather, kvlen, stream); break;
      case 96: e = c.rb == 2 ? dispatch_two_blocks<96>(p, gather, stream) : dispatch_flags<96>(p, gather, kvlen, stream); break;
      case 128: e = dispatch_flags<128>(p, gather, kvlen, stream); break;
      default: return SAFE_ERR_UNSUPPORTED;
    }
  }
  return e == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
