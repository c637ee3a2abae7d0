// Attention forward: launch planning and the mask-free instances ("SAFE-DiT" Eq. 2
// with m empty, Eq. 16-18).  The kernels themselves are in attn_kernel.h; the masked
// instances are compiled in attn_masked.hip.
#include "attn_kernel.h"

namespace safe {
namespace {

template <int D>
hipError_t dispatch_flags(const AttnParams& p, bool gather, bool kvlen, hipStream_t s) {
  if (gather) return kvlen ? launch<D, true, true, kMaskNone>(p, s) : launch<D, true, false, kMaskNone>(p, s);
  return kvlen ? launch<D, false, true, kMaskNone>(p, s) : launch<D, false, false, kMaskNone>(p, s);
}

int resident_for(int d, bool gather) {
  switch (d) {
    case 32: return gather ? resident_workgroups<32, true, false, kMaskNone>() : resident_workgroups<32, false, false, kMaskNone>();
    case 64: return gather ? resident_workgroups<64, true, false, kMaskNone>() : resident_workgroups<64, false, false, kMaskNone>();
    case 72: return gather ? resident_workgroups<72, true, false, kMaskNone>() : resident_workgroups<72, false, false, kMaskNone>();
    case 96: return gather ? resident_workgroups<96, true, false, kMaskNone>() : resident_workgroups<96, false, false, kMaskNone>();
    case 128: return gather ? resident_workgroups<128, true, false, kMaskNone>() : resident_workgroups<128, false, false, kMaskNone>();
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

// Tail split plan.  With S workgroups resident, T whole tiles run in rounds of S; the
// last round holds tail = T mod S tiles (all of them when T < S).  Splitting each of
// those along the keys into up to S / tail ranges (at least kMinSplitTiles key tiles
// each, at most kMaxSplit ranges) fills that round with short workgroups instead.
struct SplitPlan {
  int n_full = 0, nsplit = 1, split_tiles = 0, tail = 0;
  int64_t bytes = 0;
};
constexpr int kMinSplitTiles = 4;
constexpr int kMaxSplit = 16;

SplitPlan plan_split(const safe_attn_args* a, int64_t total_tiles) {
  SplitPlan pl;
  pl.n_full = (int)total_tiles;
  if (a->kv_len != nullptr || total_tiles <= 0 || a->Nk <= 0) return pl;
  const int mt = mask_kind(a);
  const bool gather = a->q_rows != nullptr;
  const int S = mt == kMaskNone ? resident_for(a->d, gather) : attn_masked_resident(a->d, gather, mt);
  if (S <= 0) return pl;
  const int64_t tail = total_tiles % S;
  if (tail == 0) return pl;
  const int nk_tiles = (a->Nk + BN - 1) / BN;
  int nsplit = (int)std::min<int64_t>(S / tail, kMaxSplit);
  nsplit = std::min(nsplit, nk_tiles / kMinSplitTiles);
  if (nsplit < 2) return pl;
  pl.split_tiles = (nk_tiles + nsplit - 1) / nsplit;
  pl.nsplit = (nk_tiles + pl.split_tiles - 1) / pl.split_tiles;   // every range non-empty
  if (pl.nsplit < 2) return SplitPlan{(int)total_tiles};
  pl.tail = (int)tail;
  pl.n_full = (int)(total_tiles - tail);
  pl.bytes = (int64_t)pl.tail * pl.nsplit * BM * ((int64_t)a->d * 4 + 8);
  return pl;
}

}  // namespace

int64_t attn_workspace_bytes(const safe_attn_args* a) {
  const int64_t total = (int64_t)((a->n_rows + BM - 1) / BM) * a->H * a->B;
  if (a->n_rows == 0 || total == 0 || total > 0x7fffffff) return 0;
  return plan_split(a, total).bytes;
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
  p.n_row_tiles = (a->n_rows + BM - 1) / BM;
  const int64_t total = (int64_t)p.n_row_tiles * a->H * a->B;
  if (total > 0x7fffffff) return SAFE_ERR_SHAPE;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.scatter = (a->flags & SAFE_ATTN_SCATTER_OUT) ? 1 : 0;
  const int mt = mask_kind(a);
  p.mask = static_cast<const char*>(mt == kMaskNone ? nullptr : a->mask);
  p.ms0 = a->mask_stride[0]; p.ms1 = a->mask_stride[1]; p.ms2 = a->mask_stride[2];
  p.inv_scale = 1.0f / scale;
  SplitPlan pl;
  pl.n_full = (int)total;
  if (a->workspace != nullptr && a->workspace_bytes > 0) {
    pl = plan_split(a, total);
    if (pl.tail == 0 || a->workspace_bytes < pl.bytes) pl = SplitPlan{(int)total};
  }
  p.n_full = pl.n_full;
  p.nsplit = pl.nsplit;
  p.split_tiles = pl.split_tiles;
  p.n_slots = pl.tail * pl.nsplit;
  p.part = pl.tail > 0 ? static_cast<float*>(a->workspace) : nullptr;
  p.total_wg = pl.n_full + p.n_slots;
  const bool gather = a->q_rows != nullptr;
  const bool kvlen = a->kv_len != nullptr;
  hipError_t e;
  if (mt != kMaskNone) {
    e = attn_masked_dispatch(p, a->d, gather, mt, stream);
  } else {
    switch (a->d) {
      case 32: e = dispatch_flags<32>(p, gather, kvlen, stream); break;
      case 64: e = dispatch_flags<64>(p, gather, kvlen, stream); break;
      case 72: e = dispatch_flags<72>(p, gather, kvlen, stream); break;
      case 96: e = dispatch_flags<96>(p, gather, kvlen, stream); break;
      case 128: e = dispatch_flags<128>(p, gather, kvlen, stream); break;
      default: return SAFE_ERR_UNSUPPORTED;
    }
  }
  return e == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
