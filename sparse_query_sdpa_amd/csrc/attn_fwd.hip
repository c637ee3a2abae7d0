// Attention forward for gfx950: bf16 MFMA for Q K^T and P V, fp32 online softmax.
//
// Computes, per sample b, head h and selected query row, softmax over the valid
// keys of scale * q . k, times V ("SAFE-DiT" Eq. 2 with no mask; Eq. 16 SRSU
// self-attention on the gathered rows of S; Eq. 17 cross-attention with the text
// padding kept as a per-sample valid key count; Eq. 18 dense anchor pass).
//
// Work decomposition
//   workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32 rows.
//   Keys stream in tiles of 64 through LDS (double buffered, one barrier per tile).
//   Per wave and tile:
//     S^T[64 keys x 32 queries] = K_tile . Q^T     (v_mfma_f32_32x32x16_bf16)
//       A = K rows straight from LDS (d contiguous), B = the wave's Q^T held in
//       registers for the whole loop.  In the 32x32 accumulator layout lane l
//       holds query column l%32 and 16 keys, so every lane owns one query and
//       the row max / row sum need only the partner lane l^32.
//     O^T[d x 32 queries] += V^T . P^T             (same MFMA)
//       B = P^T: the lane's own probabilities, converted to bf16 in registers
//       (no LDS round trip); A = V^T rows from LDS.  V is written to LDS
//       transposed ([d][key]) with keys permuted inside each group of 16 so the
//       A operand's k-slots line up with the accumulator rows of S^T.
//   Online softmax in the log2 domain with a lazily moved reference max: the
//   reference only moves (and O, l are rescaled) when a tile's max exceeds it
//   by more than 2^8, so probabilities stay <= 256 and rescaling is rare.
//   Workgroups are remapped so all row tiles of one (b, h) sit on one XCD and
//   share its L2 for the K/V stream.
#include "common.h"

namespace safe {
namespace {

constexpr int BM = 128;       // query rows per workgroup
constexpr int BN = 64;        // keys per tile
constexpr int NTHREADS = 256;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

struct AttnParams {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  const int32_t* q_rows;
  int64_t qr_bs;
  const int32_t* kv_len;
  float* lse;
  int B, H, Nq, Nk, n_rows, n_row_tiles, total_wg;
  float scale_log2;
  int scatter;
};

// Slot of key-subgroup sg (4 keys) inside a 16-key group of the transposed V tile:
// storage order is keys {0-3, 8-11, 4-7, 12-15}.
__device__ __forceinline__ int vslot(int kg) {
  const int sg = kg & 3;
  return (kg & ~3) * 4 + (((sg & 1) << 1) | (sg >> 1)) * 4;
}

template <int D>
struct TileRegs {
  static constexpr int KCH = BN * D / 8;                       // 16-byte K chunks per tile
  static constexpr int KPT = (KCH + NTHREADS - 1) / NTHREADS;   // per thread
  static constexpr int VTASKS = (BN / 4) * (D / 8);             // 4 keys x 8 d tasks
  u32x4 kr[KPT];
  u32x4 vr[4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, const u16* kbase, const u16* vbase, int64_t ks1,
                                          int64_t vs1, int j0, int nvalid, int tid) {
  constexpr int PARTS = D / 8;
#pragma unroll
  for (int c = 0; c < TileRegs<D>::KPT; ++c) {
    const int chunk = tid + c * NTHREADS;
    const int key = chunk / PARTS, part = chunk % PARTS;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (chunk < TileRegs<D>::KCH && j0 + key < nvalid) val = ld16(kbase + (int64_t)(j0 + key) * ks1 + part * 8);
    t.kr[c] = val;
  }
  if (tid < TileRegs<D>::VTASKS) {
    const int kg = tid / PARTS, part = tid % PARTS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kg * 4 + i;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (j0 + key < nvalid) val = ld16(vbase + (int64_t)(j0 + key) * vs1 + part * 8);
      t.vr[i] = val;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, u16 (*Ks)[D + 8], u16 (*Vs)[BN + 8], int tid) {
  constexpr int PARTS = D / 8;
#pragma unroll
  for (int c = 0; c < TileRegs<D>::KPT; ++c) {
    const int chunk = tid + c * NTHREADS;
    if (chunk < TileRegs<D>::KCH) {
      const int key = chunk / PARTS, part = chunk % PARTS;
      st16(&Ks[key][part * 8], t.kr[c]);
    }
  }
  if (tid < TileRegs<D>::VTASKS) {
    const int kg = tid / PARTS, part = tid % PARTS;
    const int slot = vslot(kg);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // d = part*8 + 2w (low halves) and + 2w + 1 (high halves), keys kg*4 + 0..3
      const u32 a0 = t.vr[0][w], a1 = t.vr[1][w], a2 = t.vr[2][w], a3 = t.vr[3][w];
      u32x2 lo, hi;
      lo[0] = (a0 & 0xFFFFu) | (a1 << 16);
      lo[1] = (a2 & 0xFFFFu) | (a3 << 16);
      hi[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
      hi[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
      st8(&Vs[part * 8 + 2 * w][slot], lo);
      st8(&Vs[part * 8 + 2 * w + 1][slot], hi);
    }
  }
}

template <int D, bool GATHER, bool KVLEN>
__global__ __launch_bounds__(NTHREADS) void attn_fwd_kernel(AttnParams p) {
  constexpr int KS = D / 16;   // k-steps of the Q K^T product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) u16 Ks[2][BN][D + 8];
  __shared__ __attribute__((aligned(16))) u16 Vs[2][D][BN + 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column owned by this lane
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group this lane holds

  const int logical = xcd_remap(blockIdx.x, p.total_wg);
  const int tile = logical % p.n_row_tiles;
  const int bh = logical / p.n_row_tiles;
  const int h = bh % p.H;
  const int b = bh / p.H;

  // ---- this lane's query row --------------------------------------------------
  const int rr = tile * BM + wave * 32 + col;  // output row (compact index)
  const bool row_ok = rr < p.n_rows;
  int qi = rr;
  if (GATHER) qi = row_ok ? p.q_rows[(int64_t)b * p.qr_bs + rr] : -1;
  const bool q_ok = row_ok && qi >= 0 && qi < p.Nq;

  bf16x8 qf[KS];
  {
    const u16* qp = p.q + (int64_t)b * p.qs0 + (int64_t)(q_ok ? qi : 0) * p.qs1 + (int64_t)h * p.qs2 + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q_ok) v = ld16(qp + s * 16);
      qf[s] = as_bf16x8(v);
    }
  }

  int nkeys = p.Nk;
  if (KVLEN) {
    int L = p.kv_len[b];
    nkeys = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  const int ntiles = (nkeys + BN - 1) / BN;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_ref = -INFINITY;  // reference max, log2 domain
  float l_run = 0.f;        // this lane's share of the row sum

  const u16* kbase = p.k + (int64_t)b * p.ks0 + (int64_t)h * p.ks2;
  const u16* vbase = p.v + (int64_t)b * p.vs0 + (int64_t)h * p.vs2;
  const float sl2 = p.scale_log2;

  TileRegs<D> tr;
  if (ntiles > 0) {
    load_tile<D>(tr, kbase, vbase, p.ks1, p.vs1, 0, nkeys, tid);
    store_tile<D>(tr, Ks[0], Vs[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int j0 = it * BN;
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile<D>(tr, kbase, vbase, p.ks1, p.vs1, j0 + BN, nkeys, tid);

    // ---- S^T = K Q^T for 64 keys (two 32-key blocks) -------------------------
    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = as_bf16x8(ld16(&Ks[buf][blk * 32 + col][s * 16 + half * 8]));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], acc, 0, 0, 0);
      }
      sacc[blk] = acc;
    }

    // ---- mask keys past the valid length (last tile only) -------------------
    if (j0 + BN > nkeys) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + blk * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= nkeys) sacc[blk][r] = -INFINITY;
        }
    }

    // ---- tile max (raw scores) over the lane pair ---------------------------
    float mt = sacc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[1][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mt2 = mt * sl2;

    // ---- lazy reference move + rescale (wave-uniform branch) ----------------
    const bool move = mt2 > m_ref + kRescaleThreshold;
    if (__any(move)) {
      const float m_new = move ? mt2 : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // exp2(-inf) = 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      m_ref = m_new;
    }

    // ---- probabilities, row-sum share, bf16 B operands ------------------------
    bf16x8 pb[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 packed;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][8 * t + 2 * e], sl2, -m_ref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][8 * t + 2 * e + 1], sl2, -m_ref));
          l_run += p0 + p1;
          packed[e] = pack_bf16x2(p0, p1);
        }
        pb[blk][t] = as_bf16x8(packed);
      }
    }

    // ---- O^T += V^T P^T --------------------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 vf = as_bf16x8(ld16(&Vs[buf][db * 32 + col][blk * 32 + t * 16 + half * 8]));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[blk][t], oacc[db], 0, 0, 0);
        }
    }

    if (has_next) store_tile<D>(tr, Ks[buf ^ 1], Vs[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- epilogue: normalise, store O (bf16) and LSE ------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const int orow = (GATHER && p.scatter) ? qi : rr;
  if (!GATHER || !p.scatter || q_ok) {
    u16* op = p.o + (int64_t)b * p.os0 + (int64_t)orow * p.os1 + (int64_t)h * p.os2;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        st8(op + db * 32 + 8 * g + 4 * half, w);
      }
  }
  if (p.lse != nullptr && half == 0) {
    const float lse = l_tot > 0.f ? (m_ref + __builtin_log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    p.lse[((int64_t)b * p.H + h) * p.n_rows + rr] = lse;
  }
}

template <int D, bool G, bool KV>
hipError_t launch(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, G, KV>), dim3(p.total_wg), dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_flags(const AttnParams& p, bool gather, bool kvlen, hipStream_t s) {
  if (gather) return kvlen ? launch<D, true, true>(p, s) : launch<D, true, false>(p, s);
  return kvlen ? launch<D, false, true>(p, s) : launch<D, false, false>(p, s);
}

}  // namespace

// Enqueue the attention kernel.  Arguments were validated by the caller.
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
  p.total_wg = (int)total;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.scatter = (a->flags & SAFE_ATTN_SCATTER_OUT) ? 1 : 0;
  const bool gather = a->q_rows != nullptr;
  const bool kvlen = a->kv_len != nullptr;
  hipError_t e;
  switch (a->d) {
    case 32: e = dispatch_flags<32>(p, gather, kvlen, stream); break;
    case 64: e = dispatch_flags<64>(p, gather, kvlen, stream); break;
    case 96: e = dispatch_flags<96>(p, gather, kvlen, stream); break;
    case 128: e = dispatch_flags<128>(p, gather, kvlen, stream); break;
    default: return SAFE_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
