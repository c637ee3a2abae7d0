// Attention over a short key set with per-sample key lengths: the image-text
// cross-attention of the rows of S ("SAFE-DiT" Eq. 17: the text padding kept as a
// per-sample valid key count), the same result as attn_fwd_kernel with key lengths.
//
// With a few hundred text keys a workgroup of the general kernel spends most of its life
// waiting for its query rows and then for its output stores: one (b, h, 128-row tile)
// per workgroup has too little work to hide either.  Here a workgroup owns 128 query
// rows of one sample and a group of heads and walks its (head, 32-key tile) steps as one
// software pipeline (the same structure as the PCSP accumulation):
//   * each step waits for the copies the step before issued, then starts the next
//     step's direct-to-LDS copies: the next 32 keys and values (two LDS stages), and at a
//     head's last step the next head's 128 query rows (an LDS buffer, read into registers
//     at that head's first step);
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 in the layouts of
//     attn_fwd_kernel (each lane owns one query row; V^T read with the LDS transpose
//     load; P^T packed to bf16 in registers), one 32-key block per step;
//   * the softmax keeps a lazy reference as there: the max of a head's first block, then
//     probabilities against it, the max taken again only when a block's per-lane sum
//     leaves [0, 2^16];
//   * at a head's last step the rows are normalised and stored (and the LSE).
// Rows outside the selection (index past Nq or negative) read a zero query row, as in
// the general kernel; blocks wholly past the key length are skipped.
#include "attn_kernel.h"

namespace safe {
namespace {

constexpr int SBN = 32;    // keys per step
constexpr int SBM = 128;   // query rows per workgroup (4 waves x 32)
constexpr int SWAVES = 4;
constexpr float kShortSumLimit = 65536.f;
constexpr float kShortMoveMargin = 8.f;

template <int D>
struct ShortTile {
  using T = Tile<D>;
  static constexpr int CH = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int K_BYTES = SBN * T::K_ROWB;
  static constexpr int V_BYTES = SBN * T::V_ROWB;
  static constexpr int KCH = SBN * T::K_SLOTS;           // 16-byte chunks of a key tile
  static constexpr int VCH = SBN * T::V_SLOTS;
  static constexpr int KCOPY = (KCH + 63) / 64;          // wave-wide copies (the last may be partial)
  static constexpr int VCOPY = (VCH + 63) / 64;
  static constexpr int NCOPY = KCOPY + VCOPY;
  static constexpr int PER_WAVE = (NCOPY + SWAVES - 1) / SWAVES;
  static constexpr int Q_BYTES = SBM * D * 2;            // the workgroup's query rows, packed
  static constexpr int QPER_WAVE = SBM * CH / 64 / SWAVES;
  static_assert(D % 32 == 0 && SBM * CH % (64 * SWAVES) == 0, "whole blocks and query copies");
};

struct ShortParams {
  AttnParams a;
  int row_tiles;        // 128-row tiles per sample
  int heads_per_group;
  int total;            // workgroups: row_tiles x B x head groups
};

__device__ __forceinline__ void lds_copy16_s(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}

template <int D, bool GATHER>
__global__ __launch_bounds__(SWAVES * 64, D >= 128 ? 2 : 3) void attn_short_kernel(ShortParams sp) {
  using S = ShortTile<D>;
  using T = Tile<D>;
  constexpr int KS = S::KS, DB = S::DB;
  const AttnParams& p = sp.a;
  __shared__ __attribute__((aligned(1024))) char kst0[S::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char kst1[S::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char vst0[S::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vst1[S::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char qst[S::Q_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // consecutive logical ids (the row tiles of one sample and head group, which share
  // their keys and values) run on one XCD and share its L2
  const int logical = xcd_remap(blockIdx.x, sp.total);
  const int tile = logical % sp.row_tiles;
  const int b = (logical / sp.row_tiles) % p.B;
  const int h_first = (logical / sp.row_tiles / p.B) * sp.heads_per_group;
  const int h_end = min(p.H, h_first + sp.heads_per_group);

  // this lane's output row and its query token
  const int rr = tile * SBM + wave * 32 + col;
  const bool row_ok = rr < p.n_rows;
  int qi = rr;
  if (GATHER) qi = row_ok ? p.q_rows[(int64_t)b * p.qr_bs + rr] : -1;
  const bool q_ok = row_ok && qi >= 0 && qi < p.Nq;

  int nkeys = p.Nk;
  if (p.kv_len != nullptr) {
    const int L = p.kv_len[b];
    nkeys = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  const int ntiles = (nkeys + SBN - 1) / SBN;
  const float sl2 = p.scale_log2;

  // copy plans, fixed per lane: query copy m moves chunk `chunk` of tile row `row` (the
  // token it selects; a row outside the selection copies token 0 and is zeroed when read);
  // key/value copy m moves chunk `chunk` (pad chunks: chunk 0) of key row `row` of a tile
  const char* qbase = reinterpret_cast<const char*>(p.q + (int64_t)b * p.qs0);
  const char* kbase = reinterpret_cast<const char*>(p.k + (int64_t)b * p.ks0);
  const char* vbase = reinterpret_cast<const char*>(p.v + (int64_t)b * p.vs0);
  const int64_t krow_b = p.ks1 * 2, vrow_b = p.vs1 * 2;
  // (32-bit: the host routes calls whose query rows or key tiles span 2 GiB elsewhere)
  uint32_t qoff[S::QPER_WAVE], coff[S::PER_WAVE];
#pragma unroll
  for (int m = 0; m < S::QPER_WAVE; ++m) {
    const int sigma = (wave + SWAVES * m) * 64 + lane;
    const int row = sigma / S::CH;
    const int chunk = sigma - row * S::CH;
    const int r = tile * SBM + row;
    int tok = r < p.n_rows ? r : 0;
    if (GATHER) tok = r < p.n_rows ? p.q_rows[(int64_t)b * p.qr_bs + r] : 0;
    if (tok < 0 || tok >= p.Nq) tok = 0;
    qoff[m] = (uint32_t)tok * (uint32_t)(p.qs1 * 2) + (uint32_t)(chunk * 16);
  }
#pragma unroll
  for (int m = 0; m < S::PER_WAVE; ++m) {
    const int c = wave + SWAVES * m;
    const bool isk = c < S::KCOPY;
    const int slots = isk ? T::K_SLOTS : T::V_SLOTS;
    const int sigma = (isk ? c : c - S::KCOPY) * 64 + lane;
    const int row = sigma / slots;
    int chunk = sigma - row * slots;
    if (chunk >= S::CH) chunk = 0;
    coff[m] = (uint32_t)(row * (isk ? krow_b : vrow_b) + chunk * 16);
  }
  auto issue_q = [&](int h) {
    const char* qb = qbase + (int64_t)h * p.qs2 * 2;
#pragma unroll
    for (int m = 0; m < S::QPER_WAVE; ++m) lds_copy16_s(qb + qoff[m], qst + (wave + SWAVES * m) * 1024);
  };
  // keys and values [j0, j0 + 32) of head h; on a partial tile rows past the length fetch
  // the tile's row 0 (their scores are masked)
  auto issue = [&](int h, int j0, char* kst, char* vst) {
    const char* kb = kbase + (int64_t)h * p.ks2 * 2 + (int64_t)j0 * krow_b;
    const char* vb = vbase + (int64_t)h * p.vs2 * 2 + (int64_t)j0 * vrow_b;
    const int nvalid = nkeys - j0;
    // the lane index laundered for the partial-tile rows, so that they are not hoisted out
    // of the step loop into registers live across it
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int m = 0; m < S::PER_WAVE; ++m) {
      const int c = wave + SWAVES * m;   // wave-uniform
      if (c >= S::NCOPY) continue;
      const bool isk = c < S::KCOPY;
      const int cc = isk ? c : c - S::KCOPY;
      const int nch = isk ? S::KCH : S::VCH;
      if (cc * 64 + lane >= nch) continue;   // past the tile's last chunk
      char* dst = (isk ? kst : vst) + cc * 1024;
      if (nvalid >= SBN) {
        lds_copy16_s((isk ? kb : vb) + coff[m], dst);
      } else {
        const int slots = isk ? T::K_SLOTS : T::V_SLOTS;
        const int row = (cc * 64 + ln) / slots;
        const int64_t rowb = isk ? krow_b : vrow_b;
        lds_copy16_s((isk ? kb : vb) + (coff[m] - (row < nvalid ? 0u : (uint32_t)(row * rowb))), dst);
      }
    }
  };

  // LDS addresses of this lane's operand reads
  const int k_lane = col * T::K_ROWB + half * 16;
  const int grp = (lane >> 4) & 3, src = lane & 15;
  const int v_lane = (4 * (grp >> 1) + (src >> 2)) * T::V_ROWB + (16 * (grp & 1) + 4 * (src & 3)) * 2;
  const char* q_lane = qst + (wave * 32 + col) * (D * 2) + half * 16;

  // the output of head h for this lane's row (o unnormalised, l its row sum share)
  auto store_head = [&](int h, const f32x16 (&o)[DB], float l_run, float m_ref) {
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
          w[0] = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
          w[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
          st8(op + db * 32 + 8 * g + 4 * half, w);
        }
    }
    if (p.lse != nullptr && half == 0) {
      const float lse = l_tot > 0.f ? (m_ref + __builtin_log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
      p.lse[((int64_t)b * p.H + h) * p.n_rows + rr] = lse;
    }
  };

  if (ntiles == 0) {   // no valid key: zero rows and LSE -inf for every head of the group
    f32x16 zero[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) zero[db] = f32x16{};
    for (int h = h_first; h < h_end; ++h) store_head(h, zero, 0.f, -FLT_MAX);
    return;
  }
  if (h_first >= h_end) return;

  int h = h_first, t = 0;
  issue_q(h);
  issue(h, 0, kst0, vst0);
  bf16x8 qc[KS];
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_ref = -FLT_MAX, l_run = 0.f;

  auto step = [&](const char* kcur, const char* vcur, char* knext, char* vnext) -> bool {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies (and stores) done
    __syncthreads();                      // ... everyone's, and the other stage is free
    const int j0 = t * SBN;
    const bool last = t + 1 == ntiles;
    const bool next_head = last && h + 1 < h_end;
    if (t == 0) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 v = ld16(q_lane + s * 32);
        if (!q_ok) v = u32x4{0u, 0u, 0u, 0u};
        qc[s] = as_bf16x8(v);
      }
      // a one-tile head refills qst in this same step: every wave has read it first
      if (next_head) __syncthreads();
    }
    if (!last) {
      issue(h, j0 + SBN, knext, vnext);
    } else if (next_head) {
      issue(h + 1, 0, knext, vnext);
      issue_q(h + 1);
    }

    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kf = as_bf16x8(ld16(kcur + k_lane + s * 32));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qc[s], sc, 0, 0, 0);
    }
    if (j0 + SBN > nkeys) {   // keys past the length get -inf
      const int lim = nkeys - j0 - 4 * half;   // valid: 8 (r / 4) + r % 4 < lim
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
    }
    bf16x8 pb[2];
    float ts;
    auto probs = [&]() {
      ts = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 packed;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * tt + 2 * e], sl2, -m_ref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * tt + 2 * e + 1], sl2, -m_ref));
          packed[e] = pack_bf16x2(p0, p1);
          ts += p0 + p1;
        }
        pb[tt] = as_bf16x8(packed);
      }
    };
    // the row's max over both lanes holding it: finite, since key j0 < nkeys is valid
    auto block_max = [&]() {
      float mt = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
      return fmaxf(mt, __shfl_xor(mt, 32)) * sl2;
    };
    // a head's first block (wave-uniform; O and l are 0): the reference is its max, so the
    // trial pass against the empty reference is skipped
    if (t == 0) m_ref = block_max();
    probs();
    if (__any(!(ts <= kShortSumLimit))) {   // wave-uniform and rare: scores rose past the reference
      const float mt = block_max();
      const float m_new = mt > m_ref + kShortMoveMargin ? mt : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_ref = m_new;
      probs();
    }
    l_run += ts;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const char* vp = vcur + v_lane + tt * 16 * T::V_ROWB + db * 64;
        const i16x4 lo = lds_read_tr(vp);
        const i16x4 hi = lds_read_tr(vp + 8 * T::V_ROWB);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[tt], oacc[db], 0, 0, 0);
      }
    if (last) {
      store_head(h, oacc, l_run, m_ref);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
      m_ref = -FLT_MAX;
      l_run = 0.f;
      ++h;
      t = 0;
    } else {
      ++t;
    }
    return !last || h < h_end;
  };
  for (;;) {
    if (!step(kst0, vst0, kst1, vst1)) break;
    if (!step(kst1, vst1, kst0, vst0)) break;
  }
}

template <int D, bool GATHER>
hipError_t short_launch(const ShortParams& sp, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_short_kernel<D, GATHER>), grid, dim3(SWAVES * 64), 0, s, sp);
  return hipGetLastError();
}

template <int D, bool GATHER>
int short_resident() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_short_kernel<D, GATHER>, SWAVES * 64, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 0;
  v = cus * per_cu;
  cached.store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

// The short-key path applies to mask-free calls with per-sample key lengths (no fused
// K/V map) whose key axis is at most kShortMaxKeys, at head dims that are multiples of 32.
constexpr int kShortMaxKeys = 1024;
bool attn_short_applies(const safe_attn_args* a) {
  const int64_t two_gib = int64_t(1) << 31;
  return a->kv_len != nullptr && a->mask == nullptr && a->kv_src == nullptr && a->Nk <= kShortMaxKeys &&
         (a->d == 64 || a->d == 96 || a->d == 128) && (int64_t)a->Nq * a->q_stride[1] * 2 < two_gib &&
         (int64_t)SBN * a->k_stride[1] * 2 < two_gib && (int64_t)SBN * a->v_stride[1] * 2 < two_gib;
}

// Heads per workgroup: several heads per workgroup (the next head's query rows then load
// while the current head computes) only where that still leaves about two full rounds of
// the resident workgroups.  Samples usually differ in key length (the conditional and the
// unconditional prompt of a guidance pair), so a workgroup's time differs by sample and
// more, shorter workgroups balance the CUs: at the 160x160 workload with key lengths
// (195, 32) one head per workgroup takes 43 us against 52 us with two; with equal
// lengths (195, 195) it costs 59 against 56 us.
hipError_t attn_short_launch(const AttnParams& p, int d, hipStream_t s) {
  ShortParams sp;
  sp.a = p;
  sp.row_tiles = (p.n_rows + SBM - 1) / SBM;
  const bool gather = p.q_rows != nullptr;
  int resident = 0;
  switch (d) {
    case 64: resident = gather ? short_resident<64, true>() : short_resident<64, false>(); break;
    case 96: resident = gather ? short_resident<96, true>() : short_resident<96, false>(); break;
    case 128: resident = gather ? short_resident<128, true>() : short_resident<128, false>(); break;
    default: return hipErrorInvalidValue;
  }
  const int64_t items = (int64_t)sp.row_tiles * p.B;
  int hpg = 1;
  if (resident > 0 && items > 0) {
    while (hpg < p.H && items * ((p.H + 2 * hpg - 1) / (2 * hpg)) >= 2 * (int64_t)resident) hpg *= 2;
  }
  hpg = std::min(hpg, std::max(p.H, 1));
  sp.heads_per_group = hpg;
  const int64_t total = items * ((p.H + hpg - 1) / hpg);
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  sp.total = (int)total;
  const dim3 grid((unsigned)total);
  switch (d) {
    case 64: return gather ? short_launch<64, true>(sp, grid, s) : short_launch<64, false>(sp, grid, s);
    case 96: return gather ? short_launch<96, true>(sp, grid, s) : short_launch<96, false>(sp, grid, s);
    case 128: return gather ? short_launch<128, true>(sp, grid, s) : short_launch<128, false>(sp, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace safe
