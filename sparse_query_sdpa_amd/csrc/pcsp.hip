// Prompt-Conditioned Sensitivity Partitioning ("SAFE-DiT" Eq. 9-12).
//
// ACCUM (Eq. 9-10): acc[b,i] += sum_{h in head set} sum_{j<L_b} w[b,j] softmax_j(scale q_i.k_j).
//   A workgroup owns 128 image tokens of one sample (4 waves x 32) and one group of
//   heads: with a workspace the heads are split into groups so the grid holds a few
//   thousand workgroups, each group's per-token sum goes to its own slice of the
//   workspace, and pcsp_reduce_kernel adds the slices to acc in group order (the
//   result does not depend on scheduling); without one, one group holds every head
//   and the sum is added to acc directly.  The workgroup walks its (head, key tile)
//   steps as one software pipeline: a tile's 64 text keys and weights are copied
//   straight into LDS (two stages) one step ahead, and the next head's 128 query rows
//   are copied into an LDS buffer during the last step of the head before (and read
//   into registers at the head's first step), so each step waits only for copies
//   issued one step earlier.  S^T = K_txt Q^T
//   runs on v_mfma_f32_32x32x16_bf16 exactly as in the attention kernel (each lane
//   owns one image token), and instead of a P V product each lane keeps an online
//   softmax numerator sum_j w_j p_j and denominator sum_j p_j.  The probabilities are
//   never stored: only the N-vector acc is kept, as the paper's instrumentation does.
// SELECT (Eq. 11-12): the separable Gaussian (rows, then columns, one thread per
//   token, in-grid taps renormalised) runs as two grid-wide kernels; then one
//   workgroup per sample (1024 threads, the sample's keys held in LDS when they fit)
//   does the min-max normalisation for the optional score output and an exact top-k:
//   order-preserving 32-bit keys (-0 folded to +0, NaN lowest), a 4 x 8-bit radix
//   select of the k-th key, and an ordered compaction that keeps every key above
//   it plus the lowest-index ties, so the result is a deterministic ascending list.
#include <limits.h>

#include <algorithm>

#include "common.h"

namespace safe {
namespace {

// ============================== ACCUM ========================================
constexpr int ABM = 128;   // image tokens per workgroup
constexpr int ABN = 32;    // text keys per tile (one 32 x 32 score block per wave)
constexpr int ANT = 256;
constexpr int AWAVES = ANT / 64;
constexpr float kAccSumLimit = 65536.f;   // a 32-key block's per-lane sum of probabilities kept below this
constexpr float kAccMoveMargin = 8.f;     // the reference moves to a max more than 2^8 above it

typedef __attribute__((address_space(3))) void lds_void;

// One direct-to-LDS copy per lane of 16 (4) bytes from src; lds_dst is the wave's LDS base,
// the lane's bytes land at lds_dst + 16 (4) * lane.
__device__ __forceinline__ void lds_copy16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 4, 0, 0);
}

// LDS layout of a key tile: ABN rows of SLOTS 16-byte chunks (an odd count, so the 16
// lanes of a fragment read hit distinct banks); the copies fill it in order, one
// wave-wide 1 KB copy per 64 chunks (lanes past the tile's last chunk idle), and pad
// chunks fetch chunk 0 of their row.
template <int D>
struct AccTile {
  static constexpr int CH = D / 8;        // 16-byte chunks of a key row
  static constexpr int KS = D / 16;       // k-steps of the S^T product
  static constexpr int SLOTS = CH | 1;
  static constexpr int ROWB = SLOTS * 16;
  static constexpr int BYTES = ABN * ROWB;
  static constexpr int NCHUNK = ABN * SLOTS;              // 16-byte chunks of a tile
  static constexpr int NCOPY = (NCHUNK + 63) / 64;          // wave-wide copies (the last may be partial)
  static constexpr int PER_WAVE = (NCOPY + AWAVES - 1) / AWAVES;
  static constexpr int QBYTES = ABM * D * 2;            // the workgroup's query rows, packed
  static constexpr int QPER_WAVE = ABM * CH / 64 / AWAVES;
  static_assert(D % 16 == 0 && ABM * CH % (64 * AWAVES) == 0, "whole k-steps and query copies");
};

struct AccParams {
  const u16* q; int64_t qs0, qs1, qs2;
  const u16* kt; int64_t ks0, ks1, ks2;
  const int32_t* kv_len;
  const float* w;
  float* acc;
  float* part;        // [groups][B][N] per-group sums, or nullptr: add into acc
  uint64_t head_mask;
  int B, N, M, H, tiles_per_b, heads_per_group;
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(ANT, D >= 128 ? 3 : 4) void pcsp_accum_kernel(AccParams p) {
  using T = AccTile<D>;
  constexpr int KS = T::KS;
  // two stages as separate objects, so a read of one is not held for a copy into the other
  __shared__ __attribute__((aligned(1024))) char kst0[T::BYTES];
  __shared__ __attribute__((aligned(1024))) char kst1[T::BYTES];
  __shared__ __attribute__((aligned(256))) float wst0[ABN];
  __shared__ __attribute__((aligned(256))) float wst1[ABN];
  __shared__ __attribute__((aligned(1024))) char qst[T::QBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int b = blockIdx.x / p.tiles_per_b;
  const int tile = blockIdx.x % p.tiles_per_b;
  const int i = tile * ABM + wave * 32 + col;
  const bool ok = i < p.N;

  int L = p.kv_len ? p.kv_len[b] : p.M;
  L = L < 0 ? 0 : (L > p.M ? p.M : L);
  const int ntiles = (L + ABN - 1) / ABN;
  const float sl2 = p.scale_log2;
  const int g = blockIdx.y;
  const int h_first = g * p.heads_per_group;
  const int h_end = min(p.H, h_first + p.heads_per_group);
  auto next_head = [&](int h) {   // the next head of the set in this group, or h_end
    for (++h; h < h_end; ++h)
      if (p.head_mask == 0 || ((p.head_mask >> h) & 1ull)) break;
    return h;
  };

  // Copy plans, fixed per lane: query copy m moves chunk `chunk` of row `row` of the
  // workgroup's token tile (a token past N copies the tile's first token: finite scores,
  // never written out); key copy m moves chunk `chunk` (pad chunks: chunk 0) of key row
  // `row` of a tile.  The byte offsets stay in registers for the whole loop.
  const char* qbase = reinterpret_cast<const char*>(p.q + (int64_t)b * p.qs0 + (int64_t)tile * ABM * p.qs1);
  const char* kbase = reinterpret_cast<const char*>(p.kt + (int64_t)b * p.ks0);
  const int64_t krow_b = p.ks1 * 2;
  const float* wrow = p.w + (int64_t)b * p.M;
  int64_t qoff[T::QPER_WAVE], koff[T::PER_WAVE];
#pragma unroll
  for (int m = 0; m < T::QPER_WAVE; ++m) {
    const int sigma = (wave + AWAVES * m) * 64 + lane;
    const int row = sigma / T::CH;
    const int chunk = sigma - row * T::CH;
    qoff[m] = (int64_t)(tile * ABM + row < p.N ? row : 0) * p.qs1 * 2 + chunk * 16;
  }
#pragma unroll
  for (int m = 0; m < T::PER_WAVE; ++m) {
    const int sigma = (wave + AWAVES * m) * 64 + lane;
    const int row = sigma / T::SLOTS;
    int chunk = sigma - row * T::SLOTS;
    if (chunk >= T::CH) chunk = 0;
    koff[m] = (int64_t)row * krow_b + chunk * 16;
  }
  auto issue_q = [&](int h) {   // head h's query rows -> qst (row r = token tile * 128 + r)
    const char* qb = qbase + (int64_t)h * p.qs2 * 2;
#pragma unroll
    for (int m = 0; m < T::QPER_WAVE; ++m) {
      lds_copy16(qb + qoff[m], qst + (wave + AWAVES * m) * 1024);
    }
  };
  // keys and weights of step (h, j0); on a partial tile, key rows past L fetch the tile's
  // row 0 and weights past L weight 0 of the tile (their scores are masked); the weights
  // are dwords (w rows need not be aligned), copied by the last wave
  auto issue = [&](int h, int j0, char* kst, float* wst) {
    const char* kb = kbase + (int64_t)h * p.ks2 * 2 + (int64_t)j0 * krow_b;
    const int nvalid = L - j0;
    if (nvalid >= ABN) {
#pragma unroll
      for (int m = 0; m < T::PER_WAVE; ++m) {
        const int c = wave + AWAVES * m;
        if (c < T::NCOPY && (T::NCHUNK % 64 == 0 || c * 64 + lane < T::NCHUNK))   // c: wave-uniform
          lds_copy16(kb + koff[m], kst + c * 1024);
      }
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int m = 0; m < T::PER_WAVE; ++m) {
        const int c = wave + AWAVES * m;
        if (c < T::NCOPY && (T::NCHUNK % 64 == 0 || c * 64 + ln < T::NCHUNK)) {
          const int sigma = c * 64 + ln;
          const int row = sigma / T::SLOTS;
          int chunk = sigma - row * T::SLOTS;
          if (chunk >= T::CH) chunk = 0;
          lds_copy16(kb + (int64_t)(row < nvalid ? row : 0) * krow_b + chunk * 16, kst + c * 1024);
        }
      }
    }
    if (wave == AWAVES - 1 && lane < ABN) {
      const int r = lane < nvalid ? lane : 0;
      lds_copy4(wrow + j0 + r, wst);
    }
  };

  float total = 0.f;
  int h = next_head(h_first - 1);
  if (ntiles > 0 && h < h_end) {
    bf16x8 qc[KS];   // this lane's query row of the current head
    issue_q(h);
    issue(h, 0, kst0, wst0);
    int hn = next_head(h), t = 0;
    // online softmax of the current head against a lazy reference m (log2 domain): the
    // max of the head's first block, then probabilities are taken as exp2(s - m) and the
    // reference moves only when a 32-key block's sum leaves [0, kAccSumLimit] (scores more
    // than kAccMoveMargin above m); num and den are rescaled with it
    float m = -INFINITY, num = 0.f, den = 0.f;
    const int k_lane = col * T::ROWB + half * 16;
    const char* q_lane = qst + (wave * 32 + col) * (D * 2) + half * 16;

    // One step: wait for what the step before issued (this step's keys and weights,
    // and at a head's first step its query rows), start the next step's copies into the
    // other stage (and, at a head's last step, the next head's query rows), then scores,
    // online softmax and the weighted sums.
    auto step = [&](const char* kcur, const float* wcur, char* knext, float* wnext) -> bool {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
      __syncthreads();                      // ... everyone's, and the other stage is free
      const int j0 = t * ABN;
      const bool last = t + 1 == ntiles;
      if (t == 0) {
#pragma unroll
        for (int s = 0; s < KS; ++s) qc[s] = as_bf16x8(ld16(q_lane + s * 32));
        // a one-tile head refills qst in this same step: every wave has read it first
        if (last && hn < h_end) __syncthreads();
      }
      const bool more = !last || hn < h_end;
      if (!last) {
        issue(h, j0 + ABN, knext, wnext);
      } else if (hn < h_end) {
        issue(hn, 0, knext, wnext);
        issue_q(hn);
      }

      // the tile's 32-key blocks in turn; a block wholly past L is skipped (the first
      // always holds key j0 < L)
#pragma unroll
      for (int blk = 0; blk < ABN / 32; ++blk) {
        const int kh = j0 + blk * 32;   // first key of the block
        if (blk > 0 && kh >= L) break;
        f32x16 sc = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kf = as_bf16x8(ld16(kcur + k_lane + blk * 32 * T::ROWB + s * 32));
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qc[s], sc, 0, 0, 0);
        }
        if (kh + 32 > L) {   // keys past L get -inf
          const int lim = L - kh - 4 * half;   // valid: 8 (r / 4) + r % 4 < lim
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
        }
        float ts, tn;   // this lane's share of the block's sum of p and of w p
        auto probs = [&]() {
          ts = 0.f;
          tn = 0.f;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 wv = *reinterpret_cast<const f32x4*>(wcur + blk * 32 + 8 * r4 + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * r4 + e], sl2, -m));
              ts += pr;
              tn = __builtin_fmaf(pr, wv[e], tn);
            }
          }
        };
        // the token's max over both lanes holding it: finite, since key kh < L is valid
        auto block_max = [&]() {
          float mt = sc[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
          return fmaxf(mt, __shfl_xor(mt, 32)) * sl2;
        };
        // a head's first block (wave-uniform; num and den are 0): the reference is its max,
        // so the trial pass against the empty reference is skipped
        if (t == 0 && blk == 0) m = block_max();
        probs();
        if (__any(!(ts <= kAccSumLimit))) {   // wave-uniform and rare: scores rose past the reference
          const float mt = block_max();
          const float m_new = mt > m + kAccMoveMargin ? mt : m;
          const float alpha = __builtin_amdgcn_exp2f(m - m_new);
          num *= alpha;
          den *= alpha;
          m = m_new;
          probs();
        }
        den += ts;
        num += tn;
      }
      if (last) {   // the head's last tile: its share of the sum over heads
        const float num_t = num + __shfl_xor(num, 32);
        const float den_t = den + __shfl_xor(den, 32);
        if (den_t > 0.f) total += num_t / den_t;
        m = -INFINITY;
        num = 0.f;
        den = 0.f;
        h = hn;
        hn = next_head(hn);
        t = 0;
      } else {
        ++t;
      }
      return more;
    };
    for (;;) {
      if (!step(kst0, wst0, kst1, wst1)) break;
      if (!step(kst1, wst1, kst0, wst0)) break;
    }
  }
  if (p.part != nullptr) {
    if (ok && half == 0) p.part[((int64_t)g * p.B + b) * p.N + i] = total;
  } else if (ok && half == 0 && L > 0) {
    p.acc[(int64_t)b * p.N + i] += total;
  }
}

// acc[x] += sum over head groups of part[g][x], in group order
__global__ __launch_bounds__(256) void pcsp_reduce_kernel(const float* part, float* acc, int64_t n, int groups) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  float s = 0.f;
  for (int g = 0; g < groups; ++g) s += part[(int64_t)g * n + x];
  acc[x] += s;
}

// Head groups for the accumulation: enough workgroups (about 4800) to fill the GPU several
// times, which also evens out samples whose text lengths differ (2400 ran 3-7% slower at the
// 160x160 workload, 9600 as fast as 2400).
struct AccPlan {
  int groups = 1, heads_per_group = 0;
};
AccPlan plan_accum(const safe_pcsp_args* a) {
  AccPlan pl;
  pl.heads_per_group = a->H;
  const int64_t items = (int64_t)a->B * ((a->N + ABM - 1) / ABM);
  if (items <= 0 || a->H <= 1) return pl;
  const int64_t want = (4800 + items - 1) / items;
  if (want <= 1) return pl;
  const int g = (int)std::min<int64_t>(want, a->H);
  pl.heads_per_group = (a->H + g - 1) / g;
  pl.groups = (a->H + pl.heads_per_group - 1) / pl.heads_per_group;
  return pl;
}

// ============================== SELECT =======================================
constexpr int SNT = 1024;
constexpr int SUNR = 8;    // field elements per thread loaded together
constexpr int MAX_TAPS = 2 * 96 + 1;  // sigma <= 32 -> radius <= 96

struct SelParams {
  const float* acc;
  float* score_out;
  int32_t* idx_out;
  float* ws;           // smoothed field: sample b at ws + b * ws_bs
  int64_t ws_bs;
  int N, gh, gw, k, radius;
  float sigma;
};

__device__ __forceinline__ u32 order_key(float f) {
  u32 u = __builtin_bit_cast(u32, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;      // NaN: lowest
  if (u == 0x80000000u) u = 0u;                          // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block (1024 threads); returns the block total in *total.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < SNT; off <<= 1) {
    const int add = t >= off ? sh[t - off] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  const int incl = sh[t];
  *total = sh[SNT - 1];
  __syncthreads();
  return incl - v;
}

// ---- Eq. 11: separable Gaussian, renormalised at the borders ------------------
// One thread per token; rows then columns.  Taps exp(-t^2 / (2 sigma^2)) in LDS.
__device__ __forceinline__ void load_taps(float* taps, int R, float sigma) {
  const float inv2s2 = 1.0f / (2.0f * sigma * sigma);
  for (int i = threadIdx.x; i <= 2 * R; i += blockDim.x) {
    const float d = (float)(i - R);
    taps[i] = expf(-d * d * inv2s2);
  }
  __syncthreads();
}

template <bool ROWS>
__global__ __launch_bounds__(256) void pcsp_smooth_kernel(const float* in, float* out, int N, int gh, int gw,
                                                         int R, float sigma, int64_t in_bs, int64_t out_bs) {
  __shared__ float taps[MAX_TAPS];
  load_taps(taps, R, sigma);
  const int b = blockIdx.y;
  const int pos = blockIdx.x * 256 + threadIdx.x;
  if (pos >= N) return;
  const float* src = in + (int64_t)b * in_bs;
  const int y = pos / gw, x = pos % gw;
  float num = 0.f, den = 0.f;
  if (ROWS) {
    const int lo = max(-R, -x), hi = min(R, gw - 1 - x);
    for (int d = lo; d <= hi; ++d) {
      num = __builtin_fmaf(taps[d + R], src[y * gw + x + d], num);
      den += taps[d + R];
    }
  } else {
    const int lo = max(-R, -y), hi = min(R, gh - 1 - y);
    for (int d = lo; d <= hi; ++d) {
      num = __builtin_fmaf(taps[d + R], src[(y + d) * gw + x], num);
      den += taps[d + R];
    }
  }
  out[(int64_t)b * out_bs + pos] = num / den;
}

// ---- Norm and Eq. 12: one workgroup per sample --------------------------------
// KEYS_IN_LDS: the N order keys are loaded into LDS once (N <= kKeyCap: grids up to
// 192 x 192, 144 KB of the workgroup's LDS) and every radix pass and the compaction read
// them there; otherwise they are recomputed from the field in global memory.  Histograms aggregate equal bins within a wave first
// (the leading passes see few distinct bins), and the bin holding the k-th key is
// found by a suffix scan over the 256 counts on the first wave.
constexpr int kKeyCap = 36864;

__device__ __forceinline__ void hist_add(int* hist, u32 bin, bool act) {
  const int lane = threadIdx.x & 63;
  uint64_t pending = __ballot(act);
  for (int round = 0; round < 4 && pending != 0; ++round) {
    const int leader = __builtin_ctzll(pending);
    const u32 lb = __builtin_amdgcn_readlane(bin, leader);
    const uint64_t same = __ballot(act && bin == lb);
    const int n = __builtin_popcountll(same);
    if (lane == leader) atomicAdd(&hist[lb], n);
    if (act && bin == lb) act = false;
    pending &= ~same;
    if (n < 8) break;   // bins are spread: plain atomics for the rest
  }
  if (act) atomicAdd(&hist[bin], 1);
}

template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(SNT) void pcsp_select_kernel(SelParams p) {
  __shared__ u32 kbuf[KEYS_IN_LDS ? kKeyCap : 1];
  __shared__ int hist[256];
  __shared__ int scan_buf[SNT];
  __shared__ float red_min[SNT / 64], red_max[SNT / 64];
  __shared__ u32 red_kmin[SNT / 64], red_kmax[SNT / 64];
  __shared__ u32 sh_prefix;
  __shared__ int sh_krem;

  const int t = threadIdx.x, lane = t & 63;
  const int b = blockIdx.x;
  const int N = p.N;
  const float* src = (p.sigma > 0.f ? p.ws : p.acc) + (int64_t)b * (p.sigma > 0.f ? p.ws_bs : N);
  auto key_at = [&](int pos) -> u32 {
    if constexpr (KEYS_IN_LDS) return kbuf[pos];
    else return order_key(src[pos]);
  };

  // the field is read SUNR elements per thread at a time, all loads issued before the
  // first is used (a load per iteration would pay the full memory latency N / SNT times)
  float lo = INFINITY, hi = -INFINITY;
  u32 kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int base = t; base < N; base += SNT * SUNR) {
    float v[SUNR];
#pragma unroll
    for (int u = 0; u < SUNR; ++u) {
      const int pos = base + u * SNT;
      v[u] = pos < N ? src[pos] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < SUNR; ++u) {
      const int pos = base + u * SNT;
      if (pos < N) {
        const u32 key = order_key(v[u]);
        if constexpr (KEYS_IN_LDS) kbuf[pos] = key;
        lo = fminf(lo, v[u]);
        hi = fmaxf(hi, v[u]);
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (u32)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (u32)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) { red_kmin[t >> 6] = kmin; red_kmax[t >> 6] = kmax; }
  // ---- Norm: min-max scaling (optional output) --------------------------------
  if (p.score_out != nullptr) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, off));
      hi = fmaxf(hi, __shfl_xor(hi, off));
    }
    if (lane == 0) { red_min[t >> 6] = lo; red_max[t >> 6] = hi; }
    __syncthreads();
    lo = red_min[0]; hi = red_max[0];
    for (int w = 1; w < SNT / 64; ++w) { lo = fminf(lo, red_min[w]); hi = fmaxf(hi, red_max[w]); }
    const float span = hi - lo;
    float* so = p.score_out + (int64_t)b * N;
    for (int base = t; base < N; base += SNT * SUNR) {
      float v[SUNR];
#pragma unroll
      for (int u = 0; u < SUNR; ++u) {
        const int pos = base + u * SNT;
        v[u] = pos < N ? src[pos] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < SUNR; ++u) {
        const int pos = base + u * SNT;
        if (pos < N) so[pos] = span > 0.f ? (v[u] - lo) / span : 0.f;
      }
    }
  }

  // ---- Eq. 12: exact top-k ------------------------------------------------------
  const int k = p.k;
  if (k == 0) return;
  int32_t* out = p.idx_out + (int64_t)b * k;
  // radix select of the k-th largest key, 8-bit digits below the bits that every key
  // shares (those of the smallest and largest key agree on them)
  __syncthreads();
  kmin = red_kmin[0]; kmax = red_kmax[0];
  for (int w = 1; w < SNT / 64; ++w) { kmin = min(kmin, red_kmin[w]); kmax = max(kmax, red_kmax[w]); }
  const int free_bits = kmin == kmax ? 0 : 32 - __builtin_clz(kmin ^ kmax);
  if (t == 0) {
    sh_prefix = free_bits == 32 ? 0u : (kmax & ~((1u << free_bits) - 1u));
    sh_krem = k;
  }
  __syncthreads();   // also when no pass runs (all keys equal)
  for (int top = free_bits; top > 0; top -= 8) {
    const int shift = top > 8 ? top - 8 : 0;
    const u32 digit_mask = (1u << (top - shift)) - 1u;
    if (t < 256) hist[t] = 0;
    __syncthreads();
    const u32 prefix = sh_prefix;
    const u32 hmask = top == 32 ? 0u : (0xFFFFFFFFu << top);
    for (int base = 0; base < N; base += SNT) {   // every lane of a wave runs each step
      const int pos = base + t;
      u32 key = 0u;
      if (pos < N) key = key_at(pos);
      hist_add(hist, (key >> shift) & digit_mask, pos < N && (key & hmask) == prefix);
    }
    __syncthreads();
    if (t < 64) {
      // suffix counts over the 256 bins (lane l owns bins 4l..4l+3), then the bin where
      // the k-th largest key falls: suffix(bin) >= rem > suffix(bin + 1)
      const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
      int suf = c0 + c1 + c2 + c3;   // becomes the sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
      }
      const int above = suf - (c0 + c1 + c2 + c3);   // keys in bins above this lane's four
      const int rem = sh_krem;
      // lane holding the bin: above < rem <= above + its four counts
      int bin = -1, left = 0;
      if (above < rem && rem <= suf) {
        int acc3 = above + c3;
        if (rem <= acc3) { bin = 4 * lane + 3; left = rem - above; }
        else {
          int acc2 = acc3 + c2;
          if (rem <= acc2) { bin = 4 * lane + 2; left = rem - acc3; }
          else {
            int acc1 = acc2 + c1;
            if (rem <= acc1) { bin = 4 * lane + 1; left = rem - acc2; }
            else { bin = 4 * lane; left = rem - acc1; }
          }
        }
      }
      const uint64_t has = __ballot(bin >= 0);
      if (has == 0) {
        if (lane == 0) sh_prefix = prefix;   // fewer than rem keys left (cannot happen for k <= N)
      } else if (lane == __builtin_ctzll(has)) {
        sh_prefix = prefix | ((u32)bin << shift);
        sh_krem = left;  // how many to take from within this bin (and deeper)
      }
    }
    __syncthreads();
  }
  const u32 T = sh_prefix;
  const int need_eq = sh_krem;  // keys equal to T to keep (lowest indices first)

  // ordered compaction: each thread owns a contiguous segment
  const int seg = (N + SNT - 1) / SNT;
  const int beg = min(N, t * seg), end = min(N, beg + seg);
  int n_eq = 0, n_gt = 0;
  for (int pos = beg; pos < end; ++pos) {
    const u32 key = key_at(pos);
    n_eq += key == T;
    n_gt += key > T;
  }
  int tot;
  const int eq_base = block_exclusive_scan(n_eq, scan_buf, &tot);
  const int eq_take = max(0, min(n_eq, need_eq - eq_base));
  const int sel_base = block_exclusive_scan(n_gt + eq_take, scan_buf, &tot);
  {
    int r = eq_base, o = sel_base;
    for (int pos = beg; pos < end; ++pos) {
      const u32 key = key_at(pos);
      bool take = false;
      if (key > T) take = true;
      else if (key == T) { take = r < need_eq; ++r; }
      if (take && o < k) out[o++] = pos;
    }
  }
}

}  // namespace

size_t pcsp_select_workspace(const safe_pcsp_args* a) {
  if (!(a->flags & SAFE_PCSP_SELECT)) return 0;
  const size_t n = (size_t)(a->B > 0 ? a->B : 0) * 2 * (size_t)(a->N > 0 ? a->N : 0) * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

size_t pcsp_accum_workspace(const safe_pcsp_args* a) {
  if (!(a->flags & SAFE_PCSP_ACCUM) || a->B <= 0 || a->N <= 0) return 0;
  const AccPlan pl = plan_accum(a);
  if (pl.groups <= 1) return 0;
  const size_t n = (size_t)pl.groups * (size_t)a->B * (size_t)a->N * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

// ws_bytes: usable workspace bytes (0 when unknown); the accumulation is split only
// when its partial sums fit.
int pcsp_launch(const safe_pcsp_args* a, float scale, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (a->flags & SAFE_PCSP_ACCUM) {
    if ((int64_t)a->B * a->N * a->H > 0 && a->M > 0) {
      AccParams p;
      p.q = static_cast<const u16*>(a->q);
      p.qs0 = a->q_stride[0]; p.qs1 = a->q_stride[1]; p.qs2 = a->q_stride[2];
      p.kt = static_cast<const u16*>(a->k_text);
      p.ks0 = a->k_stride[0]; p.ks1 = a->k_stride[1]; p.ks2 = a->k_stride[2];
      p.kv_len = a->kv_len;
      p.w = a->w;
      p.acc = a->acc;
      p.head_mask = a->head_mask;
      p.B = a->B; p.N = a->N; p.M = a->M; p.H = a->H;
      p.tiles_per_b = (a->N + ABM - 1) / ABM;
      p.scale_log2 = scale * 1.4426950408889634f;
      AccPlan pl = plan_accum(a);
      const size_t need = pcsp_accum_workspace(a);
      if (pl.groups > 1 && (workspace == nullptr || need == 0 || ws_bytes < need)) pl = AccPlan{1, a->H};
      p.heads_per_group = pl.heads_per_group;
      p.part = pl.groups > 1 ? static_cast<float*>(workspace) : nullptr;
      const int64_t grid = (int64_t)p.tiles_per_b * a->B;
      if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
      const dim3 g3((unsigned)grid, (unsigned)pl.groups);
      switch (a->d) {
        case 32: hipLaunchKernelGGL(pcsp_accum_kernel<32>, g3, dim3(ANT), 0, s, p); break;
        case 64: hipLaunchKernelGGL(pcsp_accum_kernel<64>, g3, dim3(ANT), 0, s, p); break;
        case 96: hipLaunchKernelGGL(pcsp_accum_kernel<96>, g3, dim3(ANT), 0, s, p); break;
        case 128: hipLaunchKernelGGL(pcsp_accum_kernel<128>, g3, dim3(ANT), 0, s, p); break;
        default: return SAFE_ERR_UNSUPPORTED;
      }
      if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
      if (pl.groups > 1) {
        const int64_t n = (int64_t)a->B * a->N;
        hipLaunchKernelGGL(pcsp_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           (const float*)p.part, a->acc, n, pl.groups);
        if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
      }
    }
  }
  if (a->flags & SAFE_PCSP_SELECT) {
    if (a->B > 0 && a->N > 0) {
      SelParams p;
      p.acc = a->acc;
      p.score_out = a->score_out;
      p.idx_out = a->idx_out;
      p.ws = nullptr;
      p.ws_bs = a->N;
      p.N = a->N; p.gh = a->grid_h; p.gw = a->grid_w; p.k = a->k;
      p.sigma = a->sigma;
      p.radius = a->sigma > 0.f ? (int)ceilf(3.0f * a->sigma) : 0;
      if (p.radius > (MAX_TAPS - 1) / 2) return SAFE_ERR_RANGE;
      if (a->sigma > 0.f) {
        if (workspace == nullptr) return SAFE_ERR_WORKSPACE;
        // workspace: row-smoothed field [B][N], then the smoothed field [B][N]
        float* tmp = static_cast<float*>(workspace);
        float* sbar = tmp + (int64_t)a->B * a->N;
        const dim3 g((unsigned)((a->N + 255) / 256), (unsigned)a->B);
        hipLaunchKernelGGL(pcsp_smooth_kernel<true>, g, dim3(256), 0, s, (const float*)a->acc, tmp, a->N,
                           a->grid_h, a->grid_w, p.radius, p.sigma, (int64_t)a->N, (int64_t)a->N);
        hipLaunchKernelGGL(pcsp_smooth_kernel<false>, g, dim3(256), 0, s, (const float*)tmp, sbar, a->N,
                           a->grid_h, a->grid_w, p.radius, p.sigma, (int64_t)a->N, (int64_t)a->N);
        if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
        p.ws = sbar;
      }
      if (a->N <= kKeyCap) hipLaunchKernelGGL(pcsp_select_kernel<true>, dim3(a->B), dim3(SNT), 0, s, p);
      else hipLaunchKernelGGL(pcsp_select_kernel<false>, dim3(a->B), dim3(SNT), 0, s, p);
      if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
    }
  }
  return SAFE_OK;
}

}  // namespace safe
