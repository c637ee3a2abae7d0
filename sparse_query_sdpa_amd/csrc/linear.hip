// Row-wise linear maps of the block around attention ("SAFE-DiT" Eq. 15: the
// row-selective block computes its projections, residual updates and MLP only for
// the rows of S): out[ro(r)] = epilogue(A[ra(r)] . W^T) with gathered input rows,
// scattered output rows, bias, tanh-GELU and a (gathered) residual.
//
// gfx950 design
//   The product runs transposed, D^T = W . A^T, with v_mfma_f32_16x16x32_bf16: the
//   MFMA A operand is 16 rows of W (output features n), the B operand 16 rows of A
//   (tokens m); both are read 16 bytes per lane from LDS rows of k, so neither needs a
//   transpose, and in the accumulator lane l owns token m = l % 16 and a run of four
//   consecutive features.  The 16x16x32 shape moves the same LDS bytes per FLOP as
//   32x32x16 for a given wave tile (the fragment reuse is set by the tile), and on this
//   power-limited chip it runs 10-18% faster on these maps: with random operands it draws
//   less energy per FLOP, so the clock stays higher (the outputs are bit-identical).
//   Two tile shapes: 256 x 256 (8 waves of 64 features x 128 tokens, one workgroup per
//   CU: 12 LDS fragment reads feed 32 MFMAs per 32 k) when the problem fills the GPU at
//   least once, else 128 x 128 (4 waves of 64 x 64, two workgroups per CU).  k advances 64
//   per stage; A and W tiles are copied global -> LDS with global_load_lds_dwordx4 (no
//   staging registers).  An LDS row holds the stage's 8 chunks of 16 bytes in an order
//   rotated by the row (chunk c of row r sits at position c ^ ((r >> 1) & 7)): the 16
//   rows one fragment read touches then cover all 64 banks, and no copy bytes are spent
//   on padding.  The copies fetch the chunks already in that order, so the LDS side stays
//   lane-linear.  Gathered A rows use per-lane 64-bit source pointers, fixed for the whole
//   k loop; W rows use a scalar base and 32-bit offsets.
//   The epilogue goes through LDS: the accumulators (fp32) are written into the freed
//   stage buffers, then read back a token row at a time, so bias, GELU, residual and
//   the bf16 store run along the row and every store instruction writes whole 256-byte
//   runs of two rows (written straight from the accumulator layout, a store touched 16
//   rows, and the tile's drain was a fifth of the kernel).
#include "common.h"

namespace safe {
namespace {

constexpr int LK = 64;           // k per stage
constexpr int LSLOTS = 8;        // 16-byte chunks per LDS row, stored rotated (see above)
constexpr int LROWB = LSLOTS * 16;

// Tile shapes: WN x WM waves, each owning BNB x BMB 32 x 32 MFMA blocks (features x tokens).
template <int WN_, int WM_, int BNB_, int BMB_>
struct LinCfg {
  static constexpr int WN = WN_, WM = WM_, BNB = BNB_, BMB = BMB_;
  // a wave's 32-row blocks are NI x NJ v_mfma_f32_16x16x32_bf16 blocks of 16 features x 16 tokens
  static constexpr int NI = BNB * 2, NJ = BMB * 2;
  static constexpr int WAVES = WN * WM;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int TN = WN * BNB * 32;                 // features per tile
  static constexpr int TM = WM * BMB * 32;                 // tokens per tile
  static constexpr int COPY_A = TM * LSLOTS / 64;          // wave-wide 1 KB copies per stage
  static constexpr int COPY_W = TN * LSLOTS / 64;
  static constexpr int NCOPY = COPY_A + COPY_W;
  static constexpr int PER_WAVE = NCOPY / WAVES;
  static constexpr int A_BYTES = TM * LROWB;
  static constexpr int STAGE = (TM + TN) * LROWB;          // A tile then W tile
  static constexpr int MIN_BLOCKS = 4 * STAGE <= 160 * 1024 ? 2 : 1;
  // epilogue: the two stage buffers hold ER fp32 token rows of TN features
  static constexpr int EROWB = TN * 4;
  static constexpr int ER = 2 * STAGE / EROWB;
  static_assert(TM * LSLOTS % 64 == 0 && TN * LSLOTS % 64 == 0 && NCOPY % WAVES == 0, "copy plan");
};
// 128 x 128 tiles, 4 waves of 64 x 64 (two workgroups per CU), and 256 x 256 tiles, 8 waves
// of 64 x 128 (one workgroup per CU): 12 LDS reads feed 32 MFMAs instead of 8 feeding 16.
typedef LinCfg<2, 2, 2, 2> LinSmall;
typedef LinCfg<4, 2, 2, 4> LinLarge;

struct LinParams {
  const char* a; const char* w; const float* bias; const char* res; char* out;
  int64_t a_bs, a_s, w_s, res_bs, res_s, out_bs, out_s;   // byte strides
  const int32_t* a_rows; const int32_t* res_rows; const int32_t* out_rows;
  int64_t rows_bs;
  int M, N, K, Ntok, act, tiles_m, tiles_n, batches;
  // Launch split: the 256 x 256 kernel takes logical tiles [0, grid); the 128 x 128 kernel
  // with tail_first >= 0 takes the last partial round, large tiles tail_first.., as four
  // 128 x 128 sub-tiles each (tiles_m / tiles_n count 256 x 256 tiles then).
  int tail_first;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void lcopy16(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}

// tanh-form GELU: x/2 (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), with
// tanh(u) = 1 - 2 / (1 + e^{2u}) (saturates to +-1 without overflow trouble).  The
// reciprocal is the hardware's (1 ulp): its error in tanh is ~2^-23, far below the bf16
// rounding of the result, and it replaces the ten-instruction IEEE division.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * x, x * x, x);
  const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * u);   // e^{2u}
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
  return 0.5f * x * (1.0f + t);
}

__device__ __forceinline__ int bounded_row(const int32_t* rows, int64_t bs, int b, int r, int limit) {
  const int v = rows[(int64_t)b * bs + r];
  return (v >= 0 && v < limit) ? v : -1;
}

// Logical tile -> (batch, first token, first feature).  Tiles are ordered in groups of
// kGroupM along m: with consecutive logical tiles on one XCD (xcd_remap, or the persistent
// walk below), the ~32 tiles that run side by side there cover 8 (m) x 4 (n), so both
// their A and their W panels are shared in its L2 (+8-9% over a plain m-fastest order,
// where every A panel came from HBM).
__device__ __forceinline__ void lin_tile(const LinParams& p, int logical, int TM, int TN, int& b, int& m0, int& n0) {
  constexpr int kGroupM = 8;
  const int per_b = p.tiles_m * p.tiles_n;
  b = logical / per_b;
  const int t = logical - b * per_b;
  const int group = t / (kGroupM * p.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, p.tiles_m - first_m);
  const int gi = t - group * kGroupM * p.tiles_n;
  m0 = (first_m + gi % gm) * TM;
  n0 = (gi / gm) * TN;
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS operations, not for
// its vector-memory ones (copies into other buffers stay in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Staged epilogue of one tile, ER token rows a round.  Write: lane l of 16 x 16 block (i, j)
// holds token wm*BMB*32 + 16j + l % 16 and features wn*BNB*32 + 16i + 4(l / 16) + [0, 4): a
// 16-byte chunk c = feature / 4 of the token's fp32 row, stored at position c ^ (token & 15)
// (the 16 rows of one write then cover all banks).  Read: 32 lanes per
// row, lane u holding chunks u, u + 32, ...; then bias, GELU, residual, bf16 and an
// 8-byte store per chunk, 256 contiguous bytes per 32 lanes.  A lane finishes IT rows a
// round; their index-list entries and residual runs are loaded before the round's LDS work,
// so each round waits for memory once instead of once per row.  rowp(tt) is the LDS row
// of staged token tt (rows of one 32-token block are contiguous).  The caller has made the
// staging rows free (barrier); the function ends with them free again.
template <typename CFG, int ER, typename RowPtr>
__device__ __forceinline__ void lin_epilogue(const LinParams& p, const f32x4 (&acc)[CFG::NI][CFG::NJ],
                                             int b, int m0, int n0, int wave, int lane, RowPtr rowp) {
  constexpr int BNB = CFG::BNB, BMB = CFG::BMB, LWAVES = CFG::WAVES;
  constexpr int CPR = CFG::TN / 4;          // 16-byte fp32 chunks per staged row
  constexpr int CPL = CPR / 32;             // of which each reading lane holds CPL
  constexpr int ROUNDS = CFG::TM / ER;
  constexpr int IT = ER / (2 * LWAVES);     // rows a lane finishes per round
  static_assert(ER % 32 == 0 && CFG::TM % ER == 0 && CPR % 32 == 0 && ER % (2 * LWAVES) == 0, "epilogue plan");
  const int col = lane & 31, half = lane >> 5;
  const int wn = wave % CFG::WN, wm = wave / CFG::WN;
  f32x4 bias[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int n = n0 + 4 * (col + 32 * u);
    bias[u] = (p.bias != nullptr && n < p.N) ? __builtin_bit_cast(f32x4, ld16(p.bias + n)) : f32x4{};
  }
#pragma unroll
  for (int rnd = 0; rnd < ROUNDS; ++rnd) {
    // this lane's rows: output row (-1: skipped) and residual row (-1: none)
    int ro[IT], rres[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int rr = m0 + rnd * ER + (wave * IT + it) * 2 + half;
      ro[it] = -1; rres[it] = -1;
      if (rr < p.M) {
        ro[it] = p.out_rows != nullptr ? bounded_row(p.out_rows, p.rows_bs, b, rr, p.Ntok) : rr;
        if (p.res != nullptr) rres[it] = p.res_rows != nullptr ? bounded_row(p.res_rows, p.rows_bs, b, rr, p.Ntok) : rr;
      }
    }
    u32x2 rv[IT][CPL];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int n = n0 + 4 * (col + 32 * u);
        rv[it][u] = u32x2{0u, 0u};
        if (ro[it] >= 0 && rres[it] >= 0 && n < p.N)
          rv[it][u] = *reinterpret_cast<const u32x2*>(p.res + (int64_t)b * p.res_bs + (int64_t)rres[it] * p.res_s + n * 2);
      }
#pragma unroll
    for (int j = 0; j < CFG::NJ; ++j) {
      if ((wm * BMB * 32 + j * 16) / ER != rnd) continue;   // wave-uniform
      const int tt = wm * BMB * 32 + j * 16 - rnd * ER + (lane & 15);
      char* row = rowp(tt);
#pragma unroll
      for (int i = 0; i < CFG::NI; ++i) {
        const int c = (wn * BNB * 32 + i * 16 + 4 * (lane >> 4)) >> 2;
        *reinterpret_cast<f32x4*>(row + ((c ^ (tt & 15)) << 4)) = acc[i][j];
      }
    }
    lds_barrier();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int tt = (wave * IT + it) * 2 + half;
      const char* row = rowp(tt);
      f32x4 y[CPL];
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        y[u] = *reinterpret_cast<const f32x4*>(row + (((col + 32 * u) ^ (tt & 15)) << 4));
      if (ro[it] < 0) continue;   // past M, or an invalid scatter index: skipped
      char* op = p.out + (int64_t)b * p.out_bs + (int64_t)ro[it] * p.out_s;
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int n = n0 + 4 * (col + 32 * u);
        if (n >= p.N) continue;
        float e[4] = {y[u][0], y[u][1], y[u][2], y[u][3]};
        if (p.bias != nullptr) {
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] += bias[u][q];
        }
        if (p.act == SAFE_ACT_GELU_TANH) {
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = gelu_tanh(e[q]);
        }
        if (rres[it] >= 0) {
          const f32x2 lo = __builtin_bit_cast(f32x2, rv[it][u] << 16);
          const f32x2 hi = __builtin_bit_cast(f32x2, rv[it][u] & 0xFFFF0000u);
          e[0] += lo[0]; e[1] += hi[0]; e[2] += lo[1]; e[3] += hi[1];
        }
        u32x2 w;
        w[0] = pack_bf16x2(e[0], e[1]);
        w[1] = pack_bf16x2(e[2], e[3]);
        st8(op + n * 2, w);
      }
    }
    lds_barrier();   // the rows are free for the next round (or the caller)
  }
}

// Lane addressing of the fragment reads.  Lane l reads row l % 16 of a 16-row block (plus
// multiples of 16, so the row's rotation (row >> 1) & 7 depends on the lane alone) and k-step
// s (32 k) takes its chunk 4s + l / 16, at position (4s + l/16) ^ rot = rq ^ 4s.
template <typename CFG>
struct LinLanes {
  int a, w, rq;
  __device__ __forceinline__ LinLanes(int lane, int wn, int wm) {
    const int r = lane & 15;
    a = (wm * CFG::BMB * 32 + r) * LROWB;   // B operand: token rows
    w = (wn * CFG::BNB * 32 + r) * LROWB;   // A operand: feature rows
    rq = (lane >> 4) ^ ((r >> 1) & 7);
  }
};

// One k stage (64 k) of MFMAs: At / Wt are the stage's A and W tiles (LROWB-byte rotated rows).
template <typename CFG>
__device__ __forceinline__ void lin_stage(f32x4 (&acc)[CFG::NI][CFG::NJ], const char* At, const char* Wt,
                                          const LinLanes<CFG>& ln) {
  constexpr int NI = CFG::NI, NJ = CFG::NJ;
#pragma unroll
  for (int s = 0; s < LK / 32; ++s) {
    const int co = (ln.rq ^ (4 * s)) << 4;
    bf16x8 af[NJ], wf[NI];
#pragma unroll
    for (int j = 0; j < NJ; ++j) af[j] = as_bf16x8(ld16(At + ln.a + j * 16 * LROWB + co));
#pragma unroll
    for (int i = 0; i < NI; ++i) wf[i] = as_bf16x8(ld16(Wt + ln.w + i * 16 * LROWB + co));
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
  }
}

template <typename CFG>
__global__ __launch_bounds__(CFG::THREADS, CFG::MIN_BLOCKS) void linear_kernel(LinParams p) {
  constexpr int LWAVES = CFG::WAVES, LPER_WAVE = CFG::PER_WAVE, LCOPY_A = CFG::COPY_A;
  __shared__ __attribute__((aligned(1024))) char lds[2 * CFG::STAGE];
  char* const st0 = lds;
  char* const st1 = lds + CFG::STAGE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % CFG::WN, wm = wave / CFG::WN;       // this wave's block of the tile
  int b, m0, n0;
  if (p.tail_first >= 0) {   // sub-tile q % 4 of large tile tail_first + q / 4
    const int q = xcd_remap(blockIdx.x, gridDim.x);
    lin_tile(p, p.tail_first + q / 4, 2 * CFG::TM, 2 * CFG::TN, b, m0, n0);
    m0 += (q & 1) * CFG::TM;
    n0 += ((q >> 1) & 1) * CFG::TN;
  } else {
    lin_tile(p, xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n * p.batches), CFG::TM, CFG::TN, b, m0, n0);
  }

  // ---- copy plan: copy c < LCOPY_A fills A slots [64c, 64c+64), the rest W slots --
  // slot sigma: row sigma / 8, position sigma % 8, which holds chunk position ^ ((row >> 1)
  // & 7) of the row.  Rows past M (tokens) or N (features) fetch row 0.
  const char* aptr[LPER_WAVE];    // A copies: per-lane 64-bit source (k = 0)
  uint32_t woff[LPER_WAVE];       // W copies: byte offset from the tile's first row
  const char* wbase = p.w + (int64_t)n0 * p.w_s;
#pragma unroll
  for (int m = 0; m < LPER_WAVE; ++m) {
    const int c = wave + LWAVES * m;
    const bool isa = c < LCOPY_A;
    const int sigma = (isa ? c : c - LCOPY_A) * 64 + lane;
    const int row = sigma / LSLOTS;
    const int chunk = (sigma % LSLOTS) ^ ((row >> 1) & 7);
    if (isa) {
      const int r = m0 + row;
      int src = 0;
      if (r < p.M) {
        src = r;
        if (p.a_rows != nullptr) {
          src = bounded_row(p.a_rows, p.rows_bs, b, r, p.Ntok);
          if (src < 0) src = 0;
        }
      }
      aptr[m] = p.a + (int64_t)b * p.a_bs + (int64_t)src * p.a_s + chunk * 16;
      woff[m] = 0;
    } else {
      const int n = n0 + row < p.N ? row : 0;
      woff[m] = (uint32_t)(n * p.w_s + chunk * 16);
      aptr[m] = nullptr;
    }
  }
  auto issue = [&](int k0, char* stage) {
    int wl = wave * 1024;
    asm volatile("" : "+s"(wl));
#pragma unroll
    for (int m = 0; m < LPER_WAVE; ++m) {
      const int c = wave + LWAVES * m;
      const bool all_a = LWAVES * m + LWAVES - 1 < LCOPY_A;   // compile-time per unrolled m
      const bool all_w = LWAVES * m >= LCOPY_A;
      char* dst = stage + wl + m * LWAVES * 1024;
      if (all_a || (!all_w && c < LCOPY_A)) {
        lcopy16(aptr[m] + (int64_t)k0 * 2, dst);
      } else {
        uint32_t o = woff[m];
        asm volatile("" : "+v"(o));
        lcopy16(wbase + (int64_t)k0 * 2 + o, dst);
      }
    }
  };

  f32x4 acc[CFG::NI][CFG::NJ];
#pragma unroll
  for (int i = 0; i < CFG::NI; ++i)
#pragma unroll
    for (int j = 0; j < CFG::NJ; ++j) acc[i][j] = f32x4{};
  const LinLanes<CFG> ln(lane, wn, wm);
  auto compute = [&](const char* stage) { lin_stage<CFG>(acc, stage, stage + CFG::A_BYTES, ln); };

  const int nst = p.K / LK;
  if (nst > 0) issue(0, st0);
  int s = 0;
  for (; s + 2 <= nst; s += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
    __syncthreads();                      // everyone's; the other stage is free
    if (s + 1 < nst) issue((s + 1) * LK, st1);
    compute(st0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (s + 2 < nst) issue((s + 2) * LK, st0);
    compute(st1);
  }
  if (s < nst) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    compute(st0);
  }

  __syncthreads();   // every wave is done with the stage buffers
  lin_epilogue<CFG, CFG::ER>(p, acc, b, m0, n0, wave, lane, [&](int tt) { return lds + tt * CFG::EROWB; });
}

// ---- 256 x 256 tiles through a ring of half-stage buffers ------------------------------
// The copies run through five half-stage buffers (the A or the W tile of one k stage, 32 KB
// each, 160 KB): while stage s is multiplied, stage s + 1 and the A tile of stage s + 2 are
// in flight (96 KB per CU instead of the 64 KB of a double-buffered stage), and each step
// waits only for the copies it needs (vmcnt of the younger half-stage), with a barrier that
// does not drain the copy queue.  Each step then issues the next two half-stages into the
// buffers the previous step freed.  (A persistent form that also ran the ring on into the
// next tile, so its first copies overlapped this tile's epilogue, measured no faster.)
constexpr int PHALF = LinLarge::STAGE / 2;   // bytes of one half-stage buffer
constexpr int PRING = 5;                     // half-stage buffers in the ring

template <typename CFG>
__global__ __launch_bounds__(CFG::THREADS, 1) void linear_ring_kernel(LinParams p) {
  constexpr int LWAVES = CFG::WAVES;
  static_assert(CFG::COPY_A == 4 * LWAVES && CFG::COPY_W == 4 * LWAVES && CFG::A_BYTES == PHALF, "ring copy plan");
  static_assert(PRING * PHALF <= 160 * 1024 && 2 * CFG::STAGE <= PRING * PHALF, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[PRING * PHALF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % CFG::WN, wm = wave / CFG::WN;
  int b, m0, n0;
  lin_tile(p, xcd_remap(blockIdx.x, gridDim.x), CFG::TM, CFG::TN, b, m0, n0);

  // Copy plan: copy mm of the A (W) half-stage fills slots 64 (wave + 8 mm) + lane; slot
  // sigma = row sigma / 8, position sigma % 8 holding chunk position ^ ((row >> 1) & 7).
  // Rows past M (tokens) or N (features) fetch row 0.
  const char* aptr[4];
  uint32_t woff[4];
  const char* wbase = p.w + (int64_t)n0 * p.w_s;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    const int sigma = (wave + LWAVES * mm) * 64 + lane;
    const int row = sigma / LSLOTS;
    const int chunk = (sigma % LSLOTS) ^ ((row >> 1) & 7);
    const int r = m0 + row;
    int src = 0;
    if (r < p.M) {
      src = r;
      if (p.a_rows != nullptr) {
        src = bounded_row(p.a_rows, p.rows_bs, b, r, p.Ntok);
        if (src < 0) src = 0;
      }
    }
    aptr[mm] = p.a + (int64_t)b * p.a_bs + (int64_t)src * p.a_s + chunk * 16;
    const int n = n0 + row < p.N ? row : 0;
    woff[mm] = (uint32_t)(n * p.w_s + chunk * 16);
  }
  // half-stage h: the A tile of stage h / 2 if h is even, else its W tile; buffer h % PRING
  auto issue_half = [&](int h) {
    const int64_t k2 = (int64_t)(h >> 1) * (LK * 2);
    int wl = (h % PRING) * PHALF + wave * 1024;
    asm volatile("" : "+s"(wl));
    char* dst = lds + wl;
    if ((h & 1) == 0) {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) lcopy16(aptr[mm] + k2, dst + mm * LWAVES * 1024);
    } else {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        uint32_t o = woff[mm];
        asm volatile("" : "+v"(o));
        lcopy16(wbase + k2 + o, dst + mm * LWAVES * 1024);
      }
    }
  };

  f32x4 acc[CFG::NI][CFG::NJ];
#pragma unroll
  for (int i = 0; i < CFG::NI; ++i)
#pragma unroll
    for (int j = 0; j < CFG::NJ; ++j) acc[i][j] = f32x4{};
  const LinLanes<CFG> ln(lane, wn, wm);
  const int nst = p.K / LK, nh = 2 * nst;
  int issued = 0;
  for (; issued < nh && issued < 2; ++issued) issue_half(issued);   // stage 0 alone: it is needed first
  for (int s = 0; s < nst; ++s) {
    // this wave's copies of half-stages up to 2s + 1 have landed; younger ones (4 copies
    // each) may stay in flight
    const int out = issued - (2 * s + 2);
    if (out >= 3) __builtin_amdgcn_s_waitcnt(0x0F7C);        // vmcnt(12)
    else if (out == 2) __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
    else if (out == 1) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0)
    lds_barrier();   // everyone's have; step s - 1's buffers are free
    for (; issued < nh && issued <= 2 * s + PRING - 1; ++issued) issue_half(issued);
    lin_stage<CFG>(acc, lds + ((2 * s) % PRING) * PHALF, lds + ((2 * s + 1) % PRING) * PHALF, ln);
  }
  lds_barrier();   // every wave is done with the stage buffers (all copies have landed)
  lin_epilogue<CFG, CFG::ER>(p, acc, b, m0, n0, wave, lane, [&](int tt) { return lds + tt * CFG::EROWB; });
}

}  // namespace

// Enqueue the linear map.  Arguments were validated by the caller.
int linear_launch(const safe_linear_args* a, hipStream_t s) {
  if ((int64_t)a->batches * a->M * a->N == 0) return SAFE_OK;
  LinParams p;
  p.a = static_cast<const char*>(a->a);
  p.w = static_cast<const char*>(a->w);
  p.bias = a->bias;
  p.res = static_cast<const char*>(a->res);
  p.out = static_cast<char*>(a->out);
  p.a_bs = a->a_stride[0] * 2; p.a_s = a->a_stride[1] * 2;
  p.w_s = a->w_stride * 2;
  p.res_bs = a->res_stride[0] * 2; p.res_s = a->res_stride[1] * 2;
  p.out_bs = a->out_stride[0] * 2; p.out_s = a->out_stride[1] * 2;
  p.a_rows = a->a_rows; p.res_rows = a->res_rows; p.out_rows = a->out_rows;
  p.rows_bs = a->rows_bstride;
  p.M = a->M; p.N = a->N; p.K = a->K; p.Ntok = a->Ntok; p.act = a->act;
  p.batches = a->batches;
  // Large tiles when they fill the GPU at least once (one workgroup per CU); otherwise the
  // small ones, whose 4x as many workgroups spread better over a short problem.
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int64_t large_tiles = ceil_div64(a->M, LinLarge::TM) * ceil_div64(a->N, LinLarge::TN) * a->batches;
  const bool large = large_tiles >= cus;
  const int TM = large ? LinLarge::TM : LinSmall::TM, TN = large ? LinLarge::TN : LinSmall::TN;
  p.tiles_m = (a->M + TM - 1) / TM;
  p.tiles_n = (a->N + TN - 1) / TN;
  p.tail_first = -1;
  const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * a->batches;
  if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
  if (!large) {
    hipLaunchKernelGGL(linear_kernel<LinSmall>, dim3((unsigned)grid), dim3(LinSmall::THREADS), 0, s, p);
    return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
  }
  // The last round of large tiles, when it would leave more than half the CUs idle, runs as
  // 128 x 128 sub-tiles instead (two workgroups per CU): the 4 x rem sub-tiles finish in a
  // quarter to a half of a large tile's time.  A tile's sums are the same either way (same
  // MFMA shape, same k order), so the split does not change the result.
  const int64_t rem = grid % cus;
  const bool tail = rem > 0 && 4 * rem <= 2 * (int64_t)cus;
  const int64_t head = tail ? grid - rem : grid;
  hipLaunchKernelGGL(linear_ring_kernel<LinLarge>, dim3((unsigned)head), dim3(LinLarge::THREADS), 0, s, p);
  if (tail) {
    if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
    p.tail_first = (int)head;
    hipLaunchKernelGGL(linear_kernel<LinSmall>, dim3((unsigned)(4 * rem)), dim3(LinSmall::THREADS), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
