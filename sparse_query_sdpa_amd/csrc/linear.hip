// Row-wise linear maps of the block around attention ("SAFE-DiT" Eq. 15: the
// row-selective block computes its projections, residual updates and MLP only for
// the rows of S): out[ro(r)] = epilogue(A[ra(r)] . W^T) with gathered input rows,
// scattered output rows, bias, tanh-GELU and a (gathered) residual.
//
// gfx950 design
//   The product runs transposed, D^T = W . A^T, with v_mfma_f32_32x32x16_bf16: the
//   MFMA A operand is 32 rows of W (output features n), the B operand 32 rows of A
//   (tokens m); both are read 16 bytes per lane from LDS rows of k, so neither needs a
//   transpose, and in the accumulator lane l owns token m = l % 32 and runs of four
//   consecutive features -- the epilogue stores 8 bytes per run.
//   Two tile shapes: 256 x 256 (8 waves of 64 features x 128 tokens, one workgroup per
//   CU: 6 LDS fragment reads feed 8 MFMAs) when the problem fills the GPU at least once,
//   else 128 x 128 (4 waves of 64 x 64, two workgroups per CU).  k advances 64 per
//   stage; A and W tiles are copied global -> LDS with global_load_lds_dwordx4 (no
//   staging registers), double buffered, one barrier per stage.  LDS rows are 9 chunks
//   of 16 bytes (8 used): an odd chunk count keeps the 16-lane row reads conflict-free.
//   Gathered A rows use per-lane 64-bit source pointers, fixed for the whole k loop; W
//   rows use a scalar base and 32-bit offsets.
#include "common.h"

namespace safe {
namespace {

constexpr int LK = 64;           // k per stage
constexpr int LSLOTS = 9;        // 16-byte chunks per LDS row (8 used)
constexpr int LROWB = LSLOTS * 16;

// Tile shapes: WN x WM waves, each owning BNB x BMB 32 x 32 MFMA blocks (features x tokens).
template <int WN_, int WM_, int BNB_, int BMB_>
struct LinCfg {
  static constexpr int WN = WN_, WM = WM_, BNB = BNB_, BMB = BMB_;
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
  static_assert(TM * LSLOTS % 64 == 0 && TN * LSLOTS % 64 == 0 && NCOPY % WAVES == 0, "copy plan");
};
// 128 x 128 tiles, 4 waves of 64 x 64 (two workgroups per CU), and 256 x 256 tiles, 8 waves
// of 64 x 128 (one workgroup per CU): 6 LDS reads feed 8 MFMAs instead of 4 feeding 4.
typedef LinCfg<2, 2, 2, 2> LinSmall;
typedef LinCfg<4, 2, 2, 4> LinLarge;

struct LinParams {
  const char* a; const char* w; const float* bias; const char* res; char* out;
  int64_t a_bs, a_s, w_s, res_bs, res_s, out_bs, out_s;   // byte strides
  const int32_t* a_rows; const int32_t* res_rows; const int32_t* out_rows;
  int64_t rows_bs;
  int M, N, K, Ntok, act, tiles_m, tiles_n, batches;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void lcopy16(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}

// tanh-form GELU: x/2 (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), with
// tanh(u) = 1 - 2 / (1 + e^{2u}) (saturates to +-1 without overflow trouble).
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * x, x * x, x);
  const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * u);   // e^{2u}
  const float t = 1.0f - 2.0f / (1.0f + e);
  return 0.5f * x * (1.0f + t);
}

__device__ __forceinline__ int bounded_row(const int32_t* rows, int64_t bs, int b, int r, int limit) {
  const int v = rows[(int64_t)b * bs + r];
  return (v >= 0 && v < limit) ? v : -1;
}

template <typename CFG>
__global__ __launch_bounds__(CFG::THREADS, CFG::MIN_BLOCKS) void linear_kernel(LinParams p) {
  constexpr int LWAVES = CFG::WAVES, LPER_WAVE = CFG::PER_WAVE, LCOPY_A = CFG::COPY_A;
  constexpr int BNB = CFG::BNB, BMB = CFG::BMB;
  __shared__ __attribute__((aligned(1024))) char st0[CFG::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[CFG::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int wn = wave % CFG::WN, wm = wave / CFG::WN;       // this wave's block of the tile
  // Consecutive logical tiles share an XCD (xcd_remap) and are ordered in groups of
  // kGroupM tiles along m: the 32 or so tiles that run side by side on one XCD cover
  // 8 (m) x 4 (n), so both their A and their W panels are shared in its L2 (+8-9% over
  // a plain m-fastest order, where every A panel came from HBM).
  constexpr int kGroupM = 8;
  const int per_b = p.tiles_m * p.tiles_n;
  const int logical = xcd_remap(blockIdx.x, per_b * p.batches);
  const int b = logical / per_b, t = logical - b * per_b;
  const int group = t / (kGroupM * p.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, p.tiles_m - first_m);
  const int gi = t - group * kGroupM * p.tiles_n;
  const int tm = first_m + gi % gm, tn = gi / gm;
  const int m0 = tm * CFG::TM, n0 = tn * CFG::TN;

  // ---- copy plan: copy c < LCOPY_A fills A slots [64c, 64c+64), the rest W slots --
  // slot sigma: row sigma / 9, chunk sigma % 9 (chunk 8 is padding: it fetches chunk 0
  // of its row, never read back).  Rows past M (tokens) or N (features) fetch row 0.
  const char* aptr[LPER_WAVE];    // A copies: per-lane 64-bit source (k = 0)
  uint32_t woff[LPER_WAVE];       // W copies: byte offset from the tile's first row
  const char* wbase = p.w + (int64_t)n0 * p.w_s;
#pragma unroll
  for (int m = 0; m < LPER_WAVE; ++m) {
    const int c = wave + LWAVES * m;
    const bool isa = c < LCOPY_A;
    const int sigma = (isa ? c : c - LCOPY_A) * 64 + lane;
    const int row = sigma / LSLOTS;
    int chunk = sigma % LSLOTS;
    if (chunk >= 8) chunk = 0;
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

  f32x16 acc[BNB][BMB];
#pragma unroll
  for (int i = 0; i < BNB; ++i)
#pragma unroll
    for (int j = 0; j < BMB; ++j) acc[i][j] = f32x16{};
  const int a_lane = (wm * BMB * 32 + col) * LROWB + half * 16;   // B operand: token rows
  const int w_lane = (wn * BNB * 32 + col) * LROWB + half * 16;   // A operand: feature rows

  auto compute = [&](const char* stage) {
    const char* At = stage;
    const char* Wt = stage + CFG::A_BYTES;
#pragma unroll
    for (int s = 0; s < LK / 16; ++s) {
      bf16x8 af[BMB], wf[BNB];
#pragma unroll
      for (int j = 0; j < BMB; ++j) af[j] = as_bf16x8(ld16(At + a_lane + j * 32 * LROWB + s * 32));
#pragma unroll
      for (int i = 0; i < BNB; ++i) wf[i] = as_bf16x8(ld16(Wt + w_lane + i * 32 * LROWB + s * 32));
#pragma unroll
      for (int i = 0; i < BNB; ++i)
#pragma unroll
        for (int j = 0; j < BMB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
  };

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

  // ---- epilogue: lane owns token m and, per feature block i, four runs of 4 features --
  const int r = m0 + wm * BMB * 32;   // + j * 32 + col
#pragma unroll
  for (int j = 0; j < BMB; ++j) {
    const int rr = r + j * 32 + col;
    if (rr >= p.M) continue;
    int ro = rr, rres = rr;
    if (p.out_rows != nullptr) ro = bounded_row(p.out_rows, p.rows_bs, b, rr, p.Ntok);
    if (ro < 0) continue;   // an invalid scatter index is skipped
    if (p.res != nullptr && p.res_rows != nullptr) rres = bounded_row(p.res_rows, p.rows_bs, b, rr, p.Ntok);
    const char* resp = (p.res != nullptr && rres >= 0) ? p.res + (int64_t)b * p.res_bs + (int64_t)rres * p.res_s : nullptr;
    char* op = p.out + (int64_t)b * p.out_bs + (int64_t)ro * p.out_s;
#pragma unroll
    for (int i = 0; i < BNB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * BNB * 32 + i * 32 + 8 * g + 4 * half;
        if (n >= p.N) continue;
        float y[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (p.bias != nullptr) {
          const f32x4 bv = __builtin_bit_cast(f32x4, ld16(p.bias + n));
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += bv[e];
        }
        if (p.act == SAFE_ACT_GELU_TANH) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = gelu_tanh(y[e]);
        }
        if (resp != nullptr) {
          const u32x2 rv = *reinterpret_cast<const u32x2*>(resp + n * 2);
          const f32x2 lo = __builtin_bit_cast(f32x2, rv << 16);
          const f32x2 hi = __builtin_bit_cast(f32x2, rv & 0xFFFF0000u);
          y[0] += lo[0]; y[1] += hi[0]; y[2] += lo[1]; y[3] += hi[1];
        }
        u32x2 w;
        w[0] = pack_bf16x2(y[0], y[1]);
        w[1] = pack_bf16x2(y[2], y[3]);
        st8(op + n * 2, w);
      }
  }
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
  const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * a->batches;
  if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
  if (large) hipLaunchKernelGGL(linear_kernel<LinLarge>, dim3((unsigned)grid), dim3(LinLarge::THREADS), 0, s, p);
  else hipLaunchKernelGGL(linear_kernel<LinSmall>, dim3((unsigned)grid), dim3(LinSmall::THREADS), 0, s, p);
  return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
