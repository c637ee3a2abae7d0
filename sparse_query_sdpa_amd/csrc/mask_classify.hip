// Row-constant mask certifier ("SAFE-DiT" Eq. 6-8).
//
// For every stored row of a [B, H, Nq, Nk] mask (broadcast dims stored once) the
// scan decides whether the row is one real constant (class R: all-valid Boolean,
// all-zero or row-constant additive) or which kept pattern it is (text key
// padding, non-constant, blocked, non-finite).  The overall class is the maximum
// row class; a key-padding mask is reported with its per-sample valid length when
// every row of a sample has the same one.
//
// Kernels: init (clear the reduction slots) -> scan (HBM stream: each wave walks a
// contiguous range of rows in steps of 8 KB, two steps of loads in flight across row
// boundaries) -> finalize (one thread: overall class, verdict, per-sample lengths).  Element tests work on bit patterns: -inf is the blocked
// value, NaN/+inf are non-finite, equality is IEEE equality (so -0 == +0).
#include <limits.h>

#include "common.h"

namespace safe {
namespace {

constexpr int NT = 256;
constexpr int WAVES_PER_BLOCK = NT / kWave;
// Scan shape, measured on the 160x160 workload's [2,1,N,N] bf16 mask (2.62 GB) and the
// 192x192 workload's [1,1,N,N] fp32 mask (5.44 GB), fraction of 8 TB/s: 4 waves per CU
// (1024 waves on the chip, ~50 rows each) with 8 chunks per lane per step and two steps in
// flight reach 83% / 85%; 16 waves per CU 73% / 78%, 8 waves 79-80% / 80-82%, 2-3 waves
// 44-67%.  Fewer concurrent row streams keep the DRAM pages better used, as long as each
// wave keeps two steps of loads in flight.
constexpr int MASK_UNR = 8;            // 16-byte chunks per lane per step
constexpr int MASK_WAVES_PER_CU = 4;

// Workspace layout (bytes)
constexpr size_t WS_INFO = 0;        // safe_mask_info (32 bytes), device copy of the result
constexpr size_t WS_MAXCLS = 32;     // u32 max row class
constexpr size_t WS_FIRSTBAD = 40;   // u64 min bad row (UINT64_MAX = none)
constexpr size_t WS_LEN = 64;        // per stored batch index: int32 min L, int32 max L

struct BoolT { typedef uint8_t U; static constexpr bool is_bool = true; static constexpr U NEG_INF = 0, EXP = 0, ABS = 0; };
struct Bf16T { typedef uint16_t U; static constexpr bool is_bool = false; static constexpr U NEG_INF = 0xFF80u, EXP = 0x7F80u, ABS = 0x7FFFu; };
struct F16T { typedef uint16_t U; static constexpr bool is_bool = false; static constexpr U NEG_INF = 0xFC00u, EXP = 0x7C00u, ABS = 0x7FFFu; };
struct F32T { typedef uint32_t U; static constexpr bool is_bool = false; static constexpr U NEG_INF = 0xFF800000u, EXP = 0x7F800000u, ABS = 0x7FFFFFFFu; };

struct RowAcc {
  bool neq;        // a valid entry differs from the first entry
  bool nonfinite;  // NaN or +inf seen
  int min_blocked; // first blocked position (Nk if none)
  int max_valid;   // last valid position (-1 if none)
};

template <class T>
__device__ __forceinline__ bool is_blocked(typename T::U x) {
  return x == T::NEG_INF;  // for bool, NEG_INF == 0 == false
}

template <class T>
__device__ __forceinline__ void visit(RowAcc& a, typename T::U x, typename T::U first, int pos) {
  if (is_blocked<T>(x)) {
    a.min_blocked = min(a.min_blocked, pos);
    return;
  }
  a.max_valid = max(a.max_valid, pos);
  if (!T::is_bool) {
    if ((x & T::EXP) == T::EXP) a.nonfinite = true;              // NaN or +inf (-inf handled above)
    const bool eq = (x == first) || (((x | first) & T::ABS) == 0);  // IEEE ==, +-0 equal
    if (!eq) a.neq = true;
  }
}

struct ScanParams {
  const uint8_t* mask;   // byte pointer
  int64_t s0, s1, s2;    // element strides
  int64_t S1, S2;        // sizes of dims 1, 2
  int64_t rows;
  int Nk;
  int rows_per_wave;
  int vec;               // rows start 16-byte aligned
  uint8_t* row_class;
  unsigned char* ws;
};

template <class T>
__device__ __forceinline__ void flush_len(unsigned char* ws, int b, int lmin, int lmax) {
  int* len = reinterpret_cast<int*>(ws + WS_LEN);
  atomicMin(&len[2 * b], lmin);
  atomicMax(&len[2 * b + 1], lmax);
}

// Class of one scanned row from its wave-reduced facts (see the file header).
template <class T>
__device__ __forceinline__ unsigned row_class_of(int Nk, bool neq, bool nonfinite, int mb, int mv,
                                                 typename T::U first, int& L) {
  L = -1;
  if (Nk == 0) {
    L = 0;
    return T::is_bool ? SAFE_MASK_ALL_VALID : SAFE_MASK_ZERO;
  }
  if (nonfinite) return SAFE_MASK_NONFINITE;
  if (mb < Nk) {
    if (mb >= 1 && mv < mb && !neq) {
      L = mb;
      return SAFE_MASK_KEY_PADDING;
    }
    return SAFE_MASK_BLOCKED;
  }
  L = Nk;
  if (T::is_bool) return SAFE_MASK_ALL_VALID;
  if (!neq) return (((u32)first & T::ABS) == 0) ? SAFE_MASK_ZERO : SAFE_MASK_ROW_CONST;
  L = -1;
  return SAFE_MASK_NONCONST;
}

// One wave scans the contiguous stored rows [r_begin, r_end).  Rows whose start is 16-byte
// aligned stream as 16-byte chunks, UNR per lane per step; the steps of all the wave's rows
// form one sequence, software-pipelined: the loads of step j + 1 (possibly the next row's
// first step, with that row's first element) are issued before step j's chunks are compared,
// so the per-row wave reduction and the atomics run while the next loads are in flight.
// Every load is unconditional (lanes past the row's last chunk re-read that chunk and ignore
// it), so the compiler's wait counts are exact.
template <class T>
__global__ __launch_bounds__(NT) void mask_scan_kernel(ScanParams p) {
  typedef typename T::U U;
  constexpr int EPC = 16 / sizeof(U);  // elements per 16-byte chunk
  constexpr int UNR = MASK_UNR;        // chunks per lane per step
  constexpr int PER_STEP = kWave * UNR;
  const int lane = threadIdx.x & 63;
  // the wave index made uniform, so the row range, the cursors and the loop are scalar
  const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_BLOCK + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r_begin = wave * p.rows_per_wave;
  const int64_t r_end = min(r_begin + (int64_t)p.rows_per_wave, p.rows);
  const int Nk = p.Nk;

  unsigned wave_max = 0;
  int64_t wave_first_bad = -1;
  int cur_b = -1, lmin = INT_MAX, lmax = -1;

  auto row_ptr = [&](int64_t r, int& b) -> const U* {
    const int64_t i = r % p.S2;
    const int64_t hb = r / p.S2;
    const int64_t hh = hb % p.S1;
    b = (int)(hb / p.S1);
    return reinterpret_cast<const U*>(p.mask) + b * p.s0 + hh * p.s1 + i * p.s2;
  };
  // wave reduction of a finished row, its class, and the per-wave reductions
  auto finish_row = [&](int64_t r, int b, const RowAcc& a, U first) {
    const bool neq = __any(a.neq);
    const bool nonfinite = __any(a.nonfinite);
    int mb = a.min_blocked, mv = a.max_valid;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mb = min(mb, __shfl_xor(mb, off));
      mv = max(mv, __shfl_xor(mv, off));
    }
    int L;
    const unsigned cls = row_class_of<T>(Nk, neq, nonfinite, mb, mv, first, L);
    if (lane == 0 && p.row_class != nullptr) p.row_class[r] = (uint8_t)cls;
    wave_max = max(wave_max, cls);
    if (cls > SAFE_MASK_ROW_CONST && wave_first_bad < 0) wave_first_bad = r;
    if (cls <= SAFE_MASK_KEY_PADDING) {
      if (b != cur_b) {
        if (cur_b >= 0 && lane == 0) flush_len<T>(p.ws, cur_b, lmin, lmax);
        cur_b = b; lmin = INT_MAX; lmax = -1;
      }
      lmin = min(lmin, L);
      lmax = max(lmax, L);
    }
  };

  if (p.vec && Nk >= EPC && Nk % EPC == 0) {
    const int nchunks = Nk / EPC;                                // >= 1, whole chunks
    const int nit = (nchunks + PER_STEP - 1) / PER_STEP;         // steps per row
    const int64_t total = (r_end - r_begin) * nit;
    // A cursor walks the wave's rows step by step; the row's (b, h, i) and its address are
    // advanced incrementally (wave-uniform values, no division per step).
    struct Cursor {
      int64_t r;
      int it, i, hh, b;
      const U* row;
    };
    auto start = [&](int64_t r) {
      Cursor c;
      c.r = r;
      c.it = 0;
      c.i = (int)(r % p.S2);
      const int64_t hb = r / p.S2;
      c.hh = (int)(hb % p.S1);
      c.b = (int)(hb / p.S1);
      c.row = reinterpret_cast<const U*>(p.mask) + c.b * p.s0 + c.hh * p.s1 + c.i * p.s2;
      return c;
    };
    auto advance = [&](Cursor& c) {
      if (++c.it < nit) return;
      c.it = 0;
      ++c.r;
      if (++c.i == p.S2) {
        c.i = 0;
        if (++c.hh == p.S1) {
          c.hh = 0;
          ++c.b;
        }
      }
      c.row = reinterpret_cast<const U*>(p.mask) + c.b * p.s0 + c.hh * p.s1 + c.i * p.s2;
    };
    Cursor ci = start(r_begin), cp = ci;
    u32x4 bA[UNR], bB[UNR];
    auto issue = [&](u32x4 (&buf)[UNR]) {
      const u32x4* rv = reinterpret_cast<const u32x4*>(ci.row);
      const int c0 = ci.it * PER_STEP + lane;
#pragma unroll
      for (int u = 0; u < UNR; ++u) buf[u] = __builtin_nontemporal_load(rv + min(c0 + u * kWave, nchunks - 1));
      advance(ci);
    };
    RowAcc a = {false, false, Nk, -1};
    U first = 0;
    u32 fw = 0;
    bool first_blocked = false;
    auto process = [&](const u32x4 (&buf)[UNR]) {
      if (cp.it == 0) {
        // the row's first element: the low bytes of lane 0's first chunk of its first step
        a = RowAcc{false, false, Nk, -1};
        first = (U)__builtin_amdgcn_readfirstlane(buf[0][0]);
        // the first element replicated as a 16-byte pattern
        if (sizeof(U) == 1) fw = (u32)first * 0x01010101u;
        else if (sizeof(U) == 2) fw = (u32)first | ((u32)first << 16);
        else fw = (u32)first;
        first_blocked = is_blocked<T>(first);
      }
      const int c0 = cp.it * PER_STEP;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < nchunks) {
          const u32x4 v = buf[u];
          if (v[0] == fw && v[1] == fw && v[2] == fw && v[3] == fw) {
            // every element bitwise equal to the first
            if (first_blocked) a.min_blocked = min(a.min_blocked, c * EPC);
            else a.max_valid = max(a.max_valid, c * EPC + EPC - 1);
          } else {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
              const u32 w = v[(e * (int)sizeof(U)) / 4];
              const U x = (U)(w >> (8 * ((e * (int)sizeof(U)) % 4)));
              visit<T>(a, x, first, c * EPC + e);
            }
          }
        }
      }
      if (cp.it == nit - 1) {
        if (!T::is_bool && lane == 0 && !first_blocked && (first & T::EXP) == T::EXP) a.nonfinite = true;
        finish_row(cp.r, cp.b, a, first);
      }
      advance(cp);
    };
    // two buffers in flight: A holds step j, B step j + 1; the steady-state loop has no
    // conditional load, so every wait is "all but the other buffer's loads"
    if (total >= 4) {
      // both issues unconditional here, so the compiler counts both buffers in flight
      issue(bA);
      issue(bB);
      int64_t j = 0;
      for (; j + 4 <= total; j += 2) {
        process(bA);
        issue(bA);      // step j + 2
        process(bB);
        issue(bB);      // step j + 3
      }
      // the last two or three steps
      process(bA);
      if (j + 2 < total) issue(bA);
      process(bB);
      if (j + 2 < total) process(bA);
    } else {
      for (int64_t j = 0; j < total; ++j) {
        issue(bA);
        process(bA);
      }
    }
  } else {
    for (int64_t r = r_begin; r < r_end; ++r) {
      int b;
      const U* row = row_ptr(r, b);
      RowAcc a = {false, false, Nk, -1};
      const U first = Nk > 0 ? row[0] : (U)0;
      for (int e = lane; e < Nk; e += kWave) visit<T>(a, row[e], first, e);
      finish_row(r, b, a, first);
    }
  }
  if (lane == 0) {
    if (cur_b >= 0) flush_len<T>(p.ws, cur_b, lmin, lmax);
    if (r_begin < r_end) atomicMax(reinterpret_cast<unsigned*>(p.ws + WS_MAXCLS), wave_max);
    if (wave_first_bad >= 0)
      atomicMin(reinterpret_cast<unsigned long long*>(p.ws + WS_FIRSTBAD), (unsigned long long)wave_first_bad);
  }
}

__global__ void mask_init_kernel(unsigned char* ws, int nb) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t == 0) {
    *reinterpret_cast<unsigned*>(ws + WS_MAXCLS) = 0u;
    *reinterpret_cast<unsigned long long*>(ws + WS_FIRSTBAD) = ~0ull;
  }
  int* len = reinterpret_cast<int*>(ws + WS_LEN);
  for (int b = t; b < nb; b += gridDim.x * blockDim.x) {
    len[2 * b] = INT_MAX;
    len[2 * b + 1] = -1;
  }
}

__global__ void mask_finalize_kernel(unsigned char* ws, int nb, int64_t rows, int is_bool, int32_t* kv_len_out) {
  // one block; thread 0 decides, all threads write kv_len_out
  __shared__ int overall_s;
  const int* len = reinterpret_cast<const int*>(ws + WS_LEN);
  if (threadIdx.x == 0) {
    int overall;
    if (rows == 0) overall = is_bool ? SAFE_MASK_ALL_VALID : SAFE_MASK_ZERO;
    else overall = (int)*reinterpret_cast<const unsigned*>(ws + WS_MAXCLS);
    if (overall == SAFE_MASK_KEY_PADDING) {
      for (int b = 0; b < nb; ++b)
        if (len[2 * b] != len[2 * b + 1]) { overall = SAFE_MASK_BLOCKED; break; }
    }
    const unsigned long long fb = *reinterpret_cast<const unsigned long long*>(ws + WS_FIRSTBAD);
    safe_mask_info info;
    info.verdict = overall <= SAFE_MASK_ROW_CONST ? 1 : 0;
    info.mask_class = overall;
    info.first_bad_row = fb == ~0ull ? -1 : (int64_t)fb;
    info.rows = rows;
    *reinterpret_cast<safe_mask_info*>(ws + WS_INFO) = info;
    overall_s = overall;
  }
  __syncthreads();
  if (kv_len_out != nullptr) {
    const bool pad = overall_s == SAFE_MASK_KEY_PADDING;
    for (int b = threadIdx.x; b < nb; b += blockDim.x) kv_len_out[b] = pad ? len[2 * b] : -1;
  }
}

template <class T>
hipError_t launch_scan(ScanParams& p, hipStream_t s) {
  // MASK_WAVES_PER_CU waves per CU (256 CUs), contiguous row ranges
  const int64_t max_waves = 256 * MASK_WAVES_PER_CU;
  int64_t waves = p.rows < max_waves ? p.rows : max_waves;
  if (waves < 1) waves = 1;
  p.rows_per_wave = (int)((p.rows + waves - 1) / waves);
  const int64_t wv = (p.rows + p.rows_per_wave - 1) / p.rows_per_wave;
  const int blocks = (int)((wv + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK);
  hipLaunchKernelGGL(mask_scan_kernel<T>, dim3(blocks), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

size_t mask_classify_workspace(const int64_t size[4]) {
  const size_t need = WS_LEN + 8 * (size_t)(size[0] > 0 ? size[0] : 1);
  return (need + 255) & ~(size_t)255;
}

int mask_classify_launch(const void* mask, int32_t dtype, const int64_t size[4], const int64_t stride[4],
                         uint32_t flags, safe_mask_info* info, uint8_t* row_class, int32_t* kv_len_out,
                         void* workspace, hipStream_t s) {
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const int nb = (int)(size[0] > 0 ? size[0] : 0);
  const int64_t rows = size[0] * size[1] * size[2];
  const int esize = dtype == SAFE_DT_BOOL ? 1 : (dtype == SAFE_DT_F32 ? 4 : 2);
  hipLaunchKernelGGL(mask_init_kernel, dim3(nb > 256 ? (nb + 255) / 256 : 1), dim3(256), 0, s, ws, nb);
  if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
  if (rows > 0) {
    if (rows > (int64_t)INT_MAX * 256) return SAFE_ERR_SHAPE;
    ScanParams p;
    p.mask = static_cast<const uint8_t*>(mask);
    p.s0 = stride[0]; p.s1 = stride[1]; p.s2 = stride[2];
    p.S1 = size[1]; p.S2 = size[2];
    p.rows = rows;
    p.Nk = (int)size[3];
    p.row_class = row_class;
    p.ws = ws;
    const bool base_ok = (reinterpret_cast<uintptr_t>(mask) & 15u) == 0;
    const bool strides_ok = ((stride[0] * esize) % 16 == 0 || size[0] == 1) &&
                            ((stride[1] * esize) % 16 == 0 || size[1] == 1) &&
                            ((stride[2] * esize) % 16 == 0 || size[2] == 1);
    p.vec = (base_ok && strides_ok) ? 1 : 0;
    hipError_t e;
    switch (dtype) {
      case SAFE_DT_BOOL: e = launch_scan<BoolT>(p, s); break;
      case SAFE_DT_BF16: e = launch_scan<Bf16T>(p, s); break;
      case SAFE_DT_F16: e = launch_scan<F16T>(p, s); break;
      default: e = launch_scan<F32T>(p, s); break;
    }
    if (e != hipSuccess) return SAFE_ERR_HIP;
  }
  hipLaunchKernelGGL(mask_finalize_kernel, dim3(1), dim3(256), 0, s, ws, nb, rows, dtype == SAFE_DT_BOOL ? 1 : 0,
                     kv_len_out);
  if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
  if (!(flags & SAFE_CLASSIFY_ASYNC)) {
    if (hipMemcpyAsync(info, ws + WS_INFO, sizeof(safe_mask_info), hipMemcpyDeviceToHost, s) != hipSuccess)
      return SAFE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SAFE_ERR_HIP;
  }
  return SAFE_OK;
}

}  // namespace safe
