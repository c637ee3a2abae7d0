// Measurement aids beside the method's kernels: the rates the chip itself sustains, which the
// method's kernels are read against.
//
// Matrix-core rate probe: the MFMA throughput on random bf16 operands with nothing else
// running.  On MI355X the attention and linear kernels are limited by the board's power cap
// rather than by issue, and this rate (which also drops under the cap) is their ceiling.
//
// Every lane draws eight A and eight B fragments (8 bf16 each, uniform in [-2, 2)) from a
// counter-based hash of (seed, global lane, fragment), keeps them in registers, and each round
// issues 16 MFMAs into four independent accumulators, pairing A fragment q % 8 with B fragment
// (q + q / 8) % 8 so that consecutive instructions always see different operands.  The lane
// writes the sum of its accumulator elements, which keeps every product live.
#include <type_traits>

#include "common.h"

namespace safe {
namespace {

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {   // a 32-bit integer mixer
  x ^= x >> 16; x *= 0x7feb352dU;
  x ^= x >> 15; x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// bf16 value of draw (seed, lane, f, e): (u / 2^24 - 0.5) * 4, rounded to nearest even
__device__ __forceinline__ bf16x8 probe_fragment(uint32_t seed, uint32_t lane_g, int f) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = probe_hash(seed ^ probe_hash(lane_g * 64u + (uint32_t)(f * 8 + e)));
    v[e] = ((float)(h >> 8) * (1.0f / 16777216.0f) - 0.5f) * 4.0f;
  }
  u32x4 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  w[2] = pack_bf16x2(v[4], v[5]);
  w[3] = pack_bf16x2(v[6], v[7]);
  return as_bf16x8(w);
}

template <int SHAPE>
__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(int iters, uint32_t seed, float* out) {
  typedef typename std::conditional<SHAPE == 32, f32x16, f32x4>::type Acc;
  constexpr int NE = SHAPE == 32 ? 16 : 4;
  const uint32_t lane_g = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    a[f] = probe_fragment(seed, lane_g, f);
    b[f] = probe_fragment(seed, lane_g, 8 + f);
  }
  Acc acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = Acc{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (SHAPE == 32)
        acc[q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q & 7], b[(q + (q >> 3)) & 7], acc[q & 3], 0, 0, 0);
      else
        acc[q & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q & 7], b[(q + (q >> 3)) & 7], acc[q & 3], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < NE; ++e) s += acc[c][e];
  out[lane_g] = s;
}

// Streaming probe: every 16-byte chunk of the source read once with non-temporal loads, four
// chunks in flight per thread (grid-stride: chunk c belongs to thread c mod the thread count),
// and either xor-folded into one word per thread (read) or stored to the same offset of the
// destination (copy).  The read form is the box's streaming-read bandwidth that the classifier
// is read against; the copy form the read+write rate the K/V assembly is read against.
template <bool COPY>
__global__ __launch_bounds__(256) void hbm_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t nchunks, uint32_t* __restrict__ out) {
  constexpr int U = 4;
  const int64_t T = (int64_t)gridDim.x * 256;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0u;
  int64_t c = g;
  for (; c + (U - 1) * T < nchunks; c += U * T) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + c + u * T);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (COPY) __builtin_nontemporal_store(v[u], dst + c + u * T);
      else x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
  }
  for (; c < nchunks; c += T) {
    const u32x4 v = __builtin_nontemporal_load(src + c);
    if constexpr (COPY) __builtin_nontemporal_store(v, dst + c);
    else x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if constexpr (!COPY) out[g] = x;
}

}  // namespace

// Arguments were validated by the caller.
int hbm_probe_launch(int mode, const void* src, void* dst, int64_t bytes, int blocks, uint32_t* out, hipStream_t s) {
  const int64_t nchunks = bytes / 16;
  const u32x4* in = reinterpret_cast<const u32x4*>(src);
  if (mode == 1)
    hipLaunchKernelGGL(hbm_probe_kernel<true>, dim3(blocks), dim3(256), 0, s, in, reinterpret_cast<u32x4*>(dst), nchunks,
                       out);
  else
    hipLaunchKernelGGL(hbm_probe_kernel<false>, dim3(blocks), dim3(256), 0, s, in, nullptr, nchunks, out);
  return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

// Arguments were validated by the caller.
int mfma_probe_launch(int shape, int iters, int blocks, uint32_t seed, float* out, hipStream_t s) {
  if (shape == 32) hipLaunchKernelGGL(mfma_probe_kernel<32>, dim3(blocks), dim3(256), 0, s, iters, seed, out);
  else hipLaunchKernelGGL(mfma_probe_kernel<16>, dim3(blocks), dim3(256), 0, s, iters, seed, out);
  return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
