// Sensitivity-weighted classifier-free guidance ("SAFE-DiT" Eq. 20, 21).
//
// out[b,i,:] = f_u[b,i,:] + gamma_i * (f_c[b,i,:] - f_u[b,i,:]) with gamma_i from the
// token's normalised sensitivity score (Eq. 20), from membership in S (the binary
// variant), or the global scale.  A streaming kernel: a workgroup owns 16 tokens of
// one image and walks their values as a flat run of 16-byte chunks, four per thread
// per step, both predictions loaded non-temporally before the results are stored.
// For the binary variant the workgroup finds which of its tokens are in S with one
// binary search of the ascending list plus a 16-entry map in LDS (the list values
// only decide membership, so out-of-range entries simply match nothing).
#include "common.h"

namespace safe {
namespace {

constexpr int GT = 16;    // tokens per workgroup
constexpr int GNT = 256;  // threads
constexpr int GU = 4;     // chunks per thread per step

struct CfgParams {
  const char* fc; const char* fu; char* out;
  int64_t sb, si;                 // byte strides of b and i
  const float* s; int64_t s_bs;
  const int32_t* idx; int k; int64_t idx_bs;
  int N, cpt, tiles_per_b;        // cpt: 16-byte chunks per token
  float g_ctx, g_sens;
};

__device__ __forceinline__ float bf16_lo(u32 w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

template <bool BF16>
__global__ __launch_bounds__(GNT) void sw_cfg_kernel(CfgParams p) {
  __shared__ float gamma[GT];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.tiles_per_b;
  const int i0 = (blockIdx.x % p.tiles_per_b) * GT;
  const int ntok = min(GT, p.N - i0);
  if (tid < GT) {
    float g = p.g_ctx;
    if (p.s != nullptr && tid < ntok) g = p.g_ctx + (p.g_sens - p.g_ctx) * p.s[(int64_t)b * p.s_bs + i0 + tid];
    gamma[tid] = g;
  }
  __syncthreads();
  if (p.idx != nullptr && p.k > 0 && tid < GT) {
    const int32_t* idx = p.idx + (int64_t)b * p.idx_bs;
    int lo = 0, hi = p.k;   // lower bound of i0 in the ascending list
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx[mid] < i0) lo = mid + 1; else hi = mid;
    }
    const int r = lo + tid;
    if (r < p.k) {
      const int j = idx[r];
      if (j >= i0 && j < i0 + ntok) gamma[j - i0] = p.g_sens;
    }
  }
  __syncthreads();

  const int total = ntok * p.cpt;
  const float inv_cpt = 1.0f / (float)p.cpt;
  for (int base = 0; base < total; base += GU * GNT) {
    u32x4 vc[GU], vu[GU];
    int tok[GU];
    int64_t off[GU];
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int c = base + u * GNT + tid;
      tok[u] = -1;
      if (c < total) {
        int t = (int)((float)c * inv_cpt);   // token of the chunk (t < 16): one correction
        if (t * p.cpt > c) --t;
        else if ((t + 1) * p.cpt <= c) ++t;
        tok[u] = t;
        off[u] = (int64_t)b * p.sb + (int64_t)(i0 + t) * p.si + (int64_t)(c - t * p.cpt) * 16;
        vc[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.fc + off[u]));
        vu[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.fu + off[u]));
      }
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      if (tok[u] < 0) continue;
      const float g = gamma[tok[u]];
      u32x4 r;
      if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float c0 = bf16_lo(vc[u][w]), c1 = bf16_hi(vc[u][w]);
          const float u0 = bf16_lo(vu[u][w]), u1 = bf16_hi(vu[u][w]);
          r[w] = pack_bf16x2(__builtin_fmaf(g, c0 - u0, u0), __builtin_fmaf(g, c1 - u1, u1));
        }
      } else {
        // whole-vector reinterpretation: a bit_cast of a single element of a vector value
        // has been miscompiled (the element index dropped), so none is used
        const f32x4 cf = __builtin_bit_cast(f32x4, vc[u]), uf = __builtin_bit_cast(f32x4, vu[u]);
        f32x4 rf;
#pragma unroll
        for (int w = 0; w < 4; ++w) rf[w] = __builtin_fmaf(g, cf[w] - uf[w], uf[w]);
        r = __builtin_bit_cast(u32x4, rf);
      }
      __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p.out + off[u]));
    }
  }
}

}  // namespace

// Enqueue the guidance kernel.  Arguments were validated by the caller.
int sw_cfg_launch(const safe_cfg_args* a, hipStream_t s) {
  if ((int64_t)a->B * a->N * a->C == 0) return SAFE_OK;
  const int esz = a->dtype == SAFE_DT_BF16 ? 2 : 4;
  CfgParams p;
  p.fc = static_cast<const char*>(a->f_c);
  p.fu = static_cast<const char*>(a->f_u);
  p.out = static_cast<char*>(a->out);
  p.sb = a->stride[0] * esz;
  p.si = a->stride[1] * esz;
  p.s = a->s;
  p.s_bs = a->s_bstride;
  p.idx = a->idx;
  p.k = a->k;
  p.idx_bs = a->idx_bstride;
  p.N = a->N;
  p.cpt = (int)((int64_t)a->C * esz / 16);
  p.tiles_per_b = (a->N + GT - 1) / GT;
  p.g_ctx = a->g_ctx;
  p.g_sens = a->g_sens;
  const int64_t grid = (int64_t)p.tiles_per_b * a->B;
  if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
  if (a->dtype == SAFE_DT_BF16) hipLaunchKernelGGL(sw_cfg_kernel<true>, dim3((unsigned)grid), dim3(GNT), 0, s, p);
  else hipLaunchKernelGGL(sw_cfg_kernel<false>, dim3((unsigned)grid), dim3(GNT), 0, s, p);
  return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
