// Global K/V assembly for SRSU ("SAFE-DiT" Eq. 14 and 16): the fresh rows of the
// sensitive set S are placed, in the original token order, over the cached
// context rows of the last anchor.
//
// Out of place: a workgroup owns 4 (packed rows) or 32 consecutive tokens of one
// sample.  It finds
// which of them are in S with one binary search of the ascending index list
// (lower bound of the first token) plus a 32-entry map in LDS, then streams each
// token's K and V rows from their single source to the output in 16-byte chunks.
// Every output byte is read once and written once.
// In place (output == cache): a workgroup copies one (packed rows) or 32 fresh rows to
// their tokens; context rows are not touched.
// Index entries outside [0, N) are skipped, so no index value can address
// memory outside the tensors.
#include "common.h"

namespace safe {
namespace {

constexpr int TOK = 32;
constexpr int NT = 256;

struct KvParams {
  const u16* kf; const u16* vf; int64_t fs0, fs1, fs2;
  const int32_t* idx; int64_t ibs;
  const u16* kc; const u16* vc; int64_t cs0, cs1, cs2;
  u16* ko; u16* vo; int64_t os0, os1, os2;
  int B, N, H, d8, nsel, blocks_per_b;
};

__global__ __launch_bounds__(NT) void kv_assemble_kernel(KvParams p) {
  __shared__ int src_row[TOK];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.blocks_per_b;
  const int j0 = (blockIdx.x % p.blocks_per_b) * TOK;
  const int32_t* idx = p.idx + (int64_t)b * p.ibs;

  if (tid < TOK) src_row[tid] = -1;
  __syncthreads();
  if (p.nsel > 0 && tid < TOK) {
    // lower bound of j0 in the ascending list (each of the 32 threads searches; cheap)
    int lo = 0, hi = p.nsel;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx[mid] < j0) lo = mid + 1; else hi = mid;
    }
    const int r = lo + tid;
    if (r < p.nsel) {
      const int j = idx[r];
      if (j >= j0 && j < j0 + TOK && j < p.N) src_row[j - j0] = r;
    }
  }
  __syncthreads();

  const int ntok = min(TOK, p.N - j0);
  const int cpr = p.H * p.d8;  // 16-byte chunks per token row
  for (int c = tid; c < cpr; c += NT) {
    const int hh = c / p.d8, part = c % p.d8;
    const int64_t fo = (int64_t)b * p.fs0 + (int64_t)hh * p.fs2 + part * 8;
    const int64_t co = (int64_t)b * p.cs0 + (int64_t)hh * p.cs2 + part * 8;
    const int64_t oo = (int64_t)b * p.os0 + (int64_t)hh * p.os2 + part * 8;
    constexpr int U = 8;
    for (int t0 = 0; t0 < ntok; t0 += U) {
      u32x4 kv[U], vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u;
        if (t < ntok) {
          const int r = src_row[t];
          const u16* ks = r >= 0 ? p.kf + fo + (int64_t)r * p.fs1 : p.kc + co + (int64_t)(j0 + t) * p.cs1;
          const u16* vs = r >= 0 ? p.vf + fo + (int64_t)r * p.fs1 : p.vc + co + (int64_t)(j0 + t) * p.cs1;
          kv[u] = ld16(ks);
          vv[u] = ld16(vs);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u;
        if (t < ntok) {
          st16(p.ko + oo + (int64_t)(j0 + t) * p.os1, kv[u]);
          st16(p.vo + oo + (int64_t)(j0 + t) * p.os1, vv[u]);
        }
      }
    }
  }
}

// Packed rows (stride_h == d for every tensor): a token's K (or V) row for all heads
// is one contiguous run of R = H*d/8 16-byte chunks.  A workgroup owns 4 tokens and
// walks their K rows, then their V rows, as one flat run of chunks: four chunks per
// thread per step (1024 consecutive chunks, 16 KB, per workgroup), every load of a
// step in flight before its stores, non-temporal on both sides since nothing is
// re-read.  (Measured on a plain 1 GiB copy: four 16-byte chunks in flight per thread
// stream at 5.85 TB/s, eight at 5.43, sixteen at 4.73; at the 160x160 grid 4 tokens
// per workgroup move 6.0 TB/s, 8 tokens 5.4, 16 tokens 4.9.)
constexpr int PTOK = 4;
constexpr int PU = 4;   // chunks per thread per step
// The packed in-place scatter moves 4 k H d bytes (236 MB at the 160x160 grid, rho 25%):
// one fresh row (2 x 288 chunks) per workgroup of 256 threads, two chunks per thread, reached
// 69% of 8 TB/s (42.8 us); 2, 4, 8 and 16 rows per workgroup 67, 63, 58 and 56%, 64- to
// 192-thread workgroups 63-69%.  At this size the launch and drain take a tenth of the time.
constexpr int SROWS = 1;     // fresh rows per workgroup
constexpr int SPU = 2;       // chunks per thread per step
constexpr int SNT = 256;     // threads per workgroup
__global__ __launch_bounds__(NT) void kv_assemble_packed_kernel(KvParams p) {
  __shared__ int src_row[PTOK];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.blocks_per_b;
  const int j0 = (blockIdx.x % p.blocks_per_b) * PTOK;
  const int32_t* idx = p.idx + (int64_t)b * p.ibs;
  if (tid < PTOK) src_row[tid] = -1;
  __syncthreads();
  if (p.nsel > 0 && tid < PTOK) {
    int lo = 0, hi = p.nsel;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx[mid] < j0) lo = mid + 1; else hi = mid;
    }
    const int r = lo + tid;
    if (r < p.nsel) {
      const int j = idx[r];
      if (j >= j0 && j < j0 + PTOK && j < p.N) src_row[j - j0] = r;
    }
  }
  __syncthreads();
  const int ntok = min(PTOK, p.N - j0);
  const int R = p.H * p.d8;          // 16-byte chunks per row
  const int per = ntok * R;          // chunks of one tensor in this workgroup
  const int total = 2 * per;
  const float inv_r = 1.0f / (float)R;
  const int64_t fb = (int64_t)b * p.fs0, cb = (int64_t)b * p.cs0, ob = (int64_t)b * p.os0;
  for (int base = 0; base < total; base += PU * NT) {
    u32x4 v[PU];
    u32x4* dst[PU];
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int c = base + u * NT + tid;
      dst[u] = nullptr;
      if (c < total) {
        const bool isv = c >= per;
        const int cc = isv ? c - per : c;
        int t = (int)((float)cc * inv_r);          // row of the chunk, t < PTOK: one correction
        if (t * R > cc) --t;
        else if ((t + 1) * R <= cc) ++t;
        const int ch = cc - t * R;
        const int r = src_row[t];
        const u16* src = r >= 0 ? (isv ? p.vf : p.kf) + fb + (int64_t)r * p.fs1
                                : (isv ? p.vc : p.kc) + cb + (int64_t)(j0 + t) * p.cs1;
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + ch);
        dst[u] = reinterpret_cast<u32x4*>((isv ? p.vo : p.ko) + ob + (int64_t)(j0 + t) * p.os1) + ch;
      }
    }
#pragma unroll
    for (int u = 0; u < PU; ++u)
      if (dst[u] != nullptr) __builtin_nontemporal_store(v[u], dst[u]);
  }
}

__global__ __launch_bounds__(NT) void kv_scatter_kernel(KvParams p) {
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.blocks_per_b;
  const int r0 = (blockIdx.x % p.blocks_per_b) * TOK;
  const int32_t* idx = p.idx + (int64_t)b * p.ibs;
  const int nr = min(TOK, p.nsel - r0);
  const int cpr = p.H * p.d8;
  for (int c = tid; c < cpr; c += NT) {
    const int hh = c / p.d8, part = c % p.d8;
    const int64_t fo = (int64_t)b * p.fs0 + (int64_t)hh * p.fs2 + part * 8;
    const int64_t oo = (int64_t)b * p.os0 + (int64_t)hh * p.os2 + part * 8;
    constexpr int U = 8;
    for (int t0 = 0; t0 < nr; t0 += U) {
      u32x4 kv[U], vv[U];
      int dst[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + t0 + u;
        dst[u] = -1;
        if (t0 + u < nr) {
          const int j = idx[r];
          if (j >= 0 && j < p.N) {
            dst[u] = j;
            kv[u] = ld16(p.kf + fo + (int64_t)r * p.fs1);
            vv[u] = ld16(p.vf + fo + (int64_t)r * p.fs1);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (dst[u] >= 0) {
          st16(p.ko + oo + (int64_t)dst[u] * p.os1, kv[u]);
          st16(p.vo + oo + (int64_t)dst[u] * p.os1, vv[u]);
        }
      }
    }
  }
}

// In place with packed rows: a workgroup owns SROWS fresh rows of one sample and copies
// their K rows, then their V rows, to the tokens the index list names, as one flat run of
// 16-byte chunks (SPU per thread per step, non-temporal on both sides), so at the 160x160
// grid 12800 workgroups stream instead of 400.  Rows whose token is outside [0, N) are
// skipped.
__global__ __launch_bounds__(SNT) void kv_scatter_packed_kernel(KvParams p) {
  __shared__ int dst_tok[SROWS];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.blocks_per_b;
  const int r0 = (blockIdx.x % p.blocks_per_b) * SROWS;
  const int nr = min(SROWS, p.nsel - r0);
  if (tid < SROWS) {
    const int j = tid < nr ? p.idx[(int64_t)b * p.ibs + r0 + tid] : -1;
    dst_tok[tid] = (j >= 0 && j < p.N) ? j : -1;
  }
  __syncthreads();
  const int R = p.H * p.d8;          // 16-byte chunks per row
  const int per = nr * R;            // chunks of one tensor in this workgroup
  const int total = 2 * per;
  const float inv_r = 1.0f / (float)R;
  const int64_t fb = (int64_t)b * p.fs0, ob = (int64_t)b * p.os0;
  for (int base = 0; base < total; base += SPU * SNT) {
    u32x4 v[SPU];
    u32x4* dst[SPU];
#pragma unroll
    for (int u = 0; u < SPU; ++u) {
      const int c = base + u * SNT + tid;
      dst[u] = nullptr;
      if (c < total) {
        const bool isv = c >= per;
        const int cc = isv ? c - per : c;
        int t = (int)((float)cc * inv_r);          // row of the chunk, t < SROWS: one correction
        if (t * R > cc) --t;
        else if ((t + 1) * R <= cc) ++t;
        const int ch = cc - t * R;
        const int j = dst_tok[t];
        if (j >= 0) {
          const u16* src = (isv ? p.vf : p.kf) + fb + (int64_t)(r0 + t) * p.fs1;
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + ch);
          dst[u] = reinterpret_cast<u32x4*>((isv ? p.vo : p.ko) + ob + (int64_t)j * p.os1) + ch;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < SPU; ++u)
      if (dst[u] != nullptr) __builtin_nontemporal_store(v[u], dst[u]);
  }
}

// Source map of the fused global K/V read: src[b, j] = r when idx[b, r] == j, else -1.
// A workgroup owns NT consecutive tokens of one sample: one binary search (lower bound
// of its first token in the ascending list) finds the entries that land in its range,
// which are then consecutive in the list (at most NT of them).
__global__ __launch_bounds__(NT) void kv_srcmap_kernel(KvParams p, int32_t* src) {
  __shared__ int map[NT];
  __shared__ int lo_s;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.blocks_per_b;
  const int t0 = (blockIdx.x % p.blocks_per_b) * NT;
  const int32_t* idx = p.idx + (int64_t)b * p.ibs;
  map[tid] = -1;
  if (tid == 0) {
    int lo = 0, hi = p.nsel;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx[mid] < t0) lo = mid + 1;
      else hi = mid;
    }
    lo_s = lo;
  }
  __syncthreads();
  const int r = lo_s + tid;
  if (r < p.nsel) {
    const int j = idx[r];
    if (j >= t0 && j < t0 + NT && j < p.N) map[j - t0] = r;
  }
  __syncthreads();
  const int j = t0 + tid;
  if (j < p.N) src[(int64_t)b * p.N + j] = map[tid];
}

}  // namespace

int kv_source_map_launch(const safe_kv_args* a, int32_t* src, hipStream_t s) {
  KvParams p = {};
  p.idx = a->idx;
  p.ibs = a->idx_bstride;
  p.B = a->B; p.N = a->N; p.nsel = a->nsel;
  p.blocks_per_b = (a->N + NT - 1) / NT;
  const int64_t grid = (int64_t)p.blocks_per_b * a->B;
  if (grid == 0) return SAFE_OK;
  if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
  hipLaunchKernelGGL(kv_srcmap_kernel, dim3((unsigned)grid), dim3(NT), 0, s, p, src);
  return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

int kv_assemble_launch(const safe_kv_args* a, bool in_place, hipStream_t s) {
  KvParams p;
  p.kf = static_cast<const u16*>(a->k_fresh);
  p.vf = static_cast<const u16*>(a->v_fresh);
  p.fs0 = a->fresh_stride[0]; p.fs1 = a->fresh_stride[1]; p.fs2 = a->fresh_stride[2];
  p.idx = a->idx;
  p.ibs = a->idx_bstride;
  p.kc = static_cast<const u16*>(a->k_cache);
  p.vc = static_cast<const u16*>(a->v_cache);
  p.cs0 = a->cache_stride[0]; p.cs1 = a->cache_stride[1]; p.cs2 = a->cache_stride[2];
  p.ko = static_cast<u16*>(a->k_out);
  p.vo = static_cast<u16*>(a->v_out);
  p.os0 = a->out_stride[0]; p.os1 = a->out_stride[1]; p.os2 = a->out_stride[2];
  p.B = a->B; p.N = a->N; p.H = a->H; p.d8 = a->d / 8; p.nsel = a->nsel;
  if (in_place) {
    if (a->nsel == 0) return SAFE_OK;
    const bool packed = a->fresh_stride[2] == a->d && a->out_stride[2] == a->d &&
                        (int64_t)a->H * (a->d / 8) * SROWS * 2 < 0x7fffffff;
    const int rows = packed ? SROWS : TOK;
    p.blocks_per_b = (a->nsel + rows - 1) / rows;
    const int64_t grid = (int64_t)p.blocks_per_b * a->B;
    if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
    if (packed) hipLaunchKernelGGL(kv_scatter_packed_kernel, dim3((unsigned)grid), dim3(SNT), 0, s, p);
    else hipLaunchKernelGGL(kv_scatter_kernel, dim3((unsigned)grid), dim3(NT), 0, s, p);
  } else {
    const bool packed = a->fresh_stride[2] == a->d && a->cache_stride[2] == a->d && a->out_stride[2] == a->d &&
                        (int64_t)a->H * (a->d / 8) * PTOK * 2 < 0x7fffffff;
    if (packed) {
      p.blocks_per_b = (a->N + PTOK - 1) / PTOK;
      const int64_t grid = (int64_t)p.blocks_per_b * a->B;
      if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
      hipLaunchKernelGGL(kv_assemble_packed_kernel, dim3((unsigned)grid), dim3(NT), 0, s, p);
      return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
    }
    p.blocks_per_b = (a->N + TOK - 1) / TOK;
    const int64_t grid = (int64_t)p.blocks_per_b * a->B;
    if (grid > 0x7fffffff) return SAFE_ERR_SHAPE;
    hipLaunchKernelGGL(kv_assemble_kernel, dim3((unsigned)grid), dim3(NT), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? SAFE_OK : SAFE_ERR_HIP;
}

}  // namespace safe
