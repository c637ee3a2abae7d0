// Internal helpers shared by the libsafe kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/safe.h"

namespace safe {

typedef unsigned short u16;
typedef unsigned int u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

// Workgroup id -> logical id such that consecutive logical ids run on the same XCD.
// The dispatcher places workgroup L on XCD L % 8; XCD x receives ceil/floor(total/8)
// workgroups, and its s-th one gets logical id (first id of x) + s.
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / kNumXcd, rem = total % kNumXcd;
  const int x = L % kNumXcd, s = L / kNumXcd;
  return x * per + (x < rem ? x : rem) + s;
}

// A wave-uniform pointer made explicitly uniform (both halves read from the first lane), so
// the compiler keeps it in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float pair -> packed bfloat16 (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, bf16x2));
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace safe
