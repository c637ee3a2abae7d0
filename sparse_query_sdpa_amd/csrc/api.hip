// libsafe C ABI: argument validation (host only, before any HIP call) and dispatch.
#include <math.h>
#include <string.h>

#include <atomic>
#include <vector>

#include "common.h"

namespace safe {
int attn_fwd_launch(const safe_attn_args* a, float scale, hipStream_t stream);
int64_t attn_workspace_bytes(const safe_attn_args* a);
int attn_plan(const safe_attn_args* a, safe_attn_plan_info* out);
int sw_cfg_launch(const safe_cfg_args* a, hipStream_t stream);
int linear_launch(const safe_linear_args* a, hipStream_t stream);
int mfma_probe_launch(int shape, int iters, int blocks, uint32_t seed, float* out, hipStream_t stream);
int hbm_probe_launch(int mode, const void* src, void* dst, int64_t bytes, int blocks, uint32_t* out, hipStream_t stream);
int kv_assemble_launch(const safe_kv_args* a, bool in_place, hipStream_t stream);
int kv_source_map_launch(const safe_kv_args* a, int32_t* src, hipStream_t stream);
int mask_classify_launch(const void* mask, int32_t dtype, const int64_t size[4], const int64_t stride[4],
                         uint32_t flags, safe_mask_info* info, uint8_t* row_class, int32_t* kv_len_out,
                         void* workspace, hipStream_t stream);
size_t mask_classify_workspace(const int64_t size[4]);
int pcsp_launch(const safe_pcsp_args* a, float scale, void* workspace, size_t ws_bytes, hipStream_t stream);
size_t pcsp_select_workspace(const safe_pcsp_args* a);
size_t pcsp_accum_workspace(const safe_pcsp_args* a);
}  // namespace safe

using namespace safe;

namespace {

bool supported_head_dim(int d) { return d == 32 || d == 64 || d == 72 || d == 96 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A [B, N, H, d] 16-bit tensor read or written in 16-byte chunks: every row start
// must be 16-byte aligned (strides multiples of 8 elements) and strides >= 0.
int check_bnhd(const void* p, const int64_t st[3], bool need) {
  if (p == nullptr) return need ? SAFE_ERR_NULL : SAFE_OK;
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return SAFE_ERR_SHAPE;
    if (st[i] % 8 != 0) return SAFE_ERR_ALIGN;
  }
  if (!aligned16(p)) return SAFE_ERR_ALIGN;
  return SAFE_OK;
}

float resolve_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / sqrtf((float)d); }

template <typename T>
int copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t s) {
  dst.resize(n);
  if (n == 0) return SAFE_OK;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s) != hipSuccess) return SAFE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SAFE_ERR_HIP;
  return SAFE_OK;
}

// SAFE_FLAG_CHECK: index lists ascending? (attention only needs range; assembly
// needs range and distinctness, which ascending order guarantees.)
int check_rows(const int32_t* rows, int B, int n, int64_t bstride, int limit, bool ascending, hipStream_t s) {
  const int nb = bstride == 0 ? 1 : B;
  for (int b = 0; b < nb; ++b) {
    std::vector<int32_t> h;
    int st = copy_to_host(h, rows + (int64_t)b * bstride, (size_t)n, s);
    if (st != SAFE_OK) return st;
    for (int i = 0; i < n; ++i) {
      if (h[i] < 0 || h[i] >= limit) return SAFE_ERR_RANGE;
      if (ascending && i > 0 && h[i] <= h[i - 1]) return SAFE_ERR_RANGE;
    }
  }
  return SAFE_OK;
}

int check_lengths(const int32_t* len, int B, int limit, hipStream_t s) {
  std::vector<int32_t> h;
  int st = copy_to_host(h, len, (size_t)B, s);
  if (st != SAFE_OK) return st;
  for (int b = 0; b < B; ++b)
    if (h[b] < 0 || h[b] > limit) return SAFE_ERR_RANGE;
  return SAFE_OK;
}

}  // namespace

extern "C" {

int safe_abi_version(void) { return SAFE_ABI_VERSION; }

const char* safe_status_str(int status) {
  switch (status) {
    case SAFE_OK: return "SAFE_OK";
    case SAFE_ERR_NULL: return "SAFE_ERR_NULL: a required pointer is NULL";
    case SAFE_ERR_SHAPE: return "SAFE_ERR_SHAPE: sizes or strides inconsistent or out of range";
    case SAFE_ERR_DTYPE: return "SAFE_ERR_DTYPE: unknown dtype code";
    case SAFE_ERR_RANGE: return "SAFE_ERR_RANGE: a scalar or device value is out of range";
    case SAFE_ERR_UNSUPPORTED: return "SAFE_ERR_UNSUPPORTED: valid request the library does not implement";
    case SAFE_ERR_WORKSPACE: return "SAFE_ERR_WORKSPACE: workspace missing or too small";
    case SAFE_ERR_HIP: return "SAFE_ERR_HIP: a HIP runtime call failed";
    case SAFE_ERR_ALIGN: return "SAFE_ERR_ALIGN: pointer or stride breaks 16-byte alignment";
    default: return "unknown status";
  }
}

// Size, scale and flag checks shared by the call and its workspace query (no pointers read).
static int check_attn_sizes(const safe_attn_args* a) {
  if (a == nullptr) return SAFE_ERR_NULL;
  if (a->B < 0 || a->H < 0 || a->Nq < 0 || a->Nk < 0 || a->n_rows < 0) return SAFE_ERR_SHAPE;
  if (!supported_head_dim(a->d)) return SAFE_ERR_UNSUPPORTED;
  if (!(isfinite(a->scale))) return SAFE_ERR_RANGE;
  if (a->q_rows == nullptr && a->n_rows != a->Nq) return SAFE_ERR_SHAPE;
  if (a->q_rows == nullptr && (a->flags & SAFE_ATTN_SCATTER_OUT)) return SAFE_ERR_SHAPE;
  if (a->q_rows != nullptr && a->q_rows_bstride < 0) return SAFE_ERR_SHAPE;
  if (a->q_rows != nullptr && a->q_rows_bstride != 0 && a->q_rows_bstride < a->n_rows) return SAFE_ERR_SHAPE;
  if (a->flags & ~(SAFE_ATTN_SCATTER_OUT | SAFE_FLAG_CHECK)) return SAFE_ERR_RANGE;
  if (a->workspace_bytes < 0) return SAFE_ERR_WORKSPACE;
  if (a->kv_src != nullptr) {   // fused global K/V: no key lengths, no mask
    if (a->kv_len != nullptr || a->mask != nullptr) return SAFE_ERR_UNSUPPORTED;
    if (a->n_fresh < 0 || a->kv_src_bstride < 0 || (a->kv_src_bstride != 0 && a->kv_src_bstride < a->Nk))
      return SAFE_ERR_SHAPE;
  }
  if (a->mask != nullptr) {
    if (a->mask_dtype < SAFE_DT_BOOL || a->mask_dtype > SAFE_DT_F32) return SAFE_ERR_DTYPE;
    if (a->kv_len != nullptr) return SAFE_ERR_UNSUPPORTED;
    const int esz = a->mask_dtype == SAFE_DT_BOOL ? 1 : (a->mask_dtype == SAFE_DT_F32 ? 4 : 2);
    for (int i = 0; i < 3; ++i) {
      if (a->mask_stride[i] < 0) return SAFE_ERR_SHAPE;
      if (a->mask_stride[i] * esz % 16 != 0) return SAFE_ERR_ALIGN;
    }
  }
  return SAFE_OK;
}


int64_t safe_attn_workspace_bytes(const safe_attn_args* a) {
  const int st = check_attn_sizes(a);
  if (st != SAFE_OK) return st;
  return attn_workspace_bytes(a);
}

int safe_attn_plan(const safe_attn_args* a, safe_attn_plan_info* out) {
  if (out == nullptr) return SAFE_ERR_NULL;
  const int st = check_attn_sizes(a);
  if (st != SAFE_OK) return st;
  return attn_plan(a, out);
}

// Every host-side check of an attention call (sizes, flags, pointers, alignment).
static int check_attn_call(const safe_attn_args* a) {
  int st = check_attn_sizes(a);
  if (st != SAFE_OK) return st;
  if (a->workspace != nullptr && !aligned16(a->workspace)) return SAFE_ERR_ALIGN;
  if (a->mask != nullptr && !aligned16(a->mask)) return SAFE_ERR_ALIGN;
  const bool work = (int64_t)a->B * a->H * a->n_rows > 0;
  if ((st = check_bnhd(a->q, a->q_stride, work)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->k, a->k_stride, work && a->Nk > 0)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->v, a->v_stride, work && a->Nk > 0)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->o, a->o_stride, work)) != SAFE_OK) return st;
  if (a->kv_src != nullptr) {
    const bool fresh = work && a->Nk > 0 && a->n_fresh > 0;
    if ((st = check_bnhd(a->k_fresh, a->fresh_stride, fresh)) != SAFE_OK) return st;
    if ((st = check_bnhd(a->v_fresh, a->fresh_stride, fresh)) != SAFE_OK) return st;
  }
  if (!work) return SAFE_OK;
  // key/value token strides: the kernel addresses a 64-key tile with 32-bit byte offsets
  // (63 rows of 2 * stride bytes plus a row), so strides stay below 2^25 elements
  if (a->k_stride[1] >= (int64_t(1) << 25) || a->v_stride[1] >= (int64_t(1) << 25)) return SAFE_ERR_UNSUPPORTED;
  return SAFE_OK;
}

int safe_attn_fwd(const safe_attn_args* a, void* stream) {
  int st = check_attn_call(a);
  if (st != SAFE_OK) return st;
  if ((int64_t)a->B * a->H * a->n_rows == 0) return SAFE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->flags & SAFE_FLAG_CHECK) {
    if (a->q_rows != nullptr &&
        (st = check_rows(a->q_rows, a->B, a->n_rows, a->q_rows_bstride, a->Nq, false, s)) != SAFE_OK)
      return st;
    if (a->kv_len != nullptr && (st = check_lengths(a->kv_len, a->B, a->Nk, s)) != SAFE_OK) return st;
  }
  return attn_fwd_launch(a, resolve_scale(a->scale, a->d), s);
}

// ---- safe_attn_fwd_noalloc: the split partials in a static device array ----------------

// The scratch of the allocation-free attention entry point.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is resolved once per device
// with hipGetSymbolAddress and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[SAFE_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxScratchDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// Device address of this device's copy of `scratch` (resolved on the first call on the
// device, with the device current; racing first calls store the same address).
static int current_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAFE_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return SAFE_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SAFE_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SAFE_OK;
}

int safe_attn_fwd_noalloc(const safe_attn_args* a, void* stream) {
  if (a == nullptr) return SAFE_ERR_NULL;
  if (a->workspace != nullptr || a->workspace_bytes != 0) return SAFE_ERR_WORKSPACE;
  if (a->flags & SAFE_FLAG_CHECK) return SAFE_ERR_UNSUPPORTED;
  int st = check_attn_call(a);
  if (st != SAFE_OK) return st;
  if ((int64_t)a->B * a->H * a->n_rows == 0) return SAFE_OK;
  safe_attn_args c = *a;
  if ((st = current_scratch(&c.workspace)) != SAFE_OK) return st;
  c.workspace_bytes = (int64_t)SAFE_NOALLOC_SCRATCH_BYTES;
  // the plan takes a split only when its partials fit the array; checked, not assumed
  safe_attn_plan_info plan;
  if ((st = attn_plan(&c, &plan)) != SAFE_OK) return st;
  if (plan.workspace_bytes > (int64_t)SAFE_NOALLOC_SCRATCH_BYTES) return SAFE_ERR_WORKSPACE;
  return attn_fwd_launch(&c, resolve_scale(c.scale, c.d), static_cast<hipStream_t>(stream));
}

// ---- safe_sdpa: the Eq. 8 rewrite as one call ------------------------------------------

// Stored sizes and element strides of the mask of an attention call: a zero stride marks
// a broadcast dimension, which is stored with size 1; keys are contiguous.
static void mask_geometry(const safe_attn_args* a, int64_t size[4], int64_t stride[4]) {
  const int64_t full[3] = {a->B, a->H, a->Nq};
  for (int i = 0; i < 3; ++i) {
    size[i] = a->mask_stride[i] == 0 ? 1 : full[i];
    stride[i] = a->mask_stride[i];
  }
  size[3] = a->Nk;
  stride[3] = 1;
}

// Layout of safe_sdpa's scratch: the classifier's workspace, its per-stored-sample key
// lengths, and (for a mask shared by the batch) those lengths repeated for every sample.
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static size_t sdpa_scratch(const safe_attn_args* a, const int64_t size[4], size_t* off_len, size_t* off_rep) {
  *off_len = align256(mask_classify_workspace(size));
  *off_rep = *off_len + align256((size_t)size[0] * sizeof(int32_t));
  return *off_rep + align256((size_t)a->B * sizeof(int32_t));
}

static __global__ void kv_len_repeat_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[0];
}

int safe_sdpa(const safe_attn_args* a, void* classify_ws, size_t* classify_ws_bytes, safe_sdpa_info* info,
              void* stream) {
  if (a == nullptr) return SAFE_ERR_NULL;
  if (info != nullptr) *info = safe_sdpa_info{SAFE_ROUTE_NO_MASK, -1, -1};
  // the mask-free call must be valid whatever the route: check it before any scan
  safe_attn_args c = *a;
  c.mask = nullptr;
  int st = check_attn_call(&c);
  if (st != SAFE_OK) return st;
  int64_t size[4] = {0, 0, 0, 0}, stride[4] = {0, 0, 0, 1};
  size_t off_len = 0, off_rep = 0, need = 0;
  if (a->mask != nullptr) {
    if (a->kv_len != nullptr || a->kv_src != nullptr) return SAFE_ERR_UNSUPPORTED;
    if (a->mask_dtype < SAFE_DT_BOOL || a->mask_dtype > SAFE_DT_F32) return SAFE_ERR_DTYPE;
    for (int i = 0; i < 3; ++i)
      if (a->mask_stride[i] < 0) return SAFE_ERR_SHAPE;
    mask_geometry(a, size, stride);
    need = sdpa_scratch(a, size, &off_len, &off_rep);
  }
  if (classify_ws == nullptr && classify_ws_bytes != nullptr) {   // size query: nothing runs
    *classify_ws_bytes = need;
    return SAFE_OK;
  }
  if (a->mask == nullptr) return safe_attn_fwd(a, stream);
  if (classify_ws == nullptr) return SAFE_ERR_WORKSPACE;
  if (classify_ws_bytes != nullptr && *classify_ws_bytes < need) return SAFE_ERR_WORKSPACE;
  if (!aligned16(classify_ws)) return SAFE_ERR_ALIGN;

  char* ws = static_cast<char*>(classify_ws);
  int32_t* len = reinterpret_cast<int32_t*>(ws + off_len);
  int32_t* rep = reinterpret_cast<int32_t*>(ws + off_rep);
  size_t cls_bytes = mask_classify_workspace(size);
  safe_mask_info mi;
  st = safe_mask_classify(a->mask, a->mask_dtype, size, stride, 0, &mi, nullptr, len, ws, &cls_bytes, stream);
  if (st != SAFE_OK) return st;
  int route = SAFE_ROUTE_MASK;
  c = *a;
  if (mi.verdict) {
    route = SAFE_ROUTE_NO_MASK;
    c.mask = nullptr;
  } else if (mi.mask_class == SAFE_MASK_KEY_PADDING) {
    route = SAFE_ROUTE_KV_LEN;
    c.mask = nullptr;
    c.kv_len = len;
    if (size[0] != a->B && a->B > 0) {   // one mask batch row serves every sample
      hipLaunchKernelGGL(kv_len_repeat_kernel, dim3((a->B + 255) / 256), dim3(256), 0,
                         static_cast<hipStream_t>(stream), len, rep, a->B);
      if (hipGetLastError() != hipSuccess) return SAFE_ERR_HIP;
      c.kv_len = rep;
    }
  }
  if (info != nullptr) *info = safe_sdpa_info{route, mi.mask_class, mi.first_bad_row};
  return safe_attn_fwd(&c, stream);
}

int safe_kv_assemble(const safe_kv_args* a, void* stream) {
  if (a == nullptr) return SAFE_ERR_NULL;
  if (a->B < 0 || a->N < 0 || a->H < 0 || a->d < 0 || a->nsel < 0) return SAFE_ERR_SHAPE;
  if (a->d % 8 != 0) return SAFE_ERR_ALIGN;
  if (a->nsel > a->N) return SAFE_ERR_SHAPE;
  if (a->idx_bstride < 0 || (a->idx_bstride != 0 && a->idx_bstride < a->nsel)) return SAFE_ERR_SHAPE;
  if (a->flags & ~SAFE_FLAG_CHECK) return SAFE_ERR_RANGE;
  const bool any = (int64_t)a->B * a->N * a->H * a->d > 0;
  const bool sel = any && a->nsel > 0;
  int st;
  if ((st = check_bnhd(a->k_cache, a->cache_stride, any)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->v_cache, a->cache_stride, any)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->k_out, a->out_stride, any)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->v_out, a->out_stride, any)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->k_fresh, a->fresh_stride, sel)) != SAFE_OK) return st;
  if ((st = check_bnhd(a->v_fresh, a->fresh_stride, sel)) != SAFE_OK) return st;
  if (sel && a->idx == nullptr) return SAFE_ERR_NULL;
  if (!any) return SAFE_OK;
  const bool k_same = a->k_out == a->k_cache, v_same = a->v_out == a->v_cache;
  const bool same_strides = memcmp(a->out_stride, a->cache_stride, sizeof(a->out_stride)) == 0;
  if (k_same != v_same) return SAFE_ERR_SHAPE;            // half in place is not supported
  if (k_same && !same_strides) return SAFE_ERR_SHAPE;     // aliasing with different strides
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((a->flags & SAFE_FLAG_CHECK) && sel &&
      (st = check_rows(a->idx, a->B, a->nsel, a->idx_bstride, a->N, true, s)) != SAFE_OK)
    return st;
  return kv_assemble_launch(a, k_same, s);
}

int safe_kv_source_map(const safe_kv_args* a, int32_t* kv_src, void* stream) {
  if (a == nullptr) return SAFE_ERR_NULL;
  if (a->B < 0 || a->N < 0 || a->nsel < 0 || a->nsel > a->N) return SAFE_ERR_SHAPE;
  if (a->idx_bstride < 0 || (a->idx_bstride != 0 && a->idx_bstride < a->nsel)) return SAFE_ERR_SHAPE;
  if (a->flags & ~SAFE_FLAG_CHECK) return SAFE_ERR_RANGE;
  if ((int64_t)a->B * a->N == 0) return SAFE_OK;
  if (kv_src == nullptr || (a->nsel > 0 && a->idx == nullptr)) return SAFE_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st;
  if ((a->flags & SAFE_FLAG_CHECK) && a->nsel > 0 &&
      (st = check_rows(a->idx, a->B, a->nsel, a->idx_bstride, a->N, true, s)) != SAFE_OK)
    return st;
  return kv_source_map_launch(a, kv_src, s);
}

int safe_mask_classify(const void* mask, int32_t dtype, const int64_t size[4], const int64_t stride[4],
                       uint32_t flags, safe_mask_info* info, uint8_t* row_class, int32_t* kv_len_out,
                       void* workspace, size_t* workspace_bytes, void* stream) {
  if (size == nullptr || stride == nullptr) return SAFE_ERR_NULL;
  if (dtype < SAFE_DT_BOOL || dtype > SAFE_DT_F32) return SAFE_ERR_DTYPE;
  for (int i = 0; i < 4; ++i)
    if (size[i] < 0 || stride[i] < 0) return SAFE_ERR_SHAPE;
  if (size[3] > 1 && stride[3] != 1) return SAFE_ERR_SHAPE;
  if (size[0] > 0x7fffffff || size[3] > 0x7fffffff) return SAFE_ERR_SHAPE;
  if (flags & ~SAFE_CLASSIFY_ASYNC) return SAFE_ERR_RANGE;
  const size_t need = mask_classify_workspace(size);
  if (workspace == nullptr) {
    if (workspace_bytes == nullptr) return SAFE_ERR_WORKSPACE;
    *workspace_bytes = need;
    return SAFE_OK;
  }
  if (workspace_bytes != nullptr && *workspace_bytes < need) return SAFE_ERR_WORKSPACE;
  if (!(flags & SAFE_CLASSIFY_ASYNC) && info == nullptr) return SAFE_ERR_NULL;
  const int64_t rows = size[0] * size[1] * size[2];
  if (rows > 0 && size[3] > 0 && mask == nullptr) return SAFE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return SAFE_ERR_ALIGN;
  return mask_classify_launch(mask, dtype, size, stride, flags, info, row_class, kv_len_out, workspace,
                              static_cast<hipStream_t>(stream));
}

int safe_pcsp_select(const safe_pcsp_args* a, void* workspace, size_t* workspace_bytes, void* stream) {
  if (a == nullptr) return SAFE_ERR_NULL;
  const uint32_t ops = a->flags & (SAFE_PCSP_ACCUM | SAFE_PCSP_SELECT);
  if (ops == 0 || (a->flags & ~(SAFE_PCSP_ACCUM | SAFE_PCSP_SELECT))) return SAFE_ERR_RANGE;
  if (a->B < 0 || a->N < 0 || a->M < 0 || a->H < 0) return SAFE_ERR_SHAPE;
  const bool sel = (a->flags & SAFE_PCSP_SELECT) != 0;
  const bool accum = (a->flags & SAFE_PCSP_ACCUM) != 0;
  // workspace == NULL with a size pointer is a query (both uses share one buffer:
  // the accumulation's per-head-group sums are consumed before the selection runs)
  const size_t need_sel = pcsp_select_workspace(a);
  const size_t need_acc = accum ? pcsp_accum_workspace(a) : 0;
  if (workspace == nullptr && workspace_bytes != nullptr) {
    *workspace_bytes = need_sel > need_acc ? need_sel : need_acc;
    return SAFE_OK;
  }
  if (sel) {
    if (workspace == nullptr && need_sel > 0) return SAFE_ERR_WORKSPACE;
    if (workspace_bytes != nullptr && *workspace_bytes < need_sel) return SAFE_ERR_WORKSPACE;
    if (a->grid_h < 0 || a->grid_w < 0 || (int64_t)a->grid_h * a->grid_w != a->N) return SAFE_ERR_SHAPE;
    if (!(a->sigma >= 0.f && a->sigma <= 32.f)) return SAFE_ERR_RANGE;
    if (a->k < 0 || a->k > a->N) return SAFE_ERR_RANGE;
    if (a->B > 0 && a->N > 0 && a->acc == nullptr) return SAFE_ERR_NULL;
    if (a->B > 0 && a->k > 0 && a->idx_out == nullptr) return SAFE_ERR_NULL;
  }
  if (accum) {
    if (!supported_head_dim(a->d)) return SAFE_ERR_UNSUPPORTED;
    if (a->M > 1024) return SAFE_ERR_UNSUPPORTED;
    if (a->head_mask != 0 && a->H > 64) return SAFE_ERR_RANGE;
    if (a->head_mask != 0 && a->H < 64 && (a->head_mask >> a->H) != 0) return SAFE_ERR_RANGE;
    if (!isfinite(a->scale)) return SAFE_ERR_RANGE;
    const bool work = (int64_t)a->B * a->N * a->H > 0 && a->M > 0;
    int st;
    if ((st = check_bnhd(a->q, a->q_stride, work)) != SAFE_OK) return st;
    if ((st = check_bnhd(a->k_text, a->k_stride, work)) != SAFE_OK) return st;
    if (work && (a->w == nullptr || a->acc == nullptr)) return SAFE_ERR_NULL;
  }
  if (workspace != nullptr && !aligned16(workspace)) return SAFE_ERR_ALIGN;
  return pcsp_launch(a, accum ? resolve_scale(a->scale, a->d) : 0.f, workspace,
                     workspace_bytes != nullptr ? *workspace_bytes : 0, static_cast<hipStream_t>(stream));
}

int safe_sw_cfg(const safe_cfg_args* a, void* stream) {
  if (a == nullptr) return SAFE_ERR_NULL;
  if (a->B < 0 || a->N < 0 || a->C < 0) return SAFE_ERR_SHAPE;
  if (a->dtype != SAFE_DT_BF16 && a->dtype != SAFE_DT_F32) return SAFE_ERR_DTYPE;
  if (!isfinite(a->g_ctx) || !isfinite(a->g_sens)) return SAFE_ERR_RANGE;
  if (a->s != nullptr && a->idx != nullptr) return SAFE_ERR_SHAPE;
  if (a->stride[0] < 0 || a->stride[1] < 0) return SAFE_ERR_SHAPE;
  if ((int64_t)a->B * a->N * a->C == 0) return SAFE_OK;
  const int64_t esz = a->dtype == SAFE_DT_BF16 ? 2 : 4;
  if (a->f_c == nullptr || a->f_u == nullptr || a->out == nullptr) return SAFE_ERR_NULL;
  if ((a->C * esz) % 16 != 0 || (a->stride[0] * esz) % 16 != 0 || (a->stride[1] * esz) % 16 != 0) return SAFE_ERR_ALIGN;
  if (!aligned16(a->f_c) || !aligned16(a->f_u) || !aligned16(a->out)) return SAFE_ERR_ALIGN;
  // token rows and images must not overlap (every row is written once)
  if (a->N > 1 && a->stride[1] < a->C) return SAFE_ERR_SHAPE;
  if (a->B > 1 && a->stride[0] < (int64_t)(a->N - 1) * a->stride[1] + a->C) return SAFE_ERR_SHAPE;
  if (a->s != nullptr && (a->s_bstride < 0 || (a->s_bstride != 0 && a->s_bstride < a->N))) return SAFE_ERR_SHAPE;
  if (a->idx != nullptr) {
    if (a->k < 0 || a->idx_bstride < 0 || (a->idx_bstride != 0 && a->idx_bstride < a->k)) return SAFE_ERR_SHAPE;
  } else if (a->k != 0) {
    return SAFE_ERR_NULL;
  }
  return sw_cfg_launch(a, static_cast<hipStream_t>(stream));
}

// A bf16 row block: 16-byte aligned rows (strides multiples of 8 elements, >= 0).
static int check_rows2(const void* p, const int64_t st[2], bool need) {
  if (p == nullptr) return need ? SAFE_ERR_NULL : SAFE_OK;
  for (int i = 0; i < 2; ++i) {
    if (st[i] < 0) return SAFE_ERR_SHAPE;
    if (st[i] % 8 != 0) return SAFE_ERR_ALIGN;
  }
  return aligned16(p) ? SAFE_OK : SAFE_ERR_ALIGN;
}

int safe_linear(const safe_linear_args* a, void* stream) {
  if (a == nullptr) return SAFE_ERR_NULL;
  if (a->batches < 0 || a->M < 0 || a->N < 0 || a->K < 0 || a->Ntok < 0) return SAFE_ERR_SHAPE;
  if (a->K % 64 != 0) return SAFE_ERR_UNSUPPORTED;
  if (a->N % 8 != 0) return SAFE_ERR_ALIGN;
  if (a->act != SAFE_ACT_NONE && a->act != SAFE_ACT_GELU_TANH) return SAFE_ERR_RANGE;
  if (a->flags & ~SAFE_FLAG_CHECK) return SAFE_ERR_RANGE;
  const bool lists = a->a_rows != nullptr || a->res_rows != nullptr || a->out_rows != nullptr;
  if (lists && (a->rows_bstride < 0 || (a->rows_bstride != 0 && a->rows_bstride < a->M))) return SAFE_ERR_SHAPE;
  const bool work = (int64_t)a->batches * a->M * a->N > 0;
  if (work && a->a_rows != nullptr && a->K > 0 && a->Ntok < 1) return SAFE_ERR_SHAPE;   // row 0 must exist
  int st;
  if ((st = check_rows2(a->a, a->a_stride, work && a->K > 0)) != SAFE_OK) return st;
  if ((st = check_rows2(a->out, a->out_stride, work)) != SAFE_OK) return st;
  if ((st = check_rows2(a->res, a->res_stride, false)) != SAFE_OK) return st;
  if (work && a->K > 0) {
    if (a->w == nullptr) return SAFE_ERR_NULL;
    if (a->w_stride < a->K || a->w_stride >= (int64_t(1) << 23)) return SAFE_ERR_SHAPE;
    if (a->w_stride % 8 != 0 || !aligned16(a->w)) return SAFE_ERR_ALIGN;
  }
  if (a->bias != nullptr && !aligned16(a->bias)) return SAFE_ERR_ALIGN;
  if (!work) return SAFE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->flags & SAFE_FLAG_CHECK) {
    const int32_t* l3[3] = {a->a_rows, a->res_rows, a->out_rows};
    for (const int32_t* l : l3)
      if (l != nullptr && (st = check_rows(l, a->batches, a->M, a->rows_bstride, a->Ntok, false, s)) != SAFE_OK)
        return st;
  }
  return linear_launch(a, s);
}

int safe_mfma_probe(int32_t shape, int32_t iters, int32_t blocks, uint32_t seed, float* out, void* stream) {
  if (shape != 32 && shape != 16) return SAFE_ERR_RANGE;
  if (iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > (1 << 24)) return SAFE_ERR_RANGE;
  if (out == nullptr) return SAFE_ERR_NULL;
  return mfma_probe_launch(shape, iters, blocks, seed, out, static_cast<hipStream_t>(stream));
}

int safe_hbm_probe(int32_t mode, const void* src, void* dst, int64_t bytes, int32_t blocks, uint32_t* out,
                   void* stream) {
  if (mode != 0 && mode != 1) return SAFE_ERR_RANGE;
  if (bytes < 16 || bytes > ((int64_t)1 << 40) || bytes % 16 != 0) return SAFE_ERR_SHAPE;
  if (blocks < 1 || blocks > (1 << 20)) return SAFE_ERR_RANGE;
  if (src == nullptr || (mode == 1 && dst == nullptr) || (mode == 0 && out == nullptr)) return SAFE_ERR_NULL;
  if (!aligned16(src) || (mode == 1 && !aligned16(dst))) return SAFE_ERR_ALIGN;
  if (mode == 1) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + (uint64_t)bytes && b < a + (uint64_t)bytes) return SAFE_ERR_RANGE;   // overlapping copy
  }
  return hbm_probe_launch(mode, src, dst, bytes, blocks, out, static_cast<hipStream_t>(stream));
}

}  // extern "C"
