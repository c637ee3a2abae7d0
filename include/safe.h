/*
 * safe.h -- C ABI of libsafe, the MI355X (gfx950) hot path of SAFE-DiT
 * ("SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
 * Diffusion Transformers", arXiv 2606.29360).
 *
 * Four operations, each enqueued on a caller-supplied HIP stream:
 *   safe_mask_classify  Eq. 6-8   is an attention mask in the row-constant class R?
 *   safe_pcsp_select    Eq. 9-12  image->text sensitivity scores and the top-k set S
 *   safe_kv_assemble    Eq. 14,16 global K/V: fresh rows of S over cached context rows
 *   safe_attn_fwd       Eq. 2,16-18 attention on all rows (dense anchor pass) or on the
 *                       gathered rows of S, with optional per-sample valid key lengths
 *                       (or, for masks the rewrite cannot drop, a dense mask)
 *   safe_sdpa           Eq. 8     the rewrite as one call: certify the mask, then run
 *                                 safe_attn_fwd without it, with per-sample key lengths
 *                                 (text padding) or with it, and report which
 *   safe_sw_cfg         Eq. 20-21 sensitivity-weighted classifier-free guidance
 *   safe_linear         Eq. 15    the row-wise linear maps of the block around attention
 *                                 (projections, residual updates, MLP) on gathered rows
 *
 * Common conventions
 *   - Tensors are DEVICE pointers owned by the caller; the library never allocates,
 *     frees or retains device memory.  Scratch space, where an operation needs it,
 *     is a caller-provided workspace whose size is queried first (see each call).
 *   - Activations are token-major [B, N, H, d] with d contiguous; the three other
 *     strides are given in ELEMENTS as stride[0] = batch, stride[1] = token,
 *     stride[2] = head.  bf16 tensors are passed as 16-bit storage.
 *   - Every argument is validated on the host before any HIP call; a failed check
 *     returns a negative status and enqueues nothing.  Values that live in device
 *     memory (index lists, key lengths) are NOT read by the host unless
 *     SAFE_FLAG_CHECK is set; the kernels bound every such value before using it
 *     as an address, so a bad value yields a documented result, never a stray
 *     access.
 *   - No call throws; no call keeps state between calls; calls on different
 *     streams with separate outputs and workspaces may run concurrently.
 *   - `stream` is a hipStream_t (NULL = the default stream).
 */
#ifndef SAFE_DIT_SAFE_H
#define SAFE_DIT_SAFE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAFE_ABI_VERSION 10

/* ---- status codes (negative = error) ----------------------------------- */
enum {
  SAFE_OK = 0,
  SAFE_ERR_NULL = -1,        /* a required pointer is NULL                          */
  SAFE_ERR_SHAPE = -2,       /* sizes/strides inconsistent or out of range          */
  SAFE_ERR_DTYPE = -3,       /* unknown dtype code                                  */
  SAFE_ERR_RANGE = -4,       /* a scalar argument, or (with SAFE_FLAG_CHECK) a device
                                value such as an index or a key length, out of range */
  SAFE_ERR_UNSUPPORTED = -5, /* valid request the library does not implement (e.g. d) */
  SAFE_ERR_WORKSPACE = -6,   /* workspace missing or too small                      */
  SAFE_ERR_HIP = -7,         /* a HIP runtime call failed                            */
  SAFE_ERR_ALIGN = -8        /* a pointer or stride breaks the 16-byte vector access */
};

/* ---- flags ------------------------------------------------------------- */
#define SAFE_FLAG_CHECK        (1u << 0)  /* copy device index/length inputs to the host,
                                             check them, return SAFE_ERR_RANGE on a bad
                                             value (synchronises the stream)            */
#define SAFE_ATTN_SCATTER_OUT  (1u << 1)  /* safe_attn_fwd: write row r at token q_rows[r]
                                             of an [B, Nq, H, d] output instead of the
                                             compact [B, n_rows, H, d] layout           */
#define SAFE_CLASSIFY_ASYNC    (1u << 2)  /* safe_mask_classify: do not wait; `info` is
                                             not written (it may be NULL); the summary is
                                             left in the workspace's first 32 bytes as a
                                             safe_mask_info                             */
#define SAFE_PCSP_ACCUM        (1u << 3)  /* safe_pcsp_select: add Eq. 9-10 scores to acc */
#define SAFE_PCSP_SELECT       (1u << 4)  /* safe_pcsp_select: Eq. 11-12 from acc         */

/* ---- element types ----------------------------------------------------- */
enum {
  SAFE_DT_BOOL = 0,  /* uint8: nonzero = attend, 0 = blocked              */
  SAFE_DT_BF16 = 1,  /* additive bias, bfloat16                           */
  SAFE_DT_F16 = 2,   /* additive bias, IEEE half                          */
  SAFE_DT_F32 = 3    /* additive bias, IEEE single                        */
};

/* ---- mask row classes (ordered: the overall class is the maximum) ------- */
enum {
  SAFE_MASK_ALL_VALID = 0,   /* Boolean row, every entry attends          } class R:   */
  SAFE_MASK_ZERO = 1,        /* additive row of zeros (-0 == +0)          } removable  */
  SAFE_MASK_ROW_CONST = 2,   /* additive row, one finite nonzero constant } (Eq. 6)    */
  SAFE_MASK_KEY_PADDING = 3, /* keys [0,L) valid and equal, [L,Nk) blocked, 1 <= L < Nk */
  SAFE_MASK_NONCONST = 4,    /* finite, not all equal                                  */
  SAFE_MASK_BLOCKED = 5,     /* any other row with -inf / false entries (incl. L = 0)  */
  SAFE_MASK_NONFINITE = 6    /* a NaN or +inf entry                                    */
};

typedef struct {
  int32_t verdict;        /* 1: every stored row is in R, so the mask may be dropped   */
  int32_t mask_class;     /* overall class (max over rows; KEY_PADDING only if every
                             row of each stored batch index has the same L, rows in R
                             counting as L = Nk; otherwise BLOCKED)                    */
  int64_t first_bad_row;  /* lowest flat stored row (b,h,i row-major) not in R, or -1  */
  int64_t rows;           /* number of stored rows = size[0]*size[1]*size[2]           */
} safe_mask_info;

/*
 * safe_mask_classify -- certify whether an attention mask is removable.
 *
 * Defined by the paper's Eq. 6 (the row-constant class R), the rule that
 * batched or head-specific masks are classified on every broadcast query row, the
 * statements after Eq. 7 (all-valid Boolean and all-zero additive masks are in
 * R; finite non-uniform biases and masks with blocked positions are kept) and
 * the Eq. 8 rewrite (drop the mask iff it is in R).  A mask whose rows are all
 * KEY_PADDING with one L per sample is the text-padding mask of Eq. 4/17 and is
 * reported with kv_len_out[b] = L, so the caller can run safe_attn_fwd with
 * per-sample key lengths instead of the mask.
 *
 * mask       device; 4-D [size0, size1, size2, size3] = [B, H, Nq, Nk] as STORED
 *            (broadcast dims stored with size 1); element type `dtype`.
 * stride     element strides of the four dims, >= 0; stride[3] must be 1 when
 *            size[3] > 1.  Any alignment is accepted (rows whose start is 16-byte
 *            aligned are scanned with vector loads).
 * info       host; written on return unless SAFE_CLASSIFY_ASYNC.
 * row_class  device, optional: uint8 [rows] class of every stored row.
 * kv_len_out device, optional: int32 [size0]; L per stored batch index when the
 *            overall class is KEY_PADDING, else -1.
 * workspace  device scratch of *workspace_bytes; call first with workspace == NULL
 *            to have the required size written to *workspace_bytes (returns SAFE_OK).
 * Blocking unless SAFE_CLASSIFY_ASYNC: waits for the stream and reads 32 bytes back.
 * A mask with zero rows is removable (class ALL_VALID for bool, ZERO otherwise).
 */
int safe_mask_classify(const void* mask, int32_t dtype, const int64_t size[4], const int64_t stride[4],
                       uint32_t flags, safe_mask_info* info, uint8_t* row_class, int32_t* kv_len_out,
                       void* workspace, size_t* workspace_bytes, void* stream);

/*
 * safe_pcsp_select -- Prompt-Conditioned Sensitivity Partitioning.
 *
 * SAFE_PCSP_ACCUM (Eq. 9-10): for every image token i and head h in the head set,
 *   A_h[i, j] = softmax over j < kv_len[b] of scale * q[b,i,h,:] . k_text[b,j,h,:]
 *   acc[b, i] += sum_h sum_{j < kv_len[b]} w[b, j] * A_h[i, j]
 * Call once per warm-up step and layer; the 1/(|W||L||H|) factor of Eq. 10 is a
 * positive constant and is left out (it changes neither order nor Norm).
 * SAFE_PCSP_SELECT (Eq. 11-12): s_bar = G_sigma * acc on the grid_h x grid_w
 * row-major raster (token i = row*grid_w + col): separable Gaussian taps
 * exp(-t^2/(2 sigma^2)), |t| <= ceil(3 sigma), renormalised over the taps inside
 * the grid; sigma == 0 leaves acc unchanged.  score_out (optional) receives
 * Norm(s_bar) = (s_bar - min)/(max - min) (0 for a constant field).  idx_out
 * receives the k tokens ranking highest by s_bar (descending value, ties to the
 * lower index, -0 == +0, NaN last), in ASCENDING token order.  Norm is
 * increasing, so ranking s_bar selects the same set as ranking Norm(s_bar).
 * Both flags may be given in one call (accumulate, then select).
 *
 * Workspace: a call with workspace == NULL and workspace_bytes != NULL only writes
 * the bytes it can use (no launch).  SAFE_PCSP_SELECT needs that much.  For
 * SAFE_PCSP_ACCUM it is optional: given a workspace of at least that size (the size
 * passed in *workspace_bytes), the heads are split into groups over more workgroups and
 * the group sums are added to acc in group order by a second kernel; with workspace
 * and workspace_bytes both NULL the accumulation runs unsplit.  Accumulation alone
 * rounds a little differently split and unsplit; each form is deterministic.
 * Limits: H <= 64 when head_mask != 0; d in {32, 64, 96, 128}; M <= 1024;
 * 0 <= k <= N; acc is caller-zeroed before the first accumulation.
 */
typedef struct {
  uint32_t flags;                  /* SAFE_PCSP_ACCUM | SAFE_PCSP_SELECT                */
  int32_t B, N, M, H, d;
  const void* q;      int64_t q_stride[3];   /* [B, N, H, d] bf16 image queries (ACCUM) */
  const void* k_text; int64_t k_stride[3];   /* [B, M, H, d] bf16 text keys (ACCUM)     */
  const int32_t* kv_len;           /* device [B] valid text keys (suffix padding); NULL = M;
                                      values are clamped to [0, M]                      */
  const float* w;                  /* device [B, M] content weights (ACCUM): 0 on padding
                                      and special tokens, summing to 1 over content     */
  uint64_t head_mask;              /* bit h set = head h is in the head set; 0 = all    */
  float scale;                     /* logit scale; <= 0 means 1/sqrt(d)                 */
  float* acc;                      /* device [B, N] fp32 (ACCUM adds; SELECT reads)     */
  int32_t grid_h, grid_w;          /* SELECT: grid_h * grid_w == N                      */
  float sigma;                     /* SELECT: Gaussian width in tokens, >= 0, <= 32     */
  int32_t k;                       /* SELECT: 0 <= k <= N                               */
  float* score_out;                /* device [B, N], optional (SELECT)                  */
  int32_t* idx_out;                /* device [B, k] (SELECT)                            */
} safe_pcsp_args;

int safe_pcsp_select(const safe_pcsp_args* a, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * safe_kv_assemble -- global keys and values for SRSU (Eq. 14, 16).
 *
 *   k_out[b, j] = k_fresh[b, r]  if idx[b, r] == j
 *               = k_cache[b, j]  otherwise          (same for v)
 * i.e. the fresh rows of the sensitive set S placed, in the original token order,
 * over the cached context rows of the last anchor.  idx holds nsel ascending
 * distinct token indices per sample (shared by all samples when idx_bstride == 0).
 * Out of place: every output row is read once from its source and written once.
 * In place (k_out == k_cache, v_out == v_cache, equal strides): only the nsel
 * fresh rows are written (the cache refresh of Eq. 19 with S = all rows is the
 * same call with nsel == N and idx = 0..N-1).
 * Index entries outside [0, N) are skipped (no write); with SAFE_FLAG_CHECK they
 * return SAFE_ERR_RANGE instead.  Elements are 16-bit (bf16 / fp16); every
 * pointer and stride must give 16-byte aligned rows, and d % 8 == 0.
 */
typedef struct {
  int32_t B, N, H, d, nsel;
  const void* k_fresh; const void* v_fresh; int64_t fresh_stride[3]; /* [B, nsel, H, d] */
  const int32_t* idx; int64_t idx_bstride;                           /* [B, nsel] int32  */
  const void* k_cache; const void* v_cache; int64_t cache_stride[3]; /* [B, N, H, d]     */
  void* k_out; void* v_out; int64_t out_stride[3];                   /* [B, N, H, d]     */
  uint32_t flags;                                                    /* SAFE_FLAG_CHECK  */
} safe_kv_args;

int safe_kv_assemble(const safe_kv_args* a, void* stream);

/* Source map of the fused global K/V read (see safe_attn_fwd.kv_src): writes kv_src,
 * device int32 [B, N] row-major (sample stride N), with kv_src[b][j] = r when
 * idx[b][r] == j and -1 for the other tokens.  Of a, only B, N, idx, nsel, idx_bstride
 * and flags are read; idx must be ascending (SAFE_FLAG_CHECK verifies it and the range,
 * SAFE_ERR_RANGE).  Entries outside [0, N) are skipped.  Enqueued on stream; one launch. */
int safe_kv_source_map(const safe_kv_args* a, int32_t* kv_src, void* stream);

/*
 * safe_attn_fwd -- scaled dot-product attention, normally without a mask tensor.
 *
 * For each sample b, head h and output row r (query token i = q_rows[b][r], or
 * i = r when q_rows is NULL), with L = kv_len[b] (or Nk):
 *   O[b, r, h, :] = sum_{j < L} softmax_j(scale * q[b,i,h,:] . k[b,j,h,:] + m[b,h,i,j]) v[b,j,h,:]
 *   lse[b, h, r]  = natural-log log-sum-exp of those scaled logits
 * With mask == NULL (m = 0) this is Eq. 2 with m = empty (also the Eq. 8 rewrite of a
 * removable mask), the SRSU row-selective forms Eq. 16 (self-attention: every key
 * visible) and Eq. 17 (cross-attention: text padding kept as the valid length L), and
 * the dense anchor pass of Eq. 18 (q_rows == NULL).  A row with no attended key
 * (L == 0, or every key blocked by the mask) gives O = 0 and lse = -inf.
 * Inputs bf16; softmax and accumulation in fp32; O is written as bf16.
 *
 * q_rows        device int32 [B, n_rows] (sample stride q_rows_bstride; 0 = one list
 *               shared by every sample) or NULL (n_rows must then equal Nq).  Entries
 *               outside [0, Nq) read a zero query row (SAFE_FLAG_CHECK: error).
 * kv_len        device int32 [B] or NULL; values are clamped to [0, Nk].
 * lse           device fp32 [B, H, n_rows], optional.
 * o             bf16; compact [B, n_rows, H, d] unless SAFE_ATTN_SCATTER_OUT.
 * Limits: d in {32, 64, 72, 96, 128}; pointers and strides give 16-byte aligned rows;
 * k and v token strides (stride[1]) below 2^25 elements (else SAFE_ERR_UNSUPPORTED).
 *
 * mask          optional device mask of Eq. 2 (NULL: none), for masks the Eq. 8 rewrite
 *               cannot remove and for measuring what the rewrite saves.  Element
 *               (b, h, i, j) -- i the query TOKEN, not the output row -- is at
 *               mask + b*mask_stride[0] + h*mask_stride[1] + i*mask_stride[2] + j
 *               (element strides; 0 broadcasts, e.g. one [Nq, Nk] mask for all b, h
 *               or a key-only [B, 1, 1, Nk] mask).  mask_dtype: SAFE_DT_BOOL (nonzero
 *               = attend; blocked keys get -inf), SAFE_DT_BF16, SAFE_DT_F16 or
 *               SAFE_DT_F32 (additive bias, -inf allowed).  The bias is added in fp32
 *               as scale * (q . k + bias / scale), so entries beyond about
 *               FLT_MAX * scale in magnitude act as -inf / +inf.  Rows are read in
 *               16-byte pieces: the pointer 16-byte aligned and every stride a multiple
 *               of 16 bytes (SAFE_ERR_ALIGN).  Not combinable with kv_len
 *               (SAFE_ERR_UNSUPPORTED).
 *               Rows whose token is outside [0, Nq) read a zero query row and mask
 *               row 0 of their (b, h) (with Nq == 0 the mask has no rows and is not
 *               read).  mask_dtype and mask_stride are ignored when mask is NULL.
 *
 * workspace     optional device scratch of workspace_bytes bytes (16-byte aligned),
 *               owned by the caller and not retained.  The rows are processed in
 *               tiles of 128 or 256 rows of one (b, h), one workgroup each (the size
 *               is chosen per call, see safe_attn_plan); when the tile count leaves
 *               the last round of workgroups on the GPU partly empty, the tiles of that round
 *               are split along the keys into partial results (unnormalised fp32 O,
 *               running max and sum per row) kept in the workspace and merged by a
 *               second kernel on the same stream.  The result is the same attention,
 *               rounded differently for those rows.  With workspace NULL or smaller
 *               than safe_attn_workspace_bytes() reports, no tile is split.  Calls that
 *               share a workspace must be ordered on one stream.
 *
 * kv_src        optional fused global K/V (Eq. 14 and 16 read in place of a separate
 *               safe_kv_assemble pass): device int32 [B, Nk] (sample stride
 *               kv_src_bstride, 0 = one map for every sample).  Key j of sample b is
 *               read from row kv_src[b][j] of k_fresh / v_fresh ([B, n_fresh, H, d] bf16,
 *               element strides fresh_stride) when that value is in [0, n_fresh), and
 *               from k / v (the cache) otherwise.  safe_kv_source_map builds the map
 *               from the ascending index list of S.  The result is attention on the
 *               assembled K/V (bit for bit where safe_attn_plan reports the same schedule
 *               for both calls; the split of long key ranges may differ).  Not combinable with kv_len or a mask
 *               (SAFE_ERR_UNSUPPORTED).  NULL: k and v are read as given.
 */
typedef struct {
  int32_t B, H, Nq, Nk, d;
  const void* q; int64_t q_stride[3];     /* [B, Nq, H, d] bf16 */
  const void* k; int64_t k_stride[3];     /* [B, Nk, H, d] bf16 */
  const void* v; int64_t v_stride[3];     /* [B, Nk, H, d] bf16 */
  void* o;       int64_t o_stride[3];     /* bf16, see above    */
  const int32_t* q_rows; int32_t n_rows; int64_t q_rows_bstride;
  const int32_t* kv_len;
  float scale;                            /* <= 0 means 1/sqrt(d) (Eq. 2) */
  float* lse;
  uint32_t flags;                         /* SAFE_ATTN_SCATTER_OUT | SAFE_FLAG_CHECK */
  void* workspace; int64_t workspace_bytes;   /* optional, see above */
  const void* mask; int32_t mask_dtype; int64_t mask_stride[3];   /* optional, see above */
  const int32_t* kv_src; int64_t kv_src_bstride;                   /* optional, see below */
  const void* k_fresh; const void* v_fresh; int64_t fresh_stride[3]; int32_t n_fresh;
} safe_attn_args;

int safe_attn_fwd(const safe_attn_args* a, void* stream);

/*
 * safe_attn_fwd_noalloc -- safe_attn_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The partials of the split tail tiles go to a library-owned static device array of
 * SAFE_NOALLOC_SCRATCH_BYTES bytes (one per GPU, held until the process ends) instead of a
 * caller workspace: the call runs the schedule safe_attn_fwd runs with a workspace of that
 * size (bit for bit the same result), so a shape whose split needs more runs unsplit and no
 * call can exceed the array.  No allocation, no free, no host synchronisation.
 *
 * a             as for safe_attn_fwd, except: workspace must be NULL and workspace_bytes 0
 *               (SAFE_ERR_WORKSPACE otherwise: the scratch is the library's), and
 *               SAFE_FLAG_CHECK is refused (SAFE_ERR_UNSUPPORTED: it copies device values
 *               to host memory).
 * The first call on a device resolves the array's address there (hipGetSymbolAddress;
 * SAFE_ERR_HIP if that fails).  Every call on a GPU shares that GPU's array and leaves
 * its partials in it; no call reads a byte of it that the same call has not written first,
 * so nothing needs clearing, but calls that overlap on one GPU (other streams, other host
 * threads) race on the array: order them on one stream.
 */
#define SAFE_NOALLOC_SCRATCH_BYTES (64ull << 20)
int safe_attn_fwd_noalloc(const safe_attn_args* a, void* stream);

/* Workspace bytes that let safe_attn_fwd split the last round of tiles for these
 * arguments on the current device (0: this shape gains nothing from a split, the
 * key-length form is never split, or no device is visible).  Of the pointer fields
 * only whether mask and q_rows are NULL is read.  Negative: the SAFE_ERR_* status
 * safe_attn_fwd would return for the sizes. */
int64_t safe_attn_workspace_bytes(const safe_attn_args* a);

/* The schedule safe_attn_fwd runs for these arguments on the current device: rows per
 * tile (128 or 256), the tile count (tiles per (b, h) x H x B), how many tiles of the
 * last round are split along the keys and into how many ranges of how many keys, and
 * the workspace bytes those partials take.  Reads the sizes, flags, workspace_bytes and
 * whether workspace, q_rows, kv_len and mask are NULL, like the call; dereferences no
 * pointer of a.  out is a host pointer, filled on SAFE_OK (all zero when there is no
 * row to compute).  Errors: SAFE_ERR_NULL (a or out NULL) and the size errors of
 * safe_attn_fwd.  The plan depends only on these values and on the device (its
 * compute units and the kernels' occupancy), so repeated calls give the same plan. */
typedef struct {
  int32_t rows_per_tile;
  int32_t row_tiles;
  int32_t split_tiles;      /* 0: nothing is split */
  int32_t key_ranges;       /* ranges per split tile (1 when nothing is split) */
  int32_t keys_per_range;   /* keys per range (the last range may hold fewer) */
  int64_t workspace_bytes;  /* partials of the split tiles */
} safe_attn_plan_info;

int safe_attn_plan(const safe_attn_args* a, safe_attn_plan_info* out);

/*
 * safe_sdpa -- the Eq. 8 rewrite as one call.  The paper's SAFE-SDPA replaces an SDPA
 * call whose mask lies in the row-constant class R (Eq. 6; every stored row one real
 * constant, all-valid Boolean and all-zero additive masks included) by the mask-free
 * call, which Eq. 7 makes exact, and keeps every other mask; the text padding of the
 * cross-attention (Eq. 4/17) is kept as well.  This call certifies a->mask with the
 * classifier of safe_mask_classify and then runs safe_attn_fwd on a copy of a:
 *   SAFE_ROUTE_NO_MASK  mask NULL, or every stored row in R      -> mask dropped
 *   SAFE_ROUTE_KV_LEN   every row KEY_PADDING with one valid length L per sample
 *                       (rows in R counting as L = Nk)          -> mask dropped,
 *                       kv_len[b] = L of the mask row that serves sample b
 *   SAFE_ROUTE_MASK     anything else (finite non-constant biases, other blocked
 *                       patterns, NaN / +inf entries)           -> the mask is kept
 * Correctness never depends on the rewrite firing: every route computes the attention
 * of Eq. 2 with the given mask (up to the rounding of the kernels).
 *
 * a             as for safe_attn_fwd (its workspace serves the attention as there);
 *               the mask is described by mask, mask_dtype and mask_stride as there:
 *               a zero stride marks a broadcast dimension, stored with size 1, so the
 *               classifier scans the [B|1, H|1, Nq|1, Nk] rows as stored.  kv_len must
 *               be NULL when a mask is given (SAFE_ERR_UNSUPPORTED).  The classifier
 *               accepts any alignment; the masked route needs the 16-byte mask rows
 *               safe_attn_fwd requires (else SAFE_ERR_ALIGN, returned after the scan).
 * classify_ws   device scratch for the classifier and the per-sample lengths, of
 *               *classify_ws_bytes bytes (16-byte aligned); classify_ws == NULL writes
 *               the required size to *classify_ws_bytes and returns SAFE_OK.  Not
 *               needed (may be NULL) when mask is NULL.
 * info          host, optional: the route taken, the mask's overall class and its
 *               first row outside R (-1 if none; route NO_MASK without a mask: class
 *               -1, row -1).
 * Blocking when a mask is given (the verdict is a host decision: the stream is
 * synchronised once); the attention itself is enqueued on stream and not waited for.
 */
enum { SAFE_ROUTE_NO_MASK = 0, SAFE_ROUTE_KV_LEN = 1, SAFE_ROUTE_MASK = 2 };
typedef struct {
  int32_t route;          /* SAFE_ROUTE_*                                     */
  int32_t mask_class;     /* overall class of the mask (SAFE_MASK_*), or -1  */
  int64_t first_bad_row;  /* lowest stored row outside R, or -1              */
} safe_sdpa_info;

int safe_sdpa(const safe_attn_args* a, void* classify_ws, size_t* classify_ws_bytes, safe_sdpa_info* info,
              void* stream);

/* Human-readable name of a status code (static storage). */
const char* safe_status_str(int status);
/*
 * safe_sw_cfg -- sensitivity-weighted classifier-free guidance (Eq. 20, 21).
 *
 * For image b, token i and value c (f_c, f_u: conditional and unconditional
 * predictions, token-major [B, N, C] with C contiguous):
 *   gamma_i = g_ctx + (g_sens - g_ctx) * s[b, i]     with a score row s (Eq. 20; s is
 *                                                     the normalised score of Eq. 11)
 *   gamma_i = g_sens if i is in idx[b], else g_ctx    with an index list (the binary
 *                                                     variant: S gets g_sens)
 *   gamma_i = g_ctx                                   with neither (global guidance)
 *   out[b, i, c] = f_u + gamma_i * (f_c - f_u)        (Eq. 21)
 * computed in fp32 (one subtraction and one fused multiply-add) and stored in the
 * tensors' dtype (bf16 rounds to nearest even).  out may alias f_c or f_u.
 *
 * dtype         SAFE_DT_BF16 or SAFE_DT_F32 for all three tensors.
 * stride        element strides of b and i, shared by f_c, f_u and out; C * element
 *               size must be a multiple of 16 bytes and every row 16-byte aligned.
 * s             device fp32 [B, N] (sample stride s_bstride; 0 = one row for all).
 * idx           device int32 [B, k] ascending token indices (sample stride
 *               idx_bstride; 0 = one list for all); entries outside [0, N) match no
 *               token.  Give at most one of s and idx.
 */
typedef struct {
  int32_t B, N, C, dtype;
  const void* f_c; const void* f_u; void* out;   /* [B, N, C] */
  int64_t stride[2];                            /* b, i (elements) */
  const float* s; int64_t s_bstride;
  const int32_t* idx; int32_t k; int64_t idx_bstride;
  float g_ctx, g_sens;
} safe_cfg_args;

int safe_sw_cfg(const safe_cfg_args* a, void* stream);

/*
 * safe_linear -- the row-wise linear maps of the DiT block around attention.  Eq. 15:
 * at a non-anchor step the block computes its attention inputs and outputs, residual
 * updates and row-wise MLP only for the rows of S; this is that computation for any
 * row list (or all rows, the dense block of Eq. 18).  For batch b and row r < M:
 *   y[n] = sum_k A[b, ra(r), k] * W[n, k] + bias[n]         ra(r) = a_rows[b][r] or r
 *   y[n] = gelu_tanh(y[n])                                  if act == SAFE_ACT_GELU_TANH
 *   y[n] = y[n] + R[b, rr(r), n]                            rr(r) = res_rows[b][r] or r
 *   out[b, ro(r), n] = bf16(y[n])                           ro(r) = out_rows[b][r] or r
 * with gelu_tanh(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); products and sums
 * in fp32, one rounding to bf16 (nearest even) on store.
 *
 * a, res, out   bf16 rows (K values for a, N for res and out); element strides
 *               stride[0] = batch, stride[1] = row; 16-byte aligned rows.
 * w             bf16 [N, K]: row n holds output feature n's weights (K contiguous),
 *               row stride w_stride elements (< 2^23: a tile's 256 rows are addressed
 *               with 32-bit byte offsets).
 * bias          fp32 [N] (16-byte aligned) or NULL.
 * a_rows, res_rows, out_rows  device int32 [batches, M] (batch stride rows_bstride; 0 =
 *               one list for all) or NULL; entries index rows [0, Ntok).  Out of range:
 *               an A row reads row 0, a residual row adds nothing, an output row is not
 *               written (SAFE_FLAG_CHECK: SAFE_ERR_RANGE).  With out_rows the untouched
 *               output rows keep their contents (e.g. the cached context rows).
 * Limits: K a multiple of 64, N a multiple of 8 (else SAFE_ERR_UNSUPPORTED /
 * SAFE_ERR_ALIGN).  out may alias res only row for row (same rows, same strides).
 */
#define SAFE_ACT_NONE      0
#define SAFE_ACT_GELU_TANH 1
typedef struct {
  int32_t batches, M, N, K;
  const void* a; int64_t a_stride[2];
  const void* w; int64_t w_stride;
  const float* bias;
  int32_t act;
  const void* res; int64_t res_stride[2];
  void* out; int64_t out_stride[2];
  const int32_t* a_rows; const int32_t* res_rows; const int32_t* out_rows;
  int64_t rows_bstride;
  int32_t Ntok;
  uint32_t flags;                          /* SAFE_FLAG_CHECK */
} safe_linear_args;

int safe_linear(const safe_linear_args* a, void* stream);

/*
 * safe_mfma_probe -- a measurement aid beside the method (no equation of the pages): the
 * matrix-core rate the GPU sustains on random bf16 operands with nothing else running, the
 * ceiling the attention and linear kernels are read against on a power-capped chip.
 * `blocks` workgroups of 256 threads (two per CU fill the chip as the attention kernel does)
 * each run `iters` rounds; a round is 16 MFMAs per wave into four independent accumulators,
 * every instruction on a different pair of the lane's eight A and eight B register fragments:
 *   shape 32: v_mfma_f32_32x32x16_bf16 (32768 FLOP each), shape 16: v_mfma_f32_16x16x32_bf16
 *   (16384 FLOP each); FLOP per launch = blocks * 4 waves * iters * 16 * FLOP per MFMA.
 * Operands: lane g = 256 * block + thread holds, in fragment f (A: f = 0..7, B: f = 8..15),
 * element e = bf16_rne((h / 2^24 - 0.5) * 4) with h = H(seed ^ H(64 g + 8 f + e)) >> 8 and H the
 * 32-bit mixer x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b; x ^= x >> 16.
 * Round q (0..15) multiplies A fragment q % 8 by B fragment (q + q / 8) % 8 into accumulator q % 4.
 * out: device float[blocks * 256], lane g's sum of its accumulator elements (keeps the
 * products live; the sum over a wave's lanes is the sum of every product it issued).
 * Errors: SAFE_ERR_RANGE (shape not 16 or 32, iters or blocks outside [1, 2^24]), SAFE_ERR_NULL.
 */
int safe_mfma_probe(int32_t shape, int32_t iters, int32_t blocks, uint32_t seed, float* out, void* stream);

/*
 * safe_hbm_probe -- a measurement aid beside the method (no equation of the pages): the
 * streaming bandwidth of the device memory, against which the bandwidth-bound steps (the
 * classifier reads its mask once, the K/V assembly reads and writes each row once) are read.
 * `blocks` workgroups of 256 threads; chunk c (16 bytes) of src belongs to thread
 * c mod (256 * blocks), which loads it non-temporally with three more of its chunks in flight.
 *   mode 0 (read):  out[t] = xor of every 32-bit word of thread t's chunks (0 for a thread
 *                   with none); out is device uint32[256 * blocks], dst is unused.
 *   mode 1 (copy):  dst[0, bytes) = src[0, bytes), stored non-temporally; out is unused.
 * src and dst are device pointers, 16-byte aligned, not overlapping; bytes a multiple of 16 in
 * [16, 2^40].  Enqueued on stream; one launch.
 * Errors: SAFE_ERR_RANGE (mode not 0 or 1, blocks outside [1, 2^20], overlapping copy),
 * SAFE_ERR_SHAPE (bytes), SAFE_ERR_NULL, SAFE_ERR_ALIGN.
 */
int safe_hbm_probe(int32_t mode, const void* src, void* dst, int64_t bytes, int32_t blocks, uint32_t* out,
                   void* stream);

/* SAFE_ABI_VERSION of the built library. */
int safe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAFE_DIT_SAFE_H */
