// Attention forward for gfx950: bf16 MFMA for Q K^T and P V, fp32 online softmax.
//
// Computes, per sample b, head h and selected query row, softmax over the valid
// keys of scale * q . k (+ mask), times V ("SAFE-DiT" Eq. 2; with no mask also the
// Eq. 8 rewrite of a removable one; Eq. 16 SRSU self-attention on the gathered rows
// of S; Eq. 17 cross-attention with the text padding kept as a per-sample valid key
// count; Eq. 18 dense anchor pass).  The masked instances read a dense mask: the
// call that the rewrite removes, kept for masks outside R.
//
// Work decomposition
//   workgroup = 4 waves of one (b, h); each wave owns RB row blocks of 32 query rows
//   (RB = 1: 128 rows per workgroup, three workgroups per CU, <= 168 registers per
//   lane; two for d = 128 and for the masked instances.  RB = 2, compiled for d = 96
//   and 72 without mask or key lengths: 256 rows, two workgroups per CU, and every K
//   and V fragment read from LDS feeds two MFMAs).  The waves on a SIMD overlap one
//   another's MFMA and softmax work; wave priorities (s_setprio) let the wave whose
//   softmax is on its critical path issue first.  Keys stream in tiles of 64 through
//   LDS, double buffered (two separate LDS objects, loop unrolled by two), one barrier
//   per tile.
//   K and V tiles are copied global -> LDS by the direct-to-LDS loads
//   (global_load_lds_dwordx4): no staging registers, no LDS store instructions.
//   Both tiles keep the natural [key][d] layout; row strides are chosen for
//   conflict-free LDS reads (see Tile).
//   Per wave, row block and tile:
//     S^T[64 keys x 32 queries] = K_tile . Q^T     (v_mfma_f32_32x32x16_bf16)
//       A = K rows from LDS (ds_read_b128, d contiguous); B = the wave's Q^T,
//       held in registers for the whole loop.  In the 32x32 accumulator layout
//       lane l holds query column l%32 and 16 keys, so each lane owns one query
//       and the row max / row sum need only the partner lane l^32.
//     O^T[d x 32 queries] += V^T . P^T             (same MFMA)
//       B = P^T: the lane's own probabilities packed to bf16 in registers.
//       A = V^T, read with the LDS transpose load ds_read_b64_tr_b16: in each
//       16-lane group, output lane i element j comes from source lane 4j + i/4,
//       element i%4; pointing source lane s at V[key0 + s/4][d0 + 4(s%4)] gives
//       output lane i the four keys key0..key0+3 of column d0 + i, which are
//       exactly the k-slots the S^T accumulator layout assigns to P^T.
//   A head dimension that is not a multiple of 16 (d = 72) runs the products on the
//   next multiples (80 for Q K^T, 96 for P V): the missing Q columns are zero, the
//   padded K and V columns in LDS hold copies of real data, and O rows past d are
//   dropped.
//   Online softmax in the log2 domain with a lazily moved reference max.  A tile's
//   probabilities are first computed against the current reference, with no tile
//   max at all; only when some lane's share of the tile sum exceeds 2^16 or is not
//   finite (always on the first tile, against the initial reference) does the wave take
//   the exact pair max, move the reference of the rows whose max exceeds it by more
//   than 2^8 (rescaling O and l), and recompute the tile.  Probabilities stay below
//   2^16, far inside the range of bf16 P and the fp32 accumulators, and the common
//   path skips the 32-value max reduction.  The reference starts at -FLT_MAX, not
//   -inf, so a row whose keys are all masked so far gets exp2(-inf) = 0, not NaN.
//   The mask, when present, is loaded one tile ahead -- coalesced into registers and
//   redistributed through a per-wave LDS area, so each lane ends up with its keys in
//   runs of four (the accumulator layout's grouping) -- and folded into the scores as
//   s + bias / scale (Boolean: -inf where blocked) before the softmax.
//   Workgroups are remapped so all row tiles of one (b, h) sit on one XCD and
//   share its L2 for the K/V stream.
#pragma once

#include "common.h"

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <type_traits>

namespace safe {

// mask element type of an instance
constexpr int kMaskNone = 0, kMaskBool = 1, kMaskBf16 = 2, kMaskF16 = 3, kMaskF32 = 4;

struct AttnParams {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  const int32_t* q_rows;
  int64_t qr_bs;
  const int32_t* kv_len;
  float* lse;
  int B, H, Nq, Nk, n_rows, n_row_tiles, total_wg;
  float scale_log2;
  int scatter;
  // Tail split: workgroups [0, n_full) take whole row tiles (logical tiles 0..n_full-1);
  // workgroup n_full + t takes key range t % nsplit (split_tiles key tiles each) of
  // logical tile n_full + t / nsplit and leaves unnormalised partials in `part`:
  // O as fp32 [n_slots][rows][d], then (max, sum) as fp32 [n_slots][rows][2], rows = the
  // instance's query rows per workgroup.
  int n_full, nsplit, split_tiles, n_slots;
  float* part;
  // consecutive logical tiles cycle through head_group heads of one row tile (1: all row
  // tiles of a head in turn), so a per-row mask shared by the heads is read once per group
  // from L2
  int head_group;
  // dense mask (masked instances): element (b, h, query token i, key j) at
  // mask + b*ms0 + h*ms1 + i*ms2 + j elements; bias is added as bias * inv_scale
  const char* mask;
  int64_t ms0, ms1, ms2;
  float inv_scale;
  // fused global K/V (source-map instances): key j of sample b comes from fresh row
  // kv_src[b * src_bs + j] when that is >= 0, else from k / v (the cache)
  const int32_t* kv_src;
  int64_t src_bs;
  int nsel;                 // fresh rows per sample; map entries outside [0, nsel) read the cache
  const u16* kf;
  const u16* vf;
  int64_t fs0, fs1, fs2;
};

hipError_t attn_masked_dispatch(const AttnParams& p, int d, bool gather, int mt, hipStream_t s);
int attn_masked_resident(int d, bool gather, int mt);
// short key sets with per-sample key lengths (text cross-attention): attn_short.hip
bool attn_short_applies(const safe_attn_args* a);
hipError_t attn_short_launch(const AttnParams& p, int d, hipStream_t s);

namespace {

constexpr int BN = 64;        // keys per tile
constexpr int NTHREADS = 256;
constexpr int NWAVES = NTHREADS / 64;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
// Query row blocks (of 32) per wave, RB: each K and V^T fragment read from LDS feeds RB
// MFMAs, and a K/V tile copied into LDS serves NWAVES * 32 * RB query rows.
constexpr int tile_rows(int rb) { return NWAVES * 32 * rb; }
constexpr float kSumLimit = 65536.0f;          // a lane's tile-sum share above this moves the reference

// LDS tile geometry.  K rows are read 16 bytes per lane, 16 lanes on 16 rows at once:
// conflict-free on the 64 four-byte banks when the row stride is an odd number of
// 16-byte chunks.  V rows are read by the transpose load, 4 rows x 32 bytes per
// 16-lane group: conflict-free when the stride is 64 or 192 bytes modulo 256.
// K rows hold at least the 2 * KS chunks the Q K^T steps read, V rows the 4 * DB
// chunks the P V blocks read; chunks past d are padding.
template <int D>
struct Tile {
  static constexpr int CH = D / 8;                                   // 16-byte chunks of a row
  static constexpr int KS = (D + 15) / 16;                           // k-steps of Q K^T
  static constexpr int DB = (D + 31) / 32;                           // 32-row blocks of O^T
  static constexpr int KC = CH > 2 * KS ? CH : 2 * KS;
  static constexpr int VC = CH > 4 * DB ? CH : 4 * DB;
  static constexpr int K_SLOTS = KC | 1;                             // odd chunk count
  static constexpr int V_SLOTS = (VC % 16 == 4 || VC % 16 == 12) ? VC : (VC | 3) + (((VC | 3) % 16 == 7 || (VC | 3) % 16 == 15) ? 5 : 1);
  static constexpr int K_ROWB = K_SLOTS * 16;
  static constexpr int V_ROWB = V_SLOTS * 16;
  static constexpr int K_BYTES = BN * K_ROWB;
  static constexpr int V_BYTES = BN * V_ROWB;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int NCOPY = K_SLOTS + V_SLOTS;                    // wave-wide 1 KB copies per tile
  static constexpr int PER_WAVE = (NCOPY + NWAVES - 1) / NWAVES;
  static_assert(D % 8 == 0, "rows are whole 16-byte chunks");
  static_assert((V_SLOTS % 16) == 4 || (V_SLOTS % 16) == 12, "V stride must be 64 or 192 mod 256 bytes");
  static_assert(V_SLOTS >= VC && K_SLOTS >= KC, "rows must fit");
};

// A mask run of four consecutive keys as loaded: 4 bytes (Boolean), 8 (16-bit), 16 (fp32).
template <int MT> struct MaskRun { typedef u32 type; static constexpr int esz = 1; };
template <> struct MaskRun<kMaskBf16> { typedef u32x2 type; static constexpr int esz = 2; };
template <> struct MaskRun<kMaskF16> { typedef u32x2 type; static constexpr int esz = 2; };
template <> struct MaskRun<kMaskF32> { typedef u32x4 type; static constexpr int esz = 4; };

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Fold a run into scores sc[4g .. 4g+3]: blocked -> -inf, or + bias * inv_scale.
// (Whole-vector reinterpretations only.)
template <int MT>
__device__ __forceinline__ void fold_run(f32x16& sc, int g, const typename MaskRun<MT>::type& c, float inv_scale) {
  if constexpr (MT == kMaskBool) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (((c >> (8 * e)) & 0xFFu) == 0u) sc[4 * g + e] = -INFINITY;
  } else if constexpr (MT == kMaskBf16) {
    const f32x2 lo = __builtin_bit_cast(f32x2, c << 16);
    const f32x2 hi = __builtin_bit_cast(f32x2, c & 0xFFFF0000u);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      sc[4 * g + 2 * k] = __builtin_fmaf(lo[k], inv_scale, sc[4 * g + 2 * k]);
      sc[4 * g + 2 * k + 1] = __builtin_fmaf(hi[k], inv_scale, sc[4 * g + 2 * k + 1]);
    }
  } else if constexpr (MT == kMaskF16) {
    const f16x4 h = __builtin_bit_cast(f16x4, c);
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[4 * g + e] = __builtin_fmaf((float)h[e], inv_scale, sc[4 * g + e]);
  } else if constexpr (MT == kMaskF32) {
    const f32x4 f = __builtin_bit_cast(f32x4, c);
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[4 * g + e] = __builtin_fmaf(f[e], inv_scale, sc[4 * g + e]);
  }
}

// Logical tile -> (row tile, head, sample): all row tiles of head 0, then head 1, ...
// Consecutive logical tiles share an XCD (xcd_remap), so the workgroups that run side
// by side share one head's K/V in L2.  With head_group G > 1 (a mask broadcast over the
// heads) the order is row tile-major within groups of G heads: the ~64 tiles side by side
// on an XCD are 64 / G row tiles of G heads, sharing each mask tile G ways and each
// head's K/V 64 / G ways (G = 4: 5% faster than G = 1 on the 160x160 masked call, G = 8 17%
// slower).
__device__ __forceinline__ void split_logical(int logical, const AttnParams& p, int& tile, int& h, int& b) {
  if (p.head_group > 1) {
    const int G = p.head_group;
    const int hi = logical % G;
    const int rest = logical / G;
    tile = rest % p.n_row_tiles;
    const int r2 = rest / p.n_row_tiles;
    const int ng = p.H / G;
    h = (r2 % ng) * G + hi;
    b = r2 / ng;
    return;
  }
  tile = logical % p.n_row_tiles;
  const int bh = logical / p.n_row_tiles;
  h = bh % p.H;
  b = bh / p.H;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void copy16_to_lds(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

template <int D, bool GATHER, bool KVLEN, int MT, int RB, bool KVMAP = false>
__global__ __launch_bounds__(NTHREADS, (D >= 128 || MT != kMaskNone || RB > 1) ? 2 : 3)
void attn_fwd_kernel(AttnParams p) {
  using T = Tile<D>;
  constexpr int TBM = tile_rows(RB);   // query rows per workgroup
  static_assert(RB == 1 || MT == kMaskNone, "masked instances use one row block per wave");
  using MR = MaskRun<MT>;
  typedef typename MR::type MRun;
  constexpr int KS = T::KS;   // k-steps of the Q K^T product
  constexpr int DB = T::DB;   // 32-row blocks of O^T
  constexpr bool HAS_MASK = MT != kMaskNone;
  // two stages as separate objects: the compiler can then tell a copy into one stage
  // from reads of the other and does not wait for the copy before those reads
  __shared__ __attribute__((aligned(1024))) char stage0[T::STAGE];  // K tile, then V tile
  __shared__ __attribute__((aligned(1024))) char stage1[T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar copy bookkeeping
  const int col = lane & 31;   // query column owned by this lane
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group this lane holds

  // whole row tile (slot < 0), or key range [kb0, kb0 + split_tiles * BN) of a tail tile
  int logical, slot = -1, kb0 = 0;
  if ((int)blockIdx.x < p.n_full) {
    logical = xcd_remap(blockIdx.x, p.n_full);
  } else {
    slot = (int)blockIdx.x - p.n_full;
    logical = p.n_full + slot / p.nsplit;
    kb0 = (slot % p.nsplit) * p.split_tiles * BN;
  }
  int tile, h, b;
  split_logical(logical, p, tile, h, b);

  // ---- this lane's query rows (one per row block) ------------------------------
  int rr[RB], qi[RB];
  bool row_ok[RB], q_ok[RB];
  bf16x8 qf[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    rr[rb] = tile * TBM + (wave * RB + rb) * 32 + col;  // output row (compact index)
    row_ok[rb] = rr[rb] < p.n_rows;
    qi[rb] = rr[rb];
    if (GATHER) qi[rb] = row_ok[rb] ? p.q_rows[(int64_t)b * p.qr_bs + rr[rb]] : -1;
    q_ok[rb] = row_ok[rb] && qi[rb] >= 0 && qi[rb] < p.Nq;
    const u16* qp = p.q + (int64_t)b * p.qs0 + (int64_t)(q_ok[rb] ? qi[rb] : 0) * p.qs1 + (int64_t)h * p.qs2 + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      // columns past d (the upper half of the last k-step when d % 16 == 8) stay zero
      const bool in_row = s * 16 + 16 <= D || half == 0;
      if (q_ok[rb] && in_row) v = ld16(qp + s * 16);
      qf[rb][s] = as_bf16x8(v);
    }
  }

  int nkeys = p.Nk;
  if (KVLEN) {
    int L = p.kv_len[b];
    nkeys = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  const int kend = slot < 0 ? nkeys : min(nkeys, kb0 + p.split_tiles * BN);
  const int ntiles = (kend - kb0 + BN - 1) / BN;   // key ranges of splits are never empty

  // ---- per-lane copy plan ------------------------------------------------------
  // A tile is NCOPY wave-wide copies of 1 KB: copy c < K_SLOTS fills K slots
  // [64c, 64c + 64), the rest fill V.  Slot sigma is row sigma / SLOTS, chunk
  // sigma % SLOTS; pad chunks fetch chunk 0 of their row, so every lane is active.
  // Wave w issues copies c = w + NWAVES * m.  Rounds m < FULL are issued by every
  // wave and whether a round is K, V or mixed is a compile-time fact, so a full tile
  // costs one scalar select per mixed round and one uniform branch for the partial
  // last round: no per-copy branches (a taken branch refetches the wave's
  // instructions).
  constexpr int FULL = T::NCOPY / NWAVES;
  const char* kbase = reinterpret_cast<const char*>(p.k + (int64_t)b * p.ks0 + (int64_t)h * p.ks2);
  const char* vbase = reinterpret_cast<const char*>(p.v + (int64_t)b * p.vs0 + (int64_t)h * p.vs2);
  const int64_t krow_b = p.ks1 * 2, vrow_b = p.vs1 * 2;   // bytes between consecutive keys
  const char* kfresh = nullptr;                             // fused global K/V: fresh rows of (b, h)
  const char* vfresh = nullptr;
  if constexpr (KVMAP) {   // uniform, kept in scalar registers (the vector ones are all taken)
    kfresh = uniform_ptr(reinterpret_cast<const char*>(p.kf + (int64_t)b * p.fs0 + (int64_t)h * p.fs2));
    vfresh = uniform_ptr(reinterpret_cast<const char*>(p.vf + (int64_t)b * p.fs0 + (int64_t)h * p.fs2));
  }
  // This lane's copy plan, per copy: the byte offset of its chunk in a tile, or for the fused
  // global K/V, the byte offset of its row's K or V source address in a tile's address table
  // (below) << 16 | the chunk's bytes.  The fused form with two row blocks keeps the plan in
  // LDS (plan[wave][m][lane]), read back when a tile's copies issue: there the registers are
  // all taken by the products.
  constexpr bool PLAN_LDS = KVMAP && RB > 1;
  uint32_t coff[PLAN_LDS ? 1 : T::PER_WAVE];
  __shared__ __attribute__((aligned(256))) uint32_t planbuf[PLAN_LDS ? NWAVES * T::PER_WAVE * 64 : 1];
#pragma unroll
  for (int m = 0; m < T::PER_WAVE; ++m) {
    const int c = wave + NWAVES * m;
    const bool isk = c < T::K_SLOTS;
    const int slots = isk ? T::K_SLOTS : T::V_SLOTS;
    const int sigma = (isk ? c : c - T::K_SLOTS) * 64 + lane;
    const int row = sigma / slots;
    int chunk = sigma % slots;
    if (chunk >= T::CH) chunk = 0;
    uint32_t e = (uint32_t)(row * (isk ? krow_b : vrow_b) + chunk * 16);
    if constexpr (KVMAP) e = ((uint32_t)((row & (BN - 1)) * 16 + (isk ? 0 : 8)) << 16) | (uint32_t)(chunk * 16);
    if constexpr (PLAN_LDS) planbuf[(wave * T::PER_WAVE + m) * 64 + lane] = e;
    else coff[m] = e;
  }
  // Fused global K/V: each copy reads its key's row from the fresh rows or the cache, as the
  // source map says.  One wave (wave t % 4 for tile t, so the work rotates over the SIMDs)
  // turns a tile's 64 map entries into a table of the 64 keys' K and V source addresses
  // (addr[slot][row] = {K, V}, 16 bytes), two tiles ahead; a copy then costs one LDS read of
  // its row's address and one add.  The map of tile t reaches LDS (one dword copy) at step
  // t-3 into map slot t % 2, becomes table slot t % 2 at step t-2, and is read by every wave
  // for the copies of tile t at step t-1: each handover is ordered by a step's wait-and-
  // barrier, and a slot is rewritten only after the barrier that follows its last read.  Rows
  // past the valid keys take the tile's first key.
  __shared__ __attribute__((aligned(256))) int mapbuf[KVMAP ? 2 * BN : 1];
  __shared__ __attribute__((aligned(256))) char addrbuf[KVMAP ? 2 * BN * 16 : 1];
  const int32_t* smap =
      KVMAP ? reinterpret_cast<const int32_t*>(uniform_ptr(reinterpret_cast<const char*>(p.kv_src + (int64_t)b * p.src_bs)))
            : nullptr;
  auto load_map = [&](int t) {   // map entries of tile t (one wave)
    const int j0 = kb0 + t * BN;
    const int r = lane < nkeys - j0 ? lane : 0;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(smap + j0 + r),
                                     (lds_void*)(mapbuf + (t & 1) * BN), 4, 0, 0);
  };
  auto store_table = [&](int t, int src) {   // source addresses of tile t from its map entries (one wave)
    const int j0 = kb0 + t * BN;
    const int key = j0 + (lane < nkeys - j0 ? lane : 0);
    const bool fresh = (unsigned)src < (unsigned)p.nsel;
    const int64_t fo = (int64_t)src * p.fs1 * 2;
    u64x2 a;
    a[0] = reinterpret_cast<uint64_t>(fresh ? kfresh + fo : kbase + (int64_t)key * krow_b);
    a[1] = reinterpret_cast<uint64_t>(fresh ? vfresh + fo : vbase + (int64_t)key * vrow_b);
    *reinterpret_cast<u64x2*>(addrbuf + ((t & 1) * BN + lane) * 16) = a;
  };
  // A tile's copies through the table: every plan entry, then every address, is read before
  // the first copy issues (a copy writes LDS, so a read placed after one waits for it), and
  // the reads can be issued well before the copies.
  struct SrcPlan {
    uint32_t e[KVMAP ? T::PER_WAVE : 1];
    const char* from[KVMAP ? T::PER_WAVE : 1];
  };
  auto fetch_sources = [&](int j0, SrcPlan& sp) {
    const char* table = addrbuf + (((j0 - kb0) / BN) & 1) * BN * 16;
    // the plan's address redefined each tile, so no plan entry is hoisted into a register
    uint32_t pa = (uint32_t)((wave * T::PER_WAVE * 64 + lane) * 4);
    asm volatile("" : "+v"(pa));
    const char* plan = reinterpret_cast<const char*>(planbuf) + pa;
#pragma unroll
    for (int m = 0; m < T::PER_WAVE; ++m) {
      if (m < FULL || wave + NWAVES * m < T::NCOPY) {
        if constexpr (PLAN_LDS) {
          sp.e[m] = *reinterpret_cast<const uint32_t*>(plan + m * 256);
        } else {
          asm volatile("" : "+v"(coff[m]));
          sp.e[m] = coff[m];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < T::PER_WAVE; ++m)
      if (m < FULL || wave + NWAVES * m < T::NCOPY) sp.from[m] = *reinterpret_cast<const char* const*>(table + (sp.e[m] >> 16));
  };
  auto issue_sources = [&](const SrcPlan& sp, char* stage) {
    int wlds = __builtin_amdgcn_readfirstlane(wave * 1024);
    asm volatile("" : "+s"(wlds));
#pragma unroll
    for (int m = 0; m < T::PER_WAVE; ++m)
      if (m < FULL || wave + NWAVES * m < T::NCOPY)
        copy16_to_lds(sp.from[m] + (sp.e[m] & 0xffffu), stage + wlds + m * NWAVES * 1024);
  };
  auto issue_tile = [&](int j0, char* stage) {
    const char* kb = kbase + (int64_t)j0 * krow_b;
    const char* vb = vbase + (int64_t)j0 * vrow_b;
    const int nrow_valid = nkeys - j0;
    if constexpr (KVMAP) {
      // every copy from its row's source address in the tile's table (rows past the valid
      // keys hold the first key's), plus the chunk's bytes
      SrcPlan sp;
      fetch_sources(j0, sp);
      issue_sources(sp, stage);
      return;
    }
    if (nrow_valid >= BN) {
      // The empty asm statements redefine the offsets in place each tile: the 32-bit
      // lane offsets are then not widened and hoisted out of the loop (the copy keeps
      // the scalar-base form, base in SGPRs + 32-bit lane offset), and the LDS
      // destinations are one scalar add each instead of precomputed registers.
      int wlds = wave * 1024;
      asm volatile("" : "+s"(wlds));
#pragma unroll
      for (int m = 0; m < T::PER_WAVE; ++m) {
        const int c = wave + NWAVES * m;
        const bool all_k = NWAVES * m + NWAVES - 1 < T::K_SLOTS;  // compile-time per unrolled m
        const bool all_v = NWAVES * m >= T::K_SLOTS;
        const char* base = all_k ? kb : (all_v ? vb : (c < T::K_SLOTS ? kb : vb));
        asm volatile("" : "+v"(coff[m]));
        if (m < FULL || c < T::NCOPY) copy16_to_lds(base + coff[m], stage + wlds + m * NWAVES * 1024);
      }
    } else {
      // last, partial tile: rows past the valid keys fetch row 0 of the tile instead
      // (lane laundered so none of this is hoisted into registers live across the loop)
      int ln = lane, wv = wave;
      asm volatile("" : "+v"(ln), "+s"(wv));
#pragma unroll
      for (int m = 0; m < T::PER_WAVE; ++m) {
        const int c = wv + NWAVES * m;
        if (c < T::NCOPY) {
          const bool isk = c < T::K_SLOTS;
          const int row = ((isk ? c : c - T::K_SLOTS) * 64 + ln) / (isk ? T::K_SLOTS : T::V_SLOTS);
          const uint32_t off = row < nrow_valid ? coff[m] : coff[m] - (uint32_t)(row * (isk ? krow_b : vrow_b));
          copy16_to_lds((isk ? kb : vb) + off, stage + c * 1024);
        }
      }
    }
  };

  // ---- mask runs: run i of a tile covers keys 32 (i / 4) + 8 (i % 4) + 4 half + 0..3 ----
  // Whole tiles are loaded one tile ahead.  Staged (when the LDS leaves room for two
  // workgroups per CU): the wave's 32 rows of the next tile are copied straight into the
  // wave's own LDS rows (NMI direct-to-LDS copies per lane, issued with the K/V copies and
  // covered by the same wait), then read back as runs -- a copy touches 8 or fewer cache
  // lines instead of the 32 a run load would, and no registers or LDS writes stage them.
  // Row r's 16-byte chunk c sits at position c ^ rot(r), rot(r) = (r / (16 / CPR)) % CPR, so
  // the 16 rows one run read touches cover all banks.  Otherwise the runs are loaded
  // directly (8 loads per lane).
  constexpr int CPR = 4 * MR::esz;                                  // 16-byte chunks per row of a tile
  constexpr int NMI = HAS_MASK ? 32 * CPR / 64 : 1;                 // staging copies per lane
  constexpr int MRS = CPR * 16;                                     // LDS row stride (no padding)
  constexpr int RPB = 16 / CPR;                                     // rows per 256 bytes of LDS
  constexpr bool STAGED = HAS_MASK && 2 * T::STAGE + NWAVES * 32 * MRS <= 80 * 1024;
  __shared__ __attribute__((aligned(1024))) char mstage[STAGED ? NWAVES * 32 * MRS : 16];
  char* const mw = mstage + (STAGED ? wave * 32 * MRS : 0);          // this wave's LDS rows
  const char* mrow = nullptr;   // this lane's own row (and half): direct and partial-tile loads
  const char* mld[NMI];         // the row chunk this lane copies, its rotation included
  if constexpr (HAS_MASK) {
    const char* mbh = p.mask + ((int64_t)b * p.ms0 + (int64_t)h * p.ms1) * MR::esz;
    const int qrow = q_ok[0] ? qi[0] : 0;
    mrow = mbh + ((int64_t)qrow * p.ms2 + 4 * half) * MR::esz;
#pragma unroll
    for (int i = 0; i < NMI; ++i) {
      const int q = i * 64 + lane;            // LDS slot: row q / CPR, position q % CPR
      const int r = q / CPR;
      const int src_row = __shfl(qrow, r);    // lane r < 32 holds row r's token
      const int chunk = (q % CPR) ^ ((r / RPB) % CPR);
      mld[i] = mbh + (int64_t)src_row * p.ms2 * MR::esz + chunk * 16;
    }
  }
  typedef u32x4 MStage[1];   // (unused: the staged rows go straight to LDS)
  auto stage_load = [&](int j0, MStage&) {
    if constexpr (STAGED) {
      // this wave's run reads of the rows must be done before the copies overwrite them
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
#pragma unroll
      for (int i = 0; i < NMI; ++i) copy16_to_lds(mld[i] + (int64_t)j0 * MR::esz, mw + i * 1024);
    }
  };
  auto stage_runs = [&](const MStage&, MRun (&r)[8]) {   // the wave's LDS rows -> runs
    if constexpr (STAGED) {
      const int rot = (col / RPB) % CPR;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int byte = (32 * (i >> 2) + 8 * (i & 3) + 4 * half) * MR::esz;
        r[i] = *reinterpret_cast<const MRun*>(mw + col * MRS + (((byte >> 4) ^ rot) << 4) + (byte & 15));
      }
    }
  };
  auto load_runs = [&](int j0, MRun (&r)[8]) {        // direct: a whole tile, every key valid
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = *reinterpret_cast<const MRun*>(mrow + (int64_t)(j0 + 32 * (i >> 2) + 8 * (i & 3)) * MR::esz);
  };
  auto load_runs_partial = [&](int j0, MRun (&r)[8]) {   // element loads below nkeys
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      MRun c = {};
      if constexpr (MT == kMaskBool) c = 0x01010101u;   // neutral: attend (masked by length later)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rel = 32 * (i >> 2) + 8 * (i & 3) + e;
        if (j0 + 4 * half + rel < nkeys) {
          const char* ep = mrow + (int64_t)(j0 + rel) * MR::esz;
          if constexpr (MT == kMaskBool) {
            c = (c & ~(0xFFu << (8 * e))) | ((u32)*reinterpret_cast<const unsigned char*>(ep) << (8 * e));
          } else if constexpr (MT != kMaskNone && MR::esz == 2) {
            c[e >> 1] |= (u32)*reinterpret_cast<const u16*>(ep) << (16 * (e & 1));
          } else if constexpr (MR::esz == 4) {
            c[e] = *reinterpret_cast<const u32*>(ep);
          }
        }
      }
      r[i] = c;
    }
  };

  f32x16 oacc[RB][DB];
  float m_ref[RB], l_run[RB];   // reference max (log2 domain; -FLT_MAX: none yet), this lane's row-sum share
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[rb][i] = f32x16{};
    m_ref[rb] = -FLT_MAX;
    l_run[rb] = 0.f;
  }
  const float sl2 = p.scale_log2;

  // LDS addresses of this lane's operand reads (byte offsets inside a tile)
  const int k_lane = col * T::K_ROWB + half * 16;
  const int grp = (lane >> 4) & 3, src = lane & 15;
  const int v_lane = (4 * (grp >> 1) + (src >> 2)) * T::V_ROWB + (16 * (grp & 1) + 4 * (src & 3)) * 2;

  // Per-lane pieces of a tile.  A tile's two 32-key halves are independent once
  // scores exist: probabilities are taken against the current reference, so the
  // softmax of one half can run between the MFMAs of the other half.
  auto s_half = [&](const char* Kt, int blk, f32x16 (&acc)[RB]) {   // S^T rows blk*32.. of the tile
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kf = as_bf16x8(ld16(Kt + k_lane + blk * 32 * T::K_ROWB + s * 32));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[rb][s], acc[rb], 0, 0, 0);
    }
  };
  auto fold_half = [&](f32x16& sc, int blk, const MRun (&r)[8]) {
    if constexpr (HAS_MASK) {
#pragma unroll
      for (int g = 0; g < 4; ++g) fold_run<MT>(sc, g, r[4 * blk + g], p.inv_scale);
    }
  };
  // bf16 P^T operands of one half and this lane's share of its sum
  auto probs_half = [&](const f32x16& sc, bf16x8 (&pb)[2], int rb) -> float {
    float ts = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * t + 2 * e], sl2, -m_ref[rb]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * t + 2 * e + 1], sl2, -m_ref[rb]));
        packed[e] = pack_bf16x2(p0, p1);
        ts = (t == 0 && e == 0) ? p0 + p1 : ts + (p0 + p1);   // 0 + x is not folded (signed zeros)
      }
      pb[t] = as_bf16x8(packed);
    }
    return ts;
  };
  // Reference move (rare, wave-uniform): the first half-tile (reference -FLT_MAX gives
  // +inf), or a half whose probabilities grew past 2^16 / 16 somewhere.  The rows
  // whose pair max exceeds the reference by more than 2^8 move it; O and l (which
  // hold every earlier half) are rescaled and the half is recomputed.  A row whose
  // keys are all blocked so far (-inf scores) keeps the reference at -FLT_MAX, its
  // probabilities exp2(-inf) = 0 and O and l zero.
  auto settle_half = [&](const f32x16& sc, bf16x8 (&pb)[2], float ts, int rb) -> float {
    if (__any(!(ts <= kSumLimit))) {
      float mt = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mt2 = mt * sl2;
      const bool move = mt2 > m_ref[rb] + kRescaleThreshold;
      const float m_new = move ? mt2 : m_ref[rb];
      const float alpha = __builtin_amdgcn_exp2f(m_ref[rb] - m_new);  // 0 on the first move
      l_run[rb] *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[rb][i] *= alpha;
      m_ref[rb] = m_new;
      ts = probs_half(sc, pb, rb);
    }
    return ts;
  };
  auto pv_half = [&](const char* Vt, int blk, const bf16x8 (&pb)[RB][2]) {   // O^T += V^T P^T, one half
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const char* vp = Vt + v_lane + (blk * 32 + t * 16) * T::V_ROWB + db * 64;
        const i16x4 lo = lds_read_tr(vp);
        const i16x4 hi = lds_read_tr(vp + 8 * T::V_ROWB);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[rb][t], oacc[rb][db], 0, 0, 0);
      }
  };
  // keys past the valid length get -inf (the partial last tile only)
  auto mask_half = [&](f32x16& sc, int j0, int blk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + blk * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key >= nkeys) sc[r] = -INFINITY;
    }
  };

  // One tile: wait for its copies (and mask data), start the next tile's copies into
  // the other stage (and its mask loads into the other register set), then S^T half 0;
  // [S^T half 1 | softmax half 0]; [PV half 0 | softmax half 1]; PV half 1.  Each
  // bracket is one basic block, so the scheduler interleaves the MFMAs of one half
  // with the VALU work of the other; the rare reference moves sit between them.
  // MASKED is the partial last tile: it loads its own mask runs, masks by length and
  // issues no copies.  The fused global K/V reads the next tile's source addresses at the
  // top and issues its copies after S^T half 0, so the two LDS round trips of those reads
  // are hidden behind products instead of delaying them.
  auto tile_step = [&](auto masked, int it, const char* cur, char* nxt, MRun (&mc)[8], MRun (&mn)[8],
                       MStage& sc_, MStage& sn_) {
    constexpr bool MASKED = decltype(masked)::value;
    const int j0 = kb0 + it * BN;
    SrcPlan sp;       // fused global K/V: the next tile's sources
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile `it` landed
    __syncthreads();                     // ... everyone's, and tile it-1 is no longer read
    if constexpr (!MASKED) {
      if constexpr (STAGED) stage_runs(sc_, mc);
      // the next tile's copies go out first at the top priority: the sooner they are in
      // flight, the more of the tile hides their latency (+1-2%)
      __builtin_amdgcn_s_setprio(2);
      if (it + 1 < ntiles) {
        // the fused global K/V reads its sources here and copies after the first products
        if constexpr (KVMAP) fetch_sources(j0 + BN, sp);
        else issue_tile(j0 + BN, nxt);
        if constexpr (HAS_MASK) {
          if (j0 + 2 * BN <= kend) {
            if constexpr (STAGED) stage_load(j0 + BN, sn_);
            else load_runs(j0 + BN, mn);
          }
        }
      }
      if constexpr (KVMAP) {
        // one wave, in turn: the table of tile it+2 from its map (landed before this step's
        // barrier), then the map of tile it+3 into the slot that the map of tile it+1 left
        // (read in the step before, so no wait)
        if (wave == ((it + 2) & (NWAVES - 1)) && it + 2 < ntiles) {
          store_table(it + 2, mapbuf[((it + 2) & 1) * BN + lane]);
          if (it + 3 < ntiles) load_map(it + 3);
        }
      }
    } else if constexpr (HAS_MASK) {
      load_runs_partial(j0, mc);
    }
    const char* Kt = cur;
    const char* Vt = cur + T::K_BYTES;
    __builtin_amdgcn_s_setprio(0);

    f32x16 s0[RB], s1[RB];
    bf16x8 pb0[RB][2], pb1[RB][2];
    float ts0[RB], ts1[RB];
    s_half(Kt, 0, s0);
    if constexpr (KVMAP && !MASKED) {   // the sources were read at the top: no wait here
      if (it + 1 < ntiles) issue_sources(sp, nxt);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      fold_half(s0[rb], 0, mc);
      if constexpr (MASKED) mask_half(s0[rb], j0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // The two middle brackets carry the softmax: their VALU work is this wave's critical
    // path, so the wave issues ahead of its SIMD partner (whose own S^T half 0 or P V
    // half 1 is MFMA work only) until P V half 1 (+2-3%).
    __builtin_amdgcn_s_setprio(1);
    s_half(Kt, 1, s1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      fold_half(s1[rb], 1, mc);
      if constexpr (MASKED) mask_half(s1[rb], j0, 1);
      ts0[rb] = probs_half(s0[rb], pb0[rb], rb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ts0[rb] = settle_half(s0[rb], pb0[rb], ts0[rb], rb);
      l_run[rb] += ts0[rb];
    }
    pv_half(Vt, 0, pb0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ts1[rb] = probs_half(s1[rb], pb1[rb], rb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ts1[rb] = settle_half(s1[rb], pb1[rb], ts1[rb], rb);
      l_run[rb] += ts1[rb];
    }
    __builtin_amdgcn_s_setprio(0);
    pv_half(Vt, 1, pb1);
  };

  const std::integral_constant<bool, false> kFull;
  const std::integral_constant<bool, true> kMasked;
  MRun mA[8], mB[8];        // mask runs of the even / odd tiles (unused without a mask)
  MStage sA, sB;            // staged mask loads of the even / odd tiles (unused unless STAGED)
  const int nfull = (kend - kb0) / BN;   // tiles whose 64 keys are all valid
  if constexpr (KVMAP) {
    // the tables of tiles 0 and 1, and the map of tile 2, before the first copies
    if (ntiles > 0) {
      if (wave == 0) {
        load_map(0);
        if (ntiles > 1) load_map(1);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the maps landed
      __syncthreads();
      if (wave == 0) {
        store_table(0, mapbuf[lane]);
        if (ntiles > 1) store_table(1, mapbuf[BN + lane]);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): map slot 0 has been read
        if (ntiles > 2) load_map(2);
      }
      __syncthreads();                       // the tables are visible
    }
  }
  if (ntiles > 0) issue_tile(kb0, stage0);
  if constexpr (HAS_MASK) {
    if (nfull > 0) {
      if constexpr (STAGED) stage_load(kb0, sA);
      else load_runs(kb0, mA);
    }
  }
  int it = 0;
  for (; it + 2 <= nfull; it += 2) {
    tile_step(kFull, it, stage0, stage1, mA, mB, sA, sB);
    tile_step(kFull, it + 1, stage1, stage0, mB, mA, sB, sA);
  }
  if (it < nfull) {
    tile_step(kFull, it, stage0, stage1, mA, mB, sA, sB);
    ++it;
  }
  if (it < ntiles) tile_step(kMasked, it, (it & 1) ? stage1 : stage0, nullptr, mA, mB, sA, sB);

  // ---- epilogue: normalise, store O (bf16) and LSE ------------------------------
  float l_tot[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) l_tot[rb] = l_run[rb] + __shfl_xor(l_run[rb], 32);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!row_ok[rb]) continue;
    if (slot >= 0) {  // partial of a split tile: unnormalised O and this range's (max, sum)
      const int rloc = (wave * RB + rb) * 32 + col;
      float* po = p.part + ((int64_t)slot * TBM + rloc) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (db * 32 + 8 * g >= D) continue;   // padded O rows (d % 32 != 0)
          const f32x4 w = {oacc[rb][db][4 * g + 0], oacc[rb][db][4 * g + 1], oacc[rb][db][4 * g + 2], oacc[rb][db][4 * g + 3]};
          st16(po + db * 32 + 8 * g + 4 * half, __builtin_bit_cast(u32x4, w));
        }
      if (half == 0) {
        float* pm = p.part + (int64_t)p.n_slots * TBM * D + ((int64_t)slot * TBM + rloc) * 2;
        pm[0] = m_ref[rb];
        pm[1] = l_tot[rb];
      }
      continue;
    }
    const float inv = l_tot[rb] > 0.f ? 1.0f / l_tot[rb] : 0.f;
    const int orow = (GATHER && p.scatter) ? qi[rb] : rr[rb];
    if (!GATHER || !p.scatter || q_ok[rb]) {
      u16* op = p.o + (int64_t)b * p.os0 + (int64_t)orow * p.os1 + (int64_t)h * p.os2;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (db * 32 + 8 * g >= D) continue;   // padded O rows (d % 32 != 0)
          u32x2 w;
          w[0] = pack_bf16x2(oacc[rb][db][4 * g + 0] * inv, oacc[rb][db][4 * g + 1] * inv);
          w[1] = pack_bf16x2(oacc[rb][db][4 * g + 2] * inv, oacc[rb][db][4 * g + 3] * inv);
          st8(op + db * 32 + 8 * g + 4 * half, w);
        }
    }
    if (p.lse != nullptr && half == 0) {
      const float lse = l_tot[rb] > 0.f ? (m_ref[rb] + __builtin_log2f(l_tot[rb])) * 0.69314718055994530942f : -INFINITY;
      p.lse[((int64_t)b * p.H + h) * p.n_rows + rr[rb]] = lse;
    }
  }
}

// Merge the key-range partials of each split tail tile: M = max of the ranges' maxima,
// L = sum of their sums scaled by 2^(max - M), O = sum of their O scaled the same way
// over L; the same output rules as the whole-tile epilogue.  A workgroup takes 32 rows
// of a tile, MergeShape<D>::TPR threads per row, each owning DT consecutive columns.
constexpr int MERGE_ROWS = 32;
template <int D>
struct MergeShape {
  static constexpr int TPR = D % 32 == 0 ? 8 : 6;   // threads per row
  static constexpr int DT = D / TPR;                // columns per thread: 4, 8, 12 or 16
  static_assert(D % (4 * TPR) == 0, "whole 4-column groups per thread");
};
template <int D, bool GATHER, int TBM>
__global__ __launch_bounds__(MERGE_ROWS * 8) void attn_merge_kernel(AttnParams p) {
  constexpr int TPR = MergeShape<D>::TPR;
  constexpr int DT = MergeShape<D>::DT;
  const int ti = blockIdx.x;
  const int logical = p.n_full + ti;
  int tile, h, b;
  split_logical(logical, p, tile, h, b);
  const int rloc = blockIdx.y * MERGE_ROWS + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  const int rr = tile * TBM + rloc;
  if (rr >= p.n_rows) return;
  int qi = rr;
  if (GATHER) qi = p.q_rows[(int64_t)b * p.qr_bs + rr];
  const bool q_ok = qi >= 0 && qi < p.Nq;

  const float* pml = p.part + (int64_t)p.n_slots * TBM * D;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, pml[((int64_t)(ti * p.nsplit + s) * TBM + rloc) * 2]);
  float acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = 0.f;
  float L = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const int64_t sl = (int64_t)(ti * p.nsplit + s) * TBM + rloc;
    const float w = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pml[sl * 2] - M);
    L += w * pml[sl * 2 + 1];
    const float* po = p.part + sl * D + part * DT;
#pragma unroll
    for (int i = 0; i < DT; i += 4) {
      const f32x4 v = __builtin_bit_cast(f32x4, ld16(po + i));
      acc[i] += w * v[0]; acc[i + 1] += w * v[1]; acc[i + 2] += w * v[2]; acc[i + 3] += w * v[3];
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int orow = (GATHER && p.scatter) ? qi : rr;
  if (!GATHER || !p.scatter || q_ok) {
    u16* op = p.o + (int64_t)b * p.os0 + (int64_t)orow * p.os1 + (int64_t)h * p.os2 + part * DT;
#pragma unroll
    for (int i = 0; i < DT; i += 4) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[i] * inv, acc[i + 1] * inv);
      w[1] = pack_bf16x2(acc[i + 2] * inv, acc[i + 3] * inv);
      st8(op + i, w);
    }
  }
  if (p.lse != nullptr && part == 0) {
    const float lse = L > 0.f ? (M + __builtin_log2f(L)) * 0.69314718055994530942f : -INFINITY;
    p.lse[((int64_t)b * p.H + h) * p.n_rows + rr] = lse;
  }
}

template <int D, bool G, bool KV, int MT, int RB, bool KVMAP = false>
hipError_t launch(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, G, KV, MT, RB, KVMAP>), dim3(p.total_wg), dim3(NTHREADS), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_slots == 0) return e;
  hipLaunchKernelGGL((attn_merge_kernel<D, G, tile_rows(RB)>), dim3(p.n_slots / p.nsplit, tile_rows(RB) / MERGE_ROWS),
                     dim3(MERGE_ROWS * MergeShape<D>::TPR), 0, s, p);
  return hipGetLastError();
}

// Workgroups of one kernel instance resident on the whole device (0 if unknown).
// Cached per device and instance; racing first calls store the same value.
template <int D, bool G, bool KV, int MT, int RB, bool KVMAP = false>
int resident_workgroups() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_kernel<D, G, KV, MT, RB, KVMAP>, NTHREADS, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  v = per_cu * cus;
  if (v > 0) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace
}  // namespace safe
