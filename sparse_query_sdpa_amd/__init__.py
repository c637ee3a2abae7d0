"""Python binding of libsafe, the MI355X (gfx950) SAFE-DiT attention hot path.

Argument marshalling only: every step runs in the HIP kernels of libsafe.so;
PyTorch supplies device memory and the current HIP stream.  There is no CPU
fallback: importing the package fails loudly when the library is missing.

Entry points (the C ABI in include/safe.h, same names without the safe_ prefix):
  mask_classify   -- Eq. 6-8 row-constant certification of an attention mask
  pcsp_accumulate -- Eq. 9-10 image->text sensitivity scores (safe_pcsp_select, ACCUM)
  pcsp_select     -- Eq. 11-12 smoothing, Norm and the ascending top-k set S (SELECT)
  kv_assemble     -- Eq. 14, 16 global K/V from fresh rows over cached rows
  kv_source_map   -- the per-token map of the fused global K/V read (Eq. 14, 16 in one pass)
  attn_fwd        -- Eq. 2, 16-18 attention, dense or on gathered rows, with kv_len or a mask
  sdpa            -- Eq. 8 the rewrite as one call: certify the mask, run the exact cheapest form
  attn_plan, attn_workspace_bytes -- the schedule and split workspace of an attn_fwd call
  sw_cfg          -- Eq. 20-21 sensitivity-weighted classifier-free guidance
  linear          -- Eq. 15 row-wise linear maps on gathered rows (the block around attention)
  block_dense, block_srsu -- that block as a sequence of the calls above
  mfma_probe, hbm_probe -- measurement aids: the matrix-core and streaming memory rates of the GPU
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SAFE_LIB_PATH selects another build of the same library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("SAFE_LIB_PATH") or os.path.join(_HERE, "libsafe.so")

SAFE_OK = 0
STATUS = {0: "SAFE_OK", -1: "SAFE_ERR_NULL", -2: "SAFE_ERR_SHAPE", -3: "SAFE_ERR_DTYPE", -4: "SAFE_ERR_RANGE",
          -5: "SAFE_ERR_UNSUPPORTED", -6: "SAFE_ERR_WORKSPACE", -7: "SAFE_ERR_HIP", -8: "SAFE_ERR_ALIGN"}

FLAG_CHECK = 1 << 0
ATTN_SCATTER_OUT = 1 << 1
CLASSIFY_ASYNC = 1 << 2
PCSP_ACCUM = 1 << 3
PCSP_SELECT = 1 << 4

ABI_VERSION = 10  # struct layouts below match include/safe.h of this version
DT_BOOL, DT_BF16, DT_F16, DT_F32 = 0, 1, 2, 3
MASK_CLASS_NAMES = ("ALL_VALID", "ZERO", "ROW_CONST", "KEY_PADDING", "NONCONST", "BLOCKED", "NONFINITE")

_i64x3 = ctypes.c_int64 * 3
_i64x4 = ctypes.c_int64 * 4


class MaskInfo(ctypes.Structure):
    _fields_ = [("verdict", ctypes.c_int32), ("mask_class", ctypes.c_int32),
                ("first_bad_row", ctypes.c_int64), ("rows", ctypes.c_int64)]


class PcspArgs(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("M", ctypes.c_int32),
                ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("q_stride", _i64x3),
                ("k_text", ctypes.c_void_p), ("k_stride", _i64x3),
                ("kv_len", ctypes.c_void_p), ("w", ctypes.c_void_p), ("head_mask", ctypes.c_uint64),
                ("scale", ctypes.c_float), ("acc", ctypes.c_void_p),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32), ("sigma", ctypes.c_float),
                ("k", ctypes.c_int32), ("score_out", ctypes.c_void_p), ("idx_out", ctypes.c_void_p)]


class KvArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("nsel", ctypes.c_int32),
                ("k_fresh", ctypes.c_void_p), ("v_fresh", ctypes.c_void_p), ("fresh_stride", _i64x3),
                ("idx", ctypes.c_void_p), ("idx_bstride", ctypes.c_int64),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("cache_stride", _i64x3),
                ("k_out", ctypes.c_void_p), ("v_out", ctypes.c_void_p), ("out_stride", _i64x3),
                ("flags", ctypes.c_uint32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32),
                ("d", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("q_stride", _i64x3),
                ("k", ctypes.c_void_p), ("k_stride", _i64x3),
                ("v", ctypes.c_void_p), ("v_stride", _i64x3),
                ("o", ctypes.c_void_p), ("o_stride", _i64x3),
                ("q_rows", ctypes.c_void_p), ("n_rows", ctypes.c_int32), ("q_rows_bstride", ctypes.c_int64),
                ("kv_len", ctypes.c_void_p), ("scale", ctypes.c_float), ("lse", ctypes.c_void_p),
                ("flags", ctypes.c_uint32), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
                ("mask", ctypes.c_void_p), ("mask_dtype", ctypes.c_int32), ("mask_stride", _i64x3),
                ("kv_src", ctypes.c_void_p), ("kv_src_bstride", ctypes.c_int64),
                ("k_fresh", ctypes.c_void_p), ("v_fresh", ctypes.c_void_p), ("fresh_stride", _i64x3),
                ("n_fresh", ctypes.c_int32)]


class SdpaInfo(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int32), ("mask_class", ctypes.c_int32), ("first_bad_row", ctypes.c_int64)]


ROUTE_NAMES = ("no_mask", "kv_len", "mask")


class AttnPlanInfo(ctypes.Structure):
    _fields_ = [("rows_per_tile", ctypes.c_int32), ("row_tiles", ctypes.c_int32),
                ("split_tiles", ctypes.c_int32), ("key_ranges", ctypes.c_int32),
                ("keys_per_range", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]


class CfgArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("C", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("f_c", ctypes.c_void_p), ("f_u", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("stride", ctypes.c_int64 * 2),
                ("s", ctypes.c_void_p), ("s_bstride", ctypes.c_int64),
                ("idx", ctypes.c_void_p), ("k", ctypes.c_int32), ("idx_bstride", ctypes.c_int64),
                ("g_ctx", ctypes.c_float), ("g_sens", ctypes.c_float)]


class LinearArgs(ctypes.Structure):
    _fields_ = [("batches", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("a", ctypes.c_void_p), ("a_stride", ctypes.c_int64 * 2),
                ("w", ctypes.c_void_p), ("w_stride", ctypes.c_int64),
                ("bias", ctypes.c_void_p), ("act", ctypes.c_int32),
                ("res", ctypes.c_void_p), ("res_stride", ctypes.c_int64 * 2),
                ("out", ctypes.c_void_p), ("out_stride", ctypes.c_int64 * 2),
                ("a_rows", ctypes.c_void_p), ("res_rows", ctypes.c_void_p), ("out_rows", ctypes.c_void_p),
                ("rows_bstride", ctypes.c_int64), ("Ntok", ctypes.c_int32), ("flags", ctypes.c_uint32)]


ACT_NONE, ACT_GELU_TANH = 0, 1


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libsafe.so not found at {LIB_PATH}: build it with "
                          "`python sparse_query_sdpa_amd/build.py` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.safe_abi_version.restype = ctypes.c_int
    if lib.safe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.safe_abi_version()}, this binding needs "
                          f"{ABI_VERSION}: rebuild with `python sparse_query_sdpa_amd/build.py`")
    lib.safe_status_str.restype = ctypes.c_char_p
    lib.safe_status_str.argtypes = [ctypes.c_int]
    lib.safe_attn_fwd.restype = ctypes.c_int
    lib.safe_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.safe_attn_fwd_noalloc.restype = ctypes.c_int
    lib.safe_attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.safe_sdpa.restype = ctypes.c_int
    lib.safe_sdpa.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                              ctypes.POINTER(SdpaInfo), ctypes.c_void_p]
    lib.safe_sw_cfg.restype = ctypes.c_int
    lib.safe_sw_cfg.argtypes = [ctypes.POINTER(CfgArgs), ctypes.c_void_p]
    lib.safe_attn_workspace_bytes.restype = ctypes.c_int64
    lib.safe_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs)]
    lib.safe_attn_plan.restype = ctypes.c_int
    lib.safe_attn_plan.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(AttnPlanInfo)]
    lib.safe_kv_assemble.restype = ctypes.c_int
    lib.safe_kv_assemble.argtypes = [ctypes.POINTER(KvArgs), ctypes.c_void_p]
    lib.safe_kv_source_map.restype = ctypes.c_int
    lib.safe_kv_source_map.argtypes = [ctypes.POINTER(KvArgs), ctypes.c_void_p, ctypes.c_void_p]
    lib.safe_pcsp_select.restype = ctypes.c_int
    lib.safe_pcsp_select.argtypes = [ctypes.POINTER(PcspArgs), ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.c_void_p]
    lib.safe_linear.restype = ctypes.c_int
    lib.safe_linear.argtypes = [ctypes.POINTER(LinearArgs), ctypes.c_void_p]
    lib.safe_mfma_probe.restype = ctypes.c_int
    lib.safe_mfma_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.safe_hbm_probe.restype = ctypes.c_int
    lib.safe_hbm_probe.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.safe_mask_classify.restype = ctypes.c_int
    lib.safe_mask_classify.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.c_uint32, ctypes.POINTER(MaskInfo),
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    return lib


lib = _load()


class SafeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {lib.safe_status_str(status).decode()} ({status})")
        self.status = status


def _check(fn: str, status: int):
    if status != SAFE_OK:
        raise SafeError(fn, status)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    """Device address of a tensor passed to the library (every tensor argument is device memory)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments must be device tensors")
    return t.data_ptr()


def _need(t: torch.Tensor, shape, name: str):
    """A caller-provided tensor must have exactly the shape the call reads or writes."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _bnhd(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, N, H, d]")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name}: the head dimension d must be contiguous")
    return _i64x3(t.stride(0), t.stride(1), t.stride(2))


def _bits16(t: torch.Tensor, name: str):
    """Every attention, assembly and linear operand is read and written as bfloat16 (the
    C ABI has no dtype field for them): any other dtype is refused, fp16 included."""
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a torch.bfloat16 tensor, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _i32(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_cuda:
        raise TypeError(f"{name} must be an int32 device tensor")
    return t


def _lengths(t: Optional[torch.Tensor], B: int, name: str = "kv_len"):
    """Per-sample lengths: an int32 device tensor of exactly B entries (one per sample)."""
    t = _i32(t, name)
    if t is not None and (t.dim() != 1 or t.shape[0] != B or (B > 1 and t.stride(0) != 1)):
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape [{B}], got {list(t.shape)}")
    return t


def _row_lists(t: Optional[torch.Tensor], B: int, name: str):
    """(rows per sample, sample stride) of an index list [n] / [1, n] (shared by every
    sample: stride 0) or [B, n] (one list per sample); rows contiguous."""
    if t is None:
        return None, 0
    if t.dim() == 1:
        if t.shape[0] > 1 and t.stride(0) != 1:
            raise ValueError(f"{name} must be contiguous")
        return t.shape[0], 0
    if t.dim() != 2 or t.shape[0] not in (1, B) or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be [n], [1, n] or [{B}, n] with contiguous rows, got {list(t.shape)}")
    return t.shape[1], (0 if t.shape[0] == 1 else t.stride(0))


# ---------------------------------------------------------------------------------
_ATTN_WS = {}      # (device index, stream handle) -> uint8 workspace tensor, grown on demand
_RETIRED_WS = []   # superseded workspaces: never freed, a captured graph may still write them


def _cached_workspace(cache: dict, key, need: int, device: torch.device, what: str) -> torch.Tensor:
    """The workspace cached for (device, stream), grown when a call needs more.  A buffer
    that a HIP graph may have captured must outlive the graph, so a superseded buffer is
    kept alive rather than returned to the allocator; during capture nothing is allocated
    (run the call once eagerly on the capture stream first, or pass a workspace tensor)."""
    ws = cache.get(key)
    if ws is None or ws.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(f"{what}: the cached workspace of this stream is smaller than the captured call "
                               f"needs ({need} bytes); run the call once before capturing it, or pass an explicit "
                               "workspace tensor")
        if ws is not None:
            _RETIRED_WS.append(ws)
        ws = torch.empty(int(need), dtype=torch.uint8, device=device)
        cache[key] = ws
    return ws


def _attn_workspace(a: AttnArgs, device: torch.device, stream_handle) -> Optional[torch.Tensor]:
    need = lib.safe_attn_workspace_bytes(ctypes.byref(a))
    if need < 0:
        _check("safe_attn_workspace_bytes", int(need))
    if need <= 0:
        return None
    return _cached_workspace(_ATTN_WS, (device.index, stream_handle), int(need), device, "attn_fwd")


def _attn_mask(mask: Optional[torch.Tensor], B: int, H: int, Nq: int, Nk: int):
    """(pointer, dtype code, element strides of b, h, i) of a [B|1, H|1, Nq|1, Nk] mask."""
    if mask is None:
        return None, 0, (0, 0, 0)
    if mask.dim() != 4 or mask.dtype not in _MASK_DT:
        raise ValueError("mask must be a 4-D bool/uint8/bfloat16/float16/float32 tensor [B|1, H|1, Nq|1, Nk]")
    for got, full in zip(mask.shape, (B, H, Nq, Nk)):
        if got != full and got != 1:
            raise ValueError(f"mask shape {tuple(mask.shape)} does not broadcast to {(B, H, Nq, Nk)}")
    if mask.shape[3] != Nk or (Nk > 1 and mask.stride(3) != 1):
        raise ValueError("mask keys must be the last, contiguous dimension")
    st = tuple(0 if mask.shape[i] == 1 else mask.stride(i) for i in range(3))
    return _ptr(mask), _MASK_DT[mask.dtype], st


def _attn_call(q, k, v, q_rows, kv_len, scale, out, return_lse, scatter_out, check, mask, kv_src, k_fresh,
               v_fresh):
    """Checked AttnArgs of a call plus its output tensors: (args or None when there is nothing
    to compute, out, lse)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bits16(t, n)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k and v must be 4-D [B, N, H, d]")
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    if k.shape != (B, Nk, H, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Nk, H, d] matching q")
    q_rows = _i32(q_rows, "q_rows")
    kv_len = _lengths(kv_len, B)
    if q_rows is not None:
        n_rows, bstride = _row_lists(q_rows, B, "q_rows")
    else:
        n_rows, bstride = Nq, 0
    if out is None:
        out = torch.empty((B, Nq if scatter_out else n_rows, H, d), dtype=q.dtype, device=q.device)
    _bits16(out, "out")
    _need(out, (B, Nq if scatter_out else n_rows, H, d), "out")
    lse = torch.empty((B, H, n_rows), dtype=torch.float32, device=q.device) if return_lse else None
    if q_rows is not None and n_rows == 0:   # an empty row list has no storage pointer: nothing to compute
        return None, out, lse
    a = AttnArgs(B, H, Nq, Nk, d, _ptr(q), _bnhd(q, "q"), _ptr(k), _bnhd(k, "k"), _ptr(v), _bnhd(v, "v"),
                 _ptr(out), _bnhd(out, "out"), _ptr(q_rows), n_rows, bstride, _ptr(kv_len),
                 0.0 if scale is None else float(scale), _ptr(lse),
                 (ATTN_SCATTER_OUT if scatter_out else 0) | (FLAG_CHECK if check else 0), None, 0)
    a.mask, a.mask_dtype, ms = _attn_mask(mask, B, H, Nq, Nk)
    a.mask_stride[:] = ms
    _attn_kv_src(a, kv_src, k_fresh, v_fresh, B, Nk, H, d)
    return a, out, lse


def _attn_set_workspace(a: AttnArgs, workspace, device: torch.device, st: int):
    """Point a at the split workspace: "auto" (cached per device and stream), None, or a tensor."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a device tensor")
        workspace = _attn_workspace(a, device, st)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_rows: Optional[torch.Tensor] = None,
             kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             return_lse: bool = False, scatter_out: bool = False, check: bool = False, stream=None,
             workspace="auto", mask: Optional[torch.Tensor] = None, kv_src: Optional[torch.Tensor] = None,
             k_fresh: Optional[torch.Tensor] = None, v_fresh: Optional[torch.Tensor] = None):
    """Attention on all rows (q_rows None) or on gathered rows q_rows [n] / [1|B, n]; see safe.h.

    kv_len: int32 [B] valid key counts.  kv_src: optional source map [Nk] / [1|B, Nk] int32
    (kv_source_map) for the fused global K/V read: key j comes from row kv_src[.., j] of
    k_fresh / v_fresh [B, n_fresh, H, d] when that is in [0, n_fresh), else from k / v (the
    cache).  workspace: "auto" (a buffer cached per device and stream, sized by
    safe_attn_workspace_bytes; under HIP graph capture it must already be large enough),
    None (no tail split), or a uint8 device tensor.  mask: optional dense mask
    [B|1, H|1, Nq|1, Nk] (size-1 dims broadcast), indexed by query token; bool/uint8
    attend-where-nonzero or an additive bf16/f16/f32 bias."""
    a, out, lse = _attn_call(q, k, v, q_rows, kv_len, scale, out, return_lse, scatter_out, check, mask, kv_src,
                             k_fresh, v_fresh)
    if a is not None:
        st = _stream(stream)
        _attn_set_workspace(a, workspace, q.device, st)
        _check("safe_attn_fwd", lib.safe_attn_fwd(ctypes.byref(a), st))
    return (out, lse) if return_lse else out


_SDPA_WS = {}   # (device index, stream handle) -> classifier scratch of sdpa


def sdpa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Optional[torch.Tensor] = None,
         q_rows: Optional[torch.Tensor] = None, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
         return_lse: bool = False, scatter_out: bool = False, stream=None, workspace="auto"):
    """The Eq. 8 rewrite as one call (safe_sdpa): certify `mask` on the GPU, then run the
    attention without it (every stored row in R), with per-sample key lengths (a text-padding
    mask with one valid length per sample) or with it (anything else).  mask as for attn_fwd
    ([B|1, H|1, Nq|1, Nk], size-1 dims broadcast).  Returns (out[, lse], info) with info a
    dict: route ("no_mask", "kv_len" or "mask"), mask_class (name, or None without a mask)
    and first_bad_row.  Blocks on the classifier's verdict when a mask is given."""
    a, out, lse = _attn_call(q, k, v, q_rows, None, scale, out, return_lse, scatter_out, False, mask, None,
                             None, None)
    if a is None:
        res = {"route": None, "mask_class": None, "first_bad_row": -1}
        return (out, lse, res) if return_lse else (out, res)
    st = _stream(stream)
    # the split workspace is sized for the mask-free form; a route whose plan needs more runs unsplit
    free = AttnArgs.from_buffer_copy(a)
    free.mask = None
    _attn_set_workspace(free, workspace, q.device, st)
    a.workspace, a.workspace_bytes = free.workspace, free.workspace_bytes
    need = ctypes.c_size_t(0)
    _check("safe_sdpa", lib.safe_sdpa(ctypes.byref(a), None, ctypes.byref(need), None, st))
    cws = None
    if need.value > 0:
        cws = _cached_workspace(_SDPA_WS, (q.device.index, st), int(need.value), q.device, "sdpa")
    info = SdpaInfo()
    size = ctypes.c_size_t(0 if cws is None else cws.numel())
    _check("safe_sdpa", lib.safe_sdpa(ctypes.byref(a), _ptr(cws), ctypes.byref(size) if cws is not None else None,
                                      ctypes.byref(info), st))
    res = {"route": ROUTE_NAMES[info.route],
           "mask_class": MASK_CLASS_NAMES[info.mask_class] if info.mask_class >= 0 else None,
           "first_bad_row": int(info.first_bad_row)}
    return (out, lse, res) if return_lse else (out, res)


def _attn_kv_src(a, kv_src, k_fresh, v_fresh, B, Nk, H, d):
    """Fill the fused global K/V fields of AttnArgs (all three tensors or none)."""
    if kv_src is None:
        if k_fresh is not None or v_fresh is not None:
            raise ValueError("k_fresh / v_fresh need kv_src")
        return
    kv_src = _i32(kv_src, "kv_src")
    if kv_src.dim() not in (1, 2) or kv_src.shape[-1] != Nk or kv_src.stride(-1) != 1 \
            or (kv_src.dim() == 2 and kv_src.shape[0] not in (1, B)):
        raise ValueError("kv_src must be [Nk], [1, Nk] or [B, Nk] with contiguous rows")
    if k_fresh is None or v_fresh is None:
        raise ValueError("kv_src needs k_fresh and v_fresh")
    _bits16(k_fresh, "k_fresh")
    _bits16(v_fresh, "v_fresh")
    if k_fresh.dim() != 4 or k_fresh.shape[0] != B or k_fresh.shape[2:] != (H, d) or v_fresh.shape != k_fresh.shape:
        raise ValueError("k_fresh and v_fresh must be [B, n_fresh, H, d]")
    fs = _bnhd(k_fresh, "k_fresh")
    if _bnhd(v_fresh, "v_fresh")[:] != fs[:]:
        raise ValueError("k_fresh and v_fresh must share strides")
    shared = kv_src.dim() == 1 or kv_src.shape[0] == 1
    a.kv_src, a.kv_src_bstride = _ptr(kv_src), (0 if shared else kv_src.stride(0))
    a.k_fresh, a.v_fresh, a.n_fresh = _ptr(k_fresh), _ptr(v_fresh), k_fresh.shape[1]
    a.fresh_stride[:] = fs[:]


def kv_source_map(idx: torch.Tensor, n_tokens: int, batch: Optional[int] = None, out: Optional[torch.Tensor] = None,
                  check: bool = False, stream=None) -> torch.Tensor:
    """Source map [B, N] int32 of the fused global K/V read: r where idx[b, r] == j, else -1.

    idx: ascending int32 token list [nsel] (shared by the batch, B = batch) or [B, nsel]."""
    idx = _i32(idx, "idx")
    if idx.dim() == 1:
        B = 1 if batch is None else int(batch)
    elif idx.dim() == 2:
        B = idx.shape[0] if batch is None or idx.shape[0] != 1 else int(batch)
    else:
        raise ValueError("idx must be [nsel] or [B, nsel]")
    nsel, ibs = _row_lists(idx, B, "idx")
    if out is None:
        out = torch.empty((B, n_tokens), dtype=torch.int32, device=idx.device)
    if out.dtype != torch.int32 or out.shape != (B, n_tokens) or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous int32 device tensor [B, N]")
    a = KvArgs()
    a.B, a.N, a.nsel, a.idx, a.idx_bstride = B, n_tokens, nsel, _ptr(idx), ibs
    a.flags = FLAG_CHECK if check else 0
    _check("safe_kv_source_map", lib.safe_kv_source_map(ctypes.byref(a), _ptr(out), _stream(stream)))
    return out


def attn_workspace_bytes(q: torch.Tensor, k: torch.Tensor, q_rows: Optional[torch.Tensor] = None,
                         kv_len: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                         kv_src: Optional[torch.Tensor] = None) -> int:
    """Workspace bytes attn_fwd would use on the current device for these shapes (0: no split)."""
    B, Nq, H, d = q.shape
    if q_rows is None:
        n_rows = Nq
    else:
        n_rows = q_rows.shape[-1]
    a = AttnArgs()
    a.B, a.H, a.Nq, a.Nk, a.d, a.n_rows = B, H, Nq, k.shape[1], d, n_rows
    a.q_rows = None if q_rows is None else _ptr(q_rows)
    a.kv_len = None if kv_len is None else _ptr(kv_len)
    a.mask, a.mask_dtype, ms = _attn_mask(mask, B, a.H, Nq, a.Nk)
    a.mask_stride[:] = ms
    a.kv_src = None if kv_src is None else 16   # only its being non-NULL is read
    n = lib.safe_attn_workspace_bytes(ctypes.byref(a))
    if n < 0:
        _check("safe_attn_workspace_bytes", int(n))
    return int(n)


def attn_plan(q: torch.Tensor, k: torch.Tensor, q_rows: Optional[torch.Tensor] = None,
              kv_len: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
              workspace_bytes: Optional[int] = None, kv_src: Optional[torch.Tensor] = None) -> dict:
    """The schedule attn_fwd runs for these shapes on the current device (safe_attn_plan):
    rows per tile, tile count, split tiles, key ranges, keys per range, workspace bytes.
    workspace_bytes None: the workspace attn_fwd allocates by default; 0: no workspace."""
    B, Nq, H, d = q.shape
    a = AttnArgs()
    a.B, a.H, a.Nq, a.Nk, a.d = B, H, Nq, k.shape[1], d
    a.n_rows = Nq if q_rows is None else q_rows.shape[-1]
    a.q_rows = None if q_rows is None else _ptr(q_rows)
    a.q_rows_bstride = _row_lists(q_rows, B, "q_rows")[1]
    a.kv_len = None if kv_len is None else _ptr(kv_len)
    a.mask, a.mask_dtype, ms = _attn_mask(mask, B, a.H, Nq, a.Nk)
    a.mask_stride[:] = ms
    a.kv_src = None if kv_src is None else 16   # only its being non-NULL is read
    if workspace_bytes is None:
        workspace_bytes = attn_workspace_bytes(q, k, q_rows=q_rows, kv_len=kv_len, mask=mask, kv_src=kv_src)
    if workspace_bytes > 0:
        a.workspace = 16          # only its being non-NULL is read
        a.workspace_bytes = int(workspace_bytes)
    info = AttnPlanInfo()
    _check("safe_attn_plan", lib.safe_attn_plan(ctypes.byref(a), ctypes.byref(info)))
    return {f: int(getattr(info, f)) for f, _ in AttnPlanInfo._fields_}


def kv_assemble(k_fresh: torch.Tensor, v_fresh: torch.Tensor, idx: torch.Tensor, k_cache: torch.Tensor,
                v_cache: torch.Tensor, k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                in_place: bool = False, check: bool = False, stream=None):
    """Global K/V = fresh rows (token idx) over cached rows; see safe.h.  Returns (k_out, v_out)."""
    for t, n in ((k_fresh, "k_fresh"), (v_fresh, "v_fresh"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _bits16(t, n)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be 4-D [B, N, H, d]")
    B, N, H, d = k_cache.shape
    idx = _i32(idx, "idx")
    nsel, ibs = _row_lists(idx, B, "idx")
    if k_fresh.shape != (B, nsel, H, d) or v_fresh.shape != k_fresh.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch: fresh [B, nsel, H, d], cache [B, N, H, d]")
    if in_place:
        k_out, v_out = k_cache, v_cache
    else:
        if k_out is None:
            k_out = torch.empty_like(k_cache)
        if v_out is None:
            v_out = torch.empty_like(v_cache)
        for t, n in ((k_out, "k_out"), (v_out, "v_out")):
            _bits16(t, n)
            _need(t, k_cache.shape, n)
    a = KvArgs(B, N, H, d, nsel, _ptr(k_fresh), _ptr(v_fresh), _bnhd(k_fresh, "k_fresh"), _ptr(idx), ibs,
               _ptr(k_cache), _ptr(v_cache), _bnhd(k_cache, "k_cache"), _ptr(k_out), _ptr(v_out),
               _bnhd(k_out, "k_out"), FLAG_CHECK if check else 0)
    if _bnhd(v_fresh, "v_fresh")[:] != a.fresh_stride[:] or _bnhd(v_cache, "v_cache")[:] != a.cache_stride[:] \
            or _bnhd(v_out, "v_out")[:] != a.out_stride[:]:
        raise ValueError("k and v tensors must share strides")
    _check("safe_kv_assemble", lib.safe_kv_assemble(ctypes.byref(a), _stream(stream)))
    return k_out, v_out


_MASK_DT = {torch.bool: DT_BOOL, torch.uint8: DT_BOOL, torch.bfloat16: DT_BF16, torch.float16: DT_F16,
            torch.float32: DT_F32}


def mask_classify(mask: torch.Tensor, row_class: bool = False, kv_len: bool = False, workspace=None,
                  asynchronous: bool = False, stream=None) -> dict:
    """Certify a [B, H, Nq, Nk] mask (as stored); returns a dict with verdict, class, first bad row, rows."""
    if mask.dim() != 4:
        raise ValueError("mask must be 4-D [B, H, Nq, Nk] (broadcast dims stored with size 1)")
    if mask.dtype not in _MASK_DT:
        raise TypeError(f"unsupported mask dtype {mask.dtype}")
    if not mask.is_cuda:
        raise ValueError("mask must be a device tensor")
    dt = _MASK_DT[mask.dtype]
    size = _i64x4(*mask.shape)
    stride = _i64x4(*mask.stride())
    need = ctypes.c_size_t(0)
    s = _stream(stream)
    _check("safe_mask_classify", lib.safe_mask_classify(None, dt, size, stride, 0, None, None, None, None,
                                                        ctypes.byref(need), s))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=mask.device)
    rc = torch.empty(mask.shape[0] * mask.shape[1] * mask.shape[2], dtype=torch.uint8, device=mask.device) \
        if row_class else None
    kl = torch.empty(mask.shape[0], dtype=torch.int32, device=mask.device) if kv_len else None
    info = MaskInfo()
    flags = CLASSIFY_ASYNC if asynchronous else 0
    # torch.bool storage is one byte per element (0/1): read as uint8
    _check("safe_mask_classify", lib.safe_mask_classify(_ptr(mask), dt, size, stride, flags, ctypes.byref(info),
                                                        _ptr(rc), _ptr(kl), _ptr(workspace), ctypes.byref(need), s))
    out = {"row_class": rc, "kv_len": kl, "workspace": workspace}
    if not asynchronous:
        out.update(verdict=info.verdict, mask_class=info.mask_class, first_bad_row=info.first_bad_row,
                   rows=info.rows, class_name=MASK_CLASS_NAMES[info.mask_class])
    return out


_PCSP_WS = {}  # (device index, stream handle) -> uint8 workspace tensor for the head-group split


def pcsp_accumulate(q_c: torch.Tensor, k_txt: torch.Tensor, w: torch.Tensor, acc: torch.Tensor,
                    kv_len: Optional[torch.Tensor] = None, head_mask: int = 0, scale: Optional[float] = None,
                    stream=None, workspace="auto") -> torch.Tensor:
    """acc[b, i] += sum_h sum_j w[b, j] softmax_j(scale q_c[b,i,h] . k_txt[b,j,h])  (Eq. 9-10).

    workspace: "auto" (cached per device and stream), None (unsplit), or a uint8 device tensor."""
    _bits16(q_c, "q_c")
    _bits16(k_txt, "k_txt")
    B, N, H, d = q_c.shape
    M = k_txt.shape[1]
    if w.dtype != torch.float32 or w.shape != (B, M) or not w.is_contiguous():
        raise ValueError("w must be contiguous float32 [B, M]")
    if acc.dtype != torch.float32 or acc.shape != (B, N) or not acc.is_contiguous():
        raise ValueError("acc must be contiguous float32 [B, N]")
    kv_len = _lengths(kv_len, B)
    a = PcspArgs()
    a.flags = PCSP_ACCUM
    a.B, a.N, a.M, a.H, a.d = B, N, M, H, d
    a.q, a.q_stride = _ptr(q_c), _bnhd(q_c, "q_c")
    a.k_text, a.k_stride = _ptr(k_txt), _bnhd(k_txt, "k_txt")
    a.kv_len, a.w, a.head_mask = _ptr(kv_len), _ptr(w), head_mask
    a.scale = 0.0 if scale is None else float(scale)
    a.acc = _ptr(acc)
    st = _stream(stream)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a device tensor")
        need = ctypes.c_size_t(0)
        _check("safe_pcsp_select", lib.safe_pcsp_select(ctypes.byref(a), None, ctypes.byref(need), st))
        workspace = None
        if need.value > 0:
            workspace = _cached_workspace(_PCSP_WS, (acc.device.index, st), int(need.value), acc.device,
                                          "pcsp_accumulate")
    if workspace is None:
        _check("safe_pcsp_select", lib.safe_pcsp_select(ctypes.byref(a), None, None, st))
    else:
        size = ctypes.c_size_t(workspace.numel() * workspace.element_size())
        _check("safe_pcsp_select", lib.safe_pcsp_select(ctypes.byref(a), _ptr(workspace), ctypes.byref(size), st))
    return acc


def pcsp_select(acc: torch.Tensor, grid_h: int, grid_w: int, sigma: float, k: int, score_out: bool = False,
                workspace=None, stream=None):
    """Eq. 11-12: smoothed field, optional Norm output, ascending top-k indices [B, k] int32."""
    if acc.dtype != torch.float32 or acc.dim() != 2 or not acc.is_contiguous():
        raise ValueError("acc must be contiguous float32 [B, N]")
    B, N = acc.shape
    a = PcspArgs()
    a.flags = PCSP_SELECT
    a.B, a.N = B, N
    a.acc = _ptr(acc)
    a.grid_h, a.grid_w, a.sigma, a.k = grid_h, grid_w, float(sigma), k
    idx = torch.empty((B, k), dtype=torch.int32, device=acc.device)
    so = torch.empty_like(acc) if score_out else None
    a.score_out, a.idx_out = _ptr(so), _ptr(idx)
    need = ctypes.c_size_t(0)
    s = _stream(stream)
    _check("safe_pcsp_select", lib.safe_pcsp_select(ctypes.byref(a), None, ctypes.byref(need), s))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=acc.device)
    _check("safe_pcsp_select", lib.safe_pcsp_select(ctypes.byref(a), _ptr(workspace), ctypes.byref(need), s))
    return (idx, so) if score_out else idx


def sw_cfg(f_c: torch.Tensor, f_u: torch.Tensor, g_ctx: float, g_sens: Optional[float] = None,
           s: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Eq. 20-21: out = f_u + gamma * (f_c - f_u) per token, gamma from the score row s [B, N] (or [N]),
    from membership in the ascending index list idx [B, k] (or [k]), or g_ctx everywhere."""
    if f_c.shape != f_u.shape or f_c.dim() != 3 or f_c.dtype != f_u.dtype:
        raise ValueError("f_c and f_u must be [B, N, C] of one dtype")
    if f_c.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("predictions must be bfloat16 or float32")
    if f_c.stride() != f_u.stride() or f_c.stride(2) != 1:
        raise ValueError("f_c and f_u must share strides with C contiguous")
    B, N, C = f_c.shape
    if out is None:
        out = torch.empty_like(f_c)
    if out.shape != f_c.shape or out.stride() != f_c.stride() or out.dtype != f_c.dtype:
        raise ValueError("out must match f_c in shape, strides and dtype")
    a = CfgArgs()
    a.B, a.N, a.C = B, N, C
    a.dtype = DT_BF16 if f_c.dtype == torch.bfloat16 else DT_F32
    a.f_c, a.f_u, a.out = _ptr(f_c), _ptr(f_u), _ptr(out)
    a.stride[:] = [f_c.stride(0), f_c.stride(1)]
    if s is not None and idx is not None:
        raise ValueError("give at most one of s and idx")
    if s is not None:
        if s.dtype != torch.float32 or s.dim() not in (1, 2) or s.shape[-1] != N:
            raise ValueError("s must be float32 [N], [1, N] or [B, N]")
        _, sbs = _row_lists(s, B, "s")
        a.s, a.s_bstride = _ptr(s), sbs
    idx = _i32(idx, "idx")
    if idx is not None:
        kk, ibs = _row_lists(idx, B, "idx")
        a.idx, a.k, a.idx_bstride = _ptr(idx), kk, ibs
    a.g_ctx = float(g_ctx)
    a.g_sens = float(g_ctx if g_sens is None else g_sens)
    _check("safe_sw_cfg", lib.safe_sw_cfg(ctypes.byref(a), _stream(stream)))
    return out


__all__ = ["attn_fwd", "attn_plan", "attn_workspace_bytes", "kv_assemble", "kv_source_map", "mask_classify",
           "pcsp_accumulate", "pcsp_select", "sdpa", "sw_cfg", "linear", "block_dense", "block_srsu", "lib",
           "mfma_probe", "hbm_probe", "SafeError", "LIB_PATH", "MASK_CLASS_NAMES", "ROUTE_NAMES"]


def _rows3(t: torch.Tensor, name: str):
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be [batches, rows, features] with features contiguous")
    _bits16(t, name)
    return (t.stride(0) if t.shape[0] > 1 else 0, t.stride(1))


def linear(a: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, gelu: bool = False,
           res: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           a_rows: Optional[torch.Tensor] = None, res_rows: Optional[torch.Tensor] = None,
           out_rows: Optional[torch.Tensor] = None, check: bool = False, stream=None) -> torch.Tensor:
    """out[b, ro(r)] = [gelu](a[b, ra(r)] @ w.T + bias) + res[b, rr(r)] in bf16; see safe_linear in safe.h.

    a [B, Ta, K], w [N, K], res [B, Tr, N], out [B, To, N] (bf16, last dim contiguous);
    the row lists are [B, M] or [M] int32 and index tensors of equal row count."""
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be [N, K] with K contiguous")
    _bits16(w, "w")
    B, Ta, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K] matching a")
    lists = [_i32(x, n) for x, n in ((a_rows, "a_rows"), (res_rows, "res_rows"), (out_rows, "out_rows"))]
    given = [x for x in lists if x is not None]
    M = given[0].shape[-1] if given else Ta
    bst = 0
    for x in given:
        if x.shape[-1] != M or (x.dim() == 2 and (x.shape[0] != B or x.stride(1) != 1)):
            raise ValueError("row lists must all be [M] or [B, M] with contiguous rows")
    if given:
        strides = {x.stride(0) if x.dim() == 2 else 0 for x in given}
        if len(strides) != 1:
            raise ValueError("row lists must share one batch stride")
        bst = strides.pop()
    ntok = 0
    for x, t in ((lists[0], a), (lists[1], res), (lists[2], out)):
        if x is not None:
            if t is None:
                raise ValueError("a row list needs its tensor")
            if ntok and t.shape[1] != ntok:
                raise ValueError("tensors indexed by row lists must have equal row counts")
            ntok = t.shape[1]
    if out is None:
        if out_rows is not None:
            raise ValueError("out_rows needs an output tensor holding the other rows")
        out = torch.empty((B, M, N), dtype=a.dtype, device=a.device)
    # without a row list, row r of a tensor is its row r: it needs at least M rows
    # (with one, every listed tensor has the same row count, checked above)
    for t, x, n, shared in ((out, out_rows, "out", False), (res, res_rows, "res", True)):
        if t is None:
            continue
        if t.dim() != 3 or t.shape[2] != N or t.shape[0] not in ((1, B) if shared else (B,)) \
                or (x is None and t.shape[1] < M):
            raise ValueError(f"{n} must be [B{'|1' if shared else ''}, rows >= {M}, {N}], got {list(t.shape)}")
    if a_rows is None and Ta < M:
        raise ValueError(f"a without a row list needs at least {M} rows")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (N,) or not bias.is_contiguous()):
        raise ValueError("bias must be contiguous float32 [N]")
    args = LinearArgs()
    args.batches, args.M, args.N, args.K = B, M, N, K
    args.a, args.w, args.w_stride = _ptr(a), _ptr(w), w.stride(0)
    args.a_stride[:] = _rows3(a, "a")
    args.bias = _ptr(bias)
    args.act = ACT_GELU_TANH if gelu else ACT_NONE
    if res is not None:
        args.res = _ptr(res)
        args.res_stride[:] = _rows3(res, "res")
    args.out = _ptr(out)
    args.out_stride[:] = _rows3(out, "out")
    args.a_rows, args.res_rows, args.out_rows = (_ptr(x) for x in lists)
    args.rows_bstride, args.Ntok = bst, ntok
    args.flags = FLAG_CHECK if check else 0
    _check("safe_linear", lib.safe_linear(ctypes.byref(args), _stream(stream)))
    return out


# ---- the block around attention (Eq. 15-18): sequencing of the entry points above ----

def _heads(t: torch.Tensor, i: int, C: int, H: int) -> torch.Tensor:
    """Part i (0 = Q, 1 = K, 2 = V) of a [B, n, 3C] projection as a [B, n, H, d] view."""
    return t[..., i * C:(i + 1) * C].unflatten(-1, (H, C // H))


def block_dense(x: torch.Tensor, w: dict, H: int, stream=None):
    """The dense block (anchor step, Eq. 18) of the stand-in block
        qkv = x Wqkv^T;  a = SDPA(q, k, v);  y = x + a Wo^T;  z = y + gelu_tanh(y W1^T + b1) W2^T + b2
    with every map a libsafe call.  Returns (z [B, N, C], qkv [B, N, 3C]); qkv's K and V parts
    are the key/value cache of the following non-anchor steps (Eq. 14, 19)."""
    B, N, C = x.shape
    qkv = linear(x, w["w_qkv"], stream=stream)
    a = attn_fwd(_heads(qkv, 0, C, H), _heads(qkv, 1, C, H), _heads(qkv, 2, C, H), stream=stream)
    y = linear(a.view(B, N, C), w["w_o"], res=x, stream=stream)
    u = linear(y, w["w1"], bias=w["b1"], gelu=True, stream=stream)
    z = linear(u, w["w2"], bias=w["b2"], res=y, stream=stream)
    return z, qkv


def block_srsu(x: torch.Tensor, idx: torch.Tensor, z: torch.Tensor, qkv_cache: torch.Tensor, w: dict, H: int,
               stream=None):
    """The row-selective block (Eq. 15-16) for ascending token lists idx [B, k]: the rows of S
    are projected from the current state x and their query, key and value rows are written
    straight over the cached ones in qkv_cache at their tokens (the projection's row scatter:
    the cache then holds the global K/V of Eq. 16 in token order, with no assembly pass),
    their attention (queries gathered from the same buffer), residual and MLP outputs are
    computed, and their outputs are written over the cached outputs in z (in place: the
    context rows of z stay the cached ones, Eq. 15).  Returns z."""
    B, N, C = x.shape
    k = idx.shape[-1]
    linear(x, w["w_qkv"], a_rows=idx, out=qkv_cache, out_rows=idx, stream=stream)
    a_s = attn_fwd(_heads(qkv_cache, 0, C, H), _heads(qkv_cache, 1, C, H), _heads(qkv_cache, 2, C, H),
                   q_rows=idx, stream=stream)
    y_s = linear(a_s.view(B, k, C), w["w_o"], res=x, res_rows=idx, stream=stream)
    u_s = linear(y_s, w["w1"], bias=w["b1"], gelu=True, stream=stream)
    linear(u_s, w["w2"], bias=w["b2"], res=y_s, out=z, out_rows=idx, stream=stream)
    return z


def mfma_probe(shape: int, iters: int, blocks: int, seed: int = 1, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """The matrix-core rate probe (safe_mfma_probe, a measurement aid): `blocks` workgroups of
    4 waves issue iters x 16 MFMAs each on random bf16 register operands (shape 32:
    v_mfma_f32_32x32x16_bf16, 32768 FLOP; 16: v_mfma_f32_16x16x32_bf16, 16384 FLOP).  Returns the
    float32 per-lane checksums [blocks * 256]."""
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() < blocks * 256:
        raise ValueError("out must be a contiguous float32 tensor of at least blocks * 256 elements")
    _check("safe_mfma_probe", lib.safe_mfma_probe(int(shape), int(iters), int(blocks), int(seed) & 0xFFFFFFFF,
                                                  _ptr(out), _stream(stream)))
    return out


def hbm_probe(src: torch.Tensor, blocks: int, dst: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              stream=None) -> Optional[torch.Tensor]:
    """The streaming probe (safe_hbm_probe, a measurement aid) over the bytes of the contiguous
    device tensor `src`: with `dst` (a contiguous tensor of the same byte size) a non-temporal
    copy into it, returning None; without, a read that returns the per-thread xor words
    (uint32 as int32, [blocks * 256]; thread t owns 16-byte chunks t, t + 256 * blocks, ...)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst is not None:
        if not dst.is_cuda or not dst.is_contiguous() or dst.numel() * dst.element_size() != nbytes:
            raise ValueError("dst must be a contiguous device tensor of the same byte size as src")
        _check("safe_hbm_probe", lib.safe_hbm_probe(1, _ptr(src), _ptr(dst), nbytes, int(blocks), None,
                                                    _stream(stream)))
        return None
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.int32, device=src.device)
    if out.dtype != torch.int32 or not out.is_contiguous() or out.numel() < blocks * 256:
        raise ValueError("out must be a contiguous int32 tensor of at least blocks * 256 elements")
    _check("safe_hbm_probe", lib.safe_hbm_probe(0, _ptr(src), None, nbytes, int(blocks), _ptr(out), _stream(stream)))
    return out
