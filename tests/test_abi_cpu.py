"""CPU-only checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "safe.h")

sq = pytest.importorskip("sparse_query_sdpa_amd", reason="libsafe.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int64_t|int|const char\*)\s+(safe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("safe_mask_classify", "safe_pcsp_select", "safe_kv_assemble", "safe_attn_fwd", "safe_sw_cfg", "safe_linear",
              "safe_attn_workspace_bytes", "safe_attn_plan", "safe_kv_source_map", "safe_sdpa", "safe_status_str",
              "safe_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(sq.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    assert sq.lib.safe_abi_version() == 10 == sq.ABI_VERSION
    for code, name in sq.STATUS.items():
        assert sq.lib.safe_status_str(code).decode().startswith(name)
    assert sq.lib.safe_status_str(12345) == b"unknown status"


def _attn_args(**kw):
    a = sq.AttnArgs()
    a.B, a.H, a.Nq, a.Nk, a.d = 1, 1, 128, 128, 96
    fake = 0x10000  # never dereferenced: validation fails or returns first
    a.q = a.k = a.v = a.o = fake
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(a, name)[:] = [128 * 96, 96, 96]
    a.n_rows = 128
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(d=48), -5), (dict(d=256), -5), (dict(B=-1), -2), (dict(q=None), -1), (dict(o=None), -1),
    (dict(n_rows=5), -2), (dict(scale=float("nan")), -4), (dict(scale=float("inf")), -4),
    (dict(q=0x10008), -8), (dict(flags=1 << 7), -4), (dict(flags=2), -2),
])
def test_attn_rejects_bad_arguments_without_gpu(kw, status):
    a = _attn_args(**kw)
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == status


def test_sdpa_validates_and_sizes_its_scratch_without_gpu():
    """safe_sdpa (the Eq. 8 rewrite as one call) checks the attention call and the mask on the
    host, answers the scratch-size query, and refuses a missing or misaligned scratch before
    any HIP call."""
    need = ctypes.c_size_t(123)
    a = _attn_args()
    assert sq.lib.safe_sdpa(ctypes.byref(a), None, ctypes.byref(need), None, None) == 0
    assert need.value == 0, "no mask: no scratch"
    a = _attn_args(mask=0x30000, mask_dtype=1)
    a.mask_stride[:] = [0, 0, 128]                       # one [Nq, Nk] mask for every (b, h)
    assert sq.lib.safe_sdpa(ctypes.byref(a), None, ctypes.byref(need), None, None) == 0
    assert need.value > 0 and need.value % 256 == 0
    assert sq.lib.safe_sdpa(ctypes.byref(a), None, None, None, None) == -6           # scratch missing
    small = ctypes.c_size_t(need.value - 1)
    assert sq.lib.safe_sdpa(ctypes.byref(a), 0x40000, ctypes.byref(small), None, None) == -6
    assert sq.lib.safe_sdpa(ctypes.byref(a), 0x40008, ctypes.byref(need), None, None) == -8
    for kw, status in ((dict(mask_dtype=9), -3), (dict(kv_len=0x50000), -5), (dict(d=48), -5),
                       (dict(kv_src=0x50000), -5), (dict(q=None), -1)):
        b = _attn_args(**{"mask": 0x30000, "mask_dtype": 1, **kw})
        assert sq.lib.safe_sdpa(ctypes.byref(b), None, ctypes.byref(need), None, None) == status, kw
    b = _attn_args(mask=0x30000, mask_dtype=1)
    b.mask_stride[:] = [0, -1, 128]
    assert sq.lib.safe_sdpa(ctypes.byref(b), None, ctypes.byref(need), None, None) == -2
    # an unaligned mask row stride is accepted by the classifier (the masked route checks it later)
    b.mask_stride[:] = [0, 0, 127]
    assert sq.lib.safe_sdpa(ctypes.byref(b), None, ctypes.byref(need), None, None) == 0


def test_noalloc_validates_on_the_host_without_gpu():
    """safe_attn_fwd_noalloc owns its scratch: a caller workspace or the host-side check flag
    is refused, and the size checks of safe_attn_fwd apply, all before any HIP call."""
    f = sq.lib.safe_attn_fwd_noalloc
    assert f(None, None) == -1
    a = _attn_args(workspace=0x60000, workspace_bytes=1 << 20)
    assert f(ctypes.byref(a), None) == -6
    a = _attn_args(workspace_bytes=16)
    assert f(ctypes.byref(a), None) == -6
    a = _attn_args(flags=1)
    assert f(ctypes.byref(a), None) == -5
    for kw, status in ((dict(d=48), -5), (dict(B=-1), -2), (dict(q=None), -1), (dict(n_rows=5), -2)):
        assert f(ctypes.byref(_attn_args(**kw)), None) == status, kw
    a = _attn_args(n_rows=0, q_rows=0x20000)    # nothing to compute: no HIP call, OK
    assert f(ctypes.byref(a), None) == 0


def test_attn_stride_checks():
    a = _attn_args()
    a.k_stride[1] = 100  # not a multiple of 8 elements
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == -8
    a = _attn_args()
    a.v_stride[0] = -96
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == -2
    a = _attn_args(q_rows=0x20000, n_rows=10, q_rows_bstride=5)  # per-sample lists overlap
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == -2
    # a 64-key tile is addressed with 32-bit byte offsets: 63 * 2 * 2^25 + row > 2^32
    for name in ("k_stride", "v_stride"):
        a = _attn_args()
        getattr(a, name)[1] = 1 << 25
        assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == -5


def test_attn_plan_arguments_without_gpu():
    info = sq.AttnPlanInfo()
    assert sq.lib.safe_attn_plan(None, ctypes.byref(info)) == -1
    assert sq.lib.safe_attn_plan(ctypes.byref(_attn_args()), None) == -1
    for kw, status in ((dict(d=48), -5), (dict(B=-1), -2), (dict(n_rows=5), -2), (dict(flags=1 << 7), -4),
                       (dict(workspace_bytes=-1), -6)):
        assert sq.lib.safe_attn_plan(ctypes.byref(_attn_args(**kw)), ctypes.byref(info)) == status, kw
    # no row to compute: an all-zero plan, no device needed
    info.rows_per_tile = 7
    assert sq.lib.safe_attn_plan(ctypes.byref(_attn_args(n_rows=0, Nq=0)), ctypes.byref(info)) == 0
    assert (info.rows_per_tile, info.row_tiles, info.split_tiles, info.workspace_bytes) == (0, 0, 0, 0)


def test_attn_workspace_arguments_without_gpu():
    # the size query validates like the call and reads no pointer
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(d=48))) == -5
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(n_rows=5))) == -2
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(q=None, k=None, v=None, o=None))) >= 0
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(kv_len=0x30000))) == 0  # never split
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(workspace_bytes=-1)), None) == -6
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(workspace=0x40004, workspace_bytes=64)), None) == -8


def test_attn_mask_arguments_without_gpu():
    m = 0x60000
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(mask=m, mask_dtype=7)), None) == -3
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(mask=m, mask_dtype=-1)), None) == -3
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(mask=m, mask_dtype=1, kv_len=0x30000)), None) == -5
    for i, bad, status in ((2, 130, -8), (0, -4, -2), (1, 2, -8)):
        a = _attn_args(mask=m, mask_dtype=1)
        a.mask_stride[:] = [128 * 128, 0, 128]
        a.mask_stride[i] = bad
        assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == status
    # rows are read in 16-byte pieces: 16-byte aligned pointer, strides of 16 bytes
    for dtype, ptr in ((0, m + 2), (1, m + 4), (2, m + 8), (3, m + 8)):
        a = _attn_args(mask=ptr, mask_dtype=dtype)
        a.mask_stride[:] = [0, 0, 128]
        assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == -8, dtype
    for dtype, stride in ((0, 8), (1, 4), (2, 12), (3, 2)):   # 8, 8, 24, 8 bytes
        a = _attn_args(mask=m, mask_dtype=dtype)
        a.mask_stride[:] = [0, 0, stride]
        assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == -8, dtype
    # the size query checks the mask fields too; a NULL mask ignores them
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(mask=m, mask_dtype=9))) == -3
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(mask_dtype=9))) >= 0
    # d = 72 is a supported head dimension (the size query runs without a device)
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(d=72))) >= 0


def test_attn_fused_kv_arguments_without_gpu():
    src, fresh = 0x70000, 0x80000
    ok = dict(kv_src=src, n_fresh=4, k_fresh=fresh, v_fresh=fresh)
    # no key lengths or mask with the fused read
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(kv_len=0x30000, **ok)), None) == -5
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(mask=0x60000, mask_dtype=1, **ok)), None) == -5
    for kw, status in ((dict(n_fresh=-1), -2), (dict(kv_src_bstride=5), -2), (dict(kv_src_bstride=-128), -2),
                       (dict(k_fresh=None), -1), (dict(v_fresh=0x80004), -8)):
        assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(**{**ok, **kw})), None) == status, kw
    a = _attn_args(**ok)
    a.fresh_stride[:] = [4 * 96, 100, 96]   # not a multiple of 8 elements
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == -8
    # the size query and the plan validate the same fields
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(kv_len=0x30000, **ok))) == -5
    assert sq.lib.safe_attn_workspace_bytes(ctypes.byref(_attn_args(**ok))) >= 0
    # empty work returns before any pointer is read
    assert sq.lib.safe_attn_fwd(ctypes.byref(_attn_args(B=0, **ok)), None) == 0


def test_kv_source_map_arguments_without_gpu():
    a = _kv_args()
    assert sq.lib.safe_kv_source_map(None, 0x90000, None) == -1
    assert sq.lib.safe_kv_source_map(ctypes.byref(a), None, None) == -1
    for kw, status in ((dict(nsel=65), -2), (dict(N=-1), -2), (dict(idx_bstride=3), -2), (dict(flags=4), -4),
                       (dict(idx=None), -1)):
        assert sq.lib.safe_kv_source_map(ctypes.byref(_kv_args(**kw)), 0x90000, None) == status, kw
    # nothing to write: no pointer is read
    assert sq.lib.safe_kv_source_map(ctypes.byref(_kv_args(B=0, idx=None)), None, None) == 0
    assert sq.lib.safe_kv_source_map(ctypes.byref(_kv_args(N=0, nsel=0, idx=None)), None, None) == 0


def test_attn_empty_work_is_ok_without_gpu():
    a = _attn_args(B=0)
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == 0
    a = _attn_args(q_rows=0x20000, n_rows=0)
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == 0
    a = _attn_args(B=0, q=None, k=None, v=None, o=None)
    assert sq.lib.safe_attn_fwd(ctypes.byref(a), None) == 0


def _kv_args(**kw):
    a = sq.KvArgs()
    a.B, a.N, a.H, a.d, a.nsel = 1, 64, 2, 96, 8
    fake = 0x10000
    a.k_fresh = a.v_fresh = a.k_cache = a.v_cache = fake
    a.k_out, a.v_out = 0x40000, 0x50000
    a.idx = 0x20000
    for name in ("fresh_stride", "cache_stride", "out_stride"):
        getattr(a, name)[:] = [64 * 192, 192, 96]
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(d=12), -8), (dict(nsel=65), -2), (dict(idx=None), -1), (dict(k_cache=None), -1),
    (dict(k_out=0x10000), -2), (dict(idx_bstride=3), -2), (dict(k_fresh=0x10004), -8), (dict(flags=4), -4),
])
def test_kv_rejects_bad_arguments_without_gpu(kw, status):
    a = _kv_args(**kw)
    assert sq.lib.safe_kv_assemble(ctypes.byref(a), None) == status


def test_kv_in_place_with_other_strides_is_rejected():
    a = _kv_args(k_out=0x10000, v_out=0x10000)
    a.out_stride[1] = 200
    assert sq.lib.safe_kv_assemble(ctypes.byref(a), None) == -2


def _classify(size, stride, dtype=1, flags=0, ws=None, need=None, info=True, mask=0x10000):
    sz = (ctypes.c_int64 * 4)(*size)
    st = (ctypes.c_int64 * 4)(*stride)
    inf = sq.MaskInfo()
    nb = ctypes.c_size_t(0) if need is None else ctypes.c_size_t(need)
    rc = sq.lib.safe_mask_classify(mask, dtype, sz, st, flags, ctypes.byref(inf) if info else None, None, None, ws,
                                   ctypes.byref(nb), None)
    return rc, nb.value


def test_classify_workspace_query_and_errors():
    rc, need = _classify([2, 1, 100, 100], [10000, 10000, 100, 1])
    assert rc == 0 and need >= 64 + 16 and need % 256 == 0
    assert _classify([1, 1, 4, 4], [16, 16, 4, 1], dtype=7)[0] == -3
    assert _classify([1, 1, 4, 4], [16, 16, 4, 2])[0] == -2          # last dim not contiguous
    assert _classify([1, 1, -4, 4], [16, 16, 4, 1])[0] == -2
    assert _classify([1, 1, 4, 4], [16, 16, 4, 1], flags=64)[0] == -4
    assert _classify([1, 1, 4, 4], [16, 16, 4, 1], ws=0x30000, need=1)[0] == -6
    assert _classify([1, 1, 4, 4], [16, 16, 4, 1], ws=0x30000, need=4096, info=False)[0] == -1
    assert _classify([1, 1, 4, 4], [16, 16, 4, 1], ws=0x30008, need=4096)[0] == -8
    assert _classify([1, 1, 4, 4], [16, 16, 4, 1], ws=0x30000, need=4096, mask=None)[0] == -1


def _pcsp(**kw):
    a = sq.PcspArgs()
    a.flags = sq.PCSP_ACCUM
    a.B, a.N, a.M, a.H, a.d = 1, 64, 16, 2, 96
    a.q = a.k_text = 0x10000
    a.q_stride[:] = [64 * 192, 192, 96]
    a.k_stride[:] = [16 * 192, 192, 96]
    a.w = a.acc = 0x20000
    a.grid_h, a.grid_w, a.k = 8, 8, 4
    a.idx_out = 0x30000
    for k, v in kw.items():
        setattr(a, k, v)
    need = ctypes.c_size_t(1 << 20)
    return sq.lib.safe_pcsp_select(ctypes.byref(a), 0x40000, ctypes.byref(need), None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=0), -4), (dict(flags=1 << 9), -4), (dict(d=40), -5), (dict(M=2048), -5), (dict(w=None), -1),
    (dict(head_mask=1 << 5), -4), (dict(scale=float("nan")), -4), (dict(q_stride=(ctypes.c_int64 * 3)(1, 2, 3)), -8),
    (dict(flags=sq.PCSP_SELECT, grid_h=7), -2), (dict(flags=sq.PCSP_SELECT, k=65), -4),
    (dict(flags=sq.PCSP_SELECT, sigma=-1.0), -4), (dict(flags=sq.PCSP_SELECT, sigma=40.0), -4),
    (dict(flags=sq.PCSP_SELECT, idx_out=None), -1),
])
def test_pcsp_rejects_bad_arguments_without_gpu(kw, status):
    assert _pcsp(**kw) == status


def test_pcsp_accumulate_workspace_query():
    # the head-group split of the accumulation is sized by the query (no launch)
    a = sq.PcspArgs()
    a.flags = sq.PCSP_ACCUM
    a.B, a.N, a.M, a.H, a.d = 2, 25600, 256, 24, 96
    need = ctypes.c_size_t(0)
    assert sq.lib.safe_pcsp_select(ctypes.byref(a), None, ctypes.byref(need), None) == 0
    groups = need.value // (2 * 25600 * 4)
    assert 2 <= groups <= 24 and need.value >= groups * 2 * 25600 * 4
    a.H = 1   # nothing to split
    assert sq.lib.safe_pcsp_select(ctypes.byref(a), None, ctypes.byref(need), None) == 0
    assert need.value == 0


def test_pcsp_select_workspace_query():
    a = sq.PcspArgs()
    a.flags = sq.PCSP_SELECT
    a.B, a.N, a.grid_h, a.grid_w, a.k = 2, 100, 10, 10, 5
    need = ctypes.c_size_t(0)
    assert sq.lib.safe_pcsp_select(ctypes.byref(a), None, ctypes.byref(need), None) == 0
    assert need.value >= 2 * 2 * 100 * 4


def _cfg_args(**kw):
    a = sq.CfgArgs()
    a.B, a.N, a.C, a.dtype = 2, 50, 16, sq.DT_F32
    a.f_c = a.f_u = a.out = 0x10000  # never dereferenced: validation fails or returns first
    a.stride[:] = [50 * 16, 16]
    a.g_ctx, a.g_sens = 4.0, 7.0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=sq.DT_F16), -3), (dict(B=-1), -2), (dict(f_c=None), -1), (dict(out=None), -1),
    (dict(C=6), -8), (dict(f_u=0x10008), -8), (dict(g_sens=float("nan")), -4),
    (dict(s=0x20000, idx=0x30000, k=3), -2), (dict(k=3), -1), (dict(s=0x20000, s_bstride=10), -2),
    (dict(idx=0x30000, k=5, idx_bstride=2), -2), (dict(stride=(ctypes.c_int64 * 2)(50 * 16, 8)), -2),
])
def test_sw_cfg_rejects_bad_arguments_without_gpu(kw, status):
    assert sq.lib.safe_sw_cfg(ctypes.byref(_cfg_args(**kw)), None) == status


def test_sw_cfg_empty_work_is_ok_without_gpu():
    assert sq.lib.safe_sw_cfg(ctypes.byref(_cfg_args(N=0, f_c=None, f_u=None, out=None)), None) == 0


def _lin_args(**kw):
    a = sq.LinearArgs()
    a.batches, a.M, a.N, a.K = 2, 100, 64, 128
    a.a, a.w, a.out = 0x10000, 0x20000, 0x30000
    a.a_stride[:] = [100 * 128, 128]
    a.out_stride[:] = [100 * 64, 64]
    a.w_stride = 128
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), -5), (dict(N=12), -8), (dict(M=-1), -2), (dict(act=5), -4), (dict(flags=1 << 5), -4),
    (dict(a=None), -1), (dict(out=None), -1), (dict(w=None), -1), (dict(a=0x10008), -8),
    (dict(w_stride=64), -2), (dict(w_stride=1 << 23), -2), (dict(w_stride=132), -8), (dict(bias=0x40004), -8),
    (dict(a_rows=0x50000, rows_bstride=50), -2), (dict(a_rows=0x50000, Ntok=0), -2),
    (dict(res=0x60000), -2),
])
def test_linear_rejects_bad_arguments_without_gpu(kw, status):
    a = _lin_args(**kw)
    if "res" in kw:
        a.res_stride[:] = [-64, 64]
    assert sq.lib.safe_linear(ctypes.byref(a), None) == status


def test_linear_empty_work_is_ok_without_gpu():
    for kw in (dict(M=0), dict(batches=0), dict(N=0, a=None, w=None, out=None)):
        assert sq.lib.safe_linear(ctypes.byref(_lin_args(**kw)), None) == 0, kw


def test_kv_source_map_binding_rejects_host_tensors():
    idx = torch.arange(4, dtype=torch.int32)
    with pytest.raises(TypeError):
        sq.kv_source_map(idx, 16)          # the index list must be a device tensor


def test_binding_rejects_host_output_tensors():
    # no tensor of host memory reaches a kernel, outputs included
    with pytest.raises(ValueError):
        sq._ptr(torch.empty(4, dtype=torch.int32))
    assert sq._ptr(None) is None


def test_probe_arguments_without_gpu():
    lib, fake, out = sq.lib, 0x10000, 0x20000     # never dereferenced: validation fails first
    assert lib.safe_mfma_probe(8, 1, 1, 1, out, None) == -4
    assert lib.safe_mfma_probe(32, 0, 1, 1, out, None) == -4
    assert lib.safe_mfma_probe(16, 1, 1 << 25, 1, out, None) == -4
    assert lib.safe_mfma_probe(32, 1, 1, 1, None, None) == -1
    assert lib.safe_hbm_probe(3, fake, None, 4096, 1, out, None) == -4
    assert lib.safe_hbm_probe(0, fake, None, 8, 1, out, None) == -2
    assert lib.safe_hbm_probe(0, fake, None, (1 << 40) + 16, 1, out, None) == -2
    assert lib.safe_hbm_probe(0, fake, None, 4096, 1 << 21, out, None) == -4
    assert lib.safe_hbm_probe(0, None, None, 4096, 1, out, None) == -1
    assert lib.safe_hbm_probe(1, fake, fake + 8, 4096, 1, None, None) == -8
    assert lib.safe_hbm_probe(1, fake, fake + 4096, 8192, 1, None, None) == -4   # overlap
    assert lib.safe_hbm_probe(1, fake + 4096, fake, 8192, 1, None, None) == -4
