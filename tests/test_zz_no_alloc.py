"""safe_attn_fwd_noalloc through the C ABI: the attention entry point for callers that cannot
allocate keeps its split partials in the library's static device array and must give, call
after call, the result safe_attn_fwd gives with a workspace of the same size (bit for bit),
and stay within the oracle's bounds (Eq. 2, 16, 18)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attn_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")

SCRATCH = 64 << 20   # SAFE_NOALLOC_SCRATCH_BYTES


def _noalloc(q, k, v, q_rows=None, out=None):
    """One safe_attn_fwd_noalloc call with the arguments the binding marshals for attn_fwd."""
    a, out, _ = sq._attn_call(q, k, v, q_rows, None, None, out, False, False, False, None, None, None, None)
    st = sq.lib.safe_attn_fwd_noalloc(ctypes.byref(a), int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, sq.lib.safe_status_str(st).decode()
    return out


def _reference(q, k, v, q_rows=None):
    """safe_attn_fwd with a caller workspace of the static array's size (or none at all when
    the split does not fit it: the no-alloc call then runs unsplit too)."""
    need = sq.attn_workspace_bytes(q, k, q_rows=q_rows)
    ws = torch.empty(SCRATCH, dtype=torch.uint8, device="cuda") if 0 < need <= SCRATCH else None
    return sq.attn_fwd(q, k, v, q_rows=q_rows, workspace=ws), need


def test_noalloc_matches_attn_fwd_on_consecutive_calls():
    # first call: a split dense pass whose partials fill part of the array
    B, N, H, d = 1, 2000, 4, 96
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=90)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    ref, need = _reference(qd, kd, vd)
    assert 0 < need <= SCRATCH, need
    got = _noalloc(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "first call"
    rows = np.arange(0, N, 7)
    r, _ = oracle.sdpa(q.value, k.value, v.value, q_rows=rows[::9])
    assert_attn_close(got[:, torch.from_numpy(rows[::9]).long()], r, "no-alloc dense")
    # second, smaller call on the same array: gathered rows, another head dimension
    B2, N2, H2, d2 = 1, 900, 3, 64
    q2, k2, v2 = W.attention_inputs(B2, N2, N2, H2, d2, seed=91)
    qd2, kd2, vd2 = to_dev_bf16(q2), to_dev_bf16(k2), to_dev_bf16(v2)
    sel = W.random_rows(np.random.default_rng(92), N2, 333)
    ref2, need2 = _reference(qd2, kd2, vd2, q_rows=to_dev(sel))
    assert 0 < need2 < need, (need2, need)
    got2 = _noalloc(qd2, kd2, vd2, q_rows=to_dev(sel))
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2), "second, smaller call"
    r2, _ = oracle.sdpa(q2.value, k2.value, v2.value, q_rows=sel)
    assert_attn_close(got2, r2, "no-alloc gathered")
    # the first shape again: the array holds the second call's partials, nothing leaks through
    assert torch.equal(_noalloc(qd, kd, vd), ref), "repeat of the first call"


def test_noalloc_with_a_split_larger_than_the_array_runs_unsplit():
    """The 160x160-grid dense pass wants ~154 MB of partials: more than the array, so the
    no-alloc call runs the unsplit schedule, like safe_attn_fwd without a workspace."""
    B, N, H, d = 2, 25600, 24, 96
    g = torch.Generator(device="cuda").manual_seed(93)
    q, k, v = (torch.randn((B, N, H, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    ref, need = _reference(q, k, v)
    assert need > SCRATCH, need
    assert torch.equal(_noalloc(q, k, v), ref)


def test_noalloc_fused_global_kv_read():
    """The fused global K/V read (source map, fresh rows over the cache) through the
    no-alloc entry point: bit for bit what attn_fwd gives with a workspace of the array's size."""
    B, N, H, d, nsel = 2, 3000, 4, 96, 900
    q, kc, vc = W.attention_inputs(B, N, N, H, d, seed=93)
    kf, vf, _ = W.attention_inputs(B, nsel, nsel, H, d, seed=94)
    S = np.stack([W.random_rows(np.random.default_rng(95 + b), N, nsel) for b in range(B)])
    qd, kcd, vcd, kfd, vfd = (to_dev_bf16(t) for t in (q, kc, vc, kf, vf))
    Sd = to_dev(S)
    src = sq.kv_source_map(Sd, N)
    need = sq.attn_workspace_bytes(qd, kcd, q_rows=Sd, kv_src=src)
    ws = torch.empty(SCRATCH, dtype=torch.uint8, device="cuda") if 0 < need <= SCRATCH else None
    ref = sq.attn_fwd(qd, kcd, vcd, q_rows=Sd, workspace=ws, kv_src=src, k_fresh=kfd, v_fresh=vfd)
    a, got, _ = sq._attn_call(qd, kcd, vcd, Sd, None, None, None, False, False, False, None, src, kfd, vfd)
    st = sq.lib.safe_attn_fwd_noalloc(ctypes.byref(a), int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, sq.lib.safe_status_str(st).decode()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    kg = oracle.kv_assemble(kf.value, S, kc.value)
    vg = oracle.kv_assemble(vf.value, S, vc.value)
    samp = np.array([0, 1, 450, nsel - 1])
    r, _ = oracle.sdpa(q.value, kg, vg, q_rows=S[:, samp])
    assert_attn_close(got[:, torch.from_numpy(samp).long()], r, "no-alloc fused read")


def test_noalloc_refuses_a_workspace_and_the_check_flag():
    q, k, v = W.attention_inputs(1, 256, 256, 2, 64, seed=94)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    a, _, _ = sq._attn_call(qd, kd, vd, None, None, None, None, False, False, False, None, None, None, None)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    assert sq.lib.safe_attn_fwd_noalloc(ctypes.byref(a), None) == -6
    a.workspace, a.workspace_bytes = None, 0
    a.flags = 1
    assert sq.lib.safe_attn_fwd_noalloc(ctypes.byref(a), None) == -5
