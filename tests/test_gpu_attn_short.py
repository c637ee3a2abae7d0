"""GPU parity of the short-key path of safe_attn_fwd (per-sample key lengths over at most
1024 keys, head dims 64/96/128: the text cross-attention of Eq. 17) against the fp64 oracle:
lengths on and around the 32-key step edges, row counts that leave a partial 128-row tile,
several head groups per call, gathered, scattered and invalid rows, LSE."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attn_close, assert_lse_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("gather", [False, True])
def test_short_keys_against_oracle(d, gather):
    B, Nq, Nk, H = 6, 333, 300, 7
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=500 + d + gather)
    kv = np.array([0, 1, 31, 32, 33, 300], dtype=np.int32)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rows = None
    if gather:
        rng = np.random.default_rng(d)
        rows = np.stack([W.random_rows(rng, Nq, 201) for _ in range(B)])
    o, lse = sq.attn_fwd(qd, kd, vd, q_rows=None if rows is None else to_dev(rows), kv_len=to_dev(kv),
                         return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, q_rows=rows, kv_len=kv)
    assert_attn_close(o, ref, f"short d={d} gather={gather}")
    assert_lse_close(lse, ref_lse, f"short d={d} gather={gather}")
    assert torch.all(o[0] == 0) and torch.all(torch.isinf(lse[0])), "kv_len 0: zero rows, LSE -inf"
    again = sq.attn_fwd(qd, kd, vd, q_rows=None if rows is None else to_dev(rows), kv_len=to_dev(kv))
    assert torch.equal(again, o), "repeated calls are bitwise identical"


def test_short_keys_scatter_and_invalid_rows():
    """Scattered output lands at the selected tokens and leaves the others untouched; an
    index outside [0, Nq) reads a zero query row (compact output) and is skipped when
    scattering."""
    B, Nq, Nk, H, d = 2, 400, 256, 3, 96
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=77)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    kv = np.array([195, 32], dtype=np.int32)
    rng = np.random.default_rng(3)
    rows = np.stack([W.random_rows(rng, Nq, 150) for _ in range(B)])
    out = torch.full((B, Nq, H, d), 7.0, dtype=torch.bfloat16, device=qd.device)
    sq.attn_fwd(qd, kd, vd, q_rows=to_dev(rows), kv_len=to_dev(kv), out=out, scatter_out=True)
    ref, _ = oracle.sdpa(q.value, k.value, v.value, q_rows=rows, kv_len=kv)
    g = out.float().cpu().numpy()
    for b in range(B):
        assert_attn_close(out[b][torch.from_numpy(rows[b]).long()].unsqueeze(0), ref[b:b + 1], "scatter")
        rest = np.ones(Nq, bool)
        rest[rows[b]] = False
        assert np.all(g[b][rest] == 7.0)
    bad = rows.copy()
    bad[0, 5], bad[1, 140] = -1, Nq + 3
    o = sq.attn_fwd(qd, kd, vd, q_rows=to_dev(bad), kv_len=to_dev(kv))
    for b, r in ((0, 5), (1, 140)):
        zero_ref, _ = oracle.sdpa(np.zeros((1, 1, H, d)), k.value[b:b + 1], v.value[b:b + 1], kv_len=kv[b:b + 1])
        assert_attn_close(o[b:b + 1, r:r + 1], zero_ref, "zero query row")
    out2 = torch.full((B, Nq, H, d), 7.0, dtype=torch.bfloat16, device=qd.device)
    sq.attn_fwd(qd, kd, vd, q_rows=to_dev(bad), kv_len=to_dev(kv), out=out2, scatter_out=True)
    written = np.zeros(Nq, bool)
    written[np.delete(rows[0], 5)] = True       # entry 5 of sample 0 is the invalid one
    assert np.all(out2[0].float().cpu().numpy()[~written] == 7.0), "the invalid entry writes nothing"


def test_short_keys_strided_views_and_many_heads():
    """Query, key, value and output views inside wider buffers; 24 heads (several head
    groups per call) and the full key axis of 1024."""
    B, Nq, Nk, H, d = 2, 700, 1024, 24, 64
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=91)
    dev = torch.device("cuda:0")
    qw = torch.zeros((B, Nq, H, d + 32), dtype=torch.bfloat16, device=dev)
    kw = torch.zeros((B, Nk, H + 1, d), dtype=torch.bfloat16, device=dev)
    vw = torch.zeros((B, Nk, H, 2 * d), dtype=torch.bfloat16, device=dev)
    qw[..., 16:16 + d] = to_dev_bf16(q)
    kw[:, :, 1:] = to_dev_bf16(k)
    vw[..., d:] = to_dev_bf16(v)
    kv = np.array([1024, 517], dtype=np.int32)
    ow = torch.zeros((B, Nq, H, d + 8), dtype=torch.bfloat16, device=dev)
    sq.attn_fwd(qw[..., 16:16 + d], kw[:, :, 1:], vw[..., d:], kv_len=to_dev(kv), out=ow[..., :d])
    ref, _ = oracle.sdpa(q.value, k.value, v.value, kv_len=kv)
    assert_attn_close(ow[..., :d], ref, "strided short")
    assert torch.all(ow[..., d:] == 0), "nothing written past the output view"


@pytest.mark.parametrize("H", [7, 24])
def test_short_keys_several_heads_per_workgroup(H):
    """Enough rows that each workgroup walks several heads (the next head's query rows
    prefetched during the current one), with a head count the groups do not divide evenly
    (H = 7): the oracle on sampled rows of every sample and head."""
    B, Nq, Nk, d = 4, 16384, 300, 64
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=123 + H)
    kv = np.array([300, 1, 64, 211], dtype=np.int32)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    o, lse = sq.attn_fwd(qd, kd, vd, kv_len=to_dev(kv), return_lse=True)
    rng = np.random.default_rng(H)
    samp = np.unique(np.concatenate([[0, 127, 128, Nq - 1], rng.choice(Nq, 60, replace=False)]))
    rows = np.broadcast_to(samp, (B, len(samp))).copy()
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, q_rows=rows, kv_len=kv)
    assert_attn_close(o[:, torch.from_numpy(samp).long()], ref, f"H={H} sampled rows")
    assert_lse_close(lse[:, :, torch.from_numpy(samp).long()], ref_lse, f"H={H} sampled LSE")
