"""GPU parity of safe_attn_fwd with a dense mask (Eq. 2 with m given) against the fp64
oracle, and the exactness of dropping a removable mask (Eq. 7-8) on this kernel."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attn_close, assert_lse_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")

TORCH_DT = {"bool": torch.bool, "bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def padded_mask(values: np.ndarray, kind: str, pad_to: int = 16) -> torch.Tensor:
    """A device mask holding `values` [.., Nk] in rows padded to a multiple of `pad_to`
    elements (rows must start 16-byte aligned), returned as the [.., :Nk] view."""
    nk = values.shape[-1]
    width = -(-nk // pad_to) * pad_to
    store = np.zeros(values.shape[:-1] + (width,), dtype=values.dtype)
    store[..., :nk] = values
    t = torch.from_numpy(store).to(TORCH_DT[kind]).to("cuda:0")
    return t[..., :nk]


def additive_values(rng, shape, kind):
    """Random finite biases with ~30% -inf, rounded to the mask dtype (the oracle gets the
    rounded values), with one fully blocked query row and one row blocked on its first 200 keys."""
    m = rng.uniform(-4.0, 4.0, size=shape)
    m[rng.random(shape) < 0.3] = -np.inf
    m[..., 3, :] = -np.inf
    m[..., 5, :200] = -np.inf
    m[..., 5, 200] = 0.0
    exact = torch.from_numpy(m).to(TORCH_DT[kind]).to(torch.float64).numpy()
    return exact


@pytest.mark.parametrize("kind", ["bool", "bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [32, 72, 96, 128])
def test_masked_against_oracle(d, kind):
    B, Nq, Nk, H = 2, 301, 333, 3
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=300 + d)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rng = np.random.default_rng(d * 7 + len(kind))
    if kind == "bool":
        keep = rng.random((1, H, Nq, Nk)) < 0.6
        keep[..., 3, :] = False                      # a row with no attended key
        keep[..., 5, :] = False
        keep[..., 5, 250:] = True                    # attended keys only from tile 3 on
        mask = padded_mask(keep.astype(np.uint8), kind).bool()
        ref_mask = oracle.mask.to_additive(keep, True)
    else:
        vals = additive_values(rng, (B, 1, Nq, Nk), kind)
        mask = padded_mask(vals, kind)
        ref_mask = vals
    o, lse = sq.attn_fwd(qd, kd, vd, mask=mask, return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, mask=ref_mask)
    assert_attn_close(o, ref, f"masked dense d={d} {kind}")
    assert_lse_close(lse, ref_lse, f"masked dense d={d} {kind}")
    assert torch.all(o[:, 3] == 0), "a fully blocked row gives zero output"
    # gathered per-sample rows (the mask row is the query token's), scattered output
    rows = np.stack([W.random_rows(rng, Nq, 77) for _ in range(B)])
    rows[:, 0] = 3
    rows[:, 1] = 5
    rows.sort(axis=1)
    out = torch.full((B, Nq, H, d), 5.0, dtype=torch.bfloat16, device=qd.device)
    _, lse = sq.attn_fwd(qd, kd, vd, q_rows=to_dev(rows), mask=mask, out=out, scatter_out=True, return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, q_rows=rows, mask=ref_mask)
    for b in range(B):
        assert_attn_close(out[b][torch.from_numpy(rows[b]).long()].unsqueeze(0), ref[b:b + 1], "masked scatter")
    assert_lse_close(lse, ref_lse, f"masked rows d={d} {kind}")


@pytest.mark.parametrize("H", [4, 6, 8])
def test_head_shared_row_mask_groups_heads(H):
    """A per-row mask shared by the heads ([B, 1, Nq, Nk]) runs its tiles in groups of four
    (H = 4, 8) or two (H = 6) heads of one row tile: every head's rows still get their own
    outputs and LSE (oracle), on all rows and on gathered rows."""
    B, Nq, Nk, d = 2, 1500, 700, 64
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=600 + H)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rng = np.random.default_rng(600 + H)
    vals = additive_values(rng, (B, 1, Nq, Nk), "bf16")
    mask = padded_mask(vals, "bf16")
    o, lse = sq.attn_fwd(qd, kd, vd, mask=mask, return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, mask=vals)
    assert_attn_close(o, ref, f"head-shared mask H={H}")
    assert_lse_close(lse, ref_lse, f"head-shared mask H={H}")
    rows = np.stack([W.random_rows(rng, Nq, 333) for _ in range(B)])
    o2 = sq.attn_fwd(qd, kd, vd, q_rows=to_dev(rows), mask=mask)
    ref2, _ = oracle.sdpa(q.value, k.value, v.value, q_rows=rows, mask=vals)
    assert_attn_close(o2, ref2, f"head-shared mask rows H={H}")


def test_removable_masks_are_exact_to_drop():
    """Eq. 7-8 on this kernel: an all-valid Boolean mask and a zero additive mask give
    bit-identical outputs to the mask-free call (same scores, same softmax order); a
    row-constant additive mask stays within tolerance of the oracle's mask-free result."""
    B, N, H, d = 2, 528, 4, 96
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=31)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    plain = sq.attn_fwd(qd, kd, vd, workspace=None)
    ones = torch.ones((B, 1, N, N), dtype=torch.bool, device=qd.device)
    assert torch.equal(sq.attn_fwd(qd, kd, vd, mask=ones, workspace=None), plain)
    zeros = torch.zeros((B, 1, N, N), dtype=torch.bfloat16, device=qd.device)
    assert torch.equal(sq.attn_fwd(qd, kd, vd, mask=zeros, workspace=None), plain)
    rng = np.random.default_rng(8)
    c = rng.uniform(-5, 5, size=(1, 1, N, 1)).astype(np.float32)
    row_const = torch.from_numpy(np.broadcast_to(c, (1, 1, N, N)).copy()).to("cuda:0")
    o = sq.attn_fwd(qd, kd, vd, mask=row_const)
    ref, _ = oracle.sdpa(q.value, k.value, v.value)
    assert_attn_close(o, ref, "row-constant mask")


def test_broadcast_key_mask_equals_key_lengths():
    """A [B, 1, 1, Nk] Boolean key-padding mask (query stride 0) gives the kv_len result."""
    B, Nq, Nk, H, d = 3, 200, 256, 2, 64
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=33)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    kv = np.array([256, 1, 130], dtype=np.int32)
    keep = np.arange(Nk)[None, :] < kv[:, None]
    mask = torch.from_numpy(keep[:, None, None, :]).to("cuda:0")
    o, lse = sq.attn_fwd(qd, kd, vd, mask=mask, return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, kv_len=kv)
    assert_attn_close(o, ref, "key mask")
    assert_lse_close(lse, ref_lse, "key mask")
    o2 = sq.attn_fwd(qd, kd, vd, kv_len=to_dev(kv))
    assert (o.float() - o2.float()).abs().max().item() <= 1e-2


def test_masked_tail_split_and_invalid_rows():
    """Split tail tiles carry the mask through the key ranges; rows outside [0, Nq) read a
    zero query and mask row 0."""
    B, Nq, Nk, H, d = 1, 300, 3000, 2, 96
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=35)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rng = np.random.default_rng(35)
    vals = additive_values(rng, (1, H, Nq, Nk), "bf16")
    vals[..., 7, :2900] = -np.inf                   # only the last key range attends
    mask = padded_mask(vals, "bf16")
    assert sq.attn_workspace_bytes(qd, kd, mask=mask) > 0, "this shape must be split"
    o, lse = sq.attn_fwd(qd, kd, vd, mask=mask, return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, mask=vals)
    assert_attn_close(o, ref, "masked split")
    assert_lse_close(lse, ref_lse, "masked split")
    plain = sq.attn_fwd(qd, kd, vd, mask=mask, workspace=None)
    assert (o.float() - plain.float()).abs().max().item() <= 2e-2
    rows = to_dev(np.array([7, Nq + 3, -1, 12], dtype=np.int32))
    o = sq.attn_fwd(qd, kd, vd, q_rows=rows, mask=mask)
    ref0, _ = oracle.sdpa(np.zeros((1, 1, H, d)), k.value, v.value, mask=vals[:, :, 0:1, :])
    assert_attn_close(o[:, 1:3], np.concatenate([ref0, ref0], axis=1), "invalid rows use mask row 0")
    ref7, _ = oracle.sdpa(q.value, k.value, v.value, q_rows=[7, 12], mask=vals)
    assert_attn_close(o[:, [0, 3]], ref7, "valid rows")


def test_mask_argument_errors():
    B, N, H, d = 1, 64, 1, 64
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=37)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    m = torch.ones((1, 1, N, N), dtype=torch.bool, device=qd.device)
    with pytest.raises(sq.SafeError) as e:
        sq.attn_fwd(qd, kd, vd, mask=m, kv_len=to_dev(np.array([10], np.int32)))
    assert e.value.status == -5
    odd = torch.ones((1, 1, N, N + 8), dtype=torch.bool, device=qd.device)[..., :N]   # row stride 72 bytes
    with pytest.raises(sq.SafeError) as e:
        sq.attn_fwd(qd, kd, vd, mask=odd)
    assert e.value.status == -8
    with pytest.raises(ValueError):
        sq.attn_fwd(qd, kd, vd, mask=torch.ones((1, 1, N, N - 1), dtype=torch.bool, device=qd.device))
