"""GPU parity of safe_sdpa, the Eq. 8 rewrite as one call, against the oracle's safe_sdpa:
for masks of every row class (Eq. 6 and the statements after Eq. 7) the call certifies the
mask, takes the route the oracle takes (mask dropped, text padding kept as per-sample key
lengths, or mask kept) and matches the oracle's output; dropped masks give the mask-free
call's output bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attn_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")

B, NQ, NK, H, D = 2, 200, 176, 3, 64      # NK: whole 16-byte mask rows, a partial 64-key tile


def _inputs(seed):
    q, k, v = W.attention_inputs(B, NQ, NK, H, D, seed=seed)
    return q, k, v, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)


def _masks(rng):
    """(name, stored mask values, torch dtype, Boolean?, expected overall class)."""
    pad = np.zeros((B, 1, NQ, NK), np.float32)
    pad[0, ..., 37:] = -np.inf                              # sample 0: 37 valid keys; sample 1: all valid
    shared_pad = np.zeros((1, 1, NQ, NK), np.float32)
    shared_pad[..., 50:] = -np.inf                          # one text-padding mask for both samples
    bool_pad = np.ones((B, 1, 1, NK), np.uint8)
    bool_pad[0, ..., 100:] = 0
    bool_pad[1, ..., 9:] = 0
    blocked = rng.uniform(-2, 2, (1, H, NQ, NK)).astype(np.float32)
    blocked[0, 1, 7, 13] = -np.inf                          # a blocked key that is not a suffix
    nonfinite = np.zeros((B, 1, NQ, NK), np.float32)
    nonfinite[1, 0, 11, 5] = np.nan
    return [
        ("all_valid_bool", np.ones((B, H, NQ, NK), np.uint8), torch.bool, True, oracle.ALL_VALID),
        ("zero_bf16", np.zeros((1, 1, NQ, NK), np.float32), torch.bfloat16, False, oracle.ZERO),
        ("row_const_f32", W.mask_row_constant_f32(rng, NQ, NK, -5.0, 5.0), torch.float32, False, oracle.ROW_CONST),
        ("key_padding_f32", pad, torch.float32, False, oracle.KEY_PADDING),
        ("key_padding_shared_f16", shared_pad, torch.float16, False, oracle.KEY_PADDING),
        ("key_padding_bool_keys", bool_pad, torch.bool, True, oracle.KEY_PADDING),
        ("nonconst_f32", rng.standard_normal((1, 1, NQ, NK)).astype(np.float32), torch.float32, False,
         oracle.NONCONST),
        ("blocked_bf16_per_head", blocked, torch.bfloat16, False, oracle.BLOCKED),
        ("nonfinite_f32", nonfinite, torch.float32, False, oracle.NONFINITE),
    ]


@pytest.mark.parametrize("case", range(9))
def test_sdpa_routes_and_values_match_the_oracle(case):
    rng = np.random.default_rng(70 + case)
    name, values, tdt, is_bool, cls = _masks(rng)[case]
    q, k, v, qd, kd, vd = _inputs(71)
    mask = torch.from_numpy(values).to(tdt).to("cuda:0")
    stored = mask.to(torch.float64).cpu().numpy() if not is_bool else values   # the bits the GPU reads
    ref_o, _, verdict, ref_route = oracle.safe_sdpa(q.value, k.value, v.value, stored, is_bool=is_bool)
    assert verdict.mask_class == cls, (name, verdict.mask_class)
    out, info = sq.sdpa(qd, kd, vd, mask=mask)
    route = {"none": "no_mask", "kv_len": "kv_len", "mask": "mask"}[ref_route]
    assert info["route"] == route, (name, info)
    assert info["mask_class"] == oracle.CLASS_NAMES[cls], (name, info)
    assert info["first_bad_row"] == verdict.first_bad_row, (name, info)
    # a query row whose mask row holds NaN or +inf has no softmax (Eq. 2 is undefined there):
    # such rows are left out of the comparison; every other row must match
    full = np.broadcast_to(stored, (B, H, NQ, NK)) if not is_bool else None
    undefined = np.zeros((B, NQ), bool) if full is None else \
        (np.isnan(full) | (full == np.inf)).any(axis=(1, 3))
    if undefined.any():
        for b in range(B):
            sel = np.nonzero(~undefined[b])[0]
            assert_attn_close(out[b:b + 1, torch.from_numpy(sel).long()], ref_o[b:b + 1, sel], f"{name} b={b}")
    else:
        assert_attn_close(out, ref_o, name)
    if route == "no_mask":
        assert torch.equal(out, sq.attn_fwd(qd, kd, vd)), f"{name}: a dropped mask is the mask-free call"
    elif route == "kv_len":
        L = torch.from_numpy(np.broadcast_to(verdict.kv_len, (B,)).astype(np.int32).copy()).cuda()
        assert torch.equal(out, sq.attn_fwd(qd, kd, vd, kv_len=L)), f"{name}: padding kept as key lengths"


def test_sdpa_on_gathered_rows_and_without_a_mask():
    """The rewrite on the SRSU form (gathered query rows, the mask indexed by query token)
    and the no-mask call (nothing to certify)."""
    rng = np.random.default_rng(80)
    q, k, v, qd, kd, vd = _inputs(81)
    rows = np.stack([W.random_rows(rng, NQ, 61) for _ in range(B)])
    rows_t = to_dev(rows)
    vals = rng.standard_normal((B, 1, NQ, NK)).astype(np.float32)
    mask = torch.from_numpy(vals).cuda()
    out, info = sq.sdpa(qd, kd, vd, mask=mask, q_rows=rows_t)
    assert info["route"] == "mask" and info["mask_class"] == "NONCONST"
    ref, _ = oracle.sdpa(q.value, k.value, v.value, q_rows=rows, mask=vals.astype(np.float64))
    assert_attn_close(out, ref, "gathered rows, kept mask")
    const = torch.from_numpy(W.mask_row_constant_f32(rng, NQ, NK, -3.0, 3.0)).cuda()
    out, info = sq.sdpa(qd, kd, vd, mask=const, q_rows=rows_t)
    assert info["route"] == "no_mask" and info["mask_class"] == "ROW_CONST"
    assert torch.equal(out, sq.attn_fwd(qd, kd, vd, q_rows=rows_t))
    out, lse, info = sq.sdpa(qd, kd, vd, return_lse=True)
    assert info == {"route": "no_mask", "mask_class": None, "first_bad_row": -1}
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value)
    assert_attn_close(out, ref, "no mask")


def test_sdpa_unaligned_mask_rows():
    """The classifier reads masks of any alignment: a removable mask whose rows are not
    16-byte aligned is dropped and the call runs; a kept one needs the masked kernel's
    aligned rows and is refused (SAFE_ERR_ALIGN) after the scan, with nothing written."""
    _, _, _, qd, kd, vd = _inputs(82)
    store = torch.zeros((1, 1, NQ, NK + 1), dtype=torch.float32, device="cuda")
    out, info = sq.sdpa(qd, kd, vd, mask=store[..., :NK])
    assert info["route"] == "no_mask" and torch.equal(out, sq.attn_fwd(qd, kd, vd))
    store[..., 3] = 1.0
    sentinel = torch.full_like(out, 9.0)
    with pytest.raises(sq.SafeError) as e:
        sq.sdpa(qd, kd, vd, mask=store[..., :NK], out=sentinel)
    assert e.value.status == -8
    assert bool((sentinel == 9.0).all())
