"""Pins of the attention oracle (Eq. 2, 5, 7, 16, 17) against things other than itself."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def torch_sdpa_f64(q, k, v, q_rows=None, kv_len=None, scale=None, attn_mask=None):
    """torch's CPU float64 scaled_dot_product_attention on BNHD inputs (library routine).

    attn_mask: a [B|1, H|1, Nq, Nk] bool (True = attend) or additive float64 mask over the
    full query range; it is gathered to the selected rows here."""
    q = torch.from_numpy(np.asarray(q, dtype=np.float64))
    k = torch.from_numpy(np.asarray(k, dtype=np.float64))
    v = torch.from_numpy(np.asarray(v, dtype=np.float64))
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    if q_rows is not None:
        rows = torch.as_tensor(np.broadcast_to(np.asarray(q_rows), (B, len(np.asarray(q_rows).reshape(B, -1)[0]))).copy()
                               if np.asarray(q_rows).ndim == 2 else np.asarray(q_rows))
        if rows.ndim == 1:
            q = q[:, rows]
        else:
            q = torch.stack([q[b, rows[b]] for b in range(B)])
    mask = None
    if kv_len is not None:
        mask = torch.arange(Nk)[None, :] < torch.as_tensor(np.asarray(kv_len))[:, None]   # True = attend
        mask = mask[:, None, None, :]
    if attn_mask is not None:
        mask = torch.as_tensor(np.asarray(attn_mask))
        if q_rows is not None:
            r = np.asarray(q_rows)
            mask = mask.expand(B, -1, -1, -1)
            mask = torch.stack([mask[b][:, torch.as_tensor(r if r.ndim == 1 else r[b])] for b in range(B)])
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3), attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "attention_hand.json")))
    q, k, v = (np.asarray(g[x], dtype=np.float64) for x in ("q", "k", "v"))
    for case in g["cases"]:
        o, lse = oracle.sdpa(q, k, v, kv_len=[case["kv_len"]])
        np.testing.assert_allclose(o[0, 0, 0], case["o"], rtol=0, atol=1e-15)
        assert abs(lse[0, 0, 0] - case["lse"]) < 1e-15


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_torch_sdpa_f64(seed):
    rng = np.random.default_rng(seed)
    B, Nq, Nk, H, d = 2, 37, 53, 3, 16
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, H, d))
    v = rng.standard_normal((B, Nk, H, d))
    o, _ = oracle.sdpa(q, k, v)
    np.testing.assert_allclose(o, torch_sdpa_f64(q, k, v), rtol=0, atol=1e-12)
    rows = np.sort(rng.choice(Nq, 11, replace=False))
    kv = np.array([53, 7])
    o, _ = oracle.sdpa(q, k, v, q_rows=rows, kv_len=kv)
    np.testing.assert_allclose(o, torch_sdpa_f64(q, k, v, q_rows=rows, kv_len=kv), rtol=0, atol=1e-12)
    o, _ = oracle.sdpa(q, k, v, scale=0.37)
    np.testing.assert_allclose(o, torch_sdpa_f64(q, k, v, scale=0.37), rtol=0, atol=1e-12)


def test_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 9, 2, 8))
    k = rng.standard_normal((1, 13, 2, 8))
    v = rng.standard_normal((1, 13, 2, 8))
    _, lse = oracle.sdpa(q, k, v, kv_len=[10])
    logits = torch.einsum("bqhd,bkhd->bhqk", torch.from_numpy(q), torch.from_numpy(k[:, :10])) / math.sqrt(8)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(7)
    B, N, H, d = 1, 6, 2, 4
    q = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    # identical keys: uniform weights over the valid keys -> mean of values
    k_same = np.broadcast_to(rng.standard_normal((1, 1, H, d)), (B, N, H, d))
    o, _ = oracle.sdpa(q, k_same, v, kv_len=[4])
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0, :4].mean(axis=0), (N, H, d)), atol=1e-14)
    # constant value rows -> that value
    k = rng.standard_normal((B, N, H, d))
    v_const = np.broadcast_to(np.arange(d, dtype=np.float64), (B, N, H, d))
    o, _ = oracle.sdpa(q, k, v_const)
    np.testing.assert_allclose(o, v_const, atol=1e-14)
    # one valid key -> its value, LSE = its logit
    o, lse = oracle.sdpa(q, k, v, kv_len=[1])
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0, 0], (N, H, d)), atol=0)
    np.testing.assert_allclose(lse[0], np.einsum("nhd,hd->hn", q[0], k[0, 0]) / 2.0, atol=1e-14)
    # zero scale -> uniform average of all values
    o, _ = oracle.sdpa(q, k, v, scale=0.0)
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0].mean(axis=0), (N, H, d)), atol=1e-14)
    # a dominant key takes all the weight
    k_dom = k.copy()
    k_dom[0, 3] = 400.0 * q[0, 2]
    o, _ = oracle.sdpa(q[:, 2:3], k_dom, v)
    np.testing.assert_allclose(o[0, 0], v[0, 3], atol=1e-12)
    # no valid key: output 0, LSE -inf (reading for kv_len = 0)
    o, lse = oracle.sdpa(q, k, v, kv_len=[0])
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_row_shift_invariance_eq7():
    rng = np.random.default_rng(11)
    B, N, H, d = 2, 20, 3, 8
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    c = rng.uniform(-5, 5, size=(B, H, N, 1))
    mask = np.broadcast_to(c, (B, H, N, N))
    o_m, lse_m = oracle.sdpa(q, k, v, mask=mask)
    o_0, lse_0 = oracle.sdpa(q, k, v)
    np.testing.assert_allclose(o_m, o_0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_m - c[..., 0], lse_0, atol=1e-12)
    # a zero additive mask leaves the logits bit-identical
    o_z, _ = oracle.sdpa(q, k, v, mask=np.zeros((1, 1, N, N)))
    assert np.array_equal(o_z, o_0)
    # a non-constant row changes the output (converse of Eq. 7)
    bump = np.zeros((1, 1, N, N))
    bump[..., 0, 1] = 1.0
    o_b, _ = oracle.sdpa(q, k, v, mask=bump)
    assert np.max(np.abs(o_b[:, 0] - o_0[:, 0])) > 1e-6
    assert np.array_equal(o_b[:, 1:], o_0[:, 1:])


def test_kv_len_is_suffix_minus_inf_mask():
    rng = np.random.default_rng(3)
    B, Nq, Nk, H, d = 2, 5, 9, 2, 4
    q = rng.standard_normal((B, Nq, H, d))
    k, v = rng.standard_normal((B, Nk, H, d)), rng.standard_normal((B, Nk, H, d))
    kv = np.array([6, 2])
    m = np.zeros((B, 1, 1, Nk))
    for b in range(B):
        m[b, ..., kv[b]:] = -np.inf
    o1, l1 = oracle.sdpa(q, k, v, kv_len=kv)
    o2, l2 = oracle.sdpa(q, k, v, mask=m)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)


def test_srsu_all_rows_equals_dense():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((2, 17, 2, 8)) for _ in range(3))
    o_d, l_d = oracle.sdpa(q, k, v)
    o_s, l_s = oracle.sdpa(q, k, v, q_rows=np.arange(17))
    assert np.array_equal(o_d, o_s) and np.array_equal(l_d, l_s)
    rows = np.array([[0, 5, 16], [2, 3, 4]])
    o_p, _ = oracle.sdpa(q, k, v, q_rows=rows)
    for b in range(2):
        assert np.array_equal(o_p[b], o_d[b, rows[b]])


def test_bruteforce_tiny_workload_rows():
    inp = W.workload_inputs(1)
    q, k, v = inp["q_x"].value, inp["k_x"].value, inp["v_x"].value
    rows = np.array([0, 1, 100, 255])
    o, lse = oracle.sdpa(q, k, v, q_rows=rows)
    ob, lb = oracle.sdpa_bruteforce(q, k, v, q_rows=rows)
    np.testing.assert_allclose(o, np.asarray(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.asarray(lb), rtol=0, atol=1e-12)
    # cross-attention against 11 valid text keys
    o, _ = oracle.sdpa(inp["q_c"].value, inp["k_txt"].value, inp["v_txt"].value, q_rows=rows, kv_len=inp["kv_len"])
    ob, _ = oracle.sdpa_bruteforce(inp["q_c"].value, inp["k_txt"].value, inp["v_txt"].value, q_rows=rows,
                                   kv_len=inp["kv_len"])
    np.testing.assert_allclose(o, np.asarray(ob), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_general_mask_matches_torch_sdpa_f64(seed):
    """Eq. 2 with a dense mask: additive (finite values and -inf) and Boolean, on all rows
    and on gathered rows (the mask is indexed by the query token)."""
    rng = np.random.default_rng(100 + seed)
    B, Nq, Nk, H, d = 2, 19, 23, 3, 8
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, H, d))
    v = rng.standard_normal((B, Nk, H, d))
    add = rng.uniform(-4, 4, size=(B, 1, Nq, Nk))
    add[rng.random(add.shape) < 0.3] = -np.inf
    add[..., 0] = rng.uniform(-1, 1, size=(B, 1, Nq))   # every row keeps a key (torch gives NaN otherwise)
    keep = rng.random((1, H, Nq, Nk)) < 0.6
    keep[..., 5] = True
    rows = np.sort(rng.choice(Nq, 7, replace=False))
    for m_oracle, m_torch in ((add, add), (oracle.mask.to_additive(keep, True), keep)):
        o, _ = oracle.sdpa(q, k, v, mask=m_oracle)
        np.testing.assert_allclose(o, torch_sdpa_f64(q, k, v, attn_mask=m_torch), rtol=0, atol=1e-12)
        o, _ = oracle.sdpa(q, k, v, q_rows=rows, mask=m_oracle)
        np.testing.assert_allclose(o, torch_sdpa_f64(q, k, v, q_rows=rows, attn_mask=m_torch), rtol=0, atol=1e-12)


def test_fully_blocked_mask_row_reading():
    """A row whose every key is blocked has no distribution: output 0 and LSE -inf (the
    same reading as kv_len = 0); the other rows are untouched."""
    rng = np.random.default_rng(7)
    B, N, H, d = 1, 6, 2, 4
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    m = np.zeros((1, 1, N, N))
    m[0, 0, 2, :] = -np.inf
    o, lse = oracle.sdpa(q, k, v, mask=m)
    o0, lse0 = oracle.sdpa(q, k, v)
    assert np.all(o[:, 2] == 0) and np.all(lse[:, :, 2] == -np.inf)
    keep = np.ones(N, bool)
    keep[2] = False
    assert np.array_equal(o[:, keep], o0[:, keep]) and np.array_equal(lse[..., keep], lse0[..., keep])
