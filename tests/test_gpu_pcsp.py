"""GPU parity of safe_pcsp_select against the oracle (Eq. 9-12)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")

GOLD = os.path.join(os.path.dirname(__file__), "golden")
ACC_RTOL = 1e-4


@pytest.mark.parametrize("number", [1, 2])
def test_accumulate_matches_oracle(number):
    inp = W.workload_inputs(number)
    w = inp["workload"]
    wts = W.pcsp_content_weights(inp["kv_len"], w.M)
    acc = torch.zeros((w.B, w.N), dtype=torch.float32, device=dev())
    qc, kt = to_dev_bf16(inp["q_c"]), to_dev_bf16(inp["k_txt"])
    sq.pcsp_accumulate(qc, kt, to_dev(wts), acc, kv_len=to_dev(inp["kv_len"]))
    ref = oracle.pcsp_accumulate(inp["q_c"].value, inp["k_txt"].value, inp["kv_len"], wts)
    np.testing.assert_allclose(acc.cpu().numpy(), ref, rtol=ACC_RTOL, atol=1e-7)
    # a second call adds (two warm-up calls), a head subset picks heads
    heads = [0, w.H - 1]
    mask = (1 << 0) | (1 << (w.H - 1))
    sq.pcsp_accumulate(qc, kt, to_dev(wts), acc, kv_len=to_dev(inp["kv_len"]), head_mask=mask)
    ref2 = oracle.pcsp_accumulate(inp["q_c"].value, inp["k_txt"].value, inp["kv_len"], wts, heads=heads, acc=ref)
    np.testing.assert_allclose(acc.cpu().numpy(), ref2, rtol=ACC_RTOL, atol=1e-7)


def test_accumulate_split_over_head_groups():
    """With a workspace the heads are split into groups whose sums a second kernel adds
    in group order: same values as unsplit up to rounding, deterministic, and groups
    holding no selected head add nothing."""
    inp = W.workload_inputs(2)
    w = inp["workload"]
    wts = to_dev(W.pcsp_content_weights(inp["kv_len"], w.M))
    qc, kt, kv = to_dev_bf16(inp["q_c"]), to_dev_bf16(inp["k_txt"]), to_dev(inp["kv_len"])
    ref = oracle.pcsp_accumulate(inp["q_c"].value, inp["k_txt"].value, inp["kv_len"], W.pcsp_content_weights(inp["kv_len"], w.M))
    split = torch.zeros((w.B, w.N), dtype=torch.float32, device=dev())
    sq.pcsp_accumulate(qc, kt, wts, split, kv_len=kv)
    plain = torch.zeros_like(split)
    sq.pcsp_accumulate(qc, kt, wts, plain, kv_len=kv, workspace=None)
    np.testing.assert_allclose(split.cpu().numpy(), ref, rtol=ACC_RTOL, atol=1e-7)
    np.testing.assert_allclose(split.cpu().numpy(), plain.cpu().numpy(), rtol=1e-5, atol=1e-7)
    again = torch.zeros_like(split)
    sq.pcsp_accumulate(qc, kt, wts, again, kv_len=kv)
    assert torch.equal(again, split), "split accumulation must be deterministic"
    heads = [3, 17]
    sub = torch.zeros_like(split)
    sq.pcsp_accumulate(qc, kt, wts, sub, kv_len=kv, head_mask=(1 << 3) | (1 << 17))
    ref_sub = oracle.pcsp_accumulate(inp["q_c"].value, inp["k_txt"].value, inp["kv_len"],
                                     W.pcsp_content_weights(inp["kv_len"], w.M), heads=heads)
    np.testing.assert_allclose(sub.cpu().numpy(), ref_sub, rtol=ACC_RTOL, atol=1e-7)


def test_accumulate_ragged_lengths():
    B, N, M, H, d = 3, 300, 80, 2, 64
    q, k, _ = W.attention_inputs(B, N, M, H, d, seed=11)
    kv = np.array([80, 1, 0], np.int32)
    wts = np.random.default_rng(0).random((B, M)).astype(np.float32)
    acc = torch.zeros((B, N), dtype=torch.float32, device=dev())
    sq.pcsp_accumulate(to_dev_bf16(q), to_dev_bf16(k), to_dev(wts), acc, kv_len=to_dev(kv))
    ref = oracle.pcsp_accumulate(q.value, k.value, kv, wts)
    np.testing.assert_allclose(acc.cpu().numpy(), ref, rtol=ACC_RTOL, atol=1e-7)
    assert torch.all(acc[2] == 0)


@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_accumulate_head_dims_and_text_lengths(d):
    """Every head dim, text lengths on and around the 64-key tile edges (0, 1, 63, 64, 65,
    the full M = 300 with a partial last tile), N not a multiple of the 128-token tile, a
    head subset, and with and without the head-group split: the oracle on all tokens."""
    B, N, M, H = 6, 333, 300, 5
    q, k, _ = W.attention_inputs(B, N, M, H, d, seed=40 + d)
    kv = np.array([0, 1, 63, 64, 65, 300], np.int32)
    wts = np.random.default_rng(d).random((B, M)).astype(np.float32)
    ref = oracle.pcsp_accumulate(q.value, k.value, kv, wts)
    for ws in ("auto", None):
        acc = torch.zeros((B, N), dtype=torch.float32, device=dev())
        kw = {} if ws == "auto" else {"workspace": None}
        sq.pcsp_accumulate(to_dev_bf16(q), to_dev_bf16(k), to_dev(wts), acc, kv_len=to_dev(kv), **kw)
        np.testing.assert_allclose(acc.cpu().numpy(), ref, rtol=ACC_RTOL, atol=1e-7)
        assert torch.all(acc[0] == 0)
    heads = [1, 4]
    acc = torch.zeros((B, N), dtype=torch.float32, device=dev())
    sq.pcsp_accumulate(to_dev_bf16(q), to_dev_bf16(k), to_dev(wts), acc, kv_len=to_dev(kv), head_mask=(1 << 1) | (1 << 4))
    ref_h = oracle.pcsp_accumulate(q.value, k.value, kv, wts, heads=heads)
    np.testing.assert_allclose(acc.cpu().numpy(), ref_h, rtol=ACC_RTOL, atol=1e-7)


def test_accumulate_strided_views_and_long_text():
    """Query and key views inside wider buffers (token and head strides not the packed
    ones) and the largest text length (M = 1024, every key valid)."""
    B, N, M, H, d = 2, 260, 1024, 3, 64
    q, k, _ = W.attention_inputs(B, N, M, H, d, seed=77)
    wts = np.random.default_rng(5).random((B, M)).astype(np.float32)
    qd = torch.zeros((B, N, H + 1, d + 16), dtype=torch.bfloat16, device=dev())
    kd = torch.zeros((B, M, H + 2, d + 8), dtype=torch.bfloat16, device=dev())
    qd[:, :, :H, :d] = to_dev_bf16(q)
    kd[:, :, 1:H + 1, 8:] = to_dev_bf16(k)
    acc = torch.zeros((B, N), dtype=torch.float32, device=dev())
    sq.pcsp_accumulate(qd[:, :, :H, :d], kd[:, :, 1:H + 1, 8:], to_dev(wts), acc)
    ref = oracle.pcsp_accumulate(q.value, k.value, np.full(B, M, np.int32), wts)
    np.testing.assert_allclose(acc.cpu().numpy(), ref, rtol=ACC_RTOL, atol=1e-7)


def _select(s: np.ndarray, k: int, gh: int, gw: int, sigma: float = 0.0):
    acc = to_dev(s.astype(np.float32))
    return sq.pcsp_select(acc, gh, gw, sigma, k, score_out=True)


def test_topk_golden_cases():
    for case in json.load(open(os.path.join(GOLD, "topk_hand.json")))["cases"]:
        s = np.asarray([[{"inf": np.inf, "-inf": -np.inf, "nan": np.nan, "-0": -0.0}.get(x, x)
                         if isinstance(x, str) else x for x in case["s"]]], dtype=np.float32)
        idx, _ = _select(s, case["k"], 1, s.shape[1])
        assert idx.cpu().numpy()[0].tolist() == case["idx"], case["why"]


@pytest.mark.parametrize("levels", [None, 8, 1])
@pytest.mark.parametrize("N,grid", [(256, (16, 16)), (4096, (64, 64)), (36864, (192, 192)), (40000, (200, 200))])
def test_topk_bit_exact_on_identical_scores(N, grid, levels):
    """Same fp32 score array on both sides (sigma = 0): identical index sets, lower index wins ties.
    N = 36864 is the largest field held in LDS; N = 40000 takes the path that reads the field
    from global memory in every pass."""
    rng = np.random.default_rng(N + (levels or 0))
    s = W.score_field(rng, 2, N, levels=levels)
    s[0, :5] = [-0.0, 0.0, np.nan, -np.inf, np.inf]
    for k in sorted({1, N // 4, (3 * N) // 10, N - 1, N}):
        idx, _ = _select(s, k, *grid)
        ref = oracle.topk_select(s.astype(np.float64), k)
        assert np.array_equal(idx.cpu().numpy(), ref), (N, levels, k)


def test_smoothing_and_norm_against_oracle():
    rng = np.random.default_rng(5)
    gh, gw = 40, 33
    s = rng.random((2, gh * gw)).astype(np.float32)
    for sigma in (0.7, 1.0, 2.5):
        idx, so = _select(s, 300, gh, gw, sigma)
        sbar = oracle.gaussian_smooth(s.astype(np.float64), gh, gw, sigma)
        ref_norm = oracle.minmax_normalize(sbar)
        np.testing.assert_allclose(so.cpu().numpy(), ref_norm, atol=2e-5)
        # selection: may differ only where the oracle's smoothed score is within a rounding band of the k-th
        ref_idx = oracle.topk_select(sbar, 300)
        for b in range(2):
            got, exp = set(idx[b].cpu().tolist()), set(ref_idx[b].tolist())
            kth = np.sort(sbar[b])[::-1][299]
            band = 1e-5 * np.abs(sbar[b]).max()
            for t in got ^ exp:
                assert abs(sbar[b, t] - kth) <= band, (sigma, t)
            assert np.all(np.diff(idx[b].cpu().numpy()) > 0)


def test_pipeline_tiny_workload():
    """Accumulate -> smooth (sigma 1) -> select on the 16x16 workload."""
    inp = W.workload_inputs(1)
    w = inp["workload"]
    wts = W.pcsp_content_weights(inp["kv_len"], w.M)
    acc = torch.zeros((w.B, w.N), dtype=torch.float32, device=dev())
    sq.pcsp_accumulate(to_dev_bf16(inp["q_c"]), to_dev_bf16(inp["k_txt"]), to_dev(wts), acc,
                       kv_len=to_dev(inp["kv_len"]))
    idx, so = sq.pcsp_select(acc, w.grid_h, w.grid_w, 1.0, w.k_for(25), score_out=True)
    _, sbar, s_norm, ref_idx = oracle.pcsp_scores(inp["q_c"].value, inp["k_txt"].value, inp["kv_len"], wts,
                                                  w.grid_h, w.grid_w, 1.0, w.k_for(25))
    np.testing.assert_allclose(so.cpu().numpy(), s_norm, atol=1e-4)
    got, exp = set(idx[0].cpu().tolist()), set(ref_idx[0].tolist())
    kth = np.sort(sbar[0])[::-1][w.k_for(25) - 1]
    for t in got ^ exp:
        assert abs(sbar[0, t] - kth) <= 1e-4 * np.abs(sbar).max()


def _norm_tol(sbar: np.ndarray) -> float:
    """Bound on |Norm_gpu - Norm_oracle| for one sample row.  The GPU smooths in fp32: each pass of
    at most 2*ceil(3 sigma) + 1 taps (renormalised weights) rounds at most ~16 times, so s_bar is
    off by <= 16 * 2^-24 * max|s_bar| per pass, two passes; min-max then subtracts the minimum
    and divides by (max - min), which turns that absolute error into a relative one scaled by
    max|s_bar| / (max - min), plus a rounding of the quotient.  A field whose spread is small
    against its magnitude (sums over 24 heads of softmax-weighted scores) therefore carries a
    larger Norm error than a unit-range field."""
    span = float(sbar.max() - sbar.min())
    return float(2 * 2 * 16 * 2.0 ** -24 * np.abs(sbar).max() / span + 2.0 ** -22)


def _sampled_tokens(rng, N, per=400):
    """The first two and last two tokens plus `per` random ones."""
    return np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.choice(N, size=per, replace=False)]))


@pytest.mark.parametrize("number", [3, 4, 5])
def test_accumulate_full_size_sampled_tokens(number):
    """Eq. 9-10 at the 128x128, 160x160 and 192x192 grids in the bench's launch configuration
    (head-group split with the binding's workspace): the oracle on sampled image tokens of
    both samples (a token's score depends only on its own query rows)."""
    inp = W.workload_inputs(number)
    w = inp["workload"]
    wts = W.pcsp_content_weights(inp["kv_len"], w.M)
    acc = torch.zeros((w.B, w.N), dtype=torch.float32, device=dev())
    sq.pcsp_accumulate(to_dev_bf16(inp["q_c"]), to_dev_bf16(inp["k_txt"]), to_dev(wts), acc,
                       kv_len=to_dev(inp["kv_len"]))
    samp = _sampled_tokens(W.rng_for(number, stream=8), w.N)
    ref = oracle.pcsp_accumulate(inp["q_c"].value[:, samp], inp["k_txt"].value, inp["kv_len"], wts)
    np.testing.assert_allclose(acc.cpu().numpy()[:, samp], ref, rtol=ACC_RTOL, atol=1e-7)


def test_select_on_the_full_size_field():
    """Eq. 11-12 on the 160x160 workload's own accumulated field (k = 3840 / 6400 / 10240):
    with sigma = 0 both sides rank the identical fp32 array, so the index sets are equal bit
    for bit; with sigma = 1 (the bench's setting) the oracle smooths the same fp32 field in
    fp64, and the sets may differ only at tokens whose oracle score lies within 1e-5 max|s|
    of the k-th score."""
    inp = W.workload_inputs(4)
    w = inp["workload"]
    wts = W.pcsp_content_weights(inp["kv_len"], w.M)
    acc = torch.zeros((w.B, w.N), dtype=torch.float32, device=dev())
    sq.pcsp_accumulate(to_dev_bf16(inp["q_c"]), to_dev_bf16(inp["k_txt"]), to_dev(wts), acc,
                       kv_len=to_dev(inp["kv_len"]))
    field = acc.cpu().numpy().astype(np.float64)
    sbar = oracle.gaussian_smooth(field, w.grid_h, w.grid_w, 1.0)
    for rho in w.rho_percent:
        k = w.k_for(rho)
        idx0 = sq.pcsp_select(acc, w.grid_h, w.grid_w, 0.0, k)
        assert np.array_equal(idx0.cpu().numpy(), oracle.topk_select(field, k)), ("sigma 0", k)
        idx1, so = sq.pcsp_select(acc, w.grid_h, w.grid_w, 1.0, k, score_out=True)
        got_norm, ref_norm = so.cpu().numpy(), oracle.minmax_normalize(sbar)
        for b in range(w.B):
            np.testing.assert_allclose(got_norm[b], ref_norm[b], atol=_norm_tol(sbar[b]))
        ref = oracle.topk_select(sbar, k)
        for b in range(w.B):
            got = idx1[b].cpu().numpy()
            assert got.shape == (k,) and np.all(np.diff(got) > 0)
            kth = np.sort(sbar[b])[::-1][k - 1]
            band = 1e-5 * np.abs(sbar[b]).max()
            diff = set(got.tolist()) ^ set(ref[b].tolist())
            assert all(abs(sbar[b, t] - kth) <= band for t in diff), ("sigma 1", k, b, len(diff))
