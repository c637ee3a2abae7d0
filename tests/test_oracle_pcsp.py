"""Pins of the PCSP oracle (Eq. 9-12)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.ndimage
import torch

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        return {"inf": np.inf, "-inf": -np.inf, "nan": np.nan, "-0": -0.0}[x]
    return float(x)


def test_accumulate_matches_torch_softmax():
    rng = np.random.default_rng(0)
    B, N, M, H, d = 2, 30, 12, 3, 8
    q = rng.standard_normal((B, N, H, d))
    kt = rng.standard_normal((B, M, H, d))
    kv = np.array([12, 5])
    w = rng.random((B, M))
    heads = [0, 2]
    acc = oracle.pcsp_accumulate(q, kt, kv, w, heads=heads)
    ref = np.zeros((B, N))
    for b in range(B):
        for h in heads:
            logits = torch.from_numpy(q[b, :, h] @ kt[b, :, h].T / math.sqrt(d))
            logits[:, kv[b]:] = -math.inf
            A = torch.softmax(logits, dim=-1).numpy()
            ref[b] += A[:, :kv[b]] @ w[b, :kv[b]]
    np.testing.assert_allclose(acc, ref, rtol=1e-13, atol=1e-15)


def test_accumulate_closed_forms():
    rng = np.random.default_rng(1)
    B, N, M, H, d = 2, 16, 10, 4, 8
    q = rng.standard_normal((B, N, H, d))
    kt = rng.standard_normal((B, M, H, d))
    kv = np.array([10, 3])
    # unit weights on valid keys: every A row sums to 1 -> acc = |H|
    ones = np.ones((B, M))
    np.testing.assert_allclose(oracle.pcsp_accumulate(q, kt, kv, ones), H, atol=1e-13)
    # one valid key: A = 1 -> acc = |H| w_0
    w = rng.random((B, M))
    np.testing.assert_allclose(oracle.pcsp_accumulate(q, kt, [1, 1], w, heads=[1, 3]),
                               2 * w[:, :1] * np.ones((B, N)), atol=1e-15)
    # zero queries: uniform A over valid keys -> acc = |H| * mean of valid weights
    acc = oracle.pcsp_accumulate(np.zeros_like(q), kt, kv, w)
    for b in range(B):
        np.testing.assert_allclose(acc[b], H * w[b, :kv[b]].mean(), atol=1e-14)
    # identical text keys: A = 1/L on every valid key -> acc = |H| * sum(w[:L]) / L
    kt_same = np.broadcast_to(kt[:, :1], kt.shape)
    acc = oracle.pcsp_accumulate(q, kt_same, kv, w)
    for b in range(B):
        np.testing.assert_allclose(acc[b], H * w[b, :kv[b]].sum() / kv[b], rtol=1e-13)
    # accumulation adds to the existing vector
    base = rng.random((B, N))
    np.testing.assert_allclose(oracle.pcsp_accumulate(q, kt, kv, w, acc=base),
                               base + oracle.pcsp_accumulate(q, kt, kv, w), atol=1e-15)
    # a fully padded sample contributes nothing
    assert np.all(oracle.pcsp_accumulate(q, kt, [0, 3], w)[0] == 0)


def test_uniform_weights_over_all_valid_keys_give_a_constant_field():
    """Why special tokens must get zero weight (Eq. 10): rows of A sum to 1."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 9, 2, 4))
    kt = rng.standard_normal((2, 7, 2, 4))
    kv = np.array([7, 4])
    w_all = np.zeros((2, 7))
    w_all[0, :7] = 1 / 7
    w_all[1, :4] = 1 / 4
    acc = oracle.pcsp_accumulate(q, kt, kv, w_all)
    np.testing.assert_allclose(acc[0], acc[0, 0], rtol=1e-13)
    np.testing.assert_allclose(acc[1], acc[1, 0], rtol=1e-13)
    w = W.pcsp_content_weights(kv, 7)
    assert np.all(w[:, 0] == 0) and np.all(w[1, 4:] == 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    acc = oracle.pcsp_accumulate(q, kt, kv, w)
    assert np.ptp(acc[0]) > 1e-3 and np.ptp(acc[1]) > 1e-3


def test_smoothing_identity_constant_impulse():
    rng = np.random.default_rng(3)
    s = rng.random((2, 12 * 9))
    assert np.array_equal(oracle.gaussian_smooth(s, 12, 9, 0.0), s)
    const = np.full((1, 12 * 9), 0.3)
    np.testing.assert_allclose(oracle.gaussian_smooth(const, 12, 9, 1.3), 0.3, atol=1e-15)
    taps = oracle.gaussian_taps(1.0)
    assert taps.size == 7 and taps[3] == 1.0 and abs(taps[0] - math.exp(-4.5)) < 1e-16
    # impulse far from the border reproduces the normalised 2-D taps
    imp = np.zeros((1, 15 * 15))
    imp[0, 7 * 15 + 7] = 1.0
    out = oracle.gaussian_smooth(imp, 15, 15, 1.0).reshape(15, 15)
    t = taps / taps.sum()
    np.testing.assert_allclose(out[4:11, 4:11], np.outer(t, t), atol=1e-16)
    assert np.all(out[:4] == 0) and np.all(out[:, 11:] == 0)


def test_smoothing_against_scipy_and_direct_2d():
    rng = np.random.default_rng(4)
    gh, gw, sigma = 11, 14, 1.5
    s = rng.random((2, gh * gw))
    ours = oracle.gaussian_smooth(s, gh, gw, sigma)
    taps = oracle.gaussian_taps(sigma)
    # library: zero-padded correlation, renormalised by the same filter applied to ones
    for b in range(2):
        g = s[b].reshape(gh, gw)
        num = scipy.ndimage.correlate1d(scipy.ndimage.correlate1d(g, taps, axis=1, mode="constant"),
                                        taps, axis=0, mode="constant")
        den = scipy.ndimage.correlate1d(scipy.ndimage.correlate1d(np.ones_like(g), taps, axis=1, mode="constant"),
                                        taps, axis=0, mode="constant")
        np.testing.assert_allclose(ours[b].reshape(gh, gw), num / den, rtol=1e-13)
    # direct 2-D window with 2-D renormalisation over in-grid taps
    r = (taps.size - 1) // 2
    g = s[0].reshape(gh, gw)
    direct = np.zeros_like(g)
    for y in range(gh):
        for x in range(gw):
            num = den = 0.0
            for dy in range(-r, r + 1):
                for dx in range(-r, r + 1):
                    if 0 <= y + dy < gh and 0 <= x + dx < gw:
                        wgt = math.exp(-(dy * dy + dx * dx) / (2 * sigma * sigma))
                        num += wgt * g[y + dy, x + dx]
                        den += wgt
            direct[y, x] = num / den
    np.testing.assert_allclose(ours[0].reshape(gh, gw), direct, rtol=1e-13)


def test_minmax_normalize():
    s = np.array([[2.0, 4.0, 3.0], [1.0, 1.0, 1.0]])
    out = oracle.minmax_normalize(s)
    np.testing.assert_allclose(out[0], [0.0, 1.0, 0.5])
    assert np.all(out[1] == 0)


def test_topk_golden():
    g = json.load(open(os.path.join(GOLD, "topk_hand.json")))
    for case in g["cases"]:
        s = np.asarray([[_num(x) for x in case["s"]]])
        assert list(oracle.topk_select(s, case["k"])[0]) == case["idx"], case["why"]


def _topk_bruteforce(row, k):
    """Token i is selected iff fewer than k tokens outrank it (O(N^2) count)."""
    def better(a, ia, b, ib):        # does (a, ia) outrank (b, ib)?
        na, nb = a != a, b != b
        if na != nb:
            return nb
        if not na and a != b:
            return a > b
        return ia < ib
    sel = [i for i in range(len(row)) if sum(better(row[j], j, row[i], i) for j in range(len(row))) < k]
    return sel


@pytest.mark.parametrize("levels", [None, 8, 2])
def test_topk_bruteforce(levels):
    rng = np.random.default_rng(5)
    s = W.score_field(rng, 2, 97, levels=levels).astype(np.float64)
    s[0, 10] = -0.0
    s[0, 11] = 0.0
    s[1, 5] = np.nan
    s[1, 6] = -np.inf
    for k in [0, 1, 13, 50, 96, 97]:
        idx = oracle.topk_select(s, k)
        for b in range(2):
            assert list(idx[b]) == _topk_bruteforce([float(x) for x in s[b]], k)


def test_pcsp_pipeline_on_tiny_workload():
    inp = W.workload_inputs(1)
    w = inp["workload"]
    wts = W.pcsp_content_weights(inp["kv_len"], w.M)
    acc, s_bar, s_norm, idx = oracle.pcsp_scores(inp["q_c"].value, inp["k_txt"].value, inp["kv_len"], wts,
                                                 w.grid_h, w.grid_w, 1.0, w.k_for(25))
    assert idx.shape == (1, 64) and np.all(np.diff(idx[0]) > 0)
    assert s_norm.min() == 0.0 and s_norm.max() == 1.0
    # selected tokens outrank every unselected token
    sel = np.zeros(w.N, bool)
    sel[idx[0]] = True
    assert s_bar[0, sel].min() >= s_bar[0, ~sel].max()
    # each row of A sums to 1 and the start token has weight 0, so a token's score
    # is |H| minus its start-token attention, scaled by 1/(L-1): within (0, |H|/(L-1))
    L = int(inp["kv_len"][0])
    assert np.all(acc > 0) and np.all(acc < w.H / (L - 1)) and np.ptp(acc) > 1e-3
