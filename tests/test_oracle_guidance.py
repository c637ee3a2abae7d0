"""CPU pins of the SW-CFG oracle (Eq. 20, 21) against things other than itself."""
import json
import os

import numpy as np
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sw_cfg_hand.json")


def _rand(seed, B=2, N=37, C=12):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, N, C)), rng.standard_normal((B, N, C)), rng.random((B, N))


def test_hand_worked_example():
    g = json.load(open(GOLD))
    gamma = oracle.guidance_scales(g["s"], g["g_ctx"], g["g_sens"])
    assert np.array_equal(gamma, np.array(g["gamma"]))
    assert np.array_equal(oracle.sw_cfg(g["f_c"], g["f_u"], gamma), np.array(g["f_hat"]))
    gb = oracle.binary_scales(g["binary_idx"], 1, 3, g["g_ctx"], g["g_sens"])
    assert np.array_equal(gb, np.array(g["binary_gamma"]))
    assert np.array_equal(oracle.sw_cfg(g["f_c"], g["f_u"], gb), np.array(g["binary_f_hat"]))


def test_equal_scales_are_global_cfg_as_library_lerp():
    f_c, f_u, s = _rand(1)
    for g in (0.0, 1.0, 4.5, 7.0):
        got = oracle.sw_cfg(f_c, f_u, oracle.guidance_scales(s, g, g))
        ref = torch.lerp(torch.from_numpy(f_u), torch.from_numpy(f_c), g).numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_scale_one_and_zero_select_the_predictions():
    f_c, f_u, _ = _rand(2)
    B, N, _ = f_c.shape
    # f_u + 1 * (f_c - f_u) equals f_c up to the rounding of the difference (a swap would be off by O(1))
    np.testing.assert_allclose(oracle.sw_cfg(f_c, f_u, np.ones((B, N))), f_c, rtol=0, atol=1e-14)
    assert np.array_equal(oracle.sw_cfg(f_c, f_u, np.zeros((B, N))), f_u)


def test_binary_variant_is_the_continuous_one_with_an_indicator_score():
    f_c, f_u, _ = _rand(3)
    B, N, _ = f_c.shape
    rng = np.random.default_rng(4)
    idx = np.stack([np.sort(rng.choice(N, 9, replace=False)) for _ in range(B)])
    ind = np.zeros((B, N))
    for b in range(B):
        ind[b, idx[b]] = 1.0
    gb = oracle.binary_scales(idx, B, N, 3.0, 8.0)
    assert np.array_equal(gb, oracle.guidance_scales(ind, 3.0, 8.0))
    assert np.array_equal(oracle.binary_scales(idx[0], B, N, 3.0, 8.0)[1], gb[0])   # a shared list
    np.testing.assert_allclose(oracle.sw_cfg(f_c, f_u, gb), oracle.sw_cfg(f_c, f_u, oracle.guidance_scales(ind, 3.0, 8.0)))


def test_affine_in_the_scale():
    # f_hat(gamma) is affine in gamma: the midpoint of two scales gives the midpoint prediction
    f_c, f_u, s = _rand(5)
    a = oracle.sw_cfg(f_c, f_u, oracle.guidance_scales(s, 1.0, 5.0))
    b = oracle.sw_cfg(f_c, f_u, oracle.guidance_scales(s, 3.0, 9.0))
    m = oracle.sw_cfg(f_c, f_u, oracle.guidance_scales(s, 2.0, 7.0))
    np.testing.assert_allclose(m, 0.5 * (a + b), rtol=1e-12, atol=1e-12)
