"""Pins of the row-selective block oracle (Eq. 15-16, 18) against things other than itself."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads as W


def _weights(C, Fh, seed):
    w = W.block_weights(C, Fh, seed)
    return {k: (v.value if hasattr(v, "value") else v).astype(np.float64) for k, v in w.items()}


def _torch_block(x, w, H):
    """The stand-in block written with torch's float64 library ops."""
    t = {k: torch.from_numpy(v) for k, v in w.items()}
    x = torch.from_numpy(x)
    B, N, C = x.shape
    d = C // H
    qkv = F.linear(x, t["w_qkv"])
    q, k, v = (qkv[..., i * C:(i + 1) * C].reshape(B, N, H, d).permute(0, 2, 1, 3) for i in range(3))
    a = F.scaled_dot_product_attention(q, k, v).permute(0, 2, 1, 3).reshape(B, N, C)
    y = x + F.linear(a, t["w_o"])
    z = y + F.linear(F.gelu(F.linear(y, t["w1"], t["b1"]), approximate="tanh"), t["w2"], t["b2"])
    return z.numpy(), k.permute(0, 2, 1, 3).numpy(), v.permute(0, 2, 1, 3).numpy()


def test_gelu_and_linear_match_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 13)) * 3
    np.testing.assert_allclose(oracle.gelu_tanh(x), F.gelu(torch.from_numpy(x), approximate="tanh").numpy(),
                               rtol=0, atol=1e-14)
    w, b = rng.standard_normal((5, 13)), rng.standard_normal(5)
    np.testing.assert_allclose(oracle.linear(x, w, b),
                               F.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy(),
                               rtol=0, atol=1e-12)


def test_dense_block_matches_torch_f64():
    B, N, H, d, Fh = 2, 40, 2, 8, 48
    C = H * d
    x = np.random.default_rng(2).standard_normal((B, N, C))
    w = _weights(C, Fh, 3)
    z, k, v = oracle.block_dense(x, w, H)
    zt, kt, vt = _torch_block(x, w, H)
    np.testing.assert_allclose(z, zt, rtol=0, atol=1e-11)
    np.testing.assert_allclose(k, kt, rtol=0, atol=1e-12)
    np.testing.assert_allclose(v, vt, rtol=0, atol=1e-12)


def test_zero_weights_leave_x_plus_b2():
    B, N, H, d, Fh = 1, 9, 2, 4, 16
    C = H * d
    x = np.random.default_rng(4).standard_normal((B, N, C))
    w = _weights(C, Fh, 5)
    for name in ("w_qkv", "w_o", "w1", "w2"):
        w[name] = np.zeros_like(w[name])
    z, _, _ = oracle.block_dense(x, w, H)
    np.testing.assert_allclose(z, x + w["b2"], rtol=0, atol=1e-15)


def test_row_selective_block_equals_dense_on_a_fresh_cache():
    """Cache from a dense pass on the same input: the row-selective block must reproduce the
    dense block for any S (the cached context rows are exactly what the dense pass gives)."""
    B, N, H, d, Fh = 2, 48, 2, 8, 32
    C = H * d
    rng = np.random.default_rng(6)
    x = rng.standard_normal((B, N, C))
    w = _weights(C, Fh, 7)
    z, k, v = oracle.block_dense(x, w, H)
    idx = np.stack([np.sort(rng.choice(N, 13, replace=False)) for _ in range(B)])
    z2, k2, v2 = oracle.block_srsu(x, idx, z, k, v, w, H)
    np.testing.assert_allclose(z2, z, rtol=0, atol=1e-12)
    np.testing.assert_allclose(k2, k, rtol=0, atol=1e-13)


def test_row_selective_block_with_stale_cache():
    """A stale cache (anchor on another input): rows outside S are the cached rows exactly;
    S = all rows is the dense block whatever the cache holds."""
    B, N, H, d, Fh = 2, 32, 2, 8, 32
    C = H * d
    rng = np.random.default_rng(8)
    x_anchor = rng.standard_normal((B, N, C))
    x = x_anchor + 0.05 * rng.standard_normal((B, N, C))
    w = _weights(C, Fh, 9)
    zc, kc, vc = oracle.block_dense(x_anchor, w, H)
    idx = np.stack([np.sort(rng.choice(N, 10, replace=False)) for _ in range(B)])
    z, kg, _ = oracle.block_srsu(x, idx, zc, kc, vc, w, H)
    for b in range(B):
        ctx = np.setdiff1d(np.arange(N), idx[b])
        assert np.array_equal(z[b, ctx], zc[b, ctx]) and np.array_equal(kg[b, ctx], kc[b, ctx])
        assert np.max(np.abs(z[b, idx[b]] - zc[b, idx[b]])) > 1e-3    # the rows of S moved
    z_all, _, _ = oracle.block_srsu(x, np.arange(N), zc, kc, vc, w, H)
    z_dense, _, _ = oracle.block_dense(x, w, H)
    np.testing.assert_allclose(z_all, z_dense, rtol=0, atol=1e-12)
