"""GPU parity of the block around attention (Eq. 15-16, 18) -- safe_linear, safe_kv_assemble
and safe_attn_fwd in sequence -- against the fp64 oracle of the stand-in block."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")

# The GPU path stores qkv, the attention output, y and the MLP hidden state in bf16 (four
# roundings of at most 2^-9 relative each) on top of the attention bound (max 1e-2, mean
# 1e-3 on unit-scale values) and the fp32 accumulation of the maps.  With unit-variance
# x and N(0, 1/fan_in) weights, |z| stays within a few units, so the compounded error is
# bounded by a few bf16 steps of the largest intermediate: max-abs 2^-4 * (1 + |z|) and
# mean-abs 2^-8 * mean(1 + |z|).
def assert_block_close(got, ref, what):
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), what
    scale = 1.0 + np.abs(ref)
    ratio = float((err / (2.0 ** -4 * scale)).max())
    mean = float(err.mean())
    print(f"{what}: max-abs {err.max():.3e} ratio {ratio:.3f} mean-abs {mean:.3e}")
    assert ratio <= 1.0, f"{what}: max-abs {err.max():.3e} beyond 2^-4 (1 + |z|)"
    assert mean <= 2.0 ** -8 * scale.mean(), f"{what}: mean-abs {mean:.3e}"


def _setup(B, N, H, d, F, seed):
    C = H * d
    x = W.bf16_normal((seed, 0), (B, N, C))
    wts = W.block_weights(C, F, seed + 1)
    w64 = {kk: (v.value if hasattr(v, "value") else v).astype(np.float64) for kk, v in wts.items()}
    wd = {kk: (to_dev_bf16(v) if hasattr(v, "value") else to_dev(v)) for kk, v in wts.items()}
    return x, w64, wd


@pytest.mark.parametrize("shape", [(2, 300, 2, 32, 256, 77), (2, 1000, 4, 96, 1536, 250), (1, 700, 8, 72, 2304, 200)])
def test_dense_and_row_selective_block(shape):
    B, N, H, d, F, k = shape
    C = H * d
    x, w64, wd = _setup(B, N, H, d, F, 60 + d)
    xd = to_dev_bf16(x)
    # anchor step: the dense block (Eq. 18) and its key/value cache
    z, qkv = sq.block_dense(xd, wd, H)
    z_ref, k_ref, v_ref = oracle.block_dense(x.value, w64, H)
    assert_block_close(z, z_ref, f"dense z {shape}")
    assert_block_close(qkv[..., C:2 * C].reshape(B, N, H, d), k_ref, "dense k")
    # a later step on a drifted state: only the rows of S are recomputed (Eq. 15-16)
    x2 = W.bf16_from_f32((x.value + W.drift((60 + d, 9), x.value.shape)).astype(np.float32))
    rng = np.random.default_rng(d)
    idx = np.stack([W.random_rows(rng, N, k) for _ in range(B)])
    z_s = sq.block_srsu(to_dev_bf16(x2), to_dev(idx), z.clone(), qkv.clone(), wd, H)
    z2_ref, _, _ = oracle.block_srsu(x2.value, idx, z_ref, k_ref, v_ref, w64, H)
    assert_block_close(z_s, z2_ref, f"srsu z {shape}")
    for b in range(B):
        ctx = np.setdiff1d(np.arange(N), idx[b])
        assert torch.equal(z_s[b, torch.from_numpy(ctx).cuda()], z[b, torch.from_numpy(ctx).cuda()]), \
            "context rows are the cached rows"


def test_row_selective_equals_dense_on_its_own_anchor():
    """On the anchor's own state the row-selective block reproduces the dense block's rows of S
    (same maps, other row tiling: within the rounding of one bf16 step of the outputs)."""
    B, N, H, d, F, k = 2, 640, 4, 64, 1024, 200
    x, _, wd = _setup(B, N, H, d, F, 70)
    xd = to_dev_bf16(x)
    z, qkv = sq.block_dense(xd, wd, H)
    idx = np.stack([W.random_rows(np.random.default_rng(b), N, k) for b in range(B)])
    z_s = sq.block_srsu(xd, to_dev(idx), z.clone(), qkv.clone(), wd, H)
    diff = (z_s.float() - z.float()).abs()
    assert diff.max().item() <= 2.0 ** -6 * (1 + z.float().abs().max().item())


def test_dense_block_stage_by_stage():
    """The same block, one intermediate at a time: each stage is compared with the oracle
    applied to the GPU's own input to that stage, so every stage carries its own derived
    bound instead of the compounded one -- the row-wise maps the linear bound (one bf16
    rounding of the result plus the fp32 accumulation bound, the GELU slope, the residual
    add), the attention the attention bound (max-abs, mean-abs, relative L2) -- and the
    stages reproduce block_dense bit for bit."""
    from gpu_util import assert_attn_close
    from test_gpu_linear import bound, check
    B, N, H, d, F = 2, 1000, 4, 96, 1536
    C = H * d
    x, w64, wd = _setup(B, N, H, d, F, 80)
    xd = to_dev_bf16(x)
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    qkv = sq.linear(xd, wd["w_qkv"])
    ref = oracle.linear(x.value, w64["w_qkv"])
    check(qkv, ref, bound(x.value, w64["w_qkv"], ref, C), "qkv projection")
    q, k, v = (qkv[..., i * C:(i + 1) * C].unflatten(-1, (H, d)) for i in range(3))
    a = sq.attn_fwd(q, k, v)
    ref_a, _ = oracle.sdpa(f64(q), f64(k), f64(v))
    assert_attn_close(a, ref_a, "attention on the projected q, k, v")
    a2 = a.view(B, N, C)
    y = sq.linear(a2, wd["w_o"], res=xd)
    ref = oracle.linear(f64(a2), w64["w_o"]) + x.value
    check(y, ref, bound(f64(a2), w64["w_o"], ref, C, res=x.value), "output projection + residual")
    u = sq.linear(y, wd["w1"], bias=wd["b1"], gelu=True)
    ref = oracle.gelu_tanh(oracle.linear(f64(y), w64["w1"], w64["b1"]))
    check(u, ref, bound(f64(y), w64["w1"], ref, C, gelu=True), "MLP up + GELU")
    z = sq.linear(u, wd["w2"], bias=wd["b2"], res=y)
    ref = oracle.linear(f64(u), w64["w2"], w64["b2"]) + f64(y)
    check(z, ref, bound(f64(u), w64["w2"], ref, F, res=f64(y)), "MLP down + residual")
    z_blk, qkv_blk = sq.block_dense(xd, wd, H)
    assert torch.equal(z_blk, z) and torch.equal(qkv_blk, qkv), "the block is this sequence of calls"
