"""GPU parity of safe_sw_cfg against the fp64 oracle (Eq. 20, 21)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


def _inputs(B, N, C, seed, dtype):
    rng = np.random.default_rng(seed)
    f_c = rng.standard_normal((B, N, C)).astype(np.float32)
    f_u = rng.standard_normal((B, N, C)).astype(np.float32)
    if dtype == torch.bfloat16:
        f_c, f_u = W.bf16_from_f32(f_c).value, W.bf16_from_f32(f_u).value
    return f_c, f_u, torch.from_numpy(f_c).to(dev()).to(dtype), torch.from_numpy(f_u).to(dev()).to(dtype)


U32 = 2.0 ** -24   # unit roundoff of fp32 (round to nearest even)


def _check(got, ref, dtype, f_c=None, f_u=None, gamma=None, g_lo=0.0, g_hi=0.0):
    g = got.float().cpu().numpy().astype(np.float64)
    if dtype == torch.float32:
        # The kernel rounds three times in fp32: gamma = g_ctx + (g_sens - g_ctx) s (at most
        # two roundings, 2u (|g_ctx| + |g_sens - g_ctx|), exact for the binary and global
        # forms), d = f_c - f_u (u |d|) and out = fma(gamma, d, f_u) (u |out|).  So
        #   |out - ref| <= u (|ref| + |gamma| |d|) + 2u (|g_lo| + |g_hi - g_lo|) |d|
        # to first order in u; the test allows 1% on top for the second-order terms.
        d = np.abs(f_c.astype(np.float64) - f_u.astype(np.float64))
        gam = np.abs(gamma)[:, :, None]
        bound = U32 * (np.abs(ref) + gam * d + 2.0 * (abs(g_lo) + abs(g_hi - g_lo)) * d) * 1.01 + 1e-30
        assert np.all(np.abs(g - ref) <= bound), float((np.abs(g - ref) / bound).max())
    else:
        # the fp32 result rounded to bf16 once: within one bf16 step of the exact value
        ulp = np.maximum(np.abs(ref), 1e-30) * 2.0 ** -7
        assert np.all(np.abs(g - ref) <= ulp + 1e-6), float((np.abs(g - ref) / ulp).max())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("B,N,C", [(1, 3, 16), (2, 300, 16), (2, 1000, 64), (3, 77, 8)])
def test_score_binary_and_global_forms(dtype, B, N, C):
    if dtype == torch.float32 and C % 4 or dtype == torch.bfloat16 and C % 8:
        pytest.skip("row not a whole number of 16-byte chunks")
    f_c, f_u, dc, du = _inputs(B, N, C, 10 + N + C, dtype)
    rng = np.random.default_rng(N)
    s = rng.random((B, N)).astype(np.float32)
    out = sq.sw_cfg(dc, du, 2.0, 7.5, s=to_dev(s))
    gam = oracle.guidance_scales(s, 2.0, 7.5)
    _check(out, oracle.sw_cfg(f_c, f_u, gam), dtype, f_c, f_u, gam, 2.0, 7.5)
    k = max(1, N // 4)
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)]).astype(np.int32)
    out = sq.sw_cfg(dc, du, 2.0, 7.5, idx=to_dev(idx))
    gam = oracle.binary_scales(idx, B, N, 2.0, 7.5)
    _check(out, oracle.sw_cfg(f_c, f_u, gam), dtype, f_c, f_u, gam)
    out = sq.sw_cfg(dc, du, 4.5)
    gam = np.full((B, N), 4.5)
    _check(out, oracle.sw_cfg(f_c, f_u, gam), dtype, f_c, f_u, gam)
    # shared score row / shared list for every image
    out = sq.sw_cfg(dc, du, 2.0, 7.5, s=to_dev(s[0]))
    gam = oracle.guidance_scales(np.broadcast_to(s[0], (B, N)), 2.0, 7.5)
    _check(out, oracle.sw_cfg(f_c, f_u, gam), dtype, f_c, f_u, gam, 2.0, 7.5)
    out = sq.sw_cfg(dc, du, 2.0, 7.5, idx=to_dev(idx[0]))
    gam = oracle.binary_scales(idx[0], B, N, 2.0, 7.5)
    _check(out, oracle.sw_cfg(f_c, f_u, gam), dtype, f_c, f_u, gam)


def test_in_place_strided_and_out_of_range_indices():
    B, N, C = 2, 129, 16
    f_c, f_u, dc, du = _inputs(B, N, C, 3, torch.float32)
    # a padded layout (token stride 24 > C) shared by all three tensors, output over f_c
    pc = torch.zeros((B, N, 24), device=dev()); pc[..., :C] = dc
    pu = torch.zeros((B, N, 24), device=dev()); pu[..., :C] = du
    idx = np.array([-5, 0, 64, 128, 129, 4000], dtype=np.int32)   # out-of-range entries match nothing
    sq.sw_cfg(pc[..., :C], pu[..., :C], 1.5, 9.0, idx=to_dev(idx), out=pc[..., :C])
    gam = oracle.binary_scales(np.array([0, 64, 128]), B, N, 1.5, 9.0)
    ref = oracle.sw_cfg(f_c, f_u, gam)
    _check(pc[..., :C], ref, torch.float32, f_c, f_u, gam)
    assert torch.all(pc[..., C:] == 0), "padding between rows must stay untouched"


def test_equal_scales_and_limits_bitwise():
    B, N, C = 2, 200, 32
    _, _, dc, du = _inputs(B, N, C, 4, torch.bfloat16)
    s = torch.rand((B, N), device=dev())
    assert torch.equal(sq.sw_cfg(dc, du, 3.0, 3.0, s=s), sq.sw_cfg(dc, du, 3.0)), "equal scales = global guidance"
    assert torch.equal(sq.sw_cfg(dc, du, 0.0), du), "scale 0 gives the unconditional prediction"
