"""GPU parity of safe_linear (the row-wise maps of the block around attention, Eq. 15)
against the fp64 oracle: plain, gathered input rows, GELU, gathered residual, scattered
output rows, ragged tiles, a stage count that is odd and even, invalid indices."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


def bound(a_rows_f64, w_f64, ref, K, gelu=False, res=None):
    """Elementwise error bound: one bf16 rounding of the result (2^-8 relative, a full
    step) plus the fp32 accumulation bound K * 2^-24 * sum_k |a_k w_k| (tanh-GELU's slope is
    below 1.13 and its own error ~1e-6 relative), plus the residual add's rounding."""
    acc = K * 2.0 ** -24 * (np.abs(a_rows_f64) @ np.abs(w_f64).T)
    if gelu:
        acc = 1.13 * acc + 1e-6 * np.abs(ref)
    if res is not None:
        acc = acc + 2.0 ** -24 * np.abs(res)
    return 2.0 ** -8 * np.abs(ref) + acc + 1e-30


def check(got, ref, bnd, what):
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), what
    worst = float((err / bnd).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error {float(err.max()):.3e} exceeds the bound (ratio {worst:.2f})"


def inputs(B, T, N, K, seed):
    a = W.bf16_normal((seed, 0), (B, T, K))
    w = W.bf16_normal((seed, 1), (N, K), std=1.0 / np.sqrt(K))
    bias = W.normal_f32((seed, 2), (N,), std=0.1)
    res = W.bf16_normal((seed, 3), (B, T, N))
    return a, w, bias, res


@pytest.mark.parametrize("K", [64, 128, 192, 320])
def test_plain_ragged_tiles(K):
    B, M, N = 2, 300, 200
    a, w, bias, _ = inputs(B, M, N, K, 10 + K)
    out = sq.linear(to_dev_bf16(a), to_dev_bf16(w), bias=to_dev(bias))
    ref = oracle.linear(a.value, w.value, bias)
    check(out, ref, bound(a.value, w.value, ref, K), f"plain K={K}")


def test_gather_gelu_residual_scatter():
    B, T, N, K, M = 2, 500, 264, 256, 137
    a, w, bias, res = inputs(B, T, N, K, 20)
    rng = np.random.default_rng(20)
    rows = np.stack([W.random_rows(rng, T, M) for _ in range(B)])
    ad, wd = to_dev_bf16(a), to_dev_bf16(w)
    # gathered A rows, compact output, GELU
    y = sq.linear(ad, wd, bias=to_dev(bias), gelu=True, a_rows=to_dev(rows))
    a_s = np.stack([a.value[b, rows[b]] for b in range(B)])
    ref = oracle.gelu_tanh(oracle.linear(a_s, w.value, bias))
    check(y, ref, bound(a_s, w.value, ref, K, gelu=True), "gather+gelu")
    # gathered residual and scattered output into a tensor holding other rows
    out = torch.full((B, T, N), 2.5, dtype=torch.bfloat16, device="cuda:0")
    resd = to_dev_bf16(res)
    sq.linear(ad, wd, res=resd, out=out, a_rows=to_dev(rows), res_rows=to_dev(rows), out_rows=to_dev(rows))
    r_s = np.stack([res.value[b, rows[b]] for b in range(B)])
    ref = oracle.linear(a_s, w.value) + r_s
    g = out.float().cpu().numpy()
    for b in range(B):
        check(out[b][torch.from_numpy(rows[b]).long()].unsqueeze(0), ref[b:b + 1],
              bound(a_s[b:b + 1], w.value, ref[b:b + 1], K, res=r_s[b:b + 1]), "scatter")
        other = np.ones(T, bool)
        other[rows[b]] = False
        assert np.all(g[b][other] == 2.5), "rows outside the list keep their contents"
    # one list shared by both samples
    shared = rows[0]
    y = sq.linear(ad, wd, a_rows=to_dev(shared))
    ref = oracle.linear(a.value[:, shared], w.value)
    check(y, ref, bound(a.value[:, shared], w.value, ref, K), "shared list")


def test_invalid_indices_and_check():
    B, T, N, K = 1, 100, 64, 64
    a, w, bias, res = inputs(B, T, N, K, 30)
    ad, wd, resd = to_dev_bf16(a), to_dev_bf16(w), to_dev_bf16(res)
    rows = np.array([[5, -1, 99, 100]], dtype=np.int32)
    with pytest.raises(sq.SafeError) as e:
        sq.linear(ad, wd, a_rows=to_dev(rows), check=True)
    assert e.value.status == -4
    y = sq.linear(ad, wd, a_rows=to_dev(rows))          # invalid A rows read row 0
    src = np.array([5, 0, 99, 0])
    ref = oracle.linear(a.value[:, src], w.value)
    check(y, ref, bound(a.value[:, src], w.value, ref, K), "invalid a rows")
    out = torch.full((B, T, N), -1.0, dtype=torch.bfloat16, device="cuda:0")
    sq.linear(ad, wd, res=resd, out=out, res_rows=to_dev(rows), out_rows=to_dev(rows))
    g = out.float().cpu().numpy()
    ref = oracle.linear(a.value[:, :4], w.value)
    ref[0, 0] += res.value[0, 5]
    ref[0, 2] += res.value[0, 99]                       # invalid residual rows add nothing
    check(out[:, [5, 99]], ref[:, [0, 2]], bound(a.value[:, [0, 2]], w.value, ref[:, [0, 2]], K, res=1.0), "rows")
    untouched = np.ones(T, bool)
    untouched[[5, 99]] = False
    assert np.all(g[0][untouched] == -1.0), "invalid scatter rows are not written"


def test_block_shapes_sampled_rows():
    """The 2560sq block's QKV projection shape on gathered rows (B=2, k=6400 of 25600,
    C=2304 -> 3C): oracle on sampled output rows."""
    B, T, C, k = 2, 25600, 2304, 6400
    g = torch.Generator(device="cpu").manual_seed(50)
    a = torch.randn((B, T, C), generator=g).to(torch.bfloat16)
    w = (torch.randn((3 * C, C), generator=g) / np.sqrt(C)).to(torch.bfloat16)
    rows = torch.stack([torch.sort(torch.randperm(T, generator=g)[:k])[0] for _ in range(B)]).to(torch.int32)
    y = sq.linear(a.cuda(), w.cuda(), a_rows=rows.cuda())
    rng = np.random.default_rng(50)
    samp = np.unique(np.concatenate([[0, 127, 128, k - 1], rng.choice(k, 40, replace=False)]))
    a64, w64 = a.double().numpy(), w.double().numpy()
    for b in range(B):
        a_s = a64[b, rows[b].numpy()[samp]]
        ref = oracle.linear(a_s, w64)
        check(y[b, torch.from_numpy(samp).cuda()], ref, bound(a_s, w64, ref, C), f"block shape b={b}")


@pytest.mark.parametrize("K,N", [(64, 4104), (128, 4104), (192, 4104), (576, 4104), (128, 6400)])
def test_large_tiles_ragged_edges(K, N):
    """Enough 256 x 256 tiles to take the large-tile kernel (its ring of half-stage buffers:
    one, two, three and nine k stages), with ragged token and feature edges, a gathered
    list, GELU and a residual.  With N = 4104 the 16 x 17 = 272 tiles leave a last round of
    16 (on 256 CUs), which runs as 128 x 128 sub-tiles; with N = 6400 the last round holds
    144 tiles and stays 256 x 256."""
    B, T, M = 1, 4100, 4000
    a, w, bias, res = inputs(B, T, N, K, 40 + K)
    rows = np.sort(np.random.default_rng(40).choice(T, M, replace=False)).astype(np.int32)[None]
    y = sq.linear(to_dev_bf16(a), to_dev_bf16(w), bias=to_dev(bias), gelu=True, res=to_dev_bf16(res),
                  a_rows=to_dev(rows), res_rows=to_dev(rows))
    a_s = a.value[:, rows[0]]
    r_s = res.value[:, rows[0]]
    ref = oracle.gelu_tanh(oracle.linear(a_s, w.value, bias)) + r_s
    check(y, ref, bound(a_s, w.value, ref, K, gelu=True, res=r_s), f"large tiles K={K} N={N}")
