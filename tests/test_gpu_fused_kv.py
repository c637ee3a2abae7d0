"""GPU parity of the fused global K/V read (Eq. 14 and 16 in one pass): the source map
bit-exact against its definition, attention through the map against the oracle on the
oracle's own assembled K/V, and bitwise against safe_kv_assemble + safe_attn_fwd where
the two calls run the same schedule."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attn_close, assert_lse_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


def _map_expected(idx: np.ndarray, B: int, N: int) -> np.ndarray:
    """src[b, j] = r where idx[b, r] == j (entries outside [0, N) skipped), else -1."""
    idx2 = np.broadcast_to(idx, (B, idx.shape[-1]))
    out = np.full((B, N), -1, np.int32)
    for b in range(B):
        for r, j in enumerate(idx2[b]):
            if 0 <= j < N:
                out[b, j] = r
    return out


@pytest.mark.parametrize("B,N,nsel,shared", [(1, 256, 0, True), (2, 1000, 300, False), (2, 4096, 4096, True),
                                             (2, 4097, 1229, False), (3, 300, 1, False)])
def test_source_map_bit_exact(B, N, nsel, shared):
    rng = np.random.default_rng(N + nsel)
    idx = W.random_rows(rng, N, nsel) if shared else np.stack([W.random_rows(rng, N, nsel) for _ in range(B)])
    got = sq.kv_source_map(to_dev(idx), N, batch=B, check=True).cpu().numpy()
    assert np.array_equal(got, _map_expected(idx, B, N))


def test_source_map_range_and_order_checks():
    idx = np.array([5, 40, 300], dtype=np.int32)
    with pytest.raises(sq.SafeError) as e:
        sq.kv_source_map(to_dev(idx), 300, check=True)
    assert e.value.status == -4
    with pytest.raises(sq.SafeError):
        sq.kv_source_map(to_dev(np.array([5, 5, 9], np.int32)), 300, check=True)
    got = sq.kv_source_map(to_dev(idx), 300).cpu().numpy()    # unchecked: 300 is skipped
    assert np.array_equal(got, _map_expected(idx, 1, 300))


def _case(B, N, H, d, nsel, seed, shared=False):
    rng = np.random.default_rng(seed)
    q, ck, cv = W.attention_inputs(B, N, N, H, d, seed=seed)
    fk, fv, _ = W.attention_inputs(B, nsel, nsel, H, d, seed=seed + 1)
    S = W.random_rows(rng, N, nsel) if shared else np.stack([W.random_rows(rng, N, nsel) for _ in range(B)])
    return rng, q, ck, cv, fk, fv, S


def _oracle_global(fk, fv, S, ck, cv):
    return oracle.kv_assemble(fk.value, S, ck.value), oracle.kv_assemble(fv.value, S, cv.value)


def _plans_match(qd, kd, rows, kv_src, ws):
    wb = 0 if ws is None else None
    return sq.attn_plan(qd, kd, q_rows=rows, workspace_bytes=wb) == \
        sq.attn_plan(qd, kd, q_rows=rows, workspace_bytes=wb, kv_src=kv_src)


@pytest.mark.parametrize("d", [32, 64, 72, 96, 128])
@pytest.mark.parametrize("gather", [False, True])
def test_fused_matches_assembled_and_oracle(d, gather):
    """Ragged N (not a multiple of 64), per-sample S, split and unsplit schedules."""
    B, N, H = 2, 1000, 3
    nsel = 301
    rng, q, ck, cv, fk, fv, S = _case(B, N, H, d, nsel, seed=70 + d + gather)
    qd, ckd, cvd, fkd, fvd = (to_dev_bf16(t) for t in (q, ck, cv, fk, fv))
    Sd = to_dev(S)
    src = sq.kv_source_map(Sd, N, check=True)
    ko, vo = sq.kv_assemble(fkd, fvd, Sd, ckd, cvd)
    rows = Sd if gather else None
    kg, vg = _oracle_global(fk, fv, S, ck, cv)
    for ws in ("auto", None):
        o_a, l_a = sq.attn_fwd(qd, ko, vo, q_rows=rows, workspace=ws, return_lse=True)
        o_f, l_f = sq.attn_fwd(qd, ckd, cvd, q_rows=rows, workspace=ws, return_lse=True, kv_src=src,
                               k_fresh=fkd, v_fresh=fvd)
        if _plans_match(qd, ckd, rows, src, ws):
            assert torch.equal(o_f.view(torch.int16), o_a.view(torch.int16)), (d, gather, ws)
            assert torch.equal(l_f, l_a), (d, gather, ws)
        # oracle on sampled outputs of every (b, h): first/last rows and a random sample
        n_out = nsel if gather else N
        samp = np.unique(np.concatenate([[0, n_out - 1], rng.choice(n_out, 20, replace=False)]))
        qrows = S[:, samp] if gather else samp
        ref, ref_lse = oracle.sdpa(q.value, kg, vg, q_rows=qrows)
        sel = torch.from_numpy(samp).long()
        assert_attn_close(o_f[:, sel], ref, f"fused d={d} gather={gather} ws={ws}")
        assert_lse_close(l_f.cpu()[:, :, sel], ref_lse, f"fused lse d={d} gather={gather} ws={ws}")


@pytest.mark.parametrize("d", [72, 96])
@pytest.mark.parametrize("gather", [False, True])
def test_fused_two_row_blocks(d, gather):
    """Shapes large enough for 256-row tiles (two row blocks per wave, the copy plan in LDS):
    ragged N, per-sample S, a split tail; bitwise against the two-pass path, the oracle on
    sampled rows."""
    B, N, H = 2, 16040, 8
    nsel = 8017
    rng, q, ck, cv, fk, fv, S = _case(B, N, H, d, nsel, seed=170 + d + gather)
    qd, ckd, cvd, fkd, fvd = (to_dev_bf16(t) for t in (q, ck, cv, fk, fv))
    Sd = to_dev(S)
    src = sq.kv_source_map(Sd, N, check=True)
    rows = Sd if gather else None
    plan = sq.attn_plan(qd, ckd, q_rows=rows, kv_src=src)
    assert plan["rows_per_tile"] == 256, plan
    o_f, l_f = sq.attn_fwd(qd, ckd, cvd, q_rows=rows, return_lse=True, kv_src=src, k_fresh=fkd, v_fresh=fvd)
    ko, vo = sq.kv_assemble(fkd, fvd, Sd, ckd, cvd)
    o_a, l_a = sq.attn_fwd(qd, ko, vo, q_rows=rows, return_lse=True)
    assert _plans_match(qd, ckd, rows, src, "auto")
    assert torch.equal(o_f.view(torch.int16), o_a.view(torch.int16)), (d, gather)
    assert torch.equal(l_f, l_a), (d, gather)
    kg, vg = _oracle_global(fk, fv, S, ck, cv)
    n_out = nsel if gather else N
    samp = np.unique(np.concatenate([[0, n_out - 1], rng.choice(n_out, 20, replace=False)]))
    ref, ref_lse = oracle.sdpa(q.value, kg, vg, q_rows=S[:, samp] if gather else samp)
    sel = torch.from_numpy(samp).long()
    assert_attn_close(o_f[:, sel], ref, f"fused two row blocks d={d} gather={gather}")
    assert_lse_close(l_f.cpu()[:, :, sel], ref_lse, f"fused two row blocks lse d={d} gather={gather}")


@pytest.mark.parametrize("N", [40, 64, 100, 150, 192, 250])
def test_fused_few_key_tiles(N):
    """One to four 64-key tiles (full and partial): the source-address tables of the first
    tiles are built before the loop, later ones inside it; bitwise against the two passes,
    the oracle on sampled rows."""
    B, H, d = 2, 3, 96
    nsel = max(1, N // 3)
    rng, q, ck, cv, fk, fv, S = _case(B, N, H, d, nsel, seed=190 + N)
    qd, ckd, cvd, fkd, fvd = (to_dev_bf16(t) for t in (q, ck, cv, fk, fv))
    Sd = to_dev(S)
    src = sq.kv_source_map(Sd, N, check=True)
    ko, vo = sq.kv_assemble(fkd, fvd, Sd, ckd, cvd)
    o_a = sq.attn_fwd(qd, ko, vo, workspace=None)
    o_f = sq.attn_fwd(qd, ckd, cvd, workspace=None, kv_src=src, k_fresh=fkd, v_fresh=fvd)
    assert torch.equal(o_f.view(torch.int16), o_a.view(torch.int16)), N
    kg, vg = _oracle_global(fk, fv, S, ck, cv)
    samp = np.unique(np.array([0, N // 2, N - 1]))
    ref, _ = oracle.sdpa(q.value, kg, vg, q_rows=samp)
    assert_attn_close(o_f[:, torch.from_numpy(samp).long()], ref, f"fused N={N}")


def test_fused_edge_sets_and_shared_map():
    """S empty (all keys from the cache), S = every token (all keys fresh), one map shared
    by the batch."""
    B, N, H, d = 2, 640, 2, 96
    q, ck, cv = W.attention_inputs(B, N, N, H, d, seed=81)
    qd, ckd, cvd = to_dev_bf16(q), to_dev_bf16(ck), to_dev_bf16(cv)
    samp = np.array([0, 1, 127, 128, 383, 639])
    sel = torch.from_numpy(samp).long()
    # S empty: the map is all -1 and the fresh tensors have no rows
    empty = torch.empty((B, 0, H, d), dtype=torch.bfloat16, device=qd.device)
    src = sq.kv_source_map(to_dev(np.zeros((0,), np.int32)), N, batch=B)
    assert bool((src == -1).all())
    o = sq.attn_fwd(qd, ckd, cvd, kv_src=src, k_fresh=empty, v_fresh=empty)
    ref, _ = oracle.sdpa(q.value, ck.value, cv.value, q_rows=samp)
    assert_attn_close(o[:, sel], ref, "S empty")
    # S = every token: K/V are the fresh tensors (Eq. 19 refresh)
    fk, fv, _ = W.attention_inputs(B, N, N, H, d, seed=82)
    src = sq.kv_source_map(to_dev(np.arange(N, dtype=np.int32)), N, batch=B)
    o = sq.attn_fwd(qd, ckd, cvd, kv_src=src, k_fresh=to_dev_bf16(fk), v_fresh=to_dev_bf16(fv))
    ref, _ = oracle.sdpa(q.value, fk.value, fv.value, q_rows=samp)
    assert_attn_close(o[:, sel], ref, "S all")
    # a [Nk] map shared by the batch equals the [B, Nk] one
    rng = np.random.default_rng(83)
    S = W.random_rows(rng, N, 200)
    fk, fv, _ = W.attention_inputs(B, 200, 200, H, d, seed=84)
    src1 = sq.kv_source_map(to_dev(S), N)[0]
    srcB = sq.kv_source_map(to_dev(S), N, batch=B)
    args = dict(k_fresh=to_dev_bf16(fk), v_fresh=to_dev_bf16(fv), q_rows=to_dev(S))
    o1 = sq.attn_fwd(qd, ckd, cvd, kv_src=src1, **args)
    oB = sq.attn_fwd(qd, ckd, cvd, kv_src=srcB, **args)
    assert torch.equal(o1.view(torch.int16), oB.view(torch.int16))
    kg, vg = _oracle_global(fk, fv, S, ck, cv)
    ref, _ = oracle.sdpa(q.value, kg, vg, q_rows=S[[0, 57, 199]])
    assert_attn_close(o1[:, torch.tensor([0, 57, 199])], ref, "shared map")


def test_fused_rejects_key_lengths_and_masks():
    B, N, H, d = 1, 128, 1, 64
    q, ck, cv = W.attention_inputs(B, N, N, H, d, seed=85)
    qd, ckd, cvd = to_dev_bf16(q), to_dev_bf16(ck), to_dev_bf16(cv)
    src = sq.kv_source_map(to_dev(np.array([3], np.int32)), N)
    f = qd[:, :1].contiguous()
    for kw in ({"kv_len": torch.tensor([64], dtype=torch.int32, device=qd.device)},
               {"mask": torch.ones((1, 1, 1, N), dtype=torch.bool, device=qd.device)}):
        with pytest.raises(sq.SafeError) as e:
            sq.attn_fwd(qd, ckd, cvd, kv_src=src, k_fresh=f, v_fresh=f, **kw)
        assert e.value.status == -5


@pytest.mark.parametrize("number", [4])
def test_full_size_srsu_step_sampled_rows(number):
    """The 160x160-grid workload (25600 tokens), SRSU self-attention at rho 25%, fused: bitwise
    against the two-pass path where the schedules agree, the oracle on sampled rows."""
    inp = W.workload_inputs(number)
    w = inp["workload"]
    rng = W.rng_for(number, stream=9)
    S = W.random_rows(rng, w.N, w.k_for(25))
    k_t = inp["k_x"].value + W.drift((1003, 10, 0), inp["k_x"].value.shape)
    v_t = inp["v_x"].value + W.drift((1003, 11, 0), inp["v_x"].value.shape)
    kb, vb = W.bf16_from_f32(k_t), W.bf16_from_f32(v_t)
    fk = W.Bf16Tensor(kb.bits[:, S], kb.value[:, S])
    fv = W.Bf16Tensor(vb.bits[:, S], vb.value[:, S])
    qd, ckd, cvd = to_dev_bf16(inp["q_x"]), to_dev_bf16(inp["k_x"]), to_dev_bf16(inp["v_x"])
    fkd, fvd, Sd = to_dev_bf16(fk), to_dev_bf16(fv), to_dev(S)
    src = sq.kv_source_map(Sd, w.N, check=True)
    o_f = sq.attn_fwd(qd, ckd, cvd, q_rows=Sd, kv_src=src, k_fresh=fkd, v_fresh=fvd)
    ko, vo = sq.kv_assemble(fkd, fvd, Sd, ckd, cvd)
    o_a = sq.attn_fwd(qd, ko, vo, q_rows=Sd)
    if _plans_match(qd, ckd, Sd, src, "auto"):
        assert torch.equal(o_f.view(torch.int16), o_a.view(torch.int16))
    samp = np.unique(np.concatenate([[0, len(S) - 1], rng.choice(len(S), 24, replace=False)]))
    kg = oracle.kv_assemble(fk.value, S, inp["k_x"].value)
    vg = oracle.kv_assemble(fv.value, S, inp["v_x"].value)
    ref, _ = oracle.sdpa(inp["q_x"].value, kg, vg, q_rows=S[samp])
    assert_attn_close(o_f[:, torch.from_numpy(samp).long()], ref, "fused full size")


def test_fused_step_in_a_hip_graph():
    """Source map + fused SRSU attention captured in a HIP graph: every replay, with eager
    work in between and the map buffer cleared, gives the eager result bitwise."""
    B, N, H, d, n_sel = 2, 3000, 4, 96, 777
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=86)
    qd, kc, vc = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rows = to_dev(np.stack([W.random_rows(np.random.default_rng(87 + b), N, n_sel) for b in range(B)]))
    g = torch.Generator(device="cuda").manual_seed(88)
    kf = torch.randn((B, n_sel, H, d), generator=g, device="cuda").to(torch.bfloat16)
    vf = torch.randn((B, n_sel, H, d), generator=g, device="cuda").to(torch.bfloat16)
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    o = torch.empty((B, n_sel, H, d), dtype=torch.bfloat16, device="cuda")

    def step():
        sq.kv_source_map(rows, N, out=src)
        sq.attn_fwd(qd, kc, vc, q_rows=rows, out=o, kv_src=src, k_fresh=kf, v_fresh=vf)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up on the capture stream (its workspace)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = o.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for rep in range(3):
        o.zero_()
        src.fill_(-1)
        eager = sq.attn_fwd(qd, kc, vc, q_rows=rows)      # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"replay {rep}"
        assert eager.shape == o.shape


@pytest.mark.parametrize("d", [64, 128])
def test_fused_strided_fresh_and_cache(d):
    """Fresh rows and the cache as views with padded rows (token stride > H·d, head stride > d),
    three samples with their own S and a ragged key count: the oracle on sampled rows."""
    B, N, H, nsel = 3, 777, 2, 200
    rng, q, ck, cv, fk, fv, S = _case(B, N, H, d, nsel, seed=90 + d)
    qd = to_dev_bf16(q)

    def padded(t, rows):
        big = torch.zeros((B, rows, H, d + 32), dtype=torch.bfloat16, device="cuda")
        big[..., :d] = to_dev_bf16(t)
        return big[..., :d]

    ckd, cvd, fkd, fvd = padded(ck, N), padded(cv, N), padded(fk, nsel), padded(fv, nsel)
    assert fkd.stride(1) == H * (d + 32) and not fkd.is_contiguous()
    src = sq.kv_source_map(to_dev(S), N, check=True)
    o = sq.attn_fwd(qd, ckd, cvd, q_rows=to_dev(S), kv_src=src, k_fresh=fkd, v_fresh=fvd)
    kg, vg = _oracle_global(fk, fv, S, ck, cv)
    samp = np.unique(np.concatenate([[0, nsel - 1], rng.choice(nsel, 16, replace=False)]))
    ref, _ = oracle.sdpa(q.value, kg, vg, q_rows=S[:, samp])
    assert_attn_close(o[:, torch.from_numpy(samp).long()], ref, f"strided d={d}")
