"""GPU parity of safe_attn_fwd against the fp64 oracle (Eq. 2, 16, 17, 18)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attn_close, assert_lse_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


def test_tiny_dense_all_rows():
    inp = W.workload_inputs(1)
    q, k, v = (to_dev_bf16(inp[n]) for n in ("q_x", "k_x", "v_x"))
    o, lse = sq.attn_fwd(q, k, v, return_lse=True)
    ref, ref_lse = oracle.sdpa(inp["q_x"].value, inp["k_x"].value, inp["v_x"].value)
    assert_attn_close(o, ref, "tiny dense")
    assert_lse_close(lse, ref_lse, "tiny dense")


def test_tiny_srsu_self_and_cross():
    inp = W.workload_inputs(1)
    w = inp["workload"]
    rows = W.random_rows(W.rng_for(1, stream=2), w.N, w.k_for(25))
    rows_t = to_dev(rows)
    q, k, v = (to_dev_bf16(inp[n]) for n in ("q_x", "k_x", "v_x"))
    o, lse = sq.attn_fwd(q, k, v, q_rows=rows_t, return_lse=True)
    ref, ref_lse = oracle.sdpa(inp["q_x"].value, inp["k_x"].value, inp["v_x"].value, q_rows=rows)
    assert_attn_close(o, ref, "tiny srsu")
    assert_lse_close(lse, ref_lse, "tiny srsu")
    qc, kt, vt = (to_dev_bf16(inp[n]) for n in ("q_c", "k_txt", "v_txt"))
    kv = to_dev(inp["kv_len"])
    o = sq.attn_fwd(qc, kt, vt, q_rows=rows_t, kv_len=kv)
    ref, _ = oracle.sdpa(inp["q_c"].value, inp["k_txt"].value, inp["v_txt"].value, q_rows=rows, kv_len=inp["kv_len"])
    assert_attn_close(o, ref, "tiny cross")


@pytest.mark.parametrize("d", [32, 64, 72, 96, 128])
def test_ragged_shapes_rows_lengths(d):
    B, Nq, Nk, H = 4, 301, 333, 3
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=100 + d)
    rng = np.random.default_rng(d)
    rows = np.stack([W.random_rows(rng, Nq, 77) for _ in range(B)])
    kv = np.array([0, 1, 333, 65], dtype=np.int32)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    # dense, no lengths (tails in both rows and keys)
    o, lse = sq.attn_fwd(qd, kd, vd, return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value)
    assert_attn_close(o, ref, f"dense d={d}")
    assert_lse_close(lse, ref_lse, f"dense d={d}")
    # gathered per-sample rows with per-sample lengths (including 0 and 1)
    o, lse = sq.attn_fwd(qd, kd, vd, q_rows=to_dev(rows), kv_len=to_dev(kv), return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, q_rows=rows, kv_len=kv)
    assert_attn_close(o, ref, f"rows+len d={d}")
    assert_lse_close(lse, ref_lse, f"rows+len d={d}")
    assert torch.all(o[0] == 0), "kv_len 0 must give zero output"
    # scattered output lands at the query tokens, other tokens untouched
    out = torch.full((B, Nq, H, d), 7.0, dtype=torch.bfloat16, device=qd.device)
    sq.attn_fwd(qd, kd, vd, q_rows=to_dev(rows), kv_len=to_dev(kv), out=out, scatter_out=True)
    g = out.float().cpu().numpy()
    for b in range(B):
        assert_attn_close(out[b][torch.from_numpy(rows[b]).long()].unsqueeze(0), ref[b:b + 1], "scatter")
        mask = np.ones(Nq, bool)
        mask[rows[b]] = False
        assert np.all(g[b][mask] == 7.0)


def test_shared_rows_and_dense_equivalence_bitwise():
    """Without tail splitting every row is computed the same way whatever the row set."""
    B, N, H, d = 2, 1000, 4, 96
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=7)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    dense = sq.attn_fwd(qd, kd, vd, workspace=None)
    all_rows = sq.attn_fwd(qd, kd, vd, q_rows=torch.arange(N, dtype=torch.int32, device=qd.device), workspace=None)
    assert torch.equal(dense, all_rows), "S = all rows must reproduce the dense pass"
    rows = W.random_rows(np.random.default_rng(3), N, 250)
    part = sq.attn_fwd(qd, kd, vd, q_rows=to_dev(rows), workspace=None)
    assert torch.equal(part, dense[:, torch.from_numpy(rows).long()])
    assert torch.equal(dense, sq.attn_fwd(qd, kd, vd, workspace=None)), "repeated calls must be bitwise identical"
    split = sq.attn_fwd(qd, kd, vd)   # workspace chosen by the binding: split schedule
    assert torch.equal(split, sq.attn_fwd(qd, kd, vd)), "repeated split calls must be bitwise identical"


def test_tail_split_against_oracle_and_unsplit():
    """Fewer row tiles than resident workgroups: every tile is split along the keys into
    partials (fp32 O, max, sum) that the merge kernel combines."""
    B, Nq, Nk, H, d = 2, 300, 3000, 3, 96
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=21)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    need = sq.attn_workspace_bytes(qd, kd)
    assert need > 0, "this shape must be split"
    o, lse = sq.attn_fwd(qd, kd, vd, return_lse=True)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value)
    assert_attn_close(o, ref, "split dense")
    assert_lse_close(lse, ref_lse, "split dense")
    plain, plain_lse = sq.attn_fwd(qd, kd, vd, return_lse=True, workspace=None)
    assert (o.float() - plain.float()).abs().max().item() <= 2e-2
    # a workspace one byte short runs unsplit
    short = torch.empty(need - 1, dtype=torch.uint8, device=qd.device)
    assert torch.equal(sq.attn_fwd(qd, kd, vd, workspace=short), plain)
    exact = torch.empty(need, dtype=torch.uint8, device=qd.device)
    assert torch.equal(sq.attn_fwd(qd, kd, vd, workspace=exact), o)
    # gathered per-sample rows, scattered output and LSE through the merge
    rng = np.random.default_rng(5)
    rows = np.stack([W.random_rows(rng, Nq, 111) for _ in range(B)])
    rows[1, 7] = Nq + 5   # out of range: reads a zero query, not written when scattering
    assert sq.attn_workspace_bytes(qd, kd, q_rows=to_dev(rows)) > 0
    out = torch.full((B, Nq, H, d), 3.0, dtype=torch.bfloat16, device=qd.device)
    _, lse = sq.attn_fwd(qd, kd, vd, q_rows=to_dev(rows), out=out, scatter_out=True, return_lse=True)
    ok_rows = np.where(rows < Nq, rows, 0)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, q_rows=ok_rows)
    g = out.float().cpu().numpy()
    for b in range(B):
        valid = rows[b] < Nq
        got = out[b][torch.from_numpy(rows[b][valid]).long()].unsqueeze(0)
        assert_attn_close(got, ref[b:b + 1, valid], "split scatter")
        assert_lse_close(lse.cpu()[b:b + 1][:, :, torch.from_numpy(valid)], ref_lse[b:b + 1][:, :, valid],
                         "split scatter lse")
        untouched = np.ones(Nq, bool)
        untouched[rows[b][valid]] = False
        assert np.all(g[b][untouched] == 3.0)


def test_invalid_rows_and_lengths():
    B, N, H, d = 1, 200, 2, 64
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=9)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    bad = to_dev(np.array([3, 250, -1, 7], dtype=np.int32))
    with pytest.raises(sq.SafeError) as e:
        sq.attn_fwd(qd, kd, vd, q_rows=bad, check=True)
    assert e.value.status == -4
    o = sq.attn_fwd(qd, kd, vd, q_rows=bad)  # out-of-range entries read a zero query row
    zero_q = np.zeros((1, 1, H, d))
    ref_zero, _ = oracle.sdpa(zero_q, k.value, v.value)
    assert_attn_close(o[:, 1:3], np.concatenate([ref_zero, ref_zero], axis=1), "zero-query rows")
    with pytest.raises(sq.SafeError):
        sq.attn_fwd(qd, kd, vd, kv_len=to_dev(np.array([201], np.int32)), check=True)
    o = sq.attn_fwd(qd, kd, vd, kv_len=to_dev(np.array([5000], np.int32)))   # clamped to Nk
    assert torch.equal(o, sq.attn_fwd(qd, kd, vd, kv_len=to_dev(np.array([N], np.int32))))
    assert (o.float() - sq.attn_fwd(qd, kd, vd).float()).abs().max().item() <= 1e-2
    empty = sq.attn_fwd(qd, kd, vd, q_rows=to_dev(np.zeros((0,), np.int32)))
    assert empty.shape == (1, 0, H, d)


@pytest.mark.parametrize("d", [64, 96])
def test_logits_growing_along_keys_and_a_late_spike(d):
    """Rows whose scores keep growing across key tiles, so the running reference max has
    to move again and again mid-row (and O, l be rescaled), plus rows where one key in a
    middle tile dwarfs everything before it."""
    B, N, H = 1, 700, 2
    rng = np.random.default_rng(40 + d)
    u = rng.standard_normal(d)
    q = u[None, None, None, :] + 0.3 * rng.standard_normal((B, N, H, d))
    alpha = np.linspace(0.0, 5.0, N)[None, :, None, None]          # scores rise by ~5 |u|^2
    k = alpha * u[None, None, None, :] + 0.3 * rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    qb, kb, vb = (W.bf16_from_f32(x.astype(np.float32)) for x in (q, k, v))
    o, lse = sq.attn_fwd(to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb), return_lse=True)
    ref, ref_lse = oracle.sdpa(qb.value, kb.value, vb.value)
    assert_attn_close(o, ref, f"growing d={d}")
    assert_lse_close(lse, ref_lse, f"growing d={d}")
    # flat scores with one spike key at 400 (tile 6 of 11)
    k2 = 0.05 * rng.standard_normal((B, N, H, d))
    k2[:, 400] = 4.0 * u
    k2b = W.bf16_from_f32(k2.astype(np.float32))
    o, lse = sq.attn_fwd(to_dev_bf16(qb), to_dev_bf16(k2b), to_dev_bf16(vb), return_lse=True)
    ref, ref_lse = oracle.sdpa(qb.value, k2b.value, vb.value)
    assert_attn_close(o, ref, f"spike d={d}")
    assert_lse_close(lse, ref_lse, f"spike d={d}")


def _sample_rows(rng, n, per=24):
    """Sampled output rows: the first, the last, rows around the 128- and 256-row tile edges
    (one and two row blocks per wave) and random ones."""
    pick = {0, n - 1, max(0, n - 129), max(0, n - 257)}
    pick.update(min(n - 1, r) for r in (127, 128, 255, 256, 383, 384))
    pick.update(rng.choice(n, size=min(n, per), replace=False).tolist())
    return np.array(sorted(pick))


@pytest.mark.parametrize("number", [2, 3, 4, 5])
def test_full_size_workloads_sampled_rows(number):
    """Full workload shapes in the bench's launch configuration; oracle on sampled output rows."""
    inp = W.workload_inputs(number)
    w = inp["workload"]
    rng = W.rng_for(number, stream=3)
    q, k, v = (to_dev_bf16(inp[n]) for n in ("q_x", "k_x", "v_x"))
    rows = W.random_rows(rng, w.N, w.k_for(w.rho_percent[0]))
    rows_t = to_dev(rows)
    # SRSU self-attention (Eq. 16)
    o = sq.attn_fwd(q, k, v, q_rows=rows_t)
    samp = _sample_rows(rng, rows.shape[0])
    ref, _ = oracle.sdpa(inp["q_x"].value, inp["k_x"].value, inp["v_x"].value, q_rows=rows[samp])
    assert_attn_close(o[:, torch.from_numpy(samp).long()], ref, f"srsu N={w.N}")
    # SRSU cross-attention with per-sample text lengths (Eq. 17)
    qc, kt, vt = (to_dev_bf16(inp[n]) for n in ("q_c", "k_txt", "v_txt"))
    o = sq.attn_fwd(qc, kt, vt, q_rows=rows_t, kv_len=to_dev(inp["kv_len"]))
    ref, _ = oracle.sdpa(inp["q_c"].value, inp["k_txt"].value, inp["v_txt"].value, q_rows=rows[samp],
                         kv_len=inp["kv_len"])
    assert_attn_close(o[:, torch.from_numpy(samp).long()], ref, f"cross N={w.N}")
    # dense anchor pass (Eq. 18)
    o = sq.attn_fwd(q, k, v)
    samp = _sample_rows(rng, w.N)
    ref, _ = oracle.sdpa(inp["q_x"].value, inp["k_x"].value, inp["v_x"].value, q_rows=samp)
    assert_attn_close(o[:, torch.from_numpy(samp).long()], ref, f"dense N={w.N}")


@pytest.mark.parametrize("H,d,Nq,n_sel", [(24, 96, 3201, 2695), (32, 72, 4225, 2440)])
def test_two_row_blocks_partial_key_tile_ragged_rows(H, d, Nq, n_sel):
    """Shapes the planner runs with 256-row tiles (two row blocks per wave) and a split tail,
    with a partial last key tile (Nk % 64 != 0) and row counts that are not a multiple of
    256: dense, gathered per-sample rows and scattered output, oracle on sampled rows of
    every (b, h)."""
    B, Nk = 2, 8250
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=40 + d)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rng = np.random.default_rng(41)
    rows = np.stack([W.random_rows(rng, Nq, n_sel) for _ in range(B)])
    rows_t = to_dev(rows)
    for name, qr in (("dense", None), ("gathered", rows_t)):
        plan = sq.attn_plan(qd, kd, q_rows=qr)
        assert plan["rows_per_tile"] == 256 and plan["split_tiles"] > 0, (name, plan)
        assert plan["keys_per_range"] % 64 == 0 and plan["key_ranges"] >= 2, (name, plan)
        # the same plan twice; the unsplit plan when no workspace is given
        assert sq.attn_plan(qd, kd, q_rows=qr) == plan
        assert sq.attn_plan(qd, kd, q_rows=qr, workspace_bytes=0)["split_tiles"] == 0
    o, lse = sq.attn_fwd(qd, kd, vd, return_lse=True)
    samp = _sample_rows(rng, Nq)
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, q_rows=samp)
    sel = torch.from_numpy(samp).long()
    assert_attn_close(o[:, sel], ref, f"dense d={d}")
    assert_lse_close(lse.cpu()[:, :, sel], ref_lse, f"dense lse d={d}")
    out = torch.full((B, Nq, H, d), 5.0, dtype=torch.bfloat16, device=qd.device)
    sq.attn_fwd(qd, kd, vd, q_rows=rows_t, out=out, scatter_out=True)
    compact = sq.attn_fwd(qd, kd, vd, q_rows=rows_t)
    samp = _sample_rows(rng, rows.shape[1])
    for b in range(B):
        ref, _ = oracle.sdpa(q.value[b:b + 1], k.value[b:b + 1], v.value[b:b + 1], q_rows=rows[b, samp])
        assert_attn_close(compact[b:b + 1, torch.from_numpy(samp).long()], ref, f"gathered b={b} d={d}")
        assert torch.equal(out[b, torch.from_numpy(rows[b]).long()], compact[b]), "scatter = compact rows"
    untouched = np.ones((B, Nq), bool)
    for b in range(B):
        untouched[b, rows[b]] = False
    assert bool((out.float().cpu().numpy()[untouched] == 5.0).all())


def test_two_row_blocks_unsplit_ragged():
    """256-row tiles with no split (the tile count fills whole rounds), a ragged last row
    tile and a partial last key tile: oracle on sampled rows of every (b, h), LSE included."""
    B, Nq, Nk, H, d = 2, 8100, 4133, 24, 96
    q, k, v = W.attention_inputs(B, Nq, Nk, H, d, seed=44)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    plan = sq.attn_plan(qd, kd)
    assert plan["rows_per_tile"] == 256 and plan["split_tiles"] == 0 and plan["workspace_bytes"] == 0, plan
    o, lse = sq.attn_fwd(qd, kd, vd, return_lse=True)
    rng = np.random.default_rng(45)
    samp = np.unique(np.concatenate([_sample_rows(rng, Nq), [Nq - 1, Nq - 2, 31 * 256, 31 * 256 - 1]]))
    ref, ref_lse = oracle.sdpa(q.value, k.value, v.value, q_rows=samp)
    sel = torch.from_numpy(samp).long()
    assert_attn_close(o[:, sel], ref, "unsplit 256-row tiles")
    assert_lse_close(lse.cpu()[:, :, sel], ref_lse, "unsplit 256-row tiles lse")


@pytest.mark.parametrize("d", [32, 64, 72, 96, 128])
def test_plan_is_consistent_with_the_workspace_query(d):
    """safe_attn_plan agrees with safe_attn_workspace_bytes, counts the tiles it says, covers
    every key with its ranges, and keeps 128-row tiles with key lengths and at head dimensions
    without a two-row-block instance."""
    dev = torch.device("cuda:0")
    for B, Nq, Nk, H, n_sel in ((2, 300, 3000, 3, None), (2, 5000, 4133, 8, 3001), (1, 20000, 700, 4, None),
                                (2, 1000, 64, 24, 17)):
        q = torch.zeros((B, Nq, H, d), dtype=torch.bfloat16, device=dev)
        k = torch.zeros((B, Nk, H, d), dtype=torch.bfloat16, device=dev)
        rows = None if n_sel is None else torch.arange(n_sel, dtype=torch.int32, device=dev)
        n_rows = Nq if rows is None else n_sel
        for kw in ({}, {"kv_len": torch.full((B,), Nk // 2, dtype=torch.int32, device=dev)}):
            plan = sq.attn_plan(q, k, q_rows=rows, **kw)
            assert plan["rows_per_tile"] in (128, 256), plan
            if kw or d not in (72, 96):
                assert plan["rows_per_tile"] == 128, plan
            assert plan["row_tiles"] == -(-n_rows // plan["rows_per_tile"]) * H * B, plan
            assert plan["workspace_bytes"] == sq.attn_workspace_bytes(q, k, q_rows=rows, **kw), plan
            if plan["split_tiles"]:
                assert not kw, "the key-length form is never split"
                assert plan["split_tiles"] <= plan["row_tiles"], plan
                assert plan["key_ranges"] >= 2 and plan["keys_per_range"] % 64 == 0
                assert (plan["key_ranges"] - 1) * plan["keys_per_range"] < Nk <= plan["key_ranges"] * plan["keys_per_range"]
                assert plan["workspace_bytes"] == plan["split_tiles"] * plan["key_ranges"] * plan["rows_per_tile"] * (4 * d + 8)
            else:
                assert plan["key_ranges"] == 1 and plan["workspace_bytes"] == 0
            assert sq.attn_plan(q, k, q_rows=rows, workspace_bytes=0, **kw)["split_tiles"] == 0


def test_side_stream_matches_default_stream():
    """The same calls enqueued on a second stream (its own workspace in the binding) give
    bitwise the same results as on the default stream, split tails included."""
    B, N, H, d = 2, 3000, 4, 96
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=46)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rows_t = to_dev(W.random_rows(np.random.default_rng(47), N, 1111))
    assert sq.attn_plan(qd, kd)["split_tiles"] > 0, "the shape must take the split path"
    ref_d, ref_lse = sq.attn_fwd(qd, kd, vd, return_lse=True)
    ref_s = sq.attn_fwd(qd, kd, vd, q_rows=rows_t)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        od, lse = sq.attn_fwd(qd, kd, vd, return_lse=True)
        os_ = sq.attn_fwd(qd, kd, vd, q_rows=rows_t)
    side.synchronize()
    assert torch.equal(od, ref_d) and torch.equal(lse, ref_lse) and torch.equal(os_, ref_s)


def test_hip_graph_replays_match_eager():
    """An SRSU step (global K/V assembly, SRSU self-attention with its split tail, dense pass)
    captured in a HIP graph: every replay, with eager work on the same buffers in between,
    gives the eager results bitwise."""
    B, N, H, d, n_sel = 2, 3000, 4, 96, 1111
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=48)
    qd, kc, vc = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rows_np = np.stack([W.random_rows(np.random.default_rng(49 + b), N, n_sel) for b in range(B)])
    rows = to_dev(rows_np)
    g = torch.Generator(device="cuda").manual_seed(50)
    kf = torch.randn((B, n_sel, H, d), generator=g, device="cuda").to(torch.bfloat16)
    vf = torch.randn((B, n_sel, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k_glob, v_glob = torch.empty_like(kc), torch.empty_like(vc)
    o_s = torch.empty((B, n_sel, H, d), dtype=torch.bfloat16, device="cuda")
    o_d = torch.empty_like(qd)

    def step():
        sq.kv_assemble(kf, vf, rows, kc, vc, k_out=k_glob, v_out=v_glob)
        sq.attn_fwd(qd, k_glob, v_glob, q_rows=rows, out=o_s)
        sq.attn_fwd(qd, kc, vc, out=o_d)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up on the capture stream (its workspace, cached plans)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_s, ref_d = o_s.clone(), o_d.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for rep in range(3):
        o_s.zero_(); o_d.zero_(); k_glob.zero_()
        eager = sq.attn_fwd(qd, kc, vc)            # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_s, ref_s) and torch.equal(o_d, ref_d), f"replay {rep}"
        assert torch.equal(eager, ref_d)


def test_caller_outputs_of_the_wrong_shape_or_memory_are_refused():
    """Outputs that the call would write past, of another dtype, or in host memory raise
    before any launch."""
    B, N, H, d = 1, 256, 2, 64
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=60)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    rows = to_dev(np.arange(0, 256, 4, dtype=np.int32))
    for bad in (torch.empty((B, 63, H, d), dtype=torch.bfloat16, device="cuda"),     # one row short
                torch.empty((B, 64, H, d), dtype=torch.float32, device="cuda"),
                torch.empty((B, 64, H, d), dtype=torch.bfloat16)):                   # host memory
        with pytest.raises((ValueError, TypeError)):
            sq.attn_fwd(qd, kd, vd, q_rows=rows, out=bad)
    with pytest.raises(ValueError):                                                  # scatter needs all rows
        sq.attn_fwd(qd, kd, vd, q_rows=rows, out=torch.empty((B, 64, H, d), dtype=torch.bfloat16,
                                                                device="cuda"), scatter_out=True)
    f = qd[:, :64].contiguous()
    with pytest.raises(ValueError):
        sq.kv_assemble(f, f, rows, kd, vd, k_out=torch.empty((B, N - 1, H, d), dtype=torch.bfloat16, device="cuda"))
    o = sq.attn_fwd(qd, kd, vd, q_rows=rows, out=torch.empty((B, 64, H, d), dtype=torch.bfloat16, device="cuda"))
    ref, _ = oracle.sdpa(q.value, k.value, v.value, q_rows=np.arange(0, 256, 4)[[0, 63]])
    assert_attn_close(o[:, [0, 63]], ref, "valid caller output")


def test_graph_replay_after_the_cached_workspace_grew():
    """A call captured with the binding's cached workspace keeps writing that buffer on replay;
    a larger eager call on the same stream afterwards grows the cache, and the superseded
    buffer must stay allocated so the replay cannot land in memory that other tensors took."""
    B, N, H, d = 2, 2000, 4, 96
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=52)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    big_q = torch.randn((B, 6000, H, d), device="cuda").to(torch.bfloat16)
    big_k = torch.randn((B, 9000, H, d), device="cuda").to(torch.bfloat16)
    small_need = sq.attn_workspace_bytes(qd, kd)
    big_need = sq.attn_workspace_bytes(big_q, big_k)
    assert 0 < small_need < big_need, (small_need, big_need)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o = torch.empty_like(qd)
    with torch.cuda.stream(side):
        sq.attn_fwd(qd, kd, vd, out=o)          # sizes this stream's cached workspace
    side.synchronize()
    ref = o.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        sq.attn_fwd(qd, kd, vd, out=o)
    with torch.cuda.stream(side):
        big = sq.attn_fwd(big_q, big_k, big_k)   # grows the cached workspace of this stream
    side.synchronize()
    fillers = [torch.full((small_need // 4 + 1,), 7.0, device="cuda") for _ in range(4)]
    for rep in range(3):
        o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"replay {rep}"
        assert all(bool((f == 7.0).all()) for f in fillers), "a replay wrote into another tensor"
    assert torch.isfinite(big.float()).all()


def test_operands_of_the_wrong_dtype_or_batch_are_refused_before_launch():
    """Every attention, assembly and linear operand is bf16 (fp16 bits would be read as bf16);
    key lengths have one entry per sample; index lists are [n], [1, n] or [B, n]."""
    B, N, H, d = 2, 256, 2, 64
    q, k, v = W.attention_inputs(B, N, N, H, d, seed=61)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    for bad in ((qd.half(), kd, vd), (qd, kd.view(torch.int16), vd), (qd, kd, vd.float())):
        with pytest.raises(TypeError):
            sq.attn_fwd(*bad)
    with pytest.raises(TypeError):
        sq.attn_fwd(qd, kd, vd, out=torch.empty_like(qd).half())
    for kv in (torch.tensor([5], dtype=torch.int32, device="cuda"),
               torch.tensor([5, 6, 7], dtype=torch.int32, device="cuda"),
               torch.tensor([[5, 6]], dtype=torch.int32, device="cuda")):
        with pytest.raises(ValueError):
            sq.attn_fwd(qd, kd, vd, kv_len=kv)
        with pytest.raises(ValueError):
            sq.pcsp_accumulate(qd, kd, torch.ones((B, N), device="cuda"), torch.zeros((B, N), device="cuda"),
                               kv_len=kv)
    rows3 = torch.zeros((3, 10), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        sq.attn_fwd(qd, kd, vd, q_rows=rows3)
    with pytest.raises(ValueError):
        sq.attn_fwd(qd, kd, vd, q_rows=torch.zeros((B, 20), dtype=torch.int32, device="cuda")[:, ::2])
    idx = torch.arange(0, N, 4, dtype=torch.int32, device="cuda")
    f = qd[:, :idx.shape[0]].contiguous()
    for bad_idx in (rows3, idx.view(1, 1, -1), torch.stack([idx, idx], 1)):
        with pytest.raises(ValueError):
            sq.kv_assemble(f, f, bad_idx, kd, vd)
    with pytest.raises(TypeError):
        sq.kv_assemble(f.half(), f.half(), idx, kd, vd)
    # a [1, n] list is shared by every sample (sample stride 0), like a [n] list
    ko1, _ = sq.kv_assemble(f, f, idx.view(1, -1), kd, vd)
    ko2, _ = sq.kv_assemble(f, f, idx, kd, vd)
    assert torch.equal(ko1, ko2)
    o1 = sq.attn_fwd(qd, kd, vd, q_rows=idx.view(1, -1))
    assert torch.equal(o1, sq.attn_fwd(qd, kd, vd, q_rows=idx))
    fc = torch.zeros((B, N, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        sq.sw_cfg(fc, fc, 3.0, 5.0, s=torch.zeros((3, N), device="cuda"))
    with pytest.raises(ValueError):
        sq.sw_cfg(fc, fc, 3.0, 5.0, idx=rows3)
