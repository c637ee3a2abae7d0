"""GPU parity of safe_kv_assemble against the oracle: bit-exact (Eq. 14, 16, 19)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_attn_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("shape", [(1, 256, 2, 32), (2, 1000, 3, 96), (2, 4096, 24, 96)])
def test_assemble_bit_exact(shape, shared):
    B, N, H, d = shape
    rng = np.random.default_rng(N + H)
    nsel = (3 * N) // 10
    cache_k, cache_v, _ = W.attention_inputs(B, N, N, H, d, seed=N)
    fk, fv, _ = W.attention_inputs(B, nsel, nsel, H, d, seed=N + 1)
    idx = W.random_rows(rng, N, nsel) if shared else np.stack([W.random_rows(rng, N, nsel) for _ in range(B)])
    ko, vo = sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(idx), to_dev_bf16(cache_k), to_dev_bf16(cache_v))
    assert np.array_equal(_bits(ko), oracle.kv_assemble(fk.bits, idx, cache_k.bits))
    assert np.array_equal(_bits(vo), oracle.kv_assemble(fv.bits, idx, cache_v.bits))


def test_in_place_scatter_and_edge_counts():
    B, N, H, d = 2, 777, 5, 64
    rng = np.random.default_rng(1)
    ck, cv, _ = W.attention_inputs(B, N, N, H, d, seed=3)
    fk, fv, _ = W.attention_inputs(B, 100, 100, H, d, seed=4)
    idx = np.stack([W.random_rows(rng, N, 100) for _ in range(B)])
    kc, vc = to_dev_bf16(ck), to_dev_bf16(cv)
    ko, vo = sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(idx), kc, vc, in_place=True)
    assert ko.data_ptr() == kc.data_ptr()
    assert np.array_equal(_bits(kc), oracle.kv_assemble(fk.bits, idx, ck.bits))
    assert np.array_equal(_bits(vc), oracle.kv_assemble(fv.bits, idx, cv.bits))
    # S empty: output is the cache; S = all rows: output is the fresh tensor (Eq. 19 refresh)
    empty = to_dev(np.zeros((0,), np.int32))
    z = torch.empty((B, 0, H, d), dtype=torch.bfloat16, device=kc.device)
    ko, vo = sq.kv_assemble(z, z, empty, to_dev_bf16(ck), to_dev_bf16(cv))
    assert np.array_equal(_bits(ko), ck.bits)
    allk, allv, _ = W.attention_inputs(B, N, N, H, d, seed=5)
    ko, vo = sq.kv_assemble(to_dev_bf16(allk), to_dev_bf16(allv), to_dev(np.arange(N, dtype=np.int32)),
                            to_dev_bf16(ck), to_dev_bf16(cv))
    assert np.array_equal(_bits(ko), allk.bits) and np.array_equal(_bits(vo), allv.bits)


def test_out_of_range_indices_are_skipped_or_rejected():
    B, N, H, d = 1, 300, 2, 32
    ck, cv, _ = W.attention_inputs(B, N, N, H, d, seed=6)
    fk, fv, _ = W.attention_inputs(B, 3, 3, H, d, seed=7)
    idx = np.array([5, 40, 300], dtype=np.int32)
    with pytest.raises(sq.SafeError) as e:
        sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(idx), to_dev_bf16(ck), to_dev_bf16(cv), check=True)
    assert e.value.status == -4
    with pytest.raises(sq.SafeError):   # not ascending
        sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(np.array([5, 5, 9], np.int32)),
                       to_dev_bf16(ck), to_dev_bf16(cv), check=True)
    kc, vc = to_dev_bf16(ck), to_dev_bf16(cv)
    sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(idx), kc, vc, in_place=True)
    exp = oracle.kv_assemble(fk.bits[:, :2], idx[:2], ck.bits)
    assert np.array_equal(_bits(kc), exp)


def test_multistep_cache_workload():
    """One anchor then three SRSU steps on the 64x64-grid workload (drift N(0, 0.05)): the
    assembly bit-exact, SRSU self- and cross-attention against the oracle at every step."""
    inp = W.workload_inputs(2)
    w = inp["workload"]
    rng = W.rng_for(2, stream=4)
    S = W.random_rows(rng, w.N, w.k_for(30))
    k_t, v_t = inp["k_x"].value.copy(), inp["v_x"].value.copy()
    cache_k, cache_v = to_dev_bf16(inp["k_x"]), to_dev_bf16(inp["v_x"])   # anchor: cache <- dense K/V (Eq. 19)
    ref_k, ref_v = inp["k_x"].bits.copy(), inp["v_x"].bits.copy()
    for step in range(3):
        k_t = k_t + W.drift((1002, 10, step), k_t.shape)
        v_t = v_t + W.drift((1002, 11, step), v_t.shape)
        kb, vb = W.bf16_from_f32(k_t), W.bf16_from_f32(v_t)
        fk = W.Bf16Tensor(kb.bits[:, S], kb.value[:, S])
        fv = W.Bf16Tensor(vb.bits[:, S], vb.value[:, S])
        ko, vo = sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(S), cache_k, cache_v)
        rk = oracle.kv_assemble(fk.bits, S, ref_k)
        rv = oracle.kv_assemble(fv.bits, S, ref_v)
        assert np.array_equal(_bits(ko), rk) and np.array_equal(_bits(vo), rv), step
        # SRSU self-attention on the assembled K/V (Eq. 16) and the text cross-attention with
        # per-sample lengths (Eq. 17), oracle on sampled rows of S in every (b, h)
        qx = to_dev_bf16(inp["q_x"])
        o_s = sq.attn_fwd(qx, ko, vo, q_rows=to_dev(S))
        o_c = sq.attn_fwd(to_dev_bf16(inp["q_c"]), to_dev_bf16(inp["k_txt"]), to_dev_bf16(inp["v_txt"]),
                          q_rows=to_dev(S), kv_len=to_dev(inp["kv_len"]))
        samp = np.unique(np.concatenate([[0, len(S) - 1], rng.choice(len(S), 24, replace=False)]))
        kg = oracle.kv_assemble(fk.value, S, inp["k_x"].value)   # the oracle's own global K/V
        vg = oracle.kv_assemble(fv.value, S, inp["v_x"].value)
        ref, _ = oracle.sdpa(inp["q_x"].value, kg, vg, q_rows=S[samp])
        assert_attn_close(o_s[:, torch.from_numpy(samp).long()], ref, f"srsu step {step}")
        ref, _ = oracle.sdpa(inp["q_c"].value, inp["k_txt"].value, inp["v_txt"].value, q_rows=S[samp],
                             kv_len=inp["kv_len"])
        assert_attn_close(o_c[:, torch.from_numpy(samp).long()], ref, f"cross step {step}")


def test_assemble_full_size_bit_exact():
    """Eq. 14/16 at the 160x160 workload in the bench's form: the drifted fresh rows of the
    PCSP-sized set (k = 6400 per sample, per-sample lists) over the cached K/V, out of place
    and in place, compared with the definition bit for bit over every element."""
    inp = W.workload_inputs(4)
    w = inp["workload"]
    k = w.k_for(25)
    rng = W.rng_for(4, stream=9)
    idx = np.stack([W.random_rows(rng, w.N, k) for _ in range(w.B)])
    fk = W.bf16_from_f32(inp["k_x"].value[np.arange(w.B)[:, None], idx] + W.drift((1004, 20), (w.B, k, w.H, w.d)))
    fv = W.bf16_from_f32(inp["v_x"].value[np.arange(w.B)[:, None], idx] + W.drift((1004, 21), (w.B, k, w.H, w.d)))
    kc, vc = to_dev_bf16(inp["k_x"]), to_dev_bf16(inp["v_x"])
    ko, vo = sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(idx), kc, vc)
    ref_k = oracle.kv_assemble(fk.bits, idx, inp["k_x"].bits)
    assert np.array_equal(_bits(ko), ref_k)
    ref_v = oracle.kv_assemble(fv.bits, idx, inp["v_x"].bits)
    assert np.array_equal(_bits(vo), ref_v)
    sq.kv_assemble(to_dev_bf16(fk), to_dev_bf16(fv), to_dev(idx), kc, vc, in_place=True)
    assert np.array_equal(_bits(kc), ref_k) and np.array_equal(_bits(vc), ref_v)
