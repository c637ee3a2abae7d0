"""The whole hot path of one step captured in one HIP graph: the asynchronous mask
certification (Eq. 6-8), the PCSP accumulation and selection (Eq. 9-12), the K/V assembly
(Eq. 14, 16), SRSU self- and cross-attention (Eq. 16-17) and the dense pass (Eq. 18), on the
64x64-grid workload.  Every replay -- with the outputs cleared and unrelated eager work in
between -- reproduces the eager step bit for bit, so no entry point allocates, synchronises
or records a memset on the captured stream."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")


def test_whole_step_in_a_hip_graph():
    inp = W.workload_inputs(2)
    w = inp["workload"]
    B, N, H, d, M = w.B, w.N, w.H, w.d, w.M
    k = w.k_for(30)
    q, kx, vx = (to_dev_bf16(inp[n]) for n in ("q_x", "k_x", "v_x"))
    qc, kt, vt = (to_dev_bf16(inp[n]) for n in ("q_c", "k_txt", "v_txt"))
    kv = to_dev(inp["kv_len"])
    wts = to_dev(W.pcsp_content_weights(inp["kv_len"], M))
    g = torch.Generator(device="cuda").manual_seed(5)
    kf = torch.randn((B, k, H, d), generator=g, device="cuda").to(torch.bfloat16)
    vf = torch.randn((B, k, H, d), generator=g, device="cuda").to(torch.bfloat16)
    mask = torch.zeros((B, 1, N, N), dtype=torch.bfloat16, device="cuda")
    acc = torch.zeros((B, N), dtype=torch.float32, device="cuda")
    k_glob, v_glob = torch.empty_like(kx), torch.empty_like(vx)
    o_s = torch.empty((B, k, H, d), dtype=torch.bfloat16, device="cuda")
    o_c, o_d = torch.empty_like(o_s), torch.empty_like(q)
    mws = sq.mask_classify(mask)["workspace"]
    sws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    state = {}

    def step():
        sq.mask_classify(mask, workspace=mws, asynchronous=True)
        acc.zero_()
        sq.pcsp_accumulate(qc, kt, wts, acc, kv_len=kv)
        idx = sq.pcsp_select(acc, w.grid_h, w.grid_w, 1.0, k, workspace=sws)
        sq.kv_assemble(kf, vf, idx, kx, vx, k_out=k_glob, v_out=v_glob)
        sq.attn_fwd(q, k_glob, v_glob, q_rows=idx, out=o_s)
        sq.attn_fwd(qc, kt, vt, q_rows=idx, kv_len=kv, out=o_c)
        sq.attn_fwd(q, kx, vx, out=o_d)
        state["idx"] = idx

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # eager step on the capture stream (its cached workspaces)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    outs = lambda: [state["idx"], acc, k_glob, v_glob, o_s, o_c, o_d, mws[:24]]   # + the 24-byte verdict
    ref = [t.clone() for t in outs()]
    assert int(ref[0].min()) >= 0 and bool(torch.all(ref[0][:, 1:] > ref[0][:, :-1])), "ascending top-k set"
    verdict = np.frombuffer(ref[7].cpu().numpy().tobytes(), dtype=np.int64)
    assert verdict[0] & 0xFFFFFFFF == 1 and verdict[1] == -1 and verdict[2] == B * N, "zero mask: removable"

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for rep in range(3):
        for t in outs()[:7]:
            t.zero_() if t.dtype != torch.int32 else t.fill_(-1)
        mws[:24].fill_(0xAB)
        eager = sq.attn_fwd(q, kx, vx, q_rows=state["idx"][:, :100].contiguous())   # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, exp) in enumerate(zip(outs(), ref)):
            assert torch.equal(got, exp), f"replay {rep}: output {i}"
        assert eager.shape == (B, 100, H, d)
