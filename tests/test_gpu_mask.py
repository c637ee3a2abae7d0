"""GPU parity of safe_mask_classify against the oracle: bit-exact (Eq. 6-8)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("sparse_query_sdpa_amd")

GOLD = os.path.join(os.path.dirname(__file__), "golden")
NP_DT = {torch.bfloat16: None, torch.float16: np.float16, torch.float32: np.float32}


def _num(x):
    if isinstance(x, str):
        return {"inf": np.inf, "-inf": -np.inf, "nan": np.nan, "-0": -0.0}[x]
    return float(x)


def _to_device_mask(values: np.ndarray, dtype) -> torch.Tensor:
    """float64 values -> device tensor of `dtype` (exact for the values used here)."""
    if dtype == torch.bfloat16:
        bits = W.f32_to_bf16_bits(values.astype(np.float32))
        nan = np.isnan(values)
        bits[nan] = W.BF16_NAN
        return torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(values.astype(NP_DT[dtype])).to(dev())


def _compare(t: torch.Tensor, m_host: np.ndarray, is_bool: bool):
    got = sq.mask_classify(t, row_class=True, kv_len=True)
    ref = oracle.classify_mask(m_host, is_bool)
    assert got["verdict"] == ref.verdict
    assert got["mask_class"] == ref.mask_class, (got["class_name"], oracle.CLASS_NAMES[ref.mask_class])
    assert got["first_bad_row"] == ref.first_bad_row
    assert got["rows"] == ref.rows
    assert np.array_equal(got["row_class"].cpu().numpy(), ref.row_class)
    assert np.array_equal(got["kv_len"].cpu().numpy(), ref.kv_len)


CASES = json.load(open(os.path.join(GOLD, "mask_cases.json")))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_cases_every_dtype(case):
    if case["bool"]:
        m = np.asarray(case["data"], dtype=np.uint8).reshape(case["shape"])
        _compare(to_dev(m), m, True)
        _compare(to_dev(m != 0), m, True)
        return
    vals = np.asarray([_num(x) for x in case["data"]], dtype=np.float64).reshape(case["shape"])
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        _compare(_to_device_mask(vals, dt), vals, False)


def test_tiny_workload_cases():
    for name, m in W.c1_mask_cases().items():
        is_bool = m.dtype == np.uint8
        _compare(to_dev(m), m, is_bool)


@pytest.mark.parametrize("Nk", [1, 7, 64, 333, 2048])
def test_fuzz_against_oracle(Nk):
    """Random rows mixing constants, padding, holes, signed zeros, NaN/inf; aligned and unaligned rows."""
    rng = np.random.default_rng(Nk)
    B, H, Nq = 2, 3, 40
    m = np.broadcast_to(rng.choice([0.0, -0.0, 1.5, -3.0], size=(B, H, Nq, 1)), (B, H, Nq, Nk)).copy()
    for r in range(B * H * Nq):
        b, h, i = r // (H * Nq), (r // Nq) % H, r % Nq
        kind = rng.integers(0, 8)
        if kind == 1:
            m[b, h, i, rng.integers(0, Nk):] = -np.inf
        elif kind == 2:
            m[b, h, i, rng.integers(0, Nk)] = rng.choice([np.nan, np.inf, -np.inf, 2.0, -0.0])
        elif kind == 3:
            m[b, h, i] = rng.standard_normal(Nk)
    # make sample 1 a consistent key-padding mask half of the time
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        vals = m if dt != torch.float16 else np.where(np.isfinite(m), np.round(m, 2), m)
        host = _to_device_mask(vals, dt).float().cpu().numpy().astype(np.float64)  # exact widening
        _compare(_to_device_mask(vals, dt), host, False)
    bm = (rng.random((B, H, Nq, Nk)) < 0.97).astype(np.uint8)
    bm[0, :, :, : max(1, Nk // 2)] = 1
    _compare(to_dev(bm), bm, True)


def test_padding_masks_give_lengths():
    B, Nq, Nk = 3, 16, 256
    lens = np.array([11, 256, 40], np.int32)
    m = np.zeros((B, 1, Nq, Nk), np.float32)
    for b in range(B):
        m[b, :, :, lens[b]:] = -np.inf
    got = sq.mask_classify(to_dev(m), kv_len=True)
    assert got["class_name"] == "KEY_PADDING"
    assert np.array_equal(got["kv_len"].cpu().numpy(), lens)
    # bool form, broadcast over queries (one stored row per sample)
    bm = (np.arange(Nk)[None, None, None, :] < lens[:, None, None, None]).astype(np.uint8)
    got = sq.mask_classify(to_dev(bm), kv_len=True)
    assert got["class_name"] == "KEY_PADDING" and np.array_equal(got["kv_len"].cpu().numpy(), lens)


def test_strided_and_expanded_views():
    base = torch.zeros((1, 1, 64, 100), dtype=torch.float32, device=dev())
    view = base.expand(2, 3, 64, 100)                 # stride-0 broadcast dims
    got = sq.mask_classify(view)
    assert got["class_name"] == "ZERO" and got["rows"] == 2 * 3 * 64
    big = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device=dev())
    big[0, 0, 5, 120] = 1.0
    got = sq.mask_classify(big[..., :100])            # rows not contiguous with each other
    assert got["class_name"] == "ZERO"
    got = sq.mask_classify(big[..., 1:125])           # rows start unaligned
    assert got["class_name"] == "NONCONST" and got["first_bad_row"] == 5
    empty = torch.zeros((1, 1, 0, 16), dtype=torch.float32, device=dev())
    got = sq.mask_classify(empty)
    assert got["verdict"] == 1 and got["rows"] == 0


def test_full_size_bf16_zero_mask_2560sq():
    """The all-valid additive mask of the 160x160 workload: [2, 1, 25600, 25600] bf16 zeros (2.6 GB)."""
    N = W.WORKLOADS[4].N
    m = torch.zeros((2, 1, N, N), dtype=torch.bfloat16, device=dev())
    got = sq.mask_classify(m, row_class=True)
    assert (got["verdict"], got["class_name"], got["first_bad_row"], got["rows"]) == (1, "ZERO", -1, 2 * N)
    assert torch.all(got["row_class"] == 1)
    # one planted entry is found at full size
    r = 12345
    m[1, 0, r, N - 1] = -0.0
    assert sq.mask_classify(m)["verdict"] == 1        # -0 == +0
    m[1, 0, r, N - 3] = 2.0 ** -20
    got = sq.mask_classify(m, row_class=True)
    row = m[1, 0, r].float().cpu().numpy()
    assert oracle.classify_row(row, False)[0] == oracle.NONCONST
    assert (got["verdict"], got["class_name"], got["first_bad_row"]) == (0, "NONCONST", N + r)
    del m
    torch.cuda.empty_cache()


def test_full_size_f32_row_constant_mask_3072sq():
    """[1, 1, 36864, 36864] fp32 row-constant mask c_i ~ U(-3, 3) (5.4 GB): certified removable."""
    N = W.WORKLOADS[5].N
    c = W.row_constants_f32(W.rng_for(5, stream=5), N, -3.0, 3.0)
    m = torch.from_numpy(c).to(dev())[None, None, :, None].expand(1, 1, N, N).contiguous()
    got = sq.mask_classify(m, row_class=True)
    assert (got["verdict"], got["class_name"], got["first_bad_row"]) == (1, "ROW_CONST", -1)
    rc = got["row_class"].cpu().numpy()
    rng = np.random.default_rng(0)
    for r in rng.choice(N, 8, replace=False):
        assert rc[r] == oracle.classify_row(m[0, 0, r].cpu().numpy(), False)[0]
    del m
    torch.cuda.empty_cache()
