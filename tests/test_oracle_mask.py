"""Pins of the mask classifier oracle (Eq. 5-8)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        return {"inf": np.inf, "-inf": -np.inf, "nan": np.nan, "-0": -0.0}[x]
    return float(x)


def golden_cases():
    g = json.load(open(os.path.join(GOLD, "mask_cases.json")))
    return g["codes"], g["cases"]


CODES, CASES = golden_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_mask_cases(case):
    if case["bool"]:
        m = np.asarray(case["data"], dtype=np.uint8).reshape(case["shape"])
    else:
        m = np.asarray([_num(x) for x in case["data"]], dtype=np.float64).reshape(case["shape"])
    v = oracle.classify_mask(m, case["bool"])
    assert [oracle.CLASS_NAMES[c] for c in v.row_class] == case["rows"]
    assert oracle.CLASS_NAMES[v.mask_class] == case["overall"]
    assert v.verdict == case["verdict"]
    assert v.first_bad_row == case["first_bad_row"]
    assert list(v.kv_len) == case["kv_len"]
    # the plain per-row loop gives the same classes
    flat = m.reshape(-1, m.shape[-1])
    assert [oracle.classify_row(r, case["bool"])[0] for r in flat] == list(v.row_class)


def test_vectorised_equals_scalar_fuzz():
    rng = np.random.default_rng(123)
    specials = np.array([0.0, -0.0, 1.5, -2.0, np.inf, -np.inf, np.nan])
    for trial in range(400):
        n = int(rng.integers(1, 7))
        R = 8
        kind = trial % 4
        if kind == 0:      # few distinct values, specials mixed in
            rows = rng.choice(specials, size=(R, n), p=[.3, .1, .2, .1, .05, .2, .05])
        elif kind == 1:    # padded rows with random L
            rows = np.zeros((R, n)) + rng.choice([0.0, 3.0], size=(R, 1))
            for r in range(R):
                L = int(rng.integers(0, n + 1))
                rows[r, L:] = -np.inf
        elif kind == 2:    # constant rows with one perturbation
            rows = np.broadcast_to(rng.standard_normal((R, 1)), (R, n)).copy()
            rows[rng.integers(0, R), rng.integers(0, n)] += rng.choice([0.0, 1.0, -np.inf])
        else:              # booleans
            rows = (rng.random((R, n)) < 0.8).astype(np.uint8)
        is_bool = kind == 3
        cls, lens = oracle.classify_rows(rows, is_bool)
        for r in range(R):
            c, L = oracle.classify_row(rows[r], is_bool)
            assert (c, L) == (cls[r], lens[r]), (rows[r], c, cls[r])


def test_tiny_workload_cases():
    cases = W.c1_mask_cases()
    expect = {"all_valid_bool": ("ALL_VALID", 1), "zero_additive": ("ZERO", 1),
              "row_constant": ("ROW_CONST", 1), "random_additive": ("NONCONST", 0),
              "text_padding": ("KEY_PADDING", 0)}
    for name, m in cases.items():
        v = oracle.classify_mask(m, m.dtype == np.uint8)
        assert (oracle.CLASS_NAMES[v.mask_class], v.verdict) == expect[name], name
    v = oracle.classify_mask(cases["text_padding"], False)
    assert list(v.kv_len) == [11]


def test_removable_rows_leave_attention_unchanged_eq7():
    """Every row in R leaves SDPA unchanged; the rewrite equals the masked call."""
    rng = np.random.default_rng(9)
    B, N, H, d = 1, 24, 2, 8
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    o0, _ = oracle.sdpa(q, k, v)
    for m, is_bool in [(np.ones((1, 1, N, N), np.uint8), True),
                       (np.zeros((1, 1, N, N)), False),
                       (W.mask_row_constant_f32(rng, N, N, -5, 5).astype(np.float64), False)]:
        o_r, _, verdict, path = oracle.safe_sdpa(q, k, v, m, is_bool)
        assert verdict.verdict == 1 and path == "none"
        o_m, _ = oracle.sdpa(q, k, v, mask=oracle.mask.to_additive(m, is_bool))
        np.testing.assert_allclose(o_m, o0, rtol=1e-12, atol=1e-13)
        assert np.array_equal(o_r, o0)


def test_key_padding_rewrite_equals_masked_call():
    rng = np.random.default_rng(10)
    B, Nq, Nk, H, d = 2, 7, 16, 2, 8
    q = rng.standard_normal((B, Nq, H, d))
    k, v = rng.standard_normal((B, Nk, H, d)), rng.standard_normal((B, Nk, H, d))
    m = np.zeros((B, 1, 1, Nk))
    m[0, ..., 11:] = -np.inf
    m[1, ..., 5:] = -np.inf
    o_r, _, verdict, path = oracle.safe_sdpa(q, k, v, m)
    assert path == "kv_len" and list(verdict.kv_len) == [11, 5]
    o_m, _ = oracle.sdpa(q, k, v, mask=m)
    np.testing.assert_allclose(o_r, o_m, atol=1e-15)
    # a non-constant finite bias keeps the mask
    bias = rng.standard_normal((1, 1, Nq, Nk))
    _, _, verdict, path = oracle.safe_sdpa(q, k, v, bias)
    assert path == "mask" and verdict.mask_class == oracle.NONCONST


def test_non_removable_rows_have_a_witness():
    """Converse after Eq. 7: rows outside R change pi at zero logits; rows in R do not."""
    rng = np.random.default_rng(12)
    rows = [np.zeros(5), np.full(5, 2.0), rng.standard_normal(5), np.array([0, 0, 0, -np.inf, -np.inf]),
            np.array([0.0, -np.inf, 0, 0, 0]), np.full(5, -np.inf), np.array([0, np.nan, 0, 0, 0]),
            np.array([0, np.inf, 0, 0, 0])]
    for r in rows:
        c, _ = oracle.classify_row(r, False)
        wit = oracle.removable_row_witness(r, False)
        if c in oracle.REMOVABLE:
            assert wit == 0.0
        else:
            assert not (wit == 0.0), (r, c, wit)
    for r in [np.array([1, 1, 1], np.uint8), np.array([1, 1, 0], np.uint8), np.array([0, 1, 1], np.uint8)]:
        c, _ = oracle.classify_row(r, True)
        assert (oracle.removable_row_witness(r, True) == 0.0) == (c in oracle.REMOVABLE)


def test_broadcast_rows_and_empty():
    # one stored row per sample, broadcast over heads and queries
    m = np.zeros((2, 1, 1, 8))
    m[1, 0, 0, 3] = 1.0
    v = oracle.classify_mask(m, False)
    assert v.rows == 2 and list(v.row_class) == [oracle.ZERO, oracle.NONCONST] and v.first_bad_row == 1
    v = oracle.classify_mask(np.zeros((1, 1, 0, 4)), False)
    assert v.verdict == 1 and v.rows == 0 and v.first_bad_row == -1
    v = oracle.classify_mask(np.zeros((1, 1, 3, 0), np.uint8), True)
    assert v.verdict == 1 and v.mask_class == oracle.ALL_VALID
