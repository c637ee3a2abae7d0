"""Pins of the K/V assembly oracle (Eq. 14, 16, 19)."""
import numpy as np

import oracle


def test_assemble_definition():
    rng = np.random.default_rng(0)
    B, N, H, d, k = 2, 20, 3, 4, 6
    cache = rng.standard_normal((B, N, H, d))
    fresh = rng.standard_normal((B, k, H, d))
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)])
    out = oracle.kv_assemble(fresh, idx, cache)
    for b in range(B):
        pos = {int(j): r for r, j in enumerate(idx[b])}
        for j in range(N):
            expect = fresh[b, pos[j]] if j in pos else cache[b, j]
            assert np.array_equal(out[b, j], expect)
    # shared index list
    out_s = oracle.kv_assemble(fresh, idx[0], cache)
    for b in range(B):
        assert np.array_equal(out_s[b, idx[0]], fresh[b])
    # the cache is not modified
    assert not np.shares_memory(out, cache)


def test_assemble_all_and_empty():
    rng = np.random.default_rng(1)
    cache = rng.standard_normal((1, 8, 2, 4))
    fresh = rng.standard_normal((1, 8, 2, 4))
    assert np.array_equal(oracle.kv_assemble(fresh, np.arange(8), cache), fresh)
    assert np.array_equal(oracle.kv_assemble(fresh[:, :0], np.arange(0), cache), cache)


def test_refresh_replaces_cache():
    k = np.arange(6.0).reshape(1, 3, 1, 2)
    v = -k
    ck, cv = oracle.car_refresh(k, v)
    assert np.array_equal(ck, k) and np.array_equal(cv, v) and not np.shares_memory(ck, k)
