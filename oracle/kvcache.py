"""Global K/V assembly and the context-cache refresh -- test infrastructure only.

Follows "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
Diffusion Transformers":
  * Eq. 14 the cache holds the context rows of the most recent anchor;
  * Eq. 16 K_{S u C}, V_{S u C} are assembled in the original token order from
    the current sensitive rows and the cached context rows;
  * Eq. 19 at an anchor the cached context rows are replaced by the dense
    result.

Reading: the cache holds per-layer keys and values [B, N, H, d] (the paper's
Eq. 14 speaks of hidden states; keys and values are fixed row-wise functions
of them, so caching them is the same schedule one projection later).

Pins (tests/test_oracle_kv.py): S = all rows returns the fresh tensor, S empty
returns the cache, every row equals exactly one of its two sources, and a
per-row brute-force loop.
"""
from __future__ import annotations

import numpy as np


def kv_assemble(fresh, idx, cache) -> np.ndarray:
    """out[b, j] = fresh[b, r] if idx[b, r] == j else cache[b, j]  (Eq. 16).

    fresh: [B, k, H, d] sensitive rows in the order of idx; idx: [k] shared or
    [B, k] ascending distinct token indices; cache: [B, N, H, d].
    """
    cache = np.asarray(cache)
    fresh = np.asarray(fresh)
    out = cache.copy()
    B = cache.shape[0]
    idx = np.asarray(idx, dtype=np.int64)
    if idx.ndim == 1:
        idx = np.broadcast_to(idx, (B, idx.shape[0]))
    for b in range(B):
        out[b, idx[b]] = fresh[b]
    return out


def car_refresh(dense_k, dense_v):
    """Eq. 19: after an anchor's dense pass the cache becomes the dense K/V."""
    return np.array(dense_k, copy=True), np.array(dense_v, copy=True)
