"""Row-selective DiT block (Eq. 15) around the attention -- test infrastructure only.

Follows "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
Diffusion Transformers", Section on selective row state update (SRSU):
  * Eq. 15 at a non-anchor step the block keeps its order and parameters but
    computes attention outputs, residual updates and row-wise MLP outputs only
    for the rows of S; the context output rows are copied from the cache;
  * Eq. 16 the sensitive queries attend to global keys and values assembled from
    the fresh rows of S and the cached context rows;
  * Eq. 18-19 at an anchor step the dense block runs and refreshes the cache.

Reading: the pages leave the block's internals to the backbone.  A plain block
stands in, with synthetic weights (C = H * d channels, F hidden MLP channels):
    Q, K, V = X Wqkv^T split in three    (Wqkv [3C, C]; head h = columns h*d..h*d+d-1)
    A       = SDPA(Q, K, V)              (Eq. 2, no mask)
    Y       = X + A Wo^T                 (Wo [C, C])
    Z       = Y + gelu_tanh(Y W1^T + b1) W2^T + b2     (W1 [F, C], W2 [C, F])
The cache holds, from the anchor step, every row's block output Z and its keys
and values K, V.  gelu_tanh(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).

Pins (tests/test_oracle_block.py): torch's float64 linear, GELU (tanh form) and
scaled_dot_product_attention (library routines); zero weights give Z = X + b2;
with the cache taken from a dense pass on the same input, the row-selective
block equals the dense block for any S; S = all rows equals the dense block for
any cache; rows outside S equal the cache exactly.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import sdpa
from .kvcache import kv_assemble


def linear(x, w, bias=None) -> np.ndarray:
    """x W^T (+ bias) in float64; x [..., K], w [N, K], bias [N]."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


def gelu_tanh(x) -> np.ndarray:
    """The tanh form of GELU, elementwise in float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def _qkv(x, weights, H):
    """Q, K, V as [B, n, H, d] from x [B, n, C]."""
    B, n, C = x.shape
    qkv = linear(x, weights["w_qkv"])
    d = C // H
    return tuple(qkv[..., i * C:(i + 1) * C].reshape(B, n, H, d) for i in range(3))


def _tail(x, a, weights):
    """Residual, output projection and MLP of the rows of x given their attention a [B, n, C]."""
    y = x + linear(a, weights["w_o"])
    return y + linear(gelu_tanh(linear(y, weights["w1"], weights["b1"])), weights["w2"], weights["b2"])


def block_dense(x, weights, H: int):
    """The dense block (anchor step, Eq. 18): returns (Z [B, N, C], K, V [B, N, H, d])."""
    x = np.asarray(x, dtype=np.float64)
    B, N, C = x.shape
    q, k, v = _qkv(x, weights, H)
    a, _ = sdpa(q, k, v)
    return _tail(x, a.reshape(B, N, C), weights), k, v


def block_srsu(x, idx, z_cache, k_cache, v_cache, weights, H: int):
    """The row-selective block (Eq. 15-16) for the ascending token lists idx [B, k]:
    only the rows of S are computed from the current state x [B, N, C]; their keys and
    values replace the cached ones (Eq. 16), their outputs replace the cached outputs,
    and every other output row is the cached one.  Returns (Z, K_glob, V_glob)."""
    x = np.asarray(x, dtype=np.float64)
    B, N, C = x.shape
    idx = np.asarray(idx, dtype=np.int64)
    if idx.ndim == 1:
        idx = np.broadcast_to(idx, (B, idx.shape[0]))
    x_s = np.stack([x[b, idx[b]] for b in range(B)])            # [B, k, C]
    q_s, k_s, v_s = _qkv(x_s, weights, H)
    k_glob = kv_assemble(k_s, idx, np.asarray(k_cache, dtype=np.float64))
    v_glob = kv_assemble(v_s, idx, np.asarray(v_cache, dtype=np.float64))
    a_s, _ = sdpa(q_s, k_glob, v_glob)                          # Eq. 16: rows of S, all keys
    z_s = _tail(x_s, a_s.reshape(B, -1, C), weights)
    z = np.array(z_cache, dtype=np.float64, copy=True)          # context rows copied from the cache
    for b in range(B):
        z[b, idx[b]] = z_s[b]
    return z, k_glob, v_glob
