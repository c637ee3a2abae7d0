"""Prompt-Conditioned Sensitivity Partitioning (PCSP) -- test infrastructure only.

Follows "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
Diffusion Transformers":
  * Eq. 9  A_{t,l,h} in [0,1]^{N x M}: image-query -> text-key probabilities
    after the model's own masking and normalisation (softmax over the valid
    text keys);
  * Eq. 10 s~_i = mean over warm-up steps, layers and heads of
    sum_{j in T} w_j A[i, j], with w_j >= 0, sum w_j = 1 over content tokens,
    zero weight on padding;
  * Eq. 11 s = Norm(G_sigma * s~) on the latent grid;
  * Eq. 12 S = TopK(s, k) with k = ceil(rho N); C is the complement.

Readings where the paper is silent or loose:
  * text padding is a suffix: keys j >= kv_len[b] are padding; the content
    weights w are an input (zero on padding and on special tokens, summing to
    one over content tokens).  With uniform weights over every valid key the
    score would be the same constant for every image token (each row of A sums
    to one over the valid keys), so the special-token zeros are what make the
    field informative;
  * the 1/(|W||L||H|) factor of Eq. 10 is left to the caller: it is a
    positive constant, so it changes neither the smoothed field's order nor
    the min-max normalised field;
  * G_sigma is a truncated Gaussian g(t) = exp(-t^2 / (2 sigma^2)) for
    |t| <= ceil(3 sigma), applied along grid rows then grid columns on the
    row-major raster (token i = row * grid_w + col); at the borders the taps
    that fall inside the grid are renormalised to sum to one; sigma = 0 is the
    identity;
  * Norm is min-max scaling to [0, 1]; a constant field maps to 0;
  * TopK ranks by score descending, ties to the lower token index, -0 == +0,
    NaN below every number; the selected indices are returned ascending (the
    "original token order" of Eq. 16).  Min-max scaling is increasing, so the
    selection is taken on G_sigma * s~ directly (rounding in the scaled field
    could only create ties).

Pins (tests/test_oracle_pcsp.py): torch softmax / scipy convolution library
routines, closed forms (one valid key -> A = 1; zero queries -> uniform A; a
constant field stays constant; a unit impulse reproduces the normalised taps),
direct 2-D convolution with 2-D renormalisation, brute-force O(N^2) ranking.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def pcsp_accumulate(q_c, k_txt, kv_len, w, heads=None, scale: Optional[float] = None,
                    acc: Optional[np.ndarray] = None) -> np.ndarray:
    """acc[b, i] += sum_{h in heads} sum_{j < kv_len[b]} w[b, j] * A_h[i, j]  (Eq. 9, 10).

    q_c: [B, N, H, d] image queries of the cross-attention; k_txt: [B, M, H, d]
    text keys; kv_len: [B]; w: [B, M] content weights (entries at j >= kv_len
    are ignored); heads: iterable of head indices or None (all heads).
    """
    q = np.asarray(q_c, dtype=np.float64)
    kt = np.asarray(k_txt, dtype=np.float64)
    B, N, H, d = q.shape
    M = kt.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if heads is None:
        heads = range(H)
    out = np.zeros((B, N), dtype=np.float64) if acc is None else np.array(acc, dtype=np.float64)
    for b in range(B):
        L = int(kv_len[b])
        if L <= 0:
            continue
        wb = np.asarray(w, dtype=np.float64)[b, :L]
        for h in heads:
            logits = (q[b, :, h, :] @ kt[b, :L, h, :].T) * scale     # [N, L]
            logits = logits - logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            A = p / p.sum(axis=1, keepdims=True)                      # Eq. 9 rows
            out[b] += A @ wb                                          # Eq. 10 inner sum
    return out


def gaussian_taps(sigma: float) -> np.ndarray:
    """Unnormalised taps exp(-t^2 / (2 sigma^2)) for t = -r..r, r = ceil(3 sigma)."""
    r = int(math.ceil(3.0 * sigma))
    t = np.arange(-r, r + 1, dtype=np.float64)
    return np.exp(-(t * t) / (2.0 * sigma * sigma))


def _smooth_axis(x: np.ndarray, taps: np.ndarray, axis: int) -> np.ndarray:
    r = (taps.size - 1) // 2
    n = x.shape[axis]
    out = np.zeros_like(x)
    norm = np.zeros(n)
    xs = np.moveaxis(x, axis, -1)
    os_ = np.moveaxis(out, axis, -1)
    for pos in range(n):
        acc = np.zeros(xs.shape[:-1])
        wsum = 0.0
        for t in range(-r, r + 1):
            src = pos + t
            if 0 <= src < n:
                acc = acc + taps[t + r] * xs[..., src]
                wsum += taps[t + r]
        os_[..., pos] = acc / wsum
        norm[pos] = wsum
    return out


def gaussian_smooth(s_tilde, grid_h: int, grid_w: int, sigma: float) -> np.ndarray:
    """G_sigma * s~ on the row-major grid, border-renormalised (Eq. 11).  [B, N] -> [B, N]."""
    s = np.asarray(s_tilde, dtype=np.float64)
    B, N = s.shape
    if N != grid_h * grid_w:
        raise ValueError("N must equal grid_h * grid_w")
    if sigma == 0.0:
        return s.copy()
    taps = gaussian_taps(sigma)
    g = s.reshape(B, grid_h, grid_w)
    g = _smooth_axis(g, taps, axis=2)   # along each grid row
    g = _smooth_axis(g, taps, axis=1)   # along each grid column
    return g.reshape(B, N)


def minmax_normalize(s_bar) -> np.ndarray:
    """Norm(.) of Eq. 11: per-sample (x - min) / (max - min); a constant field -> 0."""
    s = np.asarray(s_bar, dtype=np.float64)
    lo = s.min(axis=1, keepdims=True)
    hi = s.max(axis=1, keepdims=True)
    span = hi - lo
    return np.where(span > 0, (s - lo) / np.where(span > 0, span, 1.0), 0.0)


def _rank_key(value: float, index: int):
    if value != value:             # NaN: below every number
        return (1, 0.0, index)
    return (0, -value, index)      # -0.0 == 0.0 compare equal -> tie to lower index


def topk_select(s, k: int) -> np.ndarray:
    """Eq. 12 per sample: the k best-ranked token indices, returned ascending.  [B, N] -> int32 [B, k]."""
    s = np.asarray(s)
    B, N = s.shape
    if not (0 <= k <= N):
        raise ValueError("k must be in [0, N]")
    out = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        row = [float(x) for x in s[b]]
        order = sorted(range(N), key=lambda i: _rank_key(row[i], i))
        out[b] = np.sort(np.asarray(order[:k], dtype=np.int64)).astype(np.int32)
    return out


def pcsp_scores(q_c, k_txt, kv_len, w, grid_h: int, grid_w: int, sigma: float, k: int,
                heads=None, scale: Optional[float] = None):
    """One warm-up call through selection: returns (acc, s_bar, s_norm, idx)."""
    acc = pcsp_accumulate(q_c, k_txt, kv_len, w, heads=heads, scale=scale)
    s_bar = gaussian_smooth(acc, grid_h, grid_w, sigma)
    s_norm = minmax_normalize(s_bar)
    idx = topk_select(s_bar, k)
    return acc, s_bar, s_norm, idx
