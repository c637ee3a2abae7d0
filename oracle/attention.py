"""Scaled dot-product attention in float64 -- test infrastructure only.

Follows "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
Diffusion Transformers":
  * Eq. 2  SDPA(Q,K,V,m) = Softmax(Q K^T / sqrt(d_h) + m) V, with m = empty
    meaning a zero additive bias;
  * Eq. 5  the per-row masked distribution pi_i(m; L) = Softmax(L_i + m_i);
  * Eq. 16 SRSU self-attention: only the query rows of S are evaluated, every
    key stays visible;
  * Eq. 17 SRSU cross-attention: the same row reduction, with the text padding
    mask kept.  The padding mask is carried as a per-sample count of valid
    leading keys (suffix padding), i.e. keys j >= kv_len[b] get bias -inf.

Layout: token-major [B, N, H, d].  Readings where the paper is silent:
  * a row whose keys are all blocked (kv_len 0, or an all -inf mask row) has
    no distribution; its output is 0 and its log-sum-exp is -inf;
  * LSE is the natural-log log-sum-exp of the scaled, masked logits.

Pins (tests/test_oracle_attention.py): torch's float64 CPU
scaled_dot_product_attention (a library routine), closed forms (identical keys
-> mean of values, constant values, a single valid key, zero logits -> uniform
average, a dominant logit), the Eq. 7 shift invariance, and S = all rows
reproducing the dense result.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def sdpa(q, k, v, scale: Optional[float] = None, q_rows=None, kv_len=None,
         mask=None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention outputs for the selected query rows (Eq. 2, 16, 17).

    q: [B, Nq, H, d]; k, v: [B, Nk, H, d] (any float dtype, used in float64).
    scale: logit scale; None means 1/sqrt(d) (Eq. 2).
    q_rows: None (all Nq rows, in order), a 1-D array shared by every sample,
        or a [B, n] array; row r of the output is query q_rows[.., r].
    kv_len: None (all Nk keys) or [B] counts of valid leading keys.
    mask: None or an additive mask broadcastable to [B, H, Nq, Nk]
        (entries may be -inf); indexed by the original query row.
    Returns (O [B, n, H, d] float64, LSE [B, H, n] float64).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q_rows is None:
        rows = np.broadcast_to(np.arange(Nq), (B, Nq))
    else:
        rows = np.asarray(q_rows, dtype=np.int64)
        if rows.ndim == 1:
            rows = np.broadcast_to(rows, (B, rows.shape[0]))
    n = rows.shape[1]
    if kv_len is None:
        lengths = np.full((B,), Nk, dtype=np.int64)
    else:
        lengths = np.asarray(kv_len, dtype=np.int64)
    if mask is not None:
        mask = np.broadcast_to(_as_f64(mask), (B, H, Nq, Nk))

    out = np.zeros((B, n, H, d), dtype=np.float64)
    lse = np.full((B, H, n), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(lengths[b])
        if L <= 0 or n == 0:
            continue
        r = rows[b]
        for h in range(H):
            qs = q[b, r, h, :]                      # [n, d]  (Eq. 13 row selection)
            kk = k[b, :L, h, :]                     # [L, d]
            vv = v[b, :L, h, :]
            logits = (qs @ kk.T) * scale            # [n, L]
            if mask is not None:
                logits = logits + mask[b, h][r][:, :L]
            m = np.max(logits, axis=1, keepdims=True)
            finite = np.isfinite(m[:, 0])
            m_safe = np.where(np.isfinite(m), m, 0.0)
            p = np.exp(logits - m_safe)             # exp(-inf) = 0 for blocked keys
            denom = np.sum(p, axis=1)
            o = (p @ vv) / np.where(denom > 0, denom, 1.0)[:, None]
            o[~finite] = 0.0
            out[b, :, h, :] = o
            with np.errstate(divide="ignore"):
                lse[b, h, :] = np.where(finite, m_safe[:, 0] + np.log(np.where(denom > 0, denom, 1.0)), -np.inf)
    return out, lse


def lse_from_logits(logits) -> float:
    """log(sum(exp(x))) of a 1-D float64 array, stable; -inf for an empty or all -inf row."""
    x = _as_f64(logits)
    if x.size == 0:
        return -math.inf
    m = float(np.max(x))
    if not math.isfinite(m):
        return m
    return m + math.log(float(np.sum(np.exp(x - m))))


def sdpa_bruteforce(q, k, v, scale: Optional[float] = None, q_rows=None, kv_len=None):
    """Pure-Python loop version of `sdpa` for tiny inputs (math.exp, math.fsum).

    Returns nested lists O[b][r][h][c] and LSE[b][h][r] as Python floats.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lses = [], []
    for b in range(B):
        if q_rows is None:
            rows = list(range(Nq))
        else:
            qr = np.asarray(q_rows)
            rows = [int(x) for x in (qr[b] if qr.ndim == 2 else qr)]
        L = Nk if kv_len is None else int(kv_len[b])
        ob = [[[0.0] * d for _ in range(H)] for _ in rows]
        lb = [[-math.inf] * len(rows) for _ in range(H)]
        for ri, i in enumerate(rows):
            for h in range(H):
                if L <= 0:
                    continue
                logit = [math.fsum(float(q[b, i, h, c]) * float(k[b, j, h, c]) for c in range(d)) * scale
                         for j in range(L)]
                mx = max(logit)
                w = [math.exp(x - mx) for x in logit]
                den = math.fsum(w)
                for c in range(d):
                    ob[ri][h][c] = math.fsum(w[j] * float(v[b, j, h, c]) for j in range(L)) / den
                lb[h][ri] = mx + math.log(den)
        out.append(ob)
        lses.append(lb)
    return out, lses
