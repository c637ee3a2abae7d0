"""Sensitivity-weighted classifier-free guidance (SW-CFG) -- test infrastructure only.

Follows "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
Diffusion Transformers", Section "Sensitivity-Weighted CFG":
  * Eq. 20 the per-token guidance scale interpolates between the context scale and
    the sensitive-region scale by the normalised sensitivity score s_i of Eq. 11;
  * Eq. 21 the guided prediction moves from the unconditional prediction towards the
    conditional one by that per-token scale;
  * the binary variant gives the sensitive scale to the tokens of S and the context
    scale to the rest; equal scales are ordinary (global) classifier-free guidance.

Reading: a prediction is a token-major [B, N, C] array (C values per latent token,
for example the p x p x latent-channel block a patch embeds), and each of the B
images carries its own score row s[b] or index list S[b].

Pins (tests/test_oracle_guidance.py): equal scales against torch.lerp (the library's
linear interpolation), scale 1 and 0 giving exactly the conditional and the
unconditional prediction, the binary variant against the continuous one with an
indicator score, affinity in the scale, and a worked example computed by hand
(tests/golden/sw_cfg_hand.json).
"""
from __future__ import annotations

import numpy as np


def guidance_scales(s, g_ctx: float, g_sens: float) -> np.ndarray:
    """Eq. 20: gamma_i = g_ctx + (g_sens - g_ctx) * s_i, per image and token (s: [B, N])."""
    s = np.asarray(s, dtype=np.float64)
    return g_ctx + (g_sens - g_ctx) * s


def binary_scales(idx, B: int, N: int, g_ctx: float, g_sens: float) -> np.ndarray:
    """The binary variant: g_sens on the tokens of S (idx: [k] shared or [B, k]), g_ctx elsewhere."""
    gamma = np.full((B, N), float(g_ctx))
    idx = np.asarray(idx, dtype=np.int64)
    if idx.ndim == 1:
        idx = np.broadcast_to(idx, (B, idx.shape[0]))
    for b in range(B):
        gamma[b, idx[b]] = g_sens
    return gamma


def sw_cfg(f_c, f_u, gamma) -> np.ndarray:
    """Eq. 21: f_hat[b, i, :] = f_u[b, i, :] + gamma[b, i] * (f_c[b, i, :] - f_u[b, i, :]), in float64.

    f_c, f_u: [B, N, C] conditional and unconditional predictions; gamma: [B, N].
    """
    f_c = np.asarray(f_c, dtype=np.float64)
    f_u = np.asarray(f_u, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    return f_u + gamma[:, :, None] * (f_c - f_u)
