"""Seeded synthetic inputs for the SAFE-DiT attention hot path.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It holds only random draws, the round-to-nearest-even encoding of
float32 draws into bfloat16 bit patterns, and the workload shapes.  It holds
none of the method's arithmetic (no softmax, no classification, no selection).

Shapes follow the paper's setting (SAFE-DiT, "Semantics-Aware Fast-path
Execution for High-Resolution Diffusion Transformers", Eq. 1-4): image tokens
N on a grid_h x grid_w latent raster, M text tokens, H heads of size d.
Tensors are token-major [B, N, H, d] with d contiguous.

Recipe (stated once, used everywhere): activations N(0, 1) drawn in float32
with torch's CPU generator (Mersenne Twister, thread-count independent) seeded
from numpy's SeedSequence of (1000 + workload number, tensor id), then rounded
to bfloat16 with round-to-nearest-even; per-sample valid text lengths, sensitive
row sets and masks from numpy PCG64 seeded with 1000 + workload number (plus a
per-purpose stream offset); the drift between steps N(0, 0.05) drawn like the
activations (0.05 is a standard deviation).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


# ----------------------------------------------------------------------------
# bfloat16 encoding (storage format only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Finite inputs only (the generators never draw NaN/inf; mask cases that need
    them write the bit patterns directly).  In 32-bit arithmetic the sum cannot
    wrap for finite values (the largest, 0xFF7FFFFF, plus 0x8000 < 2^32).
    """
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.zeros(b.shape + (2,), dtype=np.uint16)   # little-endian: high half holds the bf16 bits
    out[..., 1] = b
    return out.view(np.float32).reshape(b.shape)


BF16_NEG_INF = np.uint16(0xFF80)
BF16_POS_INF = np.uint16(0x7F80)
BF16_NAN = np.uint16(0x7FC0)
BF16_NEG_ZERO = np.uint16(0x8000)


# ----------------------------------------------------------------------------
# workload shapes
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    H: int
    d: int
    grid_h: int
    grid_w: int
    M: int
    rho_percent: tuple          # sensitive fractions, in percent
    kv_len_fixed: Optional[int]  # None -> per-sample U{32..M}
    f32_inputs: bool            # activations handed over as fp32 draws rounded to bf16

    @property
    def N(self) -> int:
        return self.grid_h * self.grid_w

    def k_for(self, rho_percent: int) -> int:
        """k = ceil(rho * N) in integer arithmetic (rho given in percent)."""
        return -(-rho_percent * self.N // 100)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny-16x16", 1, 2, 32, 16, 16, 16, (25,), 11, True),
    2: Workload(2, "1024sq-64x64", 2, 24, 96, 64, 64, 256, (30,), None, False),
    3: Workload(3, "2048sq-128x128", 2, 24, 96, 128, 128, 256, (25,), None, False),
    4: Workload(4, "2560sq-160x160", 2, 24, 96, 160, 160, 256, (15, 25, 40), None, False),
    5: Workload(5, "3072sq-192x192", 2, 24, 96, 192, 192, 256, (25,), None, False),
}


def rng_for(number: int, stream: int = 0) -> np.random.Generator:
    """Seeded generator for a workload (seed 1000 + number; extra streams offset)."""
    return np.random.Generator(np.random.PCG64(1000 + number + 7919 * stream))


# ----------------------------------------------------------------------------
# activations
# ----------------------------------------------------------------------------

class Bf16Tensor:
    """A bfloat16 tensor: the bit pattern handed to the GPU and its exact value.

    `bits` is uint16; `value` (float32, exactly the bf16 value of `bits`) is
    widened on first use.
    """

    def __init__(self, bits: np.ndarray, value: Optional[np.ndarray] = None):
        self.bits = bits
        self._value = value

    @property
    def value(self) -> np.ndarray:
        if self._value is None:
            self._value = bf16_bits_to_f32(self.bits)
        return self._value

    @property
    def shape(self):
        return self.bits.shape


def _seed_of(key) -> int:
    """A 63-bit seed derived from a tuple of ints."""
    return int(np.random.SeedSequence(list(key)).generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def normal_f32(key, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draws of `shape`, deterministic in `key` (a tuple of ints).

    Drawn with torch's CPU generator (Mersenne Twister, seeded from `key`),
    whose output does not depend on the number of threads.
    """
    import torch
    g = torch.Generator().manual_seed(_seed_of(key))
    x = torch.randn(int(np.prod(shape)), generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.numpy().reshape(shape)


def _to_bf16_parallel(x: np.ndarray) -> Bf16Tensor:
    """Round to bfloat16 (nearest even) with torch's cast: identical to f32_to_bf16_bits, faster."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    bits = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return Bf16Tensor(bits)


def bf16_normal(key, shape, std: float = 1.0) -> Bf16Tensor:
    """bf16 tensor of N(0, std^2) draws (rounded to nearest even), deterministic in `key`."""
    return _to_bf16_parallel(normal_f32(key, shape, std))


def bf16_from_f32(x: np.ndarray) -> Bf16Tensor:
    return _to_bf16_parallel(np.ascontiguousarray(x, dtype=np.float32))


def attention_inputs(B: int, Nq: int, Nk: int, H: int, d: int, seed: int, std: float = 1.0):
    """q [B,Nq,H,d], k and v [B,Nk,H,d]: bf16 N(0, std^2)."""
    q = bf16_normal((seed, 0), (B, Nq, H, d), std)
    k = bf16_normal((seed, 1), (B, Nk, H, d), std)
    v = bf16_normal((seed, 2), (B, Nk, H, d), std)
    return q, k, v


def random_rows(rng: np.random.Generator, N: int, k: int) -> np.ndarray:
    """k distinct token indices in [0, N), ascending, int32."""
    return np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32)


def text_lengths(rng: np.random.Generator, B: int, M: int, lo: int = 32) -> np.ndarray:
    """Per-sample valid text lengths ~ U{lo..M}, int32."""
    return rng.integers(lo, M + 1, size=B, dtype=np.int64).astype(np.int32)


def workload_inputs(number: int) -> dict:
    """All activations of one workload, drawn in a fixed order.

    Tensor keys (1000 + number, i) for i = 0..5 in the order q_x, k_x, v_x,
    q_c, k_txt, v_txt; the per-sample text lengths come from rng_for(number).
    """
    w = WORKLOADS[number]
    rng = rng_for(number)
    B, N, H, d, M = w.B, w.N, w.H, w.d, w.M
    base = 1000 + number
    out = {"workload": w}
    out["q_x"] = bf16_normal((base, 0), (B, N, H, d))
    out["k_x"] = bf16_normal((base, 1), (B, N, H, d))
    out["v_x"] = bf16_normal((base, 2), (B, N, H, d))
    out["q_c"] = bf16_normal((base, 3), (B, N, H, d))
    out["k_txt"] = bf16_normal((base, 4), (B, M, H, d))
    out["v_txt"] = bf16_normal((base, 5), (B, M, H, d))
    if w.kv_len_fixed is not None:
        out["kv_len"] = np.full((B,), w.kv_len_fixed, dtype=np.int32)
    else:
        out["kv_len"] = text_lengths(rng, B, M)
    return out


def drift(key, shape, std: float = 0.05) -> np.ndarray:
    """float32 N(0, std^2) drift added to cached activations between steps (deterministic in key)."""
    return normal_f32(key, shape, std)


# ----------------------------------------------------------------------------
# masks for the row-constant classifier (bool as uint8, additive as bf16 bits
# or float32 values)
# ----------------------------------------------------------------------------

def mask_all_valid_bool(Nq: int, Nk: int) -> np.ndarray:
    return np.ones((1, 1, Nq, Nk), dtype=np.uint8)


def mask_zero_additive_f32(Nq: int, Nk: int) -> np.ndarray:
    return np.zeros((1, 1, Nq, Nk), dtype=np.float32)


def mask_row_constant_f32(rng: np.random.Generator, Nq: int, Nk: int, lo: float, hi: float) -> np.ndarray:
    c = rng.uniform(lo, hi, size=(Nq, 1)).astype(np.float32)
    return np.broadcast_to(c, (Nq, Nk)).reshape(1, 1, Nq, Nk).copy()


def row_constants_f32(rng: np.random.Generator, Nq: int, lo: float, hi: float) -> np.ndarray:
    """The per-row constants c_i of a row-constant mask (for building big masks on device)."""
    return rng.uniform(lo, hi, size=(Nq,)).astype(np.float32)


def mask_random_additive_f32(rng: np.random.Generator, Nq: int, Nk: int) -> np.ndarray:
    return rng.standard_normal(size=(1, 1, Nq, Nk), dtype=np.float32)


def mask_text_padding_f32(Nq: int, Nk: int, valid: int) -> np.ndarray:
    m = np.zeros((1, 1, Nq, Nk), dtype=np.float32)
    m[..., valid:] = -np.inf
    return m


def c1_mask_cases(seed_number: int = 1) -> dict:
    """The five classifier cases of the tiny workload (16x16 grid, 16 text keys, 11 valid)."""
    rng = rng_for(seed_number, stream=1)
    N, M = 256, 16
    return {
        "all_valid_bool": mask_all_valid_bool(N, N),
        "zero_additive": mask_zero_additive_f32(N, N),
        "row_constant": mask_row_constant_f32(rng, N, N, -5.0, 5.0),
        "random_additive": mask_random_additive_f32(rng, N, N),
        "text_padding": mask_text_padding_f32(N, M, 11),
    }


def pcsp_content_weights(kv_len: np.ndarray, M: int, n_special: int = 1) -> np.ndarray:
    """Synthetic content weights [B, M] float32.

    The first `n_special` text tokens stand for special (start) tokens and the
    tokens at j >= kv_len[b] are padding: both get weight 0.  The remaining
    content tokens share weight uniformly (sum 1).  A sample with no content
    token gets all-zero weights.
    """
    B = kv_len.shape[0]
    w = np.zeros((B, M), dtype=np.float32)
    for b in range(B):
        L = int(kv_len[b])
        n = L - n_special
        if n > 0:
            w[b, n_special:L] = np.float32(1.0) / np.float32(n)
    return w


def score_field(rng: np.random.Generator, B: int, N: int, levels: Optional[int] = None) -> np.ndarray:
    """float32 score vectors [B, N]; optionally quantised to `levels` values to force ties."""
    s = rng.random(size=(B, N), dtype=np.float32)
    if levels is not None:
        s = (np.floor(s * levels) / levels).astype(np.float32)
    return s


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("annotations", "dataclasses", "math", "np")]


# ----------------------------------------------------------------------------
# synthetic block weights (the row-selective block around attention)
# ----------------------------------------------------------------------------

def block_weights(C: int, F: int, seed: int) -> dict:
    """Random bf16 weights of the stand-in block: Wqkv [3C, C], Wo [C, C], W1 [F, C],
    W2 [C, F] drawn N(0, 1/fan_in) (unit-variance activations stay unit-variance), and
    fp32 biases b1 [F], b2 [C] drawn N(0, 0.1^2).  Weights are [out, in] with the input
    channels contiguous."""
    def w(i, shape):
        return bf16_normal((seed, i), shape, std=1.0 / np.sqrt(shape[1]))
    return {"w_qkv": w(0, (3 * C, C)), "w_o": w(1, (C, C)), "w1": w(2, (F, C)), "w2": w(3, (C, F)),
            "b1": normal_f32((seed, 4), (F,), std=0.1), "b2": normal_f32((seed, 5), (C,), std=0.1)}
