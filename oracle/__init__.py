"""fp64 CPU oracle of the SAFE-DiT attention hot path -- TEST INFRASTRUCTURE ONLY.

Source: "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
Diffusion Transformers" (arXiv 2606.29360), equations cited per function.

This package is plain, slow and meant to be checked by eye against the paper.
It shares no code with the HIP library (`sparse_query_sdpa_amd`) and imports
nothing from it.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import it; the product path never does.

Parts:
  mask.py      Eq. 5-8: row classes of a (broadcast) mask, the removable class R,
               the Eq. 8 rewrite decision, key-padding lengths.
  attention.py Eq. 2, 16, 17: SDPA in float64 with optional gathered query rows,
               per-sample valid key lengths and an optional explicit mask.
  pcsp.py      Eq. 9-12: image->text probability aggregation, Gaussian smoothing
               on the latent grid, min-max normalisation, top-k selection.
  kvcache.py   Eq. 14, 16, 19: global K/V assembly in original token order and
               the anchor refresh of the context cache.
  guidance.py  Eq. 20, 21: sensitivity-weighted classifier-free guidance and its
               binary variant.
  block.py     Eq. 15-16, 18: the row-selective block around attention (a plain
               stand-in block with synthetic weights) and its dense form.

Pinning status (what fixes each function other than itself) is listed in the
module docstrings; every function is pinned by the CPU tests in
tests/test_oracle_*.py.  Parity unpinned: none of the functions lacks a pin,
but no page prints a numeric worked example, so absolute values are pinned by
closed forms, library routines and brute force only.
"""
from .attention import sdpa, sdpa_bruteforce, lse_from_logits
from .mask import (ALL_VALID, ZERO, ROW_CONST, KEY_PADDING, NONCONST, BLOCKED, NONFINITE,
                   REMOVABLE, CLASS_NAMES, classify_row, classify_rows, classify_mask,
                   MaskVerdict, safe_sdpa, removable_row_witness)
from .pcsp import (pcsp_accumulate, gaussian_taps, gaussian_smooth, minmax_normalize,
                   topk_select, pcsp_scores)
from .kvcache import kv_assemble, car_refresh
from .guidance import guidance_scales, binary_scales, sw_cfg
from .block import linear, gelu_tanh, block_dense, block_srsu

__all__ = [
    "sdpa", "sdpa_bruteforce", "lse_from_logits",
    "ALL_VALID", "ZERO", "ROW_CONST", "KEY_PADDING", "NONCONST", "BLOCKED", "NONFINITE",
    "REMOVABLE", "CLASS_NAMES", "classify_row", "classify_rows", "classify_mask", "MaskVerdict",
    "safe_sdpa", "removable_row_witness",
    "guidance_scales", "binary_scales", "sw_cfg",
    "pcsp_accumulate", "gaussian_taps", "gaussian_smooth", "minmax_normalize", "topk_select",
    "pcsp_scores", "kv_assemble", "car_refresh",
    "linear", "gelu_tanh", "block_dense", "block_srsu",
]
