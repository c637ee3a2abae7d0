"""Row-constant mask classification and the exact rewrite -- test infrastructure only.

Follows "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
Diffusion Transformers":
  * Eq. 5  pi_i(m; L) = Softmax(L_i + m_i);
  * Eq. 6  the removable class R: every mask row is one real constant c_i;
  * the broadcast rule after Eq. 6: the criterion is applied to every
    (broadcast) query row of a batched or head-specific mask;
  * Eq. 7  Softmax(L_i + c_i 1) = Softmax(L_i), and its converse: a
    non-constant row changes the distribution for some logits; all-valid
    Boolean and all-zero additive masks are special cases of R; finite
    non-uniform biases and masks with blocked positions are kept;
  * Eq. 8  SAFE-SDPA(Q,K,V,m) = SDPA(Q,K,V,empty) when m is in R, otherwise the
    original call.  The case body of Eq. 8 is lost in the page text; this
    reading is the one the surrounding prose states.

Row classes (codes ordered by precedence, so the overall class of a mask is
the maximum row code):
  0 ALL_VALID   Boolean row, every entry nonzero (nonzero = attend)
  1 ZERO        additive row, every entry == 0 (IEEE: -0 == +0)
  2 ROW_CONST   additive row, all entries finite and equal, not zero
  3 KEY_PADDING entries [0, L) valid and (additive) equal to each other,
                entries [L, Nk) blocked (-inf / False), 1 <= L < Nk
  4 NONCONST    additive row, all finite, not all equal
  5 BLOCKED     any other row with a blocked entry (includes L = 0)
  6 NONFINITE   any NaN or +inf entry
Classes 0-2 form R.  A mask whose overall class is KEY_PADDING is reported as
such only when, within each stored batch index, every row has the same valid
length (rows in R count as length Nk); the length is then the per-sample key
length of Eq. 17.  Otherwise the overall class is BLOCKED.  Readings where the
paper is silent: Boolean polarity (nonzero = attend), right (suffix) padding of
text keys, -inf rows are not in R (c_i must be real), NaN/+inf never removable,
an empty row (Nk = 0) is vacuously in R.

Pins (tests/test_oracle_mask.py): hand-labelled golden masks
(tests/golden/mask_cases.json), a scalar per-row definition against the
vectorised one, the Eq. 7 invariance of `oracle.sdpa` under every R row, and the
converse witness: every row flagged non-removable gives softmax(m_i) different
from the uniform distribution at zero logits.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .attention import sdpa

ALL_VALID, ZERO, ROW_CONST, KEY_PADDING, NONCONST, BLOCKED, NONFINITE = range(7)
REMOVABLE = (ALL_VALID, ZERO, ROW_CONST)
CLASS_NAMES = ("ALL_VALID", "ZERO", "ROW_CONST", "KEY_PADDING", "NONCONST", "BLOCKED", "NONFINITE")


def classify_row(row, is_bool: bool):
    """Class and valid length of one stored mask row (plain loop form).

    Returns (class_code, L): L is the row length for rows in R, the valid
    prefix length for KEY_PADDING rows and -1 otherwise.
    """
    vals = [float(x) for x in np.asarray(row).ravel()]
    n = len(vals)
    if n == 0:
        return (ALL_VALID if is_bool else ZERO), 0
    if is_bool:
        valid = [x != 0.0 for x in vals]
        if all(valid):
            return ALL_VALID, n
        L = valid.index(False)
        if L >= 1 and not any(valid[L:]):
            return KEY_PADDING, L
        return BLOCKED, -1
    if any(x != x or x == float("inf") for x in vals):
        return NONFINITE, -1
    blocked = [x == float("-inf") for x in vals]
    if any(blocked):
        L = blocked.index(True)
        if L >= 1 and all(blocked[L:]) and all(x == vals[0] for x in vals[:L]):
            return KEY_PADDING, L
        return BLOCKED, -1
    if all(x == vals[0] for x in vals):
        return (ZERO if vals[0] == 0.0 else ROW_CONST), n
    return NONCONST, -1


def classify_rows(rows: np.ndarray, is_bool: bool):
    """Vectorised `classify_row` over a [R, n] array of stored rows.

    Returns (classes uint8 [R], lengths int64 [R]).
    """
    x = np.asarray(rows)
    R, n = x.shape
    cls = np.empty(R, dtype=np.uint8)
    lens = np.full(R, -1, dtype=np.int64)
    if n == 0:
        cls[:] = ALL_VALID if is_bool else ZERO
        lens[:] = 0
        return cls, lens
    if is_bool:
        valid = x != 0
        blocked = ~valid
        nonfinite = np.zeros(R, dtype=bool)
        eq = np.ones(R, dtype=bool)
    else:
        x = x.astype(np.float64)
        nonfinite = np.isnan(x).any(axis=1) | (x == np.inf).any(axis=1)
        blocked = x == -np.inf
        # equality of every non-blocked entry to the first entry
        eq = ((x == x[:, :1]) | blocked).all(axis=1)
    anyb = blocked.any(axis=1)
    first_blocked = np.where(anyb, np.argmax(blocked, axis=1), n)
    n_blocked = blocked.sum(axis=1)
    suffix = anyb & (first_blocked >= 1) & (n_blocked == n - first_blocked)

    all_eq = eq & ~anyb
    if is_bool:
        cls[:] = BLOCKED
        cls[~anyb] = ALL_VALID
        lens[~anyb] = n
    else:
        cls[:] = NONCONST
        zero_row = all_eq & (x[:, 0] == 0.0)
        cls[all_eq & ~zero_row] = ROW_CONST
        cls[zero_row] = ZERO
        lens[all_eq] = n
        cls[anyb] = BLOCKED
    pad = suffix & eq
    cls[pad] = KEY_PADDING
    lens[pad] = first_blocked[pad]
    cls[nonfinite] = NONFINITE
    lens[nonfinite] = -1
    return cls, lens


@dataclasses.dataclass
class MaskVerdict:
    verdict: int            # 1 if the mask is in R (removable), else 0
    mask_class: int         # overall class code
    first_bad_row: int      # lowest flat stored row not in R, or -1
    rows: int               # number of stored rows
    row_class: np.ndarray   # uint8 [rows]
    kv_len: np.ndarray      # int32 [Bm]: valid key length per stored batch index, -1 unless KEY_PADDING


def classify_mask(mask: np.ndarray, is_bool: bool, chunk_rows: int = 4096) -> MaskVerdict:
    """Classify a stored mask of shape [Bm, Hm, Nqm, Nkm] (size-1 dims broadcast).

    Rows are the stored (b, h, i) rows in row-major order: the broadcast rule
    after Eq. 6 applies the criterion to every broadcast query row, and a
    broadcast row is the same stored row for every (b, h, i) it serves.
    """
    m = np.asarray(mask)
    if m.ndim != 4:
        raise ValueError("mask must be 4-D [B, H, Nq, Nk] (size-1 dims broadcast)")
    Bm, Hm, Nq, Nk = m.shape
    flat = m.reshape(Bm * Hm * Nq, Nk)
    R = flat.shape[0]
    cls = np.empty(R, dtype=np.uint8)
    lens = np.empty(R, dtype=np.int64)
    for s in range(0, R, chunk_rows):
        c, l = classify_rows(flat[s:s + chunk_rows], is_bool)
        cls[s:s + chunk_rows] = c
        lens[s:s + chunk_rows] = l
    if R == 0:
        overall = ALL_VALID if is_bool else ZERO
    else:
        overall = int(cls.max())
    kv = np.full((Bm,), -1, dtype=np.int32)
    if overall == KEY_PADDING:
        per_b = lens.reshape(Bm, Hm * Nq)
        if np.all(per_b == per_b[:, :1]):
            kv[:] = per_b[:, 0].astype(np.int32)
        else:
            overall = BLOCKED
    bad = np.nonzero(cls > ROW_CONST)[0]
    first_bad = int(bad[0]) if bad.size else -1
    return MaskVerdict(int(overall in REMOVABLE), overall, first_bad, R, cls, kv)


def to_additive(mask: np.ndarray, is_bool: bool) -> np.ndarray:
    """Boolean masks become additive biases: attend -> 0, blocked -> -inf."""
    if is_bool:
        return np.where(np.asarray(mask) != 0, 0.0, -np.inf)
    return np.asarray(mask, dtype=np.float64)


def safe_sdpa(q, k, v, mask: Optional[np.ndarray], is_bool: bool = False, scale: Optional[float] = None):
    """The Eq. 8 rewrite in oracle form.

    Removable masks (class R) are dropped and SDPA runs with no mask; a
    key-padding mask is replaced by per-sample valid key lengths (the text
    padding semantics of Eq. 4/17 are kept); anything else runs with the
    original mask.  Returns (O, LSE, MaskVerdict or None, path) where path is
    'none', 'kv_len' or 'mask'.
    """
    if mask is None:
        o, lse = sdpa(q, k, v, scale)
        return o, lse, None, "none"
    verdict = classify_mask(mask, is_bool)
    if verdict.verdict:
        o, lse = sdpa(q, k, v, scale)
        return o, lse, verdict, "none"
    if verdict.mask_class == KEY_PADDING:
        B = np.asarray(q).shape[0]
        kv = np.broadcast_to(verdict.kv_len, (B,))
        o, lse = sdpa(q, k, v, scale, kv_len=kv)
        return o, lse, verdict, "kv_len"
    o, lse = sdpa(q, k, v, scale, mask=to_additive(mask, is_bool))
    return o, lse, verdict, "mask"


def removable_row_witness(row, is_bool: bool) -> float:
    """Distance between pi(m; L=0) and pi(empty; L=0) for one mask row (Eq. 5, 7).

    For a row in R the masked distribution at zero logits is exactly uniform,
    so the result is 0.  For a row outside R the result is positive (or NaN
    when the row holds NaN/+inf): the converse statement after Eq. 7.
    """
    add = to_additive(np.asarray(row).ravel(), is_bool)
    n = add.size
    if n == 0:
        return 0.0
    mx = np.max(add)
    if not np.isfinite(mx):
        return float("nan") if np.isnan(mx) or mx == np.inf else 1.0
    p = np.exp(add - mx)
    p = p / p.sum()
    return float(np.max(np.abs(p - 1.0 / n)))
