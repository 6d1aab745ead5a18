"""Plain fp64 CPU oracle for the draft-head projection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it exists so that tests, the smoke check and the CPU
baseline leg of the benchmark can check the HIP library against a slow,
obviously correct reading of the method.  It shares no code with the HIP path.

What is computed, and where it is defined:

* The draft head scores a hidden state of width K against LM-head rows, and
  the greedy draft is the highest-scoring row ("What I was testing" on
  krisbailey.com/articles/shortlist-mtp; greedy decoding at temperature zero in
  "Re-running the comparison fairly" there).
* A shortlisted head is the full head's weight restricted to a list of ids,
  cut at load time ("Two ways to run it" on zone-1.cobraproject.com "Masked
  MTP drafts"); a shortlisted draft can only propose ids on the list
  ("Masked MTP drafts", same page).
* The index of the winning shortlist row maps back to a vocabulary id through
  a d2t table, as in EAGLE-3's draft-to-target mapping ("Two ways to run it",
  same page).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* Inputs are bf16 bit patterns; a pattern b decodes exactly as the float32
  with bits b << 16.
* A logit is the raw dot product: no bias, scale, soft cap or temperature.
* Ties go to the smallest row index (first occurrence).
* d2t holds absolute vocabulary ids (d2t[i] = ids[i] for a trimmed head).
* The gap of a row is its best logit minus the best logit of every other
  projected row (+inf when only one row is projected).

Every bf16 x bf16 product is exact in fp64 (8 + 8 significand bits), so the
only rounding is in the fp64 sum, whose error is below K * 2**-53 times the
sum of |products| (about 1e-11 at K = 2,560 for these inputs).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "oracle_trim",
    "oracle_logits",
    "oracle_project_argmax",
    "OracleResult",
]

# Rows of W decoded to fp64 at a time (bounds memory: 8,192 x 2,560 x 8 B).
BLOCK_ROWS = 8192


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    bfloat16 is the top half of an IEEE binary32: shifting the pattern into
    the high 16 bits gives the float32 with the same value."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_trim(w_bits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Shortlisted head: row i of the result is row ids[i] of W, bit for bit.

    The head is cut once at load from a list of ids ("Two ways to run it",
    "Masked MTP drafts" on zone-1.cobraproject.com).  Every id must lie in
    [0, N); the list order is kept (row i <-> ids[i])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    ids = np.asarray(ids)
    if w_bits.ndim != 2 or ids.ndim != 1:
        raise ValueError("W must be [N, K] and ids [S]")
    n = w_bits.shape[0]
    if ids.size and (ids.min() < 0 or ids.max() >= n):
        raise IndexError("shortlist id out of range [0, N)")
    return w_bits[ids.astype(np.int64)].copy()


def oracle_logits(h_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """fp64 logits L[m, r] = sum_k h[m, k] * W[r, k] for all rows r.

    The draft head projects the hidden state onto every head row ("What I
    was testing", krisbailey.com/articles/shortlist-mtp).  W is decoded in
    row blocks so a full 248,320-row head never exists in fp64 at once."""
    h_bits = np.asarray(h_bits, dtype=np.uint16)
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if h_bits.ndim != 2 or w_bits.ndim != 2 or h_bits.shape[1] != w_bits.shape[1]:
        raise ValueError("h must be [M, K] and W [R, K] with the same K")
    h = bf16_bits_to_f64(h_bits)                    # [M, K]
    if not np.all(np.isfinite(h)):
        raise ValueError("non-finite hidden value")
    m, r = h.shape[0], w_bits.shape[0]
    out = np.empty((m, r), dtype=np.float64)
    for r0 in range(0, r, BLOCK_ROWS):
        wb = bf16_bits_to_f64(w_bits[r0:r0 + BLOCK_ROWS])   # [B, K]
        if not np.all(np.isfinite(wb)):
            raise ValueError("non-finite weight value")
        out[:, r0:r0 + wb.shape[0]] = h @ wb.T
    return out


@dataclass
class OracleResult:
    """Per hidden row m: ``id`` the proposed vocabulary id, ``idx`` the
    winning row of the projected matrix, ``logit`` its fp64 logit, ``gap``
    the margin to the best other row, ``abs_sum`` = sum_k |h[m,k] W[idx,k]|
    (the scale of the rounding error of any summation order)."""
    id: np.ndarray
    idx: np.ndarray
    logit: np.ndarray
    gap: np.ndarray
    abs_sum: np.ndarray
    logits: np.ndarray | None = None


def oracle_project_argmax(h_bits: np.ndarray, w_bits: np.ndarray,
                          d2t: np.ndarray | None = None,
                          keep_logits: bool = False) -> OracleResult:
    """Greedy draft over the projected rows, mapped through d2t.

    For each hidden row m: idx = the first r with L[m, r] equal to the row
    maximum; id = d2t[idx] (or idx when d2t is None, the full head); logit =
    L[m, idx].  The list can only offer its own ids ("Masked MTP drafts",
    zone-1.cobraproject.com); the index-to-id map is the d2t table of
    "Two ways to run it" on the same page."""
    logits = oracle_logits(h_bits, w_bits)
    m, r = logits.shape
    if r < 1:
        raise ValueError("need at least one projected row")
    idx = np.argmax(logits, axis=1)            # first occurrence of the max
    rows = np.arange(m)
    best = logits[rows, idx]
    if r == 1:
        gap = np.full(m, np.inf)
    else:
        rest = logits.copy()
        rest[rows, idx] = -np.inf
        gap = best - rest.max(axis=1)
    if d2t is None:
        ids = idx.astype(np.int64)
    else:
        d2t = np.asarray(d2t)
        if d2t.shape != (r,):
            raise ValueError("d2t must have one entry per projected row")
        ids = d2t[idx].astype(np.int64)
    h = bf16_bits_to_f64(h_bits)
    w_win = bf16_bits_to_f64(np.asarray(w_bits)[idx])
    abs_sum = np.abs(h * w_win).sum(axis=1)
    return OracleResult(ids, idx.astype(np.int64), best, gap, abs_sum,
                        logits if keep_logits else None)
