"""Plain fp64 CPU oracle for the draft-head projection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it exists so that tests, the smoke check and the CPU
baseline leg of the benchmark can check the HIP library against a slow,
obviously correct reading of the method.  It shares no code with the HIP path.

What is computed, and where it is defined:

* The draft head scores a hidden state of width K against LM-head rows, and
  the greedy draft is the highest-scoring row ("What I was testing" on
  krisbailey.com/articles/shortlist-mtp; greedy speculative decoding with
  the trim on, zone-1.cobraproject.com "Masked MTP drafts", section "Update
  (November 2026)").
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
    "oracle_project_topk",
    "oracle_scatter_logits",
    "oracle_project_argmax_indexed",
    "argmax_of_logits",
    "topk_of_logits",
    "OracleResult",
    "TopkResult",
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
    ids, idx, best, gap = argmax_of_logits(logits, d2t)
    h = bf16_bits_to_f64(h_bits)
    w_win = bf16_bits_to_f64(np.asarray(w_bits)[idx])
    abs_sum = np.abs(h * w_win).sum(axis=1)
    return OracleResult(ids, idx, best, gap, abs_sum, logits if keep_logits else None)


def argmax_of_logits(logits: np.ndarray, d2t: np.ndarray | None):
    """(id, idx, logit, gap) per hidden row of an [M, R] logit array: idx is
    the first row holding the maximum, id = d2t[idx] (or idx), gap = the
    maximum minus the best other row (+inf when R = 1)."""
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
    return ids, idx.astype(np.int64), best, gap


@dataclass
class TopkResult:
    """Per hidden row m, the k best projected rows in order: ``idx[m, j]``
    the row, ``id[m, j]`` its vocabulary id, ``logit[m, j]`` its fp64 logit;
    ``sorted_logits[m]`` every projected logit in the same order (so gaps
    around any position can be read off); ``logits`` the unsorted [M, R]."""
    id: np.ndarray
    idx: np.ndarray
    logit: np.ndarray
    sorted_logits: np.ndarray
    logits: np.ndarray


def oracle_project_topk(h_bits: np.ndarray, w_bits: np.ndarray,
                        d2t: np.ndarray | None, k: int) -> TopkResult:
    """The k highest-scoring projected rows per hidden row, best first.

    Several draft candidates per position (for sampling or a draft tree)
    are the top of the same scores whose argmax is the greedy draft; ties
    are broken by the smaller row index, as for the argmax.  Rows are
    mapped through d2t as in "Two ways to run it" (zone-1.cobraproject.com
    "Masked MTP drafts").  If fewer than k rows exist, positions past R hold
    id -1 and logit -inf."""
    return topk_of_logits(oracle_logits(h_bits, w_bits), d2t, k)


def topk_of_logits(logits: np.ndarray, d2t: np.ndarray | None, k: int) -> TopkResult:
    """The k best of [M, R] fp64 logits per row, best first, ties to the
    smaller row, mapped through d2t (the selection step of
    oracle_project_topk, shared by the heads of every format)."""
    m, r = logits.shape
    if k < 1:
        raise ValueError("k must be at least 1")
    # stable sort on -logit keeps the smaller index first among equal logits
    order = np.argsort(-logits, axis=1, kind="stable")
    srt = np.take_along_axis(logits, order, axis=1)
    kk = min(k, r)
    idx = np.full((m, k), -1, dtype=np.int64)
    lg = np.full((m, k), -np.inf)
    idx[:, :kk] = order[:, :kk]
    lg[:, :kk] = srt[:, :kk]
    if d2t is None:
        ids = idx.copy()
    else:
        d2t = np.asarray(d2t)
        if d2t.shape != (r,):
            raise ValueError("d2t must have one entry per projected row")
        ids = np.where(idx >= 0, d2t[np.clip(idx, 0, r - 1)], -1).astype(np.int64)
    return TopkResult(ids, idx, lg, srt, logits)


def oracle_scatter_logits(h_bits: np.ndarray, w_bits: np.ndarray,
                          d2t: np.ndarray | None, n: int | None = None) -> np.ndarray:
    """Logits in vocabulary space, scatter-after-matmul.

    With a d2t table the shortlist's logits are placed at their vocabulary
    ids in an [M, n] array whose other entries are -inf, the EAGLE-3 style
    map named in "Two ways to run it" (zone-1.cobraproject.com "Masked MTP
    drafts"); ids off the list can never win.  Without d2t the result is the
    [M, R] logits themselves."""
    logits = oracle_logits(h_bits, w_bits)
    if d2t is None:
        return logits
    d2t = np.asarray(d2t).astype(np.int64)
    if n is None or d2t.size and (d2t.min() < 0 or d2t.max() >= n):
        raise ValueError("d2t ids must lie in [0, n)")
    out = np.full((logits.shape[0], n), -np.inf)
    out[:, d2t] = logits
    return out


def oracle_project_argmax_indexed(h_bits: np.ndarray, w_bits: np.ndarray, ids: np.ndarray,
                                  keep_logits: bool = False) -> OracleResult:
    """Greedy draft over the rows W[ids[i]] read in place, without a trimmed
    copy: the same result as trimming the head to the list and projecting
    with d2t = ids ("Two ways to run it", zone-1.cobraproject.com "Masked MTP
    drafts": the list picks the head rows; the d2t map gives their ids).
    Entries whose id lies outside [0, N) are skipped; idx is the position in
    the list of the remaining entries, ties go to the earlier position."""
    w_bits = np.asarray(w_bits)
    ids = np.asarray(ids).astype(np.int64)
    valid = ids[(ids >= 0) & (ids < w_bits.shape[0])]
    if valid.size == 0:
        raise ValueError("no listed row is a row of W")
    return oracle_project_argmax(h_bits, oracle_trim(w_bits, valid), valid, keep_logits)
