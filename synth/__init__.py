"""Seeded synthetic inputs for the draft-head projection.

This module is shared by the oracle side and the HIP side of every test and
benchmark, so it holds no part of the method's arithmetic (no projection, no
argmax, no id map).  It only draws inputs and builds shortlists, and it does so
from numpy ``Generator(PCG64(SeedSequence(...)))`` streams so that every array
is a pure function of its seed.

What the pages fix, and what is a stand-in:

* Hidden width 2,560 and a 248,320-row head: "What I was testing" on
  krisbailey.com/articles/shortlist-mtp (the draft head and its shapes).
* The 16,000-id list is every id below 8,192, a 4,152-id structural core of
  which 3,531 ids lie above 8,192, and a frequency-ranked fill: "Building the
  16k shortlist" on the same page.  The corpus is not available, so the
  structural core is drawn uniformly and the frequency ranking is a seeded
  Zipf ranking.
* The FR-Spec list keeps the top 32,768 ids by the model's own output
  frequency, in rank order: "Masked MTP drafts" (zone-1.cobraproject.com),
  sections "Masked MTP drafts" and "Two ways to run it".
* The merged list is the sorted union of a 47,149-id list and a 9,749-id list
  of which 5,606 ids are new, 52,755 in all: "Build the draft vocabulary from
  your own text" on ai-muninn.com (qwen38-flash-next-two-sparks-checkpoint).

Zipf rankings: a seeded permutation maps rank to id, rank r gets weight
(r + 1) ** -s, counts are drawn multinomially over 224,000,000 tokens (the
size of the corpus named in "Building the 16k shortlist"), and ids are ranked
by (count descending, id ascending).
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_from_f32",
    "normal_bf16",
    "weight_matrix",
    "hidden",
    "zipf_ranking",
    "shortlist_low_struct_fill",
    "shortlist_top_ranked",
    "shortlist_union",
    "Config",
    "CONFIGS",
    "make_config",
]

# Rows per independently seeded block of a weight matrix.  Block b of a
# matrix with seed s is drawn from SeedSequence([s, b]); any block can be
# regenerated on its own, which lets a test rebuild single rows cheaply.
BLOCK_ROWS = 8192

CORPUS_TOKENS = 224_000_000


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (round to nearest, ties
    to even).  Returns uint16.  Inputs here are finite Gaussians, so NaN
    handling is not needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u
    t >>= 16
    return t.astype(np.uint16)


def _rng(*seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))


def _normal_block(seed: int, block: int, rows: int, cols: int, std: float) -> np.ndarray:
    z = _rng(seed, block).standard_normal(rows * cols, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return bf16_from_f32(z).reshape(rows, cols)


def normal_bf16(seed: int, rows: int, cols: int, std: float,
                threads: int | None = None) -> np.ndarray:
    """[rows, cols] bf16 bits (uint16), N(0, std) drawn in float32 and rounded.

    Row block b (rows b*BLOCK_ROWS ...) comes from SeedSequence([seed, b]), so
    the result does not depend on the thread count."""
    out = np.empty((rows, cols), dtype=np.uint16)
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def fill(b: int) -> None:
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        out[r0:r1] = _normal_block(seed, b, r1 - r0, cols, std)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nblk <= 1 or threads <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def normal_bf16_rows(seed: int, rows: int, cols: int, std: float,
                     which: np.ndarray) -> np.ndarray:
    """Rows ``which`` of ``normal_bf16(seed, rows, cols, std)`` without drawing
    the whole matrix (each needed block is drawn once)."""
    which = np.asarray(which, dtype=np.int64)
    out = np.empty((which.size, cols), dtype=np.uint16)
    for b in np.unique(which // BLOCK_ROWS):
        r0 = int(b) * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        blk = _normal_block(seed, int(b), r1 - r0, cols, std)
        sel = np.nonzero(which // BLOCK_ROWS == b)[0]
        out[sel] = blk[which[sel] - r0]
    return out


W_STD = 0.02   # LM-head weights ~ N(0, 0.02)
H_STD = 1.0    # hidden rows ~ N(0, 1)


def weight_matrix(seed: int, n: int, k: int) -> np.ndarray:
    return normal_bf16(seed, n, k, W_STD)


def hidden(seed: int, draw: int, m: int, k: int) -> np.ndarray:
    """Hidden rows [m, k] bf16 bits for parity draw ``draw`` of a config whose
    base seed is ``seed``: drawn from SeedSequence([seed, draw])."""
    z = _rng(seed, draw).standard_normal(m * k, dtype=np.float32)
    return bf16_from_f32(z).reshape(m, k)


def zipf_ranking(n: int, s: float, perm_seed: int,
                 total: int = CORPUS_TOKENS) -> np.ndarray:
    """All ``n`` ids ordered by sampled frequency (most frequent first).

    A seeded permutation assigns ids to ranks, rank r gets weight
    (r + 1) ** -s, ``total`` tokens are drawn multinomially, and ids are
    sorted by (count descending, id ascending)."""
    rng = _rng(perm_seed)
    rank_to_id = rng.permutation(n)
    w = np.arange(1, n + 1, dtype=np.float64) ** (-float(s))
    w /= w.sum()
    counts_by_rank = rng.multinomial(total, w)
    counts = np.empty(n, dtype=np.int64)
    counts[rank_to_id] = counts_by_rank
    # lexsort: last key is primary -> (count desc, id asc)
    ids = np.arange(n, dtype=np.int64)
    return np.lexsort((ids, -counts)).astype(np.int64)


def shortlist_low_struct_fill(n: int, size: int, low: int, struct_low: int,
                              struct_high: int, struct_seed: int,
                              ranking: np.ndarray) -> np.ndarray:
    """Every id below ``low``, plus a structural core of ``struct_low`` ids
    drawn in [0, low) and ``struct_high`` ids drawn in [low, n), plus the
    most frequent remaining ids of ``ranking`` until ``size`` ids.  Sorted."""
    rng = _rng(struct_seed)
    s_lo = rng.choice(low, size=struct_low, replace=False)
    s_hi = low + rng.choice(n - low, size=struct_high, replace=False)
    chosen = np.zeros(n, dtype=bool)
    chosen[:low] = True
    chosen[s_lo] = True
    chosen[s_hi] = True
    need = size - int(chosen.sum())
    if need < 0:
        raise ValueError("low block and structural core exceed the list size")
    fill = ranking[~chosen[ranking]][:need]
    chosen[fill] = True
    return np.nonzero(chosen)[0].astype(np.int32)


def shortlist_top_ranked(ranking: np.ndarray, size: int) -> np.ndarray:
    """The first ``size`` ids of a ranking, kept in rank order."""
    return np.ascontiguousarray(ranking[:size], dtype=np.int32)


def shortlist_union(list_a: np.ndarray, ranking_b: np.ndarray, b_in_a: int,
                    b_new: int) -> tuple[np.ndarray, np.ndarray]:
    """Build a second list by walking ``ranking_b`` and taking ids until it
    holds ``b_in_a`` ids already in ``list_a`` and ``b_new`` ids not in it.
    Returns (list_b, sorted union of list_a and list_b)."""
    in_a = np.zeros(int(max(ranking_b.max(), list_a.max())) + 1, dtype=bool)
    in_a[list_a] = True
    flags = in_a[ranking_b]
    c_in = np.cumsum(flags)
    c_new = np.cumsum(~flags)
    if c_in[-1] < b_in_a or c_new[-1] < b_new:
        raise ValueError("ranking too short for the requested second list")
    take = (flags & (c_in <= b_in_a)) | (~flags & (c_new <= b_new))
    list_b = ranking_b[take].astype(np.int32)          # walk order kept
    union = np.union1d(list_a, list_b).astype(np.int32)
    return list_b, union


@dataclass(frozen=True)
class Config:
    """One workload.  ``ms`` lists the hidden-row counts measured on it."""
    index: int
    name: str
    n: int
    k: int
    ms: tuple[int, ...]
    w_seed: int
    h_seed: tuple[int, ...]
    shortlist: str | None          # None = full vocabulary only
    full_too: bool                 # also project against the full W
    note: str = field(default="", compare=False)


FULL_N = 248_320
FULL_K = 2_560
FULL_W_SEED = 2560

CONFIGS: dict[int, Config] = {
    1: Config(1, "tiny", 4_096, 256, (1,), 256, (101,), "tiny512", True,
              "M=1 K=256 N=4096, 512-id list: ids < 256 plus the top of a "
              "Zipf(1.1) ranking"),
    2: Config(2, "full", FULL_N, FULL_K, (1,), FULL_W_SEED, (201,), None, True,
              "full-vocab draft step M=1 K=2560 N=248320"),
    3: Config(3, "mtp2_16k", FULL_N, FULL_K, (3,), FULL_W_SEED, (301,),
              "low_struct_16k", False,
              "M=3 on a 16,000-id list (low block + structural core + fill)"),
    4: Config(4, "frspec_32k", FULL_N, FULL_K, (1, 4), FULL_W_SEED, (401, 402),
              "frspec_32k", False,
              "M=1 and M=4 on the top 32,768 ids of a Zipf(1.0) ranking"),
    5: Config(5, "mtp3x8_52k", FULL_N, FULL_K, (24,), FULL_W_SEED, (501,),
              "union_52k", True,
              "M=24 (8 streams x 3 rows) on the full head and a 52,755-id union"),
}


@functools.lru_cache(maxsize=8)
def shortlist(name: str) -> np.ndarray:
    """The named shortlist as int32 ids (read-only)."""
    if name == "tiny512":
        n, low = 4_096, 256
        rk = zipf_ranking(n, 1.1, 11)
        rest = rk[rk >= low][:256]
        ids = np.union1d(np.arange(low), rest).astype(np.int32)
    elif name == "low_struct_16k":
        rk = zipf_ranking(FULL_N, 1.1, 32)
        ids = shortlist_low_struct_fill(FULL_N, 16_000, 8_192, 621, 3_531, 31, rk)
    elif name == "frspec_32k":
        ids = shortlist_top_ranked(zipf_ranking(FULL_N, 1.0, 41), 32_768)
    elif name == "union_52k":
        a = np.sort(zipf_ranking(FULL_N, 1.0, 51)[:47_149]).astype(np.int32)
        _, ids = shortlist_union(a, zipf_ranking(FULL_N, 1.0, 52), 4_143, 5_606)
    else:
        raise KeyError(name)
    ids.setflags(write=False)
    return ids


def union_parts() -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(list A, list B, union) of the 52,755-id merged list."""
    a = np.sort(zipf_ranking(FULL_N, 1.0, 51)[:47_149]).astype(np.int32)
    b, u = shortlist_union(a, zipf_ranking(FULL_N, 1.0, 52), 4_143, 5_606)
    return a, b, u


@functools.lru_cache(maxsize=2)
def _weights(seed: int, n: int, k: int) -> np.ndarray:
    w = weight_matrix(seed, n, k)
    w.setflags(write=False)
    return w


def make_config(i: int) -> dict:
    """Inputs of config ``i``: W bits, shortlist ids (or None) and the
    canonical hidden draw for each measured M."""
    c = CONFIGS[i]
    w = _weights(c.w_seed, c.n, c.k)
    ids = shortlist(c.shortlist) if c.shortlist else None
    hs = {m: hidden(seed, 0, m, c.k) for m, seed in zip(c.ms, c.h_seed)}
    return {"config": c, "W": w, "ids": ids, "h": hs}
