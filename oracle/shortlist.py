"""fp64/integer CPU oracle for shortlist maintenance.

TEST INFRASTRUCTURE ONLY, like the rest of this package: tests, the smoke
check and the CPU baseline of the benchmark use it; the product path never
imports it, and it shares no code with the HIP library.

Two operations the pages use to keep a trimmed head useful:

* A static trim can miss tokens the target still emits; on one model the
  server fixed this by learning the escaped ids into spare rows of the
  trimmed head (zone-1.cobraproject.com "Masked MTP drafts", section "Update
  (November 2026)", the Gemma 4 31B case).  Reading: an overwrite of chosen rows
  of W_trim with rows of W, and of the same d2t entries with the ids; the
  caller then projects over the grown prefix of rows.
* A list is widened by the sorted union of two id lists (ai-muninn.com
  "Qwen3.8-Flash-Next on two DGX Sparks", "Build the draft vocabulary from
  your own text": 47,149 ids and 9,749 candidates give 52,755).

Readings where the pages are silent (listed in the design notes):
* An overwrite entry whose id is outside [0, N) or whose row is outside
  [0, capacity) is skipped.  When several valid entries name the same row,
  the last one wins.
* The union is ascending and holds each id once; ids outside [0, N) are
  ignored.
"""
from __future__ import annotations

import numpy as np

__all__ = ["oracle_overwrite_rows", "oracle_union"]


def oracle_overwrite_rows(w_trim_bits, d2t, w_bits, rows, ids):
    """(W_trim', d2t') after writing W[ids[i]] into row rows[i] of W_trim and
    ids[i] into d2t[rows[i]], for i in order (so the last entry for a row
    wins); invalid entries are skipped.  Inputs are not modified."""
    w_trim = np.array(w_trim_bits, dtype=np.uint16, copy=True)
    d2t_out = np.array(d2t, dtype=np.int32, copy=True)
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    n_vocab, cap = w_bits.shape[0], w_trim.shape[0]
    if w_trim.ndim != 2 or w_bits.ndim != 2 or w_trim.shape[1] != w_bits.shape[1] or d2t_out.shape != (cap,):
        raise ValueError("W_trim [cap, K], W [N, K], d2t [cap]")
    for r, i in zip(np.asarray(rows).tolist(), np.asarray(ids).tolist()):
        if 0 <= r < cap and 0 <= i < n_vocab:
            w_trim[r] = w_bits[i]
            d2t_out[r] = i
    return w_trim, d2t_out


def oracle_union(a, b, n_vocab: int):
    """Ascending ids present in a or b (each once), ids outside [0, n_vocab)
    ignored; also (|set a|, |set b|, |set b - set a|, |union|), the four
    figures the pages print for their merge."""
    sa = {int(x) for x in np.asarray(a).tolist() if 0 <= int(x) < n_vocab}
    sb = {int(x) for x in np.asarray(b).tolist() if 0 <= int(x) < n_vocab}
    u = np.array(sorted(sa | sb), dtype=np.int32)
    return u, (len(sa), len(sb), len(sb - sa), len(sa | sb))
