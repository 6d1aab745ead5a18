"""Pins for the shortlist-maintenance part of the oracle (CPU only).

The union is pinned to the figures the pages print for their merge
(tests/golden/page_figures.json) and to numpy's union1d; the overwrite to
the gather it must stay consistent with (every row equals W at its d2t
id), to hand-built cases for skipped and repeated entries, and to the
restriction invariant of the projection after escaped ids are written into
spare rows.  ``test_shortlist_mutants_are_caught`` plants mistakes.
"""
import json
import os

import numpy as np
import pytest

import oracle.lmhead_oracle as lo
import oracle.shortlist as sl
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _rng(seed):
    return np.random.default_rng(seed)


def pin_union_page_figures(m):
    a, b, _ = synth.union_parts()
    u, counts = m.oracle_union(a, b, synth.FULL_N)
    assert list(counts) == GOLDEN["list_union"]["printed_output"]
    assert u.size == counts[3]


def pin_union_vs_numpy(m):
    rng = _rng(3)
    for n in (10, 1000, 100_000):
        a = rng.integers(-5, n + 5, size=rng.integers(0, 3 * n // 2 + 2))
        b = rng.integers(-5, n + 5, size=rng.integers(0, n // 3 + 2))
        u, counts = m.oracle_union(a, b, n)
        keep = lambda x: x[(x >= 0) & (x < n)]
        assert np.array_equal(u, np.union1d(keep(a), keep(b)).astype(np.int32))
        assert counts[0] == np.unique(keep(a)).size and counts[1] == np.unique(keep(b)).size
        assert counts[2] == np.setdiff1d(keep(b), keep(a)).size


def pin_union_edges(m):
    u, c = m.oracle_union(np.array([], np.int32), np.array([], np.int32), 7)
    assert u.size == 0 and c == (0, 0, 0, 0)
    u, c = m.oracle_union(np.array([6, 6, 0]), np.array([7, -1, 3]), 7)
    assert u.tolist() == [0, 3, 6] and c == (2, 1, 1, 3)


def pin_overwrite_consistent_with_gather(m):
    rng = _rng(4)
    w = synth.normal_bf16(4, 500, 32, 0.02)
    d2t = rng.permutation(500)[:120].astype(np.int32)
    w_trim = lo.oracle_trim(w, d2t)
    rows = rng.integers(0, 120, size=40)
    ids = rng.integers(0, 500, size=40)
    wt2, d2 = m.oracle_overwrite_rows(w_trim, d2t, w, rows, ids)
    assert np.array_equal(wt2, lo.oracle_trim(w, d2))
    untouched = np.setdiff1d(np.arange(120), rows)
    assert np.array_equal(d2[untouched], d2t[untouched])
    assert np.array_equal(w_trim, lo.oracle_trim(w, d2t))      # inputs unchanged


def pin_overwrite_last_wins_and_skips(m):
    w = synth.bf16_from_f32(np.arange(10 * 8, dtype=np.float32).reshape(10, 8))
    d2t = np.array([0, 1, 2, 3], np.int32)
    w_trim = lo.oracle_trim(w, d2t)
    rows = np.array([1, 1, 2, 4, -1, 3, 0])
    ids = np.array([5, 7, 10, 6, 6, -2, 9])
    wt2, d2 = m.oracle_overwrite_rows(w_trim, d2t, w, rows, ids)
    assert d2.tolist() == [9, 7, 2, 3]                         # row 1: last entry; 2, 3: invalid ids
    assert np.array_equal(wt2[1], w[7]) and np.array_equal(wt2[0], w[9])
    assert np.array_equal(wt2[2], w[2]) and np.array_equal(wt2[3], w[3])


def pin_learned_rows_restriction(m):
    """Escaped ids written into spare rows: the projection over the grown
    prefix equals the full projection restricted to list + escaped ids."""
    rng = _rng(5)
    n, k, s, spare = 3000, 64, 400, 64
    w = synth.normal_bf16(5, n, k, 0.02)
    ids = np.sort(rng.permutation(n)[:s]).astype(np.int32)
    cap_ids = np.concatenate([ids, np.zeros(spare, np.int32)])
    w_cap = lo.oracle_trim(w, cap_ids)
    escaped = np.setdiff1d(rng.integers(0, n, size=50), ids)[:30]
    rows = s + np.arange(escaped.size)
    wt2, d2 = m.oracle_overwrite_rows(w_cap, cap_ids, w, rows, escaped)
    live = s + escaped.size
    h = synth.hidden(6, 0, 3, k)
    got = lo.oracle_project_argmax(h, wt2[:live], d2[:live])
    full = lo.oracle_logits(h, w)
    allowed = np.concatenate([ids, escaped])
    mask = np.full(n, -np.inf)
    mask[allowed] = 0
    want = np.argmax(full + mask, axis=1)
    assert np.array_equal(got.id, want)


PINS = [pin_union_page_figures, pin_union_vs_numpy, pin_union_edges, pin_overwrite_consistent_with_gather,
        pin_overwrite_last_wins_and_skips, pin_learned_rows_restriction]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_shortlist_pin(pin):
    pin(sl)


_orig_union = sl.oracle_union
_orig_over = sl.oracle_overwrite_rows


def _mut_union_keeps_duplicates(a, b, n):
    u, c = _orig_union(a, b, n)
    extra = np.asarray(b)[(np.asarray(b) >= 0) & (np.asarray(b) < n)]
    return np.sort(np.concatenate([u, extra[:1]])).astype(np.int32), c


def _mut_union_unsorted(a, b, n):
    u, c = _orig_union(a, b, n)
    return u[::-1].copy(), c


def _mut_union_new_counts_a(a, b, n):
    u, c = _orig_union(a, b, n)
    return u, (c[0], c[1], c[3] - c[1], c[3])


def _mut_union_keeps_out_of_range(a, b, n):
    sa = {int(x) for x in np.asarray(a).tolist()}
    sb = {int(x) for x in np.asarray(b).tolist()}
    u = np.array(sorted(sa | sb), dtype=np.int32)
    return u, (len(sa), len(sb), len(sb - sa), len(sa | sb))


def _mut_over_first_wins(w_trim_bits, d2t, w_bits, rows, ids):
    rows = np.asarray(rows)[::-1]
    ids = np.asarray(ids)[::-1]
    return _orig_over(w_trim_bits, d2t, w_bits, rows, ids)


def _mut_over_keeps_d2t(w_trim_bits, d2t, w_bits, rows, ids):
    wt, _ = _orig_over(w_trim_bits, d2t, w_bits, rows, ids)
    return wt, np.array(d2t, dtype=np.int32, copy=True)


def _mut_over_wraps_ids(w_trim_bits, d2t, w_bits, rows, ids):
    n = np.asarray(w_bits).shape[0]
    return _orig_over(w_trim_bits, d2t, w_bits, rows, np.mod(np.asarray(ids), n))


MUTANTS = {
    "union_keeps_duplicates": ("oracle_union", _mut_union_keeps_duplicates),
    "union_unsorted": ("oracle_union", _mut_union_unsorted),
    "union_new_count_wrong": ("oracle_union", _mut_union_new_counts_a),
    "union_keeps_out_of_range": ("oracle_union", _mut_union_keeps_out_of_range),
    "overwrite_first_wins": ("oracle_overwrite_rows", _mut_over_first_wins),
    "overwrite_keeps_d2t": ("oracle_overwrite_rows", _mut_over_keeps_d2t),
    "overwrite_wraps_ids": ("oracle_overwrite_rows", _mut_over_wraps_ids),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_shortlist_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(sl, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(sl)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
