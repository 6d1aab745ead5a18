"""The seeded input recipe reproduces every count the pages print (CPU only)."""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "page_figures.json")))


def test_head_shape_matches_pages():
    g = GOLDEN["head_shape"]
    assert synth.FULL_K == g["hidden_width"]
    assert synth.FULL_N == g["vocab_rows"]
    for i in (2, 3, 4, 5):
        c = synth.CONFIGS[i]
        assert (c.n, c.k) == (g["vocab_rows"], g["hidden_width"])


def test_list_16k_composition():
    g = GOLDEN["list_16k"]
    ids = synth.shortlist("low_struct_16k")
    assert ids.size == g["total"] and np.unique(ids).size == ids.size
    assert np.all(np.diff(ids) > 0)                      # stored ascending
    assert np.isin(np.arange(g["low_block"]), ids).all()
    # recompute the parts with the generator's building block
    rk = synth.zipf_ranking(synth.FULL_N, 1.1, 32)
    core_lo = g["structural_core"] - g["structural_above_low_block"]
    assert core_lo == 621
    same = synth.shortlist_low_struct_fill(synth.FULL_N, g["total"], g["low_block"],
                                           core_lo, g["structural_above_low_block"], 31, rk)
    assert np.array_equal(same, ids)
    core_only = synth.shortlist_low_struct_fill(
        synth.FULL_N, g["low_block"] + g["structural_above_low_block"], g["low_block"],
        core_lo, g["structural_above_low_block"], 31, rk)
    above = core_only[core_only >= g["low_block"]]
    assert above.size == g["structural_above_low_block"]
    fill = np.setdiff1d(ids, core_only)
    assert fill.size == g["total"] - g["low_block"] - g["structural_above_low_block"] == 4277
    # the fill is the most frequent ids not already chosen, in ranking order
    rest = rk[~np.isin(rk, core_only)]
    assert np.array_equal(np.sort(rest[:fill.size]), fill)


def test_frspec_32k_is_top_of_ranking_in_rank_order():
    g = GOLDEN["frspec_trim"]
    ids = synth.shortlist("frspec_32k")
    assert ids.size == g["kept"] and np.unique(ids).size == ids.size
    rk = synth.zipf_ranking(synth.FULL_N, 1.0, 41)
    assert np.array_equal(ids, rk[:g["kept"]])
    assert not np.all(np.diff(ids) > 0)                  # rank order, not sorted
    assert round(g["vocab_rows"] / g["kept"], 1) == g["printed_ratio"]


def test_union_counts_match_printed_output():
    a, b, u = synth.union_parts()
    got = [len(set(a.tolist())), len(set(b.tolist())),
           len(set(b.tolist()) - set(a.tolist())), len(set(a.tolist()) | set(b.tolist()))]
    assert got == GOLDEN["list_union"]["printed_output"]
    assert np.array_equal(synth.shortlist("union_52k"), u)
    assert np.all(np.diff(u) > 0)


def test_tiny_list():
    ids = synth.shortlist("tiny512")
    assert ids.size == 512 and np.all(np.diff(ids) > 0)
    assert np.isin(np.arange(256), ids).all() and ids.max() < 4096


def test_zipf_ranking_is_a_permutation_ordered_by_counts():
    rk = synth.zipf_ranking(5000, 1.0, 3, total=1_000_000)
    assert np.array_equal(np.sort(rk), np.arange(5000))
    rk2 = synth.zipf_ranking(5000, 1.0, 3, total=1_000_000)
    assert np.array_equal(rk, rk2)
    assert not np.array_equal(rk, synth.zipf_ranking(5000, 1.0, 4, total=1_000_000))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200_000).astype(np.float32)
    # exact ties (low half 0x8000) with odd and even kept parts
    t = (rng.integers(0, 2 ** 31, 2000, dtype=np.uint32) & 0x7FFF0000) | 0x8000
    t = t[(t >> 23) < 0xFF]          # finite values only (the recipe draws Gaussians)
    x = np.concatenate([x, t.view(np.float32), np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    ours = synth.bf16_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert ours[-2] == 0x3F80 and ours[-1] == 0x3F82     # ties go to even


def test_weights_seeded_and_blockwise():
    a = synth.normal_bf16(99, 20_000, 64, 0.02, threads=4)
    b = synth.normal_bf16(99, 20_000, 64, 0.02, threads=1)
    assert np.array_equal(a, b)
    rows = np.array([0, 8191, 8192, 19_999, 12_345])
    assert np.array_equal(synth.normal_bf16_rows(99, 20_000, 64, 0.02, rows), a[rows])
    v = (a.astype(np.uint32) << 16).view(np.float32)
    assert abs(v.std() - 0.02) < 5e-4 and abs(v.mean()) < 5e-4


def test_hidden_draws_differ_and_repeat():
    h0 = synth.hidden(201, 0, 1, 2560)
    assert np.array_equal(h0, synth.hidden(201, 0, 1, 2560))
    assert not np.array_equal(h0, synth.hidden(201, 1, 1, 2560))
    v = (h0.astype(np.uint32) << 16).view(np.float32)
    assert abs(v.std() - 1.0) < 0.05
