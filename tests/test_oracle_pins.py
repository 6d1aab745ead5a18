"""Pins for the fp64 oracle (CPU only).

Each pin checks the oracle against something other than itself: the bfloat16
definition, torch's own bf16 conversion, brute-force correctly rounded sums,
exact integer arithmetic, closed forms (one-hot hidden rows, planted
winners, planted ties) and the invariants that follow from the method's
definition (restriction to the shortlist, scatter-after-matmul, identity
list, row independence).  ``test_mutants_are_caught`` plants plausible
mistakes in the oracle and checks that at least one pin fails for each.
"""
import math
import struct

import numpy as np
import pytest

import oracle.lmhead_oracle as lo
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_of(values):
    """bf16 bits of float values that are exactly representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def _decode_struct(b):
    """bf16 bits -> Python float via the big-endian binary32 layout."""
    return struct.unpack(">f", struct.pack(">HH", int(b), 0))[0]


def _rand_bf16(rng, shape, scale):
    return synth.bf16_from_f32(rng.standard_normal(shape).astype(np.float32) * scale)


def _int_bf16(rng, shape, lo_, hi_):
    return _bf16_of(rng.integers(lo_, hi_ + 1, size=shape).astype(np.float32))


# --------------------------------------------------------------------------
# pins, written against the module object so mutants can be patched in
# --------------------------------------------------------------------------

def pin_decode_known(m):
    # values fixed by the format: sign | 8-bit exponent (bias 127) | 7-bit fraction
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC020: -2.5, 0x4049: 3.140625,
        0x3E80: 0.25, 0x4780: 65536.0, 0x0000: 0.0, 0x0080: 2.0 ** -126,
        0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
        0x42F7: 123.5, 0xC2F7: -123.5, 0x3C00: 2.0 ** -7,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = m.bf16_bits_to_f64(bits)
    want = np.array(list(cases.values()), dtype=np.float64)
    assert np.array_equal(got, want)
    neg0 = m.bf16_bits_to_f64(np.array([0x8000], dtype=np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0


def pin_decode_all_vs_torch(m):
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = m.bf16_bits_to_f64(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_bruteforce_fsum(m):
    rng = _rng(7)
    for (mm, k, r) in [(1, 8, 5), (3, 64, 37), (4, 256, 129), (2, 24, 512)]:
        h = _rand_bf16(rng, (mm, k), 1.0)
        w = _rand_bf16(rng, (r, k), 0.02)
        got = m.oracle_logits(h, w)
        assert got.shape == (mm, r)
        hd = [[_decode_struct(b) for b in row] for row in h]
        for i in range(mm):
            for j in range(0, r, max(1, r // 23)):
                terms = [hd[i][t] * _decode_struct(w[j, t]) for t in range(k)]
                exact = math.fsum(terms)
                bound = 1e-13 * math.fsum(abs(x) for x in terms) + 1e-300
                assert abs(got[i, j] - exact) <= bound, (mm, k, r, i, j)


def pin_integer_exact(m):
    rng = _rng(11)
    for (mm, k, r) in [(1, 16, 40), (4, 256, 300), (5, 2560, 64)]:
        hi = rng.integers(-8, 9, size=(mm, k))
        wi = rng.integers(-8, 9, size=(r, k))
        h = _bf16_of(hi.astype(np.float32))
        w = _bf16_of(wi.astype(np.float32))
        exact = hi.astype(np.int64) @ wi.astype(np.int64).T
        got = m.oracle_logits(h, w)
        assert np.array_equal(got, exact.astype(np.float64))
        res = m.oracle_project_argmax(h, w)
        for i in range(mm):
            row = exact[i].tolist()
            best = max(row)
            first = row.index(best)
            assert res.idx[i] == first and res.id[i] == first
            assert res.logit[i] == best
            others = row[:first] + row[first + 1:]
            assert res.gap[i] == best - max(others)


def pin_one_hot(m):
    rng = _rng(13)
    k, r = 96, 300
    w = _rand_bf16(rng, (r, k), 0.02)
    for col in (0, 1, 47, k - 1):
        h = np.zeros((1, k), dtype=np.uint16)
        h[0, col] = 0x3F80                       # 1.0
        got = m.oracle_logits(h, w)[0]
        want = np.array([_decode_struct(b) for b in w[:, col]])
        assert np.array_equal(got, want)
        res = m.oracle_project_argmax(h, w)
        colv = want.tolist()
        assert res.idx[0] == colv.index(max(colv))


def pin_planted_winner(m):
    rng = _rng(17)
    n, k = 2000, 128
    w = _rand_bf16(rng, (n, k), 0.02)
    h = _rand_bf16(rng, (1, k), 1.0)
    hv = np.array([_decode_struct(b) for b in h[0]], dtype=np.float32)
    for j in (0, 999, n - 1):
        wj = w.copy()
        wj[j] = synth.bf16_from_f32(hv * np.float32(0.25))   # logit ~ 0.25*|h|^2
        res = m.oracle_project_argmax(h, wj)
        assert res.id[0] == j
        ids_in = np.array(sorted({3, j, 1500, 42}), dtype=np.int32)
        res_t = m.oracle_project_argmax(h, m.oracle_trim(wj, ids_in), d2t=ids_in)
        assert res_t.id[0] == j
        ids_out = np.array([i for i in (5, 77, 1234, 1999, 0) if i != j], dtype=np.int32)
        res_o = m.oracle_project_argmax(h, m.oracle_trim(wj, ids_out), d2t=ids_out)
        assert res_o.id[0] != j and res_o.id[0] in ids_out


def pin_ties_first_occurrence(m):
    k = 8
    h = _bf16_of(np.ones((1, k), np.float32))
    # row sums: 3, 5, 5, 1, 5 -> first max at index 1
    rows = [[1, 1, 1, 0, 0, 0, 0, 0], [1, 1, 1, 1, 1, 0, 0, 0], [2, 2, 1, 0, 0, 0, 0, 0],
            [1, 0, 0, 0, 0, 0, 0, 0], [5, 0, 0, 0, 0, 0, 0, 0]]
    w = _bf16_of(np.array(rows, np.float32))
    res = m.oracle_project_argmax(h, w)
    assert res.idx[0] == 1 and res.logit[0] == 5.0 and res.gap[0] == 0.0
    d2t = np.array([10, 20, 30, 40, 50], np.int32)
    assert m.oracle_project_argmax(h, w, d2t=d2t).id[0] == 20
    # all equal -> index 0
    w_eq = _bf16_of(np.full((7, k), 0.5, np.float32))
    assert m.oracle_project_argmax(h, w_eq).idx[0] == 0


def pin_gap_and_single_row(m):
    h = _bf16_of(np.array([[1.0, 2.0]], np.float32))
    w = _bf16_of(np.array([[1.0, 0.0], [0.0, 1.0], [0.5, 1.5], [-1.0, 0.0]], np.float32))
    # logits: 1, 2, 3.5, -1
    res = m.oracle_project_argmax(h, w)
    assert res.idx[0] == 2 and res.logit[0] == 3.5 and res.gap[0] == 1.5
    assert res.abs_sum[0] == 0.5 + 3.0
    one = m.oracle_project_argmax(h, w[1:2])
    assert one.idx[0] == 0 and one.logit[0] == 2.0 and np.isinf(one.gap[0])
    # negative hidden values: sign matters
    hn = _bf16_of(np.array([[-1.0, -2.0]], np.float32))
    resn = m.oracle_project_argmax(hn, w)
    assert resn.idx[0] == 3 and resn.logit[0] == 1.0


def pin_trim_rows(m):
    rng = _rng(19)
    n, k = 1000, 16
    w = np.zeros((n, k), dtype=np.uint16)
    w[:, 0] = np.arange(n, dtype=np.uint16)               # raw row tag
    w[:, 1:] = rng.integers(0, 0x7F00, size=(n, k - 1), dtype=np.uint16)
    ids = rng.permutation(n)[:300].astype(np.int32)
    t = m.oracle_trim(w, ids)
    assert t.shape == (300, k) and t.dtype == np.uint16
    assert np.array_equal(t[:, 0], ids.astype(np.uint16))
    for i in (0, 1, 150, 299):
        assert np.array_equal(t[i], w[ids[i]])
    ident = m.oracle_trim(w, np.arange(n, dtype=np.int32))
    assert np.array_equal(ident, w)
    with pytest.raises(IndexError):
        m.oracle_trim(w, np.array([0, n], dtype=np.int32))
    with pytest.raises(IndexError):
        m.oracle_trim(w, np.array([-1], dtype=np.int32))


def _tiny_inputs(draws=8):
    c = synth.CONFIGS[1]
    w = synth.weight_matrix(c.w_seed, c.n, c.k)
    ids = synth.shortlist("tiny512")
    hs = np.concatenate([synth.hidden(c.h_seed[0], d, 1, c.k) for d in range(draws)])
    return w, ids, hs


def pin_restriction_invariant(m):
    w, ids, hs = _tiny_inputs()
    full = m.oracle_logits(hs, w)
    res = m.oracle_project_argmax(hs, m.oracle_trim(w, ids), d2t=ids)
    masked = np.full_like(full, -np.inf)
    masked[:, ids] = full[:, ids]
    for i in range(hs.shape[0]):
        assert res.id[i] == int(np.flatnonzero(masked[i] == masked[i].max())[0])
        assert res.logit[i] == masked[i].max()


def pin_indexed_restriction(m):
    """Rows read through a list: the maximum of the full logits over the
    listed ids, ties to the earlier list position, with invalid entries
    (outside [0, N)) skipped."""
    w, ids, hs = _tiny_inputs()
    rng = np.random.default_rng(29)
    lst = ids[rng.permutation(ids.size)].astype(np.int64)
    lst = np.insert(lst, [0, 7, 100, lst.size], [-1, w.shape[0], w.shape[0] + 9, -20])
    # exact ties: copies of one row under two listed ids, the later one first in the list
    w = w.copy()
    a, b = int(lst[5]), int(lst[40])
    w[a] = w[b]
    res = m.oracle_project_argmax_indexed(hs, w, lst)
    full = m.oracle_logits(hs, w)
    valid = lst[(lst >= 0) & (lst < w.shape[0])]
    for i in range(hs.shape[0]):
        vals = full[i, valid]
        j = int(np.flatnonzero(vals == vals.max())[0])
        assert res.idx[i] == j and res.id[i] == valid[j] and res.logit[i] == vals.max()
    # every hidden row whose maximum is the duplicated row takes the earlier position (id a)
    hs2 = synth.bf16_from_f32(lo.bf16_bits_to_f64(w[[a]]).astype(np.float32))
    r2 = m.oracle_project_argmax_indexed(hs2, w, lst)
    assert r2.id[0] == a
    with pytest.raises(ValueError):
        m.oracle_project_argmax_indexed(hs, w, np.array([-1, w.shape[0]]))


def pin_scatter_equivalence(m):
    w, ids, hs = _tiny_inputs()
    perm = np.random.default_rng(23).permutation(ids.size)
    ids_p = ids[perm]                               # a rank-ordered list
    res = m.oracle_project_argmax(hs, m.oracle_trim(w, ids_p), d2t=ids_p,
                                  keep_logits=True)
    scat = np.full((hs.shape[0], w.shape[0]), -np.inf)
    scat[:, ids_p] = res.logits                     # scatter-after-matmul
    for i in range(hs.shape[0]):
        assert res.id[i] == int(np.argmax(scat[i]))


def pin_identity_list(m):
    w, _, hs = _tiny_inputs()
    ident = np.arange(w.shape[0], dtype=np.int32)
    a = m.oracle_project_argmax(hs, w)
    b = m.oracle_project_argmax(hs, m.oracle_trim(w, ident), d2t=ident)
    assert np.array_equal(a.id, b.id) and np.array_equal(a.logit, b.logit)


def pin_rows_independent(m):
    w, ids, hs = _tiny_inputs(draws=12)
    batch = m.oracle_project_argmax(hs, w)
    for i in range(hs.shape[0]):
        one = m.oracle_project_argmax(hs[i:i + 1], w)
        assert one.id[0] == batch.id[i] and one.logit[0] == batch.logit[i]
    t = m.oracle_project_argmax(hs, m.oracle_trim(w, ids), d2t=ids)
    perm = np.random.default_rng(29).permutation(ids.size)
    tp = m.oracle_project_argmax(hs, m.oracle_trim(w, ids[perm]), d2t=ids[perm])
    ok = t.gap > 0
    assert np.array_equal(t.id[ok], tp.id[ok])


def pin_topk_bruteforce(m):
    """Small-integer logits are exact; sort by (value desc, row asc) by hand."""
    rng = _rng(41)
    for (mm, k, r, kk) in [(1, 16, 40, 5), (3, 64, 200, 8), (2, 8, 7, 10)]:
        hi = rng.integers(-3, 4, size=(mm, k))
        wi = rng.integers(-3, 4, size=(r, k))
        exact = (hi.astype(np.int64) @ wi.astype(np.int64).T).tolist()
        res = m.oracle_project_topk(_bf16_of(hi.astype(np.float32)),
                                    _bf16_of(wi.astype(np.float32)), None, kk)
        assert res.idx.shape == (mm, kk)
        for i in range(mm):
            order = sorted(range(r), key=lambda j: (-exact[i][j], j))
            for j in range(kk):
                if j < r:
                    assert res.idx[i, j] == order[j] and res.id[i, j] == order[j]
                    assert res.logit[i, j] == exact[i][order[j]]
                else:
                    assert res.idx[i, j] == -1 and res.id[i, j] == -1
                    assert res.logit[i, j] == -np.inf


def pin_topk_ties_and_d2t(m):
    h = _bf16_of(np.ones((1, 4), np.float32))
    # row sums: 2, 4, 4, 1, 4, 3
    rows = [[1, 1, 0, 0], [2, 2, 0, 0], [1, 1, 1, 1], [1, 0, 0, 0], [4, 0, 0, 0], [3, 0, 0, 0]]
    w = _bf16_of(np.array(rows, np.float32))
    res = m.oracle_project_topk(h, w, None, 4)
    assert res.idx[0].tolist() == [1, 2, 4, 5]
    assert res.logit[0].tolist() == [4.0, 4.0, 4.0, 3.0]
    d2t = np.array([50, 40, 30, 20, 10, 0], np.int32)
    assert m.oracle_project_topk(h, w, d2t, 4).id[0].tolist() == [40, 30, 10, 0]
    one = m.oracle_project_topk(h, w, d2t, 1)
    arg = m.oracle_project_argmax(h, w, d2t)
    assert one.id[0, 0] == arg.id[0] and one.logit[0, 0] == arg.logit[0]


def pin_scatter_logits(m):
    w, ids, hs = _tiny_inputs(draws=4)
    n = w.shape[0]
    full = m.oracle_logits(hs, w)
    sc = m.oracle_scatter_logits(hs, m.oracle_trim(w, ids), ids, n)
    assert sc.shape == (hs.shape[0], n)
    off = np.ones(n, bool)
    off[ids] = False
    assert np.all(sc[:, off] == -np.inf)
    assert np.array_equal(sc[:, ids], full[:, ids])
    # argmax of the scattered vector is the shortlist draft
    arg = m.oracle_project_argmax(hs, m.oracle_trim(w, ids), d2t=ids)
    assert np.array_equal(np.argmax(sc, axis=1), arg.id)
    assert np.array_equal(m.oracle_scatter_logits(hs, w, None), full)
    with pytest.raises(ValueError):
        m.oracle_scatter_logits(hs, w[:10], np.arange(10), 5)


PINS = [pin_decode_known, pin_decode_all_vs_torch, pin_bruteforce_fsum,
        pin_integer_exact, pin_one_hot, pin_planted_winner,
        pin_ties_first_occurrence, pin_gap_and_single_row, pin_trim_rows,
        pin_restriction_invariant, pin_scatter_equivalence, pin_identity_list,
        pin_rows_independent, pin_topk_bruteforce, pin_topk_ties_and_d2t,
        pin_scatter_logits, pin_indexed_restriction]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(lo)


# --------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin
# --------------------------------------------------------------------------

_orig_decode = lo.bf16_bits_to_f64
_orig_logits = lo.oracle_logits
_orig_project = lo.oracle_project_argmax
_orig_trim = lo.oracle_trim
_orig_topk = lo.oracle_project_topk
_orig_scatter = lo.oracle_scatter_logits
_orig_indexed = lo.oracle_project_argmax_indexed


def _mut_indexed_wraps(h, w, ids, keep_logits=False):
    n = np.asarray(w).shape[0]
    return _orig_indexed(h, w, np.mod(np.asarray(ids), n), keep_logits)


def _mut_indexed_ties_by_id(h, w, ids, keep_logits=False):
    ids = np.asarray(ids)
    return _orig_indexed(h, w, np.sort(ids[(ids >= 0) & (ids < np.asarray(w).shape[0])]), keep_logits)


def _mut_decode_fp16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _mut_decode_shift15(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64)


def _mut_logits_drop_last(h, w):
    return _orig_logits(np.asarray(h)[:, :-1], np.asarray(w)[:, :-1])


def _mut_logits_drop_first_block_row(h, w):
    out = _orig_logits(h, w)
    if out.shape[1] > 1:
        out[:, 0] = out[:, 1]
    return out


def _mut_logits_sign(h, w):
    return -_orig_logits(h, w)


def _mut_logits_layout(h, w):
    w = np.asarray(w)
    r, k = w.shape
    return _orig_logits(h, np.ascontiguousarray(w.reshape(k, r).T))


def _mut_logits_hidden_reversed(h, w):
    return _orig_logits(np.asarray(h)[:, ::-1], w)


def _mut_logits_abs(h, w):
    return np.abs(_orig_logits(h, w))


def _wrap_project(post):
    def f(h, w, d2t=None, keep_logits=False):
        res = _orig_project(h, w, d2t=None, keep_logits=True)
        return post(res, np.asarray(d2t) if d2t is not None else None, keep_logits)
    return f


def _finish(res, idx, d2t, keep):
    rows = np.arange(idx.size)
    res.idx = idx
    res.logit = res.logits[rows, idx]
    res.id = idx if d2t is None else d2t[idx].astype(np.int64)
    if not keep:
        res.logits = None
    return res


def _post_last_occurrence(res, d2t, keep):
    lg = res.logits
    idx = lg.shape[1] - 1 - np.argmax(lg[:, ::-1], axis=1)
    return _finish(res, idx, d2t, keep)


def _post_argmin(res, d2t, keep):
    return _finish(res, np.argmin(res.logits, axis=1), d2t, keep)


def _post_ignore_d2t(res, d2t, keep):
    return _finish(res, res.idx, None, keep)


def _post_d2t_off_by_one(res, d2t, keep):
    r = _finish(res, res.idx, d2t, keep)
    if d2t is not None:
        r.id = d2t[np.minimum(res.idx + 1, d2t.size - 1)].astype(np.int64)
    return r


def _post_gap_second_any(res, d2t, keep):
    r = _finish(res, res.idx, d2t, keep)
    srt = np.sort(res.logits if res.logits is not None else np.zeros((1, 1)), axis=1)
    r.gap = srt[:, -1] - srt[:, 0]                 # max minus min
    return r


def _mut_trim_sorted(w, ids):
    return _orig_trim(w, np.sort(np.asarray(ids)))


def _mut_trim_off_by_one(w, ids):
    w = np.asarray(w)
    return w[np.minimum(np.asarray(ids, np.int64) + 1, w.shape[0] - 1)].copy()


def _mut_trim_no_check(w, ids):
    w = np.asarray(w)
    return w[np.asarray(ids, np.int64) % w.shape[0]].copy()


def _mut_topk_ties_large_first(h, w, d2t, k):
    res = _orig_topk(h, w, d2t, k)
    lg = res.logits
    order = np.lexsort((-np.arange(lg.shape[1])[None, :].repeat(lg.shape[0], 0), -lg), axis=1)
    kk = min(k, lg.shape[1])
    res.idx[:, :kk] = order[:, :kk]
    res.id = res.idx.copy() if d2t is None else np.where(res.idx >= 0, np.asarray(d2t)[np.clip(res.idx, 0, None)], -1)
    return res


def _mut_topk_ascending(h, w, d2t, k):
    res = _orig_topk(h, w, d2t, k)
    res.idx = res.idx[:, ::-1].copy()
    res.id = res.id[:, ::-1].copy()
    res.logit = res.logit[:, ::-1].copy()
    return res


def _mut_topk_ignores_d2t(h, w, d2t, k):
    return _orig_topk(h, w, None, k)


def _mut_topk_pads_zero(h, w, d2t, k):
    res = _orig_topk(h, w, d2t, k)
    res.logit = np.where(np.isinf(res.logit), 0.0, res.logit)
    return res


def _mut_scatter_zero_fill(h, w, d2t, n=None):
    out = _orig_scatter(h, w, d2t, n)
    return np.where(np.isinf(out), 0.0, out)


def _mut_scatter_by_position(h, w, d2t, n=None):
    logits = _orig_logits(h, w)
    if d2t is None:
        return logits
    out = np.full((logits.shape[0], n), -np.inf)
    out[:, :logits.shape[1]] = logits
    return out


MUTANTS = {
    "topk_ties_larger_first": ("oracle_project_topk", _mut_topk_ties_large_first),
    "topk_ascending": ("oracle_project_topk", _mut_topk_ascending),
    "topk_ignores_d2t": ("oracle_project_topk", _mut_topk_ignores_d2t),
    "topk_pads_zero": ("oracle_project_topk", _mut_topk_pads_zero),
    "scatter_zero_fill": ("oracle_scatter_logits", _mut_scatter_zero_fill),
    "scatter_by_position": ("oracle_scatter_logits", _mut_scatter_by_position),
    "indexed_wraps_ids": ("oracle_project_argmax_indexed", _mut_indexed_wraps),
    "indexed_sorted_list": ("oracle_project_argmax_indexed", _mut_indexed_ties_by_id),
    "decode_as_fp16": ("bf16_bits_to_f64", _mut_decode_fp16),
    "decode_shift15": ("bf16_bits_to_f64", _mut_decode_shift15),
    "logits_drop_last_k": ("oracle_logits", _mut_logits_drop_last),
    "logits_row0_wrong": ("oracle_logits", _mut_logits_drop_first_block_row),
    "logits_sign_flip": ("oracle_logits", _mut_logits_sign),
    "logits_transposed_layout": ("oracle_logits", _mut_logits_layout),
    "logits_hidden_reversed": ("oracle_logits", _mut_logits_hidden_reversed),
    "logits_abs": ("oracle_logits", _mut_logits_abs),
    "argmax_last_occurrence": ("oracle_project_argmax", _wrap_project(_post_last_occurrence)),
    "argmin": ("oracle_project_argmax", _wrap_project(_post_argmin)),
    "d2t_ignored": ("oracle_project_argmax", _wrap_project(_post_ignore_d2t)),
    "d2t_off_by_one": ("oracle_project_argmax", _wrap_project(_post_d2t_off_by_one)),
    "gap_max_minus_min": ("oracle_project_argmax", _wrap_project(_post_gap_second_any)),
    "trim_sorted_ids": ("oracle_trim", _mut_trim_sorted),
    "trim_off_by_one": ("oracle_trim", _mut_trim_off_by_one),
    "trim_wraps_ids": ("oracle_trim", _mut_trim_no_check),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(lo, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(lo)
        except (AssertionError, IndexError, ValueError, pytest.fail.Exception):
            failed.append(pin.__name__)
        except pytest.skip.Exception:
            pass
    assert failed, f"mutant {name} passed every pin"
