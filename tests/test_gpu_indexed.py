"""Projection through the listed rows of the full head (no trimmed copy),
through the C ABI, against the fp64 oracle.

draft_project_argmax_indexed(h, W, ids) must give what the oracle gives for
the list read in place (oracle_project_argmax_indexed: entries outside
[0, N) skipped, ties to the earlier position).  Because the indexed kernels
keep the same lane layout and summation order as the kernels over a
trimmed copy, a call over the list must also equal draft_project_argmax over
lmhead_trim(W, ids) with d2t = ids bit for bit on the same kernel -- a
stronger check than the tolerance alone.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from devcopy import dev_bf16, dev_i32
from parity import ParityStats, check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def paths_for(L, m, k):
    ps = [L.LMH_PATH_MFMA]
    if m <= 8 and m * ((k // 8 + 63) // 64) <= 40:
        ps.insert(0, L.LMH_PATH_VALU)
    return ps


_inputs = {}


def config_inputs(i):
    if i not in _inputs:
        _inputs.clear()
        log(f"[inputs] generating config {i}")
        _inputs[i] = synth.make_config(i)
    return _inputs[i]


def draws(c, m, n):
    seed = c.h_seed[c.ms.index(m)] if m in c.ms else c.h_seed[0]
    return [synth.hidden(seed, d, m, c.k) for d in range(n)]


def valid_entries(ids, n):
    ids = np.asarray(ids, dtype=np.int64)
    return ids[(ids >= 0) & (ids < n)].astype(np.int32)


def run_indexed(L, hs, w_np, w_dev, ids, paths, tag, compare_trim=True):
    """Each draw through the indexed call on every path: the parity rule
    against the oracle on the listed rows, and bit equality with the call
    over the trimmed copy on the same path."""
    ids_dev = dev_i32(ids)
    valid = valid_entries(ids, w_np.shape[0])
    stack = np.concatenate(hs)
    # A repeated id is the same head row: the candidates are the distinct
    # listed ids, and the parity rule is applied over them (first positions).
    _, first = np.unique(valid, return_index=True)
    uniq = valid[np.sort(first)]
    res = oracle.oracle_project_argmax_indexed(stack, w_np, uniq, keep_logits=True)
    if uniq.size == valid.size:
        assert np.array_equal(
            oracle.oracle_project_argmax_indexed(stack, w_np, ids).id, res.id)
    w_sel = oracle.oracle_trim(w_np, uniq)
    wt = L.lmhead_trim(w_dev, dev_i32(valid)) if compare_trim else None
    valid_dev = dev_i32(valid)
    for p in paths:
        st = ParityStats()
        got_i, got_l = [], []
        for h in hs:
            hd = dev_bf16(h)
            i, l = L.draft_project_argmax_indexed(hd, w_dev, ids_dev, p)
            i, l = i.cpu().numpy(), l.cpu().numpy()
            got_i.append(i)
            got_l.append(l)
            if compare_trim and valid.size == ids.size:
                ti, tl = L.draft_project_argmax_path(hd, wt, valid_dev, p)
                assert np.array_equal(i, ti.cpu().numpy()), (tag, p)
                assert np.array_equal(l.view(np.uint32), tl.cpu().numpy().view(np.uint32)), (tag, p)
        st.add(check(stack, w_sel, uniq, np.concatenate(got_i), np.concatenate(got_l), res))
        log(f"[{tag}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e} "
            f"err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


# --------------------------------------------------------------------------
# the shortlisted workloads, read in place from the full head
# --------------------------------------------------------------------------

def test_indexed_tiny(L):
    inp = config_inputs(1)
    c = inp["config"]
    hs = draws(c, 1, 32)
    run_indexed(L, hs, inp["W"], dev_bf16(inp["W"]), inp["ids"], paths_for(L, 1, c.k), "tiny list")


def test_indexed_16k_m3(L):
    inp = config_inputs(3)
    c = inp["config"]
    hs = draws(c, 3, 16)
    run_indexed(L, hs, inp["W"], dev_bf16(inp["W"]), inp["ids"], paths_for(L, 3, c.k), "16k M=3")


@pytest.mark.parametrize("m", [1, 4])
def test_indexed_32k_rank_order(L, m):
    inp = config_inputs(4)
    c = inp["config"]
    hs = draws(c, m, 16)
    run_indexed(L, hs, inp["W"], dev_bf16(inp["W"]), inp["ids"], paths_for(L, m, c.k), f"32k M={m}")


def test_indexed_52k_m24(L):
    inp = config_inputs(5)
    c = inp["config"]
    hs = draws(c, 24, 16)
    run_indexed(L, hs, inp["W"], dev_bf16(inp["W"]), inp["ids"], paths_for(L, 24, c.k), "52k M=24")


# --------------------------------------------------------------------------
# edge cases: ragged lists, K tails, invalid and duplicate entries, M classes
# --------------------------------------------------------------------------

EDGE = [
    (1, 8, 1), (1, 16, 3), (2, 24, 63), (3, 256, 64), (4, 264, 65), (1, 520, 1000),
    (1, 2560, 7), (4, 2560, 4097), (2, 4096, 333), (1, 8192, 1501), (5, 264, 129),
    (8, 2560, 33), (16, 2560, 517), (17, 256, 700), (24, 2560, 1031), (31, 520, 99),
    (32, 2560, 2050), (13, 8, 77),
]


@pytest.mark.parametrize("m,k,s", EDGE, ids=[f"M{m}-K{k}-S{s}" for m, k, s in EDGE])
def test_indexed_edge_shapes(L, m, k, s):
    n = 3 * s + 5
    w_np = synth.normal_bf16(3000 + s, n, k, 0.02)
    h_np = synth.hidden(4000 + k, m, m, k)
    rng = np.random.default_rng(s * 31 + k)
    ids = rng.permutation(n)[:s].astype(np.int32)          # unsorted, distinct
    log(f"[indexed edge] M={m} K={k} S={s} N={n}")
    run_indexed(L, [h_np], w_np, dev_bf16(w_np), ids, paths_for(L, m, k), f"edge M={m} K={k} S={s}")


@pytest.mark.parametrize("m,k", [(1, 2560), (3, 264), (4, 2560), (24, 520)])
def test_indexed_skips_entries_outside_the_head(L, m, k):
    """Ids < 0 or >= N are never read and never win; the rest of the list
    behaves as if they were not there."""
    n = 4000
    w_np = synth.normal_bf16(51 + k, n, k, 0.02)
    h_np = synth.hidden(52 + m, 0, m, k)
    rng = np.random.default_rng(53 + m)
    good = rng.permutation(n)[:700].astype(np.int32)
    ids = good.copy()
    bad_pos = rng.choice(ids.size, size=120, replace=False)
    ids[bad_pos[:40]] = -1
    ids[bad_pos[40:80]] = n
    ids[bad_pos[80:]] = np.int32(2 ** 31 - 1)
    log(f"[indexed invalid] M={m} K={k} S={ids.size}")
    run_indexed(L, [h_np], w_np, dev_bf16(w_np), ids, paths_for(L, m, k), f"invalid M={m} K={k}",
                compare_trim=False)


def test_indexed_all_entries_invalid(L):
    w_np = synth.normal_bf16(61, 300, 264, 0.02)
    h_np = synth.hidden(62, 0, 3, 264)
    ids = np.array([-5, 300, 301, -1, 1 << 30], dtype=np.int32)
    for p in paths_for(L, 3, 264):
        i, l = L.draft_project_argmax_indexed(dev_bf16(h_np), dev_bf16(w_np), dev_i32(ids), p)
        assert np.all(i.cpu().numpy() == -1), p
        assert np.all(np.isnan(l.cpu().numpy())), p


def _int_bf16(vals):
    f = np.asarray(vals, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("m", [1, 3, 5, 24])
def test_indexed_exact_ties_take_earlier_entry(L, m):
    """Small-integer inputs make every logit exact; equal maximal rows are
    planted under several ids spread over the list, out of id order, so the
    earliest list position must win whatever the workgroup order."""
    rng = np.random.default_rng(71 + m)
    n, k, s = 60_000, 256, 40_000
    wi = rng.integers(-2, 3, size=(n, k)).astype(np.float32)
    hi = rng.integers(-2, 3, size=(m, k)).astype(np.float32)
    ids = rng.permutation(n)[:s].astype(np.int32)
    want = []
    for j in range(m):
        pos = [31_000 - j, 9_000 + 11 * j, 25_000 + j, 39_999 - j]   # list positions
        for q in pos:
            wi[ids[q]] = np.sign(hi[j]) * 2
        want.append(ids[min(pos)])
    w_np, h_np = _int_bf16(wi), _int_bf16(hi)
    res = oracle.oracle_project_argmax_indexed(h_np, w_np, ids)
    assert np.array_equal(res.id, np.array(want))
    w_dev = dev_bf16(w_np)
    for p in paths_for(L, m, k):
        i, l = L.draft_project_argmax_indexed(dev_bf16(h_np), w_dev, dev_i32(ids), p)
        assert np.array_equal(i.cpu().numpy(), res.id), (p, i.cpu().numpy(), res.id)
        assert np.array_equal(l.cpu().numpy().astype(np.float64), res.logit)


def test_indexed_duplicates_and_identity(L):
    """A list with repeated ids gives the first position's id; the identity
    list 0..N-1 gives exactly the full-head call."""
    n, k = 5000, 520
    w_np = synth.normal_bf16(81, n, k, 0.02)
    w_dev = dev_bf16(w_np)
    h_np = synth.hidden(82, 0, 4, k)
    ident = np.arange(n, dtype=np.int32)
    for m in (1, 4):
        for p in paths_for(L, m, k):
            hd = dev_bf16(h_np[:m])
            i, l = L.draft_project_argmax_indexed(hd, w_dev, dev_i32(ident), p)
            fi, fl = L.draft_project_argmax_path(hd, w_dev, None, p)
            assert torch.equal(i, fi) and torch.equal(l, fl), (m, p)
    rng = np.random.default_rng(83)
    dup = np.concatenate([rng.permutation(n)[:900], rng.permutation(n)[:900]]).astype(np.int32)
    run_indexed(L, [h_np], w_np, w_dev, dup, paths_for(L, 4, k), "duplicates", compare_trim=True)


def test_indexed_bench_helper_matches_call(L):
    inp = config_inputs(1)
    w_dev = dev_bf16(inp["W"])
    ids = dev_i32(inp["ids"])
    h = dev_bf16(inp["h"][1])
    want_id, want_lg = L.draft_project_argmax_indexed(h, w_dev, ids)
    ws = L.new_workspace()
    oid = torch.empty(1, dtype=torch.int32, device="cuda")
    olg = torch.empty(1, dtype=torch.float32, device="cuda")
    for p in paths_for(L, 1, 256):
        ms = L.lmhead_bench_time_argmax_indexed(h, [w_dev, w_dev], ids, p, 5, oid, olg, ws)
        assert 0.0 < ms < 100.0
        want_id, want_lg = L.draft_project_argmax_indexed(h, w_dev, ids, p)
        assert torch.equal(oid, want_id) and torch.equal(olg, want_lg)


@pytest.mark.parametrize("m", [1, 3, 24])
def test_indexed_long_list_takes_the_large_head_loops(L, m):
    """A list of at least 131,072 entries (the size where trimmed heads at
    one and two hidden rows change their load loop; lists read in place
    keep the row-order kernel's ring loop): a shuffled 150,000-id list of
    the full head, with a few invalid ids."""
    inp = config_inputs(2)
    c = inp["config"]
    rng = np.random.default_rng(91 + m)
    ids = rng.permutation(c.n)[:150_000].astype(np.int32)
    ids[rng.choice(ids.size, 50, replace=False)] = -3
    hs = [synth.hidden(92 + m, d, m, c.k) for d in range(2 if m < 24 else 1)]
    log(f"[indexed long] M={m} S={ids.size}")
    run_indexed(L, hs, inp["W"], dev_bf16(inp["W"]), ids, paths_for(L, m, c.k), f"long list M={m}",
                compare_trim=False)
