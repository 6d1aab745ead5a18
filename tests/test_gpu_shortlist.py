"""Shortlist maintenance through the C ABI against the oracle: the device
union of two id lists and the in-place overwrite of trimmed-head rows, bit
for bit, and the projection after escaped ids are learned into spare rows
(parity rule of tests/parity.py)."""
import numpy as np
import pytest

import oracle
import synth
from parity import check
from test_gpu_parity import config_inputs, dev_bf16, dev_i32, device_weights, draws, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def gpu_union(L, a, b, n):
    out, counts = L.lmhead_shortlist_union(dev_i32(a), dev_i32(b), n)
    counts = counts.cpu().numpy()
    return out[:counts[3]].cpu().numpy(), tuple(int(c) for c in counts)


def test_union_of_the_page_lists(L):
    a, b, u = synth.union_parts()
    got, counts = gpu_union(L, a, b, synth.FULL_N)
    want, wc = oracle.oracle_union(a, b, synth.FULL_N)
    log(f"[union] counts {counts}")
    assert counts == wc == (47149, 9749, 5606, 52755)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n,na,nb", [(1, 3, 0), (31, 40, 40), (32, 0, 5), (33, 100, 1), (1000, 0, 0),
                                     (248_320, 70_000, 30_000), (1 << 19, 200_000, 5)])
def test_union_random(L, n, na, nb):
    rng = np.random.default_rng(n + na)
    a = rng.integers(-3, n + 3, size=na).astype(np.int32)
    b = rng.integers(-3, n + 3, size=nb).astype(np.int32)
    got, counts = gpu_union(L, a, b, n)
    want, wc = oracle.oracle_union(a, b, n)
    assert counts == wc
    assert np.array_equal(got, want)


def _overwrite_case(rng, n_vocab, k, cap, n):
    w = synth.normal_bf16(int(rng.integers(1 << 30)), n_vocab, k, 0.02)
    d2t = rng.permutation(n_vocab)[:cap].astype(np.int32)
    w_trim = oracle.oracle_trim(w, d2t)
    rows = rng.integers(-2, cap + 2, size=n).astype(np.int32)
    rows[: n // 4] = rows[n // 2: n // 2 + n // 4]            # repeated rows: the last entry wins
    ids = rng.integers(-2, n_vocab + 2, size=n).astype(np.int32)
    return w, d2t, w_trim, rows, ids


@pytest.mark.parametrize("n_vocab,k,cap,n", [(500, 256, 120, 40), (3000, 2560, 700, 2000), (100, 8, 7, 1),
                                             (20_000, 264, 5000, 65536)])
def test_overwrite_bit_exact(L, n_vocab, k, cap, n):
    rng = np.random.default_rng(n_vocab + n)
    w, d2t, w_trim, rows, ids = _overwrite_case(rng, n_vocab, k, cap, n)
    want_w, want_d = oracle.oracle_overwrite_rows(w_trim, d2t, w, rows, ids)
    w_dev = dev_bf16(w)
    wt_dev = dev_bf16(w_trim)
    d_dev = dev_i32(d2t)
    L.lmhead_shortlist_overwrite(w_dev, wt_dev, d_dev, dev_i32(rows), dev_i32(ids))
    torch.cuda.synchronize()
    assert np.array_equal(wt_dev.cpu().numpy().view(np.uint16), want_w)
    assert np.array_equal(d_dev.cpu().numpy(), want_d)


def test_overwrite_rejected_writes_nothing(L):
    w = dev_bf16(synth.normal_bf16(9, 100, 256, 0.02))
    wt = torch.zeros((50, 256), dtype=torch.int16, device="cuda")
    d = torch.full((50,), -7, dtype=torch.int32, device="cuda")
    rows = dev_i32(np.arange(4))
    ids = dev_i32(np.arange(4))
    lib = L.lib()
    assert lib.lmhead_shortlist_overwrite(w.data_ptr(), 100, 256, w.data_ptr() + 512, d.data_ptr(), 50,
                                          rows.data_ptr(), ids.data_ptr(), 4, None) == L.LMH_EINVAL
    assert lib.lmhead_shortlist_overwrite(w.data_ptr(), 100, 256, wt.data_ptr(), d.data_ptr(), 50,
                                          rows.data_ptr(), ids.data_ptr(), 65537, None) == L.LMH_EINVAL
    torch.cuda.synchronize()
    assert bool((wt == 0).all()) and bool((d == -7).all())


@pytest.mark.parametrize("m", [1, 4, 24])
def test_learn_escaped_ids_then_project(L, m):
    """The 32,768-id list held in a head with 1,024 spare rows: escaped ids
    written into the spare rows, then the projection over the grown prefix
    against the oracle over the same rows (which the oracle builds itself)."""
    inp = config_inputs(4)
    c, ids = inp["config"], inp["ids"]
    w_np = inp["W"]
    spare = 1024
    rng = np.random.default_rng(70 + m)
    escaped = np.setdiff1d(rng.integers(0, c.n, size=800), ids)[:600].astype(np.int32)
    cap_ids = np.concatenate([ids, np.zeros(spare, np.int32)]).astype(np.int32)
    w_dev = device_weights(4)
    wt_dev = L.lmhead_trim(w_dev, dev_i32(cap_ids))
    d_dev = dev_i32(cap_ids)
    rows = (ids.size + np.arange(escaped.size)).astype(np.int32)
    L.lmhead_shortlist_overwrite(w_dev, wt_dev, d_dev, dev_i32(rows), dev_i32(escaped))
    live = ids.size + escaped.size
    d2t_np = np.concatenate([ids, escaped]).astype(np.int32)
    assert np.array_equal(d_dev[:live].cpu().numpy(), d2t_np)
    w_live = oracle.oracle_trim(w_np, d2t_np)
    hs = draws(c, m, 2) if m in c.ms else [synth.hidden(7000 + m, d, m, c.k) for d in range(2)]
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax(stack, w_live, d2t_np, keep_logits=True)
    for p in ([L.LMH_PATH_VALU, L.LMH_PATH_MFMA] if m <= 4 else [L.LMH_PATH_MFMA]):
        gi, gl = [], []
        for h in hs:
            i, lg = L.draft_project_argmax_path(dev_bf16(h), wt_dev[:live], d_dev[:live], p)
            gi.append(i.cpu().numpy())
            gl.append(lg.cpu().numpy())
        st = check(stack, w_live, d2t_np, np.concatenate(gi), np.concatenate(gl), res)
        learned = np.isin(np.concatenate(gi), escaped).sum()
        log(f"[learn M={m}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} picked a learned id {learned}x")
        st.assert_exempt_bound()
