"""Top-k candidates and full / scattered logits through the C ABI, against
the fp64 oracle, on both kernels wherever both accept the shape."""
import numpy as np
import pytest

import oracle
import synth
from parity import check_logits, check_topk
from test_gpu_parity import config_inputs, dev_bf16, dev_i32, device_weights, draws, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def epi_paths(L, m, k=2560):
    """The top-k / logits epilogues run on the VALU kernels for M <= 4 with
    M * ceil(K / 512) <= 40, and on the matrix-core kernel for any M."""
    valu = m <= 4 and m * ((k // 8 + 63) // 64) <= 40
    return [L.LMH_PATH_VALU, L.LMH_PATH_MFMA] if valu else [L.LMH_PATH_MFMA]


def run_topk(L, hs, w_np, w_dev, d2t_np, k, tag):
    stack = np.concatenate(hs)
    res = oracle.oracle_project_topk(stack, w_np, d2t_np, k)
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in epi_paths(L, hs[0].shape[0]):
        ids, lgs = [], []
        for h in hs:
            i, l = L.draft_project_topk(dev_bf16(h), w_dev, d2t_dev, k, path=p)
            ids.append(i.cpu().numpy())
            lgs.append(l.cpu().numpy())
        st = check_topk(stack, w_np, d2t_np, np.concatenate(ids), np.concatenate(lgs), res)
        log(f"[{tag}] path={p} k={k} positions={st.rows} near_ties={st.near_ties} exempt={st.exempt} "
            f"max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


@pytest.mark.parametrize("k", [1, 3, 8, 16])
def test_topk_tiny(L, k):
    inp = config_inputs(1)
    c, ids = inp["config"], inp["ids"]
    w_dev = device_weights(1)
    hs = draws(c, 1, 16)
    run_topk(L, hs, inp["W"], w_dev, None, k, "tiny full")
    wt = L.lmhead_trim(w_dev, dev_i32(ids))
    run_topk(L, hs, oracle.oracle_trim(inp["W"], ids), wt, ids, k, "tiny trim")


def test_topk_full_head_m1_and_m3(L):
    inp = config_inputs(2)
    c = inp["config"]
    w_dev = device_weights(2)
    run_topk(L, draws(c, 1, 4), inp["W"], w_dev, None, 8, "full M=1")
    run_topk(L, [synth.hidden(c.h_seed[0] + 7, d, 3, c.k) for d in range(2)], inp["W"], w_dev, None, 4,
             "full M=3")


def test_topk_16k_m3(L):
    inp = config_inputs(3)
    c, ids = inp["config"], inp["ids"]
    wt = L.lmhead_trim(device_weights(3), dev_i32(ids))
    run_topk(L, draws(c, 3, 4), oracle.oracle_trim(inp["W"], ids), wt, ids, 10, "16k M=3")


@pytest.mark.parametrize("k", [4, 16])
def test_topk_m24_52k(L, k):
    """M = 24 with k <= 4 keeps both 16-column tiles in one pass; k = 16
    splits the hidden rows into passes of 16."""
    inp = config_inputs(5)
    c, ids = inp["config"], inp["ids"]
    wt = L.lmhead_trim(device_weights(5), dev_i32(ids))
    run_topk(L, draws(c, 24, 1), oracle.oracle_trim(inp["W"], ids), wt, ids, k, "52k M=24")


EDGE = [(1, 8, 3, 8), (2, 264, 17, 16), (4, 2560, 65, 5), (5, 520, 1000, 2), (7, 256, 9, 16),
        (17, 2560, 333, 4), (20, 2560, 200, 8), (32, 8192, 100, 16), (3, 8192, 2050, 7)]


@pytest.mark.parametrize("m,k,r,topk", EDGE, ids=[f"M{m}-K{k}-R{r}-k{t}" for m, k, r, t in EDGE])
def test_topk_edges(L, m, k, r, topk):
    w_np = synth.normal_bf16(3000 + r, r, k, 0.02)
    h_np = synth.hidden(4000 + k, m, m, k)
    d2t = (np.arange(r, dtype=np.int32)[::-1] * 3 + 1).copy()
    w_dev = dev_bf16(w_np)
    for p in epi_paths(L, m, k):
        for dd in (None, d2t):
            i, l = L.draft_project_topk(dev_bf16(h_np), w_dev, dev_i32(dd) if dd is not None else None,
                                        topk, path=p)
            check_topk(h_np, w_np, dd, i.cpu().numpy(), l.cpu().numpy())


def _int_bf16(vals):
    f = np.asarray(vals, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("m", [1, 3, 6])
def test_topk_exact_ties_order(L, m):
    """Integer inputs make every logit exact: equal logits must come out in
    row order, across workgroups."""
    rng = np.random.default_rng(77 + m)
    r, k = 120_000, 128
    wi = rng.integers(-1, 2, size=(r, k)).astype(np.float32)
    hi = rng.integers(-1, 2, size=(m, k)).astype(np.float32)
    for j in range(m):
        for rr in (90_001 + j, 3 + j, 55_555, 119_999 - j, 60_000 + 2 * j):
            wi[rr] = np.sign(hi[j])
    w_np, h_np = _int_bf16(wi), _int_bf16(hi)
    res = oracle.oracle_project_topk(h_np, w_np, None, 8)
    w_dev = dev_bf16(w_np)
    for p in epi_paths(L, m):
        i, l = L.draft_project_topk(dev_bf16(h_np), w_dev, None, 8, path=p)
        assert np.array_equal(i.cpu().numpy(), res.idx), (p, i.cpu().numpy()[:, :6], res.idx[:, :6])
        assert np.array_equal(l.cpu().numpy().astype(np.float64), res.logit)


def test_topk_1_matches_argmax(L):
    """Where argmax and top-1 run the same projection kernel (M = 1 on VALU,
    any M on the matrix cores) they agree bit for bit; M = 4 on VALU runs the
    row-order argmax kernel against the tiled top-k kernel, whose sums
    differ only by rounding."""
    inp = config_inputs(4)
    c, ids = inp["config"], inp["ids"]
    wt = L.lmhead_trim(device_weights(4), dev_i32(ids))
    d2t = dev_i32(ids)
    for m, p, exact in ((1, L.LMH_PATH_VALU, True), (1, L.LMH_PATH_MFMA, True), (4, L.LMH_PATH_MFMA, True),
                        (6, L.LMH_PATH_MFMA, True), (4, L.LMH_PATH_VALU, False)):
        for h_np in [synth.hidden(c.h_seed[0] + 31, d, m, c.k) for d in range(3)]:
            h = dev_bf16(h_np)
            a_id, a_lg = L.draft_project_argmax_path(h, wt, d2t, p)
            t_id, t_lg = L.draft_project_topk(h, wt, d2t, 1, path=p)
            if exact:
                assert torch.equal(t_id[:, 0], a_id) and torch.equal(t_lg[:, 0], a_lg), (m, p)
            else:
                assert float((t_lg[:, 0] - a_lg).abs().max()) < 1e-4
                res = oracle.oracle_project_argmax(h_np, oracle.oracle_trim(inp["W"], ids), ids)
                sure = torch.from_numpy(res.gap > 1e-3).cuda()
                assert torch.equal(t_id[:, 0][sure], a_id[sure])


# --------------------------------------------------------------------------
# logits
# --------------------------------------------------------------------------

def test_logits_tiny_full_and_scattered(L):
    inp = config_inputs(1)
    c, ids = inp["config"], inp["ids"]
    w_dev = device_weights(1)
    h_np = np.concatenate(draws(c, 1, 4))
    wt = L.lmhead_trim(w_dev, dev_i32(ids))
    for p in epi_paths(L, 4):
        out = L.draft_project_logits(dev_bf16(h_np), w_dev, None, path=p)
        check_logits(h_np, inp["W"], None, None, out.cpu().numpy())
        sc = L.draft_project_logits(dev_bf16(h_np), wt, dev_i32(ids), n=c.n, path=p)
        check_logits(h_np, oracle.oracle_trim(inp["W"], ids), ids, c.n, sc.cpu().numpy())


def test_logits_16k_scatter_m3(L):
    inp = config_inputs(3)
    c, ids = inp["config"], inp["ids"]
    wt = L.lmhead_trim(device_weights(3), dev_i32(ids))
    h_np = draws(c, 3, 1)[0]
    for p in epi_paths(L, 3):
        sc = L.draft_project_logits(dev_bf16(h_np), wt, dev_i32(ids), n=c.n, path=p)
        st = check_logits(h_np, oracle.oracle_trim(inp["W"], ids), ids, c.n, sc.cpu().numpy())
        log(f"[logits 16k M=3] path={p} max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")
        # the argmax of the scattered logits is the shortlist draft
        a_id, _ = L.draft_project_argmax(dev_bf16(h_np), wt, dev_i32(ids))
        res = oracle.oracle_project_argmax(h_np, oracle.oracle_trim(inp["W"], ids), ids)
        sure = res.gap > 1e-2
        assert np.array_equal(sc.argmax(dim=1).cpu().numpy()[sure], a_id.cpu().numpy()[sure])


def test_logits_full_head_m1_and_m8(L):
    inp = config_inputs(2)
    c = inp["config"]
    w_dev = device_weights(2)
    for m, p in ((1, L.LMH_PATH_VALU), (8, L.LMH_PATH_MFMA)):
        h_np = synth.hidden(c.h_seed[0] + 11, m, m, c.k)
        out = L.draft_project_logits(dev_bf16(h_np), w_dev, None, path=p)
        st = check_logits(h_np, inp["W"], None, None, out.cpu().numpy())
        log(f"[logits full M={m}] path={p} max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")


@pytest.mark.parametrize("m,k,r", [(1, 8, 1), (2, 264, 77), (5, 2560, 1000), (24, 520, 300), (32, 8192, 50)])
def test_logits_edges(L, m, k, r):
    w_np = synth.normal_bf16(5000 + r, r, k, 0.02)
    h_np = synth.hidden(6000 + k, m, m, k)
    n = 3 * r + 5
    d2t = (np.arange(r, dtype=np.int32) * 3 + 2)
    w_dev = dev_bf16(w_np)
    for p in epi_paths(L, m, k):
        out = L.draft_project_logits(dev_bf16(h_np), w_dev, None, path=p)
        check_logits(h_np, w_np, None, None, out.cpu().numpy())
        sc = L.draft_project_logits(dev_bf16(h_np), w_dev, dev_i32(d2t), n=n, path=p)
        check_logits(h_np, w_np, d2t, n, sc.cpu().numpy())


def test_logits_skip_ids_outside_vocabulary(L):
    """d2t entries outside [0, N) are skipped, not written out of bounds."""
    r, k, n = 50, 256, 60
    w_np = synth.normal_bf16(7001, r, k, 0.02)
    h_np = synth.hidden(7002, 0, 2, k)
    d2t = np.arange(r, dtype=np.int32)
    d2t[[3, 10, 49]] = [-5, n, 1 << 30]
    buf = torch.full((2 * n + 256,), 12345.0, device="cuda")
    out = buf[:2 * n].view(2, n)
    L.draft_project_logits(dev_bf16(h_np), dev_bf16(w_np), dev_i32(d2t), n=n, out=out)
    torch.cuda.synchronize()
    assert bool((buf[2 * n:] == 12345.0).all()), "write past the output"
    got = out.cpu().numpy()
    keep = np.ones(r, bool)
    keep[[3, 10, 49]] = False
    ref = oracle.oracle_logits(h_np, w_np)
    assert np.allclose(got[:, d2t[keep]], ref[:, keep], atol=1e-3)
    assert np.all(np.isneginf(got[:, [3, 10, 49]]))   # those columns got no row
