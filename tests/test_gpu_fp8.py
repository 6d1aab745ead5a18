"""FP8 (E4M3, one scale per row) head through the C ABI, against the fp64
oracle: the load-time quantizer bit for bit, and the argmax over the
dequantized head on both kernels wherever both accept the shape.

The oracle quantizes the bf16 head itself (no expected value comes from
the GPU); rows are independent, so the tests run it over row blocks in a
thread pool.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from parity import ParityStats, check_fp8
from test_gpu_parity import config_inputs, dev_bf16, dev_i32, device_weights, draws, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def oracle_quantize_rows(w_bits, block=4096):
    """oracle_quantize_fp8 over row blocks in threads (rows are independent)."""
    n = w_bits.shape[0]
    if n <= block:
        return oracle.oracle_quantize_fp8(w_bits)
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(lambda r0: oracle.oracle_quantize_fp8(w_bits[r0:r0 + block]), range(0, n, block)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


_oq = {}


def oracle_head(cfg, trimmed):
    """(W, codes, scale) the oracle quantized itself; the full head (shared by
    configs 2-5) stays cached, a trimmed head replaces the previous one."""
    c = synth.CONFIGS[cfg]
    key = (cfg, "trim") if trimmed else ("full", c.w_seed, c.n, c.k)
    if key not in _oq:
        inp = config_inputs(cfg)
        w = oracle.oracle_trim(inp["W"], inp["ids"]) if trimmed else inp["W"]
        log(f"[oracle] quantizing config {cfg} {'trimmed' if trimmed else 'full'} ({w.shape[0]} rows)")
        for old in [k for k in _oq if k[1] == "trim"]:
            del _oq[old]
        _oq[key] = (w, *oracle_quantize_rows(w))
    return _oq[key]


def fp8_paths(L, m):
    return [L.LMH_PATH_VALU, L.LMH_PATH_MFMA] if m <= 4 else [L.LMH_PATH_MFMA]


def gpu_quantize(L, w_dev):
    q, s = L.lmhead_quantize_fp8(w_dev)
    torch.cuda.synchronize()
    return q, s


def run_and_check_fp8(L, hs, codes, scale, q_dev, s_dev, d2t_np, tag):
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax_fp8(stack, codes, scale, d2t_np, keep_logits=True)
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in fp8_paths(L, hs[0].shape[0]):
        ids, lgs = [], []
        for h in hs:
            i, l = L.draft_project_argmax_fp8(dev_bf16(h), q_dev, s_dev, d2t_dev, p)
            ids.append(i.cpu().numpy())
            lgs.append(l.cpu().numpy())
        st = ParityStats()
        st.add(check_fp8(stack, codes, scale, d2t_np, np.concatenate(ids), np.concatenate(lgs), res))
        log(f"[{tag}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e} "
            f"err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


# --------------------------------------------------------------------------
# quantizer, bit for bit
# --------------------------------------------------------------------------

def _special_head(rng, k):
    """Rows that exercise the encoder: ties (a power-of-two scale and
    entries on E4M3 midpoints), subnormal codes, signed zeros, an all-zero
    row, a single nonzero, and ordinary rows."""
    vals = np.array([oracle.e4m3_decode(np.array([c], np.uint8))[0] for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    rows = []
    s = 2.0 ** -3
    row = np.resize(mids * s, k) * np.resize([1, -1], k)
    row[0] = 448 * s
    rows.append(row)
    row = np.resize(vals * s, k)
    row[1] = -448 * s
    rows.append(row)
    row = rng.standard_normal(k) * 1e-3
    row[:8] = [2.0 ** -20, -2.0 ** -21, 3 * 2.0 ** -22, 0.0, -0.0, 1.0, 2.0 ** -13, -(2.0 ** -12)]
    rows.append(row)
    rows.append(np.zeros(k))
    rows.append(-np.zeros(k))
    one = np.zeros(k)
    one[k // 2] = -3.5
    rows.append(one)
    for _ in range(10):
        rows.append(rng.standard_normal(k) * 0.02)
    return synth.bf16_from_f32(np.array(rows, dtype=np.float32))


@pytest.mark.parametrize("k", [16, 48, 256, 2560, 8192])
def test_quantize_bit_exact(L, k):
    rng = np.random.default_rng(900 + k)
    w = _special_head(rng, k)
    q, s = gpu_quantize(L, dev_bf16(w))
    codes, scale = oracle.oracle_quantize_fp8(w)
    assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), scale.view(np.uint32))


def test_quantize_full_head_sampled_rows(L):
    """The full 248,320-row head on the GPU; 3,000 rows compared with the
    oracle bit for bit (rows are quantized independently)."""
    inp = config_inputs(2)
    q, s = gpu_quantize(L, device_weights(2))
    rows = np.unique(np.concatenate([[0, 1, q.shape[0] - 1],
                                     np.random.default_rng(5).integers(0, q.shape[0], 3000)]))
    codes, scale = oracle.oracle_quantize_fp8(inp["W"][rows])
    sel = torch.from_numpy(rows).cuda()
    assert np.array_equal(q[sel].cpu().numpy(), codes)
    assert np.array_equal(s[sel].cpu().numpy().view(np.uint32), scale.view(np.uint32))


def test_quantize_rejects_and_writes_nothing(L):
    w = dev_bf16(synth.normal_bf16(3, 10, 40, 0.02))          # K = 40 is not a multiple of 16
    q = torch.full((10, 40), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((10,), 3.0, device="cuda")
    code = L.lib().lmhead_quantize_fp8(w.data_ptr(), 10, 40, q.data_ptr(), s.data_ptr(), None)
    assert code == L.LMH_EINVAL
    torch.cuda.synchronize()
    assert bool((q == 7).all()) and bool((s == 3.0).all())


# --------------------------------------------------------------------------
# projection + argmax over the dequantized head
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,trimmed,m,n", [
    (1, False, 1, 32), (1, True, 1, 32), (2, False, 1, 16), (3, True, 3, 16), (4, True, 1, 16),
    (4, True, 4, 16), (5, True, 24, 16), (5, False, 24, 16),
])
def test_fp8_argmax_configs(L, cfg, trimmed, m, n):
    inp = config_inputs(cfg)
    c = inp["config"]
    w, codes, scale = oracle_head(cfg, trimmed)
    d2t = inp["ids"].astype(np.int32) if trimmed else None
    if trimmed:
        w_dev = L.lmhead_trim(device_weights(cfg), dev_i32(inp["ids"]))
    else:
        w_dev = device_weights(cfg)
    q_dev, s_dev = gpu_quantize(L, w_dev)
    del w_dev
    hs = draws(c, m, n)
    run_and_check_fp8(L, hs, codes, scale, q_dev, s_dev, d2t, f"fp8 config {cfg} M={m}")


EDGE = [(1, 16, 1), (2, 16, 3), (1, 32, 2), (3, 48, 17), (4, 272, 1000), (1, 2560, 5),
        (5, 48, 700), (8, 2560, 33), (17, 256, 999), (24, 2560, 1000), (32, 8192, 40),
        (29, 2560, 600), (1, 8192, 2047), (4, 8192, 64)]


@pytest.mark.parametrize("m,k,r", EDGE, ids=[f"M{m}-K{k}-R{r}" for m, k, r in EDGE])
def test_fp8_edges(L, m, k, r):
    w = synth.normal_bf16(7000 + r, r, k, 0.02)
    codes, scale = oracle.oracle_quantize_fp8(w)
    q_dev, s_dev = gpu_quantize(L, dev_bf16(w))
    hs = [synth.hidden(8000 + k, d, m, k) for d in range(2)]
    d2t = (np.arange(r, dtype=np.int32)[::-1] * 7 + 11).copy()
    run_and_check_fp8(L, hs, codes, scale, q_dev, s_dev, None, f"fp8 edge M={m} K={k} R={r}")
    run_and_check_fp8(L, hs[:1], codes, scale, q_dev, s_dev, d2t, f"fp8 edge d2t M={m} K={k} R={r}")


@pytest.mark.parametrize("m", [1, 3, 6])
def test_fp8_exact_ties_first_row(L, m):
    """Integer weights with a power-of-two row scale make every logit exact
    in fp32: equal maxima must resolve to the smallest row, across
    workgroups."""
    rng = np.random.default_rng(31 + m)
    r, k = 150_000, 128
    wi = rng.integers(-3, 4, size=(r, k)).astype(np.float32)
    wi[:, 0] = 448.0 / 64                      # every row's maximum: scale = 2**-6 exactly
    hi = rng.integers(-1, 2, size=(m, k)).astype(np.float32)
    hi[:, 0] = 0
    for j in range(m):
        for rr in (140_001 - j, 7 + j, 77_777):
            wi[rr, 1:] = 3 * np.sign(hi[j, 1:])
    w = synth.bf16_from_f32(wi)
    h = synth.bf16_from_f32(hi)
    codes, scale = oracle.oracle_quantize_fp8(w)
    assert np.all(scale == np.float32(2.0 ** -6))
    res = oracle.oracle_project_argmax_fp8(h, codes, scale)
    q_dev, s_dev = gpu_quantize(L, dev_bf16(w))
    for p in fp8_paths(L, m):
        i, lg = L.draft_project_argmax_fp8(dev_bf16(h), q_dev, s_dev, None, p)
        assert np.array_equal(i.cpu().numpy(), res.id), (p, i.cpu().numpy(), res.id)
        assert np.array_equal(lg.cpu().numpy().astype(np.float64), res.logit)


def test_fp8_repeat_bit_identical_and_rejects(L):
    w = synth.normal_bf16(55, 5000, 2560, 0.02)
    q_dev, s_dev = gpu_quantize(L, dev_bf16(w))
    h = dev_bf16(synth.hidden(56, 0, 6, 2560))
    ws = L.new_workspace()
    a = L.draft_project_argmax_fp8(h, q_dev, s_dev, workspace=ws)
    ws.fill_(0xAB)
    b = L.draft_project_argmax_fp8(h, q_dev, s_dev, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    oid = torch.full((6,), 77, dtype=torch.int32, device="cuda")
    olg = torch.full((6,), 5.0, device="cuda")
    lib = L.lib()
    bad = [
        dict(k=2568), dict(m=0), dict(m=33), dict(r=0), dict(path=1), dict(sp=s_dev.data_ptr() + 2),
        dict(qp=q_dev.data_ptr() + 8), dict(wsb=16),
    ]
    for cs in bad:
        code = lib.draft_project_argmax_fp8(
            h.data_ptr(), cs.get("m", 6), cs.get("k", 2560), cs.get("qp", q_dev.data_ptr()),
            cs.get("sp", s_dev.data_ptr()), cs.get("r", 5000), None, oid.data_ptr(), olg.data_ptr(),
            ws.data_ptr(), cs.get("wsb", ws.numel()), cs.get("path", 0), None)
        assert code in (L.LMH_EINVAL, L.LMH_EWORKSPACE), cs
    torch.cuda.synchronize()
    assert bool((oid == 77).all()) and bool((olg == 5.0).all())


# --------------------------------------------------------------------------
# top k over the FP8 head
# --------------------------------------------------------------------------

def run_topk_fp8(L, h, codes, scale, d2t_np, topk, tag):
    from parity import check_topk_fp8
    res = oracle.oracle_project_topk_fp8(h, codes, scale, d2t_np, topk)
    q_dev, s_dev = torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda()
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
        i, lg = L.draft_project_topk_fp8(dev_bf16(h), q_dev, s_dev, d2t_dev, topk, path=p)
        st = check_topk_fp8(h, codes, scale, d2t_np, i.cpu().numpy(), lg.cpu().numpy(), res)
        log(f"[{tag}] path={p} k={topk} positions={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e} "
            f"err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


@pytest.mark.parametrize("cfg,trimmed,m,topk", [(2, False, 1, 8), (5, False, 24, 16), (3, True, 3, 4),
                                                (5, True, 24, 8)])
def test_fp8_topk_configs(L, cfg, trimmed, m, topk):
    inp = config_inputs(cfg)
    w, codes, scale = oracle_head(cfg, trimmed)
    d2t = inp["ids"].astype(np.int32) if trimmed else None
    h = draws(inp["config"], m, 1)[0]
    run_topk_fp8(L, h, codes, scale, d2t, topk, f"fp8 top-k config {cfg} M={m}")


FP8_TOPK_EDGE = [(1, 16, 1, 16), (3, 48, 5, 4), (17, 272, 1000, 16), (32, 8192, 40, 8), (24, 2560, 3001, 2)]


@pytest.mark.parametrize("m,k,r,topk", FP8_TOPK_EDGE, ids=[f"M{m}-K{k}-R{r}-k{t}" for m, k, r, t in FP8_TOPK_EDGE])
def test_fp8_topk_edges(L, m, k, r, topk):
    w = synth.normal_bf16(17000 + r, r, k, 0.02)
    codes, scale = oracle.oracle_quantize_fp8(w)
    h = synth.hidden(18000 + k, 1, m, k)
    d2t = (np.arange(r, dtype=np.int32)[::-1] * 5 + 7).copy()
    run_topk_fp8(L, h, codes, scale, None, topk, f"fp8 top-k edge M={m} K={k} R={r}")
    run_topk_fp8(L, h, codes, scale, d2t, topk, f"fp8 top-k edge d2t M={m} K={k} R={r}")


def test_fp8_topk1_matches_argmax_and_rejects(L):
    w = synth.normal_bf16(401, 20000, 2560, 0.02)
    q, s = gpu_quantize(L, dev_bf16(w))
    for m in (1, 5, 24):
        h = dev_bf16(synth.hidden(402, m, m, 2560))
        a = L.draft_project_argmax_fp8(h, q, s, None, L.LMH_PATH_MFMA)
        t = L.draft_project_topk_fp8(h, q, s, None, 1)
        assert torch.equal(t[0][:, 0], a[0]) and torch.equal(t[1][:, 0], a[1]), m
    h = dev_bf16(synth.hidden(403, 0, 2, 2560))
    with pytest.raises(L.LmheadError):
        L.draft_project_topk_fp8(h, q, s, None, 4, path=L.LMH_PATH_VALU)
