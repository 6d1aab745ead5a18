"""HIP path against the fp64 oracle on the five workloads, through the C ABI.

Every projection test runs each kernel that accepts the shape (registers /
VALU for M <= 4, matrix cores for any M) and applies the parity rule of
tests/parity.py to every hidden row of many seeded draws.  The gather is
compared bit for bit.  Full-size cases use the launch configuration the
benchmark times (the library's default kernel choice on the full head).
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from devcopy import dev_bf16, dev_i32  # noqa: F401  (also used by the other GPU modules)
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
    """Every kernel that accepts (m, k): the VALU path takes M <= 8 with
    M * ceil(K / 512) <= 40 (include/lmhead.h); the matrix-core path takes all."""
    ps = [L.LMH_PATH_MFMA]
    if m <= 8 and m * ((k // 8 + 63) // 64) <= 40:
        ps.insert(0, L.LMH_PATH_VALU)
    return ps


_inputs = {}


def config_inputs(i):
    if i not in _inputs:
        log(f"[inputs] generating config {i}")
        _inputs[i] = synth.make_config(i)
    return _inputs[i]


_dev_w = {}


def device_weights(i):
    c = synth.CONFIGS[i]
    key = (c.w_seed, c.n, c.k)
    if key not in _dev_w:
        _dev_w.clear()
        _dev_w[key] = dev_bf16(config_inputs(i)["W"])
    return _dev_w[key]


def draws(c, m, n):
    """n independent draws of an [m, K] hidden block for config c."""
    seed = c.h_seed[c.ms.index(m)] if m in c.ms else c.h_seed[0]
    return [synth.hidden(seed, d, m, c.k) for d in range(n)]


def run_and_check(L, hs, w_np, w_dev, d2t_np, paths, tag):
    """One GPU call per draw and path; the oracle is run once on all draws
    stacked (rows are independent)."""
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax(stack, w_np, d2t_np, keep_logits=True)
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in paths:
        st = ParityStats()
        ids, logits = [], []
        for h in hs:
            i, l = L.draft_project_argmax_path(dev_bf16(h), w_dev, d2t_dev, p)
            ids.append(i.cpu().numpy())
            logits.append(l.cpu().numpy())
        st.add(check(stack, w_np, d2t_np, np.concatenate(ids), np.concatenate(logits), res))
        log(f"[{tag}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e} "
            f"err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


# --------------------------------------------------------------------------
# gather
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_trim_bit_exact(L, cfg):
    inp = config_inputs(cfg)
    ids = inp["ids"]
    w_dev = device_weights(cfg)
    log(f"[trim] config {cfg} S={ids.size}")
    got = L.lmhead_trim(w_dev, dev_i32(ids))
    torch.cuda.synchronize()
    want = oracle.oracle_trim(inp["W"], ids)
    assert np.array_equal(got.cpu().numpy().view(np.uint16), want)


def test_trim_rejects_out_of_range_and_writes_nothing(L):
    w = dev_bf16(synth.normal_bf16(5, 300, 64, 0.02))
    out = torch.full((3, 64), 0x1234, dtype=torch.int16, device="cuda")
    for bad in ([0, 300, 2], [0, -1, 5]):
        code = L.lib().lmhead_trim(w.data_ptr(), 300, 64, dev_i32(bad).data_ptr(), 3,
                                   out.data_ptr(), None)
        assert code == L.LMH_ERANGE
    torch.cuda.synchronize()
    assert bool((out == 0x1234).all())


def test_trim_duplicates_and_order(L):
    w_np = synth.normal_bf16(6, 1000, 264, 0.02)
    ids = np.array([999, 0, 5, 5, 999, 17, 3], dtype=np.int32)
    got = L.lmhead_trim(dev_bf16(w_np), dev_i32(ids))
    assert np.array_equal(got.cpu().numpy().view(np.uint16), oracle.oracle_trim(w_np, ids))


# --------------------------------------------------------------------------
# projection + argmax + d2t on the five workloads
# --------------------------------------------------------------------------

def test_config1_tiny(L):
    inp = config_inputs(1)
    c = inp["config"]
    ids = inp["ids"]
    w_dev = device_weights(1)
    hs = draws(c, 1, 64)
    run_and_check(L, hs, inp["W"], w_dev, None, paths_for(L, 1, c.k), "tiny full")
    wt = L.lmhead_trim(w_dev, dev_i32(ids))
    run_and_check(L, hs, oracle.oracle_trim(inp["W"], ids), wt, ids, paths_for(L, 1, c.k),
                  "tiny trim")


def test_config2_full_m1(L):
    inp = config_inputs(2)
    c = inp["config"]
    hs = draws(c, 1, 16)
    run_and_check(L, hs, inp["W"], device_weights(2), None, paths_for(L, 1, c.k), "full M=1")


@pytest.mark.parametrize("m", [2, 3])
def test_full_head_two_and_three_rows(L, m):
    """The full head at M = 2 (the tiled kernel's unconditional loop) and
    M = 3 (the row-order kernel's two-buffer loop), on every kernel that
    takes the shape."""
    inp = config_inputs(2)
    c = inp["config"]
    hs = [synth.hidden(250 + m, d, m, c.k) for d in range(16)]
    run_and_check(L, hs, inp["W"], device_weights(2), None, paths_for(L, m, c.k), f"full M={m}")


@pytest.mark.parametrize("r", [131_071, 131_072])
def test_four_rows_at_the_head_size_boundary(L, r):
    """The argmax at M = 4 takes the VALU kernel on both sides of 131,072
    head rows (the size where the one- and two-row argmax change their load
    loop): on both sides the default call matches the oracle and, bit for
    bit, the VALU kernel, and the matrix-core kernel meets the parity rule
    too."""
    inp = config_inputs(2)
    c = inp["config"]
    w_np, w_dev = inp["W"][:r], device_weights(2)[:r]
    want = L.LMH_PATH_VALU
    assert L.draft_project_auto_path_rows(4, c.k, r) == want
    hs = [synth.hidden(4040, d, 4, c.k) for d in range(16)]
    run_and_check(L, hs, w_np, w_dev, None, [L.LMH_PATH_AUTO, L.LMH_PATH_MFMA], f"{r} rows M=4")
    for h in hs:
        a = L.draft_project_argmax_path(dev_bf16(h), w_dev, None, L.LMH_PATH_AUTO)
        b = L.draft_project_argmax_path(dev_bf16(h), w_dev, None, want)
        assert np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
        assert np.array_equal(a[1].cpu().numpy().view(np.uint32), b[1].cpu().numpy().view(np.uint32))


def test_config3_16k_m3(L):
    inp = config_inputs(3)
    c = inp["config"]
    ids = inp["ids"]
    wt = L.lmhead_trim(device_weights(3), dev_i32(ids))
    hs = draws(c, 3, 16)
    run_and_check(L, hs, oracle.oracle_trim(inp["W"], ids), wt, ids, paths_for(L, 3, c.k),
                  "16k M=3")


@pytest.mark.parametrize("m", [1, 4])
def test_config4_32k(L, m):
    inp = config_inputs(4)
    c = inp["config"]
    ids = inp["ids"]
    wt = L.lmhead_trim(device_weights(4), dev_i32(ids))
    hs = draws(c, m, 16)
    run_and_check(L, hs, oracle.oracle_trim(inp["W"], ids), wt, ids, paths_for(L, m, c.k),
                  f"32k M={m}")


def test_config5_m24_full_and_52k(L):
    inp = config_inputs(5)
    c = inp["config"]
    ids = inp["ids"]
    w_dev = device_weights(5)
    hs = draws(c, 24, 16)
    run_and_check(L, hs, inp["W"], w_dev, None, paths_for(L, 24, c.k), "full M=24")
    wt = L.lmhead_trim(w_dev, dev_i32(ids))
    run_and_check(L, hs, oracle.oracle_trim(inp["W"], ids), wt, ids, paths_for(L, 24, c.k),
                  "52k M=24")


# --------------------------------------------------------------------------
# determinism and workspace contract
# --------------------------------------------------------------------------

def test_repeated_calls_bit_identical_any_workspace_contents(L):
    """Results do not depend on what the workspace held before the call."""
    w_dev = device_weights(2)
    c = synth.CONFIGS[2]
    ws = L.new_workspace()
    for m in (1, 3, 24):
        h = dev_bf16(synth.hidden(777, 0, m, c.k))
        first = None
        for fill in (0xFF, 0x00, 0x5A, 0xFF):
            ws.fill_(fill)
            i, l = L.draft_project_argmax(h, w_dev, workspace=ws)
            got = (i.cpu().numpy().copy(), l.cpu().numpy().view(np.uint32).copy())
            if first is None:
                first = got
            assert np.array_equal(got[0], first[0]) and np.array_equal(got[1], first[1])


def test_separate_stream_and_workspace(L):
    w_np = synth.normal_bf16(8, 5000, 2560, 0.02)
    w_dev = dev_bf16(w_np)
    h_np = synth.hidden(9, 0, 2, 2560)
    s = torch.cuda.Stream()
    ws = L.new_workspace()
    with torch.cuda.stream(s):
        h = dev_bf16(h_np)
        i, l = L.draft_project_argmax(h, w_dev, workspace=ws, stream=s)
    s.synchronize()
    check(h_np, w_np, None, i.cpu().numpy(), l.cpu().numpy())


# --------------------------------------------------------------------------
# edge shapes: ragged row counts, small and large K, every M class
# --------------------------------------------------------------------------

EDGE = [
    (1, 8, 1), (1, 8, 2), (1, 16, 3), (2, 24, 63), (3, 256, 64), (4, 264, 65),
    (1, 520, 1000), (1, 2560, 1), (1, 2560, 7), (4, 2560, 4097), (2, 4096, 333),
    (1, 8192, 1501), (5, 264, 129), (8, 2560, 33), (6, 2560, 777), (7, 3072, 50), (16, 2560, 517), (17, 256, 700),
    (24, 2560, 1031), (31, 520, 99), (32, 2560, 2050), (32, 8192, 300), (13, 8, 77),
    # either side of the head size where the VALU argmax switches load loops
    (1, 264, 131_071), (1, 264, 131_072), (3, 264, 131_071), (4, 264, 131_072),
]


@pytest.mark.parametrize("m,k,r", EDGE, ids=[f"M{m}-K{k}-R{r}" for m, k, r in EDGE])
def test_edge_shapes(L, m, k, r):
    w_np = synth.normal_bf16(1000 + r, r, k, 0.02)
    h_np = synth.hidden(2000 + k, m, m, k)
    w_dev = dev_bf16(w_np)
    d2t = (np.arange(r, dtype=np.int32) * 7 + 3)
    for p in paths_for(L, m, k):
        for dd in (None, d2t):
            i, l = L.draft_project_argmax_path(dev_bf16(h_np), w_dev,
                                               dev_i32(dd) if dd is not None else None, p)
            check(h_np, w_np, dd, i.cpu().numpy(), l.cpu().numpy())


def _int_bf16(vals):
    f = np.asarray(vals, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("m", [1, 3, 5, 24])
def test_exact_ties_take_smallest_row(L, m):
    """Small-integer inputs make every logit exact in fp32, whatever the
    summation order; the maximum is planted on several far-apart rows, so
    the kernels must break the tie across waves and workgroups."""
    rng = np.random.default_rng(31 + m)
    r, k = 200_003, 256
    wi = rng.integers(-2, 3, size=(r, k)).astype(np.float32)
    hi = rng.integers(-2, 3, size=(m, k)).astype(np.float32)
    for j in range(m):
        rows = [150_001 + j, 99_000 + 17 * j, 123_456 - j, 200_002 - j]
        for rr in rows:
            wi[rr] = np.sign(hi[j]) * 2          # |logit| = 2 * sum|h| is maximal
    w_np, h_np = _int_bf16(wi), _int_bf16(hi)
    res = oracle.oracle_project_argmax(h_np, w_np)
    w_dev = dev_bf16(w_np)
    for p in paths_for(L, m, k):
        i, l = L.draft_project_argmax_path(dev_bf16(h_np), w_dev, None, p)
        assert np.array_equal(i.cpu().numpy(), res.idx), (p, i.cpu().numpy(), res.idx)
        assert np.array_equal(l.cpu().numpy().astype(np.float64), res.logit)


def test_all_rows_equal_and_negative(L):
    k = 520
    w_np = np.tile(_int_bf16(-np.ones(k)), (3000, 1))
    h_np = _int_bf16(np.ones((4, k)))
    w_dev = dev_bf16(w_np)
    for m in (1, 4):
        for p in paths_for(L, m, k):
            i, l = L.draft_project_argmax_path(dev_bf16(h_np[:m]), w_dev, None, p)
            assert np.all(i.cpu().numpy() == 0)
            assert np.all(l.cpu().numpy() == -k)


# --------------------------------------------------------------------------
# host-side rejection leaves outputs untouched
# --------------------------------------------------------------------------

def test_rejected_calls_write_nothing(L):
    w = dev_bf16(synth.normal_bf16(4, 100, 256, 0.02))
    h = dev_bf16(synth.hidden(4, 0, 2, 256))
    oid = torch.full((2,), 77, dtype=torch.int32, device="cuda")
    olog = torch.full((2,), 5.0, dtype=torch.float32, device="cuda")
    ws = L.new_workspace()
    lib = L.lib()
    cases = [
        dict(m=0), dict(m=33), dict(k=12), dict(r=0), dict(hp=h.data_ptr() + 2),
        dict(wsb=8), dict(wsp=ws.data_ptr() + 4), dict(path=9),
    ]
    ws_before = ws.clone()
    for cs in cases:
        code = lib.draft_project_argmax_path(
            cs.get("hp", h.data_ptr()), cs.get("m", 2), cs.get("k", 256), w.data_ptr(),
            cs.get("r", 100), None, oid.data_ptr(), olog.data_ptr(), cs.get("wsp", ws.data_ptr()),
            cs.get("wsb", ws.numel()), cs.get("path", 0), None)
        assert code in (L.LMH_EINVAL, L.LMH_EWORKSPACE), cs
    torch.cuda.synchronize()
    assert bool((oid == 77).all()) and bool((olog == 5.0).all())
    assert torch.equal(ws, ws_before)


# --------------------------------------------------------------------------
# the measurement helper runs the same kernels
# --------------------------------------------------------------------------

def test_binding_rejects_host_and_short_buffers(L):
    """The binding refuses a host workspace or host outputs next to device
    inputs, and outputs or a d2t of the wrong size, before any launch."""
    h = dev_bf16(synth.hidden(7, 0, 3, 512))
    W = dev_bf16(synth.normal_bf16(8, 100, 512, 0.02))
    ws_host = torch.empty(L.draft_project_workspace_bytes(32), dtype=torch.uint8)
    bad = [
        dict(workspace=ws_host),
        dict(out_id=torch.empty(3, dtype=torch.int32)),
        dict(out_logit=torch.empty(3, dtype=torch.float32)),
        dict(out_id=torch.empty(2, dtype=torch.int32, device="cuda")),
        dict(out_logit=torch.empty(3, dtype=torch.float64, device="cuda")),
    ]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)):
            L.draft_project_argmax(h, W, **kw)
    with pytest.raises(ValueError):
        L.draft_project_argmax(h, W, torch.arange(99, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        L.draft_project_argmax(h, W, torch.arange(100, dtype=torch.int32))
    q, sc = L.lmhead_quantize_fp8(W)
    with pytest.raises(ValueError):
        L.draft_project_argmax_fp8(h, q, sc, workspace=ws_host)
    with pytest.raises(ValueError):
        L.draft_project_argmax_fp8(h, q, sc, out_id=torch.empty(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()


def test_bench_time_argmax_matches_call(L):
    inp = config_inputs(1)
    c = inp["config"]
    w_dev = device_weights(1)
    h = dev_bf16(inp["h"][1])
    want_id, want_lg = L.draft_project_argmax(h, w_dev, None)
    ws = L.new_workspace()
    oid = torch.empty(1, dtype=torch.int32, device="cuda")
    olg = torch.empty(1, dtype=torch.float32, device="cuda")
    for p in paths_for(L, 1, c.k):
        ms = L.lmhead_bench_time_argmax(h, [w_dev, w_dev], None, p, 7, oid, olg, ws)
        assert 0.0 < ms < 100.0
        assert torch.equal(oid, want_id) and torch.equal(olg, want_lg)
