"""MXFP4 head (E2M1 in blocks of 32, one E8M0 scale per block) through the C
ABI, against the fp64 oracle: the load-time quantizer bit for bit, and the
argmax over the dequantized head on the matrix-core kernel (the only one
that takes this format).

The oracle quantizes every head itself and its codes are what the argmax
tests upload, so no expected value and no argmax input comes from the GPU.
Rows are quantized independently: the oracle runs over row blocks in a
thread pool, and a shortlisted head is the oracle's full-head codes at the
listed rows.

The library keeps the block scales in a tiled layout (16-row tiles, groups
of 16 blocks, 256 bytes per tile and group); tile_scales / untile_scales
below rearrange the oracle's row-major scales to and from it, following the
layout the header documents.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from devcopy import dev_u8
from parity import ParityStats, check_mxfp4
from test_gpu_parity import config_inputs, dev_bf16, dev_i32, device_weights, draws, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def tile_scales(sc, fill=0):
    """Row-major scales [R, B] -> the tiled layout [ceil(R/16), ceil(B/16),
    16, 16]: element [t, g, i, j] is the scale of row 16 t + i, block 16 g + j
    (padding = fill)."""
    r, nblk = sc.shape
    t, nb = (r + 15) // 16, (nblk + 15) // 16
    pad = np.full((t * 16, nb * 16), fill, dtype=np.uint8)
    pad[:r, :nblk] = sc
    return np.ascontiguousarray(pad.reshape(t, 16, nb, 16).transpose(0, 2, 1, 3))


def untile_scales(tiled, r, nblk):
    t, nb = tiled.shape[:2]
    return np.ascontiguousarray(tiled.transpose(0, 2, 1, 3).reshape(t * 16, nb * 16)[:r, :nblk])


def oracle_quantize_rows(w_bits, block=2048):
    """oracle_quantize_mxfp4 over row blocks in threads (rows are independent)."""
    n = w_bits.shape[0]
    if n <= block:
        return oracle.oracle_quantize_mxfp4(w_bits)
    done = [0]

    def one(r0):
        out = oracle.oracle_quantize_mxfp4(w_bits[r0:r0 + block])
        done[0] += 1
        if done[0] % 16 == 0:
            log(f"[oracle] mxfp4 blocks done: {done[0]} of {(n + block - 1) // block}")
        return out

    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(one, range(0, n, block)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


_full = {}


def oracle_full_head():
    """(codes, scales) of the full 248,320-row head, quantized by the oracle
    once per session (about a minute on 16 threads)."""
    if "q" not in _full:
        w = config_inputs(2)["W"]
        log(f"[oracle] quantizing the full head to MXFP4 ({w.shape[0]} rows)")
        _full["q"] = oracle_quantize_rows(w)
    return _full["q"]


def gpu_quantize(L, w_dev):
    q, s = L.lmhead_quantize_mxfp4(w_dev)
    torch.cuda.synchronize()
    return q, s


def run_and_check(L, hs, codes, scales, d2t_np, tag, q_dev=None, s_dev=None):
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax_mxfp4(stack, codes, scales, d2t_np, keep_logits=True)
    if q_dev is None:
        q_dev, s_dev = dev_u8(codes), dev_u8(tile_scales(scales))
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
        ids, lgs = [], []
        for h in hs:
            i, l = L.draft_project_argmax_mxfp4(dev_bf16(h), q_dev, s_dev, d2t_dev, p)
            ids.append(i.cpu().numpy())
            lgs.append(l.cpu().numpy())
        st = ParityStats()
        st.add(check_mxfp4(stack, codes, scales, d2t_np, np.concatenate(ids), np.concatenate(lgs), res))
        log(f"[{tag}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e} "
            f"err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


# --------------------------------------------------------------------------
# quantizer, bit for bit
# --------------------------------------------------------------------------

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _special_head(rng, k):
    """Rows that exercise the encoder and the block scale: every midpoint
    between neighbouring E2M1 values (ties to even) under several block
    scales, values between 6 and 8 times the scale (saturation), signed
    zeros, all-zero blocks, a lone nonzero, block maxima at extreme
    exponents (large, tiny, bf16 subnormal, clamped at -127), and ordinary
    rows of several widths."""
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    rows = []
    for s in (-7, -3, 0, 5):
        base = np.concatenate([mids, E2M1, -mids, -E2M1])              # 30 values
        row = np.resize(np.concatenate([base, [4.0, 7.5]]), k)          # 7.5 * 2^s saturates
        rows.append(row * 2.0 ** s)
    row = np.resize([7.0, 6.5, 6.25, 5.5, 4.5, 3.25, 2.75, 1.9], k)     # between 4 and 8: s = 0
    rows.append(row * np.resize([1, -1, -1, 1], k))
    rows.append(np.zeros(k))
    rows.append(-np.zeros(k))
    one = np.zeros(k)
    one[k // 2 + 3] = -3.5
    rows.append(one)
    sign = np.resize([1.0, -1.0, 1.0, 1.0, -1.0], k)
    for e in (120, 60, -60, -120, -126, -130, -133):
        rows.append(np.resize([1.0, 0.75, 0.3, 0.1, 0.02, 0.0, 1.5, 0.9], k) * 2.0 ** e * sign)
    for sd in (1.0, 0.02, 1e-4, 300.0):
        rows.append(rng.standard_normal(k) * sd)
    heavy = rng.standard_normal(k) * 0.02
    heavy[::37] *= 50                                                   # outliers inside blocks
    rows.append(heavy)
    return synth.bf16_from_f32(np.array(rows, dtype=np.float32))


@pytest.mark.parametrize("k", [32, 64, 96, 512, 2560, 8192])
def test_quantize_bit_exact(L, k):
    rng = np.random.default_rng(1900 + k)
    w = _special_head(rng, k)
    q, s = gpu_quantize(L, dev_bf16(w))
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    qn, sn = q.cpu().numpy(), untile_scales(s.cpu().numpy(), *scales.shape)
    bad = np.nonzero((qn != codes).any(axis=1) | (sn != scales).any(axis=1))[0]
    assert bad.size == 0, f"rows differing from the oracle: {bad[:10]}"
    # padding of the tiled array (rows up to a multiple of 16, blocks up to a
    # multiple of 16) is left as the binding allocated it: zero
    assert np.array_equal(s.cpu().numpy(), tile_scales(scales))


def test_quantize_ragged_row_counts(L):
    """Row counts around the launch's rows per workgroup, K = 2,560."""
    for r in (1, 3, 4, 5, 15, 16, 17, 63, 64, 65, 1000):
        w = synth.normal_bf16(40 + r, r, 2560, 0.02)
        q, s = gpu_quantize(L, dev_bf16(w))
        codes, scales = oracle.oracle_quantize_mxfp4(w)
        assert np.array_equal(q.cpu().numpy(), codes), r
        assert np.array_equal(s.cpu().numpy(), tile_scales(scales)), r


def test_quantize_full_head_every_row(L):
    """The full 248,320-row head on the GPU, every row against the oracle."""
    codes, scales = oracle_full_head()
    q, s = gpu_quantize(L, device_weights(2))
    qn, sn = q.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(untile_scales(sn, *scales.shape), scales)
    assert np.array_equal(qn, codes)


def test_quantize_rejects_and_writes_nothing(L):
    w = dev_bf16(synth.normal_bf16(3, 10, 48, 0.02))          # K = 48 is not a multiple of 32
    q = torch.full((10, 24), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((1, 1, 16, 16), 3, dtype=torch.uint8, device="cuda")
    code = L.lib().lmhead_quantize_mxfp4(w.data_ptr(), 10, 48, q.data_ptr(), s.data_ptr(), None)
    assert code == L.LMH_EINVAL
    torch.cuda.synchronize()
    assert bool((q == 7).all()) and bool((s == 3).all())
    with pytest.raises(ValueError):
        L.lmhead_quantize_mxfp4(w)


@pytest.mark.parametrize("r,k", [(1, 32), (5, 96), (16, 512), (17, 544), (1000, 2560), (4099, 8192)])
def test_tile_scales_matches_layout(L, r, k):
    """lmhead_mxfp4_tile_scales puts every row-major scale at its place in
    the tiled layout and leaves the padding alone."""
    rng = np.random.default_rng(r * 7 + k)
    sc = rng.integers(0, 256, size=(r, k // 32)).astype(np.uint8)
    out = torch.full(L.mxfp4_scale_shape(r, k), 0xEE, dtype=torch.uint8, device="cuda")
    L.lmhead_mxfp4_tile_scales(dev_u8(sc), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), tile_scales(sc, fill=0xEE))


def test_tile_scales_of_oracle_quantization_drive_the_argmax(L):
    """Scales written row-major (as the oracle writes them), tiled on the
    GPU, give the same argmax as the quantizer's own tiled scales."""
    w = synth.normal_bf16(61, 3001, 2560, 0.02)
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    s_dev = L.lmhead_mxfp4_tile_scales(dev_u8(scales))
    q_dev, s_q = gpu_quantize(L, dev_bf16(w))
    assert torch.equal(s_dev, s_q)
    h = dev_bf16(synth.hidden(62, 0, 5, 2560))
    a = L.draft_project_argmax_mxfp4(h, dev_u8(codes), s_dev)
    b = L.draft_project_argmax_mxfp4(h, q_dev, s_q)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# --------------------------------------------------------------------------
# projection + argmax over the dequantized head
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,trimmed,m,n", [
    (2, False, 1, 16), (3, True, 3, 16), (4, True, 1, 16), (4, True, 4, 16), (5, True, 24, 16), (5, False, 24, 16),
])
def test_mxfp4_argmax_configs(L, cfg, trimmed, m, n):
    inp = config_inputs(cfg)
    codes, scales = oracle_full_head()
    d2t = None
    if trimmed:
        ids = inp["ids"]
        codes, scales = codes[ids], scales[ids]
        d2t = ids.astype(np.int32)
    hs = draws(inp["config"], m, n)
    run_and_check(L, hs, codes, scales, d2t, f"mxfp4 config {cfg} M={m} {'list' if trimmed else 'full'}")


def test_mxfp4_argmax_on_gpu_quantized_head(L):
    """The chain a caller runs: lmhead_trim, then the GPU quantizer, then the
    projection; its codes are checked against the oracle's first."""
    inp = config_inputs(4)
    w_dev = L.lmhead_trim(device_weights(4), dev_i32(inp["ids"]))
    q_dev, s_dev = gpu_quantize(L, w_dev)
    del w_dev
    codes, scales = oracle_full_head()
    codes, scales = codes[inp["ids"]], scales[inp["ids"]]
    assert np.array_equal(q_dev.cpu().numpy(), codes)
    assert np.array_equal(s_dev.cpu().numpy(), tile_scales(scales))
    hs = draws(inp["config"], 4, 2)
    run_and_check(L, hs, codes, scales, inp["ids"].astype(np.int32), "mxfp4 gpu-quantized list M=4",
                  q_dev, s_dev)


EDGE = [(1, 512, 1), (2, 512, 3), (3, 1024, 17), (4, 1536, 1000), (1, 2560, 5), (5, 512, 700),
        (8, 2560, 33), (17, 512, 999), (24, 2560, 1000), (32, 8192, 40), (29, 2560, 600),
        (1, 8192, 2047), (4, 8192, 64), (16, 4096, 4099)]


@pytest.mark.parametrize("m,k,r", EDGE, ids=[f"M{m}-K{k}-R{r}" for m, k, r in EDGE])
def test_mxfp4_edges(L, m, k, r):
    w = synth.normal_bf16(17000 + r, r, k, 0.02)
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    hs = [synth.hidden(18000 + k, d, m, k) for d in range(2)]
    d2t = (np.arange(r, dtype=np.int32)[::-1] * 7 + 11).copy()
    run_and_check(L, hs, codes, scales, None, f"mxfp4 edge M={m} K={k} R={r}")
    run_and_check(L, hs[:1], codes, scales, d2t, f"mxfp4 edge d2t M={m} K={k} R={r}")


def test_mxfp4_wide_block_scales(L):
    """Blocks whose scales span 2^-100 .. 2^100 (every dequantized value
    still a normal bf16 number), with the hidden rows scaled the other way
    block by block, so that every product and logit stays moderate."""
    rng = np.random.default_rng(77)
    r, k, m = 3000, 2560, 4
    exps = rng.integers(-100, 101, size=k // 32)                  # one exponent per block column
    colscale = np.repeat(2.0 ** exps, 32)
    w = synth.bf16_from_f32((rng.standard_normal((r, k)) * 0.02 * colscale).astype(np.float32))
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    assert scales.min() < 40 and scales.max() > 215
    hs = []
    for d in range(2):
        hv = oracle.bf16_bits_to_f64(synth.hidden(78, d, m, k)) / colscale   # exact: powers of two
        hs.append(synth.bf16_from_f32(hv.astype(np.float32)))
    run_and_check(L, hs, codes, scales, None, "mxfp4 wide scales")


def test_mxfp4_tiny_block_scales(L):
    """Blocks at the bottom of the range: scale exponents down to the clamp
    at -127, where dequantized values fall below bf16's smallest normal
    number (2^-126); hidden rows scaled up block by block keep the products
    and logits moderate."""
    rng = np.random.default_rng(79)
    r, k, m = 2000, 1024, 3
    exps = rng.integers(-129, -110, size=k // 32)
    colscale = np.repeat(2.0 ** exps, 32)
    w = synth.bf16_from_f32((rng.standard_normal((r, k)) * colscale).astype(np.float32))
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    assert scales.min() == 0 and scales.max() < 20
    hs = []
    for d in range(2):
        hv = oracle.bf16_bits_to_f64(synth.hidden(80, d, m, k)) / colscale * 2.0 ** -6
        hs.append(synth.bf16_from_f32(hv.astype(np.float32)))
    run_and_check(L, hs, codes, scales, None, "mxfp4 tiny scales")


@pytest.mark.parametrize("m", [1, 3, 6, 24])
def test_mxfp4_exact_ties_first_row(L, m):
    """E2M1 values with a block maximum of 4 or 6 (scale 1) and integer
    hidden rows make every logit exact in fp32: equal maxima must resolve to
    the smallest row, across workgroups."""
    rng = np.random.default_rng(131 + m)
    r, k = 150_000, 512
    wi = rng.choice(np.array([-3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3]), size=(r, k))
    wi[:, ::32] = 4.0                          # every block's maximum: scale exponent 0
    hi = rng.integers(-1, 2, size=(m, k)).astype(np.float64)
    hi[:, ::32] = 0
    for j in range(m):
        for rr in (140_001 - j, 7 + j, 77_777):
            wi[rr] = np.where(np.arange(k) % 32 == 0, 4.0, 6.0 * np.sign(hi[j]))
    w = synth.bf16_from_f32(wi.astype(np.float32))
    h = synth.bf16_from_f32(hi.astype(np.float32))
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    assert np.all(scales == 127)
    res = oracle.oracle_project_argmax_mxfp4(h, codes, scales)
    q_dev, s_dev = dev_u8(codes), dev_u8(tile_scales(scales))
    for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
        i, lg = L.draft_project_argmax_mxfp4(dev_bf16(h), q_dev, s_dev, None, p)
        assert np.array_equal(i.cpu().numpy(), res.id), (p, i.cpu().numpy(), res.id)
        assert np.array_equal(lg.cpu().numpy().astype(np.float64), res.logit)


def test_mxfp4_repeat_bit_identical_and_rejects(L):
    w = synth.normal_bf16(155, 5000, 2560, 0.02)
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    q_dev, s_dev = dev_u8(codes), dev_u8(tile_scales(scales))
    h = dev_bf16(synth.hidden(156, 0, 6, 2560))
    ws = L.new_workspace()
    a = L.draft_project_argmax_mxfp4(h, q_dev, s_dev, workspace=ws)
    ws.fill_(0xAB)
    b = L.draft_project_argmax_mxfp4(h, q_dev, s_dev, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    oid = torch.full((6,), 77, dtype=torch.int32, device="cuda")
    olg = torch.full((6,), 5.0, device="cuda")
    lib = L.lib()
    bad = [
        dict(k=2048 + 32), dict(m=0), dict(m=33), dict(r=0), dict(path=L.LMH_PATH_VALU),
        dict(sp=s_dev.data_ptr() + 2), dict(qp=q_dev.data_ptr() + 8), dict(wsb=16), dict(qp=None),
    ]
    for cs in bad:
        code = lib.draft_project_argmax_mxfp4(
            h.data_ptr(), cs.get("m", 6), cs.get("k", 2560), cs.get("qp", q_dev.data_ptr()),
            cs.get("sp", s_dev.data_ptr()), cs.get("r", 5000), None, oid.data_ptr(), olg.data_ptr(),
            ws.data_ptr(), cs.get("wsb", ws.numel()), cs.get("path", 0), None)
        assert code in (L.LMH_EINVAL, L.LMH_EWORKSPACE), cs
    torch.cuda.synchronize()
    assert bool((oid == 77).all()) and bool((olg == 5.0).all())


def test_mxfp4_bench_helper_matches_call(L):
    w = synth.normal_bf16(255, 20000, 2560, 0.02)
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    heads = [(dev_u8(codes), dev_u8(tile_scales(scales))) for _ in range(2)]
    h = dev_bf16(synth.hidden(256, 0, 4, 2560))
    ws = L.new_workspace()
    oid = torch.empty(4, dtype=torch.int32, device="cuda")
    olg = torch.empty(4, device="cuda")
    ms = L.lmhead_bench_time_argmax_mxfp4(h, heads, None, L.LMH_PATH_AUTO, 5, oid, olg, ws)
    assert ms > 0
    i, lg = L.draft_project_argmax_mxfp4(h, heads[0][0], heads[0][1])
    assert torch.equal(oid, i) and torch.equal(olg, lg)
    res = oracle.oracle_project_argmax_mxfp4(synth.hidden(256, 0, 4, 2560), codes, scales, keep_logits=True)
    check_mxfp4(synth.hidden(256, 0, 4, 2560), codes, scales, None, i.cpu().numpy(), lg.cpu().numpy(), res)


# --------------------------------------------------------------------------
# top k over the MXFP4 head
# --------------------------------------------------------------------------

def run_topk_mx(L, h, codes, scales, d2t_np, topk, tag):
    from parity import check_topk_mxfp4
    res = oracle.oracle_project_topk_mxfp4(h, codes, scales, d2t_np, topk)
    q_dev, s_dev = dev_u8(codes), dev_u8(tile_scales(scales))
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
        i, lg = L.draft_project_topk_mxfp4(dev_bf16(h), q_dev, s_dev, d2t_dev, topk, path=p)
        st = check_topk_mxfp4(h, codes, scales, d2t_np, i.cpu().numpy(), lg.cpu().numpy(), res)
        log(f"[{tag}] path={p} k={topk} positions={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e} "
            f"err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


@pytest.mark.parametrize("cfg,trimmed,m,topk", [
    (2, False, 1, 8), (2, False, 4, 16), (5, False, 24, 4), (3, True, 3, 16), (4, True, 1, 1), (5, True, 24, 8),
])
def test_mxfp4_topk_configs(L, cfg, trimmed, m, topk):
    """Candidates from the 4-bit head: the full head and the lists."""
    inp = config_inputs(cfg)
    codes, scales = oracle_full_head()
    d2t = None
    if trimmed:
        ids = inp["ids"]
        codes, scales = codes[ids], scales[ids]
        d2t = ids.astype(np.int32)
    h = draws(inp["config"], m, 1)[0]
    run_topk_mx(L, h, codes, scales, d2t, topk, f"mxfp4 top-k config {cfg} M={m}")


TOPK_EDGE = [(1, 512, 1, 16), (3, 512, 5, 4), (2, 1024, 17, 16), (17, 1024, 1000, 16), (32, 8192, 40, 8),
             (24, 2560, 3001, 2), (5, 1536, 4099, 3)]


@pytest.mark.parametrize("m,k,r,topk", TOPK_EDGE, ids=[f"M{m}-K{k}-R{r}-k{t}" for m, k, r, t in TOPK_EDGE])
def test_mxfp4_topk_edges(L, m, k, r, topk):
    w = synth.normal_bf16(27000 + r, r, k, 0.02)
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    h = synth.hidden(28000 + k, 0, m, k)
    d2t = (np.arange(r, dtype=np.int32)[::-1] * 5 + 7).copy()
    run_topk_mx(L, h, codes, scales, None, topk, f"mxfp4 top-k edge M={m} K={k} R={r}")
    run_topk_mx(L, h, codes, scales, d2t, topk, f"mxfp4 top-k edge d2t M={m} K={k} R={r}")


def test_mxfp4_topk1_matches_argmax_and_ties(L):
    """k = 1 gives the argmax call's id and logit bits (same kernel); planted
    exact ties (E2M1 values, scale 1, integer hidden rows) come out smaller
    row first, every position equal to the oracle's."""
    w = synth.normal_bf16(301, 20000, 2560, 0.02)
    codes, scales = oracle.oracle_quantize_mxfp4(w)
    q_dev, s_dev = dev_u8(codes), dev_u8(tile_scales(scales))
    for m in (1, 4, 24):
        h = dev_bf16(synth.hidden(302, m, m, 2560))
        a = L.draft_project_argmax_mxfp4(h, q_dev, s_dev)
        t = L.draft_project_topk_mxfp4(h, q_dev, s_dev, None, 1)
        assert torch.equal(t[0][:, 0], a[0]) and torch.equal(t[1][:, 0], a[1]), m
    rng = np.random.default_rng(303)
    r, k, m = 40_000, 512, 3
    wi = rng.choice(np.array([-2, -1, 0, 1, 2], dtype=np.float64), size=(r, k))
    wi[:, ::32] = 4.0
    hi = rng.integers(-1, 2, size=(m, k)).astype(np.float64)
    hi[:, ::32] = 0
    for j in range(m):
        for rr in (39_001, 5 + j, 20_000, 12_345):
            wi[rr] = np.where(np.arange(k) % 32 == 0, 4.0, 2.0 * np.sign(hi[j]))
    wb, hb = synth.bf16_from_f32(wi.astype(np.float32)), synth.bf16_from_f32(hi.astype(np.float32))
    codes, scales = oracle.oracle_quantize_mxfp4(wb)
    res = oracle.oracle_project_topk_mxfp4(hb, codes, scales, None, 6)
    i, lg = L.draft_project_topk_mxfp4(dev_bf16(hb), dev_u8(codes), dev_u8(tile_scales(scales)), None, 6)
    assert np.array_equal(i.cpu().numpy(), res.id)
    assert np.array_equal(lg.cpu().numpy().astype(np.float64), res.logit)


def test_mxfp4_topk_rejects(L):
    """No VALU path, topk outside 1-16 rejected; a rejected call writes
    nothing."""
    w = synth.normal_bf16(311, 100, 512, 0.02)
    q, s = gpu_quantize(L, dev_bf16(w))
    h = dev_bf16(synth.hidden(312, 0, 2, 512))
    with pytest.raises(L.LmheadError):
        L.draft_project_topk_mxfp4(h, q, s, None, 4, path=L.LMH_PATH_VALU)
    oid = torch.full((2, 16), 7, dtype=torch.int32, device="cuda")
    olg = torch.full((2, 16), 5.0, device="cuda")
    ws = torch.empty(L.draft_project_topk_workspace_bytes(2, 16), dtype=torch.uint8, device="cuda")
    for topk in (0, 17):
        code = L.lib().draft_project_topk_mxfp4(h.data_ptr(), 2, 512, q.data_ptr(), s.data_ptr(), 100, None, topk,
                                                oid.data_ptr(), olg.data_ptr(), ws.data_ptr(), ws.numel(), 0, None)
        assert code == L.LMH_EINVAL
    torch.cuda.synchronize()
    assert bool((oid == 7).all()) and bool((olg == 5.0).all())
