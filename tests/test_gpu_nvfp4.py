"""NVFP4 head (E2M1 in blocks of 16, one E4M3 scale per block, one fp32 scale
per head) through the C ABI, against the fp64 oracle: the load-time
quantizer bit for bit (codes, block scales and the head's scale), and the
argmax and top k over the dequantized head on the matrix-core kernel (the
only one that takes this format).

The oracle quantizes every head itself and its codes are what the
projection tests upload, so no expected value and no projection input
comes from the GPU.  A shortlisted head is quantized as a head of its own
(its tensor scale comes from its own rows), as a trimmed head is
requantized on the pages.  Rows are quantized in threads once the tensor
scale is known.

The library keeps the block scales in a tiled layout (16-row tiles, groups
of 32 blocks, 512 bytes per tile and group); tile_scales / untile_scales
below rearrange the oracle's row-major scales to and from it, following the
layout the header documents.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import oracle.nvfp4_head as nv
import synth
from devcopy import dev_f32, dev_u8
from parity import ParityStats, check_nvfp4, check_topk_nvfp4
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
    """Row-major block scales [R, B] -> the tiled layout [ceil(R/16),
    ceil(B/32), 16, 32]: element [t, q, i, j] is the scale of row 16 t + i,
    block 32 q + j (padding = fill)."""
    r, nblk = sc.shape
    t, ng = (r + 15) // 16, (nblk + 31) // 32
    pad = np.full((t * 16, ng * 32), fill, dtype=np.uint8)
    pad[:r, :nblk] = sc
    return np.ascontiguousarray(pad.reshape(t, 16, ng, 32).transpose(0, 2, 1, 3))


def untile_scales(tiled, r, nblk):
    t, ng = tiled.shape[:2]
    return np.ascontiguousarray(tiled.transpose(0, 2, 1, 3).reshape(t * 16, ng * 32)[:r, :nblk])


def oracle_quantize_head(w_bits, block=2048):
    """oracle_quantize_nvfp4, with the rows quantized in threads once the
    head's scale is known (rows are independent given it)."""
    g = nv.tensor_scale(nv.head_amax(w_bits))
    n = w_bits.shape[0]
    if n <= block:
        c, s = nv.oracle_quantize_nvfp4_rows(w_bits, g)
        return c, s, g
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(lambda r0: nv.oracle_quantize_nvfp4_rows(w_bits[r0:r0 + block], g), range(0, n, block)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), g


_heads = {}


def oracle_head(cfg, trimmed):
    """(codes, scales, g) of the full head, or of config cfg's list as a head
    of its own; cached per session."""
    key = (cfg if trimmed else 2, trimmed)
    if key not in _heads:
        w = config_inputs(2)["W"]
        if trimmed:
            w = w[config_inputs(cfg)["ids"]]
        log(f"[oracle] quantizing a {w.shape[0]}-row head to NVFP4")
        _heads[key] = oracle_quantize_head(w)
    return _heads[key]


def gpu_quantize(L, w_dev):
    q, s, g = L.lmhead_quantize_nvfp4(w_dev)
    torch.cuda.synchronize()
    return q, s, g


def run_and_check(L, hs, codes, scales, g, d2t_np, tag, dev=None):
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax_nvfp4(stack, codes, scales, g, d2t_np, keep_logits=True)
    if dev is None:
        dev = (dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g]))
    q_dev, s_dev, g_dev = dev
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
        ids, lgs = [], []
        for h in hs:
            i, l = L.draft_project_argmax_nvfp4(dev_bf16(h), q_dev, s_dev, g_dev, d2t_dev, p)
            ids.append(i.cpu().numpy())
            lgs.append(l.cpu().numpy())
        st = ParityStats()
        st.add(check_nvfp4(stack, codes, scales, g, d2t_np, np.concatenate(ids), np.concatenate(lgs), res))
        log(f"[{tag}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} "
            f"max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


# --------------------------------------------------------------------------
# quantizer, bit for bit
# --------------------------------------------------------------------------

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
# every E4M3 midpoint between neighbouring positive values, subnormal and normal
E4M3_POS = np.array([nv.e4m3_decode(np.array([c], np.uint8))[0] for c in range(0x7F)])
E4M3_MIDS = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2


def _special_head(rng, k):
    """Rows that exercise the two-level conversion.  Row 0 holds 2,688 so
    the head's scale is 1; then: block maxima at 6 x every E4M3 midpoint
    (block-scale ties, subnormal and normal) and just below 6 x 448; blocks
    holding every E2M1 midpoint under block scale 1 (element ties to even);
    blocks of maximum 6.375, whose scale ties down to 1 so their largest
    elements saturate at 6; blocks whose scale rounds to 0 (every element a
    signed zero); zeros and signed zeros; a lone nonzero; ordinary rows."""
    rows = []
    first = np.zeros(k)
    first[0] = 2688.0
    rows.append(first)
    mids6 = np.resize(6 * E4M3_MIDS, max(k // 16, 1))
    row = np.zeros(k)
    row[::16] = mids6[:len(row[::16])]
    row[1::16] = -0.5 * mids6[:len(row[1::16])]
    rows.append(row)
    top = np.zeros(k)
    top[::16] = 6 * np.resize([447.0, 440.0, 432.0, 416.0], len(top[::16]))
    top[3::16] = -0.4 * top[::16]
    rows.append(top)
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    base = np.concatenate([[6.0], mids, E2M1[1:], [-6.0]])          # block maximum 6: scale 1
    rows.append(np.resize(np.concatenate([base, -base]), k))
    sat = np.resize([6.375, 6.25, -6.125, 6.0, 5.9, 0.1, -2.9, 4.9], k)   # scale 1.0625 ties to 1.0
    rows.append(sat)
    tiny = np.resize([6 * 2.0 ** -11, -6 * 2.0 ** -12, 2.0 ** -12, 0.0], k)   # scale code 0: signed zeros
    rows.append(tiny)
    rows.append(np.zeros(k))
    rows.append(-np.zeros(k))
    one = np.zeros(k)
    one[k // 2 + 3] = -3.5
    rows.append(one)
    for sd in (1.0, 0.02, 300.0):
        rows.append(rng.standard_normal(k) * sd)
    heavy = rng.standard_normal(k) * 0.02
    heavy[::37] *= 50
    rows.append(heavy)
    return synth.bf16_from_f32(np.array(rows, dtype=np.float32))


def _assert_quantized_equal(q, s, g, codes, scales, gw):
    qn, sn = q.cpu().numpy(), untile_scales(s.cpu().numpy(), *scales.shape)
    assert np.float32(g.cpu().numpy()[0]) == np.float32(gw), (float(g.cpu().numpy()[0]), float(gw))
    bad = np.nonzero((qn != codes).any(axis=1) | (sn != scales).any(axis=1))[0]
    assert bad.size == 0, f"rows differing from the oracle: {bad[:10]}"


@pytest.mark.parametrize("k", [16, 32, 48, 512, 2560, 8192])
def test_quantize_bit_exact(L, k):
    rng = np.random.default_rng(2900 + k)
    w = _special_head(rng, k)
    q, s, g = gpu_quantize(L, dev_bf16(w))
    codes, scales, gw = nv.oracle_quantize_nvfp4(w)
    assert gw == np.float32(1.0)
    _assert_quantized_equal(q, s, g, codes, scales, gw)
    # padding of the tiled array is left as the binding allocated it: zero
    assert np.array_equal(s.cpu().numpy(), tile_scales(scales))


@pytest.mark.parametrize("scale", [1.0, 3.0e-5, 2.0 ** -40, 700.0])
def test_quantize_tensor_scale(L, scale):
    """Heads whose largest magnitude is far from 2,688: the head's scale is
    the correctly rounded fp32 quotient, every block scale relative to it."""
    w = synth.bf16_from_f32((np.random.default_rng(7).standard_normal((300, 512)) * scale).astype(np.float32))
    q, s, g = gpu_quantize(L, dev_bf16(w))
    codes, scales, gw = nv.oracle_quantize_nvfp4(w)
    _assert_quantized_equal(q, s, g, codes, scales, gw)


def test_quantize_ragged_row_counts(L):
    for r in (1, 3, 4, 5, 15, 16, 17, 63, 64, 65, 1000):
        w = synth.normal_bf16(60 + r, r, 2560, 0.02)
        q, s, g = gpu_quantize(L, dev_bf16(w))
        codes, scales, gw = nv.oracle_quantize_nvfp4(w)
        assert np.array_equal(q.cpu().numpy(), codes), r
        assert np.array_equal(s.cpu().numpy(), tile_scales(scales)), r
        assert np.float32(g.cpu().numpy()[0]) == gw, r


def test_quantize_full_head_every_row(L):
    """The full 248,320-row head on the GPU, every row against the oracle."""
    codes, scales, gw = oracle_head(2, False)
    q, s, g = gpu_quantize(L, device_weights(2))
    _assert_quantized_equal(q, s, g, codes, scales, gw)


def test_quantize_rejects_and_writes_nothing(L):
    w = dev_bf16(synth.normal_bf16(3, 10, 40, 0.02))          # K = 40 is not a multiple of 16
    q = torch.full((10, 20), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((1, 1, 16, 32), 3, dtype=torch.uint8, device="cuda")
    g = torch.full((1,), 5.0, device="cuda")
    lib = L.lib()
    assert lib.lmhead_quantize_nvfp4(w.data_ptr(), 10, 40, q.data_ptr(), s.data_ptr(), g.data_ptr(), None) == 1
    assert lib.lmhead_quantize_nvfp4(w.data_ptr(), 10, 32, q.data_ptr(), s.data_ptr(), None, None) == 1
    assert lib.lmhead_quantize_nvfp4(w.data_ptr(), 10, 32, q.data_ptr(), s.data_ptr(), g.data_ptr() + 2, None) == 1
    torch.cuda.synchronize()
    assert bool((q == 7).all()) and bool((s == 3).all()) and bool((g == 5.0).all())
    with pytest.raises(ValueError):
        L.lmhead_quantize_nvfp4(w)


@pytest.mark.parametrize("r,k", [(1, 16), (5, 48), (16, 512), (17, 528), (1000, 2560), (4099, 8192)])
def test_tile_scales_matches_layout(L, r, k):
    """lmhead_nvfp4_tile_scales puts every row-major scale at its place in
    the tiled layout and leaves the padding alone."""
    rng = np.random.default_rng(r * 11 + k)
    sc = rng.integers(0, 256, size=(r, k // 16)).astype(np.uint8)
    out = torch.full(L.nvfp4_scale_shape(r, k), 0xEE, dtype=torch.uint8, device="cuda")
    L.lmhead_nvfp4_tile_scales(dev_u8(sc), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), tile_scales(sc, fill=0xEE))
    assert L.lmhead_nvfp4_scale_bytes(r, k) == out.numel()


# --------------------------------------------------------------------------
# projection + argmax over the dequantized head
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,trimmed,m", [
    (2, False, 1), (3, True, 3), (4, True, 1), (4, True, 4), (5, True, 24), (5, False, 24),
])
def test_nvfp4_argmax_configs(L, cfg, trimmed, m):
    inp = config_inputs(cfg)
    codes, scales, g = oracle_head(cfg, trimmed)
    d2t = inp["ids"].astype(np.int32) if trimmed else None
    hs = draws(inp["config"], m, 16)
    run_and_check(L, hs, codes, scales, g, d2t, f"nvfp4 config {cfg} M={m} {'list' if trimmed else 'full'}")


def test_nvfp4_argmax_on_gpu_quantized_list(L):
    """The chain a caller runs: lmhead_trim, the GPU quantizer over the
    trimmed head, then the projection; its codes, block scales and head
    scale are checked against the oracle's first."""
    inp = config_inputs(3)
    w_dev = L.lmhead_trim(device_weights(3), dev_i32(inp["ids"]))
    q_dev, s_dev, g_dev = gpu_quantize(L, w_dev)
    del w_dev
    codes, scales, g = oracle_head(3, True)
    _assert_quantized_equal(q_dev, s_dev, g_dev, codes, scales, g)
    hs = draws(inp["config"], 3, 4)
    run_and_check(L, hs, codes, scales, g, inp["ids"].astype(np.int32), "nvfp4 gpu-quantized 16k M=3",
                  (q_dev, s_dev, g_dev))


EDGE = [(1, 512, 1), (2, 512, 3), (3, 1024, 17), (4, 1536, 1000), (1, 2560, 5), (5, 512, 700),
        (8, 2560, 33), (17, 512, 999), (24, 2560, 1000), (32, 8192, 40), (29, 2560, 600),
        (1, 8192, 2047), (4, 8192, 64), (16, 4096, 4099)]


@pytest.mark.parametrize("m,k,r", EDGE, ids=[f"M{m}-K{k}-R{r}" for m, k, r in EDGE])
def test_nvfp4_edges(L, m, k, r):
    w = synth.normal_bf16(37000 + r, r, k, 0.02)
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    hs = [synth.hidden(38000 + k, d, m, k) for d in range(2)]
    d2t = (np.arange(r, dtype=np.int32)[::-1] * 7 + 11).copy()
    run_and_check(L, hs, codes, scales, g, None, f"nvfp4 edge M={m} K={k} R={r}")
    run_and_check(L, hs[:1], codes, scales, g, d2t, f"nvfp4 edge d2t M={m} K={k} R={r}")


def test_nvfp4_wide_block_scales(L):
    """Block scales across the whole E4M3 range, subnormal ones included
    (blocks from 448 down to 2^-9 times the largest), with the hidden rows
    scaled the other way block by block so every product and logit stays
    moderate: the decoded block scale must reach the conversion exactly."""
    rng = np.random.default_rng(97)
    r, k, m = 3000, 2560, 4
    exps = rng.integers(-17, 1, size=k // 16)                      # one exponent per block column
    colscale = np.repeat(2.0 ** exps, 16)
    w = synth.bf16_from_f32((rng.standard_normal((r, k)) * 0.02 * colscale).astype(np.float32))
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    assert scales.min() < 0x08 and scales.max() >= 0x70             # subnormal and large block scales
    hs = []
    for d in range(2):
        hv = oracle.bf16_bits_to_f64(synth.hidden(98, d, m, k)) / colscale * 2.0 ** -8
        hs.append(synth.bf16_from_f32(hv.astype(np.float32)))
    run_and_check(L, hs, codes, scales, g, None, "nvfp4 wide block scales")


@pytest.mark.parametrize("k", [512, 2560])
def test_nvfp4_hidden_rows_across_the_bf16_range(L, k):
    """The kernel takes NVFP4 products against hidden rows in f16, each row
    scaled by a power of two that moves its largest magnitude to [2^15,
    2^16) and taken off again from the row's sums.  So a hidden row times
    2^j must give the same ids and exactly 2^j times the logits, for rows
    far above and below 1 (bf16's range, not f16's).  A row with values
    more than 2^29 below its largest (which the f16 copy may round or
    flush) and an all-zero row meet the parity rule with that slack."""
    from parity import f16_hidden_slack
    w = synth.normal_bf16(41000 + k, 3001, k, 0.02)
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    dev = (dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g]))
    base = oracle.bf16_bits_to_f64(synth.hidden(42000 + k, 0, 4, k))
    ids0, lg0 = (x.cpu().numpy() for x in L.draft_project_argmax_nvfp4(dev_bf16(synth.bf16_from_f32(
        base.astype(np.float32))), *dev, None, L.LMH_PATH_MFMA))
    for j in (-100, -40, -7, 9, 40, 100):
        hj = base * 2.0 ** j
        bits = synth.bf16_from_f32(hj.astype(np.float32))
        assert np.array_equal(oracle.bf16_bits_to_f64(bits), hj)        # the scaling is exact in bf16
        for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
            i, lg = (x.cpu().numpy() for x in L.draft_project_argmax_nvfp4(dev_bf16(bits), *dev, None, p))
            assert np.array_equal(i, ids0), (j, p)
            assert np.array_equal(lg, np.ldexp(lg0, j).astype(np.float32)), (j, p)
    # a row spanning more than 2^29, and a zero row
    wide = base.copy()
    wide[0, ::7] *= 2.0 ** -40
    wide[1, 5::11] *= 2.0 ** -33
    wide[2] = 0.0
    bits = synth.bf16_from_f32(wide.astype(np.float32))
    assert np.all(f16_hidden_slack(oracle.bf16_bits_to_f64(bits))[:2].sum(axis=1) > 0)
    run_and_check(L, [bits], codes, scales, g, None, f"nvfp4 hidden beyond f16 K={k}", dev)
    res = oracle.oracle_project_argmax_nvfp4(bits, codes, scales, g)
    i, lg = (x.cpu().numpy() for x in L.draft_project_argmax_nvfp4(dev_bf16(bits), *dev, None, L.LMH_PATH_MFMA))
    assert i[2] == 0 and lg[2] == 0.0 and res.id[2] == 0


def _tie_head(rng, r, k, m, vals, planted, big):
    """E2M1 values with every block's maximum 6 (block scale 1), a row
    holding 2,688 in a column every hidden row zeroes (head scale 1, logit
    0), integer hidden rows zero on every block's first column: every logit
    exact in fp32.  Rows in `planted` take `big` x sign(h) for hidden row j."""
    wi = rng.choice(vals, size=(r, k))
    wi[:, ::16] = 6.0
    wi[1, :] = 0.0
    wi[1, 0] = 2688.0
    hi = rng.integers(-1, 2, size=(m, k)).astype(np.float64)
    hi[:, ::16] = 0
    for j in range(m):
        for rr in planted(j):
            wi[rr] = np.where(np.arange(k) % 16 == 0, 6.0, big * np.sign(hi[j]))
    return synth.bf16_from_f32(wi.astype(np.float32)), synth.bf16_from_f32(hi.astype(np.float32))


@pytest.mark.parametrize("m", [1, 3, 6, 24])
def test_nvfp4_exact_ties_first_row(L, m):
    """Equal maxima resolve to the smallest row, across workgroups."""
    rng = np.random.default_rng(231 + m)
    w, h = _tie_head(rng, 150_000, 512, m, np.array([-3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3]),
                     lambda j: (140_001 - j, 7 + j, 77_777), 6.0)
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    assert g == np.float32(1.0) and np.all(scales[2:] == 0x38)
    res = oracle.oracle_project_argmax_nvfp4(h, codes, scales, g)
    dev = (dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g]))
    for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
        i, lg = L.draft_project_argmax_nvfp4(dev_bf16(h), *dev, None, p)
        assert np.array_equal(i.cpu().numpy(), res.id), (p, i.cpu().numpy(), res.id)
        assert np.array_equal(lg.cpu().numpy().astype(np.float64), res.logit)


def test_nvfp4_repeat_bit_identical_and_rejects(L):
    w = synth.normal_bf16(255, 5000, 2560, 0.02)
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    q_dev, s_dev, g_dev = dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g])
    h = dev_bf16(synth.hidden(256, 0, 6, 2560))
    ws = L.new_workspace()
    a = L.draft_project_argmax_nvfp4(h, q_dev, s_dev, g_dev, workspace=ws)
    ws.fill_(0xAB)
    b = L.draft_project_argmax_nvfp4(h, q_dev, s_dev, g_dev, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    oid = torch.full((6,), 77, dtype=torch.int32, device="cuda")
    olg = torch.full((6,), 5.0, device="cuda")
    lib = L.lib()
    bad = [
        dict(k=2048 + 32), dict(m=0), dict(m=33), dict(r=0), dict(path=L.LMH_PATH_VALU),
        dict(sp=s_dev.data_ptr() + 2), dict(qp=q_dev.data_ptr() + 8), dict(gp=None), dict(gp=g_dev.data_ptr() + 2),
        dict(wsb=16), dict(qp=None), dict(r=1 << 30),
    ]
    for cs in bad:
        code = lib.draft_project_argmax_nvfp4(
            h.data_ptr(), cs.get("m", 6), cs.get("k", 2560), cs.get("qp", q_dev.data_ptr()),
            cs.get("sp", s_dev.data_ptr()), cs.get("gp", g_dev.data_ptr()), cs.get("r", 5000), None,
            oid.data_ptr(), olg.data_ptr(), ws.data_ptr(), cs.get("wsb", ws.numel()), cs.get("path", 0), None)
        assert code in (L.LMH_EINVAL, L.LMH_EWORKSPACE), cs
    torch.cuda.synchronize()
    assert bool((oid == 77).all()) and bool((olg == 5.0).all())


def test_nvfp4_bench_helper_matches_call(L):
    w = synth.normal_bf16(355, 20000, 2560, 0.02)
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    heads = [(dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g])) for _ in range(2)]
    h_np = synth.hidden(356, 0, 4, 2560)
    h = dev_bf16(h_np)
    ws = L.new_workspace()
    oid = torch.empty(4, dtype=torch.int32, device="cuda")
    olg = torch.empty(4, device="cuda")
    ms = L.lmhead_bench_time_argmax_nvfp4(h, heads, None, L.LMH_PATH_AUTO, 5, oid, olg, ws)
    assert ms > 0
    i, lg = L.draft_project_argmax_nvfp4(h, *heads[0])
    assert torch.equal(oid, i) and torch.equal(olg, lg)
    res = oracle.oracle_project_argmax_nvfp4(h_np, codes, scales, g, keep_logits=True)
    check_nvfp4(h_np, codes, scales, g, None, i.cpu().numpy(), lg.cpu().numpy(), res)


# --------------------------------------------------------------------------
# top k over the NVFP4 head
# --------------------------------------------------------------------------

def run_topk_nv(L, h, codes, scales, g, d2t_np, topk, tag):
    res = oracle.oracle_project_topk_nvfp4(h, codes, scales, g, d2t_np, topk)
    dev = (dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g]))
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
        i, lg = L.draft_project_topk_nvfp4(dev_bf16(h), *dev, d2t_dev, topk, path=p)
        st = check_topk_nvfp4(h, codes, scales, g, d2t_np, i.cpu().numpy(), lg.cpu().numpy(), res)
        log(f"[{tag}] path={p} k={topk} positions={st.rows} near_ties={st.near_ties} exempt={st.exempt} "
            f"max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")
        st.assert_exempt_bound()


@pytest.mark.parametrize("cfg,trimmed,m,topk", [
    (2, False, 1, 8), (2, False, 4, 16), (5, False, 24, 4), (3, True, 3, 16), (4, True, 1, 1), (4, True, 4, 4),
    (5, True, 24, 8),
])
def test_nvfp4_topk_configs(L, cfg, trimmed, m, topk):
    """A drafter's candidates scored through the NVFP4 head: the full head
    and the lists."""
    inp = config_inputs(cfg)
    codes, scales, g = oracle_head(cfg, trimmed)
    d2t = inp["ids"].astype(np.int32) if trimmed else None
    h = draws(inp["config"], m, 1)[0]
    run_topk_nv(L, h, codes, scales, g, d2t, topk, f"nvfp4 top-k config {cfg} M={m}")


TOPK_EDGE = [(1, 512, 1, 16), (3, 512, 5, 4), (2, 1024, 17, 16), (17, 1024, 1000, 16), (32, 8192, 40, 8),
             (24, 2560, 3001, 2), (5, 1536, 4099, 3)]


@pytest.mark.parametrize("m,k,r,topk", TOPK_EDGE, ids=[f"M{m}-K{k}-R{r}-k{t}" for m, k, r, t in TOPK_EDGE])
def test_nvfp4_topk_edges(L, m, k, r, topk):
    w = synth.normal_bf16(47000 + r, r, k, 0.02)
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    h = synth.hidden(48000 + k, 0, m, k)
    d2t = (np.arange(r, dtype=np.int32)[::-1] * 5 + 7).copy()
    run_topk_nv(L, h, codes, scales, g, None, topk, f"nvfp4 top-k edge M={m} K={k} R={r}")
    run_topk_nv(L, h, codes, scales, g, d2t, topk, f"nvfp4 top-k edge d2t M={m} K={k} R={r}")


def test_nvfp4_topk1_matches_argmax_and_ties(L):
    """k = 1 gives the argmax call's id and logit bits (same kernel); planted
    exact ties come out smaller row first, every position equal to the
    oracle's."""
    w = synth.normal_bf16(401, 20000, 2560, 0.02)
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    dev = (dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g]))
    for m in (1, 4, 24):
        h = dev_bf16(synth.hidden(402, m, m, 2560))
        a = L.draft_project_argmax_nvfp4(h, *dev)
        t = L.draft_project_topk_nvfp4(h, *dev, None, 1)
        assert torch.equal(t[0][:, 0], a[0]) and torch.equal(t[1][:, 0], a[1]), m
    rng = np.random.default_rng(403)
    wb, hb = _tie_head(rng, 40_000, 512, 3, np.array([-2, -1, 0, 1, 2], dtype=np.float64),
                       lambda j: (39_001, 5 + j, 20_000, 12_345), 4.0)
    codes, scales, g = nv.oracle_quantize_nvfp4(wb)
    res = oracle.oracle_project_topk_nvfp4(hb, codes, scales, g, None, 6)
    i, lg = L.draft_project_topk_nvfp4(dev_bf16(hb), dev_u8(codes), dev_u8(tile_scales(scales)), dev_f32([g]),
                                       None, 6)
    assert np.array_equal(i.cpu().numpy(), res.id)
    assert np.array_equal(lg.cpu().numpy().astype(np.float64), res.logit)


def test_nvfp4_topk_rejects(L):
    """No VALU path, topk outside 1-16 rejected; a rejected call writes
    nothing."""
    w = synth.normal_bf16(411, 100, 512, 0.02)
    q, s, g = gpu_quantize(L, dev_bf16(w))
    h = dev_bf16(synth.hidden(412, 0, 2, 512))
    with pytest.raises(L.LmheadError):
        L.draft_project_topk_nvfp4(h, q, s, g, None, 4, path=L.LMH_PATH_VALU)
    oid = torch.full((2, 16), 7, dtype=torch.int32, device="cuda")
    olg = torch.full((2, 16), 5.0, device="cuda")
    ws = torch.empty(L.draft_project_topk_workspace_bytes(2, 16), dtype=torch.uint8, device="cuda")
    for topk in (0, 17):
        code = L.lib().draft_project_topk_nvfp4(h.data_ptr(), 2, 512, q.data_ptr(), s.data_ptr(), g.data_ptr(), 100,
                                                None, topk, oid.data_ptr(), olg.data_ptr(), ws.data_ptr(), ws.numel(),
                                                0, None)
        assert code == L.LMH_EINVAL
    torch.cuda.synchronize()
    assert bool((oid == 7).all()) and bool((olg == 5.0).all())
