"""Seeded random shapes through every argmax entry point, against the fp64
oracle: bf16 heads (trimmed or full, with and without d2t), FP8 and MXFP4
heads, and lists read in place, on every kernel that accepts the shape.
The cases are drawn once from a fixed seed, so a failure names a
reproducible (format, M, K, R, path) case; they complement the hand-picked
edge shapes of the other GPU tests with combinations nobody picked.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import ParityStats, check, check_fp8, check_logits, check_mxfp4, check_topk
from test_gpu_parity import dev_bf16, dev_i32, log, paths_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 16, 17, 20, 24, 28, 31, 32]
MAX_ELEMS = 24_000_000          # R x K per case, so the oracle stays quick


def _cases(n=120, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ["bf16", "bf16", "fp8", "mx4", "idx"][i % 5]
        m = int(rng.choice(MS))
        kmax = 1024 if rng.random() < 0.5 else 8192     # half the cases with short rows (many of them)
        if fmt == "mx4":
            k = 512 * int(rng.integers(1, kmax // 512 + 1))
        elif fmt == "fp8":
            k = 16 * int(rng.integers(1, kmax // 16 + 1))
        else:
            k = 8 * int(rng.integers(1, kmax // 8 + 1))
        rmax = max(1, min(70_000, MAX_ELEMS // k))
        # half the cases small (ragged tails, a few tiles), half log-uniform up
        # to the size cap (several rounds of tiles per wave)
        if rng.random() < 0.5 or rmax <= 600:
            r = int(rng.integers(1, min(rmax, 600) + 1))
        else:
            r = int(np.exp(rng.uniform(np.log(600), np.log(rmax))))
        with_d2t = bool(rng.random() < 0.5)
        out.append((i, fmt, m, k, r, with_d2t))
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def _tile_scales(sc):
    r, nblk = sc.shape
    t, nb = (r + 15) // 16, (nblk + 15) // 16
    pad = np.zeros((t * 16, nb * 16), dtype=np.uint8)
    pad[:r, :nblk] = sc
    return np.ascontiguousarray(pad.reshape(t, 16, nb, 16).transpose(0, 2, 1, 3))


def _ids(rng, r, n):
    """r distinct vocabulary ids below n, in random order."""
    return rng.permutation(n)[:r].astype(np.int32)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-M{c[2]}-K{c[3]}-R{c[4]}{'-d2t' if c[5] else ''}"
                                             for c in CASES])
def test_random_shape(L, case):
    i, fmt, m, k, r, with_d2t = case
    log(f"[random {i}] {fmt} M={m} K={k} R={r} d2t={with_d2t}")
    rng = np.random.default_rng(1000 + i)
    hs = [synth.hidden(5000 + i, d, m, k) for d in range(2)]
    stack = np.concatenate(hs)
    st = ParityStats()
    if fmt == "idx":
        n = r + int(rng.integers(0, 3 * r + 1))
        w = synth.normal_bf16(6000 + i, n, k, 0.02)
        ids = _ids(rng, r, n)
        w_dev, ids_dev = dev_bf16(w), dev_i32(ids)
        res = oracle.oracle_project_argmax(stack, w[ids], ids, keep_logits=True)
        for p in paths_for(L, m, k):
            got = [L.draft_project_argmax_indexed(dev_bf16(h), w_dev, ids_dev, p) for h in hs]
            st.add(check(stack, w[ids], ids, np.concatenate([g[0].cpu().numpy() for g in got]),
                         np.concatenate([g[1].cpu().numpy() for g in got]), res))
    else:
        w = synth.normal_bf16(6000 + i, r, k, 0.02)
        d2t = _ids(rng, r, r + int(rng.integers(0, 2 * r + 1))) if with_d2t else None
        d2t_dev = dev_i32(d2t) if d2t is not None else None
        if fmt == "bf16":
            res = oracle.oracle_project_argmax(stack, w, d2t, keep_logits=True)
            w_dev = dev_bf16(w)
            for p in paths_for(L, m, k) + [L.LMH_PATH_AUTO]:
                got = [L.draft_project_argmax_path(dev_bf16(h), w_dev, d2t_dev, p) for h in hs]
                st.add(check(stack, w, d2t, np.concatenate([g[0].cpu().numpy() for g in got]),
                             np.concatenate([g[1].cpu().numpy() for g in got]), res))
        elif fmt == "fp8":
            codes, scale = oracle.oracle_quantize_fp8(w)
            res = oracle.oracle_project_argmax_fp8(stack, codes, scale, d2t, keep_logits=True)
            q_dev = torch.from_numpy(codes).cuda()
            s_dev = torch.from_numpy(scale).cuda()
            paths = [L.LMH_PATH_AUTO, L.LMH_PATH_MFMA] + ([L.LMH_PATH_VALU] if m <= 4 else [])
            for p in paths:
                got = [L.draft_project_argmax_fp8(dev_bf16(h), q_dev, s_dev, d2t_dev, p) for h in hs]
                st.add(check_fp8(stack, codes, scale, d2t, np.concatenate([g[0].cpu().numpy() for g in got]),
                                 np.concatenate([g[1].cpu().numpy() for g in got]), res))
        else:
            codes, scales = oracle.oracle_quantize_mxfp4(w)
            res = oracle.oracle_project_argmax_mxfp4(stack, codes, scales, d2t, keep_logits=True)
            q_dev = torch.from_numpy(codes).cuda()
            s_dev = torch.from_numpy(_tile_scales(scales)).cuda()
            for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
                got = [L.draft_project_argmax_mxfp4(dev_bf16(h), q_dev, s_dev, d2t_dev, p) for h in hs]
                st.add(check_mxfp4(stack, codes, scales, d2t, np.concatenate([g[0].cpu().numpy() for g in got]),
                                   np.concatenate([g[1].cpu().numpy() for g in got]), res))
    log(f"[random {i}] rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e} "
        f"err/bound={st.max_err_over_bound:.3f}")
    st.assert_exempt_bound()


# --------------------------------------------------------------------------
# top-k and logits epilogues
# --------------------------------------------------------------------------

def _epi_cases(n=60, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = "topk" if i % 3 else "logits"
        m = int(rng.choice(MS))
        k = 8 * int(rng.integers(1, (1024 if rng.random() < 0.5 else 8192) // 8 + 1))
        rmax = max(1, min(40_000, 12_000_000 // k))
        r = int(rng.integers(1, min(rmax, 600) + 1)) if rng.random() < 0.5 or rmax <= 600 else \
            int(np.exp(rng.uniform(np.log(600), np.log(rmax))))
        with_d2t = bool(rng.random() < 0.5)
        topk = int(rng.integers(1, 17))
        out.append((i, kind, m, k, r, with_d2t, topk))
    return out


EPI_CASES = _epi_cases()


def _epi_paths(L, m, k):
    """The top-k / logits epilogues: VALU for M <= 4 with M * ceil(K / 512)
    <= 40, matrix cores for any M."""
    valu = m <= 4 and m * ((k // 8 + 63) // 64) <= 40
    return ([L.LMH_PATH_VALU] if valu else []) + [L.LMH_PATH_MFMA, L.LMH_PATH_AUTO]


@pytest.mark.parametrize("case", EPI_CASES,
                         ids=[f"{c[0]}-{c[1]}-M{c[2]}-K{c[3]}-R{c[4]}{'-d2t' if c[5] else ''}"
                              f"{'-k' + str(c[6]) if c[1] == 'topk' else ''}" for c in EPI_CASES])
def test_random_shape_topk_logits(L, case):
    i, kind, m, k, r, with_d2t, topk = case
    log(f"[random epilogue {i}] {kind} M={m} K={k} R={r} d2t={with_d2t} topk={topk}")
    rng = np.random.default_rng(3000 + i)
    w = synth.normal_bf16(7000 + i, r, k, 0.02)
    h = synth.hidden(8000 + i, 0, m, k)
    n = r + int(rng.integers(0, 2 * r + 1))
    d2t = _ids(rng, r, n) if with_d2t else None
    w_dev, h_dev = dev_bf16(w), dev_bf16(h)
    d2t_dev = dev_i32(d2t) if d2t is not None else None
    if kind == "topk":
        res = oracle.oracle_project_topk(h, w, d2t, topk)
        for p in _epi_paths(L, m, k):
            ids, lgs = L.draft_project_topk(h_dev, w_dev, d2t_dev, topk, path=p)
            st = check_topk(h, w, d2t, ids.cpu().numpy(), lgs.cpu().numpy(), res)
    else:
        for p in _epi_paths(L, m, k):
            out = L.draft_project_logits(h_dev, w_dev, d2t_dev, n=n if with_d2t else None, path=p)
            st = check_logits(h, w, d2t, n if with_d2t else None, out.cpu().numpy())
    log(f"[random epilogue {i}] max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")


def _qtopk_cases(n=40, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = "fp8" if i % 2 else "mx4"
        m = int(rng.choice(MS))
        kmax = 1024 if rng.random() < 0.5 else 8192
        k = 512 * int(rng.integers(1, kmax // 512 + 1)) if fmt == "mx4" else 16 * int(rng.integers(1, kmax // 16 + 1))
        rmax = max(1, min(40_000, 12_000_000 // k))
        r = int(rng.integers(1, min(rmax, 600) + 1)) if rng.random() < 0.5 or rmax <= 600 else \
            int(np.exp(rng.uniform(np.log(600), np.log(rmax))))
        out.append((i, fmt, m, k, r, bool(rng.random() < 0.5), int(rng.integers(1, 17))))
    return out


QTOPK_CASES = _qtopk_cases()


@pytest.mark.parametrize("case", QTOPK_CASES,
                         ids=[f"{c[0]}-{c[1]}-M{c[2]}-K{c[3]}-R{c[4]}{'-d2t' if c[5] else ''}-k{c[6]}"
                              for c in QTOPK_CASES])
def test_random_shape_quantized_topk(L, case):
    from parity import check_topk_fp8, check_topk_mxfp4
    i, fmt, m, k, r, with_d2t, topk = case
    log(f"[random quantized top-k {i}] {fmt} M={m} K={k} R={r} d2t={with_d2t} topk={topk}")
    rng = np.random.default_rng(9000 + i)
    w = synth.normal_bf16(9100 + i, r, k, 0.02)
    h = synth.hidden(9200 + i, 0, m, k)
    d2t = _ids(rng, r, r + int(rng.integers(0, 2 * r + 1))) if with_d2t else None
    d2t_dev = dev_i32(d2t) if d2t is not None else None
    if fmt == "fp8":
        codes, scale = oracle.oracle_quantize_fp8(w)
        res = oracle.oracle_project_topk_fp8(h, codes, scale, d2t, topk)
        ids, lgs = L.draft_project_topk_fp8(dev_bf16(h), torch.from_numpy(codes).cuda(),
                                            torch.from_numpy(scale).cuda(), d2t_dev, topk)
        st = check_topk_fp8(h, codes, scale, d2t, ids.cpu().numpy(), lgs.cpu().numpy(), res)
    else:
        codes, scales = oracle.oracle_quantize_mxfp4(w)
        res = oracle.oracle_project_topk_mxfp4(h, codes, scales, d2t, topk)
        ids, lgs = L.draft_project_topk_mxfp4(dev_bf16(h), torch.from_numpy(codes).cuda(),
                                              torch.from_numpy(_tile_scales(scales)).cuda(), d2t_dev, topk)
        st = check_topk_mxfp4(h, codes, scales, d2t, ids.cpu().numpy(), lgs.cpu().numpy(), res)
    log(f"[random quantized top-k {i}] max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")


# --------------------------------------------------------------------------
# NVFP4 heads: argmax and top k over random shapes
# --------------------------------------------------------------------------

def _nv_cases(n=40, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        m = int(rng.choice(MS))
        kmax = 1024 if rng.random() < 0.5 else 8192
        k = 512 * int(rng.integers(1, kmax // 512 + 1))
        rmax = max(1, min(40_000, 12_000_000 // k))
        r = int(rng.integers(1, min(rmax, 600) + 1)) if rng.random() < 0.5 or rmax <= 600 else \
            int(np.exp(rng.uniform(np.log(600), np.log(rmax))))
        topk = int(rng.integers(1, 17)) if i % 2 else 0           # every other case a top-k call
        out.append((i, m, k, r, bool(rng.random() < 0.5), topk))
    return out


NV_CASES = _nv_cases()


def _nv_tile_scales(sc):
    """Row-major E4M3 block scales [R, K / 16] -> the library's tiled layout
    (16-row tiles, groups of 32 blocks, 512 bytes per tile and group)."""
    r, nblk = sc.shape
    t, ng = (r + 15) // 16, (nblk + 31) // 32
    pad = np.zeros((t * 16, ng * 32), dtype=np.uint8)
    pad[:r, :nblk] = sc
    return np.ascontiguousarray(pad.reshape(t, 16, ng, 32).transpose(0, 2, 1, 3))


@pytest.mark.parametrize("case", NV_CASES,
                         ids=[f"{c[0]}-nv4-M{c[1]}-K{c[2]}-R{c[3]}{'-d2t' if c[4] else ''}"
                              f"{'-k' + str(c[5]) if c[5] else ''}" for c in NV_CASES])
def test_random_shape_nvfp4(L, case):
    """NVFP4 heads quantized by the oracle (codes, tiled E4M3 scales, g): the
    argmax on the library's kernel choice and the matrix-core path, or the
    top k, against the oracle over the dequantized head."""
    from parity import check_nvfp4, check_topk_nvfp4
    import oracle.nvfp4_head as nv
    i, m, k, r, with_d2t, topk = case
    log(f"[random nvfp4 {i}] M={m} K={k} R={r} d2t={with_d2t} topk={topk}")
    rng = np.random.default_rng(11000 + i)
    w = synth.normal_bf16(11100 + i, r, k, 0.02)
    hs = [synth.hidden(11200 + i, d, m, k) for d in range(2)]
    stack = np.concatenate(hs)
    d2t = _ids(rng, r, r + int(rng.integers(0, 2 * r + 1))) if with_d2t else None
    d2t_dev = dev_i32(d2t) if d2t is not None else None
    codes, scales, g = nv.oracle_quantize_nvfp4(w)
    q_dev = torch.from_numpy(codes).cuda()
    s_dev = torch.from_numpy(_nv_tile_scales(scales)).cuda()
    g_dev = torch.tensor([float(g)], dtype=torch.float32, device="cuda")
    if topk:
        res = oracle.oracle_project_topk_nvfp4(stack, codes, scales, g, d2t, topk)
        got = [L.draft_project_topk_nvfp4(dev_bf16(h), q_dev, s_dev, g_dev, d2t_dev, topk) for h in hs]
        st = check_topk_nvfp4(stack, codes, scales, g, d2t, np.concatenate([x[0].cpu().numpy() for x in got]),
                              np.concatenate([x[1].cpu().numpy() for x in got]), res)
    else:
        res = oracle.oracle_project_argmax_nvfp4(stack, codes, scales, g, d2t, keep_logits=True)
        st = ParityStats()
        for p in (L.LMH_PATH_AUTO, L.LMH_PATH_MFMA):
            got = [L.draft_project_argmax_nvfp4(dev_bf16(h), q_dev, s_dev, g_dev, d2t_dev, p) for h in hs]
            st.add(check_nvfp4(stack, codes, scales, g, d2t, np.concatenate([x[0].cpu().numpy() for x in got]),
                               np.concatenate([x[1].cpu().numpy() for x in got]), res))
        st.assert_exempt_bound()
    log(f"[random nvfp4 {i}] max_err={st.max_err:.2e} err/bound={st.max_err_over_bound:.3f}")
