"""The single-launch argmax (draft_project_argmax_fused and its path-forcing
form) through the C ABI: workgroups merge their keys into a persistent
state with atomics, in two levels, and the workgroup that takes the last
ticket writes the outputs, so one launch replaces the projection + fold
pair.  It runs the same projection kernels with the same per-row sums, so
its outputs must equal the two-kernel call bit for bit, meet the parity rule
against the fp64 oracle, and leave the whole state at zero after every call:
both kernels, the lists and the full head, grids from one workgroup (fewer
than the 16 merge groups) to the largest, multi-pass M, exact ties planted
in different merge groups, graph replays, and the argument checks."""
import numpy as np
import pytest

import oracle
import synth
from devcopy import dev_bf16, dev_i32
from parity import ParityStats, check
from test_gpu_parity import config_inputs, device_weights, draws, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def nonzero_bytes(state):
    """Bytes of the state (tickets and keys of both levels) that are not zero."""
    return int(torch.count_nonzero(state))


def same(a, b):
    return torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def run(L, hs, w_np, w_dev, d2t_np, paths, tag):
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax(stack, w_np, d2t_np, keep_logits=True)
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    state = L.new_state("cuda")
    for p in paths:
        ids, lgs = [], []
        for h in hs:
            hd = dev_bf16(h)
            a = L.draft_project_argmax_fused_path(hd, w_dev, d2t_dev, p, state)
            b = L.draft_project_argmax_path(hd, w_dev, d2t_dev, p)
            assert same(a, b), tag
            ids.append(a[0].cpu().numpy())
            lgs.append(a[1].cpu().numpy())
        assert nonzero_bytes(state) == 0
        st = ParityStats()
        st.add(check(stack, w_np, d2t_np, np.concatenate(ids), np.concatenate(lgs), res))
        log(f"[fused {tag}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} "
            f"max_err={st.max_err:.2e}")
        st.assert_exempt_bound()


@pytest.mark.parametrize("cfg,m", [(2, 1), (2, 3), (3, 1), (3, 3), (4, 1), (4, 4), (5, 3), (5, 24)])
def test_fused_configs(L, cfg, m):
    inp = config_inputs(cfg)
    c = inp["config"]
    ids = inp["ids"]
    hs = draws(c, m, 8)
    paths = [L.LMH_PATH_VALU, L.LMH_PATH_MFMA] if m <= 4 else [L.LMH_PATH_MFMA]
    if cfg == 2:
        run(L, hs, inp["W"], device_weights(2), None, paths, f"full M={m}")
    else:
        wt = L.lmhead_trim(device_weights(cfg), dev_i32(ids))
        run(L, hs, oracle.oracle_trim(inp["W"], ids), wt, ids, paths, f"config {cfg} M={m}")


def test_fused_full_head_m24(L):
    inp = config_inputs(2)
    hs = [synth.hidden(7024, d, 24, 2560) for d in range(4)]
    run(L, hs, inp["W"], device_weights(2), None, [L.LMH_PATH_MFMA], "full M=24")


def test_auto_entry_matches_the_default_call(L):
    """draft_project_argmax_fused (the library's kernel choice) against
    draft_project_argmax, one state reused over every call."""
    inp = config_inputs(4)
    wt = L.lmhead_trim(device_weights(4), dev_i32(inp["ids"]))
    d2t = dev_i32(inp["ids"])
    state = L.new_state("cuda")
    for m in (1, 2, 3, 4, 5, 8, 16, 24, 32):
        hd = dev_bf16(synth.hidden(7100 + m, 0, m, 2560))
        assert same(L.draft_project_argmax_fused(hd, wt, d2t, state), L.draft_project_argmax(hd, wt, d2t)), m
        assert nonzero_bytes(state) == 0, m


def test_fused_shapes_share_a_state(L):
    """Launches of different grids (heads of 1 to 300,000 rows: from a
    single workgroup, fewer than the merge groups, to the largest grid; M
    from 1 to 32 with K = 8,192, which takes two passes) one after another
    on one state: every call matches the two-kernel call and leaves the
    state at zero."""
    state = L.new_state("cuda")
    for r, k, m, p in [(1, 256, 1, 1), (1, 256, 1, 2), (300_000, 256, 2, 1), (5, 2560, 3, 2), (70_000, 2560, 8, 2),
                       (3_000, 8192, 32, 2), (17, 512, 6, 1), (100_003, 1024, 1, 1), (64, 2560, 24, 2),
                       (40, 2560, 1, 1), (200, 2560, 2, 2)]:
        w_np = synth.normal_bf16(8000 + r, r, k, 0.02)
        h_np = synth.hidden(8100 + r, 0, m, k)
        w_dev, h_dev = dev_bf16(w_np), dev_bf16(h_np)
        d2t_np = (np.arange(r) * 3 + 5).astype(np.int32)
        d2t = dev_i32(d2t_np)
        a = L.draft_project_argmax_fused_path(h_dev, w_dev, d2t, p, state)
        b = L.draft_project_argmax_path(h_dev, w_dev, d2t, p)
        assert same(a, b), (r, k, m, p)
        assert nonzero_bytes(state) == 0, (r, k, m, p)
        res = oracle.oracle_project_argmax(h_np, w_np, d2t_np, keep_logits=True)
        check(h_np, w_np, d2t_np, a[0].cpu().numpy(), a[1].cpu().numpy(), res)


@pytest.mark.parametrize("m", [1, 3, 6])
def test_ties_across_merge_groups_go_to_the_smallest_row(L, m):
    """Small-integer weights and hidden rows make every logit exact; the
    largest logit is planted in rows far apart (different workgroups, so
    different merge groups) and in neighbouring rows (one workgroup): the
    fused call returns the smallest such row on both kernels."""
    rng = np.random.default_rng(950 + m)
    n, k = 60_000, 256
    wi = rng.integers(-2, 3, size=(n, k)).astype(np.float32)
    hi = rng.integers(-1, 2, size=(m, k)).astype(np.float32)
    for j in range(m):
        for r in (59_990 - j, 41_000 + j, 20_001 + j, 20_003 + j, 7_777 + 5 * j):
            wi[r] = 3.0 * np.sign(hi[j])
    w = synth.bf16_from_f32(wi)
    h = synth.bf16_from_f32(hi)
    res = oracle.oracle_project_argmax(h, w)
    assert np.all(res.gap == 0)
    w_dev, h_dev = dev_bf16(w), dev_bf16(h)
    state = L.new_state("cuda")
    for path in (L.LMH_PATH_VALU, L.LMH_PATH_MFMA):
        i, lg = L.draft_project_argmax_fused_path(h_dev, w_dev, None, path, state)
        assert np.array_equal(i.cpu().numpy(), res.id), (path, i, res.id)
        assert np.array_equal(lg.cpu().numpy().astype(np.float64), res.logit)
        assert nonzero_bytes(state) == 0


def test_fused_graph_replays_match_eager(L):
    """Fused calls of M = 1, 3 and 24 captured in one graph on one state,
    replayed with the hidden rows rewritten in place and eager calls and
    synchronizations between replays: every replay equals the eager calls,
    and the state is zero after each."""
    inp = config_inputs(3)
    wt = L.lmhead_trim(device_weights(3), dev_i32(inp["ids"]))
    d2t = dev_i32(inp["ids"])
    ms = (1, 3, 24)
    hs = {m: torch.empty((m, 2560), dtype=torch.int16, device="cuda") for m in ms}
    outs = {m: (torch.empty(m, dtype=torch.int32, device="cuda"), torch.empty(m, dtype=torch.float32, device="cuda"))
            for m in ms}
    state = L.new_state("cuda")
    draws_ = {m: [synth.hidden(7300 + m, d, m, 2560) for d in range(3)] for m in ms}
    for m in ms:
        hs[m].copy_(dev_bf16(draws_[m][0]))
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        for m in ms:
            L.draft_project_argmax_fused(hs[m], wt, d2t, state, outs[m][0], outs[m][1], cap)
    torch.cuda.synchronize()
    for rep in range(6):
        d = rep % 3
        for m in ms:
            hs[m].copy_(dev_bf16(draws_[m][d]))
        graph.replay()
        torch.cuda.synchronize()
        for m in ms:
            want = L.draft_project_argmax(dev_bf16(draws_[m][d]), wt, d2t)
            assert same(outs[m], want), (rep, m)
        assert nonzero_bytes(state) == 0, rep
        # eager fused work on the same state between replays
        L.draft_project_argmax_fused(dev_bf16(draws_[3][d]), wt, d2t, state)
        torch.cuda.synchronize()
        assert nonzero_bytes(state) == 0, rep


def test_prepared_fused_matches_the_call(L):
    inp = config_inputs(4)
    wt = L.lmhead_trim(device_weights(4), dev_i32(inp["ids"]))
    d2t = dev_i32(inp["ids"])
    for m in (1, 3, 24):
        h = torch.empty((m, 2560), dtype=torch.int16, device="cuda")
        step = L.PreparedArgmax(h, wt, d2t, state=L.new_state("cuda"))
        for d in range(3):
            h_np = synth.hidden(7400 + m, d, m, 2560)
            h.copy_(dev_bf16(h_np))
            got = step()
            assert same(got, L.draft_project_argmax(dev_bf16(h_np), wt, d2t)), (m, d)


def test_fused_rejects_and_writes_nothing(L):
    w = dev_bf16(synth.normal_bf16(3, 100, 256, 0.02))
    h = dev_bf16(synth.hidden(4, 0, 2, 256))
    oid = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    olg = torch.full((2,), 5.0, device="cuda")
    f = L.lib().draft_project_argmax_fused
    state = L.new_state("cuda")
    base = (h.data_ptr(), 2, 256, w.data_ptr(), 100, None, oid.data_ptr(), olg.data_ptr())
    assert f(*base, None, L.LMH_STATE_BYTES, None) == L.LMH_EWORKSPACE
    assert f(*base, state.data_ptr() + 8, L.LMH_STATE_BYTES - 8, None) == L.LMH_EWORKSPACE   # misaligned
    assert f(*base, state.data_ptr(), L.LMH_STATE_BYTES - 1, None) == L.LMH_EWORKSPACE        # too small
    assert f(h.data_ptr(), 0, 256, w.data_ptr(), 100, None, oid.data_ptr(), olg.data_ptr(), state.data_ptr(),
             L.LMH_STATE_BYTES, None) == L.LMH_EINVAL
    torch.cuda.synchronize()
    assert bool((oid == 7).all()) and bool((olg == 5.0).all())
    assert nonzero_bytes(state) == 0


def _random_cases(n=30, seed=20261206):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        m = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 17, 24, 31, 32]))
        k = 8 * int(rng.integers(1, (1024 if rng.random() < 0.5 else 8192) // 8 + 1))
        rmax = max(1, min(70_000, 16_000_000 // k))
        r = int(rng.integers(1, min(rmax, 600) + 1)) if rng.random() < 0.5 or rmax <= 600 else \
            int(np.exp(rng.uniform(np.log(600), np.log(rmax))))
        out.append((i, m, k, r, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("case", _random_cases(),
                         ids=lambda c: f"{c[0]}-M{c[1]}-K{c[2]}-R{c[3]}{'-d2t' if c[4] else ''}")
def test_fused_random_shapes(L, case):
    """Seeded random shapes (M, K, R, d2t) on every kernel that takes them:
    the single launch equals the two-kernel call bit for bit and leaves the
    state at zero."""
    i, m, k, r, with_d2t = case
    rng = np.random.default_rng(12000 + i)
    w_dev = dev_bf16(synth.normal_bf16(12100 + i, r, k, 0.02))
    h_dev = dev_bf16(synth.hidden(12200 + i, 0, m, k))
    d2t = dev_i32(rng.permutation(r + int(rng.integers(0, 2 * r + 1)))[:r].astype(np.int32)) if with_d2t else None
    state = L.new_state("cuda")
    paths = [L.LMH_PATH_AUTO, L.LMH_PATH_MFMA]
    if L.lib().draft_project_auto_path_rows(m, k, r) == L.LMH_PATH_VALU or m <= 8:
        paths.append(L.LMH_PATH_VALU)
    for p in paths:
        try:
            b = L.draft_project_argmax_path(h_dev, w_dev, d2t, p)
        except L.LmheadError:
            continue                                   # this kernel does not take the shape
        a = L.draft_project_argmax_fused_path(h_dev, w_dev, d2t, p, state)
        assert same(a, b), (case, p)
        assert nonzero_bytes(state) == 0, (case, p)


@pytest.mark.parametrize("m,cfg", [(1, 2), (3, 3), (24, 5)])
def test_fused_many_calls_back_to_back(L, m, cfg):
    """400 single launches queued back to back on one state (each with
    its own hidden rows and output slot, no synchronization between them),
    against the two-kernel call on the same inputs, bit for bit: every
    launch's merge must see every workgroup's maxima and leave the state
    clean for the next one.  The full head at one hidden row has the most
    workgroups per launch (the most atomics per ticket)."""
    inp = config_inputs(cfg)
    if cfg == 2:
        w = device_weights(2)
        d2t = None
    else:
        w = L.lmhead_trim(device_weights(cfg), dev_i32(inp["ids"]))
        d2t = dev_i32(inp["ids"])
    n = 400
    k = inp["config"].k
    hs = dev_bf16(np.concatenate([synth.hidden(13000 + m, d, m, k) for d in range(n)]))  # [n * m, K]
    state = L.new_state("cuda")
    fid = torch.empty((n, m), dtype=torch.int32, device="cuda")
    flg = torch.empty((n, m), dtype=torch.float32, device="cuda")
    rid = torch.empty((n, m), dtype=torch.int32, device="cuda")
    rlg = torch.empty((n, m), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(M=m)
    for i in range(n):
        h = hs[i * m:(i + 1) * m]
        L.draft_project_argmax_fused(h, w, d2t, state, fid[i], flg[i])
    for i in range(n):
        h = hs[i * m:(i + 1) * m]
        L.draft_project_argmax(h, w, d2t, rid[i], rlg[i], ws)
    torch.cuda.synchronize()
    assert torch.equal(fid, rid)
    assert torch.equal(flg.view(torch.int32), rlg.view(torch.int32))
    assert nonzero_bytes(state) == 0
