"""HIP graph capture of the per-step calls.

The projection entry points only launch kernels (no allocation, no
synchronization, no memset), so a serving loop can capture a draft step in
a graph and replay it.  Each test captures several calls, replays the graph
several times with the hidden rows rewritten in place and with eager calls
and synchronizations between the replays, and checks every replay bit for
bit against eager calls on the same inputs (the kernels are deterministic,
so graph and eager results must be identical), and one replay against the
fp64 oracle."""
import numpy as np
import pytest

import synth
from parity import check
from test_gpu_parity import dev_bf16, dev_i32, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

K = 2560
R = 20_011          # ragged: not a multiple of any tile height


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


@pytest.fixture(scope="module")
def head():
    w_np = synth.normal_bf16(4242, R, K, 0.02)
    ids = np.sort(np.random.default_rng(7).choice(248_320, R, replace=False)).astype(np.int32)
    return w_np, ids


def hidden_sets(m, n):
    return [synth.hidden(900 + m, d, m, K) for d in range(n)]


def test_argmax_and_topk_replays_match_eager(L, head):
    w_np, ids = head
    w = dev_bf16(w_np)
    d2t = dev_i32(ids)
    # calls of one step: (M, path, top k or 0); every kernel family takes part
    plan = [(1, L.LMH_PATH_AUTO, 0), (2, L.LMH_PATH_AUTO, 0), (3, L.LMH_PATH_AUTO, 0),
            (24, L.LMH_PATH_AUTO, 0), (4, L.LMH_PATH_AUTO, 8), (16, L.LMH_PATH_MFMA, 16)]
    draws = {m: hidden_sets(m, 4) for m, _, _ in plan}
    calls = []
    for m, path, k in plan:
        h = torch.empty((m, K), dtype=torch.int16, device="cuda")
        if k:
            oid = torch.empty((m, k), dtype=torch.int32, device="cuda")
            olog = torch.empty((m, k), dtype=torch.float32, device="cuda")
            ws = torch.empty(L.draft_project_topk_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
        else:
            oid = torch.empty(m, dtype=torch.int32, device="cuda")
            olog = torch.empty(m, dtype=torch.float32, device="cuda")
            ws = L.new_workspace(M=m)
        calls.append((m, path, k, h, oid, olog, ws))

    def launch(m, path, k, h, oid, olog, ws, stream=None):
        if k:
            L.draft_project_topk(h, w, d2t, k, oid, olog, ws, path, stream)
        else:
            L.draft_project_argmax_path(h, w, d2t, path, oid, olog, ws, stream)

    # eager reference results for every draw, on their own outputs
    want = {}
    for m, path, k, *_ in calls:
        for d, h_np in enumerate(draws[m]):
            if k:
                i, l = L.draft_project_topk(dev_bf16(h_np), w, d2t, k, path=path)
            else:
                i, l = L.draft_project_argmax_path(dev_bf16(h_np), w, d2t, path)
            want[(m, k, d)] = (i.cpu().numpy(), l.cpu().numpy())

    # warm up every call on the capture buffers, then capture all of them
    for c in calls:
        c[3].copy_(dev_bf16(draws[c[0]][0]))
        launch(*c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            launch(*c)
    torch.cuda.synchronize()

    spare_ws = L.new_workspace()
    for rep in range(6):
        d = rep % 4
        for c in calls:
            c[3].copy_(dev_bf16(draws[c[0]][d]))
            c[4].fill_(-7)
            c[5].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m, path, k, h, oid, olog, ws in calls:
            wi, wl = want[(m, k, d)]
            assert np.array_equal(oid.cpu().numpy(), wi), (rep, m, k)
            assert np.array_equal(olog.cpu().numpy().view(np.uint32), wl.view(np.uint32)), (rep, m, k)
        # eager work of the program between replays, on the same stream
        hx = dev_bf16(draws[3][(d + 1) % 4])
        i, l = L.draft_project_argmax(hx, w, d2t, workspace=spare_ws)
        torch.cuda.synchronize()
        assert np.array_equal(i.cpu().numpy(), want[(3, 0, (d + 1) % 4)][0])
        log(f"[graph] replay {rep}: {len(calls)} calls bit-identical to eager")

    # one replay's argmax rows against the fp64 oracle
    m = 24
    i, l = want[(m, 0, 1)]
    st = check(draws[m][1], w_np, ids, i, l)
    log(f"[graph] M=24 against the oracle: rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e}")
    st.assert_exempt_bound()


def test_quantized_heads_replay_match_eager(L, head):
    w_np, ids = head
    w = dev_bf16(w_np)
    d2t = dev_i32(ids)
    q8, s8 = L.lmhead_quantize_fp8(w)
    q4, s4 = L.lmhead_quantize_mxfp4(w)
    torch.cuda.synchronize()
    plan = [("fp8", 1), ("fp8", 24), ("mx4", 3), ("mx4", 24)]
    draws = {m: hidden_sets(m, 3) for _, m in plan}

    def launch(fmt, h, oid, olog, ws):
        if fmt == "fp8":
            L.draft_project_argmax_fp8(h, q8, s8, d2t, L.LMH_PATH_AUTO, oid, olog, ws)
        else:
            L.draft_project_argmax_mxfp4(h, q4, s4, d2t, L.LMH_PATH_AUTO, oid, olog, ws)

    calls = []
    want = {}
    for fmt, m in plan:
        h = torch.empty((m, K), dtype=torch.int16, device="cuda")
        oid = torch.empty(m, dtype=torch.int32, device="cuda")
        olog = torch.empty(m, dtype=torch.float32, device="cuda")
        ws = L.new_workspace(M=m)
        calls.append((fmt, h, oid, olog, ws))
        for d, h_np in enumerate(draws[m]):
            h.copy_(dev_bf16(h_np))
            launch(fmt, h, oid, olog, ws)
            want[(fmt, m, d)] = (oid.cpu().numpy().copy(), olog.cpu().numpy().copy())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            launch(*c)
    torch.cuda.synchronize()
    for rep in range(5):
        d = rep % 3
        for fmt, h, oid, olog, ws in calls:
            h.copy_(dev_bf16(draws[h.shape[0]][d]))
            oid.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for fmt, h, oid, olog, ws in calls:
            wi, wl = want[(fmt, h.shape[0], d)]
            assert np.array_equal(oid.cpu().numpy(), wi), (rep, fmt, h.shape[0])
            assert np.array_equal(olog.cpu().numpy().view(np.uint32), wl.view(np.uint32)), (rep, fmt)
        log(f"[graph] quantized replay {rep}: bit-identical to eager")


def test_prepared_argmax_matches_the_call(L, head):
    """PreparedArgmax (tensors checked once, one C call per step) gives the
    ordinary call's results bit for bit while the hidden rows are rewritten
    in place between steps, on each kernel family."""
    import time
    w_np, ids = head
    w = dev_bf16(w_np)
    d2t = dev_i32(ids)
    for m in (1, 2, 3, 24):
        h = torch.empty((m, K), dtype=torch.int16, device="cuda")
        step = L.PreparedArgmax(h, w, d2t, workspace=L.new_workspace(M=m))
        for d, h_np in enumerate(hidden_sets(m, 3)):
            h.copy_(dev_bf16(h_np))
            i, l = step()
            wi, wl = L.draft_project_argmax(dev_bf16(h_np), w, d2t)
            assert np.array_equal(i.cpu().numpy(), wi.cpu().numpy()), (m, d)
            assert np.array_equal(l.cpu().numpy().view(np.uint32), wl.cpu().numpy().view(np.uint32)), (m, d)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(200):
            step()
        host = (time.perf_counter() - t0) / 200 * 1e6
        torch.cuda.synchronize()
        log(f"[prepared] M={m}: bit-identical to the call; host time per queued step {host:.1f} us")
