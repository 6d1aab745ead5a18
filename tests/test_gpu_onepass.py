"""The single-launch argmax (lmhead_bench_argmax_onepass) through the C ABI:
the workgroup that takes the last ticket folds every workgroup's key, so one
launch replaces the projection + fold pair.  It runs the same projection
kernels with the same per-row sums, so its outputs must equal the two-kernel
call bit for bit, meet the parity rule against the fp64 oracle, and leave the
ticket at zero after every call (several launches of different grids on one
workspace, both kernels, a multi-pass M)."""
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


def ticket_of(L, ws, m):
    """The ticket: the workspace's first 4 bytes, whatever M."""
    return int(ws[0:4].cpu().numpy().view(np.uint32)[0])


def run(L, hs, w_np, w_dev, d2t_np, paths, tag):
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax(stack, w_np, d2t_np, keep_logits=True)
    d2t_dev = dev_i32(d2t_np) if d2t_np is not None else None
    m = hs[0].shape[0]
    ws = L.lmhead_bench_onepass_workspace("cuda", m)
    for p in paths:
        ids, lgs = [], []
        for h in hs:
            hd = dev_bf16(h)
            a = L.lmhead_bench_argmax_onepass(hd, w_dev, d2t_dev, p, ws)
            b = L.draft_project_argmax_path(hd, w_dev, d2t_dev, p)
            assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), tag
            ids.append(a[0].cpu().numpy())
            lgs.append(a[1].cpu().numpy())
        assert ticket_of(L, ws, m) == 0
        st = ParityStats()
        st.add(check(stack, w_np, d2t_np, np.concatenate(ids), np.concatenate(lgs), res))
        log(f"[onepass {tag}] path={p} rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} "
            f"max_err={st.max_err:.2e}")
        st.assert_exempt_bound()


@pytest.mark.parametrize("cfg,m", [(2, 1), (3, 3), (4, 1), (4, 4), (5, 24)])
def test_onepass_configs(L, cfg, m):
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


def test_onepass_full_head_m24(L):
    inp = config_inputs(2)
    hs = [synth.hidden(7024, d, 24, 2560) for d in range(4)]
    run(L, hs, inp["W"], device_weights(2), None, [L.LMH_PATH_MFMA], "full M=24")


def test_onepass_shapes_share_a_workspace(L):
    """Launches of different grids (heads of 1 to 300,000 rows, M from 1 to
    32 with K = 8,192, which takes two passes) one after another on one
    workspace: every call matches the two-kernel call and leaves the ticket
    at zero."""
    ws = L.lmhead_bench_onepass_workspace("cuda", 32)
    for r, k, m, p in [(1, 256, 1, 1), (300_000, 256, 2, 1), (5, 2560, 3, 2), (70_000, 2560, 8, 2),
                       (3_000, 8192, 32, 2), (17, 512, 6, 1), (100_003, 1024, 1, 1), (64, 2560, 24, 2)]:
        w_np = synth.normal_bf16(8000 + r, r, k, 0.02)
        h_np = synth.hidden(8100 + r, 0, m, k)
        w_dev, h_dev = dev_bf16(w_np), dev_bf16(h_np)
        d2t = dev_i32((np.arange(r) * 3 + 5).astype(np.int32))
        a = L.lmhead_bench_argmax_onepass(h_dev, w_dev, d2t, p, ws)
        b = L.draft_project_argmax_path(h_dev, w_dev, d2t, p)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), (r, k, m)
        assert ticket_of(L, ws, 32) == 0, (r, k, m)
        res = oracle.oracle_project_argmax(h_np, w_np, (np.arange(r) * 3 + 5).astype(np.int32), keep_logits=True)
        check(h_np, w_np, (np.arange(r) * 3 + 5).astype(np.int32), a[0].cpu().numpy(), a[1].cpu().numpy(), res)


def test_onepass_rejects(L):
    w = dev_bf16(synth.normal_bf16(3, 100, 256, 0.02))
    h = dev_bf16(synth.hidden(4, 0, 2, 256))
    oid = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    olg = torch.full((2,), 5.0, device="cuda")
    lib = L.lib()
    small = torch.zeros(L.draft_project_workspace_bytes(2), dtype=torch.uint8, device="cuda")
    code = lib.lmhead_bench_argmax_onepass(h.data_ptr(), 2, 256, w.data_ptr(), 100, None, oid.data_ptr(),
                                           olg.data_ptr(), small.data_ptr(), small.numel(), 0, None)
    assert code == L.LMH_EWORKSPACE           # no room for the ticket
    torch.cuda.synchronize()
    assert bool((oid == 7).all()) and bool((olg == 5.0).all())
