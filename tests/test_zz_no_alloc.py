"""draft_project_argmax_noalloc through the C ABI: the argmax with no
workspace (the library's static device array holds the per-workgroup keys)
must give exactly what draft_project_argmax gives with a workspace, and meet
the parity rule against the fp64 oracle, on two calls in a row, the second
on a smaller input (fewer hidden rows and head rows, so a smaller grid over
slots the first call left behind)."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from devcopy import dev_bf16, dev_i32
from parity import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from vocab_shortlisted_lm_amd import lmhead
    lmhead.lib()
    return lmhead


def call_noalloc(L, h, w, d2t, m, k, r):
    """One call of the allocation-free entry point through ctypes, into
    preallocated outputs."""
    oid = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    olg = torch.full((m,), 1e30, dtype=torch.float32, device="cuda")
    code = L.lib().draft_project_argmax_noalloc(
        ctypes.c_void_p(h.data_ptr()), m, k, ctypes.c_void_p(w.data_ptr()), r,
        ctypes.c_void_p(d2t.data_ptr()) if d2t is not None else None,
        ctypes.c_void_p(oid.data_ptr()), ctypes.c_void_p(olg.data_ptr()), None)
    assert code == L.LMH_OK, L.lmhead_status_str(code)
    return oid, olg


def call_workspace(L, h, w, d2t, m, k, r):
    oid = torch.empty((m,), dtype=torch.int32, device="cuda")
    olg = torch.empty((m,), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.draft_project_workspace_bytes(m), dtype=torch.uint8, device="cuda")
    code = L.lib().draft_project_argmax(
        h.data_ptr(), m, k, w.data_ptr(), r, d2t.data_ptr() if d2t is not None else None, oid.data_ptr(),
        olg.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert code == L.LMH_OK, L.lmhead_status_str(code)
    return oid, olg


CASES = [
    # (seed, M, K, rows, with d2t): the first is the larger call
    (11, 24, 2560, 52_755, True),
    (12, 3, 2560, 16_000, True),
    (13, 1, 2560, 248_320, False),
    (14, 2, 256, 4_096, True),
]


def test_noalloc_two_calls_then_smaller(L):
    first, second = CASES[0], CASES[1]
    for seed, m, k, r, with_d2t in (first, second):
        w_np = synth.normal_bf16(seed, r, k, 0.02)
        h_np = synth.hidden(seed + 100, 0, m, k)
        d2t_np = (np.arange(r, dtype=np.int32) * 3 + 1) if with_d2t else None
        w, h = dev_bf16(w_np), dev_bf16(h_np)
        d2t = dev_i32(d2t_np) if with_d2t else None
        a = call_noalloc(L, h, w, d2t, m, k, r)
        b = call_workspace(L, h, w, d2t, m, k, r)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]), (m, r)
        assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), (m, r)
        res = oracle.oracle_project_argmax(h_np, w_np, d2t_np, keep_logits=True)
        check(h_np, w_np, d2t_np, a[0].cpu().numpy(), a[1].cpu().numpy(), res)


def test_noalloc_shapes_in_sequence_and_rejects(L):
    """Four calls of falling and rising size on one device in a row, each
    equal to the workspace call; an invalid call is rejected before any
    launch and writes nothing."""
    for seed, m, k, r, with_d2t in CASES + [CASES[0]]:
        w_np = synth.normal_bf16(seed, r, k, 0.02)
        h_np = synth.hidden(seed + 200, 0, m, k)
        d2t_np = (np.arange(r, dtype=np.int32) * 5 + 2) if with_d2t else None
        w, h = dev_bf16(w_np), dev_bf16(h_np)
        d2t = dev_i32(d2t_np) if with_d2t else None
        a = call_noalloc(L, h, w, d2t, m, k, r)
        b = call_workspace(L, h, w, d2t, m, k, r)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), (m, r)
    w = dev_bf16(synth.normal_bf16(3, 100, 256, 0.02))
    h = dev_bf16(synth.hidden(4, 0, 2, 256))
    oid = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    olg = torch.full((2,), 5.0, device="cuda")
    f = L.lib().draft_project_argmax_noalloc
    assert f(h.data_ptr(), 33, 256, w.data_ptr(), 100, None, oid.data_ptr(), olg.data_ptr(), None) == L.LMH_EINVAL
    assert f(h.data_ptr(), 2, 256, w.data_ptr(), 0, None, oid.data_ptr(), olg.data_ptr(), None) == L.LMH_EINVAL
    assert f(h.data_ptr(), 2, 256, w.data_ptr(), 100, None, None, olg.data_ptr(), None) == L.LMH_EINVAL
    torch.cuda.synchronize()
    assert bool((oid == 7).all()) and bool((olg == 5.0).all())
