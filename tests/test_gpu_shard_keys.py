"""The one-GPU part of the vocabulary split: draft_project_argmax_keys over
contiguous slices of a head, combined by one MAX over the slices' keys (what
an all-reduce across GPUs would do), against the fp64 oracle over the whole
head, through the C ABI.

Slices: the full 248,320-row head in 2 slices of 124,160 rows (the TP = 2
shard of the Two Sparks kernel table) and in 8 slices of 31,040; and the
52,755-id list split evenly by list position into 2 (the balanced split of
"Build the draft vocabulary from your own text"), whose combined row is a
list position mapped through the list afterwards.  A slice's rows are
summed exactly as in the whole-head call (same kernel, same per-row order),
so the combined result must also equal the single call bit for bit.  Exact
ties planted across slices must go to the smallest global row.
"""
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


def decode(keys):
    """(rows, fp32 logits) of packed keys: row = 0xFFFFFFFF - low word;
    the high word holds the logit's order-preserving bits."""
    k = np.asarray(keys).view(np.uint64)
    ordb = (k >> np.uint64(32)).astype(np.uint32)
    bits = np.where(ordb & np.uint32(0x80000000), ordb & np.uint32(0x7FFFFFFF), ~ordb).astype(np.uint32)
    rows = (np.uint64(0xFFFFFFFF) - (k & np.uint64(0xFFFFFFFF))).astype(np.int64)
    return np.where(k == 0, -1, rows), bits.view(np.float32)


def combined(L, h_dev, w_dev, bounds, path=0):
    """Keys of every slice [bounds[i], bounds[i+1]) of w_dev, then the MAX."""
    keys = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        keys.append(L.draft_project_argmax_keys(h_dev, w_dev[a:b], a, path).cpu().numpy().view(np.uint64))
    return decode(np.stack(keys).max(axis=0))


def even_bounds(n, g):
    return [n * i // g for i in range(g + 1)]


@pytest.mark.parametrize("m", [1, 3, 24])
@pytest.mark.parametrize("g", [2, 8])
def test_full_head_split(L, g, m):
    inp = config_inputs(2)
    c = inp["config"]
    w_np, w_dev = inp["W"], device_weights(2)
    hs = draws(c, m, 16) if m == 1 else [synth.hidden(5000 + m, d, m, c.k) for d in range(16 if m < 24 else 6)]
    bounds = even_bounds(w_np.shape[0], g)
    assert g != 2 or bounds[1] == 124_160
    assert g != 8 or bounds[1] == 31_040
    stack = np.concatenate(hs)
    res = oracle.oracle_project_argmax(stack, w_np, None, keep_logits=True)
    rows, logits = [], []
    for h in hs:
        hd = dev_bf16(h)
        r, lg = combined(L, hd, w_dev, bounds)
        one = L.draft_project_argmax(hd, w_dev)          # the whole head in one call
        assert np.array_equal(r, one[0].cpu().numpy())
        assert np.array_equal(lg.view(np.uint32), one[1].cpu().numpy().view(np.uint32))
        rows.append(r)
        logits.append(lg)
    st = ParityStats()
    st.add(check(stack, w_np, None, np.concatenate(rows), np.concatenate(logits), res))
    log(f"[split {g} M={m}] rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e}")
    st.assert_exempt_bound()


@pytest.mark.parametrize("m", [1, 3, 24])
def test_balanced_list_split(L, m):
    """The 52,755-id list split evenly by position into 2 halves, each
    trimmed on its own; the MAX gives a list position, mapped through the
    list to the vocabulary id."""
    inp = config_inputs(5)
    ids = inp["ids"]
    w_dev = device_weights(5)
    halves = even_bounds(ids.size, 2)
    parts = [L.lmhead_trim(w_dev, dev_i32(ids[a:b])) for a, b in zip(halves[:-1], halves[1:])]
    hs = [synth.hidden(6000 + m, d, m, inp["config"].k) for d in range(16 if m < 24 else 6)]
    stack = np.concatenate(hs)
    w_trim = oracle.oracle_trim(inp["W"], ids)
    res = oracle.oracle_project_argmax(stack, w_trim, ids, keep_logits=True)
    got_ids, got_logits = [], []
    for h in hs:
        hd = dev_bf16(h)
        keys = [L.draft_project_argmax_keys(hd, p, a).cpu().numpy().view(np.uint64)
                for p, a in zip(parts, halves[:-1])]
        pos, lg = decode(np.stack(keys).max(axis=0))
        got_ids.append(ids[pos])
        got_logits.append(lg)
    st = ParityStats()
    st.add(check(stack, w_trim, ids, np.concatenate(got_ids), np.concatenate(got_logits), res))
    log(f"[list split M={m}] rows={st.rows} near_ties={st.near_ties} exempt={st.exempt} max_err={st.max_err:.2e}")
    st.assert_exempt_bound()


@pytest.mark.parametrize("m", [1, 3, 6])
def test_ties_across_slices_go_to_the_smallest_row(L, m):
    """Small-integer weights and hidden rows make every logit exact; rows
    with the largest logit are planted in several slices, and in one slice
    twice: the combined key names the smallest global row, on both
    kernels, and equals the whole-head call."""
    rng = np.random.default_rng(900 + m)
    n, k = 40_000, 256
    wi = rng.integers(-2, 3, size=(n, k)).astype(np.float32)
    hi = rng.integers(-1, 2, size=(m, k)).astype(np.float32)
    for j in range(m):
        for r in (39_990 - j, 25_000 + j, 20_001 + j, 20_003 + j):   # across and inside slices
            wi[r] = 3.0 * np.sign(hi[j])
    w = synth.bf16_from_f32(wi)
    h = synth.bf16_from_f32(hi)
    res = oracle.oracle_project_argmax(h, w)
    assert np.all(res.gap == 0)                                        # exact ties everywhere
    w_dev, h_dev = dev_bf16(w), dev_bf16(h)
    bounds = [0, 10_000, 20_002, 30_000, n]
    for path in (L.LMH_PATH_VALU, L.LMH_PATH_MFMA):
        rows, lg = combined(L, h_dev, w_dev, bounds, path)
        assert np.array_equal(rows, res.id), (path, rows, res.id)
        assert np.array_equal(lg.astype(np.float64), res.logit)
        one = L.draft_project_argmax_path(h_dev, w_dev, None, path)
        assert np.array_equal(rows, one[0].cpu().numpy())


def test_keys_reject_and_write_nothing(L):
    w = dev_bf16(synth.normal_bf16(3, 100, 256, 0.02))
    h = dev_bf16(synth.hidden(4, 0, 2, 256))
    out = torch.full((2,), 7, dtype=torch.int64, device="cuda")
    ws = L.new_workspace()
    lib = L.lib()
    f = lib.draft_project_argmax_keys
    base = (h.data_ptr(), 2, 256, w.data_ptr(), 100)
    assert f(*base, -1, out.data_ptr(), ws.data_ptr(), ws.numel(), 0, None) == L.LMH_EINVAL
    assert f(*base, (1 << 32) - 100, out.data_ptr(), ws.data_ptr(), ws.numel(), 0, None) == L.LMH_EINVAL
    assert f(*base, 0, out.data_ptr() + 4, ws.data_ptr(), ws.numel(), 0, None) == L.LMH_EINVAL
    assert f(*base, 0, None, ws.data_ptr(), ws.numel(), 0, None) == L.LMH_EINVAL
    assert f(*base, 0, out.data_ptr(), ws.data_ptr(), 8, 0, None) == L.LMH_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7).all())
    # the largest base that keeps every global row below 2^32 - 1 is taken
    k = L.draft_project_argmax_keys(h, w, (1 << 32) - 101)
    rows, _ = decode(k.cpu().numpy())
    one = L.draft_project_argmax(h, w)[0].cpu().numpy().astype(np.int64)
    assert np.array_equal(rows, (1 << 32) - 101 + one)
