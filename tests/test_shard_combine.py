"""The combine rule of the vocabulary split across GPUs, on the CPU.

Split across G devices, each device would project its own slice of head
rows and hand over, per hidden row, one 64-bit key: the order-preserving
bits of its best fp32 logit in the high half and (2^32 - 1 - global row) in
the low half.  One MAX over the G keys then names the global winner, with
the smallest row winning ties, so the all-reduce moves 8 bytes per hidden
row and no logit leaves its device.  No rank code is built here (one GPU);
these tests pin that rule against the single-device argmax of the oracle,
with fp32 logits as the GPU takes its decision in fp32."""
import numpy as np
import pytest

import oracle.lmhead_oracle as lo
import synth


def ordered_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> uint32 whose unsigned order is the float order (-0 as +0)."""
    v = np.where(v == 0, np.float32(0), v).astype(np.float32)
    b = v.view(np.uint32).astype(np.uint64)
    neg = (b >> np.uint64(31)) == 1
    return np.where(neg, ~b & np.uint64(0xFFFFFFFF), b | np.uint64(0x80000000))


def shard_keys(logits32: np.ndarray, lo_row: int, hi_row: int) -> np.ndarray:
    """One device's keys: the best row of its slice [lo_row, hi_row) per
    hidden row (first occurrence inside the slice), packed."""
    part = logits32[:, lo_row:hi_row]
    local = np.argmax(part, axis=1)
    best = part[np.arange(part.shape[0]), local]
    row = (lo_row + local).astype(np.uint64)
    return (ordered_bits(best) << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - row)


def combine(logits32: np.ndarray, bounds) -> np.ndarray:
    keys = np.stack([shard_keys(logits32, a, b) for a, b in zip(bounds[:-1], bounds[1:])])
    top = keys.max(axis=0)                                   # the one all-reduce(MAX)
    return (np.uint64(0xFFFFFFFF) - (top & np.uint64(0xFFFFFFFF))).astype(np.int64)


@pytest.mark.parametrize("g", [1, 2, 3, 8])
def test_split_then_max_equals_one_device(g):
    w = synth.normal_bf16(31, 6_000, 128, 0.02)
    h = synth.hidden(32, 0, 5, 128)
    logits32 = lo.oracle_logits(h, w).astype(np.float32)
    want = np.argmax(logits32, axis=1)                       # first occurrence on one device
    n = w.shape[0]
    even = [n * i // g for i in range(g + 1)]                # the even split of the pages' TP head
    assert np.array_equal(combine(logits32, even), want)
    rng = np.random.default_rng(g)
    cuts = np.sort(rng.choice(np.arange(1, n), size=g - 1, replace=False)) if g > 1 else []
    assert np.array_equal(combine(logits32, [0, *cuts, n]), want)


def test_ties_across_shards_go_to_the_smallest_row():
    logits32 = np.zeros((4, 12), dtype=np.float32)
    logits32[0, [2, 9]] = 5.0          # tie across two shards
    logits32[1, [7, 8]] = -1.0         # tie inside a shard, everything else lower
    logits32[1, :7] = -3.0
    logits32[1, 9:] = -3.0
    logits32[2, :] = -0.0              # all zeros of both signs
    logits32[2, 5] = 0.0
    logits32[3, [3, 11]] = np.float32(1e-30)
    got = combine(logits32, [0, 4, 8, 12])
    assert list(got) == [2, 7, 0, 3]
    assert np.array_equal(got, np.argmax(logits32, axis=1))


def test_key_order_is_float_order():
    v = np.array([-np.inf, -3.5, -1e-30, -0.0, 0.0, 1e-30, 2.0, np.inf], dtype=np.float32)
    k = ordered_bits(v)
    assert np.all(np.diff(k[[0, 1, 2, 3, 5, 6, 7]].astype(np.float64)) > 0)
    assert k[3] == k[4]                # -0 and +0 compare equal


def test_a_shortlist_splits_the_same_way():
    """A trimmed head is split by list position; d2t maps the winner."""
    w = synth.normal_bf16(41, 5_000, 64, 0.02)
    ids = np.sort(np.random.default_rng(5).choice(5_000, 777, replace=False)).astype(np.int32)
    h = synth.hidden(42, 0, 3, 64)
    trimmed = lo.oracle_trim(w, ids)
    logits32 = lo.oracle_logits(h, trimmed).astype(np.float32)
    pos = combine(logits32, [0, 200, 401, 777])
    assert np.array_equal(ids[pos], ids[np.argmax(logits32, axis=1)])
