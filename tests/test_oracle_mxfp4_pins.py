"""Pins for the MXFP4 part of the fp64 oracle (CPU).

Each pin checks the oracle against something other than itself: the E2M1
value table written out from the format (sign, 2 exponent bits with bias 1,
1 mantissa bit), the round-to-nearest-even cases at every midpoint, the
block-scale rule of the MX conversion worked by hand, an error bound any
correct quantizer meets, exact round trips of representable heads,
correctly rounded sums, and the bf16 oracle on heads whose dequantized values
are exactly bf16.  ``test_mxfp4_mutants_are_caught`` plants plausible
mistakes and checks that at least one pin fails for each.  (torch has an
E2M1 dtype but no conversions to check against.)
"""
import math

import numpy as np
import pytest

import oracle.lmhead_oracle as lo
import oracle.mxfp4_head as mx
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16_exact(values):
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    return (bits >> 16).astype(np.uint16)


def _representable_head(rng, r, k, s_lo=-12, s_hi=-4):
    """Random codes and scales, with one element of every block at magnitude
    4 or 6 so the MX scale rule gives back the same scale; returns (codes
    packed, scales, W bits) with W exactly the dequantized head."""
    nb = k // 32
    codes = rng.integers(0, 16, size=(r, k)).astype(np.uint8)
    top = rng.integers(0, 32, size=(r, nb))
    big = rng.choice(np.array([6, 7, 14, 15], np.uint8), size=(r, nb))
    for b in range(nb):
        codes[np.arange(r), b * 32 + top[:, b]] = big[:, b]
    s = rng.integers(s_lo, s_hi + 1, size=(r, nb))
    vals = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])[codes]
    w = vals * np.repeat(np.ldexp(1.0, s), 32, axis=1)
    return mx.pack_nibbles(codes), (s + 127).astype(np.uint8), _bf16_exact(w)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_decode_table(m):
    # OCP MX v1.0, E2M1: 0 00 0 = 0, 0 00 1 = 0.5 (subnormal), 0 01 0 = 1.0,
    # 0 01 1 = 1.5, 0 10 0 = 2, 0 10 1 = 3, 0 11 0 = 4, 0 11 1 = 6; bit 3 = sign
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    got = m.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert got.tolist() == want
    assert np.signbit(got[8])


def pin_encode_midpoints(m):
    # every midpoint between neighbours goes to the even code (mantissa 0)
    cases = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6,
             0.2499: 0x0, 0.2501: 0x1, 0.7499: 0x1, 0.7501: 0x2, 1.2501: 0x3, 1.7499: 0x3,
             2.4999: 0x4, 2.5001: 0x5, 3.4999: 0x5, 3.5001: 0x6, 4.9999: 0x6, 5.0001: 0x7,
             0.0: 0x0, 6.0: 0x7, 4.0: 0x6}
    x = np.array(list(cases), np.float64)
    assert m.e2m1_encode(x).tolist() == list(cases.values())
    assert m.e2m1_encode(-x).tolist() == [c | 0x8 for c in cases.values()]


def pin_encode_saturates_and_round_trips(m):
    assert m.e2m1_encode(np.array([6.5, 7.9, 1e30, -9.0])).tolist() == [0x7, 0x7, 0x7, 0xF]
    codes = np.arange(16, dtype=np.uint8)
    back = m.e2m1_encode(m.e2m1_decode(codes))
    assert back.tolist() == codes.tolist()


def pin_block_scale_by_hand(m):
    # s = floor(log2 amax) - 2: amax 6 -> 0, 1 -> -2, 0.02 -> -8 (2**-6 <= 0.02 < 2**-5),
    # 4 -> 0, 3.99 -> -1, 2**-130 -> clamped -127, 0 -> 0
    amax = np.array([6.0, 1.0, 0.02, 4.0, 3.99, 2.0 ** -130, 0.0, 1e30])
    assert m.block_scale_exponent(amax).tolist() == [0, -2, -8, 0, -1, -127, 0, 97]
    # quantizing one block by hand: amax 0.02 -> X = 2**-8; 0.02 * 256 = 5.12 -> 6
    # (bf16 of 0.02 is 0.02001953125: x 256 = 5.125 -> 6; bf16 of -0.01 is
    # -0.010009765625: x 256 = -2.5625 -> -3; 3 / 1024 x 256 = 0.75 -> 1, a tie)
    row = np.zeros(32, np.float32)
    row[0], row[1], row[2] = 0.02, -0.01, 3.0 / 1024
    bits = synth.bf16_from_f32(row)
    assert lo.bf16_bits_to_f64(bits[:3]).tolist() == [0.02001953125, -0.010009765625, 3.0 / 1024]
    c, s = m.oracle_quantize_mxfp4(bits[None, :])
    assert s.tolist() == [[119]]
    codes = m.unpack_nibbles(c)[0]
    assert codes[:3].tolist() == [0x7, 0xD, 0x2]
    assert np.all(codes[3:] == 0)


def pin_quantize_error_bound(m):
    # any correct quantizer: 4 <= amax / X < 8 for a nonzero block, and every
    # element within |w| / 4 + X / 4 of its dequantized value
    w_bits = synth.normal_bf16(5, 64, 256, 0.02)
    w = lo.bf16_bits_to_f64(w_bits)
    codes, scales = m.oracle_quantize_mxfp4(w_bits)
    deq = m.oracle_dequant_mxfp4(codes, scales)
    x = np.repeat(np.ldexp(1.0, scales.astype(np.int32) - 127), 32, axis=1)
    ratio = np.abs(w).reshape(64, 8, 32).max(axis=2) / x[:, ::32]
    assert np.all((ratio >= 4) & (ratio < 8))
    assert np.all(np.abs(w - deq) <= np.abs(w) / 4 + x / 4)
    assert np.all(np.sign(deq) * np.sign(w) >= 0)


def pin_quantize_round_trip(m):
    rng = np.random.default_rng(7)
    packed, scales, w_bits = _representable_head(rng, 40, 128)
    c2, s2 = m.oracle_quantize_mxfp4(w_bits)
    assert np.array_equal(s2, scales)
    # -0 may come back as +0 only where the input was -0 (sign kept either way)
    assert np.array_equal(m.unpack_nibbles(c2), m.unpack_nibbles(packed))


def pin_zero_block(m):
    w = np.zeros((2, 64), np.float32)
    w[1, 40] = 1.5
    c, s = m.oracle_quantize_mxfp4(_bf16_exact(w))
    assert s.tolist() == [[127, 127], [127, 125]]
    assert np.all(m.unpack_nibbles(c)[0] == 0)
    assert m.unpack_nibbles(c)[1, 40] == 0x7      # 1.5 / 2**-2 = 6


def pin_projection_equals_bf16_oracle(m):
    rng = np.random.default_rng(11)
    packed, scales, w_bits = _representable_head(rng, 300, 256)
    h = synth.hidden(12, 0, 3, 256)
    got = m.oracle_logits_mxfp4(h, packed, scales)
    want = lo.oracle_logits(h, w_bits)
    assert np.array_equal(got, want)
    ids = rng.permutation(300).astype(np.int32)
    a = m.oracle_project_argmax_mxfp4(h, packed, scales, ids)
    b = lo.oracle_project_argmax(h, w_bits, ids)
    assert np.array_equal(a.id, b.id) and np.array_equal(a.logit, b.logit)


def pin_projection_fsum(m):
    rng = np.random.default_rng(13)
    w_bits = synth.normal_bf16(14, 6, 64, 0.02)
    codes, scales = m.oracle_quantize_mxfp4(w_bits)
    h = synth.hidden(15, 0, 2, 64)
    hv = lo.bf16_bits_to_f64(h)
    vals = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    got = m.oracle_logits_mxfp4(h, codes, scales)
    for r in range(6):
        # dequantize this row by hand: nibble k of byte k // 2, scale of block k // 32
        row = [vals[(codes[r, k // 2] >> (4 * (k % 2))) & 0xF] * 2.0 ** (int(scales[r, k // 32]) - 127)
               for k in range(64)]
        for i in range(2):
            want = math.fsum(hv[i, k] * row[k] for k in range(64))
            assert abs(got[i, r] - want) <= 1e-13 * max(1.0, abs(want))
    del rng


def pin_planted_winner(m):
    k = 128
    w_bits = synth.normal_bf16(21, 500, k, 0.02)
    h = synth.hidden(22, 0, 2, k)
    hv = lo.bf16_bits_to_f64(h)
    w = lo.bf16_bits_to_f64(w_bits).astype(np.float32)
    for i, j in enumerate((77, 420)):
        w[j] = np.float32(0.05) * np.sign(hv[i]).astype(np.float32)
    codes, scales = m.oracle_quantize_mxfp4(synth.bf16_from_f32(w))
    ids = (np.arange(500) * 3 + 1).astype(np.int32)
    res = m.oracle_project_argmax_mxfp4(h, codes, scales, ids)
    assert res.id.tolist() == [77 * 3 + 1, 420 * 3 + 1]


def pin_topk_equals_bf16_oracle(m):
    """On a head whose dequantized values are bf16 numbers, the top k over
    the MXFP4 head is the bf16 oracle's top k (ids, rows and logits),
    including k past the number of rows."""
    rng = np.random.default_rng(31)
    packed, scales, w_bits = _representable_head(rng, 400, 256)
    h = synth.hidden(32, 0, 3, 256)
    ids = rng.permutation(1000)[:400].astype(np.int32)
    for k in (1, 5, 16, 400, 403):
        a = m.oracle_project_topk_mxfp4(h, packed, scales, ids, k)
        b = lo.oracle_project_topk(h, w_bits, ids, k)
        assert np.array_equal(a.id, b.id) and np.array_equal(a.idx, b.idx)
        assert np.array_equal(a.logit, b.logit)


def pin_topk_order_and_first(m):
    """Best first, the first equal to the argmax, and the k logits are the k
    largest dot products with the hand-dequantized rows."""
    w_bits = synth.normal_bf16(33, 300, 512, 0.02)
    codes, scales = m.oracle_quantize_mxfp4(w_bits)
    h = synth.hidden(34, 0, 4, 512)
    ids = (np.arange(300) * 5 + 3).astype(np.int32)
    t = m.oracle_project_topk_mxfp4(h, codes, scales, ids, 8)
    a = m.oracle_project_argmax_mxfp4(h, codes, scales, ids)
    assert np.array_equal(t.id[:, 0], a.id) and np.array_equal(t.logit[:, 0], a.logit)
    vals = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    lo_nib, hi_nib = codes & 0xF, codes >> 4
    deq = np.empty((300, 512))
    deq[:, 0::2], deq[:, 1::2] = vals[lo_nib], vals[hi_nib]
    deq *= np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    full = lo.bf16_bits_to_f64(h) @ deq.T
    for i in range(4):
        assert np.all(np.diff(t.logit[i]) <= 0)
        assert np.allclose(t.logit[i], np.sort(full[i])[::-1][:8], rtol=1e-12, atol=1e-15)
        assert np.array_equal(t.id[i], ids[t.idx[i]])


PINS = [pin_decode_table, pin_encode_midpoints, pin_encode_saturates_and_round_trips,
        pin_block_scale_by_hand, pin_quantize_error_bound, pin_quantize_round_trip, pin_zero_block,
        pin_projection_equals_bf16_oracle, pin_projection_fsum, pin_planted_winner,
        pin_topk_equals_bf16_oracle, pin_topk_order_and_first]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_mxfp4_pin(pin):
    pin(mx)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

_orig_encode = mx.e2m1_encode
_orig_decode = mx.e2m1_decode
_orig_scale = mx.block_scale_exponent
_orig_logits = mx.oracle_logits_mxfp4
_orig_project = mx.oracle_project_argmax_mxfp4
_orig_pack = mx.pack_nibbles
_orig_unpack = mx.unpack_nibbles
_orig_quantize = mx.oracle_quantize_mxfp4


def _mut_encode_ties_up(x):
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    code = _orig_encode(x)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    up = np.isin(a, mids)
    return np.where(up, (np.searchsorted(mx._POS, a) | (code & 0x8)).astype(np.uint8), code).astype(np.uint8)


def _mut_encode_truncates(x):
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 6.0)
    code = (np.searchsorted(mx._POS, a, side="right") - 1).clip(0, 7).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 3)


def _mut_encode_wraps(x):
    x = np.asarray(x, np.float64)
    code = _orig_encode(x)
    return np.where(np.abs(x) > 6, code & 0x8, code).astype(np.uint8)      # overflow to zero


def _mut_encode_ignores_sign(x):
    return _orig_encode(np.abs(np.asarray(x, np.float64)))


def _mut_decode_bias0(codes):
    c = np.asarray(codes, np.uint8)
    v = _orig_decode(c)
    return np.where((c & 0x6) != 0, v * 2, v)


def _mut_decode_no_subnormal(codes):
    c = np.asarray(codes, np.uint8)
    v = _orig_decode(c)
    return np.where((c & 0x7) == 1, np.where(c & 0x8, -1.5, 1.5), v)


def _mut_scale_emax1(amax):
    return np.where(np.asarray(amax) > 0, _orig_scale(amax) + 1, 0).astype(np.int32)


def _mut_scale_emax3(amax):
    return np.where(np.asarray(amax) > 0, _orig_scale(amax) - 1, 0).astype(np.int32)


def _mut_pack_high_first(codes):
    codes = np.asarray(codes, np.uint8)
    return ((codes[:, 0::2] << 4) | codes[:, 1::2]).astype(np.uint8)


def _mut_unpack_high_first(packed):
    packed = np.asarray(packed, np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
    out[:, 0::2] = packed >> 4
    out[:, 1::2] = packed & 0xF
    return out


def _mut_quantize_block16(w_bits):
    w_bits = np.asarray(w_bits, np.uint16)
    w = lo.bf16_bits_to_f64(w_bits)
    r, k = w.shape
    blocks = w.reshape(r, k // 16, 16)
    s16 = mx.block_scale_exponent(np.abs(blocks).max(axis=2))
    q = blocks * np.ldexp(1.0, -s16)[:, :, None]
    codes = mx.pack_nibbles(mx.e2m1_encode(q).reshape(r, k))
    return codes, (s16[:, 0::2] + 127).astype(np.uint8)


def _mut_logits_no_scale(h, codes, scales):
    return _orig_logits(h, codes, np.full_like(np.asarray(scales, np.uint8), 127))


def _mut_project_ignores_d2t(h, codes, scales, d2t=None, keep_logits=False):
    return _orig_project(h, codes, scales, None, keep_logits)


def _mut_topk_ascending(h, codes, scales, d2t, k):
    logits = _orig_logits(h, codes, scales)
    return mx.topk_of_logits(-logits, d2t, k)


MUTANTS = {
    "topk_ascending": ("oracle_project_topk_mxfp4", _mut_topk_ascending),
    "encode_ties_up": ("e2m1_encode", _mut_encode_ties_up),
    "encode_truncates": ("e2m1_encode", _mut_encode_truncates),
    "encode_overflow_wraps_to_zero": ("e2m1_encode", _mut_encode_wraps),
    "encode_ignores_sign": ("e2m1_encode", _mut_encode_ignores_sign),
    "decode_bias0": ("e2m1_decode", _mut_decode_bias0),
    "decode_no_subnormal": ("e2m1_decode", _mut_decode_no_subnormal),
    "scale_emax1": ("block_scale_exponent", _mut_scale_emax1),
    "scale_emax3": ("block_scale_exponent", _mut_scale_emax3),
    "pack_high_nibble_first": ("pack_nibbles", _mut_pack_high_first),
    "unpack_high_nibble_first": ("unpack_nibbles", _mut_unpack_high_first),
    "quantize_blocks_of_16": ("oracle_quantize_mxfp4", _mut_quantize_block16),
    "logits_without_scales": ("oracle_logits_mxfp4", _mut_logits_no_scale),
    "project_ignores_d2t": ("oracle_project_argmax_mxfp4", _mut_project_ignores_d2t),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mxfp4_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(mx, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(mx)
        except (AssertionError, IndexError, ValueError, pytest.fail.Exception):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
