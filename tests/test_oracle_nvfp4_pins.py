"""Pins for the NVFP4 part of the fp64 oracle (CPU).

Each pin checks the oracle against something other than itself:
- the tensor scale against a correctly rounded fp32 division done in exact
  rational arithmetic;
- block scales and element codes worked by hand at every kind of tie and at
  saturation;
- the block-scale code against torch's own float32 -> E4M3 conversion;
- an error bound any correct quantizer meets;
- exact round trips of heads whose values are representable;
- the bf16 oracle on such heads, and correctly rounded sums over
  hand-dequantized rows;
- the exact scaling of a whole head by a power of two.
``test_nvfp4_mutants_are_caught`` plants plausible mistakes (wrong block
size, wrong divisor, a dropped scale, truncation, ...) and checks that at
least one pin fails for each.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle.lmhead_oracle as lo
import oracle.nvfp4_head as nv
import synth

torch = pytest.importorskip("torch")

# E2M1 values by code, written out from the format (bit 3 sign, 2 exponent
# bits with bias 1, 1 mantissa bit; exponent 0 is 0 or 0.5)
E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def e4m3_by_hand(code: int) -> float:
    """OCP E4M3 value of a code with sign bit 0: exponent bias 7, 3 mantissa
    bits, exponent 0 subnormal (m x 2**-9)."""
    e, m = (code >> 3) & 0xF, code & 0x7
    return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)


def fp32_round(x: Fraction) -> np.float32:
    """The float32 nearest to the rational x, ties to even, found by exact
    comparison with the two float32 neighbours of a float64 guess."""
    guess = np.float32(float(x))
    cands = {guess, np.nextafter(guess, np.float32(np.inf)), np.nextafter(guess, np.float32(-np.inf))}
    best = sorted(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.array(c).view(np.uint32)) & 1))
    return best[0]


def _bf16_exact(values):
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "values must be bf16 numbers"
    return (bits >> 16).astype(np.uint16)


def _representable_head(rng, r, k):
    """A head whose largest magnitude is 2,688 (so g = 1) and whose every
    block holds one element at +-6 x its scale, the others E2M1 x scale:
    the quantizer must give back exactly these codes and scales.  Returns
    (codes packed, scales, W bits)."""
    nb = k // 16
    codes = rng.integers(0, 16, size=(r, k)).astype(np.uint8)
    top = rng.integers(0, 16, size=(r, nb))
    big = rng.choice(np.array([7, 15], np.uint8), size=(r, nb))
    for b in range(nb):
        codes[np.arange(r), b * 16 + top[:, b]] = big[:, b]
    sc = rng.integers(0x08, 0x7E, size=(r, nb)).astype(np.uint8)     # normal E4M3 scales
    sc[0, 0] = 0x7E                                                # 448: the head's amax is 6 x 448
    vals = E2M1[codes] * np.repeat(np.array([[e4m3_by_hand(int(c)) for c in row] for row in sc]), 16, axis=1)
    return nv.pack_nibbles(codes), sc, _bf16_exact(vals)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_tensor_scale_by_hand(m):
    # 2,688 = 448 x 6 gives g = 1 exactly; twice that gives 2; a head of zeros 1
    assert m.tensor_scale(2688.0) == np.float32(1.0)
    assert m.tensor_scale(5376.0) == np.float32(2.0)
    assert m.tensor_scale(0.0) == np.float32(1.0)
    # other maxima: the correctly rounded float32 of amax / 2688
    for amax in (0.0830078125, 1.0, 0.01171875, 3.0e-5, 7.5):
        assert m.tensor_scale(amax) == fp32_round(Fraction(amax) / 2688), amax


def pin_block_scale_by_hand(m):
    # with g = 1 the block scale is the E4M3 value nearest to amax_b / 6:
    # 6 -> 1.0 (0x38); 6.375 -> 1.0625, halfway between 1.0 (0x38) and
    # 1.125 (0x39) -> the even code 0x38; 6.75 -> 1.125 (0x39); 2688 -> 448
    # (0x7E); 3000 -> 500, saturating to 448; 6 x 2**-10 -> 2**-10, halfway
    # between 0 and the smallest subnormal 2**-9 -> the even code 0;
    # 6 x 2**-9 -> 2**-9 (0x01); 6 x 0.875 -> 0.875 (0x36)
    amax = [6.0, 6.375, 6.75, 2688.0, 3000.0, 6 * 2.0 ** -10, 6 * 2.0 ** -9, 6 * 0.875]
    assert m.block_scale_code(np.array(amax, np.float32), np.float32(1)).tolist() == [
        0x38, 0x38, 0x39, 0x7E, 0x7E, 0x00, 0x01, 0x36]
    # with g = 2 every quotient halves: 6 -> 0.5 (0x30)
    assert m.block_scale_code(np.array([6.0], np.float32), np.float32(2)).tolist() == [0x30]


def pin_quantize_rows_by_hand(m):
    # row 0 holds 2,688 (so g = 1); the blocks of row 1:
    #  0: amax 6 -> scale 1.0; 0.25 ties 0 / 0.5 -> 0 (code 0); 0.75 ties
    #     0.5 / 1 -> 1 (code 2); 2.5 ties 2 / 3 -> 2 (code 4); 5 ties 4 / 6 ->
    #     4 (code 6); -3.5 ties 3 / 4 -> -4 (code 0xE); 6 -> code 7
    #  1: amax 6.375 -> scale 1.0 (tie to even); 6.375 saturates to 6 (code 7)
    #  2: amax 6.75 -> scale 1.125; 6.75 / 1.125 = 6 (code 7); 1.6875 / 1.125
    #     = 1.5 (code 3); -0.5625 / 1.125 = -0.5 (code 9)
    #  3: amax 6 x 2**-10 -> scale 0: every element is a signed zero (0 / 8)
    w = np.zeros((2, 64), np.float32)
    w[0, 0] = 2688.0
    w[1, 0:6] = [0.25, 0.75, 2.5, 5.0, -3.5, 6.0]
    w[1, 16] = 6.375
    w[1, 32:35] = [6.75, 1.6875, -0.5625]
    w[1, 48:50] = [6 * 2.0 ** -10, -6 * 2.0 ** -10]
    codes, scales, g = m.oracle_quantize_nvfp4(_bf16_exact(w))
    assert g == np.float32(1.0)
    assert scales[1].tolist() == [0x38, 0x38, 0x39, 0x00]
    assert scales[0].tolist() == [0x7E, 0x00, 0x00, 0x00]
    c = nv.unpack_nibbles(codes)
    assert c[1, 0:6].tolist() == [0x0, 0x2, 0x4, 0x6, 0xE, 0x7]
    assert c[1, 16] == 0x7 and c[1, 32:35].tolist() == [0x7, 0x3, 0x9]
    assert c[1, 48:50].tolist() == [0x0, 0x8]
    assert c[0, 0] == 0x7 and np.all(c[0, 1:] == 0)


def pin_block_scale_matches_torch(m):
    # the block-scale code is the float32 -> E4M3 conversion of
    # fp32(fp32(amax_b / 6) / g), here against torch's float8_e4m3fn cast
    w_bits = synth.normal_bf16(41, 96, 512, 0.02)
    codes, scales, g = m.oracle_quantize_nvfp4(w_bits)
    w = lo.bf16_bits_to_f64(w_bits).astype(np.float32)
    amax_b = np.abs(w.reshape(96, 32, 16)).max(axis=2)
    q = (amax_b / np.float32(6)).astype(np.float32) / np.float32(g)
    ref = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref)


def pin_quantize_error_bound(m):
    # any correct quantizer: the block scale is within E4M3 rounding of
    # amax_b / (6 g), and every element within one E2M1 half-step (at most 1
    # unit, between 4 and 6) of its scaled value, plus the saturation a
    # rounded-down scale allows: |w - deq| <= 0.2 amax_b
    w_bits = synth.normal_bf16(5, 64, 256, 0.02)
    w = lo.bf16_bits_to_f64(w_bits)
    codes, scales, g = m.oracle_quantize_nvfp4(w_bits)
    deq = m.oracle_dequant_nvfp4(codes, scales, g)
    amax_b = np.abs(w).reshape(64, 16, 16).max(axis=2)
    dec = np.array([[e4m3_by_hand(int(c)) for c in row] for row in scales])
    want = amax_b / (6 * float(g))
    assert np.all(np.abs(dec - want) <= want / 16 + 2.0 ** -10)
    assert float(g) == pytest.approx(np.abs(w).max() / 2688, rel=2 ** -23)
    assert np.all(np.abs(w - deq) <= 0.2 * np.repeat(amax_b, 16, axis=1) + 1e-30)
    assert np.all(np.sign(deq) * np.sign(w) >= 0)


def pin_quantize_round_trip(m):
    rng = np.random.default_rng(7)
    packed, scales, w_bits = _representable_head(rng, 40, 128)
    c2, s2, g = m.oracle_quantize_nvfp4(w_bits)
    assert g == np.float32(1.0)
    assert np.array_equal(s2, scales)
    assert np.array_equal(nv.unpack_nibbles(c2), nv.unpack_nibbles(packed))


def pin_power_of_two_scaling(m):
    # scaling the whole head by 2**j (exact in bf16) scales g by 2**j and
    # leaves every code and block scale as it was, so logits scale exactly
    w_bits = synth.normal_bf16(43, 50, 256, 0.02)
    w = lo.bf16_bits_to_f64(w_bits).astype(np.float32)
    h = synth.hidden(44, 0, 2, 256)
    c0, s0, g0 = m.oracle_quantize_nvfp4(w_bits)
    for j in (-3, 5):
        c1, s1, g1 = m.oracle_quantize_nvfp4(synth.bf16_from_f32(w * np.float32(2.0 ** j)))
        assert g1 == np.float32(g0 * np.float32(2.0 ** j))
        assert np.array_equal(c1, c0) and np.array_equal(s1, s0)
        l0 = m.oracle_logits_nvfp4(h, c0, s0, g0)
        l1 = m.oracle_logits_nvfp4(h, c1, s1, g1)
        assert np.array_equal(l1, l0 * 2.0 ** j)


def pin_projection_equals_bf16_oracle(m):
    rng = np.random.default_rng(11)
    packed, scales, w_bits = _representable_head(rng, 300, 256)
    h = synth.hidden(12, 0, 3, 256)
    got = m.oracle_logits_nvfp4(h, packed, scales, np.float32(1))
    want = lo.oracle_logits(h, w_bits)
    assert np.array_equal(got, want)
    ids = rng.permutation(300).astype(np.int32)
    a = m.oracle_project_argmax_nvfp4(h, packed, scales, np.float32(1), ids)
    b = lo.oracle_project_argmax(h, w_bits, ids)
    assert np.array_equal(a.id, b.id) and np.array_equal(a.logit, b.logit)


def pin_projection_fsum(m):
    w_bits = synth.normal_bf16(14, 6, 64, 0.02)
    codes, scales, g = m.oracle_quantize_nvfp4(w_bits)
    h = synth.hidden(15, 0, 2, 64)
    hv = lo.bf16_bits_to_f64(h)
    got = m.oracle_logits_nvfp4(h, codes, scales, g)
    for r in range(6):
        # nibble k of byte k // 2, scale of block k // 16, then the tensor scale
        row = [E2M1[(codes[r, k // 2] >> (4 * (k % 2))) & 0xF] * e4m3_by_hand(int(scales[r, k // 16])) * float(g)
               for k in range(64)]
        for i in range(2):
            want = math.fsum(hv[i, k] * row[k] for k in range(64))
            assert abs(got[i, r] - want) <= 1e-13 * max(1.0, abs(want))


def pin_planted_winner(m):
    k = 128
    w_bits = synth.normal_bf16(21, 500, k, 0.02)
    h = synth.hidden(22, 0, 2, k)
    hv = lo.bf16_bits_to_f64(h)
    w = lo.bf16_bits_to_f64(w_bits).astype(np.float32)
    for i, j in enumerate((77, 420)):
        w[j] = np.float32(0.05) * np.sign(hv[i]).astype(np.float32)
    codes, scales, g = m.oracle_quantize_nvfp4(synth.bf16_from_f32(w))
    ids = (np.arange(500) * 3 + 1).astype(np.int32)
    res = m.oracle_project_argmax_nvfp4(h, codes, scales, g, ids)
    assert res.id.tolist() == [77 * 3 + 1, 420 * 3 + 1]


def pin_topk_equals_bf16_oracle(m):
    rng = np.random.default_rng(31)
    packed, scales, w_bits = _representable_head(rng, 400, 256)
    h = synth.hidden(32, 0, 3, 256)
    ids = rng.permutation(1000)[:400].astype(np.int32)
    for k in (1, 5, 16, 403):
        a = m.oracle_project_topk_nvfp4(h, packed, scales, np.float32(1), ids, k)
        b = lo.oracle_project_topk(h, w_bits, ids, k)
        assert np.array_equal(a.id, b.id) and np.array_equal(a.idx, b.idx)
        assert np.array_equal(a.logit, b.logit)


def pin_topk_order_and_first(m):
    w_bits = synth.normal_bf16(33, 300, 512, 0.02)
    codes, scales, g = m.oracle_quantize_nvfp4(w_bits)
    h = synth.hidden(34, 0, 4, 512)
    ids = (np.arange(300) * 5 + 3).astype(np.int32)
    t = m.oracle_project_topk_nvfp4(h, codes, scales, g, ids, 8)
    a = m.oracle_project_argmax_nvfp4(h, codes, scales, g, ids)
    assert np.array_equal(t.id[:, 0], a.id) and np.array_equal(t.logit[:, 0], a.logit)
    deq = np.empty((300, 512))
    deq[:, 0::2], deq[:, 1::2] = E2M1[codes & 0xF], E2M1[codes >> 4]
    dec = np.array([[e4m3_by_hand(int(c)) for c in row] for row in scales])
    deq *= np.repeat(dec, 16, axis=1) * float(g)
    full = lo.bf16_bits_to_f64(h) @ deq.T
    for i in range(4):
        assert np.all(np.diff(t.logit[i]) <= 0)
        assert np.allclose(t.logit[i], np.sort(full[i])[::-1][:8], rtol=1e-12, atol=1e-15)
        assert np.array_equal(t.id[i], ids[t.idx[i]])


PINS = [pin_tensor_scale_by_hand, pin_block_scale_by_hand, pin_quantize_rows_by_hand,
        pin_block_scale_matches_torch, pin_quantize_error_bound, pin_quantize_round_trip,
        pin_power_of_two_scaling, pin_projection_equals_bf16_oracle, pin_projection_fsum,
        pin_planted_winner, pin_topk_equals_bf16_oracle, pin_topk_order_and_first]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_nvfp4_pin(pin):
    pin(nv)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

_orig_tensor_scale = nv.tensor_scale
_orig_block_scale = nv.block_scale_code
_orig_quantize = nv.oracle_quantize_nvfp4
_orig_dequant = nv.oracle_dequant_nvfp4
_orig_logits = nv.oracle_logits_nvfp4
_orig_project = nv.oracle_project_argmax_nvfp4
_orig_e4m3_encode = nv.e4m3_encode


def _mut_divisor_448(amax):
    a = np.float32(amax)
    return np.float32(1.0) if a == 0 else np.float32(a / np.float32(448))


def _mut_divisor_6(amax):
    a = np.float32(amax)
    return np.float32(1.0) if a == 0 else np.float32(a / np.float32(6))


def _mut_block_scale_without_6(amax_b, g):
    return _orig_e4m3_encode((np.asarray(amax_b, np.float32) / np.float32(g)).astype(np.float32))


def _mut_block_scale_truncates(amax_b, g):
    q = ((np.asarray(amax_b, np.float32) / np.float32(6)).astype(np.float32) / np.float32(g)).astype(np.float32)
    code = _orig_e4m3_encode(q)
    back = nv.e4m3_decode(code)
    return np.where((back > q) & (code > 0), code - 1, code).astype(np.uint8)


def _mut_block_scale_ignores_g(amax_b, g):
    return _orig_block_scale(amax_b, np.float32(1))


def _mut_quantize_blocks_of_32(w_bits):
    saved = nv.NV_BLOCK
    nv.NV_BLOCK = 32
    try:
        codes, scales, g = _orig_quantize(w_bits)
    finally:
        nv.NV_BLOCK = saved
    return codes, np.repeat(scales, 2, axis=1), g


def _mut_dequant_ignores_g(codes, scales, g):
    return _orig_dequant(codes, scales, np.float32(1))


def _mut_dequant_ignores_block_scale(codes, scales, g):
    return _orig_dequant(codes, np.full_like(np.asarray(scales, np.uint8), 0x38), g)


def _mut_dequant_scale_of_next_block(codes, scales, g):
    return _orig_dequant(codes, np.roll(np.asarray(scales, np.uint8), 1, axis=1), g)


def _mut_project_ignores_d2t(h, codes, scales, g, d2t=None, keep_logits=False):
    return _orig_project(h, codes, scales, g, None, keep_logits)


def _mut_topk_ascending(h, codes, scales, g, d2t, k):
    return nv.topk_of_logits(-_orig_logits(h, codes, scales, g), d2t, k)


MUTANTS = {
    "tensor_divisor_448": ("tensor_scale", _mut_divisor_448),
    "tensor_divisor_6": ("tensor_scale", _mut_divisor_6),
    "block_scale_without_6": ("block_scale_code", _mut_block_scale_without_6),
    "block_scale_truncates": ("block_scale_code", _mut_block_scale_truncates),
    "block_scale_ignores_g": ("block_scale_code", _mut_block_scale_ignores_g),
    "quantize_blocks_of_32": ("oracle_quantize_nvfp4", _mut_quantize_blocks_of_32),
    "dequant_ignores_g": ("oracle_dequant_nvfp4", _mut_dequant_ignores_g),
    "dequant_ignores_block_scale": ("oracle_dequant_nvfp4", _mut_dequant_ignores_block_scale),
    "dequant_scale_of_next_block": ("oracle_dequant_nvfp4", _mut_dequant_scale_of_next_block),
    "project_ignores_d2t": ("oracle_project_argmax_nvfp4", _mut_project_ignores_d2t),
    "topk_ascending": ("oracle_project_topk_nvfp4", _mut_topk_ascending),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_nvfp4_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(nv, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(nv)
        except (AssertionError, IndexError, ValueError, pytest.fail.Exception):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
