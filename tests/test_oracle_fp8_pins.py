"""Pins for the FP8 (E4M3, one scale per row) part of the fp64 oracle (CPU).

Each pin checks the oracle against something other than itself: the E4M3
definition, torch's float8_e4m3fn conversions (a library routine), a brute
force nearest-value search over the whole code table, correctly rounded
sums, and the bf16 oracle on heads whose dequantized values are exactly
bf16 (power-of-two scales).  ``test_fp8_mutants_are_caught`` plants
plausible mistakes and checks that at least one pin fails for each.
"""
import math

import numpy as np
import pytest
import torch

import oracle.fp8_head as f8
import oracle.lmhead_oracle as lo
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rng(seed):
    return np.random.default_rng(seed)


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_exact(values):
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    return (bits >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_decode_known(m):
    # sign | exponent (4 bits, bias 7) | mantissa (3 bits); subnormals m * 2**-9
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0,
             0xFE: -448.0, 0x81: -(2.0 ** -9), 0x50: 8.0}
    got = m.e4m3_decode(np.array(list(cases), np.uint8))
    assert got.tolist() == list(cases.values())
    assert np.isnan(m.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(m.e4m3_decode(np.array([0x80], np.uint8)))[0]


def pin_decode_all_vs_torch(m):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = m.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def _encode_cases(rng):
    # every bf16 pattern with |x| <= 464, random fp32 over many binades, and
    # the midpoints between neighbouring codes with their fp32 neighbours
    b = np.arange(65536, dtype=np.uint32) << 16
    x = b.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 464)]
    mag = np.exp2(rng.uniform(-13, math.log2(464), 200_000)).astype(np.float32)
    r = mag * rng.choice(np.array([-1, 1], np.float32), mag.size)
    vals = np.array([f8._e4m3_value(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    return np.concatenate([x, r, near, -near]).astype(np.float32)


def pin_encode_vs_torch(m):
    x = _encode_cases(_rng(5))
    assert np.array_equal(m.e4m3_encode(x), _torch_encode(x))


def pin_encode_nearest_bruteforce(m):
    rng = _rng(6)
    x = (rng.standard_normal(5000) * rng.choice([0.003, 0.1, 3, 60, 300], 5000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    codes = m.e4m3_encode(x)
    table = np.array([f8._e4m3_value(c) for c in range(256)])
    finite = np.where(np.isfinite(table))[0]
    for xi, ci in zip(x.astype(np.float64), codes):
        d = np.abs(table[finite] - xi)
        best = finite[d == d.min()]
        assert ci in best or (xi == 0 and ci in (0x00, 0x80))
        if best.size > 1 and xi != 0:       # a tie: the even code wins
            assert ci % 2 == 0


def pin_encode_saturates(m):
    # reading: magnitudes above 448 saturate (torch returns NaN from 465 up)
    x = np.array([448.5, 464, 465, 479.9, 480, 1e6, 3e38, -465, -1e9], np.float32)
    assert m.e4m3_encode(x).tolist() == [0x7E] * 6 + [0x7E, 0xFE, 0xFE]


def _head(rng, r, k, std=0.02):
    return synth.bf16_from_f32((rng.standard_normal((r, k)) * std).astype(np.float32))


def pin_quantize_invariants(m):
    rng = _rng(7)
    w = _head(rng, 300, 96)
    w[5] = 0                                  # an all-zero row
    w[6] = _bf16_exact(np.full(96, -0.5, np.float32))
    codes, scale = m.oracle_quantize_fp8(w)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32 and codes.shape == w.shape
    table = np.array([f8._e4m3_value(c) for c in range(256)])
    assert np.isfinite(table[codes]).all()
    wf = lo.bf16_bits_to_f64(w)
    for r in range(w.shape[0]):
        if not wf[r].any():
            assert scale[r] == 1.0 and np.all(table[codes[r]] == 0)
            continue
        j = int(np.argmax(np.abs(wf[r])))
        assert abs(table[codes[r, j]]) == 448.0          # the largest element maps to +-448
        assert np.all(np.abs(table[codes[r]]) <= 448)
        assert scale[r] > 0 and np.isfinite(scale[r])
        # every code is a nearest value to w / scale, up to the one fp32
        # rounding of the quotient (which can move a value onto a tie)
        q = wf[r] / float(scale[r])
        err = np.abs(table[codes[r]] - q)
        nearest = np.min(np.abs(table[None, :0x7F] - np.abs(q)[:, None]), axis=1)
        assert np.all(err <= nearest + 2 * np.abs(q) * 2.0 ** -24 + 1e-30)
        assert np.all(np.signbit(table[codes[r]]) == np.signbit(wf[r]))
    assert np.all(table[codes[6]] == -448.0)


def pin_quantize_commutes_with_trim(m):
    rng = _rng(8)
    w = _head(rng, 500, 64)
    ids = rng.permutation(500)[:77]
    c_full, s_full = m.oracle_quantize_fp8(w)
    c_trim, s_trim = m.oracle_quantize_fp8(lo.oracle_trim(w, ids))
    assert np.array_equal(c_trim, c_full[ids]) and np.array_equal(s_trim, s_full[ids])


def _pow2_head(rng, r, k):
    """A head whose row maxima are 448 * 2**-j: scale = 2**-j exactly, so the
    dequantized values are exactly bf16 numbers."""
    w = synth.bf16_from_f32((rng.standard_normal((r, k)) * 0.02).astype(np.float32))
    wf = lo.bf16_bits_to_f64(w)
    j = rng.integers(5, 12, size=r)
    for i in range(r):
        col = int(rng.integers(0, k))
        amax = 448.0 * 2.0 ** -int(j[i])
        assert np.abs(wf[i]).max() < amax
        w[i, col] = _bf16_exact([amax * rng.choice([-1, 1])])[0]
    return w


def pin_projection_equals_bf16_oracle(m):
    rng = _rng(9)
    w = _pow2_head(rng, 700, 128)
    codes, scale = m.oracle_quantize_fp8(w)
    assert np.all(np.log2(scale.astype(np.float64)) == np.round(np.log2(scale.astype(np.float64))))
    deq = m.oracle_dequant_fp8(codes, scale)
    w_deq = _bf16_exact(deq.astype(np.float32))          # exact by construction
    h = synth.bf16_from_f32(rng.standard_normal((3, 128)).astype(np.float32))
    d2t = (np.arange(700, dtype=np.int32) * 5 + 3)
    a = m.oracle_project_argmax_fp8(h, codes, scale, d2t, keep_logits=True)
    b = lo.oracle_project_argmax(h, w_deq, d2t, keep_logits=True)
    assert np.array_equal(a.logits, b.logits)
    assert np.array_equal(a.id, b.id) and np.array_equal(a.gap, b.gap)
    assert np.allclose(a.abs_sum, b.abs_sum, rtol=1e-14, atol=0)


def pin_projection_fsum(m):
    rng = _rng(10)
    w = _head(rng, 40, 24)
    codes, scale = m.oracle_quantize_fp8(w)
    h = synth.bf16_from_f32(rng.standard_normal((2, 24)).astype(np.float32))
    hf = lo.bf16_bits_to_f64(h)
    table = np.array([f8._e4m3_value(c) for c in range(256)])
    got = m.oracle_logits_fp8(h, codes, scale)
    for i in range(2):
        for r in range(40):
            exact = math.fsum(hf[i, k] * table[codes[r, k]] * float(scale[r]) for k in range(24))
            assert abs(got[i, r] - exact) <= 1e-13 * max(1.0, abs(exact))


def pin_planted_winner_fp8(m):
    rng = _rng(11)
    w = _head(rng, 900, 64)
    h = synth.bf16_from_f32(rng.standard_normal((1, 64)).astype(np.float32))
    hf = lo.bf16_bits_to_f64(h)[0]
    w[417] = synth.bf16_from_f32((np.sign(hf) * 0.5).astype(np.float32))
    codes, scale = m.oracle_quantize_fp8(w)
    res = m.oracle_project_argmax_fp8(h, codes, scale)
    assert res.idx[0] == 417 and res.id[0] == 417 and res.gap[0] > 0
    d2t = np.arange(900, dtype=np.int32)[::-1].copy()
    assert m.oracle_project_argmax_fp8(h, codes, scale, d2t).id[0] == 900 - 1 - 417


def pin_topk_equals_bf16_oracle(m):
    """Power-of-two row scales make the dequantized head bf16-exact: the top
    k over the FP8 head is the bf16 oracle's top k."""
    rng = _rng(21)
    w = _pow2_head(rng, 500, 128)
    codes, scale = m.oracle_quantize_fp8(w)
    w_deq = _bf16_exact(m.oracle_dequant_fp8(codes, scale).astype(np.float32))
    h = synth.bf16_from_f32(rng.standard_normal((3, 128)).astype(np.float32))
    d2t = (np.arange(500, dtype=np.int32) * 7 + 2)
    for k in (1, 4, 16, 503):
        a = m.oracle_project_topk_fp8(h, codes, scale, d2t, k)
        b = lo.oracle_project_topk(h, w_deq, d2t, k)
        assert np.array_equal(a.id, b.id) and np.array_equal(a.logit, b.logit)
    t = m.oracle_project_topk_fp8(h, codes, scale, d2t, 6)
    a = m.oracle_project_argmax_fp8(h, codes, scale, d2t)
    assert np.array_equal(t.id[:, 0], a.id) and np.array_equal(t.logit[:, 0], a.logit)


PINS = [pin_decode_known, pin_decode_all_vs_torch, pin_encode_vs_torch,
        pin_encode_nearest_bruteforce, pin_encode_saturates, pin_quantize_invariants,
        pin_quantize_commutes_with_trim, pin_projection_equals_bf16_oracle,
        pin_projection_fsum, pin_planted_winner_fp8,
        pin_topk_equals_bf16_oracle]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_fp8_pin(pin):
    pin(f8)


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

_orig_encode = f8.e4m3_encode
_orig_decode = f8.e4m3_decode
_orig_quantize = f8.oracle_quantize_fp8
_orig_logits = f8.oracle_logits_fp8
_orig_project = f8.oracle_project_argmax_fp8


def _mut_encode_half_away(x):
    x = np.asarray(x, np.float32)
    code = _orig_encode(x)
    vals = f8._TABLE
    # where x sits exactly between two codes, take the larger magnitude
    up = np.clip((code & 0x7F).astype(np.int64) + 1, 0, 0x7E)
    mid = (np.abs(vals[code & 0x7F]) + vals[up]) / 2
    tie_down = np.abs(x.astype(np.float64)) == mid
    return np.where(tie_down, (up | (code & 0x80)).astype(np.uint8), code).astype(np.uint8)


def _mut_encode_truncate(x):
    x = np.asarray(x, np.float32)
    a = np.minimum(np.abs(x).astype(np.float64), 448.0)
    code = (np.searchsorted(f8._POS, a, side="right") - 1).clip(0, 0x7E).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def _mut_encode_no_saturation(x):
    x = np.asarray(x, np.float32)
    code = _orig_encode(x)
    big = np.abs(x) > 448
    return np.where(big, code | 0x7F, code).astype(np.uint8)


def _mut_encode_ignore_sign(x):
    return _orig_encode(np.abs(np.asarray(x, np.float32)))


def _mut_decode_bias8(codes):
    v = _orig_decode(codes)
    c = np.asarray(codes, np.uint8)
    return np.where((c & 0x78) != 0, v / 2, v)


def _mut_decode_subnormal_as_normal(codes):
    c = np.asarray(codes, np.uint8)
    v = _orig_decode(c)
    sub = ((c & 0x78) == 0) & ((c & 0x07) != 0)
    s = np.where(c & 0x80, -1.0, 1.0)
    return np.where(sub, s * (1 + (c & 7) / 8.0) * 2.0 ** -7, v)


def _mut_quantize_max240(w_bits):
    w = lo.bf16_bits_to_f64(np.asarray(w_bits, np.uint16)).astype(np.float32)
    amax = np.abs(w).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(240), np.float32(1)).astype(np.float32)
    return f8.e4m3_encode((w / scale[:, None]).astype(np.float32)), scale


def _mut_quantize_amax_by_column(w_bits):
    w = lo.bf16_bits_to_f64(np.asarray(w_bits, np.uint16)).astype(np.float32)
    amax_c = np.abs(w).max(axis=0)
    amax = np.resize(amax_c, w.shape[0])          # transposed: column maxima used as row scales
    scale = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    return f8.e4m3_encode((w / scale[:, None]).astype(np.float32)), scale


def _mut_logits_no_scale(h, codes, scale):
    return _orig_logits(h, codes, np.ones_like(np.asarray(scale, np.float32)))


def _mut_logits_scale_shift(h, codes, scale):
    s = np.asarray(scale, np.float32)
    return _orig_logits(h, codes, np.roll(s, 1))


def _mut_project_ignores_d2t(h, codes, scale, d2t=None, keep_logits=False):
    return _orig_project(h, codes, scale, None, keep_logits)


MUTANTS = {
    "encode_ties_away": ("e4m3_encode", _mut_encode_half_away),
    "encode_truncates": ("e4m3_encode", _mut_encode_truncate),
    "encode_no_saturation": ("e4m3_encode", _mut_encode_no_saturation),
    "encode_ignores_sign": ("e4m3_encode", _mut_encode_ignore_sign),
    "decode_bias8": ("e4m3_decode", _mut_decode_bias8),
    "decode_subnormal_as_normal": ("e4m3_decode", _mut_decode_subnormal_as_normal),
    "quantize_to_240": ("oracle_quantize_fp8", _mut_quantize_max240),
    "quantize_amax_by_column": ("oracle_quantize_fp8", _mut_quantize_amax_by_column),
    "logits_without_scale": ("oracle_logits_fp8", _mut_logits_no_scale),
    "logits_scale_of_other_row": ("oracle_logits_fp8", _mut_logits_scale_shift),
    "project_ignores_d2t": ("oracle_project_argmax_fp8", _mut_project_ignores_d2t),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(f8, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(f8)
        except (AssertionError, IndexError, ValueError, pytest.fail.Exception):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
