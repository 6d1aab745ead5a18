"""The parity rule's arithmetic, checked on the CPU: the f16 slack of the
NVFP4 bound and the premise behind it.

The matrix-core kernel takes an NVFP4 head's products against hidden rows
in f16, each row scaled by 2^(15 - E) (E the exponent of its largest
magnitude).  The premise: every bf16 value within 2^29 of the row's largest
is then exact in f16, and any other value is off by at most its own
magnitude.  numpy's float16 is IEEE binary16 with round-to-nearest-even, so
it checks that premise here for every bf16 magnitude over a wide range of
row maxima.
"""
import numpy as np

import oracle
import synth
from parity import f16_hidden_slack, row_bounds


def _scaled_f16(h):
    """The kernel's f16 copy of hidden rows h (fp64 values of bf16 numbers):
    h * 2^(15 - E) rounded to binary16, then scaled back."""
    a = np.abs(h).max(axis=1, keepdims=True)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    s = np.exp2(15 - e)
    return (h * s).astype(np.float16).astype(np.float64) / s


def test_every_bf16_magnitude_within_two_to_the_29_is_exact():
    # every positive finite bf16 number, both signs
    mags = oracle.bf16_bits_to_f64(np.arange(1, 0x7F80, dtype=np.uint16))
    vals = np.concatenate([mags, -mags])
    for top in (2.0 ** -120, 2.0 ** -20, 1.0, 3.0, 2.0 ** 40, 2.0 ** 127 * 1.5):
        row = np.concatenate([[top], vals[np.abs(vals) <= top]])[None, :]   # largest magnitude: top
        e = np.floor(np.log2(top))
        f16 = _scaled_f16(row)[0]
        inside = np.abs(row[0]) >= 2.0 ** (e - 29)
        sub = ~inside
        assert (sub.sum() > 0) == (e - 29 > -133), top    # bf16 reaches 2^-133
        assert np.array_equal(f16[inside], row[0][inside]), top
        # below: off by at most the value's own magnitude (rounded or flushed)
        assert np.all(np.abs(f16[sub] - row[0][sub]) <= np.abs(row[0][sub])), top


def test_slack_marks_exactly_the_values_below_two_to_the_e_minus_29():
    h = np.array([[1.5, 2.0 ** -29, 2.0 ** -30, -2.0 ** -31, 0.0, 2.0 ** -29 * 1.5],
                  [0.0] * 6,
                  [-3.0, 2.0 ** -28, -2.0 ** -28 * 0.75, 0.0, 1.0, 2.0]])
    s = f16_hidden_slack(h)
    # row 0: E = 0, so values below 2^-29 count; 2^-29 itself and above do not
    assert np.array_equal(s[0], [0.0, 0.0, 2.0 ** -30, 2.0 ** -31, 0.0, 0.0])
    assert np.all(s[1] == 0.0)
    # row 2: E = 1 (largest 3), so values below 2^-28 count
    assert np.array_equal(s[2], [0.0, 0.0, 2.0 ** -28 * 0.75, 0.0, 0.0, 0.0])


def test_slack_bounds_the_f16_copy_error():
    """|sum_k (h_k - f16copy_k) w_k| <= sum_k slack_k |w_k| on rows with a
    wide spread of magnitudes, and the bound with f16_hidden adds exactly
    that term."""
    rng = np.random.default_rng(5)
    k = 512
    h = oracle.bf16_bits_to_f64(synth.bf16_from_f32(
        (rng.standard_normal((6, k)) * np.exp2(rng.integers(-60, 20, size=(6, k)))).astype(np.float32)))
    w = rng.standard_normal((40, k))
    err = np.abs((h - _scaled_f16(h)) @ w.T)
    slack = f16_hidden_slack(h) @ np.abs(w).T
    assert np.all(err <= slack)
    assert np.all(slack > 0)
    hb = synth.bf16_from_f32(h.astype(np.float32))
    plain = row_bounds(hb, None, np.arange(40), lambda rr: w[rr], extra=2)
    with_slack = row_bounds(hb, None, np.arange(40), lambda rr: w[rr], extra=2, f16_hidden=True)
    assert np.allclose(with_slack - plain, slack, rtol=1e-9, atol=0)
