"""fp64 CPU oracle for a head stored in MXFP4: 4-bit E2M1 values in blocks of
32 along each row, one power-of-two (E8M0) scale per block.

TEST INFRASTRUCTURE ONLY, like the rest of this package: tests, the smoke
check and the CPU baseline of the benchmark use it; the product path never
imports it, and it shares no code with the HIP library.

The pages requantize the trimmed draft head to a 4-bit format at no measured
acceptance cost, and move drafter candidates onto a 4-bit head
(zone-1.cobraproject.com "Masked MTP drafts", the section of that name and
"Update (November 2026)").  Their format is NVFP4, the 4-bit format of the
GPUs they ran on.  The 4-bit format MI355X converts in hardware is OCP
MXFP4 (Open Compute Project, "OCP Microscaling Formats (MX) v1.0"), so the
head is stored in MXFP4 here.  Readings taken, each listed in the design
notes of the repository:

* Element format E2M1: sign, 2 exponent bits with bias 1, 1 mantissa bit;
  exponent 0 is subnormal (0 or 0.5); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  no infinities or NaN.
* Blocks of 32 consecutive elements of a row share one scale X = 2**s,
  stored as the E8M0 code s + 127.  Following the MX specification's
  conversion, s = floor(log2(amax)) - 2, where amax is the largest magnitude
  in the block and 2 is the exponent of the largest E2M1 normal (6 = 1.5 *
  2**2); s is clamped to [-127, 127].  A block of zeros gets s = 0.
* Element code: the E2M1 value nearest to x / X (an exact power-of-two
  scaling), ties to the even code (mantissa bit 0), magnitudes above 6
  saturating to 6; the sign bit is the input's sign bit.
* Storage: codes [R, K / 2] bytes, element k of a row in byte k // 2, the
  low nibble for even k; scales [R, K / 32] bytes.  K is a multiple of 32.
* The quantized head stands for the values decode(code) * 2**s, and logits
  are taken over exactly those values in fp64 (every product is exact).
"""
from __future__ import annotations

import numpy as np

from .lmhead_oracle import OracleResult, TopkResult, argmax_of_logits, bf16_bits_to_f64, topk_of_logits

__all__ = ["MX_BLOCK", "E2M1_MAX", "e2m1_decode", "e2m1_encode", "oracle_quantize_mxfp4",
           "oracle_dequant_mxfp4", "oracle_logits_mxfp4", "oracle_project_argmax_mxfp4",
           "unpack_nibbles", "pack_nibbles", "oracle_project_topk_mxfp4"]

MX_BLOCK = 32
E2M1_MAX = 6.0
E2M1_EMAX = 2          # exponent of the largest normal value, 6 = 1.5 * 2**2
BLOCK_ROWS = 8192


def _e2m1_value(code: int) -> float:
    """Value of one E2M1 code, from the format definition."""
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * m * 0.5                      # subnormal: 0.m * 2**(1 - 1)
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_TABLE[0x8] = -0.0
_POS = _TABLE[:8].copy()       # non-negative values, ascending with the code


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes (0..15) -> float64, exactly."""
    return _TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """float -> nearest E2M1 code (uint8 0..15), ties to the even code,
    magnitudes above 6 saturating to 6, sign bit from the input's sign."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no code here")
    a = np.minimum(np.abs(x), E2M1_MAX)
    # distance to every non-negative value; the nearest wins, and an exact
    # tie (always between adjacent codes, one even and one odd) goes to the
    # even code
    d = np.abs(a[..., None] - _POS)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1)).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 3)


def block_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """s = clamp(floor(log2(amax)) - 2, -127, 127), and 0 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(amax)                     # amax = mant * 2**ex, mant in [0.5, 1)
    s = (ex - 1) - E2M1_EMAX
    return np.where(amax > 0, np.clip(s, -127, 127), 0).astype(np.int32)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[R, K] codes -> [R, K / 2] bytes, even element in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[R, K / 2] bytes -> [R, K] codes (inverse of pack_nibbles)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def oracle_quantize_mxfp4(w_bits: np.ndarray):
    """(codes uint8 [R, K / 2], scales uint8 [R, K / 32]) of a bf16 head."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 2 or w_bits.shape[1] % MX_BLOCK:
        raise ValueError("W must be [R, K] with K a multiple of 32")
    r, k = w_bits.shape
    nb = k // MX_BLOCK
    codes = np.empty((r, k // 2), dtype=np.uint8)
    scales = np.empty((r, nb), dtype=np.uint8)
    for r0 in range(0, r, 1024):
        w = bf16_bits_to_f64(w_bits[r0:r0 + 1024])
        if not np.all(np.isfinite(w)):
            raise ValueError("non-finite weight value")
        blocks = w.reshape(w.shape[0], nb, MX_BLOCK)
        s = block_scale_exponent(np.abs(blocks).max(axis=2))          # [rows, nb]
        q = blocks * np.ldexp(1.0, -s)[:, :, None]                    # exact
        c = e2m1_encode(q).reshape(w.shape[0], k)
        codes[r0:r0 + w.shape[0]] = pack_nibbles(c)
        scales[r0:r0 + w.shape[0]] = (s + 127).astype(np.uint8)
    return codes, scales


def oracle_dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The head the codes stand for: decode(code) * 2**(scale - 127), fp64."""
    vals = e2m1_decode(unpack_nibbles(codes))
    s = np.asarray(scales, dtype=np.int32) - 127
    if vals.shape[1] != s.shape[1] * MX_BLOCK:
        raise ValueError("codes [R, K / 2] and scales [R, K / 32] disagree")
    return vals * np.repeat(np.ldexp(1.0, s), MX_BLOCK, axis=1)


def oracle_logits_mxfp4(h_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 logits of bf16 hidden rows against the dequantized head."""
    h = bf16_bits_to_f64(np.asarray(h_bits, dtype=np.uint16))
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if h.ndim != 2 or codes.ndim != 2 or h.shape[1] != 2 * codes.shape[1] or scales.shape[0] != codes.shape[0]:
        raise ValueError("h [M, K], codes [R, K / 2], scales [R, K / 32]")
    if not np.all(np.isfinite(h)):
        raise ValueError("non-finite hidden value")
    out = np.empty((h.shape[0], codes.shape[0]), dtype=np.float64)
    for r0 in range(0, codes.shape[0], BLOCK_ROWS):
        wb = oracle_dequant_mxfp4(codes[r0:r0 + BLOCK_ROWS], scales[r0:r0 + BLOCK_ROWS])
        out[:, r0:r0 + wb.shape[0]] = h @ wb.T
    return out


def oracle_project_argmax_mxfp4(h_bits, codes, scales, d2t=None, keep_logits: bool = False) -> OracleResult:
    """Greedy draft over the dequantized head, mapped through d2t (first
    row among equal maxima); abs_sum = sum_k |h[m, k] * Wdeq[idx, k]|."""
    logits = oracle_logits_mxfp4(h_bits, codes, scales)
    ids, idx, best, gap = argmax_of_logits(logits, d2t)
    h = bf16_bits_to_f64(np.asarray(h_bits, dtype=np.uint16))
    w_win = oracle_dequant_mxfp4(np.asarray(codes)[idx], np.asarray(scales)[idx])
    abs_sum = np.abs(h * w_win).sum(axis=1)
    return OracleResult(ids, idx, best, gap, abs_sum, logits if keep_logits else None)


def oracle_project_topk_mxfp4(h_bits, codes, scales, d2t, k: int) -> TopkResult:
    """The k best rows of the dequantized MXFP4 head per hidden row, best
    first, ties to the smaller row, mapped through d2t: the candidates a
    drafter takes from the target's 4-bit head (zone-1.cobraproject.com
    "Masked MTP drafts", "Update (November 2026)")."""
    return topk_of_logits(oracle_logits_mxfp4(h_bits, codes, scales), d2t, k)
