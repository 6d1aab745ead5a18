"""fp64 CPU oracle for a head stored as FP8 (E4M3) with one scale per row.

TEST INFRASTRUCTURE ONLY, like the rest of this package: tests, the smoke
check and the CPU baseline of the benchmark use it; the product path never
imports it, and it shares no code with the HIP library.

The pages convert weights that are read on every decode step to FP8 E4M3 at
load to halve the bytes read (ai-muninn.com "Qwen3.8-Flash-Next on two DGX
Sparks", "The costs: a 69% smaller KV pool and FP8 GDN weights" and the
kernel notes under "Decode runs at 80-87% of memory bandwidth"), and
requantize a trimmed head to a 4-bit format at no measured acceptance cost
(zone-1.cobraproject.com "Masked MTP drafts", section "Masked MTP drafts").
They do not fix the scaling granularity or the rounding.  Readings taken
here, each listed in the design notes of the repository:

* Format: OCP FP8 E4M3 ("E4M3FN"): sign, 4 exponent bits with bias 7, 3
  mantissa bits; subnormals m * 2**-9; no infinities; S.1111.111 is NaN;
  largest finite value 448.
* One fp32 scale per head row: scale = max_k |W[r, k]| / 448 computed in fp32
  (round to nearest even), or 1 for a row that is all zeros.
* Code of an element: the E4M3 value nearest to the fp32 quotient
  W[r, k] / scale (fp32 division), ties to the even code, magnitudes above
  448 saturating to 448; the sign bit follows the quotient's sign bit.
* The quantized head stands for the values decode(code) * scale.  Logits
  are taken over exactly those values: L[m, r] = sum_k h[m, k] *
  decode(code[r, k]) * scale[r], every product exact in fp64 (bf16 x E4M3 x
  fp32 needs 8 + 4 + 24 significand bits).
"""
from __future__ import annotations

import numpy as np

from .lmhead_oracle import OracleResult, TopkResult, argmax_of_logits, bf16_bits_to_f64, topk_of_logits

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "oracle_quantize_fp8",
           "oracle_dequant_fp8", "oracle_logits_fp8", "oracle_project_argmax_fp8",
           "oracle_project_topk_fp8"]

E4M3_MAX = 448.0
BLOCK_ROWS = 8192
QUANT_BLOCK_ROWS = 256


def _e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9               # subnormal: 0.m * 2**(1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
_TABLE[0x80] = -0.0
# non-negative finite values, ascending with the code: 0x00 .. 0x7E
_POS = _TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64, exactly."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest E4M3 code, ties to the even code, magnitudes above
    448 saturating to 448, sign bit from the input's sign bit."""
    x = np.asarray(x, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN has no code here")
    a = np.minimum(np.abs(x).astype(np.float64), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(_POS[hi] == a, hi, np.where(take_hi, hi, lo)).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def oracle_quantize_fp8(w_bits: np.ndarray):
    """(codes uint8 [R, K], scale float32 [R]) of a bf16 head, row by row
    (in blocks of QUANT_BLOCK_ROWS rows, which bounds the temporaries)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 2:
        raise ValueError("W must be [R, K]")
    codes = np.empty(w_bits.shape, dtype=np.uint8)
    scale = np.empty(w_bits.shape[0], dtype=np.float32)
    for r0 in range(0, w_bits.shape[0], QUANT_BLOCK_ROWS):
        w = bf16_bits_to_f64(w_bits[r0:r0 + QUANT_BLOCK_ROWS]).astype(np.float32)   # exact
        if not np.all(np.isfinite(w)):
            raise ValueError("non-finite weight value")
        amax = np.abs(w).max(axis=1) if w.shape[1] else np.zeros(w.shape[0], np.float32)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = (w / s[:, None]).astype(np.float32)           # fp32 division, nearest even
        codes[r0:r0 + w.shape[0]] = e4m3_encode(q)
        scale[r0:r0 + w.shape[0]] = s
    return codes, scale


def oracle_dequant_fp8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """The head the codes stand for: decode(code[r, k]) * scale[r], fp64."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]


def oracle_logits_fp8(h_bits: np.ndarray, codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp64 logits of bf16 hidden rows against the dequantized head."""
    h = bf16_bits_to_f64(np.asarray(h_bits, dtype=np.uint16))
    codes = np.asarray(codes, dtype=np.uint8)
    scale = np.asarray(scale, dtype=np.float32)
    if h.ndim != 2 or codes.ndim != 2 or h.shape[1] != codes.shape[1] or scale.shape != (codes.shape[0],):
        raise ValueError("h [M, K], codes [R, K], scale [R]")
    if not np.all(np.isfinite(h)):
        raise ValueError("non-finite hidden value")
    out = np.empty((h.shape[0], codes.shape[0]), dtype=np.float64)
    for r0 in range(0, codes.shape[0], BLOCK_ROWS):
        wb = oracle_dequant_fp8(codes[r0:r0 + BLOCK_ROWS], scale[r0:r0 + BLOCK_ROWS])
        if not np.all(np.isfinite(wb)):
            raise ValueError("NaN code or non-finite scale")
        out[:, r0:r0 + wb.shape[0]] = h @ wb.T
    return out


def oracle_project_argmax_fp8(h_bits, codes, scale, d2t=None, keep_logits: bool = False) -> OracleResult:
    """Greedy draft over the dequantized head, mapped through d2t (first
    row among equal maxima); abs_sum = sum_k |h[m, k] * Wdeq[idx, k]|."""
    logits = oracle_logits_fp8(h_bits, codes, scale)
    ids, idx, best, gap = argmax_of_logits(logits, d2t)
    h = bf16_bits_to_f64(np.asarray(h_bits, dtype=np.uint16))
    w_win = oracle_dequant_fp8(np.asarray(codes)[idx], np.asarray(scale)[idx])
    abs_sum = np.abs(h * w_win).sum(axis=1)
    return OracleResult(ids, idx, best, gap, abs_sum, logits if keep_logits else None)


def oracle_project_topk_fp8(h_bits, codes, scale, d2t, k: int) -> TopkResult:
    """The k best rows of the dequantized FP8 head per hidden row, best
    first, ties to the smaller row, mapped through d2t: several draft
    candidates per position taken from a quantized head, as the pages take a
    drafter's candidates from the target's 4-bit head
    (zone-1.cobraproject.com "Masked MTP drafts", "Update (November 2026)")."""
    return topk_of_logits(oracle_logits_fp8(h_bits, codes, scale), d2t, k)
