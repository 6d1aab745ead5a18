"""fp64 CPU oracle for a head stored in NVFP4: 4-bit E2M1 values in blocks of
16 along each row, one E4M3 scale per block, and one fp32 scale for the
whole head.

TEST INFRASTRUCTURE ONLY, like the rest of this package: tests, the smoke
check and the CPU baseline of the benchmark use it; the product path never
imports it, and it shares no code with the HIP library.

The pages requantize the trimmed draft head to NVFP4 at no measured
acceptance cost (zone-1.cobraproject.com "Masked MTP drafts", the section of
that name), and score a drafter's candidates through the target's NVFP4 head
(same page, "Update (November 2026)").  They name the format but do not give
its conversion.  NVFP4 is NVIDIA's two-level 4-bit format: E2M1 elements,
an E4M3 scale for every 16 consecutive elements, and an fp32 scale for the
tensor, so that a value stands for e2m1 x e4m3 x fp32.  Readings taken for
the conversion (each listed in the design notes of the repository):

* Tensor scale g (fp32): the head's largest magnitude divided by 2,688 =
  448 x 6 (the largest E4M3 value times the largest E2M1 value), one
  correctly rounded fp32 division; g = 1 for a head of zeros.  The largest
  block then gets a block scale near 448 and its largest element near 6.
* Block scale (E4M3 code, sign bit 0): the E4M3 value nearest to
  fp32(fp32(amax_b / 6) / g), amax_b the block's largest magnitude, ties to
  the even code, values above 448 saturating to 448 (each step a correctly
  rounded fp32 division).
* Element code: the E2M1 value nearest to fp32(x / fp32(decode(block
  scale) x g)), ties to the even code, magnitudes above 6 saturating to 6,
  the sign bit from the input; where decode(block scale) x g is 0 the
  quotient is the signed zero x * 0.
* Storage: codes [R, K / 2] bytes, element k of a row in byte k // 2, the
  low nibble for even k (as for MXFP4); block scales [R, K / 16] bytes,
  row-major; g one float32.  K is a multiple of 16.
* The quantized head stands for decode(code) x decode(block scale) x g, and
  logits are taken over exactly those values in fp64: every product of a
  bf16 hidden value, an E2M1 value, an E4M3 value and an fp32 value needs
  8 + 2 + 4 + 24 significand bits, exact in fp64's 53, and the K-term sums
  carry fp64 rounding only.
"""
from __future__ import annotations

import numpy as np

from .fp8_head import e4m3_decode, e4m3_encode
from .lmhead_oracle import OracleResult, TopkResult, argmax_of_logits, bf16_bits_to_f64, topk_of_logits
from .mxfp4_head import E2M1_MAX, e2m1_decode, e2m1_encode, pack_nibbles, unpack_nibbles

__all__ = ["NV_BLOCK", "NV_TENSOR_DIVISOR", "tensor_scale", "block_scale_code", "head_amax",
           "oracle_quantize_nvfp4", "oracle_quantize_nvfp4_rows",
           "oracle_dequant_nvfp4", "oracle_logits_nvfp4", "oracle_project_argmax_nvfp4",
           "oracle_project_topk_nvfp4"]

NV_BLOCK = 16
E4M3_MAX = 448.0
NV_TENSOR_DIVISOR = np.float32(E4M3_MAX * E2M1_MAX)     # 2,688
BLOCK_ROWS = 8192
QUANT_BLOCK_ROWS = 1024


def tensor_scale(amax) -> np.float32:
    """g = fp32(amax / 2688), or 1 when amax is 0 (the head is all zeros)."""
    a = np.float32(amax)
    if not np.isfinite(a) or a < 0:
        raise ValueError("the head's largest magnitude must be finite and >= 0")
    return np.float32(1.0) if a == 0 else np.float32(a / NV_TENSOR_DIVISOR)


def block_scale_code(amax_b, g) -> np.ndarray:
    """E4M3 code of each block's scale: nearest to fp32(fp32(amax_b / 6) / g)."""
    amax_b = np.asarray(amax_b, dtype=np.float32)
    s = (amax_b / np.float32(E2M1_MAX)).astype(np.float32)
    q = (s / np.float32(g)).astype(np.float32)
    return e4m3_encode(q)


def head_amax(w_bits: np.ndarray) -> np.float32:
    """The head's largest magnitude (a bf16 value, exact in float32)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    amax = np.float32(0.0)
    for r0 in range(0, w_bits.shape[0], QUANT_BLOCK_ROWS):
        w = bf16_bits_to_f64(w_bits[r0:r0 + QUANT_BLOCK_ROWS])
        if not np.all(np.isfinite(w)):
            raise ValueError("non-finite weight value")
        if w.size:
            amax = max(amax, np.float32(np.abs(w).max()))
    return amax


def oracle_quantize_nvfp4(w_bits: np.ndarray):
    """(codes uint8 [R, K / 2], block scales uint8 [R, K / 16], g float32)
    of a bf16 head: g from the whole head, then every row with that g."""
    g = tensor_scale(head_amax(w_bits))
    codes, scales = oracle_quantize_nvfp4_rows(w_bits, g)
    return codes, scales, g


def oracle_quantize_nvfp4_rows(w_bits: np.ndarray, g):
    """(codes, block scales) of the rows of a head whose tensor scale is g
    (rows are independent once g is known)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 2 or w_bits.shape[1] % NV_BLOCK:
        raise ValueError("W must be [R, K] with K a multiple of 16")
    r, k = w_bits.shape
    nb = k // NV_BLOCK
    g = np.float32(g)
    codes = np.empty((r, k // 2), dtype=np.uint8)
    scales = np.empty((r, nb), dtype=np.uint8)
    for r0 in range(0, r, QUANT_BLOCK_ROWS):
        w = bf16_bits_to_f64(w_bits[r0:r0 + QUANT_BLOCK_ROWS]).astype(np.float32)   # exact
        blocks = w.reshape(w.shape[0], nb, NV_BLOCK)
        sc = block_scale_code(np.abs(blocks).max(axis=2), g)                       # [rows, nb]
        denom = (e4m3_decode(sc).astype(np.float32) * g).astype(np.float32)        # fp32 product
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(denom[:, :, None] > 0, blocks / denom[:, :, None], blocks * np.float32(0.0))
        q = q.astype(np.float32)
        codes[r0:r0 + w.shape[0]] = pack_nibbles(e2m1_encode(q).reshape(w.shape[0], k))
        scales[r0:r0 + w.shape[0]] = sc
    return codes, scales


def oracle_dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """The head the codes stand for: decode(code) x decode(block scale) x g,
    in fp64."""
    vals = e2m1_decode(unpack_nibbles(codes))
    sc = e4m3_decode(np.asarray(scales, dtype=np.uint8))
    if vals.shape[1] != sc.shape[1] * NV_BLOCK or vals.shape[0] != sc.shape[0]:
        raise ValueError("codes [R, K / 2] and scales [R, K / 16] disagree")
    if not np.all(np.isfinite(sc)):
        raise ValueError("a block scale code is NaN")
    return vals * np.repeat(sc, NV_BLOCK, axis=1) * float(np.float32(g))


def oracle_logits_nvfp4(h_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """fp64 logits of bf16 hidden rows against the dequantized head."""
    h = bf16_bits_to_f64(np.asarray(h_bits, dtype=np.uint16))
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if h.ndim != 2 or codes.ndim != 2 or h.shape[1] != 2 * codes.shape[1] or scales.shape[0] != codes.shape[0]:
        raise ValueError("h [M, K], codes [R, K / 2], scales [R, K / 16]")
    if not np.all(np.isfinite(h)):
        raise ValueError("non-finite hidden value")
    out = np.empty((h.shape[0], codes.shape[0]), dtype=np.float64)
    for r0 in range(0, codes.shape[0], BLOCK_ROWS):
        wb = oracle_dequant_nvfp4(codes[r0:r0 + BLOCK_ROWS], scales[r0:r0 + BLOCK_ROWS], g)
        out[:, r0:r0 + wb.shape[0]] = h @ wb.T
    return out


def oracle_project_argmax_nvfp4(h_bits, codes, scales, g, d2t=None, keep_logits: bool = False) -> OracleResult:
    """Greedy draft over the dequantized NVFP4 head, mapped through d2t
    (first row among equal maxima); abs_sum = sum_k |h[m, k] * Wdeq[idx, k]|."""
    logits = oracle_logits_nvfp4(h_bits, codes, scales, g)
    ids, idx, best, gap = argmax_of_logits(logits, d2t)
    h = bf16_bits_to_f64(np.asarray(h_bits, dtype=np.uint16))
    w_win = oracle_dequant_nvfp4(np.asarray(codes)[idx], np.asarray(scales)[idx], g)
    abs_sum = np.abs(h * w_win).sum(axis=1)
    return OracleResult(ids, idx, best, gap, abs_sum, logits if keep_logits else None)


def oracle_project_topk_nvfp4(h_bits, codes, scales, g, d2t, k: int) -> TopkResult:
    """The k best rows of the dequantized NVFP4 head per hidden row, best
    first, ties to the smaller row, mapped through d2t: a drafter's
    candidates scored through the target's NVFP4 head (zone-1.cobraproject.com
    "Masked MTP drafts", "Update (November 2026)")."""
    return topk_of_logits(oracle_logits_nvfp4(h_bits, codes, scales, g), d2t, k)
