// lmhead.hip -- draft-head projection kernels for MI355X (gfx950) and the
// C ABI declared in include/lmhead.h.
//
// What runs on the device:
//   gather_rows             load-time shortlist gather, W_trim[i] = W[ids[i]]
//                           ("Two ways to run it", zone-1.cobraproject.com
//                           "Masked MTP drafts": the head is trimmed at load).
//   proj_valu_tiled         M = 1 (and M = 2 for the argmax): a wave walks
//                           tiles of 4 head rows in 1 KiB column stripes;
//                           packed bf16 dot products with fp32 accumulation,
//                           DPP reduction per row; hidden rows in LDS.
//   proj_valu_rows          M = 3..4 by default (M = 2 for top k and logits;
//                           forced: up to 8): one wave per head row, hidden
//                           rows in registers, two rows per step
//                           double-buffered.
//   proj_mfma               M > 4, and every M over an FP8 or MXFP4 head:
//                           coalesced 16-byte loads of 16-row tiles,
//                           transposed through a wave-private LDS stage into
//                           16x16x32 bf16 matrix-core operands; hidden rows
//                           staged in LDS.
//   proj_valu_fp8           FP8 head on the VALU path (forced only).
// Every projection kernel fuses its epilogue: for the argmax each wave keeps
// a running (logit, row) per hidden row as a 64-bit key, a workgroup folds
// its waves through LDS and stores one key per hidden row into its own
// workspace slot (top k keeps sorted key lists the same way; the logits
// epilogue stores every logit instead).
//   finalize_argmax         one workgroup per hidden row folds the slots,
//                           decodes the winner and maps it through d2t
//                           (EAGLE-3 style draft-to-target ids, "Two ways to
//                           run it").
//   finalize_topk           the same for the top-k lists.
//   fill_neg_inf            the -inf fill before logits are scattered to
//                           vocabulary ids.
//   quantize_rows_fp8, quantize_rows_mxfp4, quantize_rows_nvfp4 (with
//   nvfp4_slot_zero, nvfp4_head_amax, nvfp4_set_scale), tile_block_scales
//                           load-time copies of a head in FP8 or MXFP4.
//   overwrite_rows, union_ids
//                           shortlist maintenance (escaped ids into spare
//                           rows; the union of two lists).
// A projection kernel and its fold are ordered by the stream; no atomics,
// fences or memsets are needed, and the workspace needs no initial
// contents.  The argmax is reduced where it is computed instead of
// gathering logits, the change the fair re-run on
// krisbailey.com/articles/shortlist-mtp credits ("Re-running the comparison
// fairly").
//
// The projection is HBM-bound: at M = 1 each head row (5,120 bytes at
// K = 2,560) is used for 2,560 multiply-adds.  The kernels therefore stream
// W exactly once with 16-byte non-temporal loads and keep everything else on
// chip; logits never reach HBM.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "lmhead.h"
#include "lmhead_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// tunables (compile-time)
// ---------------------------------------------------------------------------
#ifndef LMH_VALU_ROWS
#define LMH_VALU_ROWS 2          // head rows per wave per step (VALU path)
#endif
#ifndef LMH_VALU_WG_PER_CU
#define LMH_VALU_WG_PER_CU 1     // cap on resident workgroups per CU (VALU path)
#endif
#ifndef LMH_VALU_TILE_ROWS
#define LMH_VALU_TILE_ROWS 4     // rows per tile of the tiled VALU kernel (M = 1; M = 2 argmax); 0 = row order
#endif
#ifndef LMH_VALU_PREFETCH
#define LMH_VALU_PREFETCH 1      // double-buffer rows in registers (VALU path)
#endif
#ifndef LMH_NT_LOADS
#define LMH_NT_LOADS 1           // non-temporal W loads
#endif
#ifndef LMH_MFMA_LDS_SB
#define LMH_MFMA_LDS_SB 4        // k-steps per batch of the coalesced matrix-core kernel
#endif
#ifndef LMH_MFMA_RING
#define LMH_MFMA_RING 3          // batches in the register ring of the coalesced matrix-core kernel
#endif
// LDS row padding of the matrix-core kernel, in 16-byte chunks.  Measured
// with SQ_LDS_BANK_CONFLICT over row strides and lane offsets on gfx950: a
// 16-byte read serves a half-wave at a time and is conflict-free when the
// half-wave's 32 chunk indices are distinct modulo 32.  The hidden rows are
// read as [column = lane % 16][chunk lane / 16 + 4 k], so a row stride of
// 2 (mod 4) chunks keeps 16 columns x 2 lane groups apart, while a stride of
// 1 (mod 4) makes column c of one group collide with column c + 1 of the
// next (3.6 extra cycles per read).  Those reads matter where the kernel is
// bound by its LDS traffic, the 4-bit heads at more than 16 hidden rows:
// the 2-chunk pad took the MXFP4 head at 24 rows from 74.1 to 69.9 us (the
// bank-conflict count from 12.4M to 2.5M per launch) and NVFP4 1.5-1.8%
// faster.
// The bf16 and FP8 heads are bound by HBM: a conflict-free layout there
// (hidden rows and the bf16 stage at 2, which removed every conflict of the
// bf16 kernel) changed bf16 by under 0.2% and left FP8 0.5-2.5% slower, so
// they keep the 1-chunk pads.  The FP8 stage (8-byte reads) is
// conflict-free at odd strides; the 4-bit stages (4-byte reads) reach the
// floor of such reads, 2 cycles each, at odd strides.
#ifndef LMH_MFMA_HPAD
#define LMH_MFMA_HPAD 1          // hidden rows, bf16 and FP8 heads
#endif
#ifndef LMH_MFMA_HPAD4
#define LMH_MFMA_HPAD4 2         // hidden rows, MXFP4 and NVFP4 heads
#endif
#ifndef LMH_MFMA_SPAD
#define LMH_MFMA_SPAD 1          // stages (A operand)
#endif

#ifndef LMH_WAVE_MAJOR
#define LMH_WAVE_MAJOR 0          // 1: hand out work units wave-major (see first_unit)
#endif
#ifndef LMH_RING_MAX_ROWS
#define LMH_RING_MAX_ROWS 131072  // VALU argmax at 1-2 hidden rows over fewer head rows than this: ring loop
#endif
#ifndef LMH_VALU_WAVES
#define LMH_VALU_WAVES 4          // waves per workgroup (VALU path)
#endif
constexpr int kValuMaxM = 8;
// Load loop of the VALU kernels (template parameter LOOP):
//   kLoopPair    two register buffers; the next batch is issued only if it
//                exists, which makes the compiler's wait counts cover the
//                just-issued batch too (each step drains the loads);
//   kLoopUncond  the same, issuing every batch (past the end through
//                descriptors with no records), so a step waits only for the
//                batch it scores;
//   kLoopRing    a branch-free ring of kRingDepth batches, unrolled so the
//                slots are static: exact waits, one batch always in flight.
// Measured on MI355X (interleaved runs on one machine): on the full 248,320-row
// head the draining loop is best for M = 2..4 and the unconditional one for
// M = 1 (174.6 against 177.7 us); on shortlists of 16k-53k rows the ring
// is 3-16% faster than either (the ramp and tail dominate there).
// Weight formats of the matrix-core kernel (template parameter FMT).
constexpr int kFmtBf16 = 0;  // bf16 head
constexpr int kFmtFp8 = 1;   // E4M3 codes, one fp32 scale per row
constexpr int kFmtMx4 = 2;   // MXFP4: E2M1 codes, one E8M0 scale per 32 elements
constexpr int kFmtNv4 = 3;   // NVFP4: E2M1 codes, one E4M3 scale per 16 elements, one fp32 scale per head
constexpr int kLoopPair = 0;
constexpr int kLoopUncond = 1;
constexpr int kLoopRing = 2;
constexpr int kRingDepth = 2;
constexpr int kValuMaxChunksTimesM = 40;   // register budget: 160 VGPRs of h
#ifndef LMH_VALU_AUTO_MAX_M
#define LMH_VALU_AUTO_MAX_M 4     // largest M the default choice sends to the VALU path
#endif
// Workgroup slots per hidden row in the workspace; grids are clamped to it.
constexpr int kMaxGrid = 1024;
// LDS one workgroup may use on gfx950.
constexpr int kLdsPerWorkgroup = 160 * 1024;
// Largest top-k a matrix-core lane keeps in its own registers; larger k
// keep each column's best 16 over its four lanes.
constexpr int kLaneListMaxTk = 4;
// Largest head (or list) a call takes: row arithmetic stays in int range,
// and every buffer descriptor's byte count fits its 32-bit field -- the
// largest is the id list of an indexed call, 4 bytes per entry, so
// (2^30 - 1) * 4 < 2^32 (at 2^30 entries the count would wrap to 0 and every
// id would read as 0).  The other descriptors span at most a 16-row tile of a
// head row, the hidden block, or one tile's scales.
constexpr int64_t kMaxRows = ((int64_t)1 << 30) - 1;
constexpr uint32_t kBufferWord3 = 0x00020000u;  // gfx9 raw buffer, 32-bit data
constexpr uint32_t kOobOffset = 0x80000000u;    // any offset >= num_records reads 0
// cache-policy operand of buffer loads: bit 1 = nt (streaming).  Every
// projection kernel reads whole row pieces per instruction and streams W
// once, which HBM serves best as non-temporal reads.
constexpr int kPolicyStream = LMH_NT_LOADS ? 2 : 0;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
// Raw buffer descriptor over `bytes` bytes from `base`; offsets at or past
// `bytes` read 0.  Callers keep `bytes` below 2^32 (see kMaxRows).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kBufferWord3);
}

template <int POLICY = kPolicyStream>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, POLICY);
}

// acc += sum of the eight bf16 products of one 16-byte chunk (fp32 adds).
// The pairs are taken with shufflevector from a whole-vector cast: a
// bit_cast of a single vector component (w.y) is read as component 0 by
// this compiler.
__device__ __forceinline__ float dot8(u32x4 w, u32x4 h, float acc) {
  const bf16x8 a = __builtin_bit_cast(bf16x8, w);
  const bf16x8 b = __builtin_bit_cast(bf16x8, h);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1),
                                        __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3),
                                        __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5),
                                        __builtin_shufflevector(b, b, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7),
                                        __builtin_shufflevector(b, b, 6, 7), acc, false);
  return acc;
}

// Eight E4M3 codes (bytes 0..7 of lo:hi) as eight bf16 values, exactly
// (every E4M3 value, subnormals included, is a bf16 number).  The gfx950
// conversion takes two codes from one 16-bit half of a dword; its scale
// operand is 1.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// Eight E2M1 codes (the nibbles of `packed`, element 2i in the low nibble of
// byte i) as eight bf16 values times the power-of-two scale `sc`, by the
// gfx950 conversion: exact, since an E2M1 value times a power of two in bf16
// range is a bf16 number.  Only for power-of-two scales: on MI355X an E4M3
// scale with mantissa bits passed as this operand gave NVFP4 logits up to
// 18% off the exact ones, as if only its exponent were applied.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8_scaled(uint32_t packed, float sc) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 3);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// Eight E2M1 codes times an NVFP4 block scale as eight f16 values, exactly:
// the codes convert at scale 1 to f16, and one packed f16 multiply per two
// takes the block scale `sc` (a decoded E4M3 value, exact in f16).  Every
// product has at most 6 significant bits and lies in [2^-10, 2688] or is
// zero, so it is a normal f16 number.  Two VALU operations per two
// elements, against four for the same products as bf16 (gfx950 has no
// packed bf16 multiply).
__device__ __forceinline__ u32x4 fp4x8_times_scale_to_f16x8(uint32_t packed, _Float16 sc) {
  const f16x2 s2 = f16x2{sc, sc};
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0) * s2;
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1) * s2;
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2) * s2;
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3) * s2;
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// The same with the MXFP4 block scale 2^(e - 127), e the block's E8M0
// code, placed in the exponent field of the scale operand.  The conversion
// reads only that field, as an E8M0 exponent: code 0 stands for 2^-127
// there too (blocks at that scale take part in the projection parity tests
// at full weight), so no case needs the fp32 subnormal 2^-127.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t packed, uint32_t e) {
  return fp4x8_to_bf16x8_scaled(packed, __builtin_bit_cast(float, e << 23));
}

// Value of an OCP E4M3 code (the low byte of `code`) as fp32, exactly, from
// the format: sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
// is subnormal (m x 2^-9).  The NaN code (S.1111.111) is not given a NaN:
// the NVFP4 quantizer never writes it, and a caller's scale array holding
// it gives an unspecified (in-bounds) result.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xFu;
  const uint32_t m = code & 0x7u;
  const uint32_t sign = (code & 0x80u) << 24;
  const float sub = (float)m * 0x1p-9f;  // exact
  const uint32_t normal = sign | ((e + 120u) << 23) | (m << 20);
  return e == 0u ? __builtin_bit_cast(float, sign | __builtin_bit_cast(uint32_t, sub)) : __builtin_bit_cast(float, normal);
}

// E2M1 code (OCP MX FP4: bias 1, 1 mantissa bit, subnormal 0.5) of an
// fp32 value: the magnitude is the number of rounding thresholds it
// passes, the midpoints between neighbouring values 0, 0.5, 1, 1.5, 2, 3, 4,
// 6, strict where the upper neighbour's code is odd (a tie goes to the even
// code) and inclusive where it is even; 6 and above saturate to code 7.
__device__ __forceinline__ uint32_t e2m1_encode(float q) {
  const float a = __builtin_fabsf(q);
  const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return ((__builtin_bit_cast(uint32_t, q) >> 28) & 0x8u) | mag;
}

// E4M3 code of an fp32 value (OCP FP8 E4M3: bias 7, 3 mantissa bits,
// subnormals m * 2^-9, largest finite 448): the nearest value, ties to the
// even code, magnitudes from 448 up saturating to 448; the sign bit is the
// input's.  Written from the format: below 2^-6 the step is 2^-9, so the
// code is the magnitude in units of 2^-9 rounded to nearest even; above,
// the fp32 fraction is rounded to 3 bits and a carry moves the exponent.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __builtin_fabsf(q);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling; 8 lands on 2^-6 = code 0x08
  } else {
    const uint32_t ab = __builtin_bit_cast(uint32_t, a);
    const uint32_t e = (ab >> 23) - 127u + 7u;  // 1 .. 15
    const uint32_t frac = ab & 0x7FFFFFu;
    uint32_t keep = frac >> 20;
    const uint32_t rest = frac & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
    code = (e << 3) + keep;  // keep == 8 carries into the exponent
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// Wave index inside the workgroup, as a value the compiler knows is uniform
// (so row bases and buffer descriptors live in scalar registers).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// First work unit (tile or step) of this wave; a wave then strides by
// gridDim.x * WV units.  Units go out wave-major: the first gridDim.x units
// to wave 0 of every workgroup, the next to wave 1, and so on, so a head
// with fewer units than waves (or a last partial round) still spreads over
// every CU instead of filling the first workgroups.
__device__ __forceinline__ int first_unit(int wave, int wv) {
  return LMH_WAVE_MAJOR ? wave * (int)gridDim.x + (int)blockIdx.x : (int)blockIdx.x * wv + wave;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes; every lane gets the same result, and the order of
// additions is fixed, so a row's logit is the same on every call.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8  -> every lane holds its 16-lane row sum
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a + b) + (c + d);
}

// Running argmax: keep the first row with the largest ordered logit.  A row
// replaces the best one if it is strictly larger, or if nothing ordered has
// been seen yet.  Rows reach a lane in increasing order, so this keeps the
// smallest index among equal logits.
__device__ __forceinline__ void take_best(float s, int r, float& best, int& bidx) {
  const bool better = (bidx < 0) ? (s == s) : (s > best);
  best = better ? s : best;
  bidx = better ? r : bidx;
}

// 64-bit key whose unsigned order is (logit ascending, then row descending):
// the maximum key is the largest logit at its smallest row.  Key 0 is below
// every real key and means "nothing".
__device__ __forceinline__ unsigned long long pack_key(float v, int idx) {
  if (idx < 0) return 0ull;
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  if (v == 0.0f) b = 0u;                                  // -0 == +0
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ void unpack_key(unsigned long long k, float& v, int& idx) {
  const uint32_t ord = (uint32_t)(k >> 32);
  const uint32_t b = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  v = __builtin_bit_cast(float, b);
  idx = (int)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long min_u64(unsigned long long a, unsigned long long b) {
  return a < b ? a : b;
}

// The key of lane ^ X (X = 16 or 32) with gfx950's row-swap instructions,
// on the VALU instead of a shuffle through the LDS crossbar.  Given the same
// value twice, v_permlane16_swap leaves in its first result each odd row
// holding the even row below it, and in its second each even row holding
// the odd row above it; v_permlane32_swap does the same for the two halves
// of the wave.  `row` is the lane's 16-lane row (lane / 16).
template <int X>
__device__ __forceinline__ uint32_t xrow_u32(uint32_t v, int row) {
  static_assert(X == 16 || X == 32, "a lane XOR across 16-lane rows");
  if constexpr (X == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (row & 1) ? p[0] : p[1];
  } else {
    const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (row & 2) ? q[0] : q[1];
  }
}

template <int X>
__device__ __forceinline__ unsigned long long xrow_u64(unsigned long long k, int row) {
  const uint32_t lo = xrow_u32<X>((uint32_t)k, row);
  const uint32_t hi = xrow_u32<X>((uint32_t)(k >> 32), row);
  return ((unsigned long long)hi << 32) | lo;
}

// Four wave sums at once, each with wave_sum's association, so every
// result equals wave_sum of that value bit for bit: lane pairs, then quads,
// with the four values merged into one register by lane bits 0-1 (lane
// 4 i + p of a quad ends up holding value p's quad sum), then the row
// rotations and the row swaps (xor 16, xor 32) that wave_sum's reads of
// lanes 0, 16, 32 and 48 and its (a + b) + (c + d) amount to.  About 21
// instructions for four values against four times 14.
__device__ __forceinline__ void wave_sum4(float x0, float x1, float x2, float x3, float (&out)[4]) {
  const int lane = threadIdx.x & 63;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  // even lanes keep value 0 (or 2) plus its odd neighbour's, odd lanes value 1 (or 3)
  const float p01 = (b0 ? x1 : x0) + dpp<0xB1>(b0 ? x0 : x1);  // quad_perm [1,0,3,2]
  const float p23 = (b0 ? x3 : x2) + dpp<0xB1>(b0 ? x2 : x3);
  float q = (b1 ? p23 : p01) + dpp<0x4E>(b1 ? p01 : p23);     // quad_perm [2,3,0,1]
  q += dpp<0x124>(q);  // row_ror:4
  q += dpp<0x128>(q);  // row_ror:8  -> lane p of every 16-lane row: value p's row sum
  const int row = lane >> 4;
  q += __builtin_bit_cast(float, xrow_u32<16>(__builtin_bit_cast(uint32_t, q), row));
  q += __builtin_bit_cast(float, xrow_u32<32>(__builtin_bit_cast(uint32_t, q), row));
#pragma unroll
  for (int p = 0; p < 4; ++p)
    out[p] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q), p));
}

// The wave sums of N values, four at a time (the last group padded).
template <int N>
__device__ __forceinline__ void wave_sums(const float (&x)[N], float (&out)[N]) {
#pragma unroll
  for (int g = 0; g < N; g += 4) {
    float o[4];
    wave_sum4(x[g], g + 1 < N ? x[g + 1] : 0.0f, g + 2 < N ? x[g + 2] : 0.0f, g + 3 < N ? x[g + 3] : 0.0f, o);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (g + p < N) out[g + p] = o[p];
  }
}

// A lane's running top-TK: keys in descending order, 0 = empty slot.
// push() inserts without branches over the list: position j takes
// max(old[j], min(old[j - 1], x)), which shifts every key below x down one
// place.  Keys are unique (the row is in the low bits), so the list holds
// the TK best rows seen, with the smaller row first among equal logits.
// merge() folds in another sorted list with a bitonic network: the
// element-wise maximum of one list and the other reversed holds the TK
// best of both as a bitonic sequence, which log2(TK) half-cleaner stages
// sort.
template <int TK>
struct KeyList {
  unsigned long long k[TK];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int j = 0; j < TK; ++j) k[j] = 0ull;
  }
  __device__ __forceinline__ void push(unsigned long long x) {
    if (x <= k[TK - 1]) return;  // the common case once the list is full
#pragma unroll
    for (int j = TK - 1; j >= 1; --j) k[j] = max_u64(k[j], min_u64(k[j - 1], x));
    k[0] = max_u64(k[0], x);
  }
  __device__ __forceinline__ void merge(const unsigned long long (&o)[TK]) {
#pragma unroll
    for (int j = 0; j < TK; ++j) k[j] = max_u64(k[j], o[TK - 1 - j]);
#pragma unroll
    for (int st = TK / 2; st >= 1; st >>= 1)
#pragma unroll
      for (int j = 0; j < TK; ++j)
        if ((j & st) == 0) {
          const unsigned long long a = k[j], b = k[j + st];
          k[j] = max_u64(a, b);
          k[j + st] = min_u64(a, b);
        }
  }
  // fold in the list of lane (this lane ^ x)
  template <int X>
  __device__ __forceinline__ void merge_xor(int row) {
    unsigned long long o[TK];
#pragma unroll
    for (int j = 0; j < TK; ++j) o[j] = xrow_u64<X>(k[j], row);
    merge(o);
  }
};

// Top-16 of each hidden row m < M (<= 4) spread over the 16 lanes of DPP
// row m: lane j of the row holds the j-th best (logit, row) pair, an empty
// place (-inf, -1).  The VALU kernels hand a wave its head rows in
// increasing order, so a new row r loses every tie with the rows already
// held: in key order (larger logit, then smaller row) it beats a held pair
// exactly when its logit is larger, and plain fp32 compares decide.
// Inserting: a lane whose pair is below the new one takes the smaller of
// the new pair and the pair one lane up, so pairs below it move down one
// lane; the first lane of a row sees +inf from above (bound_ctrl off keeps
// the old value).  pack_key turns a pair into the 64-bit key.
struct RowTop16 {
  float val;
  int row;
  __device__ __forceinline__ void clear() {
    val = -__builtin_inff();
    row = -1;
  }
  template <int M>
  __device__ __forceinline__ void push(const float (&sum)[M], int r, int rho) {
    const float pv = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0x7F800000, __builtin_bit_cast(int, val), 0x111, 0xF, 0xF, false));
    const int pr = __builtin_amdgcn_update_dpp(-1, row, 0x111, 0xF, 0xF, false);
    float nv = val;
    int nr = row;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (rho == m && sum[m] > val) {  // selects, no branch
        const bool here = sum[m] <= pv;
        nv = here ? sum[m] : pv;
        nr = here ? r : pr;
      }
    }
    val = nv;
    row = nr;
  }
};

// The key of lane j ^ X of this lane's 16-lane row, moved with DPP (a VALU
// operand modifier) instead of a shuffle through the LDS crossbar:
// quad_perm for X = 1 and 2, row_ror:8 for 8 (rotating 16 lanes by 8 is the
// XOR), row_mirror for 15, and for 4 the rotations by 4 and by 12, picked
// by bit 2 of the lane.  j is the lane's index within its row.
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)hi << 32) | lo;
}

template <int X>
__device__ __forceinline__ unsigned long long row_xor_u64(unsigned long long k, int j) {
  static_assert(X == 1 || X == 2 || X == 4 || X == 8 || X == 15, "a lane XOR within a 16-lane row");
  if constexpr (X == 1) {
    return dpp_u64<0xB1>(k);   // quad_perm [1,0,3,2]
  } else if constexpr (X == 2) {
    return dpp_u64<0x4E>(k);   // quad_perm [2,3,0,1]
  } else if constexpr (X == 8) {
    return dpp_u64<0x128>(k);  // row_ror:8
  } else if constexpr (X == 15) {
    return dpp_u64<0x140>(k);  // row_mirror
  } else {
    const unsigned long long by4 = dpp_u64<0x124>(k);   // row_ror:4: from lane j - 4 (mod 16)
    const unsigned long long by12 = dpp_u64<0x12C>(k);  // row_ror:12: from lane j + 4 (mod 16)
    return (j & 4) ? by4 : by12;
  }
}

template <int S>
__device__ __forceinline__ unsigned long long row_half_clean(unsigned long long c, int j) {
  const unsigned long long o = row_xor_u64<S>(c, j);
  return (j & S) == 0 ? max_u64(c, o) : min_u64(c, o);
}

// Best 16 of two lists each laid out over the 16 lanes of a DPP row (lane
// j = element j, descending): the element-wise maximum of a and b mirrored
// is bitonic and holds the best 16, which four half-cleaner stages sort.
// j = lane % 16.  Every lane of the row must take part.
__device__ __forceinline__ unsigned long long row_merge(unsigned long long a, unsigned long long b, int j) {
  unsigned long long c = max_u64(a, row_xor_u64<15>(b, j));
  c = row_half_clean<8>(c, j);
  c = row_half_clean<4>(c, j);
  c = row_half_clean<2>(c, j);
  return row_half_clean<1>(c, j);
}

// Top-16 of one hidden row in the matrix-core output layout: the 4 lanes
// g = 0..3 that hold a column each keep 4 keys, element e = 4 g + v of the
// list in register v of lane g (so lanes differ by 16 g).  Bitonic networks
// compare elements e and e ^ s: within a lane for s = 1, 2 and with the lane
// 16 s / 4 away for s = 4, 8.
template <bool ASC, int SIZE, int S>
__device__ __forceinline__ void col_cx(unsigned long long (&c)[4], int g) {
  // direction of the block of SIZE elements containing e: descending
  // where (e & SIZE) == 0, flipped for an ascending sort
  if constexpr (S >= 4) {
    constexpr int kLaneXor = 16 * (S / 4);
    const bool lower = (g & (S / 4)) == 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const bool desc = (((4 * g + v) & SIZE) == 0) != ASC;
      const unsigned long long o = xrow_u64<kLaneXor>(c[v], g);
      c[v] = (lower == desc) ? max_u64(c[v], o) : min_u64(c[v], o);
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if ((v & S) == 0) {
        const bool desc = (((4 * g + v) & SIZE) == 0) != ASC;
        const unsigned long long a = c[v], b = c[v + S];
        const unsigned long long hi = max_u64(a, b), lo = min_u64(a, b);
        c[v] = desc ? hi : lo;
        c[v + S] = desc ? lo : hi;
      }
  }
}

// the half-cleaner stages S, S / 2, ..., 1 of a block of SIZE elements
template <bool ASC, int SIZE, int S>
__device__ __forceinline__ void col_stages(unsigned long long (&c)[4], int g) {
  col_cx<ASC, SIZE, S>(c, g);
  if constexpr (S > 1) col_stages<ASC, SIZE, S / 2>(c, g);
}

// bitonic sort of the 16 elements, ascending, built up from blocks of SIZE
template <int SIZE>
__device__ __forceinline__ void col_sort_asc(unsigned long long (&c)[4], int g) {
  col_stages<true, SIZE, SIZE / 2>(c, g);
  if constexpr (SIZE < 16) col_sort_asc<SIZE * 2>(c, g);
}

// list (descending) := best 16 of list and the 16 candidates c (any order)
__device__ __forceinline__ void col_merge(unsigned long long (&list)[4], unsigned long long (&c)[4], int g) {
  col_sort_asc<2>(c, g);
  // descending list against ascending candidates: the element-wise maximum
  // is bitonic and holds the best 16; sort it descending
#pragma unroll
  for (int v = 0; v < 4; ++v) list[v] = max_u64(list[v], c[v]);
  col_stages<false, 16, 8>(list, g);
}

// Copies hidden rows 0 .. mp - 1 of h (K bf16 wide, row-major) into LDS
// rows of `stride` 16-byte chunks, writing the first `width` chunks of each
// (zero past K).  Each of the NT threads issues all of its loads of a group
// (up to MAXG) before it stores any, so staging takes one memory
// round trip per group; a plain load-then-store loop waits for every chunk
// in turn.  Buffer loads past a row's end or past the block read 0.
// MAXG bounds the group.  The registers of the largest group count towards
// the kernel's register peak even when a launch never uses it: groups of 16
// raised the matrix-core argmax kernels from 86-97 to 126-136 VGPRs, one
// wave per SIMD less, which cost MXFP4 heads their second workgroup per CU
// at a few hidden rows.  So only kernels whose LDS already holds them to one
// workgroup per CU (two 16-column tiles, more than 16 hidden rows) take 16.

template <int NT, int G>
__device__ __forceinline__ void stage_group(__amdgpu_buffer_rsrc_t hs, int K, int total, int width, int stride,
                                            u32x4* __restrict__ dst, int i0) {
  const int chunks = K >> 3;
  u32x4 v[G];
  int at[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int i = i0 + j * NT;
    const int m = i / width;
    const int c = i - m * width;
    at[j] = i < total ? m * stride + c : -1;
    v[j] = load16<0>(hs, i < total && c < chunks ? (uint32_t)(m * K + c * 8) * 2u : kOobOffset);
  }
#pragma unroll
  for (int j = 0; j < G; ++j)
    if (at[j] >= 0) dst[at[j]] = v[j];
}

template <int NT, int MAXG = 8>
__device__ __forceinline__ void stage_hidden(const uint16_t* __restrict__ h, int K, int mp, int width, int stride,
                                             u32x4* __restrict__ dst) {
  static_assert(MAXG == 8 || MAXG == 16, "groups of up to 8 or 16 loads");
  const int total = mp * width;
  const __amdgpu_buffer_rsrc_t hs = make_rsrc(h, (uint32_t)mp * (uint32_t)K * 2u);
  const int i0 = threadIdx.x;
  // the smallest group that covers the block, so no thread issues loads
  // that all read past it
  if (total <= NT) {
    stage_group<NT, 1>(hs, K, total, width, stride, dst, i0);
  } else if (total <= 2 * NT) {
    stage_group<NT, 2>(hs, K, total, width, stride, dst, i0);
  } else if (total <= 4 * NT) {
    stage_group<NT, 4>(hs, K, total, width, stride, dst, i0);
  } else if (MAXG == 8 || total <= 8 * NT) {
    for (int i = i0; i < total; i += 8 * NT) stage_group<NT, 8>(hs, K, total, width, stride, dst, i);
  } else {
    for (int i = i0; i < total; i += 16 * NT) stage_group<NT, MAXG>(hs, K, total, width, stride, dst, i);
  }
}

// Workgroup epilogue, run by wave 0 only: lane m < mcount publishes this
// workgroup's best key for hidden row m_base + m into its own slot.  Slots
// are laid out [hidden row][workgroup], so the finalize kernel reads each
// hidden row's keys contiguously.  Plain stores: the end of the kernel
// orders them before the finalize kernel on the same stream.
__device__ __forceinline__ void publish_workgroup(unsigned long long key, int lane, int mcount, int m_base,
                                                  unsigned long long* __restrict__ slots) {
  if (lane < mcount) slots[(size_t)(m_base + lane) * kMaxGrid + blockIdx.x] = key;
}

// What a projection kernel does with each (head row, hidden row) logit.
//   TK >= 1, !LOGITS: keep the TK best keys; each workgroup leaves them in
//                     slots[(hidden row * kMaxGrid + workgroup) * TK + j].
//   LOGITS:           write the logit to logits[hidden row * ld + col], col
//                     = d2t[row] (skipped unless 0 <= col < ncols) or row.
//
// Indexed kernels (template flag IDX) also read the head through a row map:
// head row r of the projection is row rowmap[r] of W, which has nw rows; a
// row whose id lies outside [0, nw) is never read and takes no part in the
// result.
//
// Single launch (argmax only): with `state` set, no slots are written:
// every workgroup merges its keys into per-hidden-row keys in `state` and
// takes a ticket; the workgroup with the last ticket maps the winners
// through fold_d2t and writes out_id / out_logit, so no fold kernel
// follows.
struct Epi {
  unsigned long long* slots;
  float* logits;
  const int32_t* d2t;
  int64_t ld;
  int64_t ncols;
  const int32_t* rowmap = nullptr;
  int nw = 0;
  char* state = nullptr;
  const int32_t* fold_d2t = nullptr;
  int32_t* out_id = nullptr;
  float* out_logit = nullptr;
};

// Layout of the single-launch state (all of it zero between launches).
// Workgroup b belongs to merge group b % kMergeGroups; each group has a
// ticket and one key per hidden row, and the final level has the same.
// Tickets sit 128 bytes apart (one L2 line each), so the groups' atomics
// do not queue on one line.
constexpr int kMergeGroups = 16;
constexpr int kStateTicket = 0;                                   // final ticket
constexpr int kStateGroupTickets = 128;                           // + 128 x group
constexpr int kStateGroupKeys = kStateGroupTickets + 128 * kMergeGroups;   // [group][LMH_MAX_M]
constexpr int kStateKeys = kStateGroupKeys + 8 * LMH_MAX_M * kMergeGroups; // [LMH_MAX_M]
constexpr int kStateBytes = kStateKeys + 8 * LMH_MAX_M;
static_assert(kStateBytes <= LMH_STATE_BYTES, "the state fits the size the header promises");

// One level of the merge, run by wave 0: lane m < mcount merges `key` (for
// hidden row m_base + m) into keys[m_base + m] with a 64-bit atomic max at
// agent scope -- atomics of that scope on one location are coherent across
// the chiplets with no L2 write-back, which is what a release fence would
// cost every workgroup.  The wave waits until the memory system has
// acknowledged every one of them, and only then lane 0 takes a ticket (a
// relaxed atomic add, same scope): when a ticket is counted, the maxima of
// its taker are in place.  (An agent-scope release on this target is that
// same wait plus an L2 write-back, and the write-back only matters for
// plain stores; here every write before the ticket is such an atomic.)
// Returns whether this wave took the last of `count` tickets; that wave
// then resets the ticket to 0.
__device__ __forceinline__ bool merge_level(unsigned long long* keys, unsigned int* ticket, unsigned int count,
                                            unsigned long long key, int lane, int mcount, int m_base) {
  if (lane < mcount && key != 0ull)
    (void)__hip_atomic_fetch_max(keys + m_base + lane, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  unsigned int t = 0u;
  if (lane == 0) t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  t = (unsigned int)__builtin_amdgcn_readfirstlane((int)t);
  if (t != count - 1u) return false;
  if (lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The last taker of a level reads the level's keys (agent-scope atomic
// loads: every taker's maxima were acknowledged before its ticket) and puts
// them back to 0 for the next launch on this state.
__device__ __forceinline__ unsigned long long take_level_key(unsigned long long* keys, int lane, int mcount,
                                                             int m_base) {
  if (lane >= mcount) return 0ull;
  unsigned long long* p = keys + m_base + lane;
  const unsigned long long k = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return k;
}

// The single-launch hand-off, run by wave 0 of every workgroup in place of
// publish_workgroup, with no fence.  Two levels, so that no location takes
// more than about grid / 16 atomics: the workgroups of a merge group merge
// into the group's keys; the last of each group merges the group's result
// into the final keys; the last group's last workgroup decodes the final
// keys, maps through d2t and stores the outputs.
__device__ __forceinline__ void merge_and_fold_if_last(const Epi& e, unsigned long long key, int lane, int mcount,
                                                       int m_base) {
  const unsigned int grid = gridDim.x;
  const unsigned int groups = grid < (unsigned)kMergeGroups ? grid : (unsigned)kMergeGroups;
  const unsigned int x = blockIdx.x % (unsigned)kMergeGroups;
  const unsigned int members = (grid - 1u - x) / (unsigned)kMergeGroups + 1u;
  unsigned long long* gkeys = reinterpret_cast<unsigned long long*>(e.state + kStateGroupKeys) + x * LMH_MAX_M;
  unsigned int* gticket = reinterpret_cast<unsigned int*>(e.state + kStateGroupTickets + 128 * x);
  if (!merge_level(gkeys, gticket, members, key, lane, mcount, m_base)) return;
  key = take_level_key(gkeys, lane, mcount, m_base);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(e.state + kStateKeys);
  unsigned int* ticket = reinterpret_cast<unsigned int*>(e.state + kStateTicket);
  if (!merge_level(keys, ticket, groups, key, lane, mcount, m_base)) return;
  key = take_level_key(keys, lane, mcount, m_base);
  if (lane < mcount) {
    const int m = m_base + lane;
    if (key == 0ull) {
      e.out_id[m] = -1;
      e.out_logit[m] = __builtin_nanf("");
    } else {
      float v;
      int idx;
      unpack_key(key, v, idx);
      e.out_id[m] = e.fold_d2t ? e.fold_d2t[idx] : idx;
      e.out_logit[m] = v;
    }
  }
}

// Id of list entry r for an indexed kernel, as a plain (unconditional)
// buffer load; entries past the list (r >= R) read 0, so the caller checks
// r < R where it uses the id.  Nothing may consume the value right after
// the load: the wait would then cover every load in flight.
__device__ __forceinline__ int load_row_id(const int32_t* rowmap, int R, int r) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(rowmap, (uint32_t)R * 4u);
  const uint32_t off = r < R ? (uint32_t)r * 4u : kOobOffset;
  return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0);
}

// List entry r (< R) with id `id` takes part if the id is a row of W.
__device__ __forceinline__ bool row_id_ok(int id, int nw) { return id >= 0 && id < nw; }

__device__ __forceinline__ void store_logit(const Epi& e, int m, int r, float v) {
  int64_t col = r;
  if (e.d2t) {
    col = e.d2t[r];
    if (col < 0 || col >= e.ncols) return;
  }
  e.logits[(int64_t)m * e.ld + col] = v;
}

// Workgroup epilogue for TK > 1, run by every thread after a barrier: the
// sorted per-wave lists of hidden row c are in LDS at lists[(w * ms + c) *
// LS + j], j < LS (LS = 16, or TK for shorter lists).  Each DPP row of the
// workgroup merges the WV lists of one hidden row (row_merge) and
// publishes its TK best keys, sorted, into the workgroup's slot.
template <int TK, int WV, int LS>
__device__ __forceinline__ void publish_rows(const unsigned long long* lists, int ms, int mcount, int m_base,
                                             unsigned long long* __restrict__ slots) {
  const int j = threadIdx.x & 15;
  const int row = threadIdx.x >> 4;
  for (int c0 = 0; c0 < mcount; c0 += (int)(blockDim.x >> 4)) {
    const int col = c0 + row;
    const int cc = col < mcount ? col : 0;  // a row with no hidden row merges row 0 and drops it
    unsigned long long k = j < LS ? lists[cc * LS + j] : 0ull;
#pragma unroll
    for (int w = 1; w < WV; ++w) k = row_merge(k, j < LS ? lists[(w * ms + cc) * LS + j] : 0ull, j);
    if (col < mcount && j < TK) slots[((size_t)(m_base + col) * kMaxGrid + blockIdx.x) * TK + j] = k;
  }
}

// One workgroup per hidden row: fold the `nslots` workgroup keys, decode
// the winner, map it through d2t and write the outputs.
__global__ void __launch_bounds__(256)
finalize_argmax(const unsigned long long* __restrict__ slots, int nslots, int m_base,
                const int32_t* __restrict__ d2t, int32_t* __restrict__ out_id,
                float* __restrict__ out_logit) {
  __shared__ unsigned long long s_wave[4];
  const int m = m_base + blockIdx.x;
  const unsigned long long* row = slots + (size_t)m * kMaxGrid;
  unsigned long long k = 0ull;
  for (int i = threadIdx.x; i < nslots; i += 256) k = row[i] > k ? row[i] : k;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)k, x);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(k >> 32), x);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    k = o > k ? o : k;
  }
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x != 0) return;
  k = s_wave[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) k = s_wave[w] > k ? s_wave[w] : k;
  if (k == 0ull) {
    out_id[m] = -1;
    out_logit[m] = __builtin_nanf("");
    return;
  }
  float v;
  int idx;
  unpack_key(k, v, idx);
  out_id[m] = d2t ? d2t[idx] : idx;
  out_logit[m] = v;
}

// Key output for a slice of a head: the same fold, then the winner's key
// re-packed with its global row row_base + idx (no d2t), so that the maximum
// over the keys of all slices of a head is the whole head's winner with the
// smallest-row tie-break.  An empty key (no ordered logit) stays 0.
__global__ void __launch_bounds__(256)
finalize_keys(const unsigned long long* __restrict__ slots, int nslots, int m_base, int64_t row_base,
              unsigned long long* __restrict__ out_key) {
  __shared__ unsigned long long s_wave[4];
  const int m = m_base + blockIdx.x;
  const unsigned long long* row = slots + (size_t)m * kMaxGrid;
  unsigned long long k = 0ull;
  for (int i = threadIdx.x; i < nslots; i += 256) k = row[i] > k ? row[i] : k;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)k, x);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(k >> 32), x);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    k = o > k ? o : k;
  }
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x != 0) return;
  k = s_wave[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) k = s_wave[w] > k ? s_wave[w] : k;
  if (k != 0ull) {
    const uint32_t idx = 0xFFFFFFFFu - (uint32_t)k;
    k = (k & 0xFFFFFFFF00000000ull) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)(row_base + idx));
  }
  out_key[m] = k;
}

// Top-TK version: one workgroup per hidden row merges the sorted TK-key
// lists of `nslots` (<= kMaxGrid) workgroups (slots laid out [hidden row]
// [workgroup][TK]) and writes the best `topk` rows, mapped through d2t, best
// first.  Each of the 64 DPP rows of the workgroup loads its lists (every
// 64th) at once and folds them (row_merge); a tree through LDS folds the 64
// rows.  Positions with no row (R < topk) get id -1 and logit -inf.
constexpr int kFinalizeTopkThreads = 1024;
constexpr int kFinalizeTopkRows = kFinalizeTopkThreads / 16;
constexpr int kFinalizeTopkPerRow = kMaxGrid / kFinalizeTopkRows;

template <int TK>
__global__ void __launch_bounds__(kFinalizeTopkThreads)
finalize_topk(const unsigned long long* __restrict__ slots, int nslots, int m_base, int topk,
              const int32_t* __restrict__ d2t, int32_t* __restrict__ out_id, float* __restrict__ out_logit) {
  __shared__ unsigned long long s_rows[kFinalizeTopkRows][16];
  const int m = m_base + blockIdx.x;
  const unsigned long long* lists = slots + (size_t)m * kMaxGrid * TK;
  const int j = threadIdx.x & 15;
  const int rr = threadIdx.x >> 4;
  unsigned long long x[kFinalizeTopkPerRow];
#pragma unroll
  for (int u = 0; u < kFinalizeTopkPerRow; ++u) {
    const int i = rr + kFinalizeTopkRows * u;
    x[u] = (i < nslots && j < TK) ? lists[(size_t)i * TK + j] : 0ull;
  }
  unsigned long long k = x[0];
#pragma unroll
  for (int u = 1; u < kFinalizeTopkPerRow; ++u)
    if (kFinalizeTopkRows * u < nslots) k = row_merge(k, x[u], j);  // uniform condition
  s_rows[rr][j] = k;
  __syncthreads();
#pragma unroll
  for (int half = kFinalizeTopkRows / 2; half >= 1; half >>= 1) {
    if (rr < half) {
      k = row_merge(k, s_rows[rr + half][j], j);
      s_rows[rr][j] = k;
    }
    __syncthreads();
  }
  if (rr == 0 && j < topk) {
    float v = -__builtin_inff();
    int idx = -1;
    if (k != 0ull) unpack_key(k, v, idx);
    out_id[(size_t)m * topk + j] = idx < 0 ? -1 : (d2t ? d2t[idx] : idx);
    out_logit[(size_t)m * topk + j] = v;
  }
}

// Fill for scatter-after-matmul: every entry of [M, N] starts at -inf.
__global__ void __launch_bounds__(256) fill_neg_inf(float* __restrict__ out, size_t n) {
  const float ninf = -__builtin_inff();
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) out[i] = ninf;
}

// ---------------------------------------------------------------------------
// gather: W_trim[i, :] = W[ids[i], :]
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
gather_rows(const uint16_t* __restrict__ W, int64_t N, int K, const int32_t* __restrict__ ids,
            int64_t S, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + wave_id();
  const int64_t nwave = (int64_t)gridDim.x * 4;
  const int chunks = K >> 3;
  for (int64_t i = wave; i < S; i += nwave) {
    const int32_t id = ids[i];
    if (id < 0 || (int64_t)id >= N) continue;  // checked on the host too
    const u32x4* src = reinterpret_cast<const u32x4*>(W + (int64_t)id * K);
    u32x4* dst = reinterpret_cast<u32x4*>(out + i * K);
    for (int c = lane; c < chunks; c += 64) {
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + c), dst + c);
    }
  }
}

// In-place refresh of a trimmed head: entry i writes row ids[i] of W into
// row rows[i] of W_trim and ids[i] into d2t[rows[i]].  One wave per entry;
// an entry with a row outside [0, cap) or an id outside [0, N) is skipped,
// and an entry is dropped when a later valid entry names the same row (the
// last one wins), so every row has exactly one writer.  Escaped ids learned
// into spare head rows are the pages' fix for a static trim that misses
// (zone-1.cobraproject.com "Masked MTP drafts", section "Update (November
// 2026)", the Gemma 4 31B case).
__global__ void __launch_bounds__(256)
overwrite_rows(const uint16_t* __restrict__ W, int64_t N, int K, uint16_t* __restrict__ W_trim, int32_t* d2t,
               int64_t cap, const int32_t* __restrict__ rows, const int32_t* __restrict__ ids, int n) {
  const int lane = threadIdx.x & 63;
  const int chunks = K >> 3;
  const int nwaves = gridDim.x * 4;
  for (int i = blockIdx.x * 4 + wave_id(); i < n; i += nwaves) {
    const int32_t r = rows[i];
    const int32_t id = ids[i];
    if (r < 0 || (int64_t)r >= cap || id < 0 || (int64_t)id >= N) continue;
    bool later = false;
    for (int j = i + 1 + lane; j < n; j += 64) {
      const int32_t jd = ids[j];
      later |= rows[j] == r && jd >= 0 && (int64_t)jd < N;
    }
    if (__any(later)) continue;
    const u32x4* src = reinterpret_cast<const u32x4*>(W + (int64_t)id * K);
    u32x4* dst = reinterpret_cast<u32x4*>(W_trim + (int64_t)r * K);
    for (int c = lane; c < chunks; c += 64) dst[c] = src[c];
    if (lane == 0) d2t[r] = id;
  }
}

// Sorted union of two id lists in one workgroup: a bitmap per list in LDS,
// counts of |A|, |B|, |B \ A| and |A u B| from them, then the union's ids in
// ascending order through a block-wide prefix sum of per-thread popcounts
// (the pages merge two lists this way: Two Sparks, "Build the draft
// vocabulary from your own text").  Ids outside [0, N) are ignored.
constexpr int kUnionThreads = 1024;
constexpr int kUnionMaxVocab = 1 << 19;   // two bitmaps of 64 KiB

__global__ void __launch_bounds__(kUnionThreads)
union_ids(const int32_t* __restrict__ a, int na, const int32_t* __restrict__ b, int nb, int N,
          int32_t* __restrict__ out, int32_t* __restrict__ counts) {
  extern __shared__ uint32_t bits[];  // [2][words]
  __shared__ uint32_t s_scan[kUnionThreads];
  __shared__ uint32_t s_cnt[4];
  const int t = threadIdx.x;
  const int words = (N + 31) >> 5;
  uint32_t* ba = bits;
  uint32_t* bb = bits + words;
  for (int w = t; w < 2 * words; w += kUnionThreads) bits[w] = 0u;
  if (t < 4) s_cnt[t] = 0u;
  __syncthreads();
  for (int i = t; i < na; i += kUnionThreads) {
    const int32_t x = a[i];
    if (x >= 0 && x < N) atomicOr(&ba[x >> 5], 1u << (x & 31));
  }
  for (int i = t; i < nb; i += kUnionThreads) {
    const int32_t x = b[i];
    if (x >= 0 && x < N) atomicOr(&bb[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  // each thread owns a contiguous run of words, so its ids come out in order
  const int per = (words + kUnionThreads - 1) / kUnionThreads;
  const int w0 = min(words, t * per), w1 = min(words, w0 + per);
  uint32_t ca = 0, cb = 0, cnew = 0, cu = 0;
  for (int w = w0; w < w1; ++w) {
    ca += __popc(ba[w]);
    cb += __popc(bb[w]);
    cnew += __popc(bb[w] & ~ba[w]);
    cu += __popc(ba[w] | bb[w]);
  }
  atomicAdd(&s_cnt[0], ca);
  atomicAdd(&s_cnt[1], cb);
  atomicAdd(&s_cnt[2], cnew);
  // inclusive scan of cu over the workgroup (Hillis-Steele in LDS)
  s_scan[t] = cu;
  __syncthreads();
  for (int d = 1; d < kUnionThreads; d <<= 1) {
    const uint32_t v = t >= d ? s_scan[t - d] : 0u;
    __syncthreads();
    s_scan[t] += v;
    __syncthreads();
  }
  uint32_t pos = s_scan[t] - cu;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = ba[w] | bb[w];
    while (m) {
      const int bit = __builtin_ctz(m);
      out[pos++] = (w << 5) + bit;
      m &= m - 1u;
    }
  }
  __syncthreads();
  if (t == 0) {
    counts[0] = (int32_t)s_cnt[0];
    counts[1] = (int32_t)s_cnt[1];
    counts[2] = (int32_t)s_cnt[2];
    counts[3] = (int32_t)s_scan[kUnionThreads - 1];
  }
}

// FP8 copy of a bf16 head, one wave per row: scale = fp32(max |W[r, :]| /
// 448) (1 for an all-zero row), code = e4m3_encode(W / scale) with both
// divisions correctly rounded.  The row stays in registers between the two
// passes (K <= 8192: at most 16 chunks of 8 values per lane).
constexpr int kQuantMaxChunksPerLane = 16;

__global__ void __launch_bounds__(256)
quantize_rows_fp8(const uint16_t* __restrict__ W, int R, int K, uint8_t* __restrict__ Wq,
                  float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int chunks = K >> 3;
  const int nwaves = gridDim.x * 4;
  for (int r = blockIdx.x * 4 + wave_id(); r < R; r += nwaves) {
    const u32x4* row = reinterpret_cast<const u32x4*>(W + (size_t)r * K);
    u32x4 v[kQuantMaxChunksPerLane];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kQuantMaxChunksPerLane; ++j) {
      const int c = lane + 64 * j;
      v[j] = c < chunks ? row[c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __builtin_bit_cast(float, v[j][e] << 16);
        const float x1 = __builtin_bit_cast(float, v[j][e] & 0xFFFF0000u);
        amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(x0), __builtin_fabsf(x1)));
      }
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, x));
    const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (lane == 0) scale[r] = sc;
    uint2* out = reinterpret_cast<uint2*>(Wq + (size_t)r * K);
#pragma unroll
    for (int j = 0; j < kQuantMaxChunksPerLane; ++j) {
      const int c = lane + 64 * j;
      if (c < chunks) {
        uint32_t b[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __builtin_bit_cast(float, v[j][e] << 16);
          const float x1 = __builtin_bit_cast(float, v[j][e] & 0xFFFF0000u);
          const uint32_t pair = e4m3_encode(__fdiv_rn(x0, sc)) | (e4m3_encode(__fdiv_rn(x1, sc)) << 8);
          b[e >> 1] |= pair << (16 * (e & 1));
        }
        out[c] = uint2{b[0], b[1]};
      }
    }
  }
}

// Place of the E8M0 scale of row r, block j (elements 32 j .. 32 j + 31) in
// the tiled scale layout: rows in tiles of 16 and blocks in groups of 16
// (one matrix-core batch), each (tile, group) a 256-byte piece of 16 rows x
// 16 bytes, the pieces of a tile in group order and the tiles in row order.
// With nb = ceil(blocks / 16) groups per row the array holds ceil(R / 16) x
// nb x 256 bytes; a tile's part starts at r0 x blocks when blocks % 16 == 0.
// NVFP4 (blocks of 16 elements) uses the same layout with groups of 32
// blocks, again 512 elements per group: GROUP = blocks per group, each
// (tile, group) piece 16 rows x GROUP bytes.
template <int GROUP>
__device__ __forceinline__ size_t tiled_scale_index(int r, int j, int blocks) {
  const int nb = (blocks + GROUP - 1) / GROUP;
  return (((size_t)(r >> 4) * nb + j / GROUP) * 16 + (r & 15)) * GROUP + (j % GROUP);
}
__device__ __forceinline__ size_t mx_scale_index(int r, int j, int blocks) { return tiled_scale_index<16>(r, j, blocks); }
__device__ __forceinline__ size_t nv_scale_index(int r, int j, int blocks) { return tiled_scale_index<32>(r, j, blocks); }

// Row-major block scales [R, blocks] into the tiled scale layout (GROUP 16:
// MXFP4, 32: NVFP4), one byte per thread (a load-time conversion of scales
// written elsewhere).
template <int GROUP>
__global__ void __launch_bounds__(256)
tile_block_scales(const uint8_t* __restrict__ src, int R, int blocks, uint8_t* __restrict__ dst) {
  const int64_t n = (int64_t)R * blocks;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / blocks);
    const int j = (int)(i - (int64_t)r * blocks);
    dst[tiled_scale_index<GROUP>(r, j, blocks)] = src[i];
  }
}

// MXFP4 copy of a bf16 head, one wave per row, one 32-element block per lane
// at a time: the block's scale exponent s = floor(log2 amax) - 2 (2 is the
// exponent of the largest E2M1 value, 6 = 1.5 x 2^2), clamped to the E8M0
// range, 0 for a block of zeros; its elements scaled by 2^-s (exact) and
// encoded to the nearest E2M1 code, ties to the even code, saturating at 6.
// Codes are packed two per byte, element 2i in the low nibble of byte i;
// the block's 16 code bytes are one 16-byte store, its scale code one byte
// at its place in the tiled scale layout (mx_scale_index).
__global__ void __launch_bounds__(256)
quantize_rows_mxfp4(const uint16_t* __restrict__ W, int R, int K, uint8_t* __restrict__ Wq,
                    uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int blocks = K >> 5;
  const int nwaves = gridDim.x * 4;
  for (int r = blockIdx.x * 4 + wave_id(); r < R; r += nwaves) {
    const u32x4* row = reinterpret_cast<const u32x4*>(W + (size_t)r * K);
    for (int blk = lane; blk < blocks; blk += 64) {
      float x[32];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = row[blk * 4 + j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * j + 2 * e] = __builtin_bit_cast(float, v[e] << 16);
          x[8 * j + 2 * e + 1] = __builtin_bit_cast(float, v[e] & 0xFFFF0000u);
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
      int s = 0;
      if (amax > 0.0f) {
        int ex = 0;
        (void)__builtin_frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
        s = min(127, max(-127, ex - 1 - 2));
      }
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 32; ++i) packed[i >> 3] |= e2m1_encode(__builtin_ldexpf(x[i], -s)) << (4 * (i & 7));
      reinterpret_cast<u32x4*>(Wq + (size_t)r * (K >> 1))[blk] = u32x4{packed[0], packed[1], packed[2], packed[3]};
      scales[mx_scale_index(r, blk, blocks)] = (uint8_t)(s + 127);
    }
  }
}

// NVFP4 copy of a bf16 head in three kernels on one stream, with the head's
// scale slot (one fp32, the caller's) as the only state between them:
//   nvfp4_head_amax      the head's largest magnitude, as the bits of a
//                        non-negative fp32 (whose unsigned order is the
//                        value order), atomicMax'ed into the slot after the
//                        slot is zeroed by nvfp4_slot_zero;
//   quantize_rows_nvfp4  per row and 16-element block: block scale and
//                        codes (below), from g = fp32(amax / 2688) (1 for a
//                        head of zeros), which every thread derives from the
//                        slot the same way;
//   nvfp4_set_scale      replaces the slot's amax by g.
constexpr float kNvTensorDivisor = 2688.0f;  // largest E4M3 value 448 x largest E2M1 value 6

__global__ void __launch_bounds__(64) nvfp4_slot_zero(float* __restrict__ slot) {
  if (threadIdx.x == 0) *slot = 0.0f;
}

__device__ __forceinline__ uint32_t abs_bits_max(uint32_t m, const u32x4& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max(v[e] & 0x7FFFu, (v[e] >> 16) & 0x7FFFu));  // |bf16| bits
  return m;
}

// Four independent 16-byte non-temporal loads per thread and step keep
// enough bytes in flight to stream the head (one load at a time read the
// 1.27 GB head at 4.6 TB/s).
__global__ void __launch_bounds__(256)
nvfp4_head_amax(const uint16_t* __restrict__ W, int64_t n16, float* __restrict__ slot) {
  uint32_t m = 0u;
  const u32x4* src = reinterpret_cast<const u32x4*>(W);
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    m = abs_bits_max(abs_bits_max(abs_bits_max(abs_bits_max(m, a), b), c), d);
  }
  for (; i < n16; i += stride) m = abs_bits_max(m, __builtin_nontemporal_load(src + i));
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, x));
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(slot), m << 16);  // as fp32 bits
}

__device__ __forceinline__ float nvfp4_tensor_scale(float amax) {
  return amax > 0.0f ? __fdiv_rn(amax, kNvTensorDivisor) : 1.0f;
}

__global__ void __launch_bounds__(64) nvfp4_set_scale(float* __restrict__ slot) {
  if (threadIdx.x == 0) *slot = nvfp4_tensor_scale(*slot);
}

// One wave per row, one 16-element block per lane at a time: block scale
// code = E4M3 nearest to fp32(fp32(amax_b / 6) / g) (e4m3_encode: ties to
// the even code, saturating at 448), then each element's E2M1 code nearest
// to fp32(x / fp32(decode(code) x g)), a signed zero where that product is
// 0.  Every division is correctly rounded (__fdiv_rn).  The block's 8 code
// bytes are one 8-byte store, its scale one byte at nv_scale_index.
__global__ void __launch_bounds__(256)
quantize_rows_nvfp4(const uint16_t* __restrict__ W, int R, int K, uint8_t* __restrict__ Wq,
                    uint8_t* __restrict__ scales, const float* __restrict__ slot) {
  const int lane = threadIdx.x & 63;
  const int blocks = K >> 4;
  const int nwaves = gridDim.x * 4;
  const float g = nvfp4_tensor_scale(*slot);
  for (int r = blockIdx.x * 4 + wave_id(); r < R; r += nwaves) {
    const u32x4* row = reinterpret_cast<const u32x4*>(W + (size_t)r * K);
    for (int blk = lane; blk < blocks; blk += 64) {
      float x[16];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 v = row[blk * 2 + j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * j + 2 * e] = __builtin_bit_cast(float, v[e] << 16);
          x[8 * j + 2 * e + 1] = __builtin_bit_cast(float, v[e] & 0xFFFF0000u);
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
      const uint32_t code = e4m3_encode(__fdiv_rn(__fdiv_rn(amax, 6.0f), g));
      const float denom = e4m3_to_f32(code) * g;
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float q = denom > 0.0f ? __fdiv_rn(x[i], denom) : __builtin_copysignf(0.0f, x[i]);
        packed[i >> 3] |= e2m1_encode(q) << (4 * (i & 7));
      }
      reinterpret_cast<uint2*>(Wq + (size_t)r * (K >> 1))[blk] = uint2{packed[0], packed[1]};
      scales[nv_scale_index(r, blk, blocks)] = (uint8_t)code;
    }
  }
}

// Epilogue of the VALU kernels, where every row sum is wave-uniform after
// the DPP reduction: the running best row per hidden row (TK == 1), the
// best 16 keys of hidden row rho = lane / 16 over that DPP row (TK > 1,
// M <= 4), or the logit itself stored by lane 0 (LOGITS).
template <int M, int WV, int TK, bool LOGITS>
struct ValuEpilogue {
  static_assert(TK == 1 || LOGITS || (M <= 4 && TK <= 16), "a DPP row holds one hidden row's top 16");
  float best[M];
  int bidx[M];
  RowTop16 top;
  // LOGITS: lane i keeps the logits of the wave's i-th pending row; every
  // 64 rows the wave stores them with M full-wave stores.  One store per
  // row and hidden row from a single lane counted towards the same wait
  // counter as the weight loads, and the loops' waits then covered them
  // (logits at 3 and 4 hidden rows took 11% longer than the argmax).
  float pend[LOGITS ? M : 1];
  int prow;
  int npend;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      best[m] = 0.0f;
      bidx[m] = -1;
    }
    top.clear();
    prow = -1;
    npend = 0;
  }
  __device__ __forceinline__ void flush_logits(int lane, const Epi& e) {
    if (lane < npend) {
#pragma unroll
      for (int m = 0; m < M; ++m) store_logit(e, m, prow, pend[m]);
    }
    npend = 0;
  }
  // head row r (< R) has logit sum[m] against hidden row m
  __device__ __forceinline__ void row(const float (&sum)[M], int r, int lane, const Epi& e) {
    if constexpr (LOGITS) {
      const bool mine = lane == npend;
#pragma unroll
      for (int m = 0; m < M; ++m) pend[m] = mine ? sum[m] : pend[m];
      prow = mine ? r : prow;
      if (++npend == 64) flush_logits(lane, e);
    } else if constexpr (TK == 1) {
#pragma unroll
      for (int m = 0; m < M; ++m) take_best(sum[m], r, best[m], bidx[m]);
    } else {
      top.push<M>(sum, r, lane >> 4);
    }
  }
  // fold the waves of the workgroup and publish its keys
  __device__ __forceinline__ void finish(int lane, int wave, const Epi& e) {
    if constexpr (LOGITS) {
      flush_logits(lane, e);
    } else if constexpr (TK == 1) {
      __shared__ unsigned long long s_key[WV][M];
      if (lane == 0) {
#pragma unroll
        for (int m = 0; m < M; ++m) s_key[wave][m] = pack_key(best[m], bidx[m]);
      }
      __syncthreads();
      if (wave != 0) return;
      unsigned long long key = 0ull;
      if (lane < M) {
#pragma unroll
        for (int w = 0; w < WV; ++w) key = s_key[w][lane] > key ? s_key[w][lane] : key;
      }
      if (e.state)
        merge_and_fold_if_last(e, key, lane, M, 0);
      else
        publish_workgroup(key, lane, M, 0, e.slots);
    } else {
      __shared__ unsigned long long s_list[WV * M * 16];
      const int rho = lane >> 4;
      if (rho < M) s_list[(wave * M + rho) * 16 + (lane & 15)] = pack_key(top.val, top.row);
      __syncthreads();
      publish_rows<TK, WV, 16>(s_list, M, M, 0, e.slots);
    }
  }
};

// ---------------------------------------------------------------------------
// VALU path: one wave per head row, hidden rows in registers
// ---------------------------------------------------------------------------
// Lane `l` owns the 16-byte chunks c = l + 64 j (j < CPL) of every row, so
// one load instruction moves 1 KiB of a row, fully coalesced.  Chunks past
// the row end get an out-of-range buffer offset and read as zero.
//
// IDX: row r is row epi.rowmap[r] of W.  The ids of the rows two steps
// ahead are fetched with a vector load (lane u < U: row u of that step)
// when a step's rows are issued, so they have arrived (loads complete in
// order) by the time their own rows are issued; a row whose id is outside
// [0, nw) reads nothing and is left out.
template <int M, int CPL, int U, int WV, int TK, bool LOGITS, bool IDX = false, int LOOP = kLoopPair>
__global__ void __launch_bounds__(64 * WV)
proj_valu_rows(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int R, int K, Epi epi) {
  static_assert(!IDX || (TK == 1 && !LOGITS && U <= 64), "indexed rows: argmax epilogue");
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int chunks = K >> 3;
  const uint32_t row_bytes = (uint32_t)K * 2u;

  uint32_t voff[CPL];
  u32x4 hf[M][CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    voff[j] = c < chunks ? (uint32_t)c * 16u : kOobOffset;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      hf[m][j] = c < chunks ? *reinterpret_cast<const u32x4*>(h + (size_t)m * K + (size_t)c * 8)
                            : u32x4{0u, 0u, 0u, 0u};
    }
  }

  ValuEpilogue<M, WV, TK, LOGITS> ep;
  ep.init();

  const int step = gridDim.x * WV * U;
  u32x4 wa[U][CPL], wb[U][CPL];

  // IDX: ids of the rows of the next two steps, one per lane u < U.
  int vid1 = -1, vid2 = -1;
  auto fetch_ids = [&](int r0) { return load_row_id(epi.rowmap, R, r0 + (lane < U ? lane : 0)); };

  // `live` gets bit u for each row that takes part.
  auto load_rows = [&](u32x4 (&w)[U][CPL], int& live, int r0) {
    int bits = 0;
    int rid[U];
    if constexpr (IDX) {
#pragma unroll
      for (int u = 0; u < U; ++u) rid[u] = __builtin_amdgcn_readlane(vid1, u);
      vid1 = vid2;
      vid2 = fetch_ids(r0 + 2 * step);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u;
      const bool ok = r < R && (!IDX || row_id_ok(rid[u], epi.nw));
      const int src = IDX ? rid[u] : r;
      bits |= ok ? (1 << u) : 0;
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(W + (size_t)(ok ? src : 0) * (size_t)K, ok ? row_bytes : 0u);
#pragma unroll
      for (int j = 0; j < CPL; ++j) w[u][j] = load16(rs, voff[j]);
    }
    live = bits;
  };
  // one wave_sum per row and hidden row: these independent chains measured
  // 0.4-0.7% faster on the full head at 3 and 4 hidden rows than wave_sums'
  // longer four-value chain
  auto score_rows = [&](const u32x4 (&w)[U][CPL], int live, int r0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sum[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) acc = dot8(w[u][j], hf[m][j], acc);
        sum[m] = wave_sum(acc);
      }
      if (r0 + u < R && (!IDX || ((live >> u) & 1))) ep.row(sum, r0 + u, lane, epi);
    }
  };

  static_assert(LOOP != kLoopUncond, "row-order kernel: pair or ring loop");
  if constexpr (LOOP == kLoopRing) {
    // The wave's steps (U rows each) in order with a ring of D batches, as
    // in proj_valu_tiled: a branch-free steady state unrolled D times, rows
    // past R read through descriptors with no records.  IDX: ring slot S
    // keeps, in lane u < U, the ids of the rows of its next step.
    constexpr int D = kRingDepth;
    const int rw = first_unit(wave, WV) * U;
    const int count = rw < R ? (R - 1 - rw) / step + 1 : 0;
    if (count > 0) {
      u32x4 ring[D][U][CPL];
      int live[D];
      int vid[IDX ? D : 1];
      int ri = rw, ra = rw, rc = rw;
      if constexpr (IDX) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
          vid[q] = fetch_ids(ra);
          ra += step;
        }
      }
      auto issue_at = [&](auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        int bits = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = ri + u;
          bool ok = r < R;
          int src = r;
          if constexpr (IDX) {
            src = __builtin_amdgcn_readlane(vid[S], u);
            ok = ok && row_id_ok(src, epi.nw);
          }
          bits |= ok ? (1 << u) : 0;
          const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + (size_t)(ok ? src : 0) * (size_t)K, ok ? row_bytes : 0u);
#pragma unroll
          for (int j = 0; j < CPL; ++j) ring[S][u][j] = load16(rs, voff[j]);
        }
        live[S] = bits;
        if constexpr (IDX) {
          vid[S] = fetch_ids(ra);
          ra += step;
        }
        ri += step;
      };
      auto consume_at = [&](auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        score_rows(ring[S], live[S], rc);
        rc += step;
      };
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (issue_at(std::integral_constant<int, J>{}), ...);
      }(std::make_integer_sequence<int, D - 1>{});
      int n = 0;
      for (; n + D <= count; n += D) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
          ((issue_at(std::integral_constant<int, (J + D - 1) % D>{}), consume_at(std::integral_constant<int, J>{})),
           ...);
        }(std::make_integer_sequence<int, D>{});
      }
      [&]<int... J>(std::integer_sequence<int, J...>) {
        ((n + J < count ? (issue_at(std::integral_constant<int, (J + D - 1) % D>{}),
                           consume_at(std::integral_constant<int, J>{}), 0)
                        : 0),
         ...);
      }(std::make_integer_sequence<int, D>{});
    }
    ep.finish(lane, wave, epi);
    return;
  }

  int r0 = first_unit(wave, WV) * U;
  int la = 0, lb = 0;
  if constexpr (IDX) {
    vid1 = fetch_ids(r0);
    vid2 = fetch_ids(r0 + step);
  }
  if constexpr (LMH_VALU_PREFETCH) {
    // Two register buffers: the next rows are in flight while these are scored.
    if (r0 < R) load_rows(wa, la, r0);
    while (r0 < R) {
      const int r1 = r0 + step;
      if (r1 < R) load_rows(wb, lb, r1);
      score_rows(wa, la, r0);
      if (r1 >= R) break;
      const int r2 = r1 + step;
      if (r2 < R) load_rows(wa, la, r2);
      score_rows(wb, lb, r1);
      r0 = r2;
    }
  } else {
    for (; r0 < R; r0 += step) {
      load_rows(wa, la, r0);
      score_rows(wa, la, r0);
    }
  }

  ep.finish(lane, wave, epi);
}

// VALU path, tiled order: a wave owns tiles of TR consecutive head rows and
// walks each tile in 1 KiB column stripes (stripe j = chunks 64 j .. 64 j + 63
// of every row of the tile), keeping one fp32 partial sum per (row, hidden
// row) in its lanes.  One batch is TR rows x 1 KiB; the next batch is in
// flight while this one is scored.  Hidden rows live in LDS, zero-padded to
// whole stripes, so the batch loop is a plain runtime loop.  The epilogue
// (argmax, top-TK or every logit) is chosen by TK and LOGITS.  Rows read in
// place through a list take the row-order kernel.
template <int M, int TR, int WV, int TK, bool LOGITS, int LOOP = kLoopPair>
__global__ void __launch_bounds__(64 * WV)
proj_valu_tiled(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int R, int K, Epi epi) {
  extern __shared__ u32x4 h_stripes[];  // [M][nb * 64] chunks, zero past K
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int chunks = K >> 3;
  const int nb = (chunks + 63) >> 6;  // stripes per row
  const int hc = nb * 64;
  const uint32_t row_bytes = (uint32_t)K * 2u;

  // The hidden rows go to LDS once the wave's first weight batch is in
  // flight (stage_and_sync below), so the two memory latencies at the start
  // overlap instead of adding up (except in the draining loop, below).
  auto stage_and_sync = [&]() __attribute__((always_inline)) {
    stage_hidden<64 * WV>(h, K, M, hc, hc, h_stripes);
    __syncthreads();
  };

  ValuEpilogue<M, WV, TK, LOGITS> ep;
  ep.init();
  float acc[TR][M];
#pragma unroll
  for (int q = 0; q < TR; ++q)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[q][m] = 0.0f;

  const int ntiles = (R + TR - 1) / TR;
  const int tstride = gridDim.x * WV;

  // One descriptor per tile covering its live rows: offsets of rows past R
  // (and of chunks past K) are >= num_records and read as zero.
  auto issue = [&](u32x4 (&w)[TR], int tile, int j) {
    const int c = lane + 64 * j;
    const int r0 = tile * TR;
    const uint32_t off = c < chunks ? (uint32_t)c * 16u : kOobOffset;
    // past the last tile (unconditional issue) the descriptor has no records
    constexpr bool kUncond = LOOP == kLoopUncond;
    const int nlive = kUncond ? __builtin_amdgcn_readfirstlane(max(0, min(TR, R - r0))) : min(TR, R - r0);
    const int rbase = kUncond ? __builtin_amdgcn_readfirstlane(nlive == 0 ? 0 : r0) : r0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + (size_t)rbase * (size_t)K, (uint32_t)nlive * row_bytes);
#pragma unroll
    for (int q = 0; q < TR; ++q) w[q] = load16(rs, off + (uint32_t)q * row_bytes);
  };
  auto consume = [&](const u32x4 (&w)[TR], int tile, int j) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const u32x4 hv = h_stripes[m * hc + j * 64 + lane];
#pragma unroll
      for (int q = 0; q < TR; ++q) acc[q][m] = dot8(w[q], hv, acc[q][m]);
    }
    if (j == nb - 1) {
      const int r0 = tile * TR;
      // the tile's TR x M sums: one row at a time at M = 1 (four
      // interleaved chains; one chain of four values measured 0.35% slower
      // on the full head), else four at a time (the same bits; at M = 2 the
      // full head 183.8 -> 180.2 us and the 32,768-row list 27.1 -> 26.8)
      float part[TR * M], tot[TR * M];
#pragma unroll
      for (int q = 0; q < TR; ++q)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          part[q * M + m] = acc[q][m];
          acc[q][m] = 0.0f;
        }
      if constexpr (M == 1) {
#pragma unroll
        for (int q = 0; q < TR; ++q) tot[q] = wave_sum(part[q]);
      } else {
        wave_sums<TR * M>(part, tot);
      }
#pragma unroll
      for (int q = 0; q < TR; ++q) {
        float sum[M];
#pragma unroll
        for (int m = 0; m < M; ++m) sum[m] = tot[q * M + m];
        if (r0 + q < R) ep.row(sum, r0 + q, lane, epi);
      }
    }
  };
  auto advance = [&](int& tile, int& j) {
    if (++j == nb) {
      j = 0;
      tile += tstride;
    }
  };

  if constexpr (LOOP == kLoopRing) {
    // The wave's (tile, stripe) positions in order, with a ring of D
    // batches: D - 1 are in flight while one is scored.  The steady state is
    // unrolled D times so ring slots are static and every slot issues and
    // consumes without conditions; positions past the wave's last one read
    // through descriptors with no records (nothing is fetched).
    constexpr int D = kRingDepth;
    const int tile0 = first_unit(wave, WV);
    const int my_tiles = tile0 < ntiles ? (ntiles - 1 - tile0) / tstride + 1 : 0;
    const int count = my_tiles * nb;
    {
      u32x4 ring[D][TR];
      int ti = tile0, ji = 0;  // next position to issue
      int tc = tile0, jc = 0;  // next position to consume
      auto issue_at = [&](auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        const int c = lane + 64 * ji;
        const uint32_t off = c < chunks ? (uint32_t)c * 16u : kOobOffset;
        const int r0 = ti * TR;
        const int nlive = __builtin_amdgcn_readfirstlane(max(0, min(TR, R - r0)));
        const int rbase = __builtin_amdgcn_readfirstlane(nlive > 0 ? r0 : 0);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + (size_t)rbase * (size_t)K, (uint32_t)nlive * row_bytes);
#pragma unroll
        for (int q = 0; q < TR; ++q) ring[S][q] = load16(rs, off + (uint32_t)q * row_bytes);
        advance(ti, ji);
      };
      auto consume_at = [&](auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        consume(ring[S], tc, jc);
        advance(tc, jc);
      };
      if (count > 0) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
          (issue_at(std::integral_constant<int, J>{}), ...);
        }(std::make_integer_sequence<int, D - 1>{});
      }
      stage_and_sync();
      int n = 0;
      for (; n + D <= count; n += D) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
          ((issue_at(std::integral_constant<int, (J + D - 1) % D>{}), consume_at(std::integral_constant<int, J>{})),
           ...);
        }(std::make_integer_sequence<int, D>{});
      }
      [&]<int... J>(std::integer_sequence<int, J...>) {
        ((n + J < count ? (issue_at(std::integral_constant<int, (J + D - 1) % D>{}),
                           consume_at(std::integral_constant<int, J>{}), 0)
                        : 0),
         ...);
      }(std::make_integer_sequence<int, D>{});
    }
    ep.finish(lane, wave, epi);
    return;
  }

  int tile = first_unit(wave, WV);
  int j = 0;
  u32x4 wa[TR], wb[TR];
  // the draining loop (top k and logits at M = 1) stages first: staged
  // after its first issue, the logits calls measured 6% slower (188 against
  // 177 us on the full head), top k unchanged
  if constexpr (LOOP == kLoopPair) stage_and_sync();
  if (tile < ntiles) issue(wa, tile, 0);
  if constexpr (LOOP != kLoopPair) stage_and_sync();
  if (tile < ntiles) {
    while (true) {
      int t1 = tile, j1 = j;
      advance(t1, j1);
      bool more = t1 < ntiles;
      if (LOOP == kLoopUncond || more) issue(wb, t1, j1);
      consume(wa, tile, j);
      if (!more) break;
      tile = t1;
      j = j1;
      advance(t1, j1);
      more = t1 < ntiles;
      if (LOOP == kLoopUncond || more) issue(wa, t1, j1);
      consume(wb, tile, j);
      if (!more) break;
      tile = t1;
      j = j1;
    }
  }

  ep.finish(lane, wave, epi);
}

// VALU path over an FP8 head (E4M3 codes, one fp32 scale per row), tiled
// like proj_valu_tiled: a wave owns tiles of TR consecutive head rows and
// walks them in 1 KiB column stripes, now 1,024 codes per stripe, so lane l
// takes codes 16 l .. 16 l + 15 and the hidden rows' matching 32 bytes from
// LDS.  Codes become bf16 in registers (exact) and meet the hidden rows in
// packed bf16 dot products with fp32 accumulation; a row's sum is then
// multiplied by its scale.  The tile's scales are read with scalar loads one
// tile ahead (the wave's next tile), so they never wait on the W stream.
template <int M, int TR, int WV, int TK, bool LOGITS>
__global__ void __launch_bounds__(64 * WV)
proj_valu_fp8(const uint16_t* __restrict__ h, const uint8_t* __restrict__ W, const float* __restrict__ wscale,
              int R, int K, Epi epi) {
  extern __shared__ u32x4 h_stripes[];  // [M][nb * 128] chunks of 8 bf16, zero past K
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wchunks = K >> 4;
  const int nb = (wchunks + 63) >> 6;  // stripes per row
  const int hc = nb * 128;
  const uint32_t row_bytes = (uint32_t)K;

  stage_hidden<64 * WV>(h, K, M, hc, hc, h_stripes);
  __syncthreads();

  ValuEpilogue<M, WV, TK, LOGITS> ep;
  ep.init();
  float acc[TR][M];
#pragma unroll
  for (int q = 0; q < TR; ++q)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[q][m] = 0.0f;

  const int ntiles = (R + TR - 1) / TR;
  const int tstride = gridDim.x * WV;
  float sc[TR];
  auto load_scales = [&](int tile) {
    const int r0 = tile * TR;
#pragma unroll
    for (int q = 0; q < TR; ++q) sc[q] = wscale[min(r0 + q, R - 1)];
  };

  auto issue = [&](u32x4 (&w)[TR], int tile, int j) {
    const int c = lane + 64 * j;
    const int r0 = tile * TR;
    const int live = min(TR, R - r0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + (size_t)r0 * (size_t)K, (uint32_t)live * row_bytes);
    const uint32_t off = c < wchunks ? (uint32_t)c * 16u : kOobOffset;
#pragma unroll
    for (int q = 0; q < TR; ++q) w[q] = load16(rs, off + (uint32_t)q * row_bytes);
  };
  auto consume = [&](const u32x4 (&w)[TR], int tile, int j) {
    u32x4 lo[TR], hi[TR];
#pragma unroll
    for (int q = 0; q < TR; ++q) {
      lo[q] = fp8x8_to_bf16x8(w[q].x, w[q].y);
      hi[q] = fp8x8_to_bf16x8(w[q].z, w[q].w);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const u32x4 h0 = h_stripes[m * hc + j * 128 + 2 * lane];
      const u32x4 h1 = h_stripes[m * hc + j * 128 + 2 * lane + 1];
#pragma unroll
      for (int q = 0; q < TR; ++q) acc[q][m] = dot8(hi[q], h1, dot8(lo[q], h0, acc[q][m]));
    }
    if (j == nb - 1) {
      const int r0 = tile * TR;
#pragma unroll
      for (int q = 0; q < TR; ++q) {
        float sum[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          sum[m] = wave_sum(acc[q][m]) * sc[q];
          acc[q][m] = 0.0f;
        }
        if (r0 + q < R) ep.row(sum, r0 + q, lane, epi);
      }
      load_scales(tile + tstride);  // the next tile this wave finishes
    }
  };
  auto advance = [&](int& tile, int& j) {
    if (++j == nb) {
      j = 0;
      tile += tstride;
    }
  };

  int tile = first_unit(wave, WV);
  int j = 0;
  u32x4 wa[TR], wb[TR];
  if (tile < ntiles) {
    load_scales(tile);
    issue(wa, tile, 0);
    while (true) {
      int t1 = tile, j1 = j;
      advance(t1, j1);
      bool more = t1 < ntiles;
      if (more) issue(wb, t1, j1);
      consume(wa, tile, j);
      if (!more) break;
      tile = t1;
      j = j1;
      advance(t1, j1);
      more = t1 < ntiles;
      if (more) issue(wa, t1, j1);
      consume(wb, tile, j);
      if (!more) break;
      tile = t1;
      j = j1;
    }
  }

  ep.finish(lane, wave, epi);
}

// ---------------------------------------------------------------------------
// matrix-core path
// ---------------------------------------------------------------------------
// NVFP4 heads take the f16 matrix instruction (see
// fp4x8_times_scale_to_f16x8), so their hidden rows go to LDS as f16.
// Hidden row m is stored as h * 2^n with n = 15 - E, E the exponent of the
// row's largest magnitude, which then lies in [2^15, 2^16); n goes to the
// row's first pad chunk (past `width`, never read as an operand).  A value
// within 2^29 of the largest becomes a normal f16 number with at most 8
// significant bits: exact.  Smaller ones are rounded to f16's subnormal
// step or flushed, an error of at most their own magnitude.  Since 2^n is
// exact, the row's sums times 2^-n are what bf16 operands would give.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  const int row = (int)(threadIdx.x & 63) >> 4;
  v = max(v, xrow_u32<16>(v, row));
  return max(v, xrow_u32<32>(v, row));
}

// n of a row from the wave's per-lane maxima of its |bf16| bits: frexp
// gives e with amax = f * 2^e, f in [0.5, 1), so E = e - 1 and n = 16 - e
// (a zero row gives e = 0 and n = 16, which scales nothing).
__device__ __forceinline__ int f16_row_shift(uint32_t lane_max) {
  return 16 - __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, wave_max_u32(lane_max) << 16));
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8_shifted(const u32x4& v, int n) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __builtin_ldexpf(__builtin_bit_cast(float, v[e] << 16), n);
    const float hi = __builtin_ldexpf(__builtin_bit_cast(float, v[e] & 0xFFFF0000u), n);
    o[e] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)lo, (_Float16)hi});
  }
  return o;
}

// Stages hidden rows [0, mp) of h ([mp, K] bf16) into LDS rows of `stride`
// chunks as above: `width` 16-byte chunks of 8 values, zero past K.  Wave w owns
// rows w, w + WV, ... and reads them straight from memory: with K <= 2,560
// (at most 5 chunks per lane and row), GR of its rows at a time with all
// their loads in flight at once, then each row's maximum (one DPP
// reduction), the conversion in registers and one LDS write per chunk.
// Longer rows go one at a time in pieces of 8 chunks per lane, read twice
// (maximum, then conversion).  The caller synchronizes afterwards.
template <int WV, int GR>
__device__ __forceinline__ void stage_hidden_f16(const uint16_t* __restrict__ h, int K, int mp, int width, int stride,
                                                 u32x4* __restrict__ lds) {
  constexpr int CPL = 5;  // chunks per lane and row on the fast path
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const __amdgpu_buffer_rsrc_t hs = make_rsrc(h, (uint32_t)mp * (uint32_t)K * 2u);
  if (width <= 64 * CPL) {
    for (int m0 = w; m0 < mp; m0 += GR * WV) {
      u32x4 v[GR][CPL];
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const int m = m0 + r * WV;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = lane + 64 * j;
          v[r][j] = load16<0>(hs, m < mp && c * 8 < K ? (uint32_t)(m * K + c * 8) * 2u : kOobOffset);
        }
      }
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const int m = m0 + r * WV;
        if (m >= mp) break;
        uint32_t mx = 0u;
#pragma unroll
        for (int j = 0; j < CPL; ++j) mx = abs_bits_max(mx, v[r][j]);
        const int n = f16_row_shift(mx);
        u32x4* row = lds + m * stride;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = lane + 64 * j;
          if (c < width) row[c] = bf16x8_to_f16x8_shifted(v[r][j], n);
        }
        if (lane == 0) reinterpret_cast<int*>(row + width)[0] = n;
      }
    }
    return;
  }
  constexpr int P = 8;  // chunks per lane and piece on the long-row path
  for (int m = w; m < mp; m += WV) {
    uint32_t mx = 0u;
    for (int c0 = 0; c0 < width; c0 += 64 * P) {
      u32x4 v[P];
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int c = c0 + lane + 64 * j;
        v[j] = load16<0>(hs, c * 8 < K ? (uint32_t)(m * K + c * 8) * 2u : kOobOffset);
      }
#pragma unroll
      for (int j = 0; j < P; ++j) mx = abs_bits_max(mx, v[j]);
    }
    const int n = f16_row_shift(mx);
    u32x4* row = lds + m * stride;
    for (int c0 = 0; c0 < width; c0 += 64 * P) {
      u32x4 v[P];
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int c = c0 + lane + 64 * j;
        v[j] = load16<0>(hs, c * 8 < K ? (uint32_t)(m * K + c * 8) * 2u : kOobOffset);
      }
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int c = c0 + lane + 64 * j;
        if (c < width) row[c] = bf16x8_to_f16x8_shifted(v[j], n);
      }
    }
    if (lane == 0) reinterpret_cast<int*>(row + width)[0] = n;
  }
}

// Matrix-core path with coalesced loads.  The MFMA operand layout wants the
// 16 lanes of a k-group to hold 16 different head rows, which makes every
// load instruction touch 16 rows x 64 bytes; HBM streams such loads at
// about 6 TB/s against 7 TB/s for whole row pieces.  Here each wave loads a
// batch of its 16-row tile with coalesced instructions (lane l: chunk l % BC
// of row l / BC, BC = 4 SB chunks = SB k-steps), writes it to a private LDS
// stage, and reads the A operands back in MFMA layout.  Hidden rows are in
// LDS as in proj_argmax_mfma.  The stage is private to the wave, so the
// exchange needs only wave-level ordering, not a workgroup barrier.
//
// IDX: the tile's 16 rows are list entries; row i of a tile is row
// epi.rowmap[tile * 16 + i] of W.  The 16 ids of the wave's next tile are
// read with scalar loads when a tile starts (one tile ahead), each lane
// forms 64-bit addresses of its rows, and the loads are plain global loads
// (past the row end, or for a row whose id is outside [0, nw), they read
// row 0 and the values are dropped).  A 16-bit mask of the rows that take
// part travels with the tile in a short history until the tile finishes.
//
// FMT selects the head's format.  A k-step is 32 head-row elements: four
// 16-byte chunks of bf16; two of E4M3 codes (kFmtFp8: codes become bf16
// when read from the stage, and a row's sum is multiplied by its fp32
// scale); or one of E2M1 codes (kFmtMx4: one E8M0 scale per k-step and row;
// each batch also loads the 16 scale bytes of each of its 16 rows, staged
// beside the codes, and the codes become bf16 times the scale, exactly); or
// NVFP4 (kFmtNv4: as MXFP4, with two E4M3 block scales per k-step and row,
// 32 scale bytes per row per batch; each code times its decoded block scale
// exactly in f16, against hidden rows in f16 scaled by a power of two per
// row (hidden_rows_to_f16), on the f16 matrix instruction; a row's sum is
// multiplied by the inverse power of two, then once by the head's fp32
// scale *gsc).
template <int NT, int SB, int WV, int D, int TK, bool LOGITS, int FMT, bool IDX = false>
__global__ void __launch_bounds__(64 * WV)
proj_mfma(const uint16_t* __restrict__ h, const void* __restrict__ Wv, const void* __restrict__ wsc,
          const float* __restrict__ gsc, int R, int K, int m_base, int mp, Epi epi, int early) {
  constexpr bool FP8 = FMT == kFmtFp8;
  constexpr bool NV4 = FMT == kFmtNv4;
  constexpr bool MX4 = FMT == kFmtMx4 || NV4;   // the E2M1 code layout and batch shape
  static_assert(!IDX || (TK == 1 && !LOGITS && FMT == kFmtBf16), "indexed rows: bf16 argmax epilogue");
  static_assert(!MX4 || SB == 16, "MXFP4 / NVFP4: a batch is 16 k-steps, one scale piece per row");
  const float* wscale = static_cast<const float*>(wsc);     // FP8: [R] fp32
  const uint8_t* mxscale = static_cast<const uint8_t*>(wsc);  // MX4: E8M0 codes; NV4: E4M3 codes (tiled)
  constexpr int SPR = NV4 ? 2 : 1;  // MX4 / NV4: 16-byte scale chunks per row per batch
  constexpr int CPS = FP8 ? 2 : (MX4 ? 1 : 4);  // 16-byte chunks per k-step
  constexpr int BC = CPS * SB;      // 16-byte chunks per row per batch
  static_assert(BC == 16 || BC == 32 || BC == 64, "a load instruction covers whole row pieces");
  constexpr int SC = BC + LMH_MFMA_SPAD;  // stage row stride in chunks
  constexpr int RPI = 64 / BC;      // rows per load instruction
  constexpr int LPB = 16 / RPI;     // load instructions per batch
  const uint8_t* W = static_cast<const uint8_t*>(Wv);
  extern __shared__ u32x4 lds[];  // [mp][row_chunks] hidden rows, then [WV][16][SC] stages
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int wchunks = FP8 ? (K >> 4) : (MX4 ? (K >> 5) : (K >> 3));  // 16-byte chunks of a head row
  const int steps = (K + 31) >> 5;
  const int s4 = steps * 4;
  const int row_chunks = s4 + (MX4 ? LMH_MFMA_HPAD4 : LMH_MFMA_HPAD);

  // The hidden rows go to LDS either first, or (early != 0) once the
  // wave's first batches are in flight: see mfma_stage_early.  NV4: as f16
  // (stage_hidden_f16), and each lane takes its columns' power-of-two
  // exponents.
  int hexp[NV4 ? NT : 1];
  auto load_hidden = [&]() __attribute__((always_inline)) {
    if constexpr (NV4)
      stage_hidden_f16<WV, (NT * 16 / WV < 3 ? NT * 16 / WV : 3)>(h + (size_t)m_base * K, K, mp, s4, row_chunks, lds);
    else
      stage_hidden<64 * WV, NT == 2 ? 16 : 8>(h + (size_t)m_base * K, K, mp, s4, row_chunks, lds);
    __syncthreads();
    if constexpr (NV4) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = nt * 16 + i16;
        hexp[nt] = reinterpret_cast<const int*>(lds + (col < mp ? col : mp - 1) * row_chunks + s4)[0];
      }
    }
  };
  if (!early) load_hidden();
  u32x4* stage = lds + mp * row_chunks + wave * 16 * SC;
  // MX4 / NV4: this wave's scale stage, SPR 16-byte chunks (16 k-steps) per row
  u32x4* sstage = lds + mp * row_chunks + WV * 16 * SC + wave * 16 * SPR;
  const u32x4* bptr[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + i16;
    bptr[nt] = lds + (col < mp ? col : mp - 1) * row_chunks + g;
  }

  // epilogue state of this lane's column (hidden row) in each 16-column
  // tile: the running best row (TK == 1); for TK <= 4 the TK best keys of
  // the rows this lane saw; for larger TK the column's best 16 spread over
  // its 4 lanes (col_merge)
  constexpr bool kLaneLists = TK > 1 && TK <= kLaneListMaxTk && !LOGITS;
  constexpr bool kColLists = TK > kLaneListMaxTk && !LOGITS;
  static_assert(TK <= 16, "a column list holds 16 keys");
  float best[NT];
  int bidx[NT];
  KeyList<TK> lists[kLaneLists ? NT : 1];
  unsigned long long clist[kColLists ? NT : 1][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    best[nt] = 0.0f;
    bidx[nt] = -1;
  }
#pragma unroll
  for (int nt = 0; nt < (kLaneLists ? NT : 1); ++nt) lists[nt].clear();
#pragma unroll
  for (int nt = 0; nt < (kColLists ? NT : 1); ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) clist[nt][v] = 0ull;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t row_bytes = FP8 ? (uint32_t)K : (MX4 ? (uint32_t)K / 2u : (uint32_t)K * 2u);
  // MX4 / NV4: scale bytes per row (a tile holds 16 rows' worth)
  const uint32_t sc_row_bytes = NV4 ? (uint32_t)K / 16u : (uint32_t)K / 32u;
  // NV4: the head's fp32 scale, one scalar load
  const float gscale = NV4 ? *gsc : 1.0f;
  const int ntiles = (R + 15) >> 4;
  const int nbatch = (steps + SB - 1) / SB;
  const int lrow = lane / BC;  // row of this lane within a load instruction
  const int lc = lane % BC;    // chunk of this lane within the batch

  const int tstride = gridDim.x * WV;  // tiles between a wave's consecutive tiles
  uint32_t rowoff[LPB];
#pragma unroll
  for (int q = 0; q < LPB; ++q) rowoff[q] = (uint32_t)(q * RPI + lrow) * row_bytes;

  // FP8: scales of head rows r0 .. r0 + 15 of a tile, read with scalar
  // loads one tile ahead (the wave's next tile), clamped to the last row.
  float sc[FP8 ? 16 : 1];
  auto load_scales = [&](int tile) __attribute__((always_inline)) {
    if constexpr (FP8) {
      const int r0 = tile * 16;
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[j] = wscale[min(r0 + j, R - 1)];
    }
  };

  // IDX state: ids of the tile being issued (snext holds the next tile's,
  // fetched one tile ahead), this lane's row addresses in it, and the
  // masks of rows that take part in the last few tiles issued (16 bits per
  // tile, newest lowest; `pushed` is the newest tile's index).
  int snext[IDX ? 16 : 1];
  const uint8_t* vrow[IDX ? LPB : 1];
  unsigned long long hist = 0ull;
  int pushed = 0;
  auto fetch_tile_ids = [&](int tile) __attribute__((always_inline)) {
    if constexpr (IDX) {
      const int r0 = tile * 16;
#pragma unroll
      for (int i = 0; i < 16; ++i) snext[i] = epi.rowmap[min(r0 + i, R - 1)];  // checked against R when used
    }
  };
  auto start_issue_tile = [&](int tile) __attribute__((always_inline)) {
    if constexpr (IDX) {
      int scur[16];
      uint32_t mask = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = tile * 16 + i < R && row_id_ok(snext[i], epi.nw);
        scur[i] = ok ? snext[i] : -1;
        mask |= ok ? (1u << i) : 0u;
      }
#pragma unroll
      for (int q = 0; q < LPB; ++q) {
        int id = scur[q * RPI];
#pragma unroll
        for (int l = 1; l < RPI; ++l) id = lrow == l ? scur[q * RPI + l] : id;
        vrow[q] = W + (size_t)(row_id_ok(id, epi.nw) ? id : 0) * row_bytes;
      }
      hist = (hist << 16) | mask;
      pushed = tile;
      fetch_tile_ids(tile + tstride);
    }
  };
  // Rows of tile `tile` (issued at most three tiles ago) that take part,
  // bit i for row i of the tile.
  auto tile_mask = [&](int tile) __attribute__((always_inline)) -> uint32_t {
    const int d = (pushed - tile) / tstride;
    return (uint32_t)(hist >> (16 * d)) & 0xFFFFu;
  };

  // Positions past the last tile get a descriptor with no records, so their
  // loads read zero without touching memory (live is clamped at 0).
  auto issue = [&](u32x4 (&buf)[LPB], u32x4& sbuf, int tile, int b) __attribute__((always_inline)) {
    if constexpr (IDX) {
      if (b == 0) start_issue_tile(tile);
      const int cg = b * BC + lc;
      const size_t coff = (size_t)(cg < wchunks ? cg : 0) * 16u;
#pragma unroll
      for (int q = 0; q < LPB; ++q)
        buf[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vrow[q] + coff));
      return;
    }
    const int r0 = tile < ntiles ? tile * 16 : 0;
    const int live = tile < ntiles ? min(16, R - r0) : 0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + (size_t)r0 * row_bytes, (uint32_t)live * row_bytes);
    // Column offset of this lane, or an offset past num_records for chunks
    // beyond K.  Selected once per batch so the loads themselves carry no
    // condition (and stay countable for the wait counters).
    const int cg = b * BC + lc;
    const uint32_t cbase = cg < wchunks ? (uint32_t)cg * 16u : kOobOffset;
#pragma unroll
    for (int q = 0; q < LPB; ++q) buf[q] = load16<kPolicyStream>(rs, cbase + rowoff[q]);
    if constexpr (MX4) {
      // lane (g < SPR, i16): scale chunk g of row i16 for k-steps b*16 ..
      // b*16 + 15, at ((b * 16 + i16) * SPR + g) * 16 in the tile's part of
      // the tiled scale layout (whole 16-row tiles, so one piece of 256
      // (MXFP4) or 512 (NVFP4) contiguous bytes per batch)
      const __amdgpu_buffer_rsrc_t ss =
          make_rsrc(mxscale + (size_t)r0 * sc_row_bytes, live > 0 ? 16u * sc_row_bytes : 0u);
      const uint32_t soff = g < SPR && i16 < live
                                ? (((uint32_t)b * 16u + (uint32_t)i16) * (uint32_t)SPR + (uint32_t)g) * 16u
                                : kOobOffset;
      sbuf = load16<kPolicyStream>(ss, soff);
    } else {
      (void)sbuf;
    }
  };
  // NV4: the lane's 8 codes of k-step sb (elements 8 g .. 8 g + 7) share
  // the block scale of block 2 sb + g / 2, byte 2 sb + g / 2 of row i16's
  // 32 scale bytes.  nv4_scales gathers that byte for 4 k-steps at once with
  // one byte permute (selector bytes g / 2, 2 + g / 2, 4 + g / 2, 6 + g / 2
  // over the 8 bytes of k-steps c0 .. c0 + 3) and decodes them to f16 with
  // two gfx950 E4M3 conversions (scale 1: exact, every E4M3 value is a
  // normal f16 number).
  const uint32_t nv_sel = 0x06040200u + (uint32_t)(g >> 1) * 0x01010101u;
  auto nv4_scales = [&](int c0, f16x2& lo, f16x2& hi) __attribute__((always_inline)) {
    const uint2 w = reinterpret_cast<const uint2*>(sstage)[i16 * 4 + (c0 >> 2)];
    const uint32_t s4 = __builtin_amdgcn_perm(w.y, w.x, nv_sel);
    lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, true);
  };
  // A operand of k-step sb of the staged batch: 8 elements of row i16 (NV4:
  // times the block scale `nsc` from nv4_scales)
  auto a_operand = [&](int sb, _Float16 nsc = (_Float16)0) __attribute__((always_inline)) -> u32x4 {
    if constexpr (FP8) {
      const uint2 raw = reinterpret_cast<const uint2*>(stage)[(i16 * SC + 2 * sb) * 2 + g];
      return fp8x8_to_bf16x8(raw.x, raw.y);
    } else if constexpr (NV4) {
      const uint32_t codes = reinterpret_cast<const uint32_t*>(stage)[(i16 * SC + sb) * 4 + g];
      return fp4x8_times_scale_to_f16x8(codes, nsc);
    } else if constexpr (MX4) {
      const uint32_t codes = reinterpret_cast<const uint32_t*>(stage)[(i16 * SC + sb) * 4 + g];
      const uint32_t e = reinterpret_cast<const uint8_t*>(sstage)[i16 * 16 + sb];
      return fp4x8_to_bf16x8(codes, e);
    } else {
      return stage[i16 * SC + 4 * sb + g];
    }
  };
  auto mma_step = [&](const u32x4& a, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 bf = bptr[nt][s * 4];
      if constexpr (NV4)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                         __builtin_bit_cast(f16x8, bf), acc[nt], 0, 0, 0);
      else
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, bf), acc[nt], 0, 0, 0);
    }
  };
  auto consume = [&](const u32x4 (&buf)[LPB], const u32x4& sbuf, int b) __attribute__((always_inline)) {
    // IDX: chunks past the row end were loaded from column 0; zero them
    const bool in_row = !IDX || b * BC + lc < wchunks;
#pragma unroll
    for (int q = 0; q < LPB; ++q) stage[(q * RPI + lrow) * SC + lc] = in_row ? buf[q] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (MX4) {
      if (g < SPR) sstage[i16 * SPR + g] = sbuf;
    }
    // lanes of this wave exchange data through the stage
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (MX4 || (b + 1) * SB <= steps) {  // MXFP4 / NVFP4 heads hold whole batches (K % 512 == 0)
      // whole batch: operand reads first, then the matrix instructions, in
      // groups of CH k-steps (MXFP4's 16 k-steps at once would not fit the
      // registers)
      constexpr int CH = MX4 ? 4 : SB;
#pragma unroll
      for (int c0 = 0; c0 < SB; c0 += CH) {
        u32x4 a[CH];
        if constexpr (NV4) {
          static_assert(CH == 4, "NV4: one scale gather per 4 k-steps");
          f16x2 lo, hi;
          nv4_scales(c0, lo, hi);
          a[0] = a_operand(c0, lo[0]);
          a[1] = a_operand(c0 + 1, lo[1]);
          a[2] = a_operand(c0 + 2, hi[0]);
          a[3] = a_operand(c0 + 3, hi[1]);
        } else {
#pragma unroll
          for (int sb = 0; sb < CH; ++sb) a[sb] = a_operand(c0 + sb);
        }
#pragma unroll
        for (int sb = 0; sb < CH; ++sb) mma_step(a[sb], b * SB + c0 + sb);
      }
    } else if constexpr (!MX4) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int s = b * SB + sb;
        if (s < steps) mma_step(a_operand(sb), s);
      }
    }
    // the next batch overwrites the stage only after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Logits without d2t: lane (g, i16) holds head rows 4 g .. 4 g + 3 of its
  // column, one 16-byte store where the row block is whole and aligned;
  // through d2t, one store per row and column.  Whole tiles are held in a
  // shift register of kLogitTiles tiles and stored together when it fills
  // and at the end (through d2t a tile at a time, after loading its
  // columns): on this chip stores count
  // towards the same wait counter as the weight loads, so a store after
  // every tile made later waits stall on its acknowledgement (the full head
  // at 16 and 24 hidden rows took 28 and 36 us longer than without the
  // stores).
  const bool vec_logits =
      LOGITS && !epi.d2t && (epi.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(epi.logits) & 15) == 0;
  constexpr int kLogitTiles = LOGITS ? 8 : 1;
  f32x4 lbuf[kLogitTiles][NT];
  int lbase[kLogitTiles];
  int nbuf = 0;
  auto flush_logits = [&]() __attribute__((always_inline)) {
    if (epi.d2t) {
      // scattered through d2t, a tile at a time: its rows' vocabulary
      // columns, then its stores (the first wait drains the loads in
      // flight once per flush, the later ones only these columns)
#pragma unroll
      for (int k = 0; k < kLogitTiles; ++k) {
        if (k < nbuf) {
          int dcol[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) dcol[v] = epi.d2t[lbase[k] + 4 * g + v];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (dcol[v] >= 0 && dcol[v] < epi.ncols) {
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) {
                const int col = nt * 16 + i16;
                if (col < mp) epi.logits[(int64_t)(m_base + col) * epi.ld + dcol[v]] = lbuf[k][nt][v];
              }
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kLogitTiles; ++k) {
        if (k < nbuf) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int col = nt * 16 + i16;
            if (col < mp)
              *reinterpret_cast<f32x4*>(epi.logits + (int64_t)(m_base + col) * epi.ld + lbase[k] + 4 * g) =
                  lbuf[k][nt];
          }
        }
      }
    }
    nbuf = 0;
  };
  auto finish_tile = [&](int tile) __attribute__((always_inline)) {
    const int r0 = tile * 16;
    if constexpr (FP8) {
      // this lane's rows are 4 g + v: pick their scales, then prefetch.
      // The pick is a sum with 0 / 1 weights (exact for finite scales): a
      // select chain would become an indexed array in scratch memory.
      const float w0 = g == 0 ? 1.0f : 0.0f, w1 = g == 1 ? 1.0f : 0.0f;
      const float w2 = g == 2 ? 1.0f : 0.0f, w3 = g == 3 ? 1.0f : 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float s = (sc[v] * w0 + sc[4 + v] * w1) + (sc[8 + v] * w2 + sc[12 + v] * w3);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][v] *= s;
      }
      load_scales(tile + tstride);
    } else if constexpr (NV4) {
      // the hidden row's power of two off (exact), then the head's scale,
      // once per row sum
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][v] = __builtin_ldexpf(acc[nt][v], -hexp[nt]) * gscale;
    }
    if (LOGITS && (vec_logits || epi.d2t) && r0 + 15 < R) {
      // a whole tile: into the shift register (static moves, no indexing)
#pragma unroll
      for (int k = kLogitTiles - 1; k > 0; --k) {
        lbase[k] = lbase[k - 1];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) lbuf[k][nt] = lbuf[k - 1][nt];
      }
      lbase[0] = r0;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        lbuf[0][nt] = acc[nt];
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (++nbuf == kLogitTiles) flush_logits();
      return;
    }
    const uint32_t live = IDX ? tile_mask(tile) >> (4 * g) : 0xFu;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 4 * g + v;
      if (r < R && ((live >> v) & 1u)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (LOGITS) {
            const int col = nt * 16 + i16;
            if (col < mp) store_logit(epi, m_base + col, r, acc[nt][v]);
          } else if constexpr (TK == 1) {
            take_best(acc[nt][v], r, best[nt], bidx[nt]);
          } else if constexpr (kLaneLists) {
            lists[nt].push(pack_key(acc[nt][v], r));
          }
        }
      }
    }
    if constexpr (kColLists) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        unsigned long long c[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = r0 + 4 * g + v;
          c[v] = r < R ? pack_key(acc[nt][v], r) : 0ull;
        }
        col_merge(clist[nt], c, g);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // The wave walks (tile, batch) pairs in order with a ring of D register
  // buffers: D - 1 batches are in flight while one is transposed and fed to
  // the matrix cores.  The loop is unrolled D times so ring slots are static.
  int ti = first_unit(wave, WV), bi = 0;  // next pair to issue
  int tc = ti, bc = 0;                      // next pair to consume
  auto advance = [&](int& t, int& bb) __attribute__((always_inline)) {
    if (++bb == nbatch) {
      bb = 0;
      t += tstride;
    }
  };
  // Number of (tile, batch) pairs this wave consumes.
  const int my_tiles = tc < ntiles ? (ntiles - 1 - tc) / tstride + 1 : 0;
  const int count = my_tiles * nbatch;
  u32x4 ring[D][LPB];
  u32x4 sring[D];  // MX4: the scale chunk of each batch in flight
  load_scales(ti);
  fetch_tile_ids(ti);
#pragma unroll
  for (int j = 0; j < D - 1; ++j) {
    issue(ring[j], sring[j], ti, bi);
    advance(ti, bi);
  }

  if (early) load_hidden();

  auto step = [&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    issue(ring[(j + D - 1) % D], sring[(j + D - 1) % D], ti, bi);
    advance(ti, bi);
    consume(ring[j], sring[j], bc);
    if (bc == nbatch - 1) finish_tile(tc);
    advance(tc, bc);
  };
  int n = 0;
  // steady state: every slot issues and consumes, no conditions on loads
  for (; n + D <= count; n += D) {
    [&]<int... J>(std::integer_sequence<int, J...>) { (step(std::integral_constant<int, J>{}), ...); }(
        std::make_integer_sequence<int, D>{});
  }
  // last partial round
  [&]<int... J>(std::integer_sequence<int, J...>) {
    ((n + J < count ? (step(std::integral_constant<int, J>{}), 0) : 0), ...);
  }(std::make_integer_sequence<int, D>{});

  if constexpr (LOGITS) {
    flush_logits();
    return;
  } else if constexpr (TK == 1) {
    // the waves' keys go to the stage area once every wave is past its main
    // loop (a static array there would cost the LDS that lets 24 hidden rows
    // of an NVFP4 head run 8-wave workgroups)
    __syncthreads();
    unsigned long long (*s_key)[32] = reinterpret_cast<unsigned long long (*)[32]>(lds + mp * row_chunks);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      unsigned long long k = pack_key(best[nt], bidx[nt]);
      // fold the four lanes (g = 0..3) that hold the same hidden row
      k = max_u64(k, xrow_u64<16>(k, g));
      k = max_u64(k, xrow_u64<32>(k, g));
      const int col = nt * 16 + i16;
      if (g == 0 && col < 32) s_key[wave][col] = k;
    }
    __syncthreads();
    if (wave != 0) return;
    unsigned long long key = 0ull;
    if (lane < mp) {
#pragma unroll
      for (int w = 0; w < WV; ++w) key = s_key[w][lane] > key ? s_key[w][lane] : key;
    }
    if (epi.state)
      merge_and_fold_if_last(epi, key, lane, mp, m_base);
    else
      publish_workgroup(key, lane, mp, m_base, epi.slots);
  } else if constexpr (kColLists) {
    // every wave is past its main loop: the stage area is free for the lists
    __syncthreads();
    unsigned long long* s_list = reinterpret_cast<unsigned long long*>(lds + mp * row_chunks);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + i16;
      if (col < mp) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s_list[(wave * 32 + col) * 16 + 4 * g + v] = clist[nt][v];
      }
    }
    __syncthreads();
    publish_rows<TK, WV, 16>(s_list, 32, mp, m_base, epi.slots);
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lists[nt].template merge_xor<16>(g);
      lists[nt].template merge_xor<32>(g);
    }
    // every wave is past its main loop: the stage area is free for the lists
    __syncthreads();
    unsigned long long* s_list = reinterpret_cast<unsigned long long*>(lds + mp * row_chunks);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + i16;
      if (g == 0 && col < mp) {
#pragma unroll
        for (int j = 0; j < TK; ++j) s_list[(wave * 32 + col) * TK + j] = lists[nt].k[j];
      }
    }
    __syncthreads();
    publish_rows<TK, WV, TK>(s_list, 32, mp, m_base, epi.slots);
  }
}

// ---------------------------------------------------------------------------
// measurement kernels
// ---------------------------------------------------------------------------
constexpr int kBenchThreads = 256;
constexpr int kBenchSinkWords = 65536;

// Practical HBM read ceiling: every lane keeps two groups of four 16-byte
// non-temporal loads in flight (the next group is issued before the current
// one is consumed).  Past the end, indexes are clamped to the last vector
// (re-read, never out of bounds).  On MI355X this reads 7.19 TB/s with one
// 256-thread workgroup per CU; more waves per CU read less (5.6 TB/s at 16).
constexpr int kStreamGroup = 4;

__global__ void __launch_bounds__(kBenchThreads)
stream_read(const u32x4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kBenchThreads;
  const size_t last = n16 - 1;
  const size_t per = (size_t)kStreamGroup * stride;
  const size_t groups = (n16 + per - 1) / per;
  size_t i = (size_t)blockIdx.x * kBenchThreads + threadIdx.x;
  uint32_t x = 0;
  u32x4 a[kStreamGroup], b[kStreamGroup];
  auto load = [&](u32x4 (&v)[kStreamGroup], size_t base) {
#pragma unroll
    for (int u = 0; u < kStreamGroup; ++u) {
      const size_t j = base + (size_t)u * stride;
      v[u] = __builtin_nontemporal_load(src + (j <= last ? j : last));
    }
  };
  auto fold = [&](const u32x4 (&v)[kStreamGroup]) {
#pragma unroll
    for (int u = 0; u < kStreamGroup; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  };
  load(a, i);
  for (size_t g = 0; g < groups; g += 2) {
    load(b, i + per);
    fold(a);
    load(a, i + 2 * per);
    fold(b);
    i += 2 * per;
  }
  // one word per workgroup
  __shared__ uint32_t s[kBenchThreads];
  s[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int t = 0; t < kBenchThreads; ++t) y ^= s[t];
    sink[blockIdx.x] = y;
  }
}

__global__ void __launch_bounds__(kBenchThreads)
copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kBenchThreads;
  for (size_t i = (size_t)blockIdx.x * kBenchThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s", what, hipGetErrorString(e));
  return LMH_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool k_ok(int64_t K) { return K >= LMH_MIN_K && K <= LMH_MAX_K && (K % 8) == 0; }

// The host-side figures a launch is planned from (CU count, resident
// workgroups per CU) are fixed per device and kernel shape, so each is
// asked of the runtime once and kept: an occupancy query costs about as
// much host time as a launch, and a short call makes two launches.
struct OccupancyKey {
  int dev;
  const void* f;
  int threads;
  size_t lds;
  int per_cu;
};
std::mutex g_query_mu;
std::vector<std::pair<int, int>> g_cu_counts;  // (device, CUs)
std::vector<OccupancyKey> g_occupancy;

int cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  {
    std::lock_guard<std::mutex> lock(g_query_mu);
    for (const auto& dc : g_cu_counts)
      if (dc.first == dev) {
        *out = dc.second;
        return LMH_OK;
      }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  *out = n < 1 ? 1 : n;
  std::lock_guard<std::mutex> lock(g_query_mu);
  g_cu_counts.emplace_back(dev, *out);
  return LMH_OK;
}

// Workgroups of kernel `f` that can be resident on one CU at once.  The
// projection kernels are persistent (each workgroup strides over rows), so
// the grid is sized to what is resident: a second, partial round of
// workgroups would double the tail.
int resident_per_cu(const void* f, int threads, size_t lds, int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  {
    std::lock_guard<std::mutex> lock(g_query_mu);
    for (const auto& k : g_occupancy)
      if (k.dev == dev && k.f == f && k.threads == threads && k.lds == lds) {
        *out = k.per_cu;
        return LMH_OK;
      }
  }
  int n = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, threads, lds);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  *out = n < 1 ? 1 : n;
  std::lock_guard<std::mutex> lock(g_query_mu);
  g_occupancy.push_back(OccupancyKey{dev, f, threads, lds, *out});
  return LMH_OK;
}

int chunks_per_lane(int64_t K) { return (int)((K / 8 + 63) / 64); }

bool valu_ok(int64_t M, int64_t K) {
  return M >= 1 && M <= kValuMaxM && k_ok(K) && M * chunks_per_lane(K) <= kValuMaxChunksTimesM;
}

// LDS bytes of one hidden row in the matrix-core kernel for a head format
int mfma_row_bytes(int64_t K, int fmt) {
  const int pad = fmt == kFmtMx4 || fmt == kFmtNv4 ? LMH_MFMA_HPAD4 : LMH_MFMA_HPAD;
  return (int)((((K + 31) / 32) * 4 + pad) * 16);
}


typedef void (*proj_fn)(const uint16_t*, const uint16_t*, int, int, Epi);

// One VALU launch shape: kernel, waves per workgroup, head rows a wave takes
// per step, LDS bytes.  The choice per M comes from measurement on MI355X
// (full 248,320 x 2,560 head): M = 1 streams fastest in 4-row tiles; M = 2..8
// in row order with one workgroup per CU (4 waves up to M = 4, else 8).
// Every epilogue (argmax, top-k, logits) uses the same shapes; top-k and
// logits take M <= 4.
struct ValuPlan {
  proj_fn fn = nullptr;
  int waves = 0;
  int rows_per_wave = 0;
  size_t lds = 0;
};

template <int M, int CPL, int WV, int TK, bool LOGITS, bool IDX, int LOOP>
void row_plan(ValuPlan& p) {
  if constexpr (M * CPL <= kValuMaxChunksTimesM) {
    // rows per step: keep each of the two row buffers at <= 10 chunks/lane,
    // and one row per step once h alone takes more than 80 registers.  The
    // ring loop at 3 and 4 hidden rows, and over rows read in place, takes
    // one row per step: 1.4-5.2% faster on the 16,000-, 32,768- and
    // 52,755-row lists and 1.1-4.5% on lists read in place (interleaved
    // builds on one machine); the pair loop at those M is 8-17% slower so.
    constexpr bool kOne = M * CPL > 20 || (LOOP == kLoopRing && (M == 3 || M == 4 || IDX));
    constexpr int U0 = kOne ? 1 : (CPL * LMH_VALU_ROWS <= 10 ? LMH_VALU_ROWS : (CPL <= 10 ? 10 / CPL : 1));
    constexpr int U = U0 < 1 ? 1 : U0;
    p.fn = proj_valu_rows<M, CPL, U, WV, TK, LOGITS, IDX, LOOP>;
    p.waves = WV;
    p.rows_per_wave = U;
    p.lds = 0;
  }
}

template <int M, int TK, bool LOGITS, bool IDX, int LOOP, int... C>
void row_plan_cpl(ValuPlan& p, int cpl, std::integer_sequence<int, C...>) {
  constexpr int WV = M <= 4 ? LMH_VALU_WAVES : 2 * LMH_VALU_WAVES;
  ((cpl == C + 1 ? (row_plan<M, C + 1, WV, TK, LOGITS, IDX, LOOP>(p), 0) : 0), ...);
}

template <int M, int TK, bool LOGITS, int LOOP>
ValuPlan tiled_plan(int K) {
  ValuPlan p;
  p.fn = proj_valu_tiled<M, LMH_VALU_TILE_ROWS, LMH_VALU_WAVES, TK, LOGITS, LOOP>;
  p.waves = LMH_VALU_WAVES;
  p.rows_per_wave = LMH_VALU_TILE_ROWS;
  p.lds = (size_t)M * chunks_per_lane(K) * 64 * 16;
  return p;
}

// Row-order plan for M = 1..4.  The argmax takes the ring loop at 3 and 4
// hidden rows on every head (with one row per step: 1.6-2.8% faster than
// the two-buffer loop on heads of 131,072-248,320 rows at three rows, up to
// 1.7% at four), over rows read in place, and at 1 and 2 rows below
// LMH_RING_MAX_ROWS head rows.  Top k takes it at 3 and 4 rows (the
// 16,000-row list at M = 3 5% faster, the full head 1.3-1.5%); logits take
// it below LMH_RING_MAX_ROWS head rows (2-6% faster on the lists, 1.7%
// slower on the full head at 3 and 4 rows, with their stores batched).
template <int M, int TK, bool LOGITS, bool IDX>
void row_plan_m(ValuPlan& p, int cpl, int64_t R) {
  using seq = std::make_integer_sequence<int, 16>;
  if constexpr (TK == 1 && !LOGITS) {
    if (M >= 3 || IDX || R < LMH_RING_MAX_ROWS) {
      row_plan_cpl<M, TK, LOGITS, IDX, kLoopRing>(p, cpl, seq{});
      return;
    }
  } else if constexpr (!LOGITS) {
    if (M >= 3) {
      row_plan_cpl<M, TK, LOGITS, IDX, kLoopRing>(p, cpl, seq{});
      return;
    }
  } else {
    if (R < LMH_RING_MAX_ROWS) {
      row_plan_cpl<M, TK, LOGITS, IDX, kLoopRing>(p, cpl, seq{});
      return;
    }
  }
  row_plan_cpl<M, TK, LOGITS, IDX, kLoopPair>(p, cpl, seq{});
}

template <int TK, bool LOGITS, bool IDX = false>
ValuPlan valu_plan(int M, int K, int64_t R) {
  ValuPlan p;
  // Two hidden rows (the verify step of a depth-1 draft): the tiled kernel
  // measured 2.2% faster than the row-order one on the full head (181.0
  // against 185.1 us) and level on lists; from three rows on it is slower
  // (198.2 against 183.5 us at three, 229.6 against 178.6 at four).  Rows
  // read in place through a list (IDX) take the row-order kernel's ring
  // loop with one row per step at one and two hidden rows too: 6-9% faster
  // than the tiled kernel on the 16,000- and 32,768-row lists at M = 1,
  // 10-11% at M = 2, 2.6% on the 52,755-row list at M = 1 (interleaved
  // builds on one machine).
  if constexpr (!IDX) {
    if constexpr (TK == 1 && !LOGITS) {
      if (M == 2 && LMH_VALU_TILE_ROWS > 0)
        return R < LMH_RING_MAX_ROWS ? tiled_plan<2, TK, LOGITS, kLoopRing>(K)
                                     : tiled_plan<2, TK, LOGITS, kLoopUncond>(K);
    }
    if (M == 1 && LMH_VALU_TILE_ROWS > 0) {
      if constexpr (TK == 1 && !LOGITS)
        return R < LMH_RING_MAX_ROWS ? tiled_plan<1, TK, LOGITS, kLoopRing>(K)
                                     : tiled_plan<1, TK, LOGITS, kLoopUncond>(K);
      else if constexpr (LOGITS)
        return R < LMH_RING_MAX_ROWS ? tiled_plan<1, TK, LOGITS, kLoopRing>(K)
                                     : tiled_plan<1, TK, LOGITS, kLoopPair>(K);
      else
        return tiled_plan<1, TK, LOGITS, kLoopPair>(K);
    }
  }
  const int cpl = chunks_per_lane(K);
  using seq = std::make_integer_sequence<int, 16>;
  switch (M) {
    case 1: row_plan_m<1, TK, LOGITS, IDX>(p, cpl, R); break;
    case 2: row_plan_m<2, TK, LOGITS, IDX>(p, cpl, R); break;
    case 3: row_plan_m<3, TK, LOGITS, IDX>(p, cpl, R); break;
    case 4: row_plan_m<4, TK, LOGITS, IDX>(p, cpl, R); break;
    default:
      if constexpr (TK == 1 && !LOGITS) {
        switch (M) {
          case 5: row_plan_cpl<5, 1, false, IDX, kLoopPair>(p, cpl, seq{}); break;
          case 6: row_plan_cpl<6, 1, false, IDX, kLoopPair>(p, cpl, seq{}); break;
          case 7: row_plan_cpl<7, 1, false, IDX, kLoopPair>(p, cpl, seq{}); break;
          case 8: row_plan_cpl<8, 1, false, IDX, kLoopPair>(p, cpl, seq{}); break;
          default: break;
        }
      }
      break;
  }
  return p;
}

// Lets kernel `f` request the whole LDS of a workgroup, once per kernel.
// Best effort: if the runtime does not take the attribute, the launch
// itself reports an LDS request it cannot meet.
void allow_full_lds(const void* f) {
  static std::mutex mu;
  static std::vector<const void*> done;
  std::lock_guard<std::mutex> lock(mu);
  if (std::find(done.begin(), done.end(), f) != done.end()) return;
  if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsPerWorkgroup) != hipSuccess)
    (void)hipGetLastError();
  done.push_back(f);
}

int clamp_grid(int64_t need, int cus, int per_cu) {
  return (int)std::max<int64_t>(1, std::min<int64_t>({need, (int64_t)cus * per_cu, (int64_t)kMaxGrid}));
}

// Persistent launch: as many workgroups as are resident (at most one round).
template <typename F, typename... Args>
int launch_persistent(F f, int threads, size_t lds, int64_t units, int units_per_wg, int cap_per_cu, int cus,
                      hipStream_t stream, const char* what, int* grid_out, Args... args) {
  allow_full_lds((const void*)f);
  int per_cu = 0;
  const int st = resident_per_cu((const void*)f, threads, lds, &per_cu);
  if (st != LMH_OK) return st;
  const int grid = clamp_grid((units + units_per_wg - 1) / units_per_wg, cus, std::min(per_cu, cap_per_cu));
  hipLaunchKernelGGL(f, dim3(grid), dim3(threads), lds, stream, args...);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  *grid_out = grid;
  return LMH_OK;
}

int launch_valu(const ValuPlan& p, const uint16_t* h, int K, const uint16_t* W, int R, const Epi& epi, int cus,
                hipStream_t stream, int* grid_out) {
  if (!p.fn) return LMH_EINVAL;
  return launch_persistent(p.fn, 64 * p.waves, p.lds, R, p.waves * p.rows_per_wave, LMH_VALU_WG_PER_CU, cus,
                           stream, "launch VALU projection", grid_out, h, W, R, K, epi);
}

// LDS of the per-wave stages of the matrix-core kernel: a 16-row code
// stage (and for MXFP4 a 16-chunk, for NVFP4 a 32-chunk scale stage) per
// wave.
size_t mfma_stage_bytes(int waves, int fmt) {
  const size_t scale_chunks = fmt == kFmtMx4 ? 16 : (fmt == kFmtNv4 ? 32 : 0);
  return (size_t)waves * 16 * (4 * LMH_MFMA_LDS_SB + LMH_MFMA_SPAD) * 16 + (size_t)waves * scale_chunks * 16;
}

// Hidden rows one launch of the matrix-core kernel can stage for K with
// `waves` waves (each with its own stages; the epilogues reuse the stage
// area), with 512 bytes to spare.
int mfma_lds_rows_fit(int64_t K, int waves, int fmt = kFmtBf16) {
  const int64_t stage = (int64_t)mfma_stage_bytes(waves, fmt);
  const int64_t fixed = stage + 512;
  const int64_t rows = (kLdsPerWorkgroup - fixed) / mfma_row_bytes(K, fmt);
  return (int)std::max<int64_t>(0, std::min<int64_t>(LMH_MAX_M, rows));
}

// Whether the matrix-core kernel stages the hidden rows after issuing its
// first batches (so the two latencies overlap) rather than before.  Measured
// on MI355X, interleaved builds on one machine: after wins at 16 and more hidden
// rows (the staging is long: 1-4% at 24 rows on the 52,755-row list) and on
// the full head in every format; before wins on short quantized lists at a
// few rows (MXFP4: 3.5% at 1, 3 and 8 rows; FP8: 1% at 1 and 3 rows), where
// waiting for the early batches delays the start.
bool mfma_stage_early(int fmt, int mp, int64_t R) {
  return R >= LMH_RING_MAX_ROWS || mp >= 16 || (mp >= 5 && fmt != kFmtMx4 && fmt != kFmtNv4);
}

// One pass of the matrix-core path over hidden rows [m_base, m_base + mp):
// 8 waves per workgroup when the hidden rows and eight stages fit the LDS
// and the head has at least 8 tiles per CU, else 4; two 16-column tiles
// when mp > 16.
// FP8 heads take twice the k-steps per batch and MXFP4 / NVFP4 heads four
// times, so a batch moves the same code bytes (and the stage has the same
// size) as for bf16.  `wsc` is the FP8 row scales or the MXFP4 / NVFP4
// block scales; `gsc` the NVFP4 head's fp32 scale (else unused).
template <int TK, bool LOGITS, int FMT, bool IDX = false>
int launch_mfma_pass(const uint16_t* h, int K, int m_base, int mp, const void* W, const void* wsc,
                     const float* gsc, int R, const Epi& epi, int cus, hipStream_t stream, int* grid_out) {
  constexpr int SB = FMT == kFmtFp8 ? 2 * LMH_MFMA_LDS_SB
                                    : (FMT == kFmtMx4 || FMT == kFmtNv4 ? 4 * LMH_MFMA_LDS_SB : LMH_MFMA_LDS_SB);
  constexpr int D = LMH_MFMA_RING;
  const void* wscale = wsc;
  const size_t hbytes = (size_t)mp * mfma_row_bytes(K, FMT);
  const int64_t tiles = (R + 15) / 16;
  // 8 waves per workgroup only when there are tiles for 8 waves on every CU:
  // a shorter head in 8-wave workgroups would leave CUs idle (a 16,000-row
  // list has 1,000 tiles, 125 such workgroups)
  const bool eight = mp <= mfma_lds_rows_fit(K, 8, FMT) && tiles >= 8LL * cus;
  const size_t lds = hbytes + mfma_stage_bytes(eight ? 8 : 4, FMT);
  const char* what = "launch matrix-core projection";
  const int early = mfma_stage_early(FMT, mp, R) ? 1 : 0;
  if (mp <= 16)
    return eight ? launch_persistent(proj_mfma<1, SB, 8, D, TK, LOGITS, FMT, IDX>, 512, lds, tiles, 8, 1 << 20, cus,
                                     stream, what, grid_out, h, W, wscale, gsc, R, K, m_base, mp, epi, early)
                 : launch_persistent(proj_mfma<1, SB, 4, D, TK, LOGITS, FMT, IDX>, 256, lds, tiles, 4, 1 << 20, cus,
                                     stream, what, grid_out, h, W, wscale, gsc, R, K, m_base, mp, epi, early);
  return eight ? launch_persistent(proj_mfma<2, SB, 8, D, TK, LOGITS, FMT, IDX>, 512, lds, tiles, 8, 1 << 20, cus,
                                   stream, what, grid_out, h, W, wscale, gsc, R, K, m_base, mp, epi, early)
               : launch_persistent(proj_mfma<2, SB, 4, D, TK, LOGITS, FMT, IDX>, 256, lds, tiles, 4, 1 << 20, cus,
                                   stream, what, grid_out, h, W, wscale, gsc, R, K, m_base, mp, epi, early);
}

// VALU path over an FP8 head: the tiled kernel for every M <= 4.
typedef void (*proj_fp8_fn)(const uint16_t*, const uint8_t*, const float*, int, int, Epi);

int launch_valu_fp8(const uint16_t* h, int M, int K, const uint8_t* Wq, const float* wscale, int R,
                    const Epi& epi, int cus, hipStream_t stream, int* grid_out) {
  constexpr int TR = LMH_VALU_TILE_ROWS > 0 ? LMH_VALU_TILE_ROWS : 4;
  constexpr int WV = LMH_VALU_WAVES;
  proj_fp8_fn fn = nullptr;
  switch (M) {
    case 1: fn = proj_valu_fp8<1, TR, WV, 1, false>; break;
    case 2: fn = proj_valu_fp8<2, TR, WV, 1, false>; break;
    case 3: fn = proj_valu_fp8<3, TR, WV, 1, false>; break;
    case 4: fn = proj_valu_fp8<4, TR, WV, 1, false>; break;
    default: return LMH_EINVAL;
  }
  const int nb = (K / 16 + 63) / 64;
  const size_t lds = (size_t)M * nb * 128 * 16;
  return launch_persistent(fn, 64 * WV, lds, R, WV * TR, LMH_VALU_WG_PER_CU, cus, stream,
                           "launch VALU FP8 projection", grid_out, h, Wq, wscale, R, K, epi);
}

int launch_finalize_argmax(unsigned long long* slots, int nslots, int m_base, int mcount, const int32_t* d2t,
                           int32_t* out_id, float* out_logit, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_argmax, dim3(mcount), dim3(256), 0, stream, slots, nslots, m_base, d2t, out_id,
                     out_logit);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch finalize_argmax");
}

int launch_finalize_keys(unsigned long long* slots, int nslots, int m_base, int mcount, int64_t row_base,
                         unsigned long long* out_key, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_keys, dim3(mcount), dim3(256), 0, stream, slots, nslots, m_base, row_base, out_key);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch finalize_keys");
}

template <int TK>
int launch_finalize_topk(unsigned long long* slots, int nslots, int m_base, int mcount, int topk,
                         const int32_t* d2t, int32_t* out_id, float* out_logit, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_topk<TK>, dim3(mcount), dim3(kFinalizeTopkThreads), 0, stream, slots, nslots, m_base,
                     topk, d2t, out_id, out_logit);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch finalize_topk");
}

// What one call asks for.  `fmt` is the head's format: bf16, or (argmax
// and top k) E4M3 codes with one fp32 scale per row in `wscale`, or MXFP4
// codes with one E8M0 scale per 32 elements in `wscale`.
struct Call {
  const uint16_t* h;
  int M;
  int K;
  const void* W;
  int R;
  const int32_t* d2t;
  int path;
  hipStream_t stream;
  bool projection_only = false;  // measurement: skip the fold (outputs untouched)
  const void* wscale = nullptr;
  int fmt = kFmtBf16;
  bool indexed = false;          // W is the whole head, read through epi.rowmap (argmax only)
  const float* gscale = nullptr; // NVFP4: the head's fp32 scale (device)
  int64_t row_base = 0;          // keys: global row of the slice's row 0
  unsigned long long* out_key = nullptr;  // keys: [M] packed keys
};

int record(hipEvent_t e, hipStream_t s) {
  const hipError_t r = hipEventRecord(e, s);
  return r == hipSuccess ? LMH_OK : hip_fail(r, "hipEventRecord");
}

// Argmax (TK == 1 with the argmax finalizer), top-TK, every logit, or the
// argmax as global-row keys of a head slice.
// MODE: 0 = argmax, 1 = top-k, 2 = logits, 3 = keys (c.out_key, c.row_base).
template <int MODE, int TK>
int run(const Call& c, const Epi& epi, int topk, int32_t* out_id, float* out_logit) {
  constexpr bool LOGITS = MODE == 2;
  int cus = 0;
  int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  auto finalize = [&](int grid, int m_base, int mcount) -> int {
    if (c.projection_only || epi.state) return LMH_OK;  // single launch: folded in the kernel
    if constexpr (MODE == 0)
      return launch_finalize_argmax(epi.slots, grid, m_base, mcount, c.d2t, out_id, out_logit, c.stream);
    else if constexpr (MODE == 1)
      return launch_finalize_topk<TK>(epi.slots, grid, m_base, mcount, topk, c.d2t, out_id, out_logit, c.stream);
    else if constexpr (MODE == 3)
      return launch_finalize_keys(epi.slots, grid, m_base, mcount, c.row_base, c.out_key, c.stream);
    else
      return LMH_OK;
  };
  const bool fp8 = c.fmt == kFmtFp8;
  const bool mx4 = c.fmt == kFmtMx4;
  const bool nv4 = c.fmt == kFmtNv4;
  if ((fp8 || mx4 || nv4) && MODE == 2) return LMH_EINVAL;  // quantized heads: argmax and top k
  if ((fp8 || mx4 || nv4) && !c.wscale) return LMH_EINVAL;
  if (nv4 && !c.gscale) return LMH_EINVAL;
  constexpr bool kIdxOk = MODE == 0 && TK == 1;
  if (c.indexed && (!kIdxOk || c.fmt != kFmtBf16 || !epi.rowmap)) return LMH_EINVAL;
  if (c.path == LMH_PATH_VALU) {
    int grid = 0;
    if (mx4 || nv4) return LMH_EINVAL;  // MXFP4 and NVFP4 heads take the matrix cores only
    if (fp8) {
      if constexpr (MODE != 0) return LMH_EINVAL;  // top k over an FP8 head: matrix cores only
      st = launch_valu_fp8(c.h, c.M, c.K, static_cast<const uint8_t*>(c.W), static_cast<const float*>(c.wscale),
                           c.R, epi, cus, c.stream, &grid);
    } else {
      ValuPlan p;
      if constexpr (kIdxOk)
        p = c.indexed ? valu_plan<TK, LOGITS, true>(c.M, c.K, c.R) : valu_plan<TK, LOGITS>(c.M, c.K, c.R);
      else
        p = valu_plan<TK, LOGITS>(c.M, c.K, c.R);
      if (!p.fn) return LMH_EINVAL;
      st = launch_valu(p, c.h, c.K, static_cast<const uint16_t*>(c.W), c.R, epi, cus, c.stream, &grid);
    }
    if (st != LMH_OK) return st;
    return finalize(grid, 0, c.M);
  }
  const int cap = mfma_lds_rows_fit(c.K, 4, c.fmt);
  if (cap < 1) return LMH_EINVAL;
  const int passes = (c.M + cap - 1) / cap;
  const int per = (c.M + passes - 1) / passes;
  for (int m0 = 0; m0 < c.M; m0 += per) {
    const int mp = std::min(per, c.M - m0);
    int grid = 0;
    if (fp8 || mx4 || nv4) {
      if constexpr (MODE != 2) {
        if (fp8)
          st = launch_mfma_pass<TK, LOGITS, kFmtFp8>(c.h, c.K, m0, mp, c.W, c.wscale, nullptr, c.R, epi, cus,
                                                     c.stream, &grid);
        else if (mx4)
          st = launch_mfma_pass<TK, LOGITS, kFmtMx4>(c.h, c.K, m0, mp, c.W, c.wscale, nullptr, c.R, epi, cus,
                                                     c.stream, &grid);
        else
          st = launch_mfma_pass<TK, LOGITS, kFmtNv4>(c.h, c.K, m0, mp, c.W, c.wscale, c.gscale, c.R, epi, cus,
                                                     c.stream, &grid);
      }
    } else if (c.indexed) {
      if constexpr (kIdxOk)
        st = launch_mfma_pass<TK, LOGITS, kFmtBf16, true>(c.h, c.K, m0, mp, c.W, nullptr, nullptr, c.R, epi, cus, c.stream,
                                                          &grid);
    } else {
      st = launch_mfma_pass<TK, LOGITS, kFmtBf16>(c.h, c.K, m0, mp, c.W, nullptr, nullptr, c.R, epi, cus, c.stream,
                                                  &grid);
    }
    if (st != LMH_OK) return st;
    st = finalize(grid, m0, mp);
    if (st != LMH_OK) return st;
  }
  return LMH_OK;
}

bool valu_epi_ok(int64_t M, int64_t K) { return M <= 4 && valu_ok(M, K); }

// Shared argument checks; returns LMH_OK and the resolved path, or a status.
// The default kernel of a call with M hidden rows (mode 0: argmax, else top
// k / logits): VALU up to 4 hidden rows, matrix cores above.  Measured under
// rocprofv3 on the full head and the 16,000-, 32,768- and 52,755-row lists
// at 3, 4, 5 and 8 hidden rows: the VALU kernel is 0.6-4.5% faster at 3
// and 4 rows on every head (one row per step in the ring loop of the
// lists), the matrix cores 2.1-10.6% faster at 5.  The head's size does
// not enter the choice, nor whether its rows are read in place.
int default_path(int64_t M, int64_t K, int mode) {
  if (M > LMH_VALU_AUTO_MAX_M || !(mode == 0 ? valu_ok(M, K) : valu_epi_ok(M, K))) return LMH_PATH_MFMA;
  return LMH_PATH_VALU;
}

int check_common(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R, int mode, int* path) {
  if (!h || !W) return LMH_EINVAL;
  if (M < 1 || M > LMH_MAX_M || !k_ok(K)) return LMH_EINVAL;
  if (R < 1 || R > kMaxRows) return LMH_EINVAL;
  if (!aligned16(h) || !aligned16(W)) return LMH_EINVAL;
  if (*path != LMH_PATH_AUTO && *path != LMH_PATH_VALU && *path != LMH_PATH_MFMA) return LMH_EINVAL;
  if (*path == LMH_PATH_AUTO) *path = default_path(M, K, mode);
  if (*path == LMH_PATH_VALU && !(mode == 0 ? valu_ok(M, K) : valu_epi_ok(M, K))) return LMH_EINVAL;
  return LMH_OK;
}

// Checks for a call over an FP8 head: as check_common, plus K a multiple
// of 16 (16-byte aligned rows of codes) and a 4-byte aligned scale array.
int check_fp8(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const float* wscale, int64_t R,
              int* path) {
  if (!h || !Wq || !wscale || (reinterpret_cast<uintptr_t>(wscale) & 3u) != 0) return LMH_EINVAL;
  if (M < 1 || M > LMH_MAX_M || !k_ok(K) || (K % 16) != 0) return LMH_EINVAL;
  if (R < 1 || R > kMaxRows) return LMH_EINVAL;
  if (!aligned16(h) || !aligned16(Wq)) return LMH_EINVAL;
  if (*path != LMH_PATH_AUTO && *path != LMH_PATH_VALU && *path != LMH_PATH_MFMA) return LMH_EINVAL;
  // Measured on MI355X (full 248,320 x 2,560 head): the matrix-core kernel
  // is faster for every M (98 us at M = 1 against 126 us for VALU, whose
  // code conversions and dot products make it ALU-bound at 1 byte/weight).
  if (*path == LMH_PATH_AUTO) *path = LMH_PATH_MFMA;
  if (*path == LMH_PATH_VALU && M > 4) return LMH_EINVAL;
  return LMH_OK;
}

// Checks for a call over an MXFP4 head: as check_common, plus K a multiple
// of 512 (a batch of the matrix-core kernel is 512 elements, and the scale
// row is a whole number of 16-byte chunks) and a 16-byte aligned scale
// array.  The matrix cores take every M.
int check_mx4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const uint8_t* scales, int64_t R,
              int* path) {
  if (!h || !Wq || !scales) return LMH_EINVAL;
  if (M < 1 || M > LMH_MAX_M || !k_ok(K) || (K % 512) != 0) return LMH_EINVAL;
  if (R < 1 || R > kMaxRows) return LMH_EINVAL;
  if (!aligned16(h) || !aligned16(Wq) || !aligned16(scales)) return LMH_EINVAL;
  if (*path != LMH_PATH_AUTO && *path != LMH_PATH_MFMA) return LMH_EINVAL;
  *path = LMH_PATH_MFMA;
  return LMH_OK;
}

// Checks for a call over an NVFP4 head: as check_mx4 (K a multiple of 512,
// the matrix cores only), plus a 4-byte aligned pointer to the head's fp32
// scale.
int check_nv4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const uint8_t* scales,
              const float* gscale, int64_t R, int* path) {
  if (!gscale || (reinterpret_cast<uintptr_t>(gscale) & 3u) != 0) return LMH_EINVAL;
  return check_mx4(h, M, K, Wq, scales, R, path);
}

// Mean projection-kernel time over `calls` back-to-back launches between two
// events, then one whole call so the outputs hold a result (bench helpers).
// `scales[i]` goes with `heads[i]` for FP8 and MXFP4 heads.
int time_projection(Call c, int nheads, const void* const* heads, const void* const* scales, const Epi& epi,
                    int32_t* out_id, float* out_logit, int calls, double* proj_ms,
                    const float* const* gscales = nullptr) {
  hipEvent_t ev[2] = {nullptr, nullptr};
  int st = LMH_OK;
  for (auto& e : ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      st = hip_fail(r, "hipEventCreate");
      break;
    }
  }
  // single-pass shapes only: the events must bracket projection kernels alone
  const int cap = mfma_lds_rows_fit(c.K, 4, c.fmt);
  if (st == LMH_OK && c.path == LMH_PATH_MFMA && (cap < 1 || c.M > cap)) st = LMH_EINVAL;
  if (st == LMH_OK) st = record(ev[0], c.stream);
  for (int i = 0; i < calls && st == LMH_OK; ++i) {
    Call ci = c;
    ci.W = heads[i % nheads];
    ci.wscale = scales ? scales[i % nheads] : nullptr;
    ci.gscale = gscales ? gscales[i % nheads] : nullptr;
    ci.projection_only = true;
    st = run<0, 1>(ci, epi, 1, out_id, out_logit);
  }
  if (st == LMH_OK) st = record(ev[1], c.stream);
  if (st == LMH_OK) {
    Call c0 = c;
    c0.W = heads[0];
    c0.wscale = scales ? scales[0] : nullptr;
    c0.gscale = gscales ? gscales[0] : nullptr;
    st = run<0, 1>(c0, epi, 1, out_id, out_logit);
  }
  if (st == LMH_OK) {
    const hipError_t r = hipStreamSynchronize(c.stream);
    if (r != hipSuccess) st = hip_fail(r, "hipStreamSynchronize");
  }
  float ms = 0.0f;
  if (st == LMH_OK) {
    const hipError_t r = hipEventElapsedTime(&ms, ev[0], ev[1]);
    if (r != hipSuccess) st = hip_fail(r, "hipEventElapsedTime");
  }
  for (hipEvent_t e : ev)
    if (e) (void)hipEventDestroy(e);
  if (st == LMH_OK) *proj_ms = (double)ms / calls;
  return st;
}

int topk_width(int64_t topk) {
  return topk <= 1 ? 1 : topk <= 2 ? 2 : topk <= 4 ? 4 : topk <= 8 ? 8 : 16;
}

// The top-k run for `topk` (1-16), on the list width that holds it.
int run_topk(const Call& c, const Epi& epi, int64_t topk, int32_t* out_id, float* out_logit) {
  switch (topk_width(topk)) {
    case 1: return run<1, 1>(c, epi, (int)topk, out_id, out_logit);
    case 2: return run<1, 2>(c, epi, (int)topk, out_id, out_logit);
    case 4: return run<1, 4>(c, epi, (int)topk, out_id, out_logit);
    case 8: return run<1, 8>(c, epi, (int)topk, out_id, out_logit);
    default: return run<1, 16>(c, epi, (int)topk, out_id, out_logit);
  }
}

}  // namespace

// Scratch of the allocation-free argmax (draft_project_argmax_noalloc): the
// per-workgroup key slots of up to LMH_MAX_M hidden rows, 256 KiB, in the
// library's own device memory.  Each GPU the library runs on holds its own
// copy until the process ends.  Host code never passes this name to a kernel
// (on the host it is only a handle): scratch_on_device() asks the runtime
// for the address on the current device once and keeps it.
static __device__ __align__(256) unsigned long long scratch[LMH_MAX_M * kMaxGrid];

namespace {

std::mutex g_scratch_mu;
std::vector<std::pair<int, void*>> g_scratch_ptrs;  // (device, address of `scratch` there)

int scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (const auto& dp : g_scratch_ptrs)
    if (dp.first == dev) {
      *out = dp.second;
      return LMH_OK;
    }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (!p) return hip_fail(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
  g_scratch_ptrs.emplace_back(dev, p);
  *out = p;
  return LMH_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int lmhead_trim(const uint16_t* W, int64_t N, int64_t K, const int32_t* ids, int64_t S,
                uint16_t* W_trim, void* stream) {
  if (S < 0 || N < 1 || N > (int64_t)0x7FFFFFFF || !k_ok(K)) return LMH_EINVAL;
  if (S == 0) return LMH_OK;
  if (!W || !ids || !W_trim || !aligned16(W) || !aligned16(W_trim)) return LMH_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> host((size_t)S);
  hipError_t e = hipMemcpyAsync(host.data(), ids, (size_t)S * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(ids)");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  for (int32_t id : host)
    if (id < 0 || (int64_t)id >= N) return LMH_ERANGE;
  int cus = 0;
  int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  const int64_t need = (S + 3) / 4;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(need, (int64_t)cus * 16));
  hipLaunchKernelGGL(gather_rows, dim3(grid), dim3(256), 0, s, W, N, (int)K, ids, S, W_trim);
  e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch gather_rows");
}

size_t draft_project_workspace_bytes(int64_t M) {
  return (M >= 1 && M <= LMH_MAX_M) ? (size_t)M * kMaxGrid * sizeof(unsigned long long) : 0;
}

int draft_project_auto_path(int64_t M, int64_t K) {
  if (M < 1 || M > LMH_MAX_M || !k_ok(K)) return -1;
  return default_path(M, K, 0);
}

int draft_project_auto_path_rows(int64_t M, int64_t K, int64_t R) {
  if (M < 1 || M > LMH_MAX_M || !k_ok(K) || R < 1 || R > kMaxRows) return -1;
  return default_path(M, K, 0);
}

int draft_project_argmax_path(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                              const int32_t* d2t, int32_t* out_id, float* out_logit, void* workspace,
                              size_t workspace_bytes, int path, void* stream) {
  int st = check_common(h, M, K, W, R, 0, &path);
  if (st != LMH_OK) return st;
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  const Call c{h, (int)M, (int)K, W, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run<0, 1>(c, epi, 1, out_id, out_logit);
}

int draft_project_argmax(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                         const int32_t* d2t, int32_t* out_id, float* out_logit, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return draft_project_argmax_path(h, M, K, W, R, d2t, out_id, out_logit, workspace, workspace_bytes,
                                   LMH_PATH_AUTO, stream);
}

int draft_project_argmax_indexed(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t N,
                                 const int32_t* ids, int64_t S, int32_t* out_id, float* out_logit, void* workspace,
                                 size_t workspace_bytes, int path, void* stream) {
  int st = check_common(h, M, K, W, S, 0, &path);
  if (st != LMH_OK) return st;
  if (N < 1 || N > (int64_t)0x7FFFFFFF || !ids || (reinterpret_cast<uintptr_t>(ids) & 3u) != 0) return LMH_EINVAL;
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, W, (int)S, ids, path, static_cast<hipStream_t>(stream)};
  c.indexed = true;
  Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  epi.rowmap = ids;
  epi.nw = (int)N;
  return run<0, 1>(c, epi, 1, out_id, out_logit);
}

size_t draft_project_topk_workspace_bytes(int64_t M, int64_t topk) {
  if (M < 1 || M > LMH_MAX_M || topk < 1 || topk > LMH_MAX_TOPK) return 0;
  return (size_t)M * kMaxGrid * topk_width(topk) * sizeof(unsigned long long);
}

// Output and workspace checks of a top-k call.
static int check_topk_io(int64_t M, int64_t topk, const int32_t* out_id, const float* out_logit,
                         const void* workspace, size_t workspace_bytes) {
  if (topk < 1 || topk > LMH_MAX_TOPK || !out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_topk_workspace_bytes(M, topk)) return LMH_EWORKSPACE;
  return LMH_OK;
}

int draft_project_topk(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                       const int32_t* d2t, int64_t topk, int32_t* out_id, float* out_logit, void* workspace,
                       size_t workspace_bytes, int path, void* stream) {
  int st = check_common(h, M, K, W, R, 1, &path);
  if (st != LMH_OK) return st;
  if ((st = check_topk_io(M, topk, out_id, out_logit, workspace, workspace_bytes)) != LMH_OK) return st;
  const Call c{h, (int)M, (int)K, W, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run_topk(c, epi, topk, out_id, out_logit);
}

int draft_project_logits(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                         const int32_t* d2t, int64_t N, float* out, int path, void* stream) {
  int st = check_common(h, M, K, W, R, 2, &path);
  if (st != LMH_OK) return st;
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u) != 0) return LMH_EINVAL;
  const int64_t ncols = d2t ? N : R;
  if (ncols < 1 || ncols > kMaxRows) return LMH_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d2t) {
    // scatter-after-matmul: columns the list does not reach stay -inf
    int cus = 0;
    st = cu_count(&cus);
    if (st != LMH_OK) return st;
    const size_t n = (size_t)M * (size_t)ncols;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)((n + 255) / 256), (int64_t)cus * 8));
    hipLaunchKernelGGL(fill_neg_inf, dim3(grid), dim3(256), 0, s, out, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch fill_neg_inf");
  }
  const Call c{h, (int)M, (int)K, W, (int)R, d2t, path, s};
  const Epi epi{nullptr, out, d2t, ncols, ncols};
  return run<2, 1>(c, epi, 0, nullptr, nullptr);
}

int lmhead_shortlist_overwrite(const uint16_t* W, int64_t N, int64_t K, uint16_t* W_trim, int32_t* d2t,
                               int64_t cap, const int32_t* rows, const int32_t* ids, int64_t n, void* stream) {
  if (n < 0 || n > LMH_MAX_OVERWRITE || N < 1 || N > (int64_t)0x7FFFFFFF || cap < 1 || cap > kMaxRows ||
      !k_ok(K))
    return LMH_EINVAL;
  if (n == 0) return LMH_OK;
  if (!W || !W_trim || !d2t || !rows || !ids || !aligned16(W) || !aligned16(W_trim)) return LMH_EINVAL;
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(W), t0 = reinterpret_cast<uintptr_t>(W_trim);
  const uintptr_t w1 = w0 + (uintptr_t)N * (uintptr_t)K * 2u, t1 = t0 + (uintptr_t)cap * (uintptr_t)K * 2u;
  if (t0 < w1 && w0 < t1) return LMH_EINVAL;  // W_trim must not overlap W
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n + 3) / 4, (int64_t)cus * 16));
  hipLaunchKernelGGL(overwrite_rows, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), W, N, (int)K,
                     W_trim, d2t, cap, rows, ids, (int)n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch overwrite_rows");
}

int lmhead_shortlist_union(const int32_t* a, int64_t na, const int32_t* b, int64_t nb, int64_t N, int32_t* out,
                           int64_t out_cap, int32_t* counts, void* stream) {
  if (na < 0 || nb < 0 || na > kMaxRows || nb > kMaxRows || N < 1 || N > kUnionMaxVocab) return LMH_EINVAL;
  if (!counts || (na > 0 && !a) || (nb > 0 && !b) || ((na + nb) > 0 && !out) || out_cap < na + nb)
    return LMH_EINVAL;
  const size_t lds = (size_t)2 * (size_t)((N + 31) / 32) * 4;
  allow_full_lds((const void*)union_ids);
  hipLaunchKernelGGL(union_ids, dim3(1), dim3(kUnionThreads), lds, static_cast<hipStream_t>(stream), a, (int)na, b,
                     (int)nb, (int)N, out, counts);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch union_ids");
}

int lmhead_quantize_fp8(const uint16_t* W, int64_t R, int64_t K, uint8_t* Wq, float* scale, void* stream) {
  if (R < 0 || R > kMaxRows || !k_ok(K) || (K % 16) != 0) return LMH_EINVAL;
  if (R == 0) return LMH_OK;
  if (!W || !Wq || !scale || !aligned16(W) || !aligned16(Wq) || (reinterpret_cast<uintptr_t>(scale) & 3u) != 0)
    return LMH_EINVAL;
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((R + 3) / 4, (int64_t)cus * 16));
  hipLaunchKernelGGL(quantize_rows_fp8, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), W, (int)R,
                     (int)K, Wq, scale);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch quantize_rows_fp8");
}

int draft_project_argmax_fp8(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const float* scale,
                             int64_t R, const int32_t* d2t, int32_t* out_id, float* out_logit, void* workspace,
                             size_t workspace_bytes, int path, void* stream) {
  int st = check_fp8(h, M, K, Wq, scale, R, &path);
  if (st != LMH_OK) return st;
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, Wq, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scale;
  c.fmt = kFmtFp8;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run<0, 1>(c, epi, 1, out_id, out_logit);
}

int draft_project_topk_fp8(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const float* scale,
                           int64_t R, const int32_t* d2t, int64_t topk, int32_t* out_id, float* out_logit,
                           void* workspace, size_t workspace_bytes, int path, void* stream) {
  int st = check_fp8(h, M, K, Wq, scale, R, &path);
  if (st != LMH_OK) return st;
  if (path != LMH_PATH_MFMA) return LMH_EINVAL;  // top k over an FP8 head: matrix cores only
  if ((st = check_topk_io(M, topk, out_id, out_logit, workspace, workspace_bytes)) != LMH_OK) return st;
  Call c{h, (int)M, (int)K, Wq, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scale;
  c.fmt = kFmtFp8;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run_topk(c, epi, topk, out_id, out_logit);
}

int draft_project_topk_mxfp4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const uint8_t* scales,
                             int64_t R, const int32_t* d2t, int64_t topk, int32_t* out_id, float* out_logit,
                             void* workspace, size_t workspace_bytes, int path, void* stream) {
  int st = check_mx4(h, M, K, Wq, scales, R, &path);
  if (st != LMH_OK) return st;
  if ((st = check_topk_io(M, topk, out_id, out_logit, workspace, workspace_bytes)) != LMH_OK) return st;
  Call c{h, (int)M, (int)K, Wq, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scales;
  c.fmt = kFmtMx4;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run_topk(c, epi, topk, out_id, out_logit);
}

int64_t lmhead_mxfp4_scale_bytes(int64_t R, int64_t K) {
  if (R < 0 || R > kMaxRows || !k_ok(K) || (K % 32) != 0) return -1;
  return (R + 15) / 16 * ((K / 32 + 15) / 16) * 256;
}

int lmhead_mxfp4_tile_scales(const uint8_t* src, int64_t R, int64_t K, uint8_t* scales, void* stream) {
  if (R < 0 || R > kMaxRows || !k_ok(K) || (K % 32) != 0) return LMH_EINVAL;
  if (R == 0) return LMH_OK;
  if (!src || !scales) return LMH_EINVAL;
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  const int64_t n = R * (K / 32);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, (int64_t)cus * 16));
  hipLaunchKernelGGL(tile_block_scales<16>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), src, (int)R,
                     (int)(K / 32), scales);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch tile_mxfp4_scales");
}

int lmhead_quantize_mxfp4(const uint16_t* W, int64_t R, int64_t K, uint8_t* Wq, uint8_t* scales, void* stream) {
  if (R < 0 || R > kMaxRows || !k_ok(K) || (K % 32) != 0) return LMH_EINVAL;
  if (R == 0) return LMH_OK;
  if (!W || !Wq || !scales || !aligned16(W) || !aligned16(Wq)) return LMH_EINVAL;
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((R + 3) / 4, (int64_t)cus * 16));
  hipLaunchKernelGGL(quantize_rows_mxfp4, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), W, (int)R,
                     (int)K, Wq, scales);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch quantize_rows_mxfp4");
}

int draft_project_argmax_mxfp4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const uint8_t* scales,
                               int64_t R, const int32_t* d2t, int32_t* out_id, float* out_logit, void* workspace,
                               size_t workspace_bytes, int path, void* stream) {
  int st = check_mx4(h, M, K, Wq, scales, R, &path);
  if (st != LMH_OK) return st;
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, Wq, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scales;
  c.fmt = kFmtMx4;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run<0, 1>(c, epi, 1, out_id, out_logit);
}

int64_t lmhead_nvfp4_scale_bytes(int64_t R, int64_t K) {
  if (R < 0 || R > kMaxRows || !k_ok(K) || (K % 16) != 0) return -1;
  return (R + 15) / 16 * ((K / 16 + 31) / 32) * 512;
}

int lmhead_nvfp4_tile_scales(const uint8_t* src, int64_t R, int64_t K, uint8_t* scales, void* stream) {
  if (R < 0 || R > kMaxRows || !k_ok(K) || (K % 16) != 0) return LMH_EINVAL;
  if (R == 0) return LMH_OK;
  if (!src || !scales) return LMH_EINVAL;
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  const int64_t n = R * (K / 16);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, (int64_t)cus * 16));
  hipLaunchKernelGGL(tile_block_scales<32>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), src, (int)R,
                     (int)(K / 16), scales);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch tile_block_scales");
}

int lmhead_quantize_nvfp4(const uint16_t* W, int64_t R, int64_t K, uint8_t* Wq, uint8_t* scales, float* gscale,
                          void* stream) {
  if (R < 0 || R > kMaxRows || !k_ok(K) || (K % 16) != 0) return LMH_EINVAL;
  if (R == 0) return LMH_OK;
  if (!W || !Wq || !scales || !gscale || !aligned16(W) || !aligned16(Wq) ||
      (reinterpret_cast<uintptr_t>(gscale) & 3u) != 0)
    return LMH_EINVAL;
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n16 = R * K / 8;
  const int agrid = (int)std::max<int64_t>(1, std::min<int64_t>((n16 + 255) / 256, (int64_t)cus * 8));
  const int qgrid = (int)std::max<int64_t>(1, std::min<int64_t>((R + 3) / 4, (int64_t)cus * 16));
  hipLaunchKernelGGL(nvfp4_slot_zero, dim3(1), dim3(64), 0, s, gscale);
  hipLaunchKernelGGL(nvfp4_head_amax, dim3(agrid), dim3(256), 0, s, W, n16, gscale);
  hipLaunchKernelGGL(quantize_rows_nvfp4, dim3(qgrid), dim3(256), 0, s, W, (int)R, (int)K, Wq, scales,
                     static_cast<const float*>(gscale));
  hipLaunchKernelGGL(nvfp4_set_scale, dim3(1), dim3(64), 0, s, gscale);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch NVFP4 quantization");
}

int draft_project_argmax_nvfp4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const uint8_t* scales,
                               const float* gscale, int64_t R, const int32_t* d2t, int32_t* out_id,
                               float* out_logit, void* workspace, size_t workspace_bytes, int path, void* stream) {
  int st = check_nv4(h, M, K, Wq, scales, gscale, R, &path);
  if (st != LMH_OK) return st;
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, Wq, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scales;
  c.gscale = gscale;
  c.fmt = kFmtNv4;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run<0, 1>(c, epi, 1, out_id, out_logit);
}

int draft_project_topk_nvfp4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* Wq, const uint8_t* scales,
                             const float* gscale, int64_t R, const int32_t* d2t, int64_t topk, int32_t* out_id,
                             float* out_logit, void* workspace, size_t workspace_bytes, int path, void* stream) {
  int st = check_nv4(h, M, K, Wq, scales, gscale, R, &path);
  if (st != LMH_OK) return st;
  if ((st = check_topk_io(M, topk, out_id, out_logit, workspace, workspace_bytes)) != LMH_OK) return st;
  Call c{h, (int)M, (int)K, Wq, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scales;
  c.gscale = gscale;
  c.fmt = kFmtNv4;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run_topk(c, epi, topk, out_id, out_logit);
}

int lmhead_bench_time_argmax_nvfp4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* const* heads,
                                   const uint8_t* const* scales, const float* const* gscales, int nheads, int64_t R,
                                   const int32_t* d2t, int32_t* out_id, float* out_logit, void* workspace,
                                   size_t workspace_bytes, int path, int calls, double* proj_ms, void* stream) {
  if (!heads || !scales || !gscales || nheads < 1 || calls < 1 || !proj_ms) return LMH_EINVAL;
  const int path_in = path;
  int st = LMH_OK;
  for (int i = 0; i < nheads; ++i) {
    path = path_in;
    if ((st = check_nv4(h, M, K, heads[i], scales[i], gscales[i], R, &path)) != LMH_OK) return st;
  }
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, heads[0], (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scales[0];
  c.gscale = gscales[0];
  c.fmt = kFmtNv4;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return time_projection(c, nheads, reinterpret_cast<const void* const*>(heads),
                         reinterpret_cast<const void* const*>(scales), epi, out_id, out_logit, calls, proj_ms,
                         gscales);
}

int draft_project_argmax_keys(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                              int64_t row_base, uint64_t* out_key, void* workspace, size_t workspace_bytes,
                              int path, void* stream) {
  int st = check_common(h, M, K, W, R, 0, &path);
  if (st != LMH_OK) return st;
  if (row_base < 0 || row_base > (int64_t)0xFFFFFFFF - R) return LMH_EINVAL;
  if (!out_key || (reinterpret_cast<uintptr_t>(out_key) & 7u) != 0) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, W, (int)R, nullptr, path, static_cast<hipStream_t>(stream)};
  c.row_base = row_base;
  c.out_key = reinterpret_cast<unsigned long long*>(out_key);
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return run<3, 1>(c, epi, 1, nullptr, nullptr);
}

int draft_project_argmax_noalloc(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                                 const int32_t* d2t, int32_t* out_id, float* out_logit, void* stream) {
  int path = LMH_PATH_AUTO;
  int st = check_common(h, M, K, W, R, 0, &path);
  if (st != LMH_OK) return st;
  if (M > LMH_NOALLOC_MAX_M) return LMH_EINVAL;  // the scratch holds LMH_NOALLOC_MAX_M rows of slots
  if (!out_id || !out_logit) return LMH_EINVAL;
  void* slots = nullptr;
  if ((st = scratch_on_device(&slots)) != LMH_OK) return st;
  const Call c{h, (int)M, (int)K, W, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  const Epi epi{static_cast<unsigned long long*>(slots), nullptr, nullptr, 0, 0};
  return run<0, 1>(c, epi, 1, out_id, out_logit);
}

int draft_project_argmax_fused_path(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                                    const int32_t* d2t, int32_t* out_id, float* out_logit, void* state,
                                    size_t state_bytes, int path, void* stream) {
  int st = check_common(h, M, K, W, R, 0, &path);
  if (st != LMH_OK) return st;
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!state || !aligned16(state) || state_bytes < (size_t)LMH_STATE_BYTES) return LMH_EWORKSPACE;
  const Call c{h, (int)M, (int)K, W, (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  Epi epi{nullptr, nullptr, nullptr, 0, 0};
  epi.state = static_cast<char*>(state);
  epi.fold_d2t = d2t;
  epi.out_id = out_id;
  epi.out_logit = out_logit;
  return run<0, 1>(c, epi, 1, out_id, out_logit);
}

int draft_project_argmax_fused(const uint16_t* h, int64_t M, int64_t K, const uint16_t* W, int64_t R,
                               const int32_t* d2t, int32_t* out_id, float* out_logit, void* state,
                               size_t state_bytes, void* stream) {
  return draft_project_argmax_fused_path(h, M, K, W, R, d2t, out_id, out_logit, state, state_bytes,
                                         LMH_PATH_AUTO, stream);
}

const char* lmhead_status_str(int status) {
  switch (status) {
    case LMH_OK: return "ok";
    case LMH_EINVAL: return "invalid argument (shape, null or misaligned pointer)";
    case LMH_ERANGE: return "shortlist id out of range [0, N)";
    case LMH_EWORKSPACE: return "workspace missing, misaligned or too small";
    case LMH_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* lmhead_last_error(void) { return g_last_error; }

int lmhead_bench_sink_words(void) { return kBenchSinkWords; }

int lmhead_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink || bytes == 0 || (bytes % 16) != 0 || !aligned16(src) || grid < 0 || grid > kBenchSinkWords)
    return LMH_EINVAL;
  int cus = 0;
  int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  if (grid == 0) grid = cus;  // one 256-thread workgroup per CU reads fastest
  grid = std::min(grid, kBenchSinkWords);
  hipLaunchKernelGGL(stream_read, dim3(grid), dim3(kBenchThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch stream_read");
}

int lmhead_bench_time_argmax(const uint16_t* h, int64_t M, int64_t K, const uint16_t* const* heads, int nheads,
                             int64_t R, const int32_t* d2t, int32_t* out_id, float* out_logit, void* workspace,
                             size_t workspace_bytes, int path, int calls, double* proj_ms, void* stream) {
  if (!heads || nheads < 1 || calls < 1 || !proj_ms) return LMH_EINVAL;
  const int path_in = path;
  int st = LMH_OK;
  for (int i = 0; i < nheads; ++i) {
    path = path_in;
    if ((st = check_common(h, M, K, heads[i], R, 0, &path)) != LMH_OK) return st;
  }
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  const Call c{h, (int)M, (int)K, heads[0], (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return time_projection(c, nheads, reinterpret_cast<const void* const*>(heads), nullptr, epi, out_id, out_logit,
                         calls, proj_ms);
}

int lmhead_bench_time_argmax_fp8(const uint16_t* h, int64_t M, int64_t K, const uint8_t* const* heads,
                                 const float* const* scales, int nheads, int64_t R, const int32_t* d2t,
                                 int32_t* out_id, float* out_logit, void* workspace, size_t workspace_bytes,
                                 int path, int calls, double* proj_ms, void* stream) {
  if (!heads || !scales || nheads < 1 || calls < 1 || !proj_ms) return LMH_EINVAL;
  const int path_in = path;
  int st = LMH_OK;
  for (int i = 0; i < nheads; ++i) {
    path = path_in;
    if ((st = check_fp8(h, M, K, heads[i], scales[i], R, &path)) != LMH_OK) return st;
  }
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, heads[0], (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scales[0];
  c.fmt = kFmtFp8;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return time_projection(c, nheads, reinterpret_cast<const void* const*>(heads),
                         reinterpret_cast<const void* const*>(scales), epi, out_id, out_logit, calls, proj_ms);
}

int lmhead_bench_time_argmax_mxfp4(const uint16_t* h, int64_t M, int64_t K, const uint8_t* const* heads,
                                   const uint8_t* const* scales, int nheads, int64_t R, const int32_t* d2t,
                                   int32_t* out_id, float* out_logit, void* workspace, size_t workspace_bytes,
                                   int path, int calls, double* proj_ms, void* stream) {
  if (!heads || !scales || nheads < 1 || calls < 1 || !proj_ms) return LMH_EINVAL;
  const int path_in = path;
  int st = LMH_OK;
  for (int i = 0; i < nheads; ++i) {
    path = path_in;
    if ((st = check_mx4(h, M, K, heads[i], scales[i], R, &path)) != LMH_OK) return st;
  }
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, heads[0], (int)R, d2t, path, static_cast<hipStream_t>(stream)};
  c.wscale = scales[0];
  c.fmt = kFmtMx4;
  const Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  return time_projection(c, nheads, reinterpret_cast<const void* const*>(heads),
                         reinterpret_cast<const void* const*>(scales), epi, out_id, out_logit, calls, proj_ms);
}

int lmhead_bench_time_argmax_indexed(const uint16_t* h, int64_t M, int64_t K, const uint16_t* const* heads,
                                     int nheads, int64_t N, const int32_t* ids, int64_t S, int32_t* out_id,
                                     float* out_logit, void* workspace, size_t workspace_bytes, int path, int calls,
                                     double* proj_ms, void* stream) {
  if (!heads || nheads < 1 || calls < 1 || !proj_ms) return LMH_EINVAL;
  const int path_in = path;
  int st = LMH_OK;
  for (int i = 0; i < nheads; ++i) {
    path = path_in;
    if ((st = check_common(h, M, K, heads[i], S, 0, &path)) != LMH_OK) return st;
  }
  if (N < 1 || N > (int64_t)0x7FFFFFFF || !ids || (reinterpret_cast<uintptr_t>(ids) & 3u) != 0) return LMH_EINVAL;
  if (!out_id || !out_logit) return LMH_EINVAL;
  if (!workspace || !aligned16(workspace)) return LMH_EWORKSPACE;
  if (workspace_bytes < draft_project_workspace_bytes(M)) return LMH_EWORKSPACE;
  Call c{h, (int)M, (int)K, heads[0], (int)S, ids, path, static_cast<hipStream_t>(stream)};
  c.indexed = true;
  Epi epi{static_cast<unsigned long long*>(workspace), nullptr, nullptr, 0, 0};
  epi.rowmap = ids;
  epi.nw = (int)N;
  return time_projection(c, nheads, reinterpret_cast<const void* const*>(heads), nullptr, epi, out_id, out_logit,
                         calls, proj_ms);
}

int lmhead_bench_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if (!src || !dst || (bytes % 16) != 0 || !aligned16(src) || !aligned16(dst) || grid < 0) return LMH_EINVAL;
  int cus = 0;
  int st = cu_count(&cus);
  if (st != LMH_OK) return st;
  if (grid == 0) grid = cus * 8;
  hipLaunchKernelGGL(copy16, dim3(grid), dim3(kBenchThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LMH_OK : hip_fail(e, "launch copy16");
}

}  // extern "C"
