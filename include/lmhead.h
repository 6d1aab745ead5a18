/*
 * lmhead.h -- skinny draft-head vocabulary projection for AMD Instinct MI355X
 * (gfx950): load-time shortlist row gather, and a fused projection + argmax +
 * d2t id map for a handful of hidden rows.
 *
 * The operation.  A speculative-decoding draft head scores a bf16 hidden
 * state of width K against every row of the bf16 LM-head weight and proposes
 * the best-scoring token ("What I was testing", krisbailey.com/articles/
 * shortlist-mtp: hidden width 2,560, 248,320 head rows, one to three rows per
 * step).  A shortlisted head scores only the rows of a list of ids, cut from
 * the full head once at load ("Two ways to run it", zone-1.cobraproject.com
 * "Masked MTP drafts"); the winning list index goes back to a vocabulary id
 * through a d2t table, as in EAGLE-3's draft-to-target map (same section).
 * The argmax is reduced where it is computed instead of gathering logits
 * ("Re-running the comparison fairly", krisbailey.com).
 *
 * Conventions for every call below:
 *  - bf16 values travel as their raw 16-bit patterns (uint16_t).
 *  - Every pointer is a DEVICE pointer on the calling thread's current HIP
 *    device, unless it is documented otherwise.
 *  - Matrices are row-major and contiguous: element (r, k) of an [R, K]
 *    matrix is at index r * K + k.
 *  - `stream` is a hipStream_t passed as void*, created on the current
 *    device; NULL means the null stream.  Launch settings (CU count,
 *    occupancy) are those of the current device.
 *    Work is queued on `stream` and the call returns without waiting, except
 *    where a call says it synchronizes.  A call that neither synchronizes
 *    nor allocates only launches kernels, so it may be captured in a HIP
 *    graph (stream capture) and replayed; make one eager call with the same
 *    shapes first, so that the per-kernel launch settings are cached outside
 *    the capture.
 *  - The caller owns every buffer.  The library never allocates or frees
 *    device memory and keeps no device state between calls, except the
 *    static slot array of draft_project_argmax_noalloc (loaded with the
 *    library; nothing in it carries from one call to the next).
 *  - Return value: an lmh_status code.  A call that returns LMH_EINVAL,
 *    LMH_ERANGE or LMH_EWORKSPACE has launched nothing and written nothing.
 *    LMH_EHIP means a HIP runtime call failed; lmhead_last_error() gives its
 *    text.  A fault inside a kernel surfaces, as usual in HIP, as an error
 *    of a later synchronizing call.
 */
#ifndef LMHEAD_H
#define LMHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMH_OK = 0,
  LMH_EINVAL = 1,      /* bad shape, null or misaligned pointer            */
  LMH_ERANGE = 2,      /* a shortlist id outside [0, N)                     */
  LMH_EWORKSPACE = 3,  /* workspace missing, misaligned or too small        */
  LMH_EHIP = 4         /* a HIP runtime call failed                         */
} lmh_status;

/* Shape limits.  K must be a multiple of 8 so a row is a whole number of
 * 16-byte vectors. */
#define LMH_MAX_M 32
#define LMH_MIN_K 8
#define LMH_MAX_K 8192
#define LMH_MAX_R ((1 << 30) - 1)  /* rows of a head or entries of a list */
#define LMH_MAX_TOPK 16
#define LMH_MAX_OVERWRITE 65536      /* entries per lmhead_shortlist_overwrite call */
#define LMH_MAX_UNION_VOCAB 524288   /* N of lmhead_shortlist_union (two LDS bitmaps) */

/* Kernel choice of the calls that take a `path` argument. */
#define LMH_PATH_AUTO 0
#define LMH_PATH_VALU 1  /* hidden rows in registers, packed bf16 dot products */
#define LMH_PATH_MFMA 2  /* hidden rows in LDS, 16x16x32 bf16 matrix-core tiles */

/*
 * lmhead_trim -- build the shortlisted head: W_trim[i, :] = W[ids[i], :].
 *
 * The head weight is cut once at load from a list of token ids ("Two ways to
 * run it", zone-1.cobraproject.com "Masked MTP drafts"; the id list file of
 * "Build the draft vocabulary from your own text", ai-muninn.com).
 *
 *  W       [N, K] bf16, 16-byte aligned.
 *  ids     [S] int32, each in [0, N); order is kept (row i <-> ids[i]);
 *          duplicates are allowed.  The same array serves as the d2t table
 *          of draft_project_argmax on W_trim.
 *  W_trim  [S, K] bf16, 16-byte aligned, written completely (bit copy).
 *  S = 0 is a no-op.  N >= 1, K as above.
 *
 * Synchronizes `stream` once: ids are copied to the host and range-checked
 * before the gather is queued, so an id outside [0, N) returns LMH_ERANGE
 * and nothing is read out of bounds.  This is a load-time call.
 */
int lmhead_trim(const uint16_t* W, int64_t N, int64_t K,
                const int32_t* ids, int64_t S,
                uint16_t* W_trim, void* stream);

/*
 * draft_project_workspace_bytes -- bytes of workspace draft_project_argmax
 * needs for M hidden rows: one 8-byte slot per hidden row per workgroup of
 * the projection kernel (M * 8 KiB; 0 if M is out of range).
 */
size_t draft_project_workspace_bytes(int64_t M);

/*
 * draft_project_argmax -- the draft head's greedy proposal, one draft step:
 * score the hidden rows against every row of the head and keep the best
 * (krisbailey.com/articles/shortlist-mtp, "What I was testing": a 2,560-wide
 * hidden state against the LM head, one row per draft step and three per
 * MTP2 verify step); over a trimmed head the winning row maps back to its
 * vocabulary id through d2t (zone-1.cobraproject.com "Masked MTP drafts",
 * "Two ways to run it").  For each hidden row m:
 *     idx[m]       = the smallest r maximizing  L[m, r] = sum_k h[m, k] * W[r, k]
 *     out_id[m]    = d2t ? d2t[idx[m]] : idx[m]
 *     out_logit[m] = L[m, idx[m]]
 * with bf16 products and fp32 accumulation.  The logit is the raw dot
 * product (no bias, scale or temperature: greedy drafting).
 *
 *  h          [M, K] bf16, 16-byte aligned, 1 <= M <= LMH_MAX_M.
 *  W          [R, K] bf16, 16-byte aligned: the full head (R = N) or a
 *             trimmed head from lmhead_trim (R = S).  1 <= R <= LMH_MAX_R
 *             (2^30 - 1).
 *  d2t        [R] int32 or NULL.  For a trimmed head pass the ids given to
 *             lmhead_trim (absolute vocabulary ids); NULL returns row indices.
 *  out_id     [M] int32.  -1 only if no logit of the row is ordered (NaN).
 *  out_logit  [M] float.
 *  workspace  at least draft_project_workspace_bytes(M) bytes, 16-byte
 *             aligned.  Scratch for one call: its contents on entry do not
 *             matter and are undefined afterwards.  Calls ordered on one
 *             stream may share a workspace; calls that may run concurrently
 *             need separate ones.
 *
 * Never synchronizes and never allocates.  Queues two kernels: the fused
 * projection + running argmax, whose workgroups each leave their best
 * (logit, row) per hidden row in the workspace, and a small kernel that
 * folds those, maps the winner through d2t and writes the outputs.  When the
 * matrix-core path cannot hold all M hidden rows in LDS at once (M * K above
 * about 75 Ki at K = 2,560) the rows are split over several such pairs.
 * Inputs with NaN or Inf give an unspecified (but in-bounds) result.
 */
int draft_project_argmax(const uint16_t* h, int64_t M, int64_t K,
                         const uint16_t* W, int64_t R,
                         const int32_t* d2t,
                         int32_t* out_id, float* out_logit,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * draft_project_argmax_fused -- draft_project_argmax as ONE kernel launch
 * (per pass of hidden rows), with a small persistent state in place of the
 * scratch workspace.  Same operation (see draft_project_argmax: the passages
 * cited there), arguments, outputs, kernel choice and errors as
 * draft_project_argmax, except:
 *
 *  state        LMH_STATE_BYTES bytes, 16-byte aligned, ALL ZERO before
 *               the first call that uses it: zero it once when it is
 *               allocated.  Every call leaves it all zero again (a call
 *               whose kernel faulted does not).  Calls ordered on one stream
 *               may share a state; calls that may run concurrently need
 *               separate ones; nothing else may write it.
 *  state_bytes  its size; a NULL or misaligned state, or a size below
 *               LMH_STATE_BYTES, is LMH_EWORKSPACE.
 *
 * Never synchronizes and never allocates.  The projection kernel's
 * workgroups merge their best keys into the state with 64-bit atomic
 * maxima at agent scope, in two levels (16 groups of workgroups, then the
 * groups), each level closed by a ticket (a relaxed atomic add taken only
 * after the wave's maxima are acknowledged); the workgroup that takes the
 * last ticket decodes the winners, maps them through d2t, writes the
 * outputs and clears the state.  No fence, no fold kernel.
 */
#define LMH_STATE_BYTES 8192
int draft_project_argmax_fused(const uint16_t* h, int64_t M, int64_t K,
                               const uint16_t* W, int64_t R,
                               const int32_t* d2t,
                               int32_t* out_id, float* out_logit,
                               void* state, size_t state_bytes,
                               void* stream);

/*
 * draft_project_argmax_noalloc -- draft_project_argmax for callers that
 * cannot allocate device memory or hold a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * operation, outputs, kernels and errors as draft_project_argmax (library's
 * own kernel choice), without the workspace arguments: the per-workgroup
 * key slots live in a static array in the library's device memory (256 KiB
 * per GPU, held until the process ends), whose address on each device is
 * looked up once, on the first call on that device.
 *
 *  M          1 .. LMH_NOALLOC_MAX_M (= LMH_MAX_M, the rows the array holds);
 *             more is LMH_EINVAL.
 * Never allocates and never synchronizes.  The array is shared by every
 * call on the device and its contents on entry do not matter (nothing in it
 * needs clearing), but calls that may overlap on one GPU -- on different
 * streams, or from several threads without ordering -- race on it: order
 * them on one stream, or use draft_project_argmax with separate workspaces.
 */
#define LMH_NOALLOC_MAX_M LMH_MAX_M
int draft_project_argmax_noalloc(const uint16_t* h, int64_t M, int64_t K,
                                 const uint16_t* W, int64_t R,
                                 const int32_t* d2t,
                                 int32_t* out_id, float* out_logit,
                                 void* stream);

/*
 * draft_project_argmax_keys -- the argmax of one slice of a head, as keys
 * that combine across slices: the unit of work of one GPU when the head is
 * split by vocabulary rows across GPUs, as a tensor-parallel lm_head is
 * (ai-muninn.com "Qwen3.8-Flash-Next on two DGX Sparks", kernel table under
 * "Decode runs at 80-87% of memory bandwidth": the 124,160-row shard of the
 * 248,320-row head at TP = 2), or when a shortlist is split evenly across
 * ranks ("Build the draft vocabulary from your own text", same page).  The
 * argmax is still reduced where it is computed; only M keys leave a slice.
 *
 * For each hidden row m, with idx[m] the smallest maximizing row of the
 * slice W (as for draft_project_argmax):
 *     out_key[m] = (ord(L[m, idx[m]]) << 32) | (0xFFFFFFFF - (row_base + idx[m]))
 * where ord is the order-preserving map of an fp32 value to 32 bits
 * (negative values: all bits inverted; others: sign bit set; -0 taken as
 * +0).  The unsigned maximum of the keys of all slices of a head is the
 * whole head's key: its largest logit, and among equal logits the smallest
 * global row.  Decode it as row = 0xFFFFFFFF - (key & 0xFFFFFFFF) and the
 * logit from the high word, then map the row through the head's d2t (for a
 * split list, row is the position in the whole list).  0 means no ordered
 * logit (NaN inputs).
 *
 *  W          [R, K] bf16, the slice (rows row_base .. row_base + R - 1 of
 *             the whole head or list), 16-byte aligned.
 *  row_base   >= 0, row_base + R <= 2^32 - 1.
 *  out_key    [M] uint64 (device, 8-byte aligned).
 *  workspace, path, h, M, K, R: as for draft_project_argmax_path.
 * Never synchronizes and never allocates; queues the projection and a
 * small fold kernel.  Errors as for draft_project_argmax.
 */
int draft_project_argmax_keys(const uint16_t* h, int64_t M, int64_t K,
                              const uint16_t* W, int64_t R, int64_t row_base,
                              uint64_t* out_key,
                              void* workspace, size_t workspace_bytes,
                              int path, void* stream);

/*
 * draft_project_topk -- the `topk` best rows per hidden row instead of one:
 * several draft candidates per position, for sampling or a draft tree.  They
 * are the top of the same scores whose argmax is the greedy draft.
 *
 *  out_id     [M, topk] int32: d2t[row] (or row), best first; among equal
 *             logits the smaller row comes first.  Positions past R hold -1.
 *  out_logit  [M, topk] float, matching; -inf past R.
 *  topk       1 .. LMH_MAX_TOPK.
 *  workspace  draft_project_topk_workspace_bytes(M, topk) bytes, 16-byte
 *             aligned; contents irrelevant, as for draft_project_argmax.
 *  path       LMH_PATH_AUTO, or LMH_PATH_VALU (M <= 4 with
 *             M * ceil(K / 512) <= 40) / LMH_PATH_MFMA.
 * Other arguments, synchronization and errors as for draft_project_argmax.
 */
size_t draft_project_topk_workspace_bytes(int64_t M, int64_t topk);
int draft_project_topk(const uint16_t* h, int64_t M, int64_t K,
                       const uint16_t* W, int64_t R,
                       const int32_t* d2t, int64_t topk,
                       int32_t* out_id, float* out_logit,
                       void* workspace, size_t workspace_bytes,
                       int path, void* stream);

/*
 * draft_project_logits -- every logit, for consumers that sample or rescore.
 * Without d2t: out is [M, R], out[m * R + r] = L[m, r].  With d2t (the
 * shortlist's vocabulary ids), the logits are scattered into vocabulary
 * space: out is [M, N], out[m * N + d2t[r]] = L[m, r] and every other entry
 * is -inf, so an id off the list can never be chosen -- EAGLE-3's d2t map,
 * scatter-after-matmul ("Two ways to run it", zone-1.cobraproject.com
 * "Masked MTP drafts").  d2t entries outside [0, N) are skipped; with
 * duplicate ids one of the rows' logits is kept.
 *
 *  out   float, 4-byte aligned, [M, R] or [M, N] as above.  No workspace.
 *  path  as for draft_project_topk.
 * Queues a -inf fill (with d2t) and the projection; never synchronizes.
 */
int draft_project_logits(const uint16_t* h, int64_t M, int64_t K,
                         const uint16_t* W, int64_t R,
                         const int32_t* d2t, int64_t N, float* out,
                         int path, void* stream);

/*
 * lmhead_quantize_fp8 -- load-time FP8 copy of a bf16 head (W or W_trim),
 * one scale per row.  The pages convert weights that every decode step
 * reads to FP8 E4M3 at load, which halves the bytes read (ai-muninn.com
 * "Qwen3.8-Flash-Next on two DGX Sparks": "The costs: a 69% smaller KV pool
 * and FP8 GDN weights", and the kernel notes under "Decode runs at 80-87%
 * of memory bandwidth").  Granularity and rounding are readings:
 *   scale[r] = max_k |W[r, k]| / 448 in fp32, or 1 for an all-zero row;
 *   Wq[r, k] = the OCP E4M3 code nearest to W[r, k] / scale[r] (fp32
 *   division), ties to the even code, magnitudes above 448 saturating.
 * The quantized head stands for decode(Wq[r, k]) * scale[r].
 *
 *  W      [R, K] bf16 (device, 16-byte aligned).  K a multiple of 16.
 *  Wq     [R, K] uint8 (device, 16-byte aligned, caller-allocated).
 *  scale  [R] float (device, 4-byte aligned, caller-allocated).
 * R = 0 is a no-op.  Asynchronous on `stream`; allocates nothing.
 * Returns LMH_EINVAL for a bad shape, a null or misaligned pointer.
 */
int lmhead_quantize_fp8(const uint16_t* W, int64_t R, int64_t K,
                        uint8_t* Wq, float* scale, void* stream);

/*
 * draft_project_argmax_fp8 -- draft_project_argmax over an FP8 head from
 * lmhead_quantize_fp8: out_logit[m] = max_r scale[r] * sum_k h[m, k] *
 * decode(Wq[r, k]), fp32 sums of exact products, then one multiply by the
 * row's scale; out_id as for draft_project_argmax (first row among equal
 * maxima, mapped through d2t).  The head streams at 1 byte per weight.
 *
 *  Wq, scale  as written by lmhead_quantize_fp8 (R rows).  K a multiple
 *             of 16, Wq 16-byte aligned, scale 4-byte aligned.
 *  path       LMH_PATH_AUTO (matrix cores for every M), LMH_PATH_VALU
 *             (M <= 4) or LMH_PATH_MFMA.
 * Other arguments, workspace, synchronization and errors as for
 * draft_project_argmax_path.
 */
int draft_project_argmax_fp8(const uint16_t* h, int64_t M, int64_t K,
                             const uint8_t* Wq, const float* scale, int64_t R,
                             const int32_t* d2t,
                             int32_t* out_id, float* out_logit,
                             void* workspace, size_t workspace_bytes,
                             int path, void* stream);

/*
 * lmhead_quantize_mxfp4 -- load-time 4-bit copy of a bf16 head (W or W_trim)
 * in OCP MXFP4: E2M1 elements in blocks of 32 consecutive elements of a
 * row, each block with one power-of-two scale stored as an E8M0 code.  The
 * pages requantize the trimmed draft head to a 4-bit format at no measured
 * acceptance cost (zone-1.cobraproject.com "Masked MTP drafts", the section
 * of that name); their format is NVFP4, the 4-bit format of their GPUs,
 * and MXFP4 is the one MI355X converts in hardware.  Rounding and scale
 * follow the MX specification's conversion:
 *   s = floor(log2(max |block|)) - 2, clamped to [-127, 127], 0 for a block
 *       of zeros; the stored code is s + 127;
 *   code = the E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives)
 *       nearest to W / 2^s, ties to the even code, above 6 saturating.
 * The quantized head stands for decode(code) * 2^s.
 *
 *  W       [R, K] bf16 (device, 16-byte aligned); K a multiple of 32.
 *  Wq      [R, K / 2] uint8 (device, 16-byte aligned): two codes per byte,
 *          element 2i in the low nibble of byte i.
 *  scales  lmhead_mxfp4_scale_bytes(R, K) bytes (device) in the tiled scale
 *          layout: with nb = ceil(K / 512), the scale of row r, block j
 *          (elements 32 j .. 32 j + 31) is byte
 *            ((r / 16 * nb + j / 16) * 16 + r % 16) * 16 + j % 16,
 *          so that the scales one 16-row tile needs for 512 elements are
 *          256 contiguous bytes.  Bytes of the padding (rows R .. up to a
 *          multiple of 16, blocks past K / 32) are not written.
 * R = 0 is a no-op.  Asynchronous on `stream`; allocates nothing.
 * Returns LMH_EINVAL for a bad shape, a null or misaligned pointer.
 */
int lmhead_quantize_mxfp4(const uint16_t* W, int64_t R, int64_t K,
                          uint8_t* Wq, uint8_t* scales, void* stream);

/*
 * lmhead_mxfp4_scale_bytes -- size in bytes of the tiled scale array of an
 * [R, K] MXFP4 head: ceil(R / 16) * ceil(K / 512) * 256.  Host only; -1 for
 * a bad shape (R outside [0, LMH_MAX_R], K not a positive multiple of 32 up
 * to the library's limit).
 */
int64_t lmhead_mxfp4_scale_bytes(int64_t R, int64_t K);

/*
 * lmhead_mxfp4_tile_scales -- row-major E8M0 block scales [R, K / 32] (the
 * order of the MX specification, for a head quantized elsewhere) into the
 * tiled scale layout of lmhead_quantize_mxfp4.
 *
 *  src     [R, K / 32] uint8 (device).
 *  scales  lmhead_mxfp4_scale_bytes(R, K) bytes (device); padding bytes are
 *          not written.
 * R = 0 is a no-op.  Asynchronous on `stream`; allocates nothing.
 * Returns LMH_EINVAL for a bad shape or a null pointer.
 */
int lmhead_mxfp4_tile_scales(const uint8_t* src, int64_t R, int64_t K, uint8_t* scales, void* stream);

/*
 * draft_project_argmax_mxfp4 -- draft_project_argmax over an MXFP4 head
 * from lmhead_quantize_mxfp4: out_logit[m] = max_r sum_k h[m, k] *
 * decode(Wq[r, k]) * 2^(s[r, k / 32]), fp32 sums of exact
 * products (every E2M1 value times a power of two is a bf16 number); out_id
 * as for draft_project_argmax (first row among equal maxima, mapped
 * through d2t).  The head streams at 0.53 bytes per weight (codes and
 * scales).  The matrix cores take every M.
 *
 *  Wq, scales as written by lmhead_quantize_mxfp4 (R rows; scales in the
 *             tiled layout, lmhead_mxfp4_scale_bytes(R, K) bytes, all of
 *             which may be read); K a multiple of 512; Wq and scales
 *             16-byte aligned.
 *  path       LMH_PATH_AUTO or LMH_PATH_MFMA.
 * Other arguments, workspace, synchronization and errors as for
 * draft_project_argmax_path.
 */
int draft_project_argmax_mxfp4(const uint16_t* h, int64_t M, int64_t K,
                               const uint8_t* Wq, const uint8_t* scales,
                               int64_t R, const int32_t* d2t,
                               int32_t* out_id, float* out_logit,
                               void* workspace, size_t workspace_bytes,
                               int path, void* stream);

/*
 * lmhead_quantize_nvfp4 -- load-time copy of a bf16 head (W or W_trim) in
 * NVFP4, the 4-bit format the pages requantize the trimmed draft head to at
 * no measured acceptance cost (zone-1.cobraproject.com "Masked MTP drafts",
 * the section of that name) and score a drafter's candidates through
 * ("Update (November 2026)", same page): E2M1 elements (0, 0.5, 1, 1.5, 2,
 * 3, 4, 6 and negatives), one E4M3 scale per 16 consecutive elements of a
 * row, and one fp32 scale g for the whole head, so that element k of row r
 * stands for e2m1(code) x e4m3(block scale) x g.  The pages do not give the
 * conversion; the one used here (every division correctly rounded in fp32):
 *   g          = max |W| / 2688 (448 x 6), or 1 for a head of zeros;
 *   block code = the E4M3 value nearest to (amax_block / 6) / g, ties to the
 *                even code, above 448 saturating to 448;
 *   code       = the E2M1 value nearest to W / (decode(block code) x g),
 *                ties to the even code, above 6 saturating to 6; a signed
 *                zero where decode(block code) x g is 0.
 *
 *  W       [R, K] bf16 (device, 16-byte aligned); K a multiple of 16.
 *  Wq      [R, K / 2] uint8 (device, 16-byte aligned): two codes per byte,
 *          element 2i in the low nibble of byte i.
 *  scales  lmhead_nvfp4_scale_bytes(R, K) bytes (device) of E4M3 block
 *          scale codes in the tiled layout: with ng = ceil(K / 512), the
 *          scale of row r, block j (elements 16 j .. 16 j + 15) is byte
 *            ((r / 16 * ng + j / 32) * 16 + r % 16) * 32 + j % 32,
 *          so the scales one 16-row tile needs for 512 elements are 512
 *          contiguous bytes.  Padding bytes are not written.
 *  gscale  one float (device, 4-byte aligned): receives g.  While the call
 *          runs it holds the head's largest magnitude; read it after the
 *          call's work has completed on `stream`.
 * R = 0 is a no-op.  Asynchronous on `stream` (four small kernels);
 * allocates nothing.  Returns LMH_EINVAL for a bad shape, a null or
 * misaligned pointer.
 */
int lmhead_quantize_nvfp4(const uint16_t* W, int64_t R, int64_t K,
                          uint8_t* Wq, uint8_t* scales, float* gscale,
                          void* stream);

/*
 * lmhead_nvfp4_scale_bytes -- size in bytes of the tiled block-scale array
 * of an [R, K] NVFP4 head: ceil(R / 16) * ceil(K / 512) * 512.  Host only;
 * -1 for a bad shape (R outside [0, LMH_MAX_R], K not a positive multiple of
 * 16 up to the library's limit).
 */
int64_t lmhead_nvfp4_scale_bytes(int64_t R, int64_t K);

/*
 * lmhead_nvfp4_tile_scales -- row-major E4M3 block scales [R, K / 16] (a
 * head quantized elsewhere, with its own g) into the tiled layout of
 * lmhead_quantize_nvfp4.
 *
 *  src     [R, K / 16] uint8 (device).
 *  scales  lmhead_nvfp4_scale_bytes(R, K) bytes (device); padding bytes are
 *          not written.
 * R = 0 is a no-op.  Asynchronous on `stream`; allocates nothing.
 * Returns LMH_EINVAL for a bad shape or a null pointer.
 */
int lmhead_nvfp4_tile_scales(const uint8_t* src, int64_t R, int64_t K, uint8_t* scales, void* stream);

/*
 * draft_project_argmax_nvfp4 -- draft_project_argmax over an NVFP4 head
 * from lmhead_quantize_nvfp4: out_logit[m] = max_r g * sum_k h[m, k] *
 * e2m1(Wq[r, k]) * e4m3(scale of block k / 16 of row r).  Each element
 * times its block scale is a normal f16 number (at most 6 significant bits)
 * and each hidden row is taken as f16 times a power of two that puts its
 * largest magnitude in [2^15, 2^16), so every product of an element and a
 * hidden value within 2^29 of its row's largest is exact (a smaller hidden
 * value may be rounded or flushed in f16, an error of at most its own
 * magnitude); the sums are fp32, the power of two comes off exactly and g
 * multiplies each row's sum once.
 * out_id as for draft_project_argmax (first row among equal maxima, mapped
 * through d2t).  The head streams at 0.5625 bytes per weight (codes and
 * block scales).  The matrix cores take every M.
 *
 *  Wq, scales, gscale  as written by lmhead_quantize_nvfp4 (R rows; scales
 *                      in the tiled layout, all of which may be read); K a
 *                      multiple of 512; Wq and scales 16-byte aligned,
 *                      gscale 4-byte aligned.
 *  path                LMH_PATH_AUTO or LMH_PATH_MFMA.
 * Other arguments, workspace, synchronization and errors as for
 * draft_project_argmax.
 */
int draft_project_argmax_nvfp4(const uint16_t* h, int64_t M, int64_t K,
                               const uint8_t* Wq, const uint8_t* scales,
                               const float* gscale, int64_t R,
                               const int32_t* d2t,
                               int32_t* out_id, float* out_logit,
                               void* workspace, size_t workspace_bytes,
                               int path, void* stream);

/*
 * draft_project_topk_fp8, draft_project_topk_mxfp4 -- draft_project_topk
 * over a quantized head: the `topk` best rows of the dequantized FP8 or
 * MXFP4 head per hidden row, best first, mapped through d2t.  The pages
 * take a drafter's candidates from the target's 4-bit head
 * (zone-1.cobraproject.com "Masked MTP drafts", "Update (November 2026)");
 * this is that scoring, several candidates per position.  Logits as for
 * draft_project_argmax_fp8 / _mxfp4; order, ties and padding (positions
 * past R hold id -1 and logit -inf) as for draft_project_topk.
 *
 *  Wq, scale / scales  the head as for draft_project_argmax_fp8 / _mxfp4.
 *  topk                1 to LMH_MAX_TOPK.
 *  workspace           draft_project_topk_workspace_bytes(M, topk) bytes.
 *  path                LMH_PATH_AUTO or LMH_PATH_MFMA (the matrix cores).
 * Errors and synchronization as for draft_project_topk.
 */
int draft_project_topk_fp8(const uint16_t* h, int64_t M, int64_t K,
                           const uint8_t* Wq, const float* scale, int64_t R,
                           const int32_t* d2t, int64_t topk,
                           int32_t* out_id, float* out_logit,
                           void* workspace, size_t workspace_bytes,
                           int path, void* stream);
int draft_project_topk_mxfp4(const uint16_t* h, int64_t M, int64_t K,
                             const uint8_t* Wq, const uint8_t* scales,
                             int64_t R, const int32_t* d2t, int64_t topk,
                             int32_t* out_id, float* out_logit,
                             void* workspace, size_t workspace_bytes,
                             int path, void* stream);

/*
 * draft_project_topk_nvfp4 -- the same over an NVFP4 head (Wq, scales,
 * gscale as for draft_project_argmax_nvfp4): the drafter's candidates
 * scored through the target's NVFP4 head (zone-1.cobraproject.com "Masked
 * MTP drafts", "Update (November 2026)").
 */
int draft_project_topk_nvfp4(const uint16_t* h, int64_t M, int64_t K,
                             const uint8_t* Wq, const uint8_t* scales,
                             const float* gscale, int64_t R,
                             const int32_t* d2t, int64_t topk,
                             int32_t* out_id, float* out_logit,
                             void* workspace, size_t workspace_bytes,
                             int path, void* stream);

/*
 * draft_project_argmax_indexed -- the shortlisted argmax read straight from
 * the full head: for each hidden row m, over the list entries i with
 * ids[i] in [0, N),
 *     best[m]      = the smallest i maximizing  L[m, i] = sum_k h[m, k] *
 *                    W[ids[i], k]   (bf16 products, fp32 sums)
 *     out_id[m]    = ids[best[m]]
 *     out_logit[m] = L[m, best[m]]
 * This is exactly draft_project_argmax over lmhead_trim(W, ids) with d2t =
 * ids, without the trimmed copy: a shortlisted head only picks which head
 * rows the draft scores, and the d2t map gives their ids ("Two ways to run
 * it", zone-1.cobraproject.com "Masked MTP drafts").  It serves when the
 * full head must stay resident anyway (the verifier reads it) and the S x K
 * copy would be extra memory, or when the list changes often; each listed
 * row is still one contiguous K x 2-byte read.
 *
 *  h          [M, K] bf16 (device, 16-byte aligned), 1 <= M <= LMH_MAX_M.
 *  W          [N, K] bf16 (device, 16-byte aligned), the full head;
 *             1 <= N <= 2^31 - 1.
 *  ids        [S] int32 (device, 4-byte aligned), 1 <= S <= LMH_MAX_R, any
 *             order, duplicates allowed.  An entry outside [0, N) is
 *             skipped (never read); if every entry is skipped, out_id = -1
 *             and out_logit is NaN.
 *  out_id, out_logit, workspace: as for draft_project_argmax.
 *  path       LMH_PATH_AUTO, LMH_PATH_VALU (M <= 8 with M * ceil(K / 512)
 *             <= 40) or LMH_PATH_MFMA.
 * Never synchronizes and never allocates.  Errors as for
 * draft_project_argmax_path.
 */
int draft_project_argmax_indexed(const uint16_t* h, int64_t M, int64_t K,
                                 const uint16_t* W, int64_t N,
                                 const int32_t* ids, int64_t S,
                                 int32_t* out_id, float* out_logit,
                                 void* workspace, size_t workspace_bytes,
                                 int path, void* stream);

/*
 * lmhead_shortlist_overwrite -- refresh rows of a trimmed head in place:
 * for each entry i, W_trim[rows[i], :] = W[ids[i], :] and d2t[rows[i]] =
 * ids[i].  This is how escaped ids are learned into spare head rows, the
 * pages' fix for a static trim that misses tokens (zone-1.cobraproject.com
 * "Masked MTP drafts", section "Update (November 2026)", the Gemma 4 31B
 * case): keep
 * W_trim and d2t with room for `cap` rows, project over the first R, write
 * newly seen ids into rows R, R + 1, ... and project over the grown prefix.
 *
 *  W       [N, K] bf16 (device, 16-byte aligned), not overlapping W_trim.
 *  W_trim  [cap, K] bf16 (device, 16-byte aligned), written in place.
 *  d2t     [cap] int32 (device), written in place.
 *  rows, ids  [n] int32 (device), 0 <= n <= LMH_MAX_OVERWRITE.
 * An entry with rows[i] outside [0, cap) or ids[i] outside [0, N) is
 * skipped.  When several valid entries name the same row, the last one
 * wins.  Asynchronous on `stream`; allocates nothing.  Order it against
 * projections that read W_trim on other streams.  LMH_EINVAL for bad
 * sizes, null or misaligned pointers, or overlapping W and W_trim.
 */
int lmhead_shortlist_overwrite(const uint16_t* W, int64_t N, int64_t K,
                               uint16_t* W_trim, int32_t* d2t, int64_t cap,
                               const int32_t* rows, const int32_t* ids,
                               int64_t n, void* stream);

/*
 * lmhead_shortlist_union -- the sorted union of two id lists, on the
 * device (the pages widen a list by merging candidates into it: ai-muninn.com
 * "Qwen3.8-Flash-Next on two DGX Sparks", "Build the draft vocabulary from
 * your own text", where 47,149 ids and 9,749 candidates, 5,606 of them new,
 * give 52,755).
 *
 *  a [na], b [nb]  int32 ids (device), any order, duplicates allowed; ids
 *                  outside [0, N) are ignored.  N <= LMH_MAX_UNION_VOCAB.
 *  out    int32 (device), room for out_cap >= na + nb entries: receives
 *         the union in ascending order, each id once.
 *  counts int32[4] (device): |set a|, |set b|, |set b minus set a|, and
 *         the union's size (the number of entries written to out).
 * Asynchronous on `stream` (one workgroup); allocates nothing.
 */
int lmhead_shortlist_union(const int32_t* a, int64_t na, const int32_t* b,
                           int64_t nb, int64_t N, int32_t* out,
                           int64_t out_cap, int32_t* counts, void* stream);

/* Which kernel draft_project_argmax picks for (M, K): an LMH_PATH_* value
 * (the VALU kernels up to 4 hidden rows where they accept K, the matrix
 * cores above), or -1 if the shape is not accepted.  The same for every
 * head size and for rows read in place through a list. */
int draft_project_auto_path(int64_t M, int64_t K);

/* The same, also checking a head of R rows: -1 if (M, K, R) is not
 * accepted (R outside [1, LMH_MAX_R]). */
int draft_project_auto_path_rows(int64_t M, int64_t K, int64_t R);

/* Static text for a status code. */
const char* lmhead_status_str(int status);

/* Text of the last HIP error seen by this thread (empty if none). */
const char* lmhead_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_H */
