/*
 * A C program that uses the library through include/lmhead.h alone, with no
 * Python and no torch: it owns its device buffers (hipMalloc), gathers a
 * shortlist at load (lmhead_trim), runs the argmax over the trimmed head
 * with d2t and over the full head without it (draft_project_argmax), the
 * same two steps as single launches (draft_project_argmax_fused, on a state
 * it zeroes once and checks is zero again) and without a workspace
 * (draft_project_argmax_noalloc), and checks that a rejected call writes
 * nothing.  The test that runs it compares its outputs with the fp64 oracle.
 *
 *   lmhead_consumer N K S M W.bin ids.bin h.bin out.bin
 *
 * W.bin: N*K bf16 bit patterns (uint16); ids.bin: S int32; h.bin: M*K
 * uint16.  out.bin receives, per hidden row, the trimmed call's id (int32)
 * and logit (float32), then the full-head call's, then the single launch's
 * over the trimmed head, then the no-workspace call's over the full head.
 */
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lmhead.h"

static int fail(const char* what, const char* detail) {
  fprintf(stderr, "lmhead_consumer: %s: %s\n", what, detail);
  return 1;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_));   \
  } while (0)

#define LMH_OK_OR_FAIL(call)                                           \
  do {                                                                 \
    int s_ = (call);                                                   \
    if (s_ != LMH_OK) {                                                \
      fprintf(stderr, "lmhead_consumer: %s: %s %s\n", #call,           \
              lmhead_status_str(s_), lmhead_last_error());             \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static int read_file(const char* path, void* dst, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) return fail("open", path);
  size_t got = fread(dst, 1, bytes, f);
  fclose(f);
  return got == bytes ? 0 : fail("short read", path);
}

int main(int argc, char** argv) {
  if (argc != 9) {
    fprintf(stderr, "usage: %s N K S M W.bin ids.bin h.bin out.bin\n", argv[0]);
    return 2;
  }
  const int64_t N = atoll(argv[1]), K = atoll(argv[2]), S = atoll(argv[3]), M = atoll(argv[4]);
  const size_t wb = (size_t)(N * K) * sizeof(uint16_t), ib = (size_t)S * sizeof(int32_t);
  const size_t hb = (size_t)(M * K) * sizeof(uint16_t), tb = (size_t)(S * K) * sizeof(uint16_t);
  uint16_t* w = malloc(wb);
  int32_t* ids = malloc(ib);
  uint16_t* h = malloc(hb);
  int32_t* out_id = malloc(4 * (size_t)M * sizeof(int32_t));
  float* out_logit = malloc(4 * (size_t)M * sizeof(float));
  if (!w || !ids || !h || !out_id || !out_logit) return fail("malloc", "host buffers");
  if (read_file(argv[5], w, wb) || read_file(argv[6], ids, ib) || read_file(argv[7], h, hb)) return 1;

  uint16_t *d_w, *d_trim, *d_h;
  int32_t *d_ids, *d_id;
  float* d_logit;
  void *d_ws, *d_state;
  const size_t wsb = draft_project_workspace_bytes(M);
  if (wsb == 0) return fail("draft_project_workspace_bytes", "rejected M");
  HIP_OK(hipMalloc((void**)&d_w, wb));
  HIP_OK(hipMalloc((void**)&d_trim, tb));
  HIP_OK(hipMalloc((void**)&d_h, hb));
  HIP_OK(hipMalloc((void**)&d_ids, ib));
  HIP_OK(hipMalloc((void**)&d_id, 4 * (size_t)M * sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_logit, 4 * (size_t)M * sizeof(float)));
  HIP_OK(hipMalloc(&d_ws, wsb));
  HIP_OK(hipMalloc(&d_state, LMH_STATE_BYTES));
  HIP_OK(hipMemset(d_state, 0, LMH_STATE_BYTES));   /* once, when the state is allocated */
  HIP_OK(hipMemcpy(d_w, w, wb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_ids, ids, ib, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_h, h, hb, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  /* load time: the shortlist rows, range-checked */
  LMH_OK_OR_FAIL(lmhead_trim(d_w, N, K, d_ids, S, d_trim, stream));
  /* a step over the trimmed head (ids mapped back through d2t = ids), then
     one over the full head (no d2t: the row is the vocabulary id) */
  LMH_OK_OR_FAIL(draft_project_argmax(d_h, M, K, d_trim, S, d_ids, d_id, d_logit, d_ws, wsb, stream));
  LMH_OK_OR_FAIL(draft_project_argmax(d_h, M, K, d_w, N, NULL, d_id + M, d_logit + M, d_ws, wsb, stream));
  /* the trimmed step again as single launches (twice: the first call
     leaves the state zero for the second), and the full-head step with no
     workspace */
  for (int rep = 0; rep < 2; ++rep)
    LMH_OK_OR_FAIL(draft_project_argmax_fused(d_h, M, K, d_trim, S, d_ids, d_id + 2 * M, d_logit + 2 * M, d_state,
                                              LMH_STATE_BYTES, stream));
  LMH_OK_OR_FAIL(draft_project_argmax_noalloc(d_h, M, K, d_w, N, NULL, d_id + 3 * M, d_logit + 3 * M, stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(out_id, d_id, 4 * (size_t)M * sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out_logit, d_logit, 4 * (size_t)M * sizeof(float), hipMemcpyDeviceToHost));
  unsigned char state_after[LMH_STATE_BYTES];
  HIP_OK(hipMemcpy(state_after, d_state, LMH_STATE_BYTES, hipMemcpyDeviceToHost));
  for (int i = 0; i < LMH_STATE_BYTES; ++i)
    if (state_after[i] != 0) return fail("draft_project_argmax_fused", "the state is not zero after the call");
  /* same kernels, same sums: the single launch equals the two-kernel call
     and the no-workspace call the ordinary one, bit for bit */
  if (memcmp(out_id, out_id + 2 * M, (size_t)M * sizeof(int32_t)) != 0 ||
      memcmp(out_logit, out_logit + 2 * M, (size_t)M * sizeof(float)) != 0)
    return fail("draft_project_argmax_fused", "differs from draft_project_argmax");
  if (memcmp(out_id + M, out_id + 3 * M, (size_t)M * sizeof(int32_t)) != 0 ||
      memcmp(out_logit + M, out_logit + 3 * M, (size_t)M * sizeof(float)) != 0)
    return fail("draft_project_argmax_noalloc", "differs from draft_project_argmax");

  /* a call the library rejects (M = 0) returns LMH_EINVAL before any launch
     and leaves the outputs alone */
  int s = draft_project_argmax(d_h, 0, K, d_w, N, NULL, d_id, d_logit, d_ws, wsb, stream);
  if (s != LMH_EINVAL) return fail("M = 0", lmhead_status_str(s));
  int32_t after[1];
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(after, d_id, sizeof(int32_t), hipMemcpyDeviceToHost));
  if (after[0] != out_id[0]) return fail("M = 0", "the rejected call wrote an output");

  FILE* f = fopen(argv[8], "wb");
  if (!f) return fail("open", argv[8]);
  for (int64_t m = 0; m < 4 * M; ++m) {
    fwrite(&out_id[m], sizeof(int32_t), 1, f);
    fwrite(&out_logit[m], sizeof(float), 1, f);
  }
  fclose(f);
  HIP_OK(hipStreamDestroy(stream));
  hipFree(d_w);
  hipFree(d_trim);
  hipFree(d_h);
  hipFree(d_ids);
  hipFree(d_id);
  hipFree(d_logit);
  hipFree(d_ws);
  hipFree(d_state);
  free(w);
  free(ids);
  free(h);
  free(out_id);
  free(out_logit);
  printf("lmhead_consumer: ok (%s)\n", lmhead_status_str(LMH_OK));
  return 0;
}
