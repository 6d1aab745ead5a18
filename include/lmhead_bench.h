/*
 * lmhead_bench.h -- measurement and test entry points of liblmhead.so, kept
 * apart from the product boundary in lmhead.h: a forced kernel choice for
 * the argmax, plain streaming kernels that find the practical HBM ceiling and
 * scale hardware counters, and timers of the projection kernel alone.  None
 * of them belongs in a decode loop.  Conventions, status codes and buffer
 * rules are those of lmhead.h.
 */
#ifndef LMHEAD_BENCH_H
#define LMHEAD_BENCH_H

#include "lmhead.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * draft_project_argmax_path -- draft_project_argmax with the kernel chosen
 * by the caller (LMH_PATH_*), for tests and measurement.  LMH_PATH_VALU
 * accepts M <= 8 with M * ceil(K / 512) <= 40; LMH_PATH_MFMA accepts every
 * shape draft_project_argmax accepts.  Other shapes give LMH_EINVAL.
 */
int draft_project_argmax_path(const uint16_t* h, int64_t M, int64_t K,
                              const uint16_t* W, int64_t R,
                              const int32_t* d2t,
                              int32_t* out_id, float* out_logit,
                              void* workspace, size_t workspace_bytes,
                              int path, void* stream);

/*
 * Measurement support (not part of the projection): plain streaming kernels
 * used to find the practical HBM ceiling and to scale hardware counters.
 *
 * lmhead_bench_stream_read: reads `bytes` (a nonzero multiple of 16,
 *   16-byte aligned `src`) with 16-byte non-temporal loads, two groups of
 *   four in flight per lane, and writes one 32-bit checksum word per
 *   workgroup into `sink` (at least lmhead_bench_sink_words() words).
 *   grid 0 = one 256-thread workgroup per CU, the fastest shape measured.
 * lmhead_bench_copy: dst[0:bytes] = src[0:bytes] (16-byte multiples/aligned).
 * `grid` = workgroups to launch (0 = the library's default).
 */
int lmhead_bench_sink_words(void);
int lmhead_bench_stream_read(const void* src, size_t bytes, uint32_t* sink,
                             int grid, void* stream);
int lmhead_bench_copy(const void* src, void* dst, size_t bytes, int grid,
                      void* stream);

/*
 * lmhead_bench_time_argmax: mean duration of the projection kernel of
 *   draft_project_argmax_path.  Between two HIP events on `stream` the
 *   library launches that kernel `calls` times back to back, launch i over
 *   heads[i % nheads] (a host array of device pointers, each [R, K]), with
 *   no fold in between; *proj_ms = elapsed milliseconds / calls.  Then one
 *   whole call over heads[0] writes out_id / out_logit.  Only shapes that
 *   take a single projection launch are accepted (LMH_EINVAL otherwise).
 *   Synchronizes; for measurement, not for the decode loop.  Other
 *   arguments as for draft_project_argmax_path.
 */
int lmhead_bench_time_argmax(const uint16_t* h, int64_t M, int64_t K,
                             const uint16_t* const* heads, int nheads,
                             int64_t R, const int32_t* d2t,
                             int32_t* out_id, float* out_logit,
                             void* workspace, size_t workspace_bytes,
                             int path, int calls, double* proj_ms,
                             void* stream);

/*
 * lmhead_bench_time_argmax_fp8: the same over FP8 heads (draft_project_
 *   argmax_fp8): launch i uses heads[i % nheads] with scales[i % nheads].
 */
int lmhead_bench_time_argmax_fp8(const uint16_t* h, int64_t M, int64_t K,
                                 const uint8_t* const* heads,
                                 const float* const* scales, int nheads,
                                 int64_t R, const int32_t* d2t,
                                 int32_t* out_id, float* out_logit,
                                 void* workspace, size_t workspace_bytes,
                                 int path, int calls, double* proj_ms,
                                 void* stream);

/*
 * lmhead_bench_time_argmax_mxfp4: the same over MXFP4 heads (draft_project_
 *   argmax_mxfp4): launch i uses heads[i % nheads] with scales[i % nheads].
 */
int lmhead_bench_time_argmax_mxfp4(const uint16_t* h, int64_t M, int64_t K,
                                   const uint8_t* const* heads,
                                   const uint8_t* const* scales, int nheads,
                                   int64_t R, const int32_t* d2t,
                                   int32_t* out_id, float* out_logit,
                                   void* workspace, size_t workspace_bytes,
                                   int path, int calls, double* proj_ms,
                                   void* stream);

/*
 * lmhead_bench_time_argmax_indexed: the same for draft_project_argmax_
 *   indexed: launch i reads full head heads[i % nheads] ([N, K] each)
 *   through the one id list `ids`.
 */
int lmhead_bench_time_argmax_indexed(const uint16_t* h, int64_t M, int64_t K,
                                     const uint16_t* const* heads, int nheads,
                                     int64_t N, const int32_t* ids, int64_t S,
                                     int32_t* out_id, float* out_logit,
                                     void* workspace, size_t workspace_bytes,
                                     int path, int calls, double* proj_ms,
                                     void* stream);

/*
 * draft_project_argmax_fused_path: draft_project_argmax_fused with the
 *   projection kernel chosen by `path` (LMH_PATH_VALU or LMH_PATH_MFMA; see
 *   draft_project_argmax_path), so that both kernels' single-launch
 *   epilogues can be checked and timed.
 */
int draft_project_argmax_fused_path(const uint16_t* h, int64_t M, int64_t K,
                                    const uint16_t* W, int64_t R,
                                    const int32_t* d2t,
                                    int32_t* out_id, float* out_logit,
                                    void* state, size_t state_bytes,
                                    int path, void* stream);

/*
 * lmhead_bench_time_argmax_nvfp4: the same over NVFP4 heads (draft_project_
 *   argmax_nvfp4): launch i uses heads[i % nheads] with scales[i % nheads]
 *   and gscales[i % nheads].
 */
int lmhead_bench_time_argmax_nvfp4(const uint16_t* h, int64_t M, int64_t K,
                                   const uint8_t* const* heads,
                                   const uint8_t* const* scales,
                                   const float* const* gscales, int nheads,
                                   int64_t R, const int32_t* d2t,
                                   int32_t* out_id, float* out_logit,
                                   void* workspace, size_t workspace_bytes,
                                   int path, int calls, double* proj_ms,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_BENCH_H */
