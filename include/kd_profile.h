/*
 * kd_profile.h -- optional per-kernel timing of libkdchunk.so.
 *
 * When enabled, every kernel that kd_chunked_fwd / kd_chunked_bwd enqueue is
 * bracketed by two HIP events recorded on the caller's stream (the stream the
 * kernel runs on), so elapsed times are measured on the device timeline.  Off
 * by default; the hot path then records nothing.  Intended for benchmarks and
 * profiling, not for concurrent use from several host threads.
 */
#ifndef KD_PROFILE_H
#define KD_PROFILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel kinds, in launch order within a chunk. */
typedef enum kd_kernel_kind {
  KD_K_PREP = 0,     /* teacher renormalisation, id sort, tile ranges          */
  KD_K_FWD_PROJ = 1, /* forward projection + online max/sum-exp + gather       */
  KD_K_MERGE = 2,    /* lse merge, row loss                                    */
  KD_K_LOSS = 3,     /* running-loss fold                                      */
  KD_K_BWD_DZ = 4,   /* backward recomputation + closed-form dZ                */
  KD_K_BWD_DH = 5,   /* dH = dZ W (split over V)                               */
  KD_K_DH_REDUCE = 6,/* fixed-order sum of the dH split partials               */
  KD_K_BWD_DW = 7,   /* dW += dZ^T H                                           */
  KD_K_DZ_CACHED = 8,/* single-call path: dZ from the forward's kept logits    */
  KD_K_TOPK_MAXIMA = 9,     /* top-K producer: projection + sampled row maxima   */
  KD_K_TOPK_THRESHOLD = 10, /* top-K producer: per-row threshold                 */
  KD_K_TOPK_COLLECT = 11,   /* top-K producer: projection + candidate collection */
  KD_K_TOPK_SELECT = 12,    /* top-K producer: per-row sort of the candidates     */
  KD_K_H_TRANSPOSE = 13,    /* backward: H_c transposed for the dW GEMM          */
  KD_K_H_TILE = 14,         /* H_c copied in k tiles for the projections         */
  KD_K_COUNT = 15
} kd_kernel_kind;

/* Turn event recording on (1) or off (0).  Either way the accumulated
 * totals are cleared.  Returns 0, or 7 (KD_ERR_LAUNCH) if events cannot be
 * created. */
int kd_profile_enable(int on);

/* Wait for every recorded event pair, add its elapsed time to the per-kind
 * totals, then report kind `kind`: its name, total milliseconds and number of
 * launches since kd_profile_enable.  Returns 0, or 2 (KD_ERR_SHAPE) when
 * `kind` is out of range; any output pointer may be NULL. */
int kd_profile_read(int kind, const char** name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* KD_PROFILE_H */
