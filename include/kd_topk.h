/*
 * kd_topk.h -- teacher top-K cache producer of libkdchunk.so (gfx950).
 *
 * The loss trains a student against a cache made once from the teacher: per
 * position, the ids and logits of the 100 most probable teacher tokens
 * (agentlenshq.com page "LLMのための効率的な知識蒸留…", section
 * "1. Top-K Logit Cachingによるオフライン蒸留"; aivibenews.ru page
 * "Дистилляция LLM на одной GPU…", section "Два приёма").  This entry point
 * makes that record from a teacher's last hidden states and output projection
 * without the positions x vocabulary grid: logits z_iv = W_T[v] . h_i are
 * formed on matrix cores one chunk of rows at a time, and per row the K
 * largest are kept.  Softmax is increasing, so they are the K most probable
 * tokens.  Readings: the record lists them largest logit first; equal logits
 * are ordered by the lower id (which also decides which of several equal
 * logits at the K-th place is kept).
 *
 * Conventions as in kd_chunked.h (device pointers, caller-owned buffers and
 * workspace, asynchronous on `stream`, host-side argument checks that
 * enqueue nothing on error).
 */
#ifndef KD_TOPK_H
#define KD_TOPK_H

#include <stddef.h>
#include <stdint.h>

#include "kd_chunked.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace kd_teacher_topk needs: per chunk 16 sampled maxima per
 * row and vocabulary tile, a threshold and a list of up to 8192 candidate
 * logits per row (8 bytes each), and the chunk's hidden states copied in
 * k tiles for the projection passes.  Uses d, v, k, chunk and x_dtype of
 * `prob` (t_dtype is ignored); independent of n.  Returns 0 for an invalid
 * problem. */
size_t kd_teacher_topk_workspace_size(const kd_problem* prob);

/* Teacher top-K record.
 *   H       [n,d]  x_dtype   teacher hidden states
 *   W       [v,d]  x_dtype   teacher output projection
 *   ids     [n,k]  int32     out: token ids, largest logit first, ties by id
 *   logits  [n,k]  float     out: their logits -- the projection's own fp32
 *                            accumulator values
 *   overflow_rows [1] int    out (optional, NULL = skip): set to the number of
 *                            rows whose candidate list overflowed
 * Per chunk: a projection pass recording, per row, the largest logit of each
 * 24-column slice of every 384-column vocabulary tile; per row the K-th
 * largest of those maxima as a threshold (they are K logits of the row, so
 * every top-K logit is at or above it); a second projection pass collecting
 * the logits at or above the threshold (about K per row for spread logits);
 * a sort of each row's candidates.  The record is exact for every row with at
 * most 8192 candidates -- always when v < 24 k -- ; a row with more (thousands
 * of logits tied at the top) gets the best K of 8192 of them and is counted in
 * *overflow_rows.
 * Returns KD_OK or an error status (nothing enqueued on error). */
int kd_teacher_topk(const kd_problem* prob, const void* H, const void* W, int32_t* ids, float* logits,
                    int* overflow_rows, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KD_TOPK_H */
