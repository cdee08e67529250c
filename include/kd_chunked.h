/*
 * kd_chunked.h -- C ABI of the fused chunked top-K KL distillation loss
 * (libkdchunk.so, AMD MI355X / gfx950).
 *
 * The operation.  A student projects hidden states H [n,d] through its output
 * projection W [v,d] to logits z_i = W h_i over the full vocabulary; a cached
 * teacher record gives, per position, K token ids and K teacher logits.  The
 * loss is, summed over unmasked positions,
 *
 *     L = sum_i m_i sum_k p_ik (log p_ik - z_{i,t_ik} + lse_i),
 *     p_i = softmax over the K cached teacher logits, lse_i = log sum_v e^{z_iv}
 *
 * i.e. KL(teacher || student) on the K cached ids (reading of the pages: the
 * teacher record is renormalised over its K entries, temperature 1, sum
 * reduction).  Sources: the offline top-100 teacher cache (agentlenshq.com
 * page "LLMのための効率的な知識蒸留…", section "1. Top-K Logit Cachingによる
 * オフライン蒸留"); the fused chunked loss that owns the output projection,
 * projects one chunk of positions at a time, folds it into a running loss and
 * discards it, and recomputes each chunk in the backward pass (same page,
 * section "2. Fused Chunked KL Loss"; aivibenews.ru page "Дистилляция LLM на
 * одной GPU…", section "Два приёма"); the closed-form gradient the aihot.vn
 * page "Tối ưu hóa chi phí chưng cất tri thức…" mentions in section "Mô hình
 * học sinh thu được":  dL/dz_iv = m_i (s_i q_iv - sum_k p_ik [t_ik = v]),
 * s_i = sum_k p_ik, q_i = softmax(z_i).
 *
 * Temperature (kd_problem.tau), a loss variant.  The aihot.vn page (section
 * "Mô hình học sinh thu được") reports ablations over the choice of loss
 * without defining any; reading: the usual temperature-scaled distillation
 * loss.  With tau != 1 the teacher and student distributions
 * are softmaxes of a / tau and z / tau and the loss is multiplied by tau^2:
 *     L = tau^2 sum_i m_i sum_k p_ik (log p_ik - z_{i,t_ik} / tau + lse_i),
 *     lse_i = log sum_v e^{z_iv / tau},
 *     dL/dz_iv = tau m_i (s_i q_iv - sum_k p_ik [t_ik = v]), q_i = softmax(z_i / tau).
 * tau = 1 (or 0, read as 1) is the loss above, with the same arithmetic.
 *
 * Conventions for every entry point:
 *  - all tensor pointers are DEVICE pointers on the current HIP device, dense
 *    row-major, and 16-byte aligned;
 *  - the caller owns and allocates every buffer, including the workspace
 *    (size from kd_chunked_workspace_size); the library allocates nothing,
 *    never synchronises, and only enqueues work on `stream` (a hipStream_t,
 *    NULL = the null stream).  Calls are asynchronous with respect to the host;
 *  - one workspace must not be used by two calls in flight at once;
 *  - arguments are checked on the host before anything is enqueued; on any
 *    error the call returns a non-zero kd_status and enqueues nothing;
 *  - no exception crosses the ABI.
 * Preconditions that are NOT checked: on unmasked rows the ids lie in [0,v);
 * the backward gets the same inputs as the forward that produced `lse`.
 * An id outside [0,v) (negative, or >= v) matches no vocabulary entry: its
 * gathered logit reads as 0 and it adds no -p term to dZ, while its p still
 * counts in sum_k p_ik and sum_k p_ik log p_ik (memory stays safe; the loss
 * is no longer a KL).  Repeated ids within a row are handled term by term.
 * Non-finite inputs propagate to the outputs; no error is raised.
 */
#ifndef KD_CHUNKED_H
#define KD_CHUNKED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kd_status {
  KD_OK = 0,
  KD_ERR_NULL = 1,      /* a required pointer is NULL                          */
  KD_ERR_SHAPE = 2,     /* n < 0, d not in [1, 65536], v < 1,
                           k not in [1, min(v,256)], chunk < 1, v > 16777215,
                           tau neither 0 nor in [0.01, 100], dw_chunks not in
                           [0, 8], or a 32-bit tile offset limit: v > 4194048
                           or chunk * max(1, dw_chunks) > 4194296 for bf16,
                           v > 2097024 or that product > 2097144 for fp32,
                           or more than 8388600 projection tiles per chunk:
                           ceil(chunk / 256) * ceil(v / 384)                   */
  KD_ERR_DTYPE = 3,     /* x_dtype / t_dtype not a kd_dtype                     */
  KD_ERR_ALIGN = 4,     /* d % 8 != 0, or a pointer not 16-byte aligned         */
  KD_ERR_WORKSPACE = 5, /* workspace_bytes < kd_chunked_workspace_size(prob)    */
  KD_ERR_DEVICE = 6,    /* the current device is not a gfx950                   */
  KD_ERR_LAUNCH = 7     /* the HIP runtime reported an error while enqueueing  */
} kd_status;

typedef enum kd_dtype { KD_F32 = 0, KD_BF16 = 1 } kd_dtype;

typedef struct kd_problem {
  int64_t n;       /* positions (batch*seq flattened), >= 0                     */
  int32_t d;       /* hidden size, multiple of 8, at most 65536                  */
  int32_t v;       /* vocabulary size                                            */
  int32_t k;       /* teacher top-K, 1 <= k <= min(v, 256)                       */
  int32_t chunk;   /* rows per chunk (the only tuning knob), >= 1               */
  int32_t x_dtype; /* kd_dtype of H and W (the projection's compute dtype)      */
  int32_t t_dtype; /* kd_dtype of the teacher logits                            */
  float tau;       /* temperature: 0 or 1 = the plain loss, else in [0.01, 100]  */
  int32_t dw_chunks; /* chunks the backward takes at once, 0..8 (0 = 1): it
                        runs each of its kernels once per group of that many
                        chunks (the workspace holds their dZ), so dW is read
                        and written once per group instead of per chunk.
                        loss, lse and dH do not change (dH is summed over the
                        V slices of one chunk's split either way); dW only in
                        the grouping of its fp32 additions, and not at all
                        when chunk is a multiple of the k tile (32 rows for
                        bf16, 16 for fp32) */
} kd_problem;

/* Bytes of workspace the fwd and bwd calls need for `prob`.  Depends on
 * (d, v, k, chunk, dtypes) only, never on n: the per-chunk logit grid lives
 * in it, the N x V grid never exists.  Returns 0 for an invalid problem. */
size_t kd_chunked_workspace_size(const kd_problem* prob);

/* Static string naming a status code (never NULL). */
const char* kd_status_string(int status);

/* Forward.  Walks the n rows in chunks of prob->chunk rows; per chunk it
 * renormalises the teacher record, runs the projection H_c W^T on matrix
 * cores with an online per-row max / sum-of-exponentials and a gather of the
 * student logits at the K teacher ids, then folds the chunk into the running
 * loss.  The forward keeps no dZ, so when the workspace (sized for the
 * backward's chunk of dZ) has room it runs up to 8 consecutive chunks per
 * pass, at most 65536 rows: each kernel launch then covers them all.  The
 * outputs are the same bit for bit (every row is computed the same way, and
 * the running loss adds chunk-sized slices in order).
 *   H        [n,d]  x_dtype   hidden states
 *   W        [v,d]  x_dtype   output projection (nn.Linear [out,in] layout)
 *   t_ids    [n,k]  int32     cached teacher token ids
 *   t_logits [n,k]  t_dtype   cached teacher logits (any order)
 *   mask     [n]    uint8     0 = position ignored (its teacher record is not
 *                             read), NULL = every position counts
 *   loss     [1]    float     out: L (fixed-order fp64 reduction, then fp32)
 *   lse      [n]    float     out: lse_i (of z_i / tau) for every row, masked
 *                             ones included
 *   row_loss [n]    float     out (optional, NULL = skip): tau^2 m_i KL_i
 *   zg       [n,k]  float     out (optional, NULL = skip): z_{i,t_ik}, the
 *                             projection's own fp32 accumulator value; 0 on
 *                             masked rows
 * Returns KD_OK or an error status (nothing enqueued on error). */
int kd_chunked_fwd(const kd_problem* prob, const void* H, const void* W,
                   const int32_t* t_ids, const void* t_logits, const uint8_t* mask,
                   float* loss, float* lse, float* row_loss, float* zg,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Backward.  Recomputes each chunk's logits, forms
 *   dZ_iv = g tau m_i (s_i exp(z_iv / tau - lse_i) - sum_k p_ik [t_ik = v])
 * in fp32 and rounds it once to x_dtype (the -p terms are applied before the
 * rounding), then dH_c = dZ_c W and dW += dZ_c^T H_c with fp32 accumulation.
 *   H, W, t_ids, t_logits, mask   as for the forward (same values, same tau)
 *   lse       [n]   float    the forward's lse output
 *   grad_loss [1]   float    device scalar g (upstream gradient), NULL = 1
 *   dH        [n,d] float    out, overwritten; masked rows are exactly zero
 *   dW        [v,d] float    in/out, accumulated (+=); prior contents kept
 * Returns KD_OK or an error status (nothing enqueued on error). */
int kd_chunked_bwd(const kd_problem* prob, const void* H, const void* W,
                   const int32_t* t_ids, const void* t_logits, const uint8_t* mask,
                   const float* lse, const float* grad_loss, float* dH, float* dW,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace kd_chunked_fwd_bwd needs for `prob`: the fwd/bwd
 * workspace plus one chunk of fp32 logits (chunk rounded up to 32 rows, x
 * 384*ceil(v/384) floats, plus 256 bytes per 32 rows).
 * Independent of n.  Returns 0 for an invalid problem. */
size_t kd_chunked_fwd_bwd_workspace_size(const kd_problem* prob);

/* Forward and backward in one call, for callers that know the upstream
 * gradient g before the forward runs.  Same chunk walk and same results as
 * kd_chunked_fwd followed by kd_chunked_bwd (loss, lse, dH and dW bit for
 * bit), except that each chunk's fp32 logits are kept in the workspace by the
 * forward projection and dZ is formed from them, instead of recomputing the
 * projection: 6 n d v flops instead of 8, for one chunk of logits more
 * workspace.  The pages' design recomputes, and note that the extra backward
 * projection costs speed at short context (aihot.vn page "Tối ưu hóa chi phí
 * chưng cất tri thức…", section "Điều này thay đổi những gì trong thực tế";
 * agentlenshq.com page, section "パフォーマンスとメモリのベンチマーク").
 *   H, W, t_ids, t_logits, mask   as for the forward
 *   grad_loss [1]   float    device scalar g, NULL = 1
 *   loss      [1]   float    out
 *   lse       [n]   float    out
 *   dH        [n,d] float    out, overwritten; masked rows are exactly zero
 *   dW        [v,d] float    in/out, accumulated (+=)
 *   workspace >= kd_chunked_fwd_bwd_workspace_size(prob) bytes
 * Returns KD_OK or an error status (nothing enqueued on error). */
int kd_chunked_fwd_bwd(const kd_problem* prob, const void* H, const void* W,
                       const int32_t* t_ids, const void* t_logits, const uint8_t* mask,
                       const float* grad_loss, float* loss, float* lse, float* dH, float* dW,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch kd_chunked_fwd_noalloc holds per GPU. */
#define KD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Forward without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same computation, arguments and results as kd_chunked_fwd
 * (loss, lse, row_loss and zg bit for bit), but the chunk workspace is a
 * file-scope device array of KD_NOALLOC_SCRATCH_BYTES inside the library
 * instead of a caller buffer; the call allocates and frees nothing.
 *  - Limit: one chunk's forward regions must fit the array, about
 *      chunk * (12 k + 10 ceil(v / 384) + 64 ceil(d x / 64) + 18) bytes
 *    (x = 2 for bf16, 4 for fp32), plus up to 256 bytes for each of its 11
 *    regions' alignment, e.g.
 *    chunk 2048 at d = 2880, v = 201088, k = 100, bf16: 25 MB.  A larger
 *    problem returns KD_ERR_WORKSPACE and enqueues nothing; pick a smaller
 *    chunk.  Consecutive chunks share a pass (one launch per kernel) when
 *    they fit together.
 *  - Each GPU has one such array, shared by every call on it; it keeps the
 *    last call's contents, none of which a later call reads.  Calls that
 *    overlap on one GPU (other streams, other host threads) race on it:
 *    serialise them.
 *  - The first call on a device looks up the array's device address
 *    (hipGetSymbolAddress); make that call before any graph capture.
 * Returns KD_OK or an error status (nothing enqueued on error). */
int kd_chunked_fwd_noalloc(const kd_problem* prob, const void* H, const void* W,
                           const int32_t* t_ids, const void* t_logits, const uint8_t* mask,
                           float* loss, float* lse, float* row_loss, float* zg, void* stream);

/* Debug check of the teacher record against what the loss assumes of it.
 * The cache holds, per position, the K most probable teacher tokens
 * (agentlenshq.com page, section "1. Top-K Logit Cachingによるオフライン
 * 蒸留"): K distinct ids of the vocabulary.  The loss calls do not check
 * this; an id outside [0,v) matches no vocabulary entry (see above).
 * This call counts, over unmasked rows only (mask NULL = every row):
 *   out[0]  rows with an id outside [0, prob->v)
 *   out[1]  rows with an id that occurs more than once in the row
 *   out[2]  the smallest row counted in out[0], or -1
 *   out[3]  the smallest row counted in out[1], or -1
 *   t_ids   [n, k] int32     mask  [n] uint8 or NULL (rows with 0 skipped)
 *   out     int64 [4], 8-byte aligned, written (prior contents ignored)
 * Only prob->n, v and k are used (d, chunk and the dtypes are still
 * checked).  The ids of masked rows are never read.  No workspace.
 * Returns KD_OK, KD_ERR_NULL (out NULL, or t_ids NULL with n > 0),
 * KD_ERR_SHAPE (as for the loss calls, or n > 4 (2^31 - 1)), KD_ERR_ALIGN
 * (out), KD_ERR_DEVICE or KD_ERR_LAUNCH; nothing is enqueued on error. */
int kd_chunked_validate(const kd_problem* prob, const int32_t* t_ids, const uint8_t* mask,
                        int64_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KD_CHUNKED_H */
