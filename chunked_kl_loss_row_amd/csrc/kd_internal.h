// Internal interface between the C ABI (kd_api.hip) and the kernels
// (kd_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kd {

// Tile shapes fixed at compile time (they also fix the workspace layout).
constexpr int kProjBM = 256;   // chunk rows per projection tile
constexpr int kProjBN = 384;   // vocabulary entries per projection tile
constexpr int kDhBM = 256;     // chunk rows per dH tile
constexpr int kDhBN = 384;     // hidden columns per dH tile
constexpr int kDwBM = 384;     // vocabulary rows per dW tile
constexpr int kDwBN = 256;     // hidden columns per dW tile
constexpr int kMaxSplit = 16;  // largest split of the dH reduction over V
constexpr int kTopkCap = 8192; // candidate keys kept per row by the teacher top-K producer
constexpr int kTopkLanes = 16; // sampled maxima per row and projection tile (one per epilogue lane)

// Everything one chunk's kernels need.  Input pointers are already offset
// to the chunk's first row; workspace pointers are chunk-local.
struct ChunkArgs {
  int rows;      // rows in this chunk (<= chunk)
  int d, v, k;
  int nvt;       // vocabulary tiles of the projection (ceil(v / kProjBN))
  int ldz;       // row stride of dZ in elements (nvt * kProjBN)
  int x_bf16;    // 1: H, W, dZ are bf16; 0: fp32
  float tau;     // temperature (1: the plain loss)
  int t_bf16;    // 1: teacher logits are bf16; 0: fp32
  const void* H;
  const void* W;
  const int32_t* ids;
  const void* logits;
  const uint8_t* mask;
  // workspace (chunk-local)
  uint32_t* keys;   // [chunk][k] teacher (id << 8 | k), ascending
  float* psort;     // [chunk][k] p in key order
  float* zgs;       // [chunk][k] gathered student logits in key order
  float* negent;    // [chunk] sum_k p log p
  float* ssum;      // [chunk] sum_k p
  uint16_t* lb;     // [chunk][nvt+1] first key index whose id >= t * kProjBN
  float* pm;        // [chunk][nvt] per-tile row max of z
  float* ps;        // [chunk][nvt] per-tile sum of exp(z - max)
  double* rl;       // [chunk] per-row loss
  double* loss_acc; // [1] running loss
  void* dz;         // dZ of the group in x dtype, blocked: [rows rounded up to 32][ldz] (blk_offset)
  int dz_row0;      // row of the dZ region where this chunk's rows start (single-call path)
  float* dhp;       // [split][chunk][d] split partials of dH
  float* zc;        // fp32 logits kept by the forward (single-call path), blocked like dZ, else null
  void* hk;         // H_c in k tiles of 64 bytes: [ceil(d / tile k)][ldk][tile k] (x dtype)
  int ldk;          // rows per k-tile block of hk (the chunk size)
  void* ht;         // H^T of the chunks of one dW group, k tiled: [ldt / tile k][d][tile k] (x dtype)
  int ldt;          // group rows ht holds (dW group rows rounded up to 32, whole k tiles)
  int ht_off;       // column of ht where this chunk's rows start
  int ht_span;      // columns this chunk writes from ht_off (its rows, zero-padded to 8 if last in group)
  int dh_split;     // number of V slices of the dH reduction
  int dh_kslice;    // V entries per slice (multiple of the k tile)
};

int dh_split_for(int chunk, int d, int ldz, int* kslice);

void launch_prep(const ChunkArgs& a, hipStream_t s);
void launch_fwd_proj(const ChunkArgs& a, hipStream_t s);
void launch_merge(const ChunkArgs& a, float* lse, float* row_loss, float* zg, hipStream_t s);
// rows summed in slices of `sub` rows, each slice added to the running loss in order
void launch_loss_fold(const ChunkArgs& a, int sub, int first, int last, float* loss, hipStream_t s);
void launch_zero_loss(float* loss, hipStream_t s);
void launch_bwd_dz(const ChunkArgs& a, const float* lse, const float* g, hipStream_t s);
void launch_dz_cached(const ChunkArgs& a, const float* lse, const float* g, hipStream_t s);
void launch_bwd_dh(const ChunkArgs& a, float* dH, hipStream_t s);
void launch_transpose_h(const ChunkArgs& a, hipStream_t s);
void launch_tile_h(const ChunkArgs& a, hipStream_t s);
void launch_validate(const int32_t* ids, const uint8_t* mask, long n, int K, int v, int64_t* out, hipStream_t s);
void launch_fill_u32(uint32_t* p, size_t words, uint32_t value, hipStream_t s);
void launch_topk_maxima(const ChunkArgs& a, uint32_t* lmax, hipStream_t s);
void launch_topk_threshold(const ChunkArgs& a, const uint32_t* lmax, uint32_t* thr, int* cnt, hipStream_t s);
void launch_topk_collect(const ChunkArgs& a, const uint32_t* thr, int* cnt, uint64_t* cand, hipStream_t s);
void launch_topk_select(const ChunkArgs& a, const int* cnt, const uint64_t* cand, int32_t* ids, float* logits,
                        int* overflow, hipStream_t s);
void launch_dh_reduce(const ChunkArgs& a, float* dH, hipStream_t s);
void launch_bwd_dw(const ChunkArgs& a, float* dW, hipStream_t s);

}  // namespace kd
