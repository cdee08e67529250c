// Kernels of the fused chunked top-K KL loss (gfx950).
//
// Per chunk of rows (the pages' "one chunk of the sequence at a time":
// agentlenshq.com page "LLMのための効率的な知識蒸留…", section
// "2. Fused Chunked KL Loss"):
//   forward (passes of up to 8 chunks): k_prep -> k_tile_h -> k_fwd_proj ->
//             k_merge -> k_loss_fold
//   backward (groups of dw_chunks chunks): k_prep -> k_tile_h -> k_bwd_dz ->
//             k_bwd_dh (+ k_dh_reduce) -> k_transpose_h -> k_bwd_dw
//   single call (forward + backward), per chunk: k_prep -> k_tile_h ->
//             k_fwd_proj keeping the chunk's fp32 logits -> k_merge ->
//             k_loss_fold -> k_dz_cached -> k_transpose_h; per group:
//             k_bwd_dh (+ k_dh_reduce) -> k_bwd_dw
//   teacher top-K producer: k_topk_pass<0> (sampled row maxima) ->
//             k_topk_threshold(_reg) -> k_topk_pass<1> (candidates) ->
//             k_topk_select
// The logit tile lives only in registers in the forward (the projections
// hold it transposed in the accumulators); in the backward the closed-form
// dZ of one group of chunks is written to the workspace in 32 x 32 blocks
// (bounded by the group's rows) and consumed by the two gradient GEMMs.
#include <math.h>

#include "kd_gemm.h"
#include "kd_internal.h"
#include "kd_util.h"

namespace kd {

// Block tiles: 256 x 384 (projection, dH) and 384 x 256 (dW), eight waves.
// The projections (forward, dZ, teacher top-K) keep three LDS stages (their
// epilogue tables need part of the rest), read H_c through its k-tiled copy
// (k_tile_h: every 128-byte line of it a load touches is read whole), issue
// their tile loads in slices between the MFMA rows (SPREAD: measured faster
// for these, slower for dH and dW) and take the tile transposed in the
// accumulators (TRANS: the epilogues work on whole row segments held in
// registers).
template <typename T>
using ProjGemmX = Gemm<T, kProjBM, kProjBN, true, true, 2, 4, 3, true, true, false, true, true>;
// dH and dW read dZ blocked (the dZ passes write it so).
template <typename T>
using DhGemm = Gemm<T, kDhBM, kDhBN, true, false, 2, 4, 4, true, false, false, false, false, true>;
// dW reads H_c^T k tiled as well (k_transpose_h writes it so).
template <typename T>
using DwGemm = Gemm<T, kDwBM, kDwBN, false, true, 2, 4, 4, false, false, true, false, false, true>;
static_assert(ProjGemmX<uint16_t>::NT == ProjGemmX<float>::NT && DhGemm<uint16_t>::NT == DhGemm<float>::NT &&
                  DwGemm<uint16_t>::NT == DwGemm<float>::NT,
              "one block size per kernel for both dtypes");

constexpr int kMaxHits = 4;  // teacher ids per (row, tile) kept in LDS; more take the slow path

// ---------------------------------------------------------------------------
// teacher record -> renormalised distribution, id-sorted keys, tile ranges
// ---------------------------------------------------------------------------
// One wave per row.  p = softmax of the K cached teacher logits divided by
// the temperature (the top-K record renormalised over its entries);
// negent = sum p log p; s = sum p.
// keys = (id << 8 | k) sorted ascending with p / zg slots in the same order;
// an id outside [0, v) takes the id field 0xFFFFFF, which no vocabulary
// entry has (v <= 0xFFFFFF) and which lies past every tile, so it matches
// nothing (the 24-bit field would otherwise alias ids >= 2^24 and negative
// ids onto vocabulary entries).  lb[t] = index of the first key whose id
// lies in vocabulary tile >= t, so the keys falling in tile t are
// [lb[t], lb[t+1]).  Masked rows read nothing and get empty ranges.
constexpr uint32_t kNoId = 0xFFFFFFu;
template <typename TT>
__global__ __launch_bounds__(256) void k_prep(const int32_t* __restrict__ ids,
                                              const TT* __restrict__ logits,
                                              const uint8_t* __restrict__ mask, int rows, int K, int v,
                                              int nvt, float inv_tau, uint32_t* __restrict__ keys,
                                              float* __restrict__ psort, float* __restrict__ zgs,
                                              float* __restrict__ negent, float* __restrict__ ssum,
                                              uint16_t* __restrict__ lb) {
  __shared__ uint32_t s_key[4][256];
  __shared__ uint32_t s_sorted[4][256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  const bool valid = row < rows;
  const bool live = valid && (mask == nullptr || mask[row] != 0);
  const long rbase = static_cast<long>(row) * K;

  uint32_t key[4];
  float p[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    key[q] = 0xFFFFFFFFu;
    p[q] = 0.f;
  }
  if (live) {
    float a[4];
    float amax = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = lane + 64 * q;
      a[q] = -INFINITY;
      if (k < K) {
        const uint32_t id = static_cast<uint32_t>(ids[rbase + k]);
        key[q] = ((id < static_cast<uint32_t>(v) ? id : kNoId) << 8) | static_cast<uint32_t>(k);
        a[q] = Elem<TT>::to_f32(logits[rbase + k]);
        amax = fmaxf(amax, a[q]);
      }
    }
    amax = wave_max(amax);
    float e[4], z = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = lane + 64 * q;
      e[q] = (k < K) ? expf((a[q] - amax) * inv_tau) : 0.f;
      z += e[q];
    }
    z = wave_sum(z);
    float ne = 0.f, s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p[q] = e[q] / z;
      ne += (p[q] > 0.f) ? p[q] * logf(p[q]) : 0.f;
      s += p[q];
    }
    ne = wave_sum(ne);
    s = wave_sum(s);
    if (lane == 0) {
      negent[row] = ne;
      ssum[row] = s;
    }
  } else if (valid && lane == 0) {
    negent[row] = 0.f;
    ssum[row] = 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) s_key[w][lane + 64 * q] = key[q];
  __syncthreads();
  if (live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = lane + 64 * q;
      if (k < K) {
        int rank = 0;
        for (int j = 0; j < K; ++j) rank += (s_key[w][j] < key[q]) ? 1 : 0;
        keys[rbase + rank] = key[q];
        psort[rbase + rank] = p[q];
        zgs[rbase + k] = 0.f;
        s_sorted[w][rank] = key[q];
      }
    }
  }
  __syncthreads();
  if (valid) {
    uint16_t* lbr = lb + static_cast<long>(row) * (nvt + 1);
    if (!live) {
      for (int t = lane; t <= nvt; t += 64) lbr[t] = 0;
    } else {
      for (int j = lane; j < K; j += 64) {
        const int vt = min(nvt, static_cast<int>((s_sorted[w][j] >> 8) / kProjBN));
        const int vprev = (j == 0) ? -1 : min(nvt, static_cast<int>((s_sorted[w][j - 1] >> 8) / kProjBN));
        for (int t = vprev + 1; t <= vt; ++t) lbr[t] = static_cast<uint16_t>(j);
        if (j == K - 1)
          for (int t = vt + 1; t <= nvt; ++t) lbr[t] = static_cast<uint16_t>(K);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// helpers shared by the two projection epilogues
// ---------------------------------------------------------------------------
// dZ before the teacher term, coef exp(z / tau - lse) with coef = g s tau,
// t2 = log2(e) / tau and lse2 = lse log2(e) (lse of z / tau), and the teacher
// term's subtraction.  Contraction is off so that every kernel forming dZ
// (recomputed or cached logits) rounds it the same way.
__device__ __forceinline__ float dz_exp(float z, float coef, float lse2, float t2) {
#pragma clang fp contract(off)
  return coef * fast_exp2(fmaf(z, t2, -lse2));
}
__device__ __forceinline__ float dz_sub(float o, float sub) {
#pragma clang fp contract(off)
  return o - sub;
}

// Tile t of a projection launch over rtn row tiles x nvt vocabulary tiles:
// groups of 8 row tiles (2048 rows), vocabulary-major inside a group, so the
// workgroups running together on one XCD share W panels and a few H panels in
// its L2, however many rows the launch covers.  Up to 8 row tiles this is
// vt = t / rtn, rt = t % rtn.
__device__ __forceinline__ void proj_tile(int t, int rtn, int nvt, int& vt, int& rt) {
  constexpr int RG = 8;
  const int g = t / (RG * nvt);
  const int gs = min(RG, rtn - g * RG);  // row tiles in this group
  const int r = t - g * RG * nvt;
  vt = r / gs;
  rt = g * RG + r % gs;
}

// ---------------------------------------------------------------------------
// forward: projection + per-tile online (max, sum exp) + top-K gather
// ---------------------------------------------------------------------------
// Tile (rt, vt): z = H[rt rows] W[vt vocab]^T on matrix cores, transposed in
// the accumulators (each lane holds 4 rows x 48 columns of its wave tile, in
// groups of 4 consecutive columns).  The epilogue works on the registers:
// each wave reduces its 96 columns of a row to (max m_w, sum of exp((z -
// m_w) / tau)), the two lanes sharing a row combine theirs, and one thread per
// row folds the four waves' pairs into the tile's (max, sum).  The lane
// holding a teacher id's column copies z there (a copy of the accumulator,
// bit for bit).  Logits reach HBM only in the single-call path (zc != null),
// which keeps the chunk's fp32 logits in the workspace for the dZ pass.
template <typename T>
__global__ __launch_bounds__(512, 1) void k_fwd_proj(const T* __restrict__ hk, int ldk, const T* __restrict__ W,
                                                     int rows, int d, int v, int nvt, int K,
                                                     const uint16_t* __restrict__ lb,
                                                     const uint32_t* __restrict__ keys,
                                                     float* __restrict__ zgs, float* __restrict__ pm,
                                                     float* __restrict__ ps, float* __restrict__ zc,
                                                     int ldz, float t2) {
  using G = ProjGemmX<T>;
  static_assert(G::WAVES_COLS == 4 && G::FN * 32 == G::WN, "the fold below takes four waves per row");
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  __shared__ int s_lo[G::BM], s_hi[G::BM];
  __shared__ uint32_t s_hit[G::BM][kMaxHits];  // (column in tile << 8) | key slot
  __shared__ float2 s_part[G::WAVES_COLS][G::BM];  // per wave: (max, sum) of its columns
  const int rtn = (rows + G::BM - 1) / G::BM;
  const int t = xcd_tile(blockIdx.x, rtn * nvt);
  if (t < 0) return;
  int vt, rt;
  proj_tile(t, rtn, nvt, vt, rt);
  const int tid = threadIdx.x;
  for (int r = tid; r < G::BM; r += G::NT) {
    const int gr = rt * G::BM + r;
    int lo = 0, hi = 0;
    if (gr < rows) {
      lo = lb[static_cast<long>(gr) * (nvt + 1) + vt];
      hi = lb[static_cast<long>(gr) * (nvt + 1) + vt + 1];
    }
    s_lo[r] = lo;
    s_hi[r] = hi;
    if (hi - lo <= kMaxHits)
      for (int q = lo; q < hi; ++q)
        s_hit[r][q - lo] = ((keys[static_cast<long>(gr) * K + q] >> 8) - vt * G::BN) << 8 | static_cast<uint32_t>(q);
  }
  f32x16 acc[G::FM][G::FN];
  const Operand<T> A{hk, ldk, static_cast<long>((d + G::BK - 1) / G::BK) * ldk * G::BK, rt * G::BM, rows, d};
  const Operand<T> B{W, d, static_cast<long>(v) * d, vt * G::BN, v, d};
  G::run(A, B, 0, d, smem, acc);  // ends with a barrier: the tables above are visible

  const int lane = tid & 63, wave = tid >> 6, wm = wave / G::WAVES_COLS, wn = wave % G::WAVES_COLS;
  const int half = lane >> 5;
  // column in tile of element e of atom j: c0 + 32 j + 8 (e >> 2) + (e & 3)
  const int c0 = wn * G::WN + 4 * half;
  const int r0 = wm * G::WM + (lane & 31);  // row in tile of atom row i: r0 + 32 i
  if (zc) {  // single-call path: keep the fp32 logits of the chunk (blocked, as dZ)
#pragma unroll
    for (int i = 0; i < G::FM; ++i) {
      const int grow = rt * G::BM + r0 + 32 * i;
      if (grow >= rows) continue;
      char* zrow = reinterpret_cast<char*>(zc) + blk_offset<4>(grow, vt * G::BN + c0, ldz);
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)  // columns c0 + 32 j + 8 g + [0, 4): one granule
          *reinterpret_cast<f32x4*>(zrow + j * 4096 + g * 1024) =
              f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    }
  }
  // Teacher ids: the lane holding (row, column) copies the accumulator.
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    const int row = r0 + 32 * i, grow = rt * G::BM + row;
    const int lo = s_lo[row], n = s_hi[row] - lo;
    for (int q = 0; q < n; ++q) {
      int col, slot;
      if (n <= kMaxHits) {
        const uint32_t u = s_hit[row][q];
        col = static_cast<int>(u >> 8);
        slot = static_cast<int>(u & 0xFFu);
      } else {
        slot = lo + q;
        col = static_cast<int>(keys[static_cast<long>(grow) * K + slot] >> 8) - vt * G::BN;
      }
      const int cw = col - wn * G::WN;
      if (cw >= 0 && cw < G::WN && ((cw >> 2) & 1) == half) {
        const int jc = cw >> 5, ec = (cw & 3) + 4 * ((cw >> 3) & 3);
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < G::FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) z = (j == jc && e == ec) ? acc[i][j][e] : z;
        zgs[static_cast<long>(grow) * K + slot] = z;
      }
    }
  }
  const int ncols = min(G::BN, v - vt * G::BN);
  if (ncols < G::BN) {  // columns past v take no part (exp2(-inf) = 0)
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (c0 + 32 * j + 8 * (e >> 2) + (e & 3) >= ncols) acc[i][j][e] = -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < G::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[i][j][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // t2 = log2(e) / tau: exp((z - mx) / tau) = 2^(z t2 - mx t2); a wave with
    // no column left (mx = -inf) sums exp2(-inf) = 0
    const float mx2 = mx == -INFINITY ? 0.f : mx * t2;
    float sm = 0.f;
#pragma unroll
    for (int j = 0; j < G::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sm += fast_exp2(fmaf(acc[i][j][e], t2, -mx2));
    sm += __shfl_xor(sm, 32, 64);
    if (half == 0) s_part[wn][r0 + 32 * i] = make_float2(mx, sm);
  }
  __syncthreads();
  for (int r = tid; r < G::BM; r += G::NT) {
    const int grow = rt * G::BM + r;
    if (grow >= rows) break;
    float2 p[G::WAVES_COLS];
#pragma unroll
    for (int w = 0; w < G::WAVES_COLS; ++w) p[w] = s_part[w][r];
    float mx = p[0].x;
#pragma unroll
    for (int w = 1; w < G::WAVES_COLS; ++w) mx = fmaxf(mx, p[w].x);
    const float mx2 = mx * t2;  // some wave holds a column below v: mx is finite
    float sm = 0.f;
#pragma unroll
    for (int w = 0; w < G::WAVES_COLS; ++w) sm += p[w].y * fast_exp2(fmaf(p[w].x, t2, -mx2));
    pm[static_cast<long>(grow) * nvt + vt] = mx;
    ps[static_cast<long>(grow) * nvt + vt] = sm;
  }
}

// ---------------------------------------------------------------------------
// forward: merge tile partials -> lse, row loss, gathered logits
// ---------------------------------------------------------------------------
// lse_i = M / tau + log sum_t s_t exp((m_t - M) / tau) over the vocabulary
// tiles (fixed order): the lse of z / tau.  row_loss_i =
// tau^2 m_i (negent_i - sum_k p_ik zg_ik / tau + s_i lse_i), tau^2 times the
// KL of the renormalised teacher from the student at the K ids.
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ pm, const float* __restrict__ ps,
                                               int nvt, const uint32_t* __restrict__ keys,
                                               const float* __restrict__ psort,
                                               const float* __restrict__ zgs,
                                               const float* __restrict__ negent,
                                               const float* __restrict__ ssum,
                                               const uint8_t* __restrict__ mask, int rows, int K,
                                               float* __restrict__ lse_out, float* __restrict__ rl_out,
                                               float* __restrict__ zg_out, double* __restrict__ rl_ws,
                                               float t2, double inv_tau, double tau2) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= rows) return;
  const long pb = static_cast<long>(row) * nvt;
  float M = -INFINITY;
  for (int t = lane; t < nvt; t += 64) M = fmaxf(M, pm[pb + t]);
  M = wave_max(M);
  float S = 0.f;
  for (int t = lane; t < nvt; t += 64) S += ps[pb + t] * fast_exp2((pm[pb + t] - M) * t2);
  S = wave_sum(S);
  const double lse = static_cast<double>(M) * inv_tau + log(static_cast<double>(S));
  const bool live = (mask == nullptr || mask[row] != 0);
  const long kb = static_cast<long>(row) * K;
  double dot = 0.0;
  if (live)
    for (int j = lane; j < K; j += 64) dot += static_cast<double>(psort[kb + j]) * static_cast<double>(zgs[kb + j]);
  dot = wave_sum(dot);
  const double rl =
      live ? tau2 * (static_cast<double>(negent[row]) - dot * inv_tau + static_cast<double>(ssum[row]) * lse) : 0.0;
  if (lane == 0) {
    lse_out[row] = static_cast<float>(lse);
    rl_ws[row] = rl;
    if (rl_out) rl_out[row] = static_cast<float>(rl);
  }
  if (zg_out) {
    for (int j = lane; j < K; j += 64) {
      if (live)
        zg_out[kb + (keys[kb + j] & 0xFFu)] = zgs[kb + j];
      else
        zg_out[kb + j] = 0.f;
    }
  }
}

// Running loss: the chunk's row losses summed in a fixed order (fp64) and
// folded into the accumulator; the last chunk writes the fp32 loss.
__global__ __launch_bounds__(256) void k_loss_fold(const double* __restrict__ rl, int rows, int sub,
                                                   double* __restrict__ acc, int first, int last,
                                                   float* __restrict__ loss) {
  // rows in slices of `sub` (the chunk size): each slice is summed by the
  // same 256-way tree and added to the running loss in order, so the result
  // does not depend on how many chunks one forward pass covers
  __shared__ double s[256];
  double a = first ? 0.0 : acc[0];
  for (int r0 = 0; r0 < rows; r0 += sub) {
    const int n = min(sub, rows - r0);
    double x = 0.0;
    for (int i = threadIdx.x; i < n; i += 256) x += rl[r0 + i];
    s[threadIdx.x] = x;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
      __syncthreads();
    }
    a += s[0];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    acc[0] = a;
    if (last) loss[0] = static_cast<float>(a);
  }
}

__global__ void k_zero_loss(float* loss) { loss[0] = 0.f; }

// ---------------------------------------------------------------------------
// backward: recompute the projection and form the closed-form dZ
// ---------------------------------------------------------------------------
// dZ_iv = g tau m_i (s_i exp(z_iv / tau - lse_i) - sum_k p_ik [t_ik = v]),
// evaluated in fp32 as (g s_i tau) exp(z_iv / tau - lse_i) - p_ik (g tau),
// the teacher terms applied before the single rounding to the storage dtype.  Masked rows and columns in
// [v, ldz) (padding of the row) are written as exact zeros.
template <typename T>
__global__ __launch_bounds__(512, 1) void k_bwd_dz(const T* __restrict__ hk, int ldk, const T* __restrict__ W,
                                                   int rows, int d, int v, int nvt, int K, int ldz,
                                                   const uint16_t* __restrict__ lb,
                                                   const uint32_t* __restrict__ keys,
                                                   const float* __restrict__ psort,
                                                   const float* __restrict__ ssum,
                                                   const uint8_t* __restrict__ mask,
                                                   const float* __restrict__ lse,
                                                   const float* __restrict__ gptr, T* __restrict__ dz,
                                                   float t2, float tau) {
  using G = ProjGemmX<T>;
  constexpr int SZ = static_cast<int>(sizeof(T)), BLK = 1024 * SZ;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  __shared__ int2 s_range[G::BM];          // the row's keys in this tile: [lo, hi)
  __shared__ f32x4 s_rc[G::BM];            // per row: lse log2(e), coefficient, g tau, live
  __shared__ int s_hcol[G::BM][kMaxHits];  // column in tile of the row's teacher ids here
  __shared__ float s_hp[G::BM][kMaxHits];  // their teacher probabilities
  __shared__ u32x4 s_hmask[G::BM];         // groups of 4 columns of the tile holding a teacher id (96 bits)
  static_assert(G::BN == 384, "the group mask covers 96 groups of 4 columns");
  const int rtn = (rows + G::BM - 1) / G::BM;
  const int t = xcd_tile(blockIdx.x, rtn * nvt);
  if (t < 0) return;
  int vt, rt;
  proj_tile(t, rtn, nvt, vt, rt);
  const int tid = threadIdx.x;
  const float g = gptr ? gptr[0] : 1.f;
  for (int r = tid; r < G::BM; r += G::NT) {
    const int gr = rt * G::BM + r;
    int lo = 0, hi = 0;
    float lse2 = 0.f, coef = 0.f, gm = 0.f;
    int live = 0;
    if (gr < rows) {
      live = (mask == nullptr || mask[gr] != 0) ? 1 : 0;
      lse2 = lse[gr] * kLog2e;
      if (live) {
        lo = lb[static_cast<long>(gr) * (nvt + 1) + vt];
        hi = lb[static_cast<long>(gr) * (nvt + 1) + vt + 1];
        gm = g * tau;
        coef = g * ssum[gr] * tau;  // g and tau folded into the row coefficient
      }
    }
    s_range[r] = make_int2(lo, hi);
    s_rc[r] = f32x4{lse2, coef, gm, live ? 1.f : 0.f};
    uint32_t hm[3] = {0u, 0u, 0u};
    for (int q = lo; q < hi; ++q) {
      const long kq = static_cast<long>(gr) * K + q;
      const int c = static_cast<int>(keys[kq] >> 8) - vt * G::BN;
      if (hi - lo <= kMaxHits) {
        s_hcol[r][q - lo] = c;
        s_hp[r][q - lo] = psort[kq];
      }
      hm[c >> 7] |= 1u << ((c >> 2) & 31);
    }
    s_hmask[r] = u32x4{hm[0], hm[1], hm[2], 0u};
  }
  f32x16 acc[G::FM][G::FN];
  const Operand<T> A{hk, ldk, static_cast<long>((d + G::BK - 1) / G::BK) * ldk * G::BK, rt * G::BM, rows, d};
  const Operand<T> B{W, d, static_cast<long>(v) * d, vt * G::BN, v, d};
  G::run(A, B, 0, d, smem, acc);  // ends with a barrier: the tables above are visible

  // The tile is transposed in the accumulators: each lane holds rows r0 + 32 i
  // and, per atom j, 4 groups of 4 consecutive columns, which are 8 (bf16) or
  // 16 (fp32) contiguous bytes of dZ's blocked layout; the lanes of a store
  // instruction cover 512 contiguous bytes.  Rows from `rows` up to a whole
  // block are written as zeros (dW reads whole blocks of rows).
  const int lane = tid & 63, wave = tid >> 6, wm = wave / G::WAVES_COLS, wn = wave % G::WAVES_COLS;
  const int half = lane >> 5;
  const int r0 = wm * G::WM + (lane & 31);
  const int c0 = wn * G::WN + 4 * half;  // column in tile of element 4 g + e of atom j: c0 + 32 j + 8 g + e
  const int rpad = (rows + 31) & ~31;
  const bool full_tile = (vt + 1) * G::BN <= v;
  char* const zb = reinterpret_cast<char*>(dz);
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    const int row = r0 + 32 * i, grow = rt * G::BM + row;
    if (grow >= rpad) continue;  // the same for the wave's 32 lanes of this row block
    const f32x4 rc = s_rc[row];
    const bool live = rc[3] != 0.f;
    char* const out = zb + blk_offset<SZ>(grow, static_cast<long>(vt) * G::BN + c0, ldz);
    // The lane's groups of 4 columns are c0 / 4 + 8 j + 2 gq: bit 8 j + 2 gq of x
    // (c0 / 4 = 24 wn + half; the 96-bit mask read as the 64 bits that hold them).
    uint32_t x;
    {
      const u32x4 hm = s_hmask[row];
      const uint64_t pr = wn < 2 ? (static_cast<uint64_t>(hm[1]) << 32 | hm[0])
                                 : (static_cast<uint64_t>(hm[2]) << 32 | hm[1]);
      x = static_cast<uint32_t>(pr >> ((c0 >> 2) - (wn < 2 ? 0 : 32)));
    }
#pragma unroll
    for (int j = 0; j < G::FN; ++j)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = live ? dz_exp(acc[i][j][4 * gq + e], rc[1], rc[0], t2) : 0.f;
        if (!full_tile) {  // columns past v: zero padding of dZ
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (vt * G::BN + c0 + 32 * j + 8 * gq + e >= v) o[e] = 0.f;
        }
        if ((x >> (8 * j + 2 * gq)) & 1u) {  // a teacher id in these 4 columns: its p, before the rounding
          const int cg = c0 + 32 * j + 8 * gq;
          const int2 rg = s_range[row];
          const int n = rg.y - rg.x;
          for (int q = 0; q < n; ++q) {  // key order: the p of a repeated id one after the other
            int c;
            float sub;
            if (n <= kMaxHits) {
              c = s_hcol[row][q];
              sub = s_hp[row][q];
            } else {
              const long kq = static_cast<long>(grow) * K + rg.x + q;
              c = static_cast<int>(keys[kq] >> 8) - vt * G::BN;
              sub = psort[kq];
            }
            const int dc = c - cg;
            if (static_cast<unsigned>(dc) < 4u) {
              const float sg = sub * rc[2];
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = dz_sub(o[e], dc == e ? sg : 0.f);
            }
          }
        }
        if constexpr (SZ == 2) {  // one nearest-even rounding per value
          *reinterpret_cast<uint2*>(out + j * BLK + gq * 512) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        } else {
          *reinterpret_cast<f32x4*>(out + j * BLK + gq * 1024) = f32x4{o[0], o[1], o[2], o[3]};
        }
      }
  }
}

// ---------------------------------------------------------------------------
// single-call path: dZ from the logits the forward kept
// ---------------------------------------------------------------------------
// The same dZ as k_bwd_dz, bit for bit (same fp32 logits, same formula),
// from the chunk's cached logits instead of a recomputed projection.  One
// thread per 8 consecutive columns of a row (ldz is a multiple of the
// projection tile width, so the 8 columns lie in one vocabulary tile); the
// 32 threads of a block's granule run are consecutive, so both the logits
// and dZ (both blocked) move in 512-byte runs.  The chunk's rows start at
// row0 of the group's dZ region, which need not be a block boundary: rows
// of the blocks it covers that belong to the chunk before are left alone,
// rows past the chunk up to a whole block are written as zeros.
template <typename T>
__global__ __launch_bounds__(256) void k_dz_cached(const float* __restrict__ zc, int ldz, int row0, int rows,
                                                   int rb0, int nrb, int v, int K, int nvt,
                                                   const uint16_t* __restrict__ lb,
                                                   const uint32_t* __restrict__ keys,
                                                   const float* __restrict__ psort,
                                                   const float* __restrict__ ssum,
                                                   const uint8_t* __restrict__ mask,
                                                   const float* __restrict__ lse,
                                                   const float* __restrict__ gptr, T* __restrict__ dz,
                                                   float t2, float tau) {
  constexpr int SZ = static_cast<int>(sizeof(T));
  // thread -> (block row rb0 + q / nvb, block column q % nvb, 8-column group, row in block)
  const int nvb = ldz / 32;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(nrb) * nvb * 128) return;
  const int m = static_cast<int>(idx & 31), g8 = static_cast<int>((idx >> 5) & 3);
  const long q = idx >> 7;
  const int cb = static_cast<int>(q % nvb);
  const long R = (rb0 + q / nvb) * 32 + m;  // row of the dZ region
  if (R < row0) return;                     // an earlier chunk's row
  const int row = static_cast<int>(R - row0), c0 = cb * 32 + g8 * 8;
  float o[8];
  if (row < rows && (mask == nullptr || mask[row] != 0)) {
    const float g = gptr ? gptr[0] : 1.f;
    const float lse2 = lse[row] * kLog2e, coef = g * ssum[row] * tau, gt = g * tau;
    const char* zr = reinterpret_cast<const char*>(zc) + blk_offset<4>(row, c0, ldz);
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(zr);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(zr + 512);  // columns c0 + 4..7: the next granule
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = dz_exp(z0[e], coef, lse2, t2);
      o[e + 4] = dz_exp(z1[e], coef, lse2, t2);
    }
    const int t = c0 / kProjBN;
    const int lo = lb[static_cast<long>(row) * (nvt + 1) + t], hi = lb[static_cast<long>(row) * (nvt + 1) + t + 1];
    for (int qq = lo; qq < hi; ++qq) {
      const long kq = static_cast<long>(row) * K + qq;
      const int c = static_cast<int>(keys[kq] >> 8) - c0;
      if (static_cast<unsigned>(c) < 8u) {
        const float sub = psort[kq] * gt;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = dz_sub(o[e], (c == e) ? sub : 0.f);
      }
    }
    if (c0 + 8 > v) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e >= v) o[e] = 0.f;
    }
  } else {  // masked rows, and rows past the chunk up to a whole block: zeros
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
  }
  char* out = reinterpret_cast<char*>(dz) + blk_offset<SZ>(R, c0, ldz);
  if constexpr (SZ == 2) {
    *reinterpret_cast<uint4*>(out) = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                                pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
  } else {
    *reinterpret_cast<f32x4*>(out) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(out + 512) = f32x4{o[4], o[5], o[6], o[7]};
  }
}

// ---------------------------------------------------------------------------
// backward: dH = dZ W (split over V, fixed-order reduce) and dW += dZ^T H
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(512, 1) void k_bwd_dh(const T* __restrict__ dz, int ldz,
                                                   const T* __restrict__ W, int rows, int d, int v,
                                                   int split, int kslice, float* __restrict__ out,
                                                   long split_stride) {
  using G = DhGemm<T>;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  const int mtn = (rows + G::BM - 1) / G::BM, ntn = (d + G::BN - 1) / G::BN;
  const int t = xcd_tile(blockIdx.x, mtn * ntn * split);
  if (t < 0) return;
  const int ks = t / (mtn * ntn), rem = t % (mtn * ntn);
  const int mt = rem / ntn, nt = rem % ntn;
  const int k0 = ks * kslice, k1 = min(ldz, k0 + kslice);
  f32x16 acc[G::FM][G::FN];
  // A(m = chunk row, k = vocab) = dZ[m][k];  B(n = hidden, k = vocab) = W[k][n]
  const Operand<T> A{dz, ldz, (rows + 31) / 32 * blk_pitch<sizeof(T)>(ldz) / static_cast<long>(sizeof(T)), mt * G::BM,
                     rows, ldz};
  const Operand<T> B{W, d, static_cast<long>(v) * d, nt * G::BN, d, v};
  G::run(A, B, k0, k1, smem, acc);
  // rows past the chunk fall outside the region; columns past d get kOOB
  const int row0 = mt * G::BM, col0 = nt * G::BN;
  const F32Region o(out + ks * split_stride + static_cast<long>(row0) * d, static_cast<long>(rows - row0) * d);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / (G::BN / G::WN), wn = wave % (G::BN / G::WN);
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      const int col = col0 + acc_col<G>(wn, j, lane);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t off = col < d ? static_cast<uint32_t>((acc_row<G>(wm, i, e, lane) * d + col) * 4) : kOOB;
        o.store(acc[i][j][e], off);
      }
    }
}

__global__ __launch_bounds__(256) void k_dh_reduce(const float* __restrict__ part, int split,
                                                   long split_stride, long count,
                                                   float* __restrict__ dH) {
  const long i4 = (static_cast<long>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i4 >= count) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i4);
  for (int k = 1; k < split; ++k) s += *reinterpret_cast<const f32x4*>(part + k * split_stride + i4);
  *reinterpret_cast<f32x4*>(dH + i4) = s;
}

// H_c in k tiles for the projections: the block of k tile t holds rows
// [0, ldk) x 64 bytes of k, element (r, k) at hk[(t ldk + r) BK + k % BK]
// with BK = 64 / sizeof(element); k past d is written as zeros.  Rows past
// `rows` are not written (the projections never read them).  A workgroup
// copies two k tiles of 32 rows: eight lanes read one row's 128 bytes (whole
// lines), and each tile's 32 rows are 2 KiB of contiguous output.  Grid: x over
// row groups (a chunk may need more than 65535 of them), y over tile pairs.
__global__ __launch_bounds__(256) void k_tile_h(const char* __restrict__ Hc, int rows, int row_bytes,
                                                char* __restrict__ hk, int ldk, int nkt) {
  const int t = threadIdx.x;
  const int r = blockIdx.x * 32 + (t >> 3);
  const int kt = blockIdx.y * 2 + ((t >> 2) & 1);
  const int byte = kt * 64 + (t & 3) * 16;  // of the row
  if (r >= rows || kt >= nkt) return;
  uint4 x = make_uint4(0u, 0u, 0u, 0u);
  if (byte < row_bytes) x = *reinterpret_cast<const uint4*>(Hc + static_cast<long>(r) * row_bytes + byte);
  *reinterpret_cast<uint4*>(hk + (static_cast<long>(kt) * ldk + r) * 64 + (t & 3) * 16) = x;
}

// H_c^T for the dW GEMM, k tiled: its k (the row within the dW group) runs
// contiguous in 64-byte tiles, element (h, q) of hidden column h and group
// row q at ht[((q / BK) d + h) BK + q % BK], BK = 64 / sizeof(element), so the
// B operand needs no transposing LDS read and each k tile is one block.  The
// chunk's rows are group rows [off, off + rows); rows [off + rows, off + span)
// are written as zeros (span rounds the last chunk of a group up to 32, a
// whole k tile).  64 x 64 tiles through LDS; the grid's x runs over chunk rows
// (a chunk may need more than 65535 row tiles), y over hidden columns.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_h(const T* __restrict__ Hc, int rows, int d, T* __restrict__ ht,
                                                     int ldt, int off, int span) {
  constexpr int BK = 64 / static_cast<int>(sizeof(T));
  __shared__ T tile[64][65];
  const int c0 = blockIdx.y * 64, r0 = blockIdx.x * 64;  // c: hidden column, r: chunk row
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < d) ? Hc[static_cast<long>(r) * d + c] : T(0);
  }
  __syncthreads();
  const int r = r0 + tx, q = off + r;
  const long qo = static_cast<long>(q / BK) * d * BK + q % BK;
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i;
    if (c < d && r < span && q < ldt) ht[qo + static_cast<long>(c) * BK] = tile[tx][i];
  }
}

// dW tile access in the accumulator layout of one wave.  Used as the
// engine's accumulator initialiser (loads) and for the write-back.  The
// fields are wave-uniform; each phase derives its per-lane part afresh from
// an opaque lane id, so no per-lane value has to stay live across the k loop
// (all registers are taken there).
//   row of element (i, e) = rbase + 32 i + 8 (e / 4) + (e % 4) + 4 (lane / 32)
//   column of atom j      = cbase + 32 j + lane % 32
// Byte offsets stay below 384 d 4 < 2^31 (d <= 65536); a column past d gets
// the top bit set, which puts it past any region (read as 0, not written).
template <class G>
struct DwTile {
  static constexpr bool kLoads = true;
  const F32Region& o;
  int d, rbase, cbase;
  struct Lane {
    int d, rbase, cbase;  // opaque copies of the fields
    uint32_t base;        // byte offset of the lane's (row, column) in the atom
    uint32_t oob[G::FN];  // 0, or the top bit for columns past d
  };
  // Every input passes through an empty volatile asm, so the values of one
  // call are not merged with those of another across the k loop.
  __device__ __forceinline__ Lane lane_part() const {
    Lane l;
    uint32_t all = ~0u;
    l.d = d;
    l.rbase = rbase;
    l.cbase = cbase;
    asm volatile("" : "+s"(all), "+s"(l.d), "+s"(l.rbase), "+s"(l.cbase));
    const int lane = static_cast<int>(__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u)));
    const int lc = lane & 31;
    l.base = static_cast<uint32_t>((4 * (lane >> 5) * l.d + lc) * 4);
#pragma unroll
    for (int j = 0; j < G::FN; ++j) l.oob[j] = lc < l.d - l.cbase - 32 * j ? 0u : kOOB;
    return l;
  }
  __device__ __forceinline__ static uint32_t offset(const Lane& l, int i, int j, int e) {
    const int urow = l.rbase + 32 * i + 8 * (e >> 2) + (e & 3);
    return (l.base + static_cast<uint32_t>((urow * l.d + l.cbase + 32 * j) * 4)) | l.oob[j];
  }
  __device__ __forceinline__ void operator()(f32x16 (&acc)[G::FM][G::FN]) const {
    const Lane l = lane_part();
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = o.load(offset(l, i, j, e));
  }
  __device__ __forceinline__ void store(const f32x16 (&acc)[G::FM][G::FN]) const {
    const Lane l = lane_part();
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) o.store(acc[i][j][e], offset(l, i, j, e));
  }
};

template <typename T>
__global__ __launch_bounds__(512, 1) void k_bwd_dw(const T* __restrict__ dz, int ldz,
                                                   const T* __restrict__ ht, int ldt, int rows, int d, int v,
                                                   float* __restrict__ dW) {
  using G = DwGemm<T>;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  const int mtn = (v + G::BM - 1) / G::BM, ntn = (d + G::BN - 1) / G::BN;
  const int t = xcd_tile(blockIdx.x, mtn * ntn);
  if (t < 0) return;
  const int mt = t / ntn, nt = t % ntn;
  // A(m = vocab, k = chunk row) = dZ[k][m];  B(n = hidden, k = chunk row) = H_c^T[n][k]
  // dZ's rows past `rows` are zero up to a whole block, so k tiles that run
  // past `rows` read zeros there
  const Operand<T> A{dz, ldz, (rows + 31) / 32 * blk_pitch<sizeof(T)>(ldz) / static_cast<long>(sizeof(T)), mt * G::BM,
                     ldz, rows};
  const Operand<T> B{ht, d, static_cast<long>(d) * ldt, nt * G::BN, d, rows};
  // dW += dZ^T H_c with the accumulators starting from the tile's current dW
  // values: they are loaded while the first operand tiles are in flight and
  // stored back after the last tile, so no read of dW waits after the
  // products are done.  Rows past v fall outside the region.
  const int row0 = mt * G::BM, col0 = nt * G::BN;
  const F32Region o(dW + static_cast<long>(row0) * d, static_cast<long>(v - row0) * d);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / (G::BN / G::WN), wn = wave % (G::BN / G::WN);
  const DwTile<G> tile{o, d, wm * G::WM, col0 + wn * G::WN};
  f32x16 acc[G::FM][G::FN];
  G::run(A, B, 0, rows, smem, acc, tile);
  tile.store(acc);
}

// ---------------------------------------------------------------------------
// teacher top-K producer: the K largest logits of every row, largest first,
// equal logits by the lower id, without the rows x vocabulary grid
// ---------------------------------------------------------------------------
// Keys: (ordered_key(z) << 32) | (0xFFFFFFFF - id) -- a larger key is a larger
// logit, or the same logit with a lower id; keys of one row are distinct.
//
// Pass 1 records, per row and tile, 16 sampled maxima, each the largest key
// of 24 of the tile's columns (each of the 8 lanes holding 48 columns of the
// row gives two): kTopkLanes x nvt sampled maxima.
// Threshold per row: the K-th largest of them.  They are keys of K distinct
// logits of the row, so at least K logits are at or above it: every logit of
// the top K is.  Rows with fewer than K sampled maxima take threshold 0 (every
// logit; then v < 24 K <= 6144 <= kTopkCap).
// One workgroup per row; the row's maxima are staged in LDS when they fit.
// Rows with at most 256 kTopkRegKeys maxima (v up to 294912): each thread
// holds its share in registers, so the 32 passes read no memory.  0 pads the
// shares (no trial threshold is 0, so padding is never counted).
constexpr int kTopkRegKeys = 48;
__global__ __launch_bounds__(256) void k_topk_threshold_reg(const uint32_t* __restrict__ lmax, int nmax, int K,
                                                            uint32_t* __restrict__ thr, int* __restrict__ cnt) {
  __shared__ int s_c[2][4];
  const int row = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint32_t* r = lmax + static_cast<long>(row) * nmax;
  uint32_t x[kTopkRegKeys];
#pragma unroll
  for (int i = 0; i < kTopkRegKeys; ++i) {
    const int t = tid + 256 * i;
    x[i] = t < nmax ? r[t] : 0u;
  }
  uint32_t res = 0;
  if (nmax >= K) {
    // MSB first: the largest res with #{maxima >= res} >= K
    for (int b = 31; b >= 0; --b) {
      const uint32_t trial = res | (1u << b);
      int c = 0;
#pragma unroll
      for (int i = 0; i < kTopkRegKeys; ++i) c += x[i] >= trial ? 1 : 0;
      c = wave_sum(c);
      if (lane == 0) s_c[b & 1][w] = c;
      __syncthreads();
      if (s_c[b & 1][0] + s_c[b & 1][1] + s_c[b & 1][2] + s_c[b & 1][3] >= K) res = trial;
    }
  }
  if (tid == 0) {
    thr[row] = res;
    cnt[row] = 0;
  }
}

// Any number of maxima: staged in LDS when they fit, else read from memory
// in every pass.
__global__ __launch_bounds__(256) void k_topk_threshold(const uint32_t* __restrict__ lmax, int nmax, int K,
                                                        uint32_t* __restrict__ thr, int* __restrict__ cnt) {
  constexpr int kLdsKeys = 16384;
  __shared__ uint32_t s_v[kLdsKeys];
  __shared__ int s_c[2][4];
  const int row = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint32_t* r = lmax + static_cast<long>(row) * nmax;
  uint32_t res = 0;
  if (nmax >= K) {
    const bool staged = nmax <= kLdsKeys;
    if (staged) {
      for (int i = tid; i < nmax; i += 256) s_v[i] = r[i];
      __syncthreads();
    }
    // MSB first: the largest res with #{maxima >= res} >= K
    for (int b = 31; b >= 0; --b) {
      const uint32_t trial = res | (1u << b);
      int c = 0;
      for (int t = tid; t < nmax; t += 256) c += (staged ? s_v[t] : r[t]) >= trial ? 1 : 0;
      c = wave_sum(c);
      if (lane == 0) s_c[b & 1][w] = c;
      __syncthreads();
      if (s_c[b & 1][0] + s_c[b & 1][1] + s_c[b & 1][2] + s_c[b & 1][3] >= K) res = trial;
    }
  }
  if (tid == 0) {
    thr[row] = res;
    cnt[row] = 0;
  }
}

// Projection tile as in the forward (transposed in the accumulators: each
// lane holds 4 rows x 48 columns).  PASS 0: per row, the lane writes the
// largest key of each half of its columns (padding columns excluded) to lmax.
// PASS 1: it appends every logit of its columns whose key is at or above its
// row's threshold to the row's candidate list (one atomic add per lane and
// row with candidates; a list longer than kTopkCap keeps kTopkCap entries and
// the select pass reports the row).
template <typename T, int PASS>
__global__ __launch_bounds__(512, 1) void k_topk_pass(const T* __restrict__ hk, int ldk, const T* __restrict__ W, int rows,
                                                      int d, int v, int nvt, uint32_t* __restrict__ lmax,
                                                      const uint32_t* __restrict__ thr, int* __restrict__ cnt,
                                                      uint64_t* __restrict__ cand) {
  using G = ProjGemmX<T>;  // H_c through its k-tiled copy, tile transposed in the accumulators
  static_assert(G::WAVES_COLS * 2 * 2 == kTopkLanes && G::FN * 4 == 12, "two maxima per lane and row");
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  __shared__ uint32_t s_thr[G::BM];
  const int rtn = (rows + G::BM - 1) / G::BM;
  const int t = xcd_tile(blockIdx.x, rtn * nvt);
  if (t < 0) return;
  int vt, rt;
  proj_tile(t, rtn, nvt, vt, rt);
  const int tid = threadIdx.x;
  if (PASS == 1)
    for (int r = tid; r < G::BM; r += G::NT) {
      const int gr = rt * G::BM + r;
      s_thr[r] = gr < rows ? thr[gr] : 0xFFFFFFFFu;
    }
  f32x16 acc[G::FM][G::FN];
  const Operand<T> A{hk, ldk, static_cast<long>((d + G::BK - 1) / G::BK) * ldk * G::BK, rt * G::BM, rows, d};
  const Operand<T> B{W, d, static_cast<long>(v) * d, vt * G::BN, v, d};
  G::run(A, B, 0, d, smem, acc);  // ends with a barrier: s_thr is visible

  const int lane = tid & 63, wave = tid >> 6, wm = wave / G::WAVES_COLS, wn = wave % G::WAVES_COLS;
  const int half = lane >> 5;
  const int c0 = wn * G::WN + 4 * half;  // column in tile of element 4 g + e of atom j: c0 + 32 j + 8 g + e
  const int r0 = wm * G::WM + (lane & 31);
  const int ncols = min(G::BN, v - vt * G::BN);
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    const int row = r0 + 32 * i, grow = rt * G::BM + row;
    if (grow >= rows) continue;
    if (PASS == 0) {
      uint32_t m[2] = {0u, 0u};  // groups j * 4 + g below 6 / from 6: 24 columns each
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c0 + 32 * j + 8 * g + e < ncols) {
              uint32_t& mm = m[(j * 4 + g) < 6 ? 0 : 1];
              mm = max(mm, ordered_key(acc[i][j][4 * g + e]));
            }
      uint32_t* out = lmax + (static_cast<long>(grow) * nvt + vt) * kTopkLanes + (wn * 2 + half) * 2;
      out[0] = m[0];  // 0: no column here
      out[1] = m[1];
      continue;
    }
    const uint32_t th = s_thr[row];
    int nh = 0;
#pragma unroll
    for (int j = 0; j < G::FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          nh += (c0 + 32 * j + 8 * g + e < ncols && ordered_key(acc[i][j][4 * g + e]) >= th) ? 1 : 0;
    if (nh > 0) {  // rare: the row's top-K region
      int base = atomicAdd(cnt + grow, nh);
      uint64_t* out = cand + static_cast<long>(grow) * kTopkCap;
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = c0 + 32 * j + 8 * g + e;
            const uint32_t key = ordered_key(acc[i][j][4 * g + e]);
            if (col < ncols && key >= th) {
              if (base < kTopkCap)
                out[base] = (static_cast<uint64_t>(key) << 32) |
                            static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(vt * G::BN + col));
              ++base;
            }
          }
    }
  }
}

// One workgroup per row: sort the row's candidate keys (bitonic, in LDS,
// descending) and write the first K.  A row with more than kTopkCap
// candidates is counted in *overflow (its record is then the best K of the
// kept ones, not necessarily the exact top K).
__global__ __launch_bounds__(256) void k_topk_select(const int* __restrict__ cnt,
                                                     const uint64_t* __restrict__ cand, int K,
                                                     int32_t* __restrict__ ids, float* __restrict__ logits,
                                                     int* __restrict__ overflow) {
  __shared__ uint64_t s[kTopkCap];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int c = cnt[row];
  const int m = c < kTopkCap ? c : kTopkCap;
  if (c > kTopkCap && tid == 0 && overflow) atomicAdd(overflow, 1);
  int P = 1;
  while (P < m) P <<= 1;
  const uint64_t* src = cand + static_cast<long>(row) * kTopkCap;
  for (int i = tid; i < P; i += 256) s[i] = i < m ? src[i] : 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P / 2; i += 256) {
        const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
        const bool desc = (lo & size) == 0;  // blocks alternate; the final merge is descending
        const uint64_t a = s[lo], b = s[hi];
        if ((a < b) == desc) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < K; j += 256) {
    const long o = static_cast<long>(row) * K + j;
    if (j < m) {
      const uint64_t key = s[j];
      ids[o] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
      logits[o] = key_value(static_cast<uint32_t>(key >> 32));
    } else {
      ids[o] = -1;
      logits[o] = -INFINITY;
    }
  }
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t words, uint32_t value) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < words) p[i] = value;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int dh_split_for(int chunk, int d, int ldz, int* kslice) {
  // Split the V reduction so the grid fills the 256 compute units with
  // little tail: the smallest split whose last wave of workgroups is >= 90%
  // full, at least 8 k tiles per slice.
  const int mt = (chunk + kDhBM - 1) / kDhBM, nt = (d + kDhBN - 1) / kDhBN;
  const int tiles = mt * nt;
  const int bk = 64;  // k tile of the bf16 engine (the fp32 engine's 32 divides it)
  int best = 1;
  for (int s = 1; s <= kMaxSplit; ++s) {
    if (static_cast<long>(ldz) / s < 8L * bk) break;
    const long wg = static_cast<long>(tiles) * s;
    const long full = (wg + 255) / 256 * 256;
    best = s;
    if (wg >= 200 && wg * 10 >= full * 9) break;
  }
  int ks = (ldz + best - 1) / best;
  ks = (ks + bk - 1) / bk * bk;
  *kslice = ks;
  return (ldz + ks - 1) / ks;
}

void launch_prep(const ChunkArgs& a, hipStream_t s) {
  const dim3 grid((a.rows + 3) / 4), block(256);
  if (a.t_bf16)
    k_prep<uint16_t><<<grid, block, 0, s>>>(a.ids, static_cast<const uint16_t*>(a.logits), a.mask, a.rows,
                                            a.k, a.v, a.nvt, 1.0f / a.tau, a.keys, a.psort, a.zgs, a.negent,
                                            a.ssum, a.lb);
  else
    k_prep<float><<<grid, block, 0, s>>>(a.ids, static_cast<const float*>(a.logits), a.mask, a.rows, a.k,
                                         a.v, a.nvt, 1.0f / a.tau, a.keys, a.psort, a.zgs, a.negent, a.ssum, a.lb);
}

void launch_fwd_proj(const ChunkArgs& a, hipStream_t s) {
  const int rtn = (a.rows + kProjBM - 1) / kProjBM;
  const dim3 grid(xcd_grid(rtn * a.nvt)), block(ProjGemmX<uint16_t>::NT);
  if (a.x_bf16)
    k_fwd_proj<uint16_t><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(a.hk), a.ldk,
                                                static_cast<const uint16_t*>(a.W), a.rows, a.d, a.v,
                                                a.nvt, a.k, a.lb, a.keys, a.zgs, a.pm, a.ps, a.zc, a.ldz,
                                                kLog2e / a.tau);
  else
    k_fwd_proj<float><<<grid, block, 0, s>>>(static_cast<const float*>(a.hk), a.ldk, static_cast<const float*>(a.W),
                                             a.rows, a.d, a.v, a.nvt, a.k, a.lb, a.keys, a.zgs, a.pm,
                                             a.ps, a.zc, a.ldz, kLog2e / a.tau);
}

void launch_merge(const ChunkArgs& a, float* lse, float* row_loss, float* zg, hipStream_t s) {
  k_merge<<<dim3((a.rows + 3) / 4), dim3(256), 0, s>>>(a.pm, a.ps, a.nvt, a.keys, a.psort, a.zgs, a.negent,
                                                      a.ssum, a.mask, a.rows, a.k, lse, row_loss, zg,
                                                      a.rl, kLog2e / a.tau, 1.0 / static_cast<double>(a.tau),
                                                      static_cast<double>(a.tau) * static_cast<double>(a.tau));
}

void launch_loss_fold(const ChunkArgs& a, int sub, int first, int last, float* loss, hipStream_t s) {
  k_loss_fold<<<dim3(1), dim3(256), 0, s>>>(a.rl, a.rows, sub, a.loss_acc, first, last, loss);
}

void launch_zero_loss(float* loss, hipStream_t s) { k_zero_loss<<<dim3(1), dim3(1), 0, s>>>(loss); }

void launch_bwd_dz(const ChunkArgs& a, const float* lse, const float* g, hipStream_t s) {
  const int rtn = (a.rows + kProjBM - 1) / kProjBM;
  const dim3 grid(xcd_grid(rtn * a.nvt)), block(ProjGemmX<uint16_t>::NT);
  if (a.x_bf16)
    k_bwd_dz<uint16_t><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(a.hk), a.ldk,
                                              static_cast<const uint16_t*>(a.W), a.rows, a.d, a.v, a.nvt,
                                              a.k, a.ldz, a.lb, a.keys, a.psort, a.ssum, a.mask, lse, g,
                                              static_cast<uint16_t*>(a.dz), kLog2e / a.tau, a.tau);
  else
    k_bwd_dz<float><<<grid, block, 0, s>>>(static_cast<const float*>(a.hk), a.ldk, static_cast<const float*>(a.W),
                                           a.rows, a.d, a.v, a.nvt, a.k, a.ldz, a.lb, a.keys, a.psort,
                                           a.ssum, a.mask, lse, g, static_cast<float*>(a.dz), kLog2e / a.tau,
                                           a.tau);
}

void launch_dz_cached(const ChunkArgs& a, const float* lse, const float* g, hipStream_t s) {
  // One thread per 8 columns of a row of the block rows the chunk touches;
  // those go in slices of at most 2^31 threads (a launch's work-item count
  // must fit in 32 bits).
  const long per_rb = static_cast<long>(a.ldz) / 32 * 128;  // threads per block row
  const long slice = (1L << 31) / per_rb;
  const long rb_first = a.dz_row0 / 32, rb_end = (static_cast<long>(a.dz_row0) + a.rows + 31) / 32;
  for (long rb = rb_first; rb < rb_end; rb += slice) {
    const int nrb = static_cast<int>(rb_end - rb < slice ? rb_end - rb : slice);
    const long threads = nrb * per_rb;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256)), block(256);
    if (a.x_bf16)
      k_dz_cached<uint16_t><<<grid, block, 0, s>>>(a.zc, a.ldz, a.dz_row0, a.rows, static_cast<int>(rb), nrb, a.v,
                                                   a.k, a.nvt, a.lb, a.keys, a.psort, a.ssum, a.mask, lse, g,
                                                   static_cast<uint16_t*>(a.dz), kLog2e / a.tau, a.tau);
    else
      k_dz_cached<float><<<grid, block, 0, s>>>(a.zc, a.ldz, a.dz_row0, a.rows, static_cast<int>(rb), nrb, a.v,
                                                a.k, a.nvt, a.lb, a.keys, a.psort, a.ssum, a.mask, lse, g,
                                                static_cast<float*>(a.dz), kLog2e / a.tau, a.tau);
  }
}

void launch_fill_u32(uint32_t* p, size_t words, uint32_t value, hipStream_t s) {
  if (words == 0) return;
  k_fill_u32<<<dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, s>>>(p, words, value);
}

void launch_topk_maxima(const ChunkArgs& a, uint32_t* lmax, hipStream_t s) {
  const int rtn = (a.rows + kProjBM - 1) / kProjBM;
  const dim3 grid(xcd_grid(rtn * a.nvt)), block(ProjGemmX<uint16_t>::NT);
  if (a.x_bf16)
    k_topk_pass<uint16_t, 0><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(a.hk), a.ldk,
                                                    static_cast<const uint16_t*>(a.W), a.rows, a.d, a.v, a.nvt,
                                                    lmax, nullptr, nullptr, nullptr);
  else
    k_topk_pass<float, 0><<<grid, block, 0, s>>>(static_cast<const float*>(a.hk), a.ldk, static_cast<const float*>(a.W),
                                                 a.rows, a.d, a.v, a.nvt, lmax, nullptr, nullptr, nullptr);
}

void launch_topk_threshold(const ChunkArgs& a, const uint32_t* lmax, uint32_t* thr, int* cnt, hipStream_t s) {
  const int nmax = a.nvt * kTopkLanes;
  if (nmax <= 256 * kTopkRegKeys)
    k_topk_threshold_reg<<<dim3(a.rows), dim3(256), 0, s>>>(lmax, nmax, a.k, thr, cnt);
  else
    k_topk_threshold<<<dim3(a.rows), dim3(256), 0, s>>>(lmax, nmax, a.k, thr, cnt);
}

void launch_topk_collect(const ChunkArgs& a, const uint32_t* thr, int* cnt, uint64_t* cand, hipStream_t s) {
  const int rtn = (a.rows + kProjBM - 1) / kProjBM;
  const dim3 grid(xcd_grid(rtn * a.nvt)), block(ProjGemmX<uint16_t>::NT);
  if (a.x_bf16)
    k_topk_pass<uint16_t, 1><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(a.hk), a.ldk,
                                                    static_cast<const uint16_t*>(a.W), a.rows, a.d, a.v, a.nvt,
                                                    nullptr, thr, cnt, cand);
  else
    k_topk_pass<float, 1><<<grid, block, 0, s>>>(static_cast<const float*>(a.hk), a.ldk, static_cast<const float*>(a.W),
                                                 a.rows, a.d, a.v, a.nvt, nullptr, thr, cnt, cand);
}

void launch_topk_select(const ChunkArgs& a, const int* cnt, const uint64_t* cand, int32_t* ids, float* logits,
                        int* overflow, hipStream_t s) {
  k_topk_select<<<dim3(a.rows), dim3(256), 0, s>>>(cnt, cand, a.k, ids, logits, overflow);
}

void launch_bwd_dh(const ChunkArgs& a, float* dH, hipStream_t s) {
  const int mtn = (a.rows + kDhBM - 1) / kDhBM, ntn = (a.d + kDhBN - 1) / kDhBN;
  const int split = a.dh_split;
  const dim3 grid(xcd_grid(mtn * ntn * split)), block(DhGemm<uint16_t>::NT);
  float* out = split == 1 ? dH : a.dhp;
  const long stride = static_cast<long>(a.rows) * a.d;
  if (a.x_bf16)
    k_bwd_dh<uint16_t><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(a.dz), a.ldz,
                                              static_cast<const uint16_t*>(a.W), a.rows, a.d, a.v, split,
                                              a.dh_kslice, out, stride);
  else
    k_bwd_dh<float><<<grid, block, 0, s>>>(static_cast<const float*>(a.dz), a.ldz,
                                           static_cast<const float*>(a.W), a.rows, a.d, a.v, split,
                                           a.dh_kslice, out, stride);
}

void launch_dh_reduce(const ChunkArgs& a, float* dH, hipStream_t s) {
  if (a.dh_split <= 1) return;
  const long count = static_cast<long>(a.rows) * a.d;  // d % 8 == 0, so count % 4 == 0
  const long nthreads = count / 4;
  k_dh_reduce<<<dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256), 0, s>>>(a.dhp, a.dh_split, count,
                                                                                       count, dH);
}

void launch_transpose_h(const ChunkArgs& a, hipStream_t s) {
  if (a.ht_span <= 0) return;
  const dim3 grid((a.ht_span + 63) / 64, (a.d + 63) / 64), block(256);
  if (a.x_bf16)
    k_transpose_h<uint16_t><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(a.H), a.rows, a.d,
                                                   static_cast<uint16_t*>(a.ht), a.ldt, a.ht_off, a.ht_span);
  else
    k_transpose_h<float><<<grid, block, 0, s>>>(static_cast<const float*>(a.H), a.rows, a.d,
                                                static_cast<float*>(a.ht), a.ldt, a.ht_off, a.ht_span);
}

void launch_tile_h(const ChunkArgs& a, hipStream_t s) {
  const int row_bytes = a.d * (a.x_bf16 ? 2 : 4);
  const int nkt = (row_bytes + 63) / 64;
  const dim3 grid(static_cast<unsigned>((a.rows + 31) / 32), static_cast<unsigned>((nkt + 1) / 2)), block(256);
  k_tile_h<<<grid, block, 0, s>>>(static_cast<const char*>(a.H), a.rows, row_bytes, static_cast<char*>(a.hk),
                                  a.ldk, nkt);
}

void launch_bwd_dw(const ChunkArgs& a, float* dW, hipStream_t s) {
  const int mtn = (a.v + kDwBM - 1) / kDwBM, ntn = (a.d + kDwBN - 1) / kDwBN;
  const dim3 grid(xcd_grid(mtn * ntn)), block(DwGemm<uint16_t>::NT);
  if (a.x_bf16)
    k_bwd_dw<uint16_t><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(a.dz), a.ldz,
                                              static_cast<const uint16_t*>(a.ht), a.ldt, a.rows, a.d, a.v, dW);
  else
    k_bwd_dw<float><<<grid, block, 0, s>>>(static_cast<const float*>(a.dz), a.ldz,
                                           static_cast<const float*>(a.ht), a.ldt, a.rows, a.d, a.v, dW);
}

}  // namespace kd
