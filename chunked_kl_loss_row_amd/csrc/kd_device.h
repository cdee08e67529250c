// Device building blocks for the fused chunked KL kernels (gfx950 / CDNA4).
//
// One block-tile GEMM engine serves all four contractions of the loss:
//   forward projection      Z  = H_c W^T     (both operands K-contiguous)
//   backward recomputation  Z  = H_c W^T     (same)
//   hidden-state gradient   dH = dZ W        (W read K-outer: rows are k)
//   weight gradient         dW = dZ^T H_c    (both operands K-outer)
// Tiles are staged through LDS in one layout -- [tile row][k], k contiguous,
// rows padded by 16 bytes -- so the matrix-core fragment reads are always one
// 16-byte ds_read per lane.  K-outer operands are transposed on the way in:
// each thread loads a VEC x VEC block (VEC rows of k, VEC consecutive columns)
// and transposes it in registers before the 16-byte LDS stores.
//
// Matrix-core atom: 16x16 output per wave instruction.  bf16 uses
// v_mfma_f32_16x16x32_bf16 (8 k-values per lane), fp32 uses four
// v_mfma_f32_16x16x4_f32 (one k-value per lane each).  A and B fragments are
// read with the same per-lane k assignment, so the product is independent of
// which k the hardware associates with a given register slot.  Output layout
// of a 16x16 atom: lane l, element r holds row 4*(l/16)+r, column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct Traits;

// bf16 stored as raw 16-bit patterns.
template <> struct Traits<uint16_t> {
  static constexpr int VEC = 8;   // elements per 16 bytes
  static constexpr int KF = 32;   // k extent of one fragment (4 lane groups x VEC)
  __device__ __forceinline__ static float to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  __device__ __forceinline__ static uint16_t from_f32(float f) {
    // round to nearest even (hardware conversion on gfx950)
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  }
  __device__ __forceinline__ static void mma(f32x4& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <> struct Traits<float> {
  static constexpr int VEC = 4;
  static constexpr int KF = 16;
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float f) { return f; }
  __device__ __forceinline__ static void mma(f32x4& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(b[j]), c,
                                               0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// reductions inside a group of 16 lanes (one row of a row-parallel pass)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float group16_max(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 16));
  return x;
}
__device__ __forceinline__ float group16_sum(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o, 16);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ---------------------------------------------------------------------------
// tile loaders: global -> registers -> LDS [R rows][BKP], k contiguous
// ---------------------------------------------------------------------------
// K-contiguous source: element (r, k) at src[r * ld + k].  Rows >= r_lim and
// k >= k_lim are zero-filled (k_lim must be a multiple of VEC).
template <typename T, int R, int NT>
struct LoaderKC {
  static constexpr int VEC = Traits<T>::VEC;
  static constexpr int BK = 128 / sizeof(T);
  static constexpr int BKP = BK + VEC;
  static constexpr int CPR = BK / VEC;           // 16-byte chunks per tile row (8)
  static constexpr int TOTAL = R * CPR;
  static constexpr int N = (TOTAL + NT - 1) / NT;
  u32x4 reg[N];

  __device__ __forceinline__ void load(const T* __restrict__ src, long ld, int r0, int r_lim,
                                       int k0, int k_lim, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPR, kc = c % CPR;
      const int gr = r0 + row, gk = k0 + kc * VEC;
      u32x4 v = {0u, 0u, 0u, 0u};
      if ((TOTAL % NT == 0 || c < TOTAL) && gr < r_lim && gk < k_lim)
        v = *reinterpret_cast<const u32x4*>(src + static_cast<long>(gr) * ld + gk);
      reg[i] = v;
    }
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT;
      if (TOTAL % NT == 0 || c < TOTAL) {
        const int row = c / CPR, kc = c % CPR;
        *reinterpret_cast<u32x4*>(lds + row * BKP + kc * VEC) = reg[i];
      }
    }
  }
};

// K-outer source: element (r, k) at src[k * ld + r].  Each thread moves
// VEC x VEC blocks; lanes vary fastest along k so the 16-byte LDS stores of a
// lane group fill one contiguous 128-byte tile row segment.  k >= k_lim and
// r >= r_lim are zero-filled (r_lim must be a multiple of VEC).
template <typename T, int R, int NT>
struct LoaderKO {
  static constexpr int VEC = Traits<T>::VEC;
  static constexpr int BK = 128 / sizeof(T);
  static constexpr int BKP = BK + VEC;
  static constexpr int KB = BK / VEC;            // blocks along k (8)
  static constexpr int TOTAL = KB * (R / VEC);
  static constexpr int N = (TOTAL + NT - 1) / NT;
  u32x4 reg[N][VEC];

  __device__ __forceinline__ void load(const T* __restrict__ src, long ld, int r0, int r_lim,
                                       int k0, int k_lim, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int b = tid + i * NT;
      const int kb = b % KB, rb = b / KB;
      const int gr = r0 + rb * VEC;
      const bool ok = (TOTAL % NT == 0 || b < TOTAL) && gr < r_lim;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int gk = k0 + kb * VEC + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok && gk < k_lim) v = *reinterpret_cast<const u32x4*>(src + static_cast<long>(gk) * ld + gr);
        reg[i][j] = v;
      }
    }
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int b = tid + i * NT;
      if (!(TOTAL % NT == 0 || b < TOTAL)) continue;
      const int kb = b % KB, rb = b / KB;
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        u32x4 o;
        if constexpr (sizeof(T) == 2) {
          // column c of the 8x8 block of 16-bit values: dword q packs rows 2q
          // (low half) and 2q+1 (high half)
          const int w = c >> 1, sh = (c & 1) * 16;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (reg[i][2 * q][w] >> sh) & 0xFFFFu;
            const uint32_t hi = (reg[i][2 * q + 1][w] >> sh) & 0xFFFFu;
            o[q] = lo | (hi << 16);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = reg[i][q][c];
        }
        *reinterpret_cast<u32x4*>(lds + (rb * VEC + c) * BKP + kb * VEC) = o;
      }
    }
  }
};

template <typename T, int R, int NT, bool KC>
struct Loader;
template <typename T, int R, int NT>
struct Loader<T, R, NT, true> : LoaderKC<T, R, NT> {};
template <typename T, int R, int NT>
struct Loader<T, R, NT, false> : LoaderKO<T, R, NT> {};

// ---------------------------------------------------------------------------
// block-tile GEMM engine
// ---------------------------------------------------------------------------
// C[BM x BN] = sum_k A[m][k] * B[n][k] over a k range, fp32 accumulation in
// registers.  WAVES_M x WAVES_N waves, each owning a (BM/WAVES_M) x
// (BN/WAVES_N) sub-tile of 16x16 atoms.
template <typename T, int BM_, int BN_, int WAVES_M, int WAVES_N, bool A_KC, bool B_KC>
struct Gemm {
  using Tr = Traits<T>;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int VEC = Tr::VEC;
  static constexpr int KF = Tr::KF;
  static constexpr int BK = 128 / sizeof(T);
  static constexpr int BKP = BK + VEC;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_ELEMS = BM * BKP, B_ELEMS = BN * BKP;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * static_cast<int>(sizeof(T));
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(BK % KF == 0, "k tile must hold whole fragments");

  using LA = Loader<T, BM, NT, A_KC>;
  using LB = Loader<T, BN, NT, B_KC>;

  // One K tile from LDS into the accumulators.
  __device__ __forceinline__ static void compute(const T* As, const T* Bs, f32x4 (&acc)[FM][FN],
                                                 int wm, int wn, int lane) {
    const int lr = lane & 15, lk = (lane >> 4) * VEC;
#pragma unroll
    for (int kk = 0; kk < BK / KF; ++kk) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const u32x4*>(As + (wm * WM + fm * 16 + lr) * BKP + kk * KF + lk);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bfr[fn] = *reinterpret_cast<const u32x4*>(Bs + (wn * WN + fn * 16 + lr) * BKP + kk * KF + lk);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) Tr::mma(acc[fm][fn], af[fm], bfr[fn]);
    }
  }

  // Accumulate over k in [k_begin, k_end).  A rows are m0.. (limit a_rlim),
  // B rows are n0.. (limit b_rlim); a_klim / b_klim bound the k index of each
  // operand's storage (zero fill past them).  Leaves LDS free on return
  // (a barrier follows the last tile).
  __device__ __forceinline__ static void run(const T* __restrict__ A, long lda, int m0, int a_rlim,
                                             int a_klim, const T* __restrict__ B, long ldb, int n0,
                                             int b_rlim, int b_klim, int k_begin, int k_end,
                                             T* lds, f32x4 (&acc)[FM][FN]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int a_kl = min(a_klim, k_end), b_kl = min(b_klim, k_end);
    const int nk = (k_end - k_begin + BK - 1) / BK;
    if (nk <= 0) return;
    LA la;
    LB lb;
    la.load(A, lda, m0, a_rlim, k_begin, a_kl, tid);
    lb.load(B, ldb, n0, b_rlim, k_begin, b_kl, tid);
    la.store(lds, tid);
    lb.store(lds + A_ELEMS, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      T* cur = lds + (kt & 1) * STAGE_ELEMS;
      T* nxt = lds + ((kt + 1) & 1) * STAGE_ELEMS;
      const bool more = kt + 1 < nk;
      if (more) {
        const int k1 = k_begin + (kt + 1) * BK;
        la.load(A, lda, m0, a_rlim, k1, a_kl, tid);
        lb.load(B, ldb, n0, b_rlim, k1, b_kl, tid);
      }
      compute(cur, cur + A_ELEMS, acc, wm, wn, lane);
      if (more) {
        la.store(nxt, tid);
        lb.store(nxt + A_ELEMS, tid);
      }
      __syncthreads();
    }
  }
};

// Workgroup -> tile mapping that keeps neighbouring tiles on one XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8); this maps
// the ids of XCD x onto a contiguous range of the linear tile order so tiles
// sharing operand panels share that XCD's L2.  Returns -1 for padding ids.
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int per = (total + 7) / 8;
  const int t = (bid % 8) * per + bid / 8;
  return t < total ? t : -1;
}
__host__ __forceinline__ int xcd_grid(int total) { return ((total + 7) / 8) * 8; }

}  // namespace kd
