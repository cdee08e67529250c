// Small device helpers shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

namespace kd {

constexpr float kLog2e = 1.4426950408889634f;

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x of another lane of the same row of 16 lanes, by a DPP lane permutation
// on the VALU (no LDS round trip).  Every lane of the row must be active.
template <int CTRL>
__device__ __forceinline__ float dpp16(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each half row
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within the row

// reductions inside a group of 16 lanes (one row of a row-parallel pass; the
// group is a DPP row: 16 aligned lanes, all active).  Partners: xor 1, xor 2,
// then the half-row mirror (quad <-> quad) and the row mirror (half <->
// half).  max and + are commutative, so every lane ends with the same bits.
__device__ __forceinline__ float group16_max(float x) {
  x = fmaxf(x, dpp16<kDppXor1>(x));
  x = fmaxf(x, dpp16<kDppXor2>(x));
  x = fmaxf(x, dpp16<kDppHalfMirror>(x));
  return fmaxf(x, dpp16<kDppMirror>(x));
}
__device__ __forceinline__ float group16_sum(float x) {
  x += dpp16<kDppXor1>(x);
  x += dpp16<kDppXor2>(x);
  x += dpp16<kDppHalfMirror>(x);
  return x + dpp16<kDppMirror>(x);
}
// reductions over the 64 lanes of a wave (fixed butterfly order)
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
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// fp32 <-> unsigned key with the same order (-0 and +0 made one value first)
__device__ __forceinline__ uint32_t ordered_key(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

}  // namespace kd
