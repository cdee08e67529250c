// Block-tile matrix-core GEMM engine for gfx950 (CDNA4).
//
// C[BM x BN] (fp32, registers) = sum over a k range of A(m, k) * B(n, k).
// Each operand is either
//   KC  -- k contiguous in memory: element (r, k) at ptr[r * ld + k], or
//   KO  -- k outer:                element (r, k) at ptr[k * ld + r], or
//   KT  -- k tiled (a KC operand re-laid out by k tile): element (r, k) at
//          ptr[(k / BK) * ld * BK + r * BK + k % BK], ld = rows per k-tile
//          block, zero-padded in k up to a whole tile.
//   BL  -- blocked (dZ, as the dZ passes write it): a row-major [rows][ld]
//          matrix whose 32 x 32 blocks are each stored as 16-byte granules of
//          consecutive columns, granule-major: element (r, c) at byte
//          blk_offset(r, c) below.  Read as KC (dH: r = chunk row, k = c) or
//          as KO (dW: r = c, k = chunk row); either way a stage's loads are
//          runs of 256 or 512 contiguous bytes.
// The four contractions of the loss use: projection (KT, KC), dH = dZ W
// (KC, KO), dW = dZ^T H (KO, KT); the teacher top-K passes (KC, KC).  A KC tile reads 64 bytes of each of its
// rows, half of each 128-byte line it touches (the other half is the next k
// tile, fetched again one tile later); a KT tile is one contiguous block, so
// every line it touches is read whole.
//
// Data movement.  Tiles go from global memory straight into LDS with
// buffer_load ... lds (16 bytes per lane, one 1 KiB LDS block per wave
// instruction); out-of-range lanes get an offset past the buffer's record
// count, which the hardware turns into zeros, so bounds need no branches.
// A k tile holds 64 bytes of k per tile row (32 bf16 / 16 fp32), so each
// operand stage is R * 64 bytes in both layouts:
//   KC: [R rows][64 B of k], 16-byte chunk c of row r stored at c ^ ((r>>2)&3);
//   KO: [BK rows of k][R entries], 16-byte chunk c of row k stored at
//       c ^ fko(k) (bf16: 4*(k&3); fp32: 8*((k>>2)&1)).
//   BL read as KO: [R / 32 blocks][granule g][BK rows of k][16 B], the k row
//       of granule g stored at k ^ bl_swz(g) (the order of the global
//       blocks, each run of granules loaded as one contiguous piece);
//   BL read as KC: [4 chunks of the k tile][R rows][16 B] (the global order
//       of the granules: lane after lane, 16-byte rows of one granule).
// The swizzles make the matrix-core fragment reads bank-conflict free:
//   KC: ds_read_b128, lane l -> row l%32, k chunk from l/32;
//   KO bf16: ds_read_b64_tr_b16 (LDS transpose read), two per fragment;
//   KO fp32: four ds_read_b32.
// Eight waves (two per SIMD), one workgroup per CU, so one wave's LDS or
// barrier wait is covered by the other's MFMAs.  NS LDS stages: the loads of
// tile k+NS-1 are issued while tile k is computed.  One barrier per tile.
// Fragment schedule (registers are the limit: a 256 x 384 block holds 192
// fp32 accumulators per lane): B fragments are double-buffered across the
// two k steps of a tile; each A fragment is re-read in place right after the
// MFMAs of its row, so the next step's A is in flight while the remaining
// rows run.  The barrier sits after the first MFMA row of the second step,
// which gives the last A read of the first step time to land.
// Matrix-core atom: 32x32 output.  bf16: v_mfma_f32_32x32x16_bf16 (8 k per
// lane); fp32: four v_mfma_f32_32x32x2_f32 (one k per lane each).  A and B
// fragments use the same per-lane k assignment (lane group h = l/32 holds k
// = 8h..8h+7 for bf16, 4h..4h+3 within each fp32 fragment).  Output of an
// atom: lane l, element r -> row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

constexpr uint32_t kOOB = 0x80000000u;  // offset past every record count we set

// Blocked layout: byte offset of element (r, c) of a [rows][ld] matrix of
// SZ-byte elements (ld a multiple of 32; rows padded to a multiple of 32).
// Each block row of 32 rows is followed by kBlPad bytes, so that block rows
// do not start at the same offset modulo the memory channel interleave (at
// ld = 201216, 32 rows of bf16 are an exact multiple of 4 KiB).
constexpr long kBlPad = 256;
template <int SZ>
__host__ __device__ __forceinline__ long blk_pitch(long ld) { return 32 * ld * SZ + kBlPad; }
template <int SZ>
__host__ __device__ __forceinline__ long blk_offset(long r, long c, long ld) {
  constexpr int VPG = 16 / SZ;  // elements per granule
  return (r >> 5) * blk_pitch<SZ>(ld) + (c >> 5) * (1024 * SZ) + ((c & 31) / VPG) * 512 + (r & 31) * 16 +
         (c % VPG) * SZ;
}
// k-row swizzle of granule g in a blocked stage read as KO (bf16: bits 2-3
// of the 32 k rows; fp32: bits 0, 1 and 3 of the 16).
template <int SZ>
__device__ __forceinline__ int bl_swz(int g) {
  return SZ == 2 ? (4 * (g & 1) | 8 * (g >> 1)) : ((g & 3) | ((g & 4) << 1));
}

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations and does not wait on the other counters (gfx9 encoding).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {  // bf16 as raw bits
  static constexpr int VEC = 8;
  __device__ __forceinline__ static float to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  __device__ __forceinline__ static uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // nearest even
  }
  __device__ __forceinline__ static void mma(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
// Two fp32 values rounded to bf16 (nearest even) and packed low, high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

template <> struct Elem<float> {
  static constexpr int VEC = 4;
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float f) { return f; }
  __device__ __forceinline__ static void mma(f32x16& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), c, 0, 0, 0);
  }
};

// Buffer resource (gfx9 layout): base address, stride 0, record count in
// bytes (capped below kOOB so that offset kOOB is always out of range), and
// the raw-buffer format word.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t n = (bytes >> 31) != 0 ? 0x7FFFFFF0u : static_cast<uint32_t>(bytes);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xFFFFu, n, 0x00020000u};
}

// 16 bytes per lane from the buffer into LDS at m0 + 16 * lane.  Issued as
// inline assembly: the compiler's wait-count pass would otherwise make every
// later LDS read wait for these loads, including those of a stage nobody is
// reading yet.  Completion is tracked explicitly with s_waitcnt vmcnt.
// The LDS address is bound to m0 through a register constraint, so the
// compiler materialises m0 itself.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

// Workgroup barrier that orders LDS only: the fences lower to
// s_waitcnt lgkmcnt(0), so global->LDS loads of later tiles stay in flight
// (a full __syncthreads() would wait for every outstanding vector-memory op).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p)));
}

// f(integral_constant<int, I>) for I = I0 .. I1-1, unrolled at compile time.
template <int I0, int I1, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, I1>(f);
  }
}

// One operand of a block tile.
template <typename T>
struct Operand {
  const T* ptr;   // storage origin
  long ld;        // leading dimension (elements)
  long extent;    // elements addressable from ptr
  int r0;         // first tile row (m or n index)
  int r_lim;      // rows >= r_lim read as zero
  int k_lim;      // k >= k_lim reads as zero (multiple of VEC)
};

// Loads of one operand stage, R tile rows, NWAVES waves.  KT (with KC): the
// operand is k tiled; the stage layout in LDS is the KC one.
template <typename T, int R, bool KC, int NWAVES, bool KT = false, bool BL = false>
struct StageLoader {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int SZ = static_cast<int>(sizeof(T));
  static constexpr int BK = 64 / SZ;
  static constexpr int GPB = 32 * SZ / 16;     // BL: granules per 32 columns of a block row
  static constexpr int BLK = 32 * 32 * SZ;     // BL: bytes per 32 x 32 block
  static constexpr int NI = R * 64 / 1024 / NWAVES;  // 1 KiB wave instructions per wave per stage
  static constexpr int CPR = R * SZ / 16;     // KO: 16-byte chunks per k row
  static_assert(R * 64 % (1024 * NWAVES) == 0, "stage must split evenly over the waves");
  static_assert(KC || (CPR % 16 == 0), "k-outer tiles need >= 256 bytes per k row");
  static_assert(KC || !KT, "a k-tiled operand is k-contiguous within its tile");
  static_assert(!(KT && BL), "one layout per operand");
  static_assert(!BL || R % 32 == 0, "blocked tiles span whole blocks");

  // byte offset from the tile's base (k part excluded for KC); kOOB when the
  // row (KC) / column chunk (KO) lies outside the operand.  kOOB plus any k
  // offset stays past every record count.
  uint32_t voff[NI];

  __device__ __forceinline__ static int fko(int k) {
    return SZ == 2 ? 4 * (k & 3) : 8 * ((k >> 2) & 1);
  }
  // k-contiguous tiles: element offset along k of the lane's chunk (the same
  // for every instruction).  k-outer tiles need no such check: their buffer
  // record ends at row k_lim.
  __device__ __forceinline__ static int rel_k(int lane) { return ((lane & 3) ^ ((lane >> 4) & 3)) * VEC; }

  __device__ __forceinline__ void init(const Operand<T>& op, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int S = (wave * NI + i) * 64 + lane;
      if (BL && KC) {  // LDS slot (chunk c, row r) <- granule c of row r (the k part is added per tile)
        const int c = S / R, r = S % R;
        voff[i] = op.r0 + r < op.r_lim ? static_cast<uint32_t>((r >> 5) * blk_pitch<SZ>(op.ld) + c * 512 + (r & 31) * 16)
                                       : kOOB;
      } else if (BL) {  // LDS slot (block cb, granule g, k row kq) <- k row kq ^ bl_swz(g)
        const int kq = S % BK, g = (S / BK) % GPB, cb = S / (BK * GPB);
        voff[i] = op.r0 + cb * 32 + g * VEC < op.r_lim
                      ? static_cast<uint32_t>(cb * BLK + g * 512 + (kq ^ bl_swz<SZ>(g)) * 16)
                      : kOOB;
      } else if (KC) {
        const int r = S >> 2, p = S & 3;
        const int c = p ^ ((r >> 2) & 3);
        const long row_bytes = KT ? 64 : op.ld * SZ;
        voff[i] = op.r0 + r < op.r_lim ? static_cast<uint32_t>(r * row_bytes + c * 16) : kOOB;
      } else {
        const int k = S / CPR, p = S % CPR;
        const int c = p ^ fko(k);
        voff[i] = op.r0 + c * VEC < op.r_lim ? static_cast<uint32_t>(k * op.ld * SZ + c * 16) : kOOB;
      }
    }
  }

  // Buffer resource of the k tile starting at k0 (wave-uniform).  For a
  // k-outer tile the record stops at row k_lim, so rows past it read as zero.
  __device__ __forceinline__ u32x4 rsrc(const Operand<T>& op, int k0) const {
    if (BL) {  // extent counts the region's bytes / SZ
      const char* p = reinterpret_cast<const char*>(op.ptr);
      // KC: the tile's first block row; KO: the block row of k tile k0, from the tile's first block
      const long base = KC ? (op.r0 >> 5) * blk_pitch<SZ>(op.ld)
                           : static_cast<long>(k0 >> 5) * blk_pitch<SZ>(op.ld) + (op.r0 >> 5) * (1024 * SZ) +
                                 (k0 & 31) * 16;
      return make_rsrc(p + base, static_cast<uint64_t>(op.extent * SZ - base));
    }
    if (KT) {  // rows [r0, ld) of the block of k tile k0 / BK (64 bytes per row)
      const long base = (static_cast<long>(k0 / BK) * op.ld + op.r0) * BK;
      return make_rsrc(op.ptr + base, static_cast<uint64_t>(op.ld - op.r0) * 64);
    }
    if (KC) {
      const long base = static_cast<long>(op.r0) * op.ld;
      return make_rsrc(op.ptr + base, static_cast<uint64_t>(op.extent - base) * SZ);
    }
    // rows [k0, k_lim) of the tile; extent >= k_lim * ld for every k-outer operand
    if (k0 >= op.k_lim) return make_rsrc(op.ptr, 0);
    const long base = static_cast<long>(k0) * op.ld + op.r0;
    return make_rsrc(op.ptr + base, static_cast<uint64_t>(static_cast<long>(op.k_lim - k0) * op.ld - op.r0) * SZ);
  }

  // Issue instructions [I0, I1) of the k tile starting at k0 into the stage
  // at LDS byte address `dst` (wave-uniform: the m0 values stay scalar).
  template <int I0, int I1>
  __device__ __forceinline__ void issue(const Operand<T>& op, const u32x4& rs, int k0, uint32_t dst,
                                        int wave) const {
    // k tiled: the buffer resource starts at the tile's block, whose k
    // padding holds zeros
    // (a blocked operand's k range is whole k tiles: no per-lane k test)
    const bool kc_ok = !KC || KT || BL || k0 + rel_k(threadIdx.x & 63) < op.k_lim;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const uint32_t o = BL ? (KC ? voff[i] + static_cast<uint32_t>((k0 >> 5) * BLK + (k0 & 31) * SZ * 32) : voff[i])
                         : (KC && !KT ? voff[i] + static_cast<uint32_t>(k0 * SZ) : voff[i]);
      lds_dma16(rs, kc_ok ? o : kOOB, dst + static_cast<uint32_t>((wave * NI + i) * 1024));
    }
  }
  __device__ __forceinline__ void issue_all(const Operand<T>& op, int k0, uint32_t dst, int wave) const {
    issue<0, NI>(op, rsrc(op, k0), k0, dst, wave);
  }
};

// Fragment read of one operand for a wave: 32 tile rows from row0, k step
// kk (16 k for bf16, 8 for fp32; two steps per k tile).
template <typename T, int R, bool KC, bool BL = false>
struct FragReader {
  static constexpr int SZ = static_cast<int>(sizeof(T));
  static constexpr int BK = 64 / SZ;
  __device__ __forceinline__ static u32x4 read(const char* stage, int row0, int kk, int lane) {
    if (BL && !KC) {  // blocked stage: [R / 32][granule][BK k rows][16 B]
      // row0 is a multiple of 32, so the lane's granule, swizzle and k rows
      // depend on the lane alone; the block and the k step are constant offsets
      const char* blk = stage + (row0 >> 5) * 2048;
      if (SZ == 2) {
        const int q = lane >> 4, s = lane & 15;
        const int g = 2 * (q & 1) + ((s & 3) >> 1), sw = bl_swz<SZ>(g);
        const int kl = 8 * (q >> 1) + (s >> 2);  // k row in the step, below 16: the swizzle keeps bit 4
        const char* p0 = blk + g * (BK * 16) + 8 * (s & 1) + kk * 256;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + ((kl ^ sw) << 4)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + (((kl + 4) ^ sw) << 4)));
        const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
        return u32x4{a[0], a[1], b[0], b[1]};
      } else {
        // the k row offsets differ per lane in their low bits (8 per lane); an
        // opaque copy of the lane id keeps the compiler from holding all 8 in
        // registers across the k loop (the fp32 dW kernel has none to spare)
        int ln;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
        const int h = ln >> 5, g = (ln & 31) >> 2, sw = bl_swz<SZ>(g);
        const char* p0 = blk + g * (BK * 16) + ((ln & 3) << 2);
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = *(const lds_u32*)(p0 + (((8 * kk + 4 * h + j) ^ sw) << 4));
        return v;
      }
    } else if (BL) {  // KC, blocked stage: [chunk][R rows][16 B]
      const int c = 2 * kk + (lane >> 5);
      return *(const lds_u32x4*)(stage + c * (R * 16) + (row0 + (lane & 31)) * 16);
    } else if (KC) {
      const int r = row0 + (lane & 31);
      const int c = 2 * kk + (lane >> 5);
      return *(const lds_u32x4*)(stage + r * 64 + ((c ^ ((r >> 2) & 3)) << 4));
    } else if (SZ == 2) {
      const int q = lane >> 4, s = lane & 15;
      const int n = row0 + 16 * (q & 1) + 4 * (s & 3);
      const int k = 16 * kk + 8 * (q >> 1) + (s >> 2);
      const int ch = ((n >> 3) ^ (4 * (k & 3))) << 4;
      const char* p0 = stage + k * (R * 2) + ch + ((n & 7) << 1);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * (R * 2)));
      const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
      return u32x4{a[0], a[1], b[0], b[1]};
    } else {
      const int n = row0 + (lane & 31), h = lane >> 5;
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 8 * kk + 4 * h + j;
        v[j] = *(const lds_u32*)(stage + k * (R * 4) + (((n >> 2) ^ (8 * h)) << 4) + ((n & 3) << 2));
      }
      return v;
    }
  }
};

// A_KT / B_KT: that operand is k tiled (KT above; requires it to be KC).
// A_BL: A is blocked (BL above).
// TRANS: the matrix cores take B as their first operand, so atom (i, j)
// holds the transposed product: element e of a lane is (row 32 i + (lane &
// 31), column 32 j + 8 (e >> 2) + 4 (lane >> 5) + (e & 3)) of the wave tile,
// i.e. each lane holds whole groups of 4 consecutive columns of FM rows.
template <typename T, int BM_, int BN_, bool A_KC, bool B_KC, int WAVES_M = 2, int WAVES_N = 4, int NS_ = 4,
          bool EARLY_BARRIER = false, bool A_KT = false, bool B_KT = false, bool SPREAD = false, bool TRANS = false,
          bool A_BL = false>
struct Gemm {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int SZ = static_cast<int>(sizeof(T));
  static constexpr int BK = 64 / SZ;             // k per tile
  static constexpr int NS = NS_;                 // LDS stages
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int WAVES_ROWS = WAVES_M, WAVES_COLS = WAVES_N;
  static constexpr int NT = 64 * NWAVES;         // two waves per SIMD by default
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * 64, B_BYTES = BN * 64;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NS * STAGE;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");

  using LA = StageLoader<T, BM, A_KC, NWAVES, A_KT, A_BL>;
  using LB = StageLoader<T, BN, B_KC, NWAVES, B_KT>;
  using RA = FragReader<T, BM, A_KC, A_BL>;
  using RB = FragReader<T, BN, B_KC>;
  static constexpr int NI = LA::NI + LB::NI;     // load instructions per wave per tile

  __device__ __forceinline__ static u32x4 read_a(const char* st, int kk, int wm, int i, int lane) {
    return RA::read(st, wm * WM + 32 * i, kk, lane);
  }
  __device__ __forceinline__ static void read_b(u32x4 (&b)[FN], const char* st, int kk, int wn, int lane) {
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = RB::read(st + A_BYTES, wn * WN + 32 * j, kk, lane);
  }
  __device__ __forceinline__ static void mma_row(f32x16 (&acc)[FM][FN], int i, const u32x4& a, const u32x4 (&b)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (TRANS)
        Elem<T>::mma(acc[i][j], b[j], a);
      else
        Elem<T>::mma(acc[i][j], a, b[j]);
    }
  }
  // wait until at most `tiles` tiles of this wave's loads are in flight
  __device__ __forceinline__ static void wait_tiles(int tiles) {
    static_assert(NS <= 5 && 4 * NI < 64, "vmcnt holds at most 63");
    if (tiles >= 4)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * NI));
    else if (tiles == 3)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * NI));
    else if (tiles == 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NI));
    else if (tiles == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  // acc = sum over k in [k_begin, k_end) of A(m, k) B(n, k).  Leaves LDS free
  // (a barrier follows the last tile).
  //   prologue: tiles 0..NS-2 in flight, wait for tile 0, barrier, read the
  //             step-0 fragments of tile 0;
  //   tile kt:  issue tile kt+NS-1 into the stage tile kt-1 used; read the
  //             step-1 B fragments; per row i: MFMAs of step 0, re-read A[i]
  //             for step 1; per row i: MFMAs of step 1 (after row 0: wait
  //             for own loads of tile kt+1, barrier, read its step-0 B), re-
  //             read A[i] for step 0 of tile kt+1.
  __device__ __forceinline__ static void run(const Operand<T>& A, const Operand<T>& B, int k_begin, int k_end,
                                             char* lds, f32x16 (&acc)[FM][FN]) {
    run(A, B, k_begin, k_end, lds, acc, ZeroAcc{});
  }
  struct ZeroAcc {
    static constexpr bool kLoads = false;
    __device__ __forceinline__ void operator()(f32x16 (&acc)[FM][FN]) const {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    }
  };
  // Same, with acc starting from what `init(acc)` puts there.  An init with
  // kLoads fills acc with vector memory loads: they are issued after the
  // prologue's tile loads (so both are in flight together) and the prologue
  // then waits for every load of the wave, so no wait for them is left for
  // the compiler to place inside the k loop.
  template <class Init>
  __device__ __forceinline__ static void run(const Operand<T>& A, const Operand<T>& B, int k_begin, int k_end,
                                             char* lds, f32x16 (&acc)[FM][FN], const Init& init) {
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int nk = (k_end - k_begin + BK - 1) / BK;
    if (nk <= 0) {
      init(acc);
      if constexpr (Init::kLoads) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      return;
    }
    Operand<T> a = A, b = B;
    a.k_lim = min(A.k_lim, k_end);
    b.k_lim = min(B.k_lim, k_end);
    LA la;
    LB lb;
    la.init(a, wave, lane);
    lb.init(b, wave, lane);
    // stage addresses as 32-bit LDS byte addresses (scalar arithmetic)
    const uint32_t lds0 = lds_addr(lds);
    auto issue_tile = [&](int t) {
      const uint32_t dst = lds0 + static_cast<uint32_t>((t % NS) * STAGE);
      la.issue_all(a, k_begin + t * BK, dst, wave);
      lb.issue_all(b, k_begin + t * BK, dst + A_BYTES, wave);
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) {
      if (t < nk) issue_tile(t);
    }
    init(acc);
    if constexpr (Init::kLoads)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else
      wait_tiles(min(NS - 2, nk - 1));
    lds_barrier();
    u32x4 af[FM], b0[FN], b1[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = read_a(lds, 0, wm, i, lane);
    read_b(b0, lds, 0, wn, lane);
    // One k tile.  LOAD: issue the loads of tile kt+NS-1; MORE: a tile kt+1
    // follows (read its step-0 fragments); wait: own tiles left in flight
    // when tile kt+1 is needed.  The loop below runs the tiles that issue a
    // load with constants for all three, so its body has no branch; the last
    // NS-1 tiles run after it.
    auto tile = [&](int kt, auto load_t, auto more_t, int wait) {
      constexpr bool LOAD = decltype(load_t)::value, MORE = decltype(more_t)::value;
      const char* cur = lds + (kt % NS) * STAGE;
      const char* nxt = lds + ((kt + 1) % NS) * STAGE;
      // SPREAD: the loads of tile kt+NS-1 go out in slices after each MFMA
      // row of step 0 (instructions [i NI / FM, (i + 1) NI / FM) after row
      // i, A's first) instead of all before the first row
      const int tn = kt + NS - 1;
      const uint32_t dst = lds0 + static_cast<uint32_t>((tn % NS) * STAGE);
      u32x4 rsa, rsb;
      if constexpr (LOAD && SPREAD) {
        rsa = la.rsrc(a, k_begin + tn * BK);
        rsb = lb.rsrc(b, k_begin + tn * BK);
      }
      if constexpr (LOAD && !SPREAD) issue_tile(tn);
      // The scheduling fences keep every fragment read where it is written:
      // left alone, the scheduler sinks reads next to their consumers and
      // exposes the LDS latency at every step.
      read_b(b1, cur, 1, wn, lane);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, FM>([&](auto I) {
        constexpr int i = decltype(I)::value;
        mma_row(acc, i, af[i], b0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LOAD && SPREAD) {
          constexpr int g0 = i * NI / FM, g1 = (i + 1) * NI / FM;
          constexpr int a0 = g0 < LA::NI ? g0 : LA::NI, a1 = g1 < LA::NI ? g1 : LA::NI;
          constexpr int b0i = g0 > LA::NI ? g0 - LA::NI : 0, b1i = g1 > LA::NI ? g1 - LA::NI : 0;
          if constexpr (a1 > a0) la.template issue<a0, a1>(a, rsa, k_begin + tn * BK, dst, wave);
          if constexpr (b1i > b0i) lb.template issue<b0i, b1i>(b, rsb, k_begin + tn * BK, dst + A_BYTES, wave);
        }
        af[i] = read_a(cur, 1, wm, i, lane);
        __builtin_amdgcn_sched_barrier(0);
      });
      // The wait and barrier for tile kt+1: after the first MFMA row of step
      // 1, or (EARLY_BARRIER) before it, where b0 is already free so the
      // first B fragments of tile kt+1 are read one MFMA row earlier.  No
      // fragment of tile kt is read from LDS in step 1 either way.
      if constexpr (EARLY_BARRIER) {
        wait_tiles(wait);
        lds_barrier();
        if constexpr (MORE) read_b(b0, nxt, 0, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        mma_row(acc, i, af[i], b1);
        __builtin_amdgcn_sched_barrier(0);
        if (!EARLY_BARRIER && i == 0) {
          wait_tiles(wait);  // tile kt+1 has landed (own loads)
          lds_barrier();     // tile kt+1 visible; stage of kt free
          if constexpr (MORE) read_b(b0, nxt, 0, wn, lane);
        }
        if constexpr (MORE) af[i] = read_a(nxt, 0, wm, i, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int kt = 0;
    for (; kt < nk - (NS - 1); ++kt) tile(kt, std::true_type{}, std::true_type{}, NS - 2);
    for (; kt < nk - 1; ++kt) tile(kt, std::false_type{}, std::true_type{}, nk - kt - 2);
    tile(kt, std::false_type{}, std::false_type{}, 0);
    __syncthreads();
  }
};

// Branch-free fp32 access to a row-major [rows][ld] region through a buffer
// resource: offsets past the region (or kOOB) read as zero / drop the write.
struct F32Region {
  __amdgpu_buffer_rsrc_t rs;
  __device__ __forceinline__ F32Region(float* base, long elems) {
    const long bytes = elems > 0 ? elems * 4 : 0;
    rs = __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0),
                                           static_cast<int>(bytes > 0x7FFFFFF0L ? 0x7FFFFFF0L : bytes),
                                           0x00020000);
  }
  // the b32 builtins move 32-bit integers: bit casts, not conversions
  __device__ __forceinline__ float load(uint32_t off) const {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
  __device__ __forceinline__ void store(float x, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, off, 0, 0);
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

// Output position of accumulator element e of atom (i, j) for a wave at
// (wm, wn): row / column inside the block tile.
template <class G>
__device__ __forceinline__ int acc_row(int wm, int i, int e, int lane) {
  return wm * G::WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
template <class G>
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * G::WN + 32 * j + (lane & 31);
}

}  // namespace kd
