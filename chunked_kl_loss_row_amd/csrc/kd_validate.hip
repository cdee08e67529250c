// Debug check of a teacher record: per unmasked row, ids outside [0, v) and
// ids that occur more than once.  The cached record lists, per position, the
// K most probable teacher tokens (agentlenshq.com page, section "1. Top-K
// Logit Cachingによるオフライン蒸留"), so a valid row holds K distinct ids of
// the vocabulary.  One wave per row; the row's ids are staged in LDS and
// every id is compared with the ids before it (K <= 256).
#include "kd_internal.h"
#include "kd_util.h"

namespace kd {

// out[0..1] = 0 (counts), out[2..3] = all ones (no row yet; -1 as int64)
__global__ __launch_bounds__(64) void k_validate_init(unsigned long long* __restrict__ out) {
  if (threadIdx.x < 4) out[threadIdx.x] = threadIdx.x < 2 ? 0ull : ~0ull;
}

// Rows [row0, row0 + n) of the record; ids and mask point at row 0.
__global__ __launch_bounds__(256) void k_validate(const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask,
                                                  long row0, long n, int K, int v,
                                                  unsigned long long* __restrict__ out) {
  __shared__ int32_t s_id[4][256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = row0 + static_cast<long>(blockIdx.x) * 4 + w;
  const bool live = row < row0 + n && (mask == nullptr || mask[row] != 0);
  int id[4];
  int out_of_range = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = lane + 64 * q;
    id[q] = (live && k < K) ? ids[row * K + k] : 0;
    if (live && k < K && (id[q] < 0 || id[q] >= v)) out_of_range = 1;
    s_id[w][k] = id[q];
  }
  __syncthreads();
  int repeated = 0;
  if (live) {
    for (int j = 0; j < K; ++j) {
      const int x = s_id[w][j];  // the same address for the whole wave
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = lane + 64 * q;
        if (j < k && k < K && x == id[q]) repeated = 1;
      }
    }
  }
  out_of_range = wave_sum(out_of_range);
  repeated = wave_sum(repeated);
  if (live && lane == 0) {
    const unsigned long long r = static_cast<unsigned long long>(row);
    if (out_of_range) {
      atomicAdd(&out[0], 1ull);
      atomicMin(&out[2], r);
    }
    if (repeated) {
      atomicAdd(&out[1], 1ull);
      atomicMin(&out[3], r);
    }
  }
}

void launch_validate(const int32_t* ids, const uint8_t* mask, long n, int K, int v, int64_t* out, hipStream_t s) {
  unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
  k_validate_init<<<1, 64, 0, s>>>(o);
  // 2^24 rows (2^30 work-items) per launch: a launch's work-item count must
  // fit in 32 bits
  constexpr long kSlice = 1L << 24;
  for (long r0 = 0; r0 < n; r0 += kSlice) {
    const long rows = n - r0 < kSlice ? n - r0 : kSlice;
    k_validate<<<static_cast<unsigned>((rows + 3) / 4), 256, 0, s>>>(ids, mask, r0, rows, K, v, o);
  }
}

}  // namespace kd
