// skv_block.h -- workgroup-wide scans for the 1024-thread selection kernels.
#pragma once
#include "skv_common.h"

namespace skv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive prefix sum of one uint32 per thread over the workgroup; *total
// receives the sum.  Uses sm_w (kSelWaves + 1 words).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sm_w, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sm_w[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kSelWaves ? sm_w[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kSelWaves; off <<= 1) {
      const uint32_t y = __shfl_up(t, off, 64);
      if (lane >= off) t += y;
    }
    if (lane < kSelWaves) sm_w[lane] = t;  // inclusive per-wave prefix
  }
  __syncthreads();
  const uint32_t before = wave == 0 ? 0u : sm_w[wave - 1];
  *total = sm_w[kSelWaves - 1];
  __syncthreads();
  return before + x - v;
}

// Rank of a true flag among the true flags of the workgroup (exclusive), and
// the number of true flags; ballot-based.
__device__ __forceinline__ uint32_t block_flag_rank(bool f, uint32_t* sm_w, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t b = __ballot(f);
  const uint32_t in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
  if (lane == 0) sm_w[wave] = (uint32_t)__popcll(b);
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t c = sm_w[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  *total = all;
  __syncthreads();
  return before + in_wave;
}

}  // namespace
}  // namespace skv
