// skv_block.h -- workgroup-wide scans for the 1024-thread selection kernels.
#pragma once
#include "skv_common.h"

namespace skv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wave, on DPP: shifts by 1, 2, 4
// and 8 lanes inside each row of 16 (lanes shifted in read zero), then the
// total of row 0 and of row 2 broadcast into rows 1 and 3 (row_bcast:15), then
// the total of rows 0-1 into rows 2 and 3 (row_bcast:31).  No LDS round trips.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum of one uint32 per thread over the workgroup; *total
// receives the sum.  Uses sm_w (kSelWaves + 1 words).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sm_w, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sm_w[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const uint32_t t = wave_incl_scan(lane < kSelWaves ? sm_w[lane] : 0u);
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
