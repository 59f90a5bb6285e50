// merge.hip -- log-sum-exp merge of split-K attention partials.
//
// Split-K decoding ("Where Activation Sparsity and KV-Cache Sparsity Cross
// ...", "Speedup Across Context" and "The Attention Baseline") cuts a head's
// key set into chunks; chunk c leaves (m_c, l_c, acc_c[d]) with m_c the chunk
// max of the log2-domain logits, l_c = sum 2^(l - m_c), acc_c = sum 2^(l - m_c) v.
// The exact softmax over the union is
//   M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  out = sum_c acc_c 2^(m_c - M) / L,
//   lse = (M + log2 L) ln 2,
// and an empty union (L = 0) gives out = 0, lse = -inf.
//
// One workgroup per output row and no barrier: each wave owns 32 columns
// (eight float4 columns) and merges them over every chunk by itself.  Lane
// (split c8 = lane / 8, column lane % 8) loads chunks c8, c8 + 8, ... in one
// round; every wave takes M over all chunks (a wave maximum), each chunk's
// weight 2^(m_c - M) is independent, and the eight chunk splits of a column
// are added across lanes in a fixed order (deterministic).
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

// Sum over the lanes l, l + 8, ..., l + 56 of a wave (the eight chunk splits
// of one column): row_ror:8 pairs lanes l and l ^ 8 inside each row of 16,
// then the 16- and 32-lane swaps.
__device__ __forceinline__ float split_sum(float y) {
  y += dpp<0x128>(y);
  y = xor16_sum(y);
  return xor32_sum(y);
}

template <int D, int kBatch>  // kBatch: chunks per lane (8 chunk splits per wave)
__global__ __launch_bounds__(2 * D) void merge_kernel(const MergeArgs a) {
  constexpr int kThreads = 2 * D;  // D / 32 waves of 32 columns
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.clear_ctr && blockIdx.x == 0)  // the one-call step's counters, for its next call
    for (int i = tid; i < a.clear_heads; i += kThreads) {
      a.clear_ctr[32 * i] = 0u;
      a.clear_ctr[32 * i + 16] = 0u;
    }
  const int Rh = a.rows_per_head;
  const int h = blockIdx.x % a.n_kv_heads;  // kv head h on the XCD that ran its chunks
  const int r = blockIdx.x / a.n_kv_heads;
  const int c8 = lane >> 3, col = wave * 8 + (lane & 7);  // col: float4 column
  const float* ml = a.part_ml + ((int64_t)h * a.cph * Rh + r) * 2;   // chunk stride Rh*2
  const float* pa = a.part_acc + ((int64_t)h * a.cph * Rh + r) * D;  // chunk stride Rh*D

  int nch = a.cph;
  float M = kNegInf, L = 0.0f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  // rounds of 8 kBatch chunks (one round for every plan but the longest
  // work lists), each rescaling what the earlier ones summed
  for (int c0 = 0; c0 < nch; c0 += 8 * kBatch) {
    float bm[kBatch], bl[kBatch];
    float4 ba[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {  // unconditional (clamped) loads, all in flight
      const int c = c0 + c8 + 8 * b;
      const int cc = c < a.cph ? c : a.cph - 1;
      bm[b] = ml[(int64_t)cc * Rh * 2];
      bl[b] = ml[(int64_t)cc * Rh * 2 + 1];
      ba[b] = *reinterpret_cast<const float4*>(pa + (int64_t)cc * Rh * D + col * 4);
    }
    if (c0 == 0 && a.nch) {  // sparse: chunks past the head's count hold stale data
      nch = a.nch[h];
      nch = nch < 1 ? 1 : (nch > a.cph ? a.cph : nch);
    }
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (c0 + c8 + 8 * b >= nch) bm[b] = kNegInf;
      mx = fmaxf(mx, bm[b]);
    }
    const float Mn = fmaxf(M, wave_max(mx));  // wave-uniform
    if (Mn != kNegInf) {
      const float sc = M == kNegInf ? 0.0f : fast_exp2(M - Mn);
      L *= sc;
      A.x *= sc; A.y *= sc; A.z *= sc; A.w *= sc;
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        // empty or unused slots (m = -inf) contribute nothing, whatever their
        // (possibly stale) l and acc hold
        const bool live = bm[b] != kNegInf;
        const float w = live ? fast_exp2(bm[b] - Mn) : 0.0f;
        L = fmaf(w, live ? bl[b] : 0.0f, L);
        const float4 av = live ? ba[b] : make_float4(0.f, 0.f, 0.f, 0.f);
        A.x = fmaf(w, av.x, A.x); A.y = fmaf(w, av.y, A.y);
        A.z = fmaf(w, av.z, A.z); A.w = fmaf(w, av.w, A.w);
      }
      M = Mn;
    }
  }
  L = split_sum(L);
  A.x = split_sum(A.x); A.y = split_sum(A.y); A.z = split_sum(A.z); A.w = split_sum(A.w);
  if (c8 == 0) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    A.x *= inv; A.y *= inv; A.z *= inv; A.w *= inv;
    const int G = a.group, Hq = a.n_kv_heads * G;
    const int64_t orow = (int64_t)(r / G) * Hq + h * G + (r % G);
    *reinterpret_cast<float4*>(a.out + orow * D + col * 4) = A;
    if (tid == 0 && a.lse) a.lse[orow] = L > 0.0f ? (M + log2f(L)) * kLn2 : kNegInf;
  }
}

template <int D>
hipError_t launch_d(const MergeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_kv_heads * a.rows_per_head));
  // the smallest batch that covers all chunks in one round of loads (8 beyond)
  const dim3 block(2 * D);
  if (a.cph <= 8)
    hipLaunchKernelGGL((merge_kernel<D, 1>), grid, block, 0, s, a);
  else if (a.cph <= 16)
    hipLaunchKernelGGL((merge_kernel<D, 2>), grid, block, 0, s, a);
  else if (a.cph <= 32)
    hipLaunchKernelGGL((merge_kernel<D, 4>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, 8>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(int d, const MergeArgs& a, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, s);
  if (d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
