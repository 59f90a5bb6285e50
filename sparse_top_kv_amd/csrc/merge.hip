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
// One workgroup per output row, two phases with no serial chain: every thread
// loads (m, l, acc[4 columns]) of its chunks in one round, the workgroup takes
// M, then each chunk weight 2^(m_c - M) is independent and the column sums are
// folded over the chunk splits through LDS in a fixed order (deterministic).
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int D, int kBatch>  // kBatch: chunks per thread per round of loads
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeArgs a) {
  constexpr int C4 = D / 4;              // float4 columns
  constexpr int NS = kThreads / C4;      // chunk splits
  __shared__ float4 sm_a[NS][C4];
  __shared__ float sm_l[NS];
  __shared__ float sm_red[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.clear_ctr && blockIdx.x == 0)  // the one-call step's counters, for its next call
    for (int i = tid; i < a.clear_heads; i += kThreads) {
      a.clear_ctr[32 * i] = 0u;
      a.clear_ctr[32 * i + 16] = 0u;
    }
  const int Rh = a.rows_per_head;
  const int h = blockIdx.x / Rh;
  const int r = blockIdx.x - h * Rh;
  const int col = tid % C4, sp = tid / C4;
  const float* ml = a.part_ml + ((int64_t)h * a.cph * Rh + r) * 2;   // chunk stride Rh*2
  const float* pa = a.part_acc + ((int64_t)h * a.cph * Rh + r) * D;  // chunk stride Rh*D

  float M_all = kNegInf;
  float L_t = 0.0f;
  float4 A_t = make_float4(0.f, 0.f, 0.f, 0.f);
  int nch = a.cph;
  // Rounds of NS * kBatch chunks (one round for every plan the host makes).
  for (int c0 = 0; c0 < nch; c0 += NS * kBatch) {
    float bm[kBatch], bl[kBatch];
    float4 ba[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {  // unconditional (clamped) loads, all in flight
      const int c = c0 + sp + b * NS;
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
      if (c0 + sp + b * NS >= nch) bm[b] = kNegInf;
      mx = fmaxf(mx, bm[b]);
    }
    mx = wave_max(mx);
    if (lane == 0) sm_red[wave] = mx;
    __syncthreads();
    float M = sm_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_red[w]);
    __syncthreads();
    if (M != kNegInf) {
      // rescale what earlier rounds summed, then add this round
      const float s = M_all == kNegInf ? 0.0f : fast_exp2(M_all - fmaxf(M_all, M));
      const float Mn = fmaxf(M_all, M);
      L_t *= s;
      A_t.x *= s; A_t.y *= s; A_t.z *= s; A_t.w *= s;
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        // empty or unused slots (m = -inf) contribute nothing, whatever their
        // (possibly stale) l and acc hold
        const bool live = bm[b] != kNegInf;
        const float w = live ? fast_exp2(bm[b] - Mn) : 0.0f;
        const float lv = live ? bl[b] : 0.0f;
        const float4 av = live ? ba[b] : make_float4(0.f, 0.f, 0.f, 0.f);
        L_t = fmaf(w, lv, L_t);
        A_t.x = fmaf(w, av.x, A_t.x); A_t.y = fmaf(w, av.y, A_t.y);
        A_t.z = fmaf(w, av.z, A_t.z); A_t.w = fmaf(w, av.w, A_t.w);
      }
      M_all = Mn;
    }
  }
  sm_a[sp][col] = A_t;
  if (col == 0) sm_l[sp] = L_t;
  __syncthreads();
  if (tid < C4) {
    float4 S = sm_a[0][tid];
    float L = sm_l[0];
#pragma unroll
    for (int k = 1; k < NS; ++k) {
      const float4 x = sm_a[k][tid];
      S.x += x.x; S.y += x.y; S.z += x.z; S.w += x.w;
      L += sm_l[k];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    S.x *= inv; S.y *= inv; S.z *= inv; S.w *= inv;
    const int G = a.group, Hq = a.n_kv_heads * G;
    const int64_t orow = (int64_t)(r / G) * Hq + h * G + (r % G);
    *reinterpret_cast<float4*>(a.out + orow * D + tid * 4) = S;
    if (tid == 0 && a.lse) a.lse[orow] = L > 0.0f ? (M_all + log2f(L)) * kLn2 : kNegInf;
  }
}

template <int D>
hipError_t launch_d(const MergeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_kv_heads * a.rows_per_head));
  constexpr int NS = kThreads / (D / 4);
  // smallest batch that covers all chunks in one round (8 beyond that)
  if (a.cph <= NS)
    hipLaunchKernelGGL((merge_kernel<D, 1>), grid, dim3(kThreads), 0, s, a);
  else if (a.cph <= 2 * NS)
    hipLaunchKernelGGL((merge_kernel<D, 2>), grid, dim3(kThreads), 0, s, a);
  else if (a.cph <= 4 * NS)
    hipLaunchKernelGGL((merge_kernel<D, 4>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, 8>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(int d, const MergeArgs& a, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, s);
  if (d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
