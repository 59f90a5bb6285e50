// select.hip -- sinks + per-head top-K of the candidate range by radix select.
//
// Method: keep the attention sinks, the run of recent entries and the
// highest-scoring history entries of each kv head ("Where Activation Sparsity
// and KV-Cache Sparsity Cross ...", header figure and "Speedup Across
// Context"; argTopK per kv head in "Sparse-to-Dense ..." Sec. 3.2; per-head K
// from the SparseMM budgets).  Order: score descending, index ascending.
//
// One 1024-thread workgroup per kv head.  Scores map to order-preserving
// 32-bit keys (score_key); three counting passes over the candidates with
// 2048/2048/1024-bin LDS histograms fix the key T of the K-th entry and how
// many entries equal to T are taken.  A final pass in index order writes, via
// block-wide ballots, every key > T and the lowest-index `take` keys == T, so
// the output is ascending without a sort and ties go to the lowest index.
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 2048;

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

__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sm_w[kSelWaves + 1];
  __shared__ uint32_t sm_digit, sm_krem;

  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const float* s = a.score + (int64_t)h * a.score_stride;
  int32_t* out = a.idx + (int64_t)h * a.idx_stride;
  const int64_t n = a.n;
  const int64_t tail = n - a.n_recent > 0 ? n - a.n_recent : 0;
  const int64_t nsink = a.n_sink < tail ? a.n_sink : tail;
  const int64_t c_lo = a.n_sink, c_hi = n - a.n_recent;
  const int64_t ncand = c_lo < c_hi ? c_hi - c_lo : 0;
  int64_t K = a.k_per_head ? a.k_per_head[h] : a.k_uniform;
  K = K < 0 ? 0 : K;
  K = K > ncand ? ncand : K;
  K = K > a.k_max ? a.k_max : K;  // never write past the index row

  for (int64_t i = tid; i < nsink; i += kSelThreads) out[i] = (int32_t)i;
  if (tid == 0) a.count[h] = (int32_t)(nsink + K);
  if (K == 0) return;
  if (K == ncand) {
    for (int64_t i = tid; i < K; i += kSelThreads) out[nsink + i] = (int32_t)(c_lo + i);
    return;
  }

  // ---- radix passes: digits [31:21], [20:10], [9:0] of the key ----------
  uint32_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)K;  // how many of the remaining keys still to take
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0u;
    __syncthreads();
    for (int64_t j = c_lo + tid; j < c_hi; j += kSelThreads) {
      const uint32_t key = score_key(s[j]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // bins are visited from the top; thread t owns nb/1024 consecutive bins
    const int per = nb / kSelThreads;
    const int top = nb - 1 - tid * per;
    uint32_t mine = 0;
    for (int i = 0; i < per; ++i) mine += hist[top - i];
    uint32_t total;
    uint32_t above = block_excl_scan(mine, sm_w, &total);
    if (above < krem && krem <= above + mine) {
      for (int i = 0; i < per; ++i) {
        const uint32_t cb = hist[top - i];
        if (krem <= above + cb) {
          sm_digit = (uint32_t)(top - i);
          sm_krem = krem - above;
          break;
        }
        above += cb;
      }
    }
    __syncthreads();
    prefix |= sm_digit << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    krem = sm_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t take = krem;  // keys equal to T to keep, lowest index first

  // ---- compaction in index order ------------------------------------------
  uint32_t base = (uint32_t)nsink, eq_seen = 0;
#pragma unroll 1
  for (int64_t t0 = c_lo; t0 < c_hi; t0 += kSelThreads) {
    const int64_t j = t0 + tid;
    const bool valid = j < c_hi;
    const uint32_t key = valid ? score_key(s[j]) : 0u;
    const bool eq = valid && key == T;
    uint32_t n_eq;
    const uint32_t eq_rank = eq_seen + block_flag_rank(eq, sm_w, &n_eq);
    const bool keep = valid && (key > T || (eq && eq_rank < take));
    uint32_t n_keep;
    const uint32_t pos = base + block_flag_rank(keep, sm_w, &n_keep);
    if (keep && pos < (uint32_t)(nsink + K)) out[pos] = (int32_t)j;  // never past the row
    base += n_keep;
    eq_seen += n_eq;
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)a.n_kv_heads), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
