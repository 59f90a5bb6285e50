// select.hip -- sinks + per-head top-K of the candidate range by radix select.
#include <limits.h>
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
#include "skv_block.h"

namespace skv {
namespace {

constexpr int kBins = 2048;

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


// ---------------------------------------------------------------------------
// Block-parallel path for long caches with few kv heads (a one-workgroup-per-
// head select would leave most CUs idle).  Candidates are cut into blocks of
// kBlk; three kernels, no global atomics, so the result is identical run to
// run.  The per-head steps between them are recomputed by every block of the
// head from the same data (cheaper than a one-workgroup-per-head launch):
//   1 per block: histogram of key bits [31:21]
//   2 per block: from all block histograms of its head, the bin d1 holding the
//                K-th key and how many to take from it, and where this block's
//                bin members go; copy them (key, index) in index order and
//                count the keys above the bin.  Block 0 records the head's
//                state, the sinks and the count.
//   3 per block: finish the radix select on the head's bin members (bits
//                [20:10], [9:0]) -> threshold key T and how many keys equal to
//                T are kept, lowest index first; this block's output offset;
//                write its kept indices
// ---------------------------------------------------------------------------
constexpr int kBlk = 4096;                 // candidates per block
constexpr int kStageCand = 8192;           // threshold-bin members staged in LDS
constexpr int kBlkPer = kBlk / kSelThreads;

struct SelGeom {  // per-head geometry shared by the three kernels
  int64_t c_lo, c_hi, ncand, nsink, K;
  int nb;         // blocks of this head
};

__device__ __forceinline__ SelGeom sel_geom(const SelectArgs& a, int h) {
  SelGeom g;
  const int64_t tail = a.n - a.n_recent > 0 ? a.n - a.n_recent : 0;
  g.nsink = a.n_sink < tail ? a.n_sink : tail;
  g.c_lo = a.n_sink;
  g.c_hi = a.n - a.n_recent;
  g.ncand = g.c_lo < g.c_hi ? g.c_hi - g.c_lo : 0;
  int64_t K = a.k_per_head ? a.k_per_head[h] : a.k_uniform;
  K = K < 0 ? 0 : K;
  K = K > g.ncand ? g.ncand : K;
  K = K > a.k_max ? a.k_max : K;
  g.K = K;
  g.nb = (int)((g.ncand + kBlk - 1) / kBlk);
  return g;
}

// Scratch layout (per kv head, nbm = blocks for the longest head).
struct SelWs {
  uint32_t* hist;    // [Hkv][nbm][2048]
  uint32_t* above;   // [Hkv][nbm]
  uint32_t* head;    // [Hkv][8]: mode, d1, krem, cbin
  uint32_t* ckey;    // [Hkv][n]
  int32_t* cidx;     // [Hkv][n]
  int nbm;
};

__host__ __device__ inline int sel_blocks_max(int64_t n) { return (int)((n + kBlk - 1) / kBlk); }

__host__ __device__ inline SelWs sel_ws(void* ws, int hkv, int64_t n) {
  SelWs w;
  w.nbm = sel_blocks_max(n);
  char* p = (char*)ws;
  auto take = [&](size_t bytes) {
    char* q = p;
    p += (bytes + 255) / 256 * 256;
    return q;
  };
  w.hist = (uint32_t*)take((size_t)hkv * w.nbm * 2048 * 4);
  w.above = (uint32_t*)take((size_t)hkv * w.nbm * 4);
  w.head = (uint32_t*)take((size_t)hkv * 8 * 4);
  w.ckey = (uint32_t*)take((size_t)hkv * n * 4);
  w.cidx = (int32_t*)take((size_t)hkv * n * 4);
  return w;
}

enum { kModeRadix = 0, kModeAll = 1, kModeNone = 2 };

__global__ __launch_bounds__(kSelThreads) void sel_hist1_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  const SelWs w = sel_ws(a.ws, a.n_kv_heads, a.n);
  const int h = blockIdx.x / w.nbm, b = blockIdx.x - h * w.nbm;
  const SelGeom g = sel_geom(a, h);
  if (b >= g.nb) return;
  const float* s = a.score + (int64_t)h * a.score_stride;
  const int tid = threadIdx.x;
  const int64_t j0 = g.c_lo + (int64_t)b * kBlk + kBlkPer * tid;  // this thread's candidates
  float sv[kBlkPer];
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) sv[u] = j0 + u < g.c_hi ? s[j0 + u] : 0.0f;
  for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u)
    if (j0 + u < g.c_hi) atomicAdd(&hist[score_key(sv[u]) >> 21], 1u);
  __syncthreads();
  uint32_t* out = w.hist + ((int64_t)h * w.nbm + b) * kBins;
  for (int i = tid; i < kBins; i += kSelThreads) out[i] = hist[i];
}

__global__ __launch_bounds__(kSelThreads) void sel_collect_kernel(const SelectArgs a) {
  __shared__ uint32_t sm_w[kSelWaves + 1];
  __shared__ uint32_t sm_digit, sm_krem, sm_base;
  const SelWs w = sel_ws(a.ws, a.n_kv_heads, a.n);
  const int h = blockIdx.x / w.nbm, b = blockIdx.x - h * w.nbm;
  const SelGeom g = sel_geom(a, h);
  if (b >= g.nb) return;
  const float* s = a.score + (int64_t)h * a.score_stride;
  const int tid = threadIdx.x;
  const int64_t j0 = g.c_lo + (int64_t)b * kBlk + kBlkPer * tid;
  float sv[kBlkPer];
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) sv[u] = j0 + u < g.c_hi ? s[j0 + u] : 0.0f;
  uint32_t* hd = w.head + (int64_t)h * 8;
  if (b == 0) {
    int32_t* out = a.idx + (int64_t)h * a.idx_stride;
    for (int64_t i = tid; i < g.nsink; i += kSelThreads) out[i] = (int32_t)i;
    if (tid == 0) a.count[h] = (int32_t)(g.nsink + g.K);
  }
  if (g.K == 0 || g.K == g.ncand) {  // nothing or everything: no radix passes
    if (b == 0 && tid == 0) hd[0] = g.K == 0 ? kModeNone : kModeAll;
    return;
  }
  // the top-11-bit bin of the K-th key, summed over the head's blocks
  const uint32_t* hist = w.hist + (int64_t)h * w.nbm * kBins;
  const int top = kBins - 1 - tid * 2;  // this thread's bins: top, top-1 (visited from the top)
  uint32_t c0 = 0, c1 = 0;
  // bins top - 1 and top are adjacent: one 8-byte load per block, eight
  // blocks in flight per round
  const uint2* hp = reinterpret_cast<const uint2*>(hist + top - 1);
  int bb = 0;
  for (; bb + 8 <= g.nb; bb += 8) {
    uint2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = hp[(int64_t)(bb + u) * (kBins / 2)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c0 += v[u].y;
      c1 += v[u].x;
    }
  }
  for (; bb < g.nb; ++bb) {
    const uint2 v = hp[(int64_t)bb * (kBins / 2)];
    c0 += v.y;
    c1 += v.x;
  }
  uint32_t total;
  const uint32_t krem = (uint32_t)g.K;
  const uint32_t above_bins = block_excl_scan(c0 + c1, sm_w, &total);
  if (above_bins < krem && krem <= above_bins + c0 + c1) {
    if (krem <= above_bins + c0) {
      sm_digit = (uint32_t)top;
      sm_krem = krem - above_bins;
    } else {
      sm_digit = (uint32_t)(top - 1);
      sm_krem = krem - above_bins - c0;
    }
  }
  __syncthreads();
  const uint32_t d1 = sm_digit;
  // members of bin d1 in the blocks before this one
  const uint32_t mine = tid < g.nb ? hist[(int64_t)tid * kBins + d1] : 0u;
  uint32_t cbin;
  const uint32_t off = block_excl_scan(mine, sm_w, &cbin);
  if (tid == b) sm_base = off;
  if (b == 0 && tid == 0) {
    hd[0] = kModeRadix;
    hd[1] = d1;
    hd[2] = sm_krem;
    hd[3] = cbin;
  }
  __syncthreads();
  // candidates in the threshold bin (kept in index order) and above it
  uint32_t key[kBlkPer], n_in = 0, n_ab = 0;
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) {
    const bool valid = j0 + u < g.c_hi;
    key[u] = score_key(sv[u]);
    n_in += (valid && (key[u] >> 21) == d1) ? 1u : 0u;
    n_ab += (valid && (key[u] >> 21) > d1) ? 1u : 0u;
  }
  uint32_t tot;  // counts <= kBlk < 2^16: both in one scan
  const uint32_t ex = block_excl_scan((n_in << 16) | n_ab, sm_w, &tot);
  uint32_t r = sm_base + (ex >> 16);
  uint32_t* ck = w.ckey + (int64_t)h * a.n;
  int32_t* ci = w.cidx + (int64_t)h * a.n;
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) {
    if (j0 + u < g.c_hi && (key[u] >> 21) == d1) {
      ck[r] = key[u];
      ci[r] = (int32_t)(j0 + u);
      ++r;
    }
  }
  if (tid == 0) w.above[(int64_t)h * w.nbm + b] = tot & 0xFFFFu;
}

__global__ __launch_bounds__(kSelThreads) void sel_write_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sm_w[kSelWaves + 1];
  __shared__ uint32_t sm_digit, sm_krem, sm_jt, sm_base;
  __shared__ uint32_t sm_kept[kSelThreads];
  // bin members staged in LDS when they fit (the usual case): the passes
  // below then read LDS instead of global memory
  __shared__ uint32_t sm_ck[kStageCand];
  __shared__ int32_t sm_ci[kStageCand];
  const SelWs w = sel_ws(a.ws, a.n_kv_heads, a.n);
  const int h = blockIdx.x / w.nbm, b = blockIdx.x - h * w.nbm;
  const SelGeom g = sel_geom(a, h);
  if (b >= g.nb) return;
  const int tid = threadIdx.x;
  const uint32_t* hd = w.head + (int64_t)h * 8;
  const uint32_t* ck = w.ckey + (int64_t)h * a.n;
  const int32_t* ci = w.cidx + (int64_t)h * a.n;
  // every independent load in one round: this block's scores, head state, the
  // blocks' counts above the bin, and (speculatively) the first kStageCand
  // bin members
  const float* s = a.score + (int64_t)h * a.score_stride;
  const int64_t j0 = g.c_lo + (int64_t)b * kBlk + kBlkPer * tid;
  float sv[kBlkPer];
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) sv[u] = j0 + u < g.c_hi ? s[j0 + u] : 0.0f;
  constexpr int kPre = kStageCand / kSelThreads;
  uint32_t pk[kPre];
  int32_t pi[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {  // rows hold n > kStageCand entries: in bounds
    pk[u] = ck[tid * kPre + u];
    pi[u] = ci[tid * kPre + u];
  }
  const uint32_t abv = tid < g.nb ? w.above[(int64_t)h * w.nbm + tid] : 0u;
  const uint32_t mode = hd[0];
  if (mode == kModeNone) return;  // uniform
  uint32_t T = 0;
  int64_t jt = INT64_MAX;  // every key >= T kept (mode all)
  uint32_t base = (uint32_t)(g.nsink + (int64_t)b * kBlk);
  if (mode == kModeRadix) {
    const uint32_t d1h = hd[1], krem0 = hd[2], C = hd[3];
    const bool staged = C <= (uint32_t)kStageCand;
    if (staged) {
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        sm_ck[tid * kPre + u] = pk[u];
        sm_ci[tid * kPre + u] = pi[u];
      }
      __syncthreads();
      ck = sm_ck;
      ci = sm_ci;
    }
    uint32_t prefix = d1h << 21, mask = 0xFFE00000u;
    uint32_t krem = krem0;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 10 : 0;
      const int nb = pass == 0 ? 2048 : 1024;
      for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < C; i += kSelThreads) {
        const uint32_t key = ck[i];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
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
    T = prefix;
    const uint32_t take = krem;
    // bin members in index order: the first `take` equal to T are kept;
    // count the kept members of every block
    sm_kept[tid] = 0u;
    if (tid == 0) sm_jt = 0xFFFFFFFFu;
    __syncthreads();
    auto keep_member = [&](uint32_t i, uint32_t key, uint32_t eq_rank) {
      const bool eq = key == T;
      if (key > T || (eq && eq_rank < take)) {
        const int32_t j = ci[i];
        atomicAdd(&sm_kept[(j - g.c_lo) / kBlk], 1u);
        if (eq && eq_rank == take - 1) sm_jt = (uint32_t)j;
      }
    };
    if (staged) {
      // kPre consecutive members per thread: one scan ranks the equal keys
      const uint32_t i0 = (uint32_t)tid * kPre;
      uint32_t n_eq = 0;
#pragma unroll
      for (int u = 0; u < kPre; ++u) n_eq += (i0 + u < C && ck[i0 + u] == T) ? 1u : 0u;
      uint32_t tot_eq;
      uint32_t eq_rank = block_excl_scan(n_eq, sm_w, &tot_eq);
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        const uint32_t i = i0 + u;
        if (i < C) {
          const uint32_t key = ck[i];
          keep_member(i, key, eq_rank);
          eq_rank += key == T ? 1u : 0u;
        }
      }
    } else {
      uint32_t eq_seen = 0;
#pragma unroll 1
      for (uint32_t t0 = 0; t0 < C; t0 += kSelThreads) {
        const uint32_t i = t0 + tid;
        const bool valid = i < C;
        const uint32_t key = valid ? ck[i] : 0u;
        uint32_t n_eq;
        const uint32_t eq_rank = eq_seen + block_flag_rank(valid && key == T, sm_w, &n_eq);
        if (valid) keep_member(i, key, eq_rank);
        eq_seen += n_eq;
      }
    }
    __syncthreads();
    // this block's output offset: sinks, then the kept keys of earlier blocks
    const uint32_t mine = tid < g.nb ? abv + sm_kept[tid] : 0u;
    uint32_t total;
    const uint32_t off = block_excl_scan(mine, sm_w, &total);
    if (tid == b) sm_base = (uint32_t)g.nsink + off;
    __syncthreads();
    base = sm_base;
    jt = take == 0 ? -1 : (int64_t)sm_jt;
  }
  bool keep[kBlkPer];
  uint32_t n_keep = 0;
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) {
    const int64_t j = j0 + u;
    const uint32_t key = score_key(sv[u]);
    keep[u] = j < g.c_hi && (key > T || (key == T && j <= jt));
    n_keep += keep[u] ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t pos = base + block_excl_scan(n_keep, sm_w, &tot);
  int32_t* out = a.idx + (int64_t)h * a.idx_stride;
  const uint32_t limit = (uint32_t)(g.nsink + g.K);
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) {
    if (keep[u]) {
      if (pos < limit) out[pos] = (int32_t)(j0 + u);  // never past the row
      ++pos;
    }
  }
}

// Block path for long rows and few heads; its per-head scans over blocks hold
// at most one block per thread (n <= kSelThreads * kBlk).
bool use_block_path(int32_t hkv, int64_t n) {
  return n > 16384 && n <= (int64_t)kSelThreads * kBlk && hkv < 64;
}

}  // namespace

size_t select_ws_bytes(int32_t n_kv_heads, int64_t n) {
  if (!use_block_path(n_kv_heads, n)) return 0;
  const SelWs w = sel_ws(nullptr, n_kv_heads, n);
  return (size_t)((char*)(w.cidx + (int64_t)n_kv_heads * n) - (char*)nullptr) + 256;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (!use_block_path(a.n_kv_heads, a.n)) {
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)a.n_kv_heads), dim3(kSelThreads), 0, stream, a);
    return hipGetLastError();
  }
  const unsigned grid_b = (unsigned)(a.n_kv_heads * sel_blocks_max(a.n));
  hipLaunchKernelGGL(sel_hist1_kernel, dim3(grid_b), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_collect_kernel, dim3(grid_b), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_write_kernel, dim3(grid_b), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
