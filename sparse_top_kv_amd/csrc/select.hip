// select.hip -- sinks + per-head top-K of the candidate range by radix select.
//
// Method: keep the attention sinks, the run of recent entries and the
// highest-scoring history entries of each kv head ("Where Activation Sparsity
// and KV-Cache Sparsity Cross ...", header figure and "Speedup Across
// Context"; argTopK per kv head in "Sparse-to-Dense ..." Sec. 3.2; per-head K
// from the SparseMM budgets).  Order: score descending, index ascending.
//
// Scores map to order-preserving 32-bit keys (score_key); counting passes over
// digits of the keys fix the key T of the K-th entry and how many entries
// equal to T are taken; a pass in index order writes every key > T and the
// lowest-index `take` keys == T, so the output is ascending without a sort and
// ties go to the lowest index.  Three launch shapes:
//   - up to 16K candidates: one 1024-thread workgroup per kv head, keys in
//     registers, 4 or 16 per thread (select_small_kernel);
//   - longer rows with many kv heads (or rows past the block path's limit):
//     one 1024-thread workgroup per kv head (select_kernel), the first 16K
//     keys staged in LDS when the grid is small;
//   - long rows with few kv heads: workgroups over 4096-candidate blocks in
//     three kernels (sel_hist1_kernel, sel_collect_kernel, sel_write_kernel).
#include <limits.h>

#include "skv_common.h"
#include "skv_kernels.h"
#include "skv_block.h"
#include "../../include/sparsekv.h"

namespace skv {
namespace {

constexpr int kBins = 2048;

constexpr int kStage = 16384;                 // keys staged in LDS (64 KB)
constexpr int kStagePer = kStage / kSelThreads;
constexpr int kStageMaxHeads = 128;           // staging pays while the grid leaves CUs to spare

// One 1024-thread workgroup per kv head: counting passes over key digits
// [31:21], [20:10], [9:0] with 2048/2048/1024-bin LDS histograms.  STAGE:
// stage the first kStage candidates in LDS (calls of up to kStageMaxHeads
// heads: 64 heads x 16K 31.3 -> 23.9 us); grids of many heads read global
// memory per pass (every CU busy; 1024 heads x 32K: 188 us, 257 with staging).
template <bool STAGE>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sm_key[STAGE ? kStage : 1];
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
  const int64_t nst = !STAGE ? 0 : (ncand < kStage ? ncand : kStage);  // staged candidates
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

  // ---- stage: every load of the first kStage candidates in one round -------
  if constexpr (STAGE) {
    float v[kStagePer];
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      const int64_t i = tid + (int64_t)u * kSelThreads;
      v[u] = i < nst ? s[c_lo + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      const int64_t i = tid + (int64_t)u * kSelThreads;
      if (i < nst) sm_key[i] = score_key(v[u]);
    }
  }
  // candidate i (0-based from c_lo): LDS when staged, else global
  auto key_at = [&](int64_t i) -> uint32_t { return i < nst ? sm_key[i] : score_key(s[c_lo + i]); };

  // ---- radix passes: digits [31:21], [20:10], [9:0] of the key ----------
  uint32_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)K;  // how many of the remaining keys still to take
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int b = tid; b < kBins; b += kSelThreads) hist[b] = 0u;
    __syncthreads();  // also orders the staging stores before the first pass
    for (int64_t i0 = 0; i0 < ncand; i0 += kSelThreads) {  // wave-uniform trip count
      const int64_t i = i0 + tid;
      const bool valid = i < ncand;
      const uint32_t key = valid ? key_at(i) : 0u;
      if (valid && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
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
  const uint32_t limit = (uint32_t)(nsink + K);

  // ---- compaction in index order ------------------------------------------
  if (STAGE && nst == ncand) {
    // all staged: thread t owns the run [t P, t P + P) of candidates, so two
    // workgroup scans rank the equal keys and the kept keys
    const int64_t P = (ncand + kSelThreads - 1) / kSelThreads;
    const int64_t i0 = tid * P;
    const int64_t i1 = i0 + P < ncand ? i0 + P : ncand;
    uint32_t n_eq = 0, n_gt = 0;
    for (int64_t i = i0; i < i1; ++i) {
      const uint32_t key = sm_key[i];
      n_eq += key == T ? 1u : 0u;
      n_gt += key > T ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t eq_rank = block_excl_scan(n_eq, sm_w, &tot);
    const uint32_t gt_before = block_excl_scan(n_gt, sm_w, &tot);
    uint32_t pos = (uint32_t)nsink + gt_before + (eq_rank < take ? eq_rank : take);
    for (int64_t i = i0; i < i1; ++i) {
      const uint32_t key = sm_key[i];
      const bool eq = key == T;
      if (key > T || (eq && eq_rank < take)) {
        if (pos < limit) out[pos] = (int32_t)(c_lo + i);  // never past the row
        ++pos;
      }
      eq_rank += eq ? 1u : 0u;
    }
    return;
  }
  uint32_t base = (uint32_t)nsink, eq_seen = 0;
#pragma unroll 1
  for (int64_t t0 = 0; t0 < ncand; t0 += kSelThreads) {
    const int64_t i = t0 + tid;
    const bool valid = i < ncand;
    const uint32_t key = valid ? key_at(i) : 0u;
    const bool eq = valid && key == T;
    uint32_t n_eq;
    const uint32_t eq_rank = eq_seen + block_flag_rank(eq, sm_w, &n_eq);
    const bool keep = valid && (key > T || (eq && eq_rank < take));
    uint32_t n_keep;
    const uint32_t pos = base + block_flag_rank(keep, sm_w, &n_keep);
    if (keep && pos < limit) out[pos] = (int32_t)(c_lo + i);  // never past the row
    base += n_keep;
    eq_seen += n_eq;
  }
}


// ---------------------------------------------------------------------------
// Rows of at most kSmallMax candidates: one workgroup per kv head.  Thread t
// holds the run of candidates [t P, t P + P), P <= PER, as keys in registers,
// loaded once.  Each radix pass takes three barriers: histogram complete,
// scan totals, digit chosen (the other of two histogram buffers is cleared in
// the same step); the compaction is one scan of the (equal, above) counts of
// every run.  PER = 4 up to 4096 candidates, 16 beyond (a run of 16 slots
// costs more per pass than the barriers of 1024 threads: 2K candidates x 8
// heads 5.3 us with 4 per thread, 7.1 us with 256 threads x 16).
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallPerShort = 4;   // keys per thread up to 4096 candidates
constexpr int kSmallPer = 16;       // ... and up to kSmallMax
constexpr int kSmallMax = kSmallThreads * kSmallPer;

// Exclusive prefix sum of one value per thread over the workgroup; sm_w holds
// kSmallWaves words that no other call touches before the next barrier.
__device__ __forceinline__ uint32_t small_excl_scan(uint32_t v, uint32_t* sm_w, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sm_w[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSmallWaves; ++w) {
    const uint32_t c = sm_w[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  *total = all;
  return before + x - v;
}

template <int PER>
__global__ __launch_bounds__(kSmallThreads) void select_small_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[2][kBins];
  __shared__ uint32_t sm_w[4][kSmallWaves];
  __shared__ uint32_t sm_digit[3], sm_krem[3];

  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const float* s = a.score + (int64_t)h * a.score_stride;
  int32_t* out = a.idx + (int64_t)h * a.idx_stride;
  const int64_t n = a.n;
  const int64_t tail = n - a.n_recent > 0 ? n - a.n_recent : 0;
  const int64_t nsink = a.n_sink < tail ? a.n_sink : tail;
  const int64_t c_lo = a.n_sink, c_hi = n - a.n_recent;
  const int ncand = c_lo < c_hi ? (int)(c_hi - c_lo) : 0;  // <= kSmallMax
  int64_t K = a.k_per_head ? a.k_per_head[h] : a.k_uniform;
  K = K < 0 ? 0 : K;
  K = K > ncand ? ncand : K;
  K = K > a.k_max ? a.k_max : K;  // never write past the index row

  for (int64_t i = tid; i < nsink; i += kSmallThreads) out[i] = (int32_t)i;
  if (tid == 0) a.count[h] = (int32_t)(nsink + K);
  if (K == 0) return;
  if (K == ncand) {
    for (int64_t i = tid; i < K; i += kSmallThreads) out[nsink + i] = (int32_t)(c_lo + i);
    return;
  }

  const int P = (ncand + kSmallThreads - 1) / kSmallThreads;
  const int i0 = tid * P;
  const int nv = ncand - i0 < 0 ? 0 : (ncand - i0 > P ? P : ncand - i0);  // keys of this run
  uint32_t key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) key[u] = u < nv ? score_key(s[c_lo + i0 + u]) : 0u;
  for (int b = tid; b < kBins; b += kSmallThreads) hist[0][b] = 0u;
  __syncthreads();

  // ---- radix passes: digits [31:21], [20:10], [9:0] ----------------------
  uint32_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)K;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    uint32_t* H = hist[pass & 1];
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (u < nv && (key[u] & mask) == prefix) atomicAdd(&H[(key[u] >> shift) & (uint32_t)(nb - 1)], 1u);
    __syncthreads();
    // thread t owns nb / 256 consecutive bins, visited from the top
    const int per = nb / kSmallThreads;
    const int top = nb - 1 - tid * per;
    uint32_t mine = 0;
    for (int i = 0; i < per; ++i) mine += H[top - i];
    uint32_t total;
    uint32_t above = small_excl_scan(mine, sm_w[pass], &total);
    if (above < krem && krem <= above + mine) {
      for (int i = 0; i < per; ++i) {
        const uint32_t cb = H[top - i];
        if (krem <= above + cb) {
          sm_digit[pass] = (uint32_t)(top - i);
          sm_krem[pass] = krem - above;
          break;
        }
        above += cb;
      }
    }
    if (pass < 2)  // the other buffer was last read before the previous pass's last barrier
      for (int b = tid; b < kBins; b += kSmallThreads) hist[(pass + 1) & 1][b] = 0u;
    __syncthreads();
    prefix |= sm_digit[pass] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    krem = sm_krem[pass];
  }
  const uint32_t T = prefix;
  const uint32_t take = krem;  // keys equal to T to keep, lowest index first
  const uint32_t limit = (uint32_t)(nsink + K);

  // ---- compaction in index order: one scan of (equal, above) per run ------
  uint32_t n_eq = 0, n_gt = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    n_eq += (u < nv && key[u] == T) ? 1u : 0u;
    n_gt += (u < nv && key[u] > T) ? 1u : 0u;
  }
  uint32_t tot;  // counts <= kSmallMax < 2^16: both in one scan
  const uint32_t ex = small_excl_scan((n_eq << 16) | n_gt, sm_w[3], &tot);
  uint32_t eq_rank = ex >> 16;
  uint32_t pos = (uint32_t)nsink + (ex & 0xFFFFu) + (eq_rank < take ? eq_rank : take);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (u < nv) {
      const bool eq = key[u] == T;
      if (key[u] > T || (eq && eq_rank < take)) {
        if (pos < limit) out[pos] = (int32_t)(c_lo + i0 + u);  // never past the row
        ++pos;
      }
      eq_rank += eq ? 1u : 0u;
    }
  }
}


// ---------------------------------------------------------------------------
// Block-parallel path for long caches with few kv heads (a one-workgroup-per-
// head select would leave most CUs idle).  Candidates are cut into blocks of
// kBlk.  Radix digits: key bits [31:20] (4096 bins), [19:9] (2048), [8:0]
// (512).  Integer histogram totals are the only global atomics, so the result
// is identical run to run.  The first-level totals live in memory that is
// zero on entry and is left zero (kernel 3 clears them after their last
// reader); kernel 1 clears the second-level totals:
//   1 per block: histogram of the first digit, kept per block and added into
//                the head's first-level totals; block 0 clears the head's
//                second-level totals
//   2 per block: from the head totals, the bin d1 holding the K-th key and the
//                rank left inside it; copy this block's bin-d1 keys (key,
//                index) in index order (offset from the other blocks' bin-d1
//                counts), count its keys above the bin, and add the histogram
//                of the second digit of its bin-d1 keys into the head's
//                second-level totals
//   3 per block: from the second-level totals, the bin d2 of the K-th key;
//                last radix pass over the bin-d1 keys with the prefix (d1, d2)
//                -> threshold key T and how many keys equal to T are kept,
//                lowest index first; the kept bin-d1 keys of every block ->
//                this block's output offset; write its kept indices.  Block 0
//                writes the sinks and the count and clears the first-level
//                totals.
// The per-head steps inside kernels 2 and 3 are recomputed by every block of
// the head from the same totals (cheaper than a one-workgroup-per-head launch).
// ---------------------------------------------------------------------------
constexpr int kBlk = 4096;                 // candidates per block
constexpr int kBlkPer = kBlk / kSelThreads;
constexpr int kBins1 = 4096;               // first digit: key >> 20
constexpr int kBins2 = 2048;               // second digit: (key >> 9) & 2047
constexpr int kStageMem = 16384;           // bin-d1 keys staged in LDS
constexpr int kPreMem = 4;                 // ... of which kPreMem per thread loaded up front
constexpr int kBatch = 8;                  // loads in flight per thread when reading global keys

struct SelGeom {  // per-head geometry shared by the kernels
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
  uint32_t* tot1;    // [Hkv][4096] head histogram of the first digit (SelectArgs::totals, zero on entry)
  uint32_t* tot2;    // [Hkv][2048] head histogram of the second digit of the bin-d1 keys
  uint32_t* hist1;   // [Hkv][nbm][4096] block histograms of the first digit
  uint32_t* above;   // [Hkv][nbm] keys above bin d1 per block
  uint32_t* moff;    // [Hkv][nbm + 1] first bin-d1 key of each block in ckey; [nb] = all
  uint32_t* head;    // [Hkv][8]: d1, rank left inside d1
  uint32_t* ckey;    // [Hkv][n] bin-d1 keys, index order
  int32_t* cidx;     // [Hkv][n]
  int nbm;
};

__host__ __device__ inline int sel_blocks_max(int64_t n) { return (int)((n + kBlk - 1) / kBlk); }

// Byte offsets of the scratch arrays (each 256-byte aligned); [7] = total.
__host__ __device__ inline void sel_offsets(int hkv, int64_t n, size_t (&off)[8]) {
  const size_t nbm = (size_t)sel_blocks_max(n);
  const size_t bytes[7] = {(size_t)hkv * kBins2 * 4, (size_t)hkv * nbm * kBins1 * 4, (size_t)hkv * nbm * 4,
                           (size_t)hkv * (nbm + 1) * 4, (size_t)hkv * 8 * 4, (size_t)hkv * n * 4,
                           (size_t)hkv * n * 4};
  size_t at = 0;
  for (int i = 0; i < 7; ++i) {
    off[i] = at;
    at += (bytes[i] + 255) / 256 * 256;
  }
  off[7] = at;
}

__host__ __device__ inline SelWs sel_ws(void* ws, uint32_t* totals, int hkv, int64_t n) {
  SelWs w;
  w.nbm = sel_blocks_max(n);
  size_t off[8];
  sel_offsets(hkv, n, off);
  char* p = (char*)ws;
  w.tot1 = totals;
  w.tot2 = (uint32_t*)(p + off[0]);
  w.hist1 = (uint32_t*)(p + off[1]);
  w.above = (uint32_t*)(p + off[2]);
  w.moff = (uint32_t*)(p + off[3]);
  w.head = (uint32_t*)(p + off[4]);
  w.ckey = (uint32_t*)(p + off[5]);
  w.cidx = (int32_t*)(p + off[6]);
  return w;
}

__device__ __forceinline__ bool sel_radix(const SelGeom& g) { return g.K > 0 && g.K < g.ncand; }

// This block's candidates: thread t holds kBlkPer consecutive ones.
__device__ __forceinline__ void load_block_scores(const SelectArgs& a, const SelGeom& g, int h, int b,
                                                  float (&sv)[kBlkPer], int64_t& j0) {
  const float* s = a.score + (int64_t)h * a.score_stride;
  j0 = g.c_lo + (int64_t)b * kBlk + kBlkPer * threadIdx.x;
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) sv[u] = j0 + u < g.c_hi ? s[j0 + u] : 0.0f;
}

// Bin of the krem-th largest key of a histogram whose NB = PER * kSelThreads
// bins are held PER per thread, thread t holding bins NB-1-PER t downwards
// (c[0] the highest); -> sm_digit, sm_krem (the rank left inside that bin).
template <int PER>
__device__ __forceinline__ void pick_bin(const uint32_t (&c)[PER], uint32_t krem, uint32_t* sm_w,
                                         uint32_t* sm_digit, uint32_t* sm_krem) {
  const int top = PER * kSelThreads - 1 - PER * (int)threadIdx.x;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += c[i];
  if (threadIdx.x == 0) {  // in range whatever the counts hold
    *sm_digit = 0u;
    *sm_krem = 1u;
  }
  uint32_t total;
  uint32_t above = block_excl_scan(mine, sm_w, &total);
  if (above < krem && krem <= above + mine) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (above < krem && krem <= above + c[i]) {
        *sm_digit = (uint32_t)(top - i);
        *sm_krem = krem - above;
      }
      above += c[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void sel_hist1_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[kBins1];
  const SelWs w = sel_ws(a.ws, a.totals, a.n_kv_heads, a.n);
  const int h = blockIdx.x % a.n_kv_heads, b = blockIdx.x / a.n_kv_heads;  // a head's blocks on one XCD
  const SelGeom g = sel_geom(a, h);
  if (b >= g.nb || !sel_radix(g)) return;
  const int tid = threadIdx.x;
  float sv[kBlkPer];
  int64_t j0;
  load_block_scores(a, g, h, b, sv, j0);
  for (int i = tid; i < kBins1; i += kSelThreads) hist[i] = 0u;
  if (b == 0)
    for (int i = tid; i < kBins2; i += kSelThreads) w.tot2[(int64_t)h * kBins2 + i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u)
    if (j0 + u < g.c_hi) atomicAdd(&hist[score_key(sv[u]) >> 20], 1u);
  __syncthreads();
  uint32_t* out = w.hist1 + ((int64_t)h * w.nbm + b) * kBins1;
  uint32_t* t1 = w.tot1 + (int64_t)h * kBins1;
  for (int i = tid; i < kBins1; i += kSelThreads) {
    const uint32_t c = hist[i];
    out[i] = c;
    if (c) atomicAdd(&t1[i], c);
  }
}

__global__ __launch_bounds__(kSelThreads) void sel_collect_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[kBins2];
  __shared__ uint32_t sm_w[kSelWaves + 1];
  __shared__ uint32_t sm_digit, sm_krem, sm_base;
  const SelWs w = sel_ws(a.ws, a.totals, a.n_kv_heads, a.n);
  const int h = blockIdx.x % a.n_kv_heads, b = blockIdx.x / a.n_kv_heads;  // a head's blocks on one XCD
  const SelGeom g = sel_geom(a, h);
  if (b >= g.nb || !sel_radix(g)) return;
  const int tid = threadIdx.x;
  float sv[kBlkPer];
  int64_t j0;
  load_block_scores(a, g, h, b, sv, j0);
  for (int i = tid; i < kBins2; i += kSelThreads) hist[i] = 0u;
  // thread t holds first-level bins 4095 - 4t .. 4092 - 4t
  const uint4 t1 = *reinterpret_cast<const uint4*>(w.tot1 + (int64_t)h * kBins1 + kBins1 - 4 - 4 * tid);
  const uint32_t c1[4] = {t1.w, t1.z, t1.y, t1.x};
  pick_bin<4>(c1, (uint32_t)g.K, sm_w, &sm_digit, &sm_krem);
  const uint32_t d1 = sm_digit;
  // bin-d1 keys in the blocks before this one
  const uint32_t* h1 = w.hist1 + (int64_t)h * w.nbm * kBins1;
  const uint32_t mine = tid < g.nb ? h1[(int64_t)tid * kBins1 + d1] : 0u;
  uint32_t cmem;
  const uint32_t off = block_excl_scan(mine, sm_w, &cmem);
  if (tid == b) sm_base = off;
  uint32_t* hd = w.head + (int64_t)h * 8;
  uint32_t* mo = w.moff + (int64_t)h * (w.nbm + 1);
  if (b == 0 && tid == 0) {
    hd[0] = d1;
    hd[1] = sm_krem;
    mo[g.nb] = cmem;
  }
  __syncthreads();
  uint32_t key[kBlkPer], n_in = 0, n_ab = 0;
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) {
    const bool valid = j0 + u < g.c_hi;
    key[u] = score_key(sv[u]);
    const bool in = valid && (key[u] >> 20) == d1;
    n_in += in ? 1u : 0u;
    n_ab += (valid && (key[u] >> 20) > d1) ? 1u : 0u;
    if (in) atomicAdd(&hist[(key[u] >> 9) & (uint32_t)(kBins2 - 1)], 1u);
  }
  uint32_t tot;  // counts <= kBlk < 2^16: both in one scan
  const uint32_t ex = block_excl_scan((n_in << 16) | n_ab, sm_w, &tot);
  uint32_t r = sm_base + (ex >> 16);
  uint32_t* ck = w.ckey + (int64_t)h * a.n;
  int32_t* ci = w.cidx + (int64_t)h * a.n;
#pragma unroll
  for (int u = 0; u < kBlkPer; ++u) {
    if (j0 + u < g.c_hi && (key[u] >> 20) == d1) {
      ck[r] = key[u];
      ci[r] = (int32_t)(j0 + u);
      ++r;
    }
  }
  if (tid == 0) {
    w.above[(int64_t)h * w.nbm + b] = tot & 0xFFFFu;
    mo[b] = sm_base;
  }
  // the block_excl_scan barriers ordered every histogram add before this
  uint32_t* t2 = w.tot2 + (int64_t)h * kBins2;
  for (int i = tid; i < kBins2; i += kSelThreads) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&t2[i], c);
  }
}

__global__ __launch_bounds__(kSelThreads) void sel_write_kernel(const SelectArgs a) {
  __shared__ uint32_t hist[kSelThreads];
  __shared__ uint32_t sm_w[kSelWaves + 1];
  __shared__ uint32_t sm_digit, sm_krem, sm_jt, sm_base;
  __shared__ uint32_t sm_kept[kSelThreads];
  __shared__ uint32_t sm_off[kSelThreads + 1];
  __shared__ uint32_t sm_ck[kStageMem];  // bin-d1 keys when they fit (the usual case)
  const SelWs w = sel_ws(a.ws, a.totals, a.n_kv_heads, a.n);
  const int h = blockIdx.x % a.n_kv_heads, b = blockIdx.x / a.n_kv_heads;  // a head's blocks on one XCD
  const SelGeom g = sel_geom(a, h);
  if (b > 0 && b >= g.nb) return;
  const int tid = threadIdx.x;
  if (b == 0) {
    int32_t* out = a.idx + (int64_t)h * a.idx_stride;
    for (int64_t i = tid; i < g.nsink; i += kSelThreads) out[i] = (int32_t)i;
    if (tid == 0) a.count[h] = (int32_t)(g.nsink + g.K);
    if (sel_radix(g))  // the previous kernel was the last reader of the first-level totals
      for (int i = tid; i < kBins1; i += kSelThreads) w.tot1[(int64_t)h * kBins1 + i] = 0u;
  }
  if (b >= g.nb || g.K == 0) return;
  const bool radix = g.K < g.ncand;
  // every independent load in one round: this block's scores, head state, the
  // blocks' counts and offsets, the second-level totals and (speculatively)
  // the first kPreMem * kSelThreads bin-d1 keys
  float sv[kBlkPer];
  int64_t j0;
  load_block_scores(a, g, h, b, sv, j0);
  uint32_t T = 0;
  int64_t jt = INT64_MAX;  // every key >= T kept (all candidates)
  uint32_t base = (uint32_t)(g.nsink + (int64_t)b * kBlk);
  if (radix) {
    const uint32_t* hd = w.head + (int64_t)h * 8;
    const uint32_t* mo = w.moff + (int64_t)h * (w.nbm + 1);
    const uint32_t* ck = w.ckey + (int64_t)h * a.n;
    const int32_t* ci = w.cidx + (int64_t)h * a.n;
    uint32_t pk[kPreMem];
#pragma unroll
    for (int u = 0; u < kPreMem; ++u) pk[u] = ck[u * kSelThreads + tid];  // rows hold n > 4096 entries
    const uint32_t abv = tid < g.nb ? w.above[(int64_t)h * w.nbm + tid] : 0u;
    const uint32_t moff = tid < g.nb ? mo[tid] : 0u;
    const uint32_t C = mo[g.nb];  // bin-d1 keys of the head
    const uint2 t2 = *reinterpret_cast<const uint2*>(w.tot2 + (int64_t)h * kBins2 + kBins2 - 2 - 2 * tid);
    const uint32_t d1 = hd[0], krem1 = hd[1];
    if (tid < g.nb) sm_off[tid] = moff;
    if (tid == 0) sm_off[g.nb] = C;
    hist[tid] = 0u;
    sm_kept[tid] = 0u;
    if (tid == 0) sm_jt = 0xFFFFFFFFu;
    const uint32_t c2[2] = {t2.y, t2.x};
    pick_bin<2>(c2, krem1, sm_w, &sm_digit, &sm_krem);  // (its barriers publish the above)
    const uint32_t P2 = (d1 << 11) | sm_digit;  // key >> 9 of the threshold
    const uint32_t krem = sm_krem;
    const bool staged = C <= (uint32_t)kStageMem;
    if (staged) {
#pragma unroll
      for (int u = 0; u < kPreMem; ++u) sm_ck[u * kSelThreads + tid] = pk[u];
      for (uint32_t i0 = kPreMem * kSelThreads; i0 < C; i0 += kBatch * kSelThreads) {
        uint32_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = i0 + u * kSelThreads + tid;
          v[u] = i < C ? ck[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = i0 + u * kSelThreads + tid;
          if (i < C) sm_ck[i] = v[u];
        }
      }
      __syncthreads();
      ck = sm_ck;
    }
    // last radix pass: bits [8:0] of the bin-d1 keys with prefix P2
    for (uint32_t i0 = 0; i0 < C; i0 += kBatch * kSelThreads) {
      uint32_t v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = i0 + u * kSelThreads + tid;
        v[u] = i < C ? ck[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = i0 + u * kSelThreads + tid;
        if (i < C && (v[u] >> 9) == P2) atomicAdd(&hist[v[u] & 511u], 1u);
      }
    }
    __syncthreads();
    {
      const uint32_t c3[1] = {hist[kSelThreads - 1 - tid]};  // bins >= 512 stay empty
      pick_bin<1>(c3, krem, sm_w, &sm_digit, &sm_krem);
    }
    T = (P2 << 9) | sm_digit;
    const uint32_t take = sm_krem;
    // bin-d1 keys in index order: every key > T and the first `take` equal to
    // T are kept.  Thread t walks the run [t R, t R + R); the kept count of the
    // block holding the run's keys is flushed whenever the run crosses into
    // the next block.
    const uint32_t R = (C + kSelThreads - 1) / kSelThreads;
    const uint32_t i0 = (uint32_t)tid * R;
    const uint32_t i1 = i0 + R < C ? i0 + R : C;
    uint32_t n_eq = 0;
    for (uint32_t i = i0; i < i1; ++i) n_eq += ck[i] == T ? 1u : 0u;
    uint32_t tot_eq;
    uint32_t eq_rank = block_excl_scan(n_eq, sm_w, &tot_eq);
    if (i0 < i1) {
      int lo = 0, hi = g.nb - 1;  // block of key i0: the last with sm_off[blk] <= i0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sm_off[mid] <= i0) lo = mid; else hi = mid - 1;
      }
      int blk = lo;
      uint32_t kept = 0;
      for (uint32_t i = i0; i < i1; ++i) {
        while (i >= sm_off[blk + 1]) {  // the run crosses a block border
          if (kept) atomicAdd(&sm_kept[blk], kept);
          kept = 0;
          ++blk;
        }
        const uint32_t key = ck[i];
        const bool eq = key == T;
        if (key > T || (eq && eq_rank < take)) {
          ++kept;
          if (eq && eq_rank == take - 1) sm_jt = (uint32_t)ci[i];
        }
        eq_rank += eq ? 1u : 0u;
      }
      if (kept) atomicAdd(&sm_kept[blk], kept);
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

static_assert((size_t)63 * kBins1 * 4 <= SKV_WS_HEADER_BYTES,
              "the block path's head totals fit the reserved workspace header");

size_t select_ws_bytes(int32_t n_kv_heads, int64_t n) {
  if (!use_block_path(n_kv_heads, n)) return 0;
  size_t off[8];
  sel_offsets(n_kv_heads, n, off);
  return off[7];
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (!use_block_path(a.n_kv_heads, a.n)) {
    const int64_t ncand = a.n - a.n_sink - a.n_recent;
    if (ncand <= kSmallThreads * kSmallPerShort) {
      hipLaunchKernelGGL(select_small_kernel<kSmallPerShort>, dim3((unsigned)a.n_kv_heads), dim3(kSmallThreads),
                         0, stream, a);
      return hipGetLastError();
    }
    if (ncand <= kSmallMax) {
      hipLaunchKernelGGL(select_small_kernel<kSmallPer>, dim3((unsigned)a.n_kv_heads), dim3(kSmallThreads), 0,
                         stream, a);
      return hipGetLastError();
    }
    if (a.n_kv_heads <= kStageMaxHeads)
      hipLaunchKernelGGL(select_kernel<true>, dim3((unsigned)a.n_kv_heads), dim3(kSelThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(select_kernel<false>, dim3((unsigned)a.n_kv_heads), dim3(kSelThreads), 0, stream, a);
    return hipGetLastError();
  }
  const unsigned grid_b = (unsigned)(a.n_kv_heads * sel_blocks_max(a.n));
  hipLaunchKernelGGL(sel_hist1_kernel, dim3(grid_b), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_collect_kernel, dim3(grid_b), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_write_kernel, dim3(grid_b), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace skv
