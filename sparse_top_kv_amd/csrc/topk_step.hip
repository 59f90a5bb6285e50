// topk_step.hip -- the per-step top-K decode step in one launch (bf16
// caches): the group-summed softmax score of one decode query
// ("Sparse-to-Dense ..." Sec. 3.2: top-K attention keeps the keys with the
// largest attention score, the scores of a GQA group summed), the selection
// of the sinks, the top-K candidates (score descending, index ascending) and
// the recent run ("Where Activation Sparsity and KV-Cache Sparsity Cross
// ...", "Speedup Across Context"), and exact attention over that kept set.
//
// Why one launch.  Done as three calls the step writes the fp32 logits of
// every query head (16.8 MB at 128K context), reads them back, and spends six
// more launches normalising, selecting, attending and merging, each launch
// boundary worth ~2 us.  Here a kv head's keys are cut into P chunks, one
// workgroup each (one per CU), and each keeps its chunk's logits in LDS:
//   A  stream K once (direct-to-LDS tiles, q.K^T on MFMA, the tile order and
//      reductions of the per-step score kernel, so the scores match it bit
//      for bit); logits -> LDS; per query head the chunk's (max, sum)   | sync
//   B  lse of every query head from the P chunks; s(j) = sum_g 2^(l - lse)
//      (stored to `score` when given); the candidates' keys (order-keeping
//      integer images of the scores); this chunk's published keys     | sync
//   C  the threshold key T (the K-th largest candidate key) and how many
//      keys equal to T are kept.  Each chunk publishes its candidate keys
//      from the 12-bit bin of local rank ~2K/P upwards and that bin's lower
//      edge (in B, before the barrier); each workgroup then finds the K-th
//      largest published key with LDS histograms.  It is T when no chunk's
//      edge lies above it (every key at or above it was published); else
//      the head's global radix levels decide: histograms of key bits
//      31..20, 19..9 and 8..0 added into device totals, then each chunk's
//      counts above and equal to T (one barrier each)
//   E  this chunk's kept indices into idx (ascending); the attention
//      partial (max, sum, acc) over the chunk's kept rows -- sinks, the
//      selected candidates, the recent run -- from the logits in LDS and
//      V rows gathered by index, written in the split-K merge kernel's
//      format; that kernel (a second launch) merges the P partials into out
//      and lse and clears the step's counters.
// "sync" is a barrier of the P workgroups of one kv head: a device-scope
// arrival counter (its own 128-byte line in the workspace header, zero on
// entry) that only counts up during the step (barrier k waits for k P
// arrivals); the merge launch resets it.  Everything one workgroup hands to
// another is written with device-scope stores, completed (s_waitcnt) before
// the arrival, and read with device-scope loads after it.
//
// Progress.  Kv head h takes the workgroups with block index = h mod Hkv,
// which draw their chunk numbers from the head's ticket when they start: a
// head's barrier only ever waits for workgroups that are running.  Waiting
// workgroups of a head number at most P - 1 while its chunks are not all
// drawn, so a device that holds (P - 1) Hkv + 1 workgroups at once (P <=
// CUs / Hkv, one workgroup per CU) never stalls, with no cooperative launch.
// The merge launch that follows resets the counters.  Spins are still
// bounded: one that runs out (other work holding the CUs far longer than a
// step) sets the header's error word, and that step's results are
// unspecified.
#include "skv_block.h"
#include "skv_common.h"
#include "skv_kernels.h"
#include "skv_mfma.h"
#include "skv_tile.h"

namespace skv {
namespace {

constexpr int kW = 8;                 // waves per workgroup
constexpr int kT = 64 * kW;
constexpr int kLgFloats = 16384;      // logits of one chunk, all query heads of the group
constexpr int kGranule = kW * kStep;  // chunk granule (one tile per wave)
constexpr uint32_t kSpinMax = 1u << 20;
constexpr int kBins1 = 4096, kBins2 = 2048, kBins3 = 512;
constexpr int kSelKpt = 8;            // keys per thread of the selection alone (chunks of 4096)
constexpr int kPubKeys = 16384;       // keys a kv head's chunks publish, at most
constexpr int kPubW = kPubKeys / kT / 4;  // 16-byte words of them per thread
constexpr int kRankMax = 512;         // keys of the threshold's bin ranked directly
constexpr int kMaxP = 1024;           // chunks per kv head

// keys per chunk and per thread for a group of G query heads: the chunk's
// logits fit kLgFloats, and its kept-row list (one word a row) the K ring
template <int D, int G>
struct Chunk {
  static constexpr int kRingWords = 2 * kW * TileGeom<D>::kTB / 4;
  static constexpr int kLim = kLgFloats / G < kRingWords ? kLgFloats / G : kRingWords;
  static constexpr int kMax = kLim / kGranule * kGranule;
  static constexpr int kPer = (kMax + kT - 1) / kT;
};

__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier of the workgroups of one kv head: wait until `target` arrivals.
__device__ __forceinline__ void head_sync(uint32_t* ctr, uint32_t target, uint32_t* err) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (ld_dev(ctr) < target) {
      if (++spins > kSpinMax) {
        st_dev(err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Exclusive prefix sum over the workgroup (kW waves); *total = the sum.
__device__ __forceinline__ uint32_t wg_excl_scan(uint32_t v, uint32_t* sm_w, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sm_w[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const uint32_t c = sm_w[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  *total = all;
  __syncthreads();
  return before + x - v;
}

// The bin of rank krem (1 = the largest key) in a head's histogram of NB
// bins (device memory, read at device scope); thread t holds bins
// NB - 1 - PER t downwards.  -> sm_digit, sm_krem (the rank left in the bin).
template <int NB>
__device__ __forceinline__ void pick_bin(const uint32_t* tot, uint32_t krem, uint32_t* sm_w,
                                         uint32_t* sm_digit, uint32_t* sm_krem) {
  constexpr int PER = NB / kT;
  static_assert(PER * kT == NB, "bins per thread");
  const int top = NB - 1 - PER * (int)threadIdx.x;
  uint32_t c[PER], mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = ld_dev(tot + top - i);
    mine += c[i];
  }
  if (threadIdx.x == 0) {  // in range whatever the counts hold
    *sm_digit = 0u;
    *sm_krem = 1u;
  }
  uint32_t total;
  uint32_t above = wg_excl_scan(mine, sm_w, &total);
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

// Scratch of one call (device memory, the caller's workspace after its header).
struct TopkWs {
  float* stats;     // [Hkv][P][G][2] chunk (max, sum) per query head
  uint32_t* tot1;   // [Hkv][4096]
  uint32_t* tot2;   // [Hkv][2048]
  uint32_t* tot3;   // [Hkv][512]
  uint32_t* cnts;   // [Hkv][P][2] keys above T and equal to T
  float* part_ml;   // [Hkv][P][G][2] attention partial (max, sum), the merge kernel's format
  float* part_acc;  // [Hkv][P][G][D] attention partial (acc)
  uint32_t* pub;    // [Hkv][P][pub_cap] each chunk's published keys
  uint32_t* edge;   // [Hkv][P][2] lower edge of the keys a chunk published; an upper bound of T
};

// Byte offsets of the scratch arrays (each 256-byte aligned); [9] = total.
inline void topk_offsets(int hkv, int p, int g, int d, size_t (&off)[10]) {
  const size_t bytes[9] = {(size_t)hkv * p * g * 2 * 4, (size_t)hkv * kBins1 * 4, (size_t)hkv * kBins2 * 4,
                           (size_t)hkv * kBins3 * 4, (size_t)hkv * p * 2 * 4, (size_t)hkv * p * g * 2 * 4,
                           (size_t)hkv * kPubKeys * 4, (size_t)hkv * p * 2 * 4, (size_t)hkv * p * g * d * 4};
  size_t at = 0;
  for (int i = 0; i < 9; ++i) {
    off[i] = at;
    at += (bytes[i] + 255) / 256 * 256;
  }
  off[9] = at;
}

inline TopkWs topk_ws_layout(const TopkArgs& a, void* scratch, int g, int d) {
  size_t off[10];
  topk_offsets(a.n_kv_heads, a.chunks_per_head, g, d, off);
  char* b = (char*)scratch;
  TopkWs w;
  w.stats = (float*)(b + off[0]);
  w.tot1 = (uint32_t*)(b + off[1]);
  w.tot2 = (uint32_t*)(b + off[2]);
  w.tot3 = (uint32_t*)(b + off[3]);
  w.cnts = (uint32_t*)(b + off[4]);
  w.part_ml = (float*)(b + off[5]);
  w.pub = (uint32_t*)(b + off[6]);
  w.edge = (uint32_t*)(b + off[7]);
  w.part_acc = (float*)(b + off[8]);
  return w;
}


// The bin of rank krem (1 = the largest key) in an LDS histogram of NB bins
// held as NC copies [NC][NB] to be summed (thread t holds bins NB - 1 - PER t
// downwards) -> sm_digit, sm_krem (the rank left in the bin); bin 0 and rank
// krem_none when the histogram holds fewer than krem keys.
template <int NB, int NC = 1>
__device__ __forceinline__ void pick_lds(const uint32_t* hist, uint32_t krem, uint32_t* sm_w,
                                         uint32_t* sm_digit, uint32_t* sm_krem, uint32_t krem_none) {
  constexpr int PER = NB / kT;
  static_assert(PER * kT == NB, "bins per thread");
  const int top = NB - 1 - PER * (int)threadIdx.x;
  uint32_t c[PER], mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = 0u;
#pragma unroll
    for (int k = 0; k < NC; ++k) c[i] += hist[k * NB + top - i];
    mine += c[i];
  }
  if (threadIdx.x == 0) {
    *sm_digit = 0u;
    *sm_krem = krem_none;
  }
  uint32_t total;
  uint32_t above = wg_excl_scan(mine, sm_w, &total);
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

// The bins of ranks ka and kb (1 = the largest key) in an LDS histogram of NB
// bins held as NC copies -> *da, *db (bin + 1; 0 when the histogram holds
// fewer keys than the rank).
template <int NB, int NC>
__device__ __forceinline__ void pick2_lds(const uint32_t* hist, uint32_t ka, uint32_t kb, uint32_t* sm_w,
                                          uint32_t* da, uint32_t* db) {
  constexpr int PER = NB / kT;
  static_assert(PER * kT == NB, "bins per thread");
  const int top = NB - 1 - PER * (int)threadIdx.x;
  uint32_t c[PER], mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = 0u;
#pragma unroll
    for (int k = 0; k < NC; ++k) c[i] += hist[k * NB + top - i];
    mine += c[i];
  }
  if (threadIdx.x == 0) {
    *da = 0u;
    *db = 0u;
  }
  uint32_t total;
  uint32_t above = wg_excl_scan(mine, sm_w, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (above < ka && ka <= above + c[i]) *da = (uint32_t)(top - i) + 1u;
    if (above < kb && kb <= above + c[i]) *db = (uint32_t)(top - i) + 1u;
    above += c[i];
  }
  __syncthreads();
}

// Sum over the lanes l, l + N, l + 2N, ... of a wave (N = 8, 16 or 32).
template <int N>
__device__ __forceinline__ float slot_sum(float y) {
  static_assert(N == 8 || N == 16 || N == 32, "lanes per row");
  if constexpr (N == 8) y += dpp<0x128>(y);  // row_ror:8 pairs lanes l and l ^ 8
  if constexpr (N <= 16) y = xor16_sum(y);
  return xor32_sum(y);
}

// Two maxima over the workgroup with one barrier pair.
__device__ __forceinline__ void wg_max2_u32(uint32_t a, uint32_t b, uint32_t* sm, uint32_t* ma, uint32_t* mb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a = max(a, (uint32_t)__shfl_xor((int)a, off, 64));
    b = max(b, (uint32_t)__shfl_xor((int)b, off, 64));
  }
  if (lane == 0) {
    sm[wave] = a;
    sm[kW + wave] = b;
  }
  __syncthreads();
  uint32_t x = 0, y = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    x = max(x, sm[w]);
    y = max(y, sm[kW + w]);
  }
  *ma = x;
  *mb = y;
  __syncthreads();
}


__device__ __forceinline__ uint4 buf_load16_dev(BufRsrc r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 16));  // sc1
}

// SEL: the selection alone over a given score row (skv_select on long rows
// with few kv heads): no K stream, no attention; the same exchange and
// threshold search, with keys of any sign.  With no merge launch after it,
// the head's last workgroup to arrive clears the head's counters.
template <int D, int G, bool SEL>
__global__ __launch_bounds__(kT) void topk_step_kernel(const TopkArgs a, const TopkWs w) {
  using TG = TileGeom<D>;
  using CK = Chunk<D, G>;
  constexpr int NI = TG::kNI, TB = TG::kTB, PPR = TG::kPPR, KS = TG::kKS;
  constexpr int KPT = SEL ? kSelKpt : CK::kPer;
  constexpr int LPR = D / 8;  // lanes per V row (16 bytes each)
  constexpr int RSL = kT / LPR;  // V rows in flight per workgroup step
  static_assert(KPT <= 32, "candidate flags fit one word per thread");

  // K ring (two stages per wave), later the histograms and the kept list
  __shared__ __attribute__((aligned(1024))) char ring[2][kW][TB];
  __shared__ __attribute__((aligned(16))) float sm_lg[SEL ? 4 : kLgFloats + 4 * 16];
  __shared__ float sm_m[kW][16], sm_l[kW][16];
  __shared__ float sm_lse2[G];
  __shared__ uint32_t sm_w[kW + 1], sm_w2[2 * kW];
  __shared__ uint32_t sm_digit, sm_krem, sm_base, sm_item;
  static_assert(2 * kW * TB >= kBins1 * 4, "the histograms fit the ring");
  // privatised copies (lane % kCopies) of the 2048-bin LDS histograms: as many
  // (a power of two, at most 8) as leave room in the ring for kRankMax keys
  constexpr int kFit = (2 * kW * TB / 4 - kRankMax - 64) / 2048;
  constexpr int kCopies = kFit >= 8 ? 8 : (kFit >= 4 ? 4 : (kFit >= 2 ? 2 : 1));
  static_assert(kFit >= 1, "a histogram and the ranked keys fit the ring");
  // the chunk's local histogram of key bits 31..20: scores are probabilities
  // in the step (keys >= 2^31: bins 2048..4095), of either sign in SEL; two
  // copies (a chunk's 4096 or fewer keys spread over its bins: four copies
  // measured 0.2 us slower in the 128K step and 0.3 us in SEL, from their
  // clearing and summing)
  constexpr int kHB = SEL ? 4096 : 2048;
  constexpr int kCopiesB = 2;
  static_assert(kCopiesB * kHB <= 2 * kW * TB / 4, "the local histograms fit the ring");
  auto hbin = [](uint32_t k) -> uint32_t { return SEL ? k >> 20 : (k >> 20) & 2047u; };
  // barriers of the head so far when C starts: one (the logits' statistics)
  // in the step, none in SEL
  constexpr uint32_t kSb = SEL ? 0u : 1u;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, li = lane & 15;
  const int P = a.chunks_per_head;
  // kv head h = block % Hkv; its chunks go out in start order from the
  // head's ticket, so a head's barriers wait only for running workgroups.
  const int h = (int)(blockIdx.x % (uint32_t)a.n_kv_heads);
  uint32_t* ctr = a.ctr + (int64_t)h * 32;  // word 0 arrivals, word 16 the ticket
  if (tid == 0) sm_item = __hip_atomic_fetch_add(ctr + 16, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int c = (int)sm_item;
  const int64_t n = a.n;
  const int64_t r0 = (int64_t)c * a.chunk;
  const int64_t rem = n - r0;
  const int rows = (int)(rem < 0 ? 0 : (rem > a.chunk ? a.chunk : rem));
  const uint32_t stride = (uint32_t)a.pos_stride_b;
  const int lg_stride = a.chunk + 4;  // floats per head row in sm_lg

  // ---- A: logits of this chunk -------------------------------------------
  if (c == 0) {  // the head's radix totals start at zero (first added after a barrier)
    for (int i = tid; i < kBins1; i += kT) st_dev(w.tot1 + (int64_t)h * kBins1 + i, 0u);
    for (int i = tid; i < kBins2; i += kT) st_dev(w.tot2 + (int64_t)h * kBins2 + i, 0u);
    for (int i = tid; i < kBins3; i += kT) st_dev(w.tot3 + (int64_t)h * kBins3 + i, 0u);
  }
  if constexpr (!SEL) {
    bf16x8_t qb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (li < G)
        v = ld16(reinterpret_cast<const char*>(a.q) + ((int64_t)(h * G + li) * D + 32 * s + 8 * q4) * 2);
      qb[s] = as_bf16x8(v);
    }
    const uint32_t span = (uint32_t)(n * a.pos_stride_b);
    const BufRsrc rk = make_rsrc(a.k + (int64_t)h * a.head_stride_b, span);
    const int grp = lane / PPR, pos = lane % PPR;
    uint32_t pk[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int t = grp * NI + u;
      pk[u] = (uint32_t)((pos ^ swz_k<D>(t)) * 16) + (uint32_t)t * stride;
    }
    const int wbase = wave * TB;
    int koff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) koff[s] = wbase + tile_byte<D>(li, (4 * s + q4) ^ swz_k<D>(li));
    const int nsteps = (rows + kStep - 1) / kStep;
    const int nst = wave < nsteps ? (nsteps - 1 - wave) / kW + 1 : 0;
    const float c2 = a.scale_log2;
    float* lg_row = sm_lg + (li < G ? li : 0) * lg_stride;
    auto issue = [&](int u, int k) {
      const int j = wave + kW * k;
      char* dst = &ring[u][wave][0];
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(r0 + (int64_t)j * kStep) * stride);
#pragma unroll
      for (int x = 0; x < NI; ++x) copy_to_lds(rk, dst + x * 1024, pk[x], soff);
    };
    float m = kNegInf, l = 0.0f;  // running max and sum of head li over this lane's keys
    auto step = [&](int u, int k) {
      if (k + 1 < nst) {
        wait_lgkm0();
        issue(u ^ 1, k + 1);
      }
      wait_newer<1, NI>(nst - 1 - k < 1 ? nst - 1 - k : 1);
      const char* base = &ring[u][0][0];
      floatx4_t cs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        cs = mfma_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(base + koff[s])), qb[s], cs);
      const int j = wave + kW * k;
      const int rb = j * kStep + 4 * q4;
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = cs[r] * c2;
      if ((j + 1) * kStep <= rows) {
        if (li < G) *reinterpret_cast<float4*>(lg_row + rb) = make_float4(sv[0], sv[1], sv[2], sv[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = rb + r < rows;
          if (ok && li < G) lg_row[rb + r] = sv[r];
          sv[r] = ok ? sv[r] : kNegInf;
        }
      }
      const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      const float mn = fmaxf(m, mx);
      if (mn != kNegInf) {
        l = l * fast_exp2(m - mn) + fast_exp2(sv[0] - mn) + fast_exp2(sv[1] - mn) +
            fast_exp2(sv[2] - mn) + fast_exp2(sv[3] - mn);
        m = mn;
      }
    };
    if (nst > 0) issue(0, 0);
    for (int k = 0; k < nst; k += 2) {
      step(0, k);
      if (k + 1 < nst) step(1, k + 1);
    }
    float M = xor16_max(m);
    M = xor32_max(M);
    float x = (m == kNegInf) ? 0.0f : l * fast_exp2(m - M);
    x = xor16_sum(x);
    x = xor32_sum(x);
    if (lane < 16) {
      sm_m[wave][lane] = M;
      sm_l[wave][lane] = x;
    }
    __syncthreads();
    if (tid < G) {
      const int g = tid;
      float Mw = sm_m[0][g];
#pragma unroll
      for (int v = 1; v < kW; ++v) Mw = fmaxf(Mw, sm_m[v][g]);
      float L = 0.0f;
#pragma unroll
      for (int v = 0; v < kW; ++v)
        L += (sm_m[v][g] == kNegInf) ? 0.0f : sm_l[v][g] * fast_exp2(sm_m[v][g] - Mw);
      float* st = w.stats + (((int64_t)h * P + c) * G + g) * 2;
      st_dev(st, Mw);
      st_dev(st + 1, L);
    }
  }
  if constexpr (!SEL) head_sync(ctr, (uint32_t)P, a.err);

  // ---- B: scores, level-1 histogram ----------------------------------------
  for (int g = wave; g < (SEL ? 0 : G); g += kW) {
    // the same reduction as the per-step score kernel's finalize
    const float* st = w.stats + (int64_t)h * P * G * 2;
    const bool in0 = lane < P;
    const float m0 = in0 ? ld_dev(st + ((int64_t)lane * G + g) * 2) : kNegInf;
    const float l0 = in0 ? ld_dev(st + ((int64_t)lane * G + g) * 2 + 1) : 0.0f;
    float M = m0;
    for (int cc = lane + 64; cc < P; cc += 64) M = fmaxf(M, ld_dev(st + ((int64_t)cc * G + g) * 2));
    M = wave_max(M);
    float L = (m0 == kNegInf) ? 0.0f : l0 * fast_exp2(m0 - M);
    for (int cc = lane + 64; cc < P; cc += 64) {
      const float mc = ld_dev(st + ((int64_t)cc * G + g) * 2);
      L += (mc == kNegInf) ? 0.0f : ld_dev(st + ((int64_t)cc * G + g) * 2 + 1) * fast_exp2(mc - M);
    }
    L = wave_sum(L);
    if (lane == 0) sm_lse2[g] = M + __log2f(L);
  }
  uint32_t* hist = reinterpret_cast<uint32_t*>(&ring[0][0][0]);
  // thread t holds chunk rows KPT t .. KPT t + KPT - 1
  const int64_t c_lo = a.n_sink, c_hi = n - a.n_recent;
  const int64_t tail = n - a.n_recent > 0 ? n - a.n_recent : 0;
  const int64_t nsink = a.n_sink < tail ? a.n_sink : tail;
  const int64_t ncand = c_lo < c_hi ? c_hi - c_lo : 0;
  int64_t kh = a.k_top;
  if constexpr (SEL)
    if (a.k_per_head) kh = a.k_per_head[h] < 0 ? 0 : a.k_per_head[h];  // clamped to [0, #candidates]
  const int64_t K = kh < ncand ? kh : ncand;
  const bool radix = K > 0 && K < ncand;  // uniform: otherwise the selection goes by index
  // (this barrier also publishes sm_lse2 to every wave)
  if (radix)
    for (int i = tid; i < kCopiesB * kHB / 4; i += kT) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (radix || !SEL) __syncthreads();
  const int rb0 = KPT * tid;
  uint32_t key[KPT];
  // bit u: row rb0 + u lies in [lo, hi) and in the chunk (chunk-relative bounds)
  auto run_mask = [&](int64_t lo, int64_t hi) -> uint32_t {
    hi = hi > rows ? rows : hi;
    lo = lo < rb0 ? 0 : (lo > rb0 + KPT ? KPT : lo - rb0);
    hi = hi < rb0 ? 0 : (hi > rb0 + KPT ? KPT : hi - rb0);
    auto below = [](int64_t x) -> uint32_t { return x >= 32 ? 0xFFFFFFFFu : (1u << x) - 1u; };
    return hi > lo ? below(hi) & ~below(lo) : 0u;
  };
  // candidates of this thread: its rows inside the chunk and inside [c_lo, c_hi)
  const int64_t cl0 = (c_lo > r0 ? c_lo : r0) - r0, ch0 = (c_hi < r0 + rows ? c_hi : r0 + rows) - r0;
  const uint32_t cand = run_mask(cl0, ch0);
  // every thread holds KPT rows and all are candidates (no sink, no recent row)
  const bool interior = rows == KPT * kT && r0 >= c_lo && r0 + rows <= c_hi;
  {
    float sc[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) sc[u] = 0.0f;
    if constexpr (SEL) {  // the given scores: 16-byte loads where the row allows them
      const float* srow = a.score + (int64_t)h * a.score_stride + r0 + rb0;
      if (((uintptr_t)a.score & 15u) == 0 && (a.score_stride & 3) == 0 && rb0 + KPT <= rows) {
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v) {
          const float4 x = reinterpret_cast<const float4*>(srow)[v];
          sc[4 * v] = x.x;
          sc[4 * v + 1] = x.y;
          sc[4 * v + 2] = x.z;
          sc[4 * v + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
          if (rb0 + u < rows) sc[u] = srow[u];
      }
    } else if (rb0 < rows) {
      // every thread with rows reads all KPT logits: rows past the chunk's
      // end read words of the LDS buffer that nothing wrote (still inside
      // it) and are masked out by the candidate flags and the stores below
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float l2 = sm_lse2[g];
        const float* lr = sm_lg + g * lg_stride + rb0;
        if constexpr (KPT % 4 == 0) {  // rows of 16-byte aligned logits
#pragma unroll
          for (int v = 0; v < KPT / 4; ++v) {
            const float4 x = reinterpret_cast<const float4*>(lr)[v];
            sc[4 * v] += fast_exp2(x.x - l2);
            sc[4 * v + 1] += fast_exp2(x.y - l2);
            sc[4 * v + 2] += fast_exp2(x.z - l2);
            sc[4 * v + 3] += fast_exp2(x.w - l2);
          }
        } else {
#pragma unroll
          for (int u = 0; u < KPT; ++u) sc[u] += fast_exp2(lr[u] - l2);
        }
      }
    }
    if (!SEL && a.score) {  // 16-byte stores where the row allows them
      float* srow = a.score + (int64_t)h * a.score_stride + r0 + rb0;
      bool vec = false;
      if constexpr (KPT % 4 == 0)
        vec = ((uintptr_t)a.score & 15u) == 0 && (a.score_stride & 3) == 0 && rb0 + KPT <= rows;
      if (vec) {
#pragma unroll
        for (int v = 0; v < KPT / 4; ++v)
          *reinterpret_cast<float4*>(srow + 4 * v) = make_float4(sc[4 * v], sc[4 * v + 1], sc[4 * v + 2], sc[4 * v + 3]);
      } else {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
          if (rb0 + u < rows) srow[u] = sc[u];
      }
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u) key[u] = score_key(sc[u]);
    if (radix) {
      if (interior) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) atomicAdd(&hist[(lane % kCopiesB) * kHB + hbin(key[u])], 1u);
      } else {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
          if ((cand >> u) & 1u) atomicAdd(&hist[(lane % kCopiesB) * kHB + hbin(key[u])], 1u);
      }
    }
  }

  // ---- C: the threshold key T and how many keys equal to T are kept ---------
  // T = 0 keeps every candidate (keys >= 2^31), T = ~0 none.
  uint32_t T = K == 0 ? 0xFFFFFFFFu : 0u, take = 0, sel_before = 0, my_take = 0;
  uint32_t pre_gt = 0, pre_eq = 0;  // published keys of earlier chunks above / equal to T (this thread's)
  bool pub_path = false;
  uint32_t nb = kSb;  // barriers of the head passed so far
  if (!radix) {
    if (K > 0) {  // every candidate: those of the chunks before this one
      const int64_t lo = r0 < c_lo ? c_lo : (r0 > c_hi ? c_hi : r0);
      sel_before = (uint32_t)(lo - c_lo);
    }
  } else {
    // Every chunk publishes its candidate keys from the 12-bit bin of local
    // rank pub_rank upwards (all of them when it has fewer), padded with zero
    // keys to pub_cap, and that bin's lower edge; after one barrier each
    // workgroup finds the K-th largest published key.  It is T whenever it is
    // not below any chunk's edge: every key at or above it was published.
    // Otherwise (a chunk holds a large share of the top K, or its boundary
    // bin is crowded) the head's global radix levels decide.
    const int mcap = a.pub_cap;
    __syncthreads();
    // bins of local rank pub_rank (the publishing edge) and ceil(K / P): some
    // chunk holds that many of the top K, so T lies below the upper edge of
    // the latter's bin in some chunk
    const int64_t share = (K + P - 1) / P;
    const int64_t rank = 2 * share + 16 < (int64_t)(mcap * 3 / 4) ? 2 * share + 16 : (int64_t)(mcap * 3 / 4);
    pick2_lds<kHB, kCopiesB>(hist, (uint32_t)(rank > 0 ? rank : 1), (uint32_t)share, sm_w, &sm_digit, &sm_krem);
    // 12-bit bins of the two ranks (their index + 1 from the pick, 0 when the
    // chunk has fewer candidates): the publishing edge dl (0: publish all)
    // and the upper edge ub of the second bin
    constexpr uint32_t kOff = SEL ? 0u : 2048u;
    const uint32_t dl = sm_digit ? sm_digit - 1u + kOff : 0u;
    const uint32_t ub = sm_krem == 0u ? 0u : (sm_krem + kOff >= 4096u ? 0xFFFFFFFFu : (sm_krem + kOff) << 20);
    uint32_t np = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) np += (((cand >> u) & 1u) && (key[u] >> 20) >= dl) ? 1u : 0u;
    uint32_t npub;
    uint32_t at = wg_excl_scan(np, sm_w, &npub);
    const bool fits = npub <= (uint32_t)mcap;
    uint32_t* pub = w.pub + ((int64_t)h * P + c) * mcap;
    if (fits) {
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (((cand >> u) & 1u) && (key[u] >> 20) >= dl) st_dev(pub + at++, key[u]);
      for (uint32_t i = npub + tid; i < (uint32_t)mcap; i += kT) st_dev(pub + i, 0u);
    }
    if (tid == 0) {
      st_dev(w.edge + ((int64_t)h * P + c) * 2, fits ? (dl << 20) : 0xFFFFFFFFu);
      st_dev(w.edge + ((int64_t)h * P + c) * 2 + 1, ub);
    }
    head_sync(ctr, (kSb + 1u) * P, a.err);
    nb = kSb + 1u;
    // the head's published keys: thread t holds words 4 (t + kT i) .. 4 (t + kT i) + 3
    const uint32_t nkeys = (uint32_t)(P * mcap);
    const BufRsrc rpub = make_rsrc(w.pub + (int64_t)h * P * mcap, nkeys * 4);
    uint4 pk[kPubW];
#pragma unroll
    for (int i = 0; i < kPubW; ++i) {
      const uint32_t e4 = (uint32_t)(tid + kT * i);
      pk[i] = 4 * e4 < nkeys ? buf_load16_dev(rpub, e4 * 16) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t em = 0, um = 0;
    for (int cc = tid; cc < P; cc += kT) {
      em = max(em, ld_dev(w.edge + ((int64_t)h * P + cc) * 2));
      um = max(um, ld_dev(w.edge + ((int64_t)h * P + cc) * 2 + 1));
    }
    uint32_t edge_max, up;  // T < up (up >= 2^31 + 2^20)
    wg_max2_u32(em, um, sm_w2, &edge_max, &up);
    // only keys >= lo can be T (the search fails when fewer than K are)
    // (above the zero padding; step scores are probabilities, keys >= 2^31)
    const uint32_t lo = edge_max > (SEL ? 1u : 0x80000000u) ? edge_max : (SEL ? 1u : 0x80000000u);
    bool valid = edge_max != 0xFFFFFFFFu && lo < up;
    if (valid) {
      // 2048 bins of width 2^sh over [lo, up) (keys above in the last one,
      // kCopies privatised copies), the bin holding the K-th largest key,
      // then that key by ranking the bin's keys (at most kRankMax, else the
      // global levels decide)
      const uint32_t span = up - 1u - lo;
      const int bl = span ? 32 - __clz(span) : 0;
      const int sh = bl > 11 ? bl - 11 : 0;
      for (int i = tid; i < kCopies * 2048 / 4; i += kT) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
      // (keys below lo go to a spare word of their lane: no branch, no conflict)
      uint32_t* spare = hist + kCopies * 2048 + kRankMax;
#pragma unroll
      for (int i = 0; i < kPubW; ++i) {
        const uint32_t kk[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          atomicAdd(kk[j] >= lo ? &hist[(lane % kCopies) * 2048 + min((kk[j] - lo) >> sh, 2047u)] : &spare[lane], 1u);
      }
      __syncthreads();
      pick_lds<2048, kCopies>(hist, (uint32_t)K, sm_w, &sm_digit, &sm_krem, 0u);
      const uint32_t d1 = sm_digit, k1 = sm_krem;  // k1 == 0: fewer than K keys >= lo
      // the bin's keys, gathered into LDS (a handful: the bins are narrow)
      uint32_t* cl = hist + kCopies * 2048;
      if (tid == 0) sm_base = 0u;
      __syncthreads();
      if (k1) {
        // bin d1 holds the keys blo .. bhi (the last bin everything above;
        // a bin reaching past 2^32 - 1 ends there)
        const uint32_t blo = lo + (d1 << sh), wb = (1u << sh) - 1u;
        const uint32_t bhi = d1 == 2047u || blo > 0xFFFFFFFFu - wb ? 0xFFFFFFFFu : blo + wb;
        uint32_t hit = 0;  // bit 4 i + j: slot (i, j) lies in the bin
#pragma unroll
        for (int i = 0; i < kPubW; ++i) {
          const uint32_t kk[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) hit |= (kk[j] >= blo && kk[j] <= bhi ? 1u : 0u) << (4 * i + j);
        }
        while (hit) {
          const int b = __builtin_ctz(hit);
          hit &= hit - 1u;
          uint32_t x = 0;
#pragma unroll
          for (int i = 0; i < kPubW; ++i) {  // slot b's key without dynamic register indexing
            const uint32_t kk[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) x = b == 4 * i + j ? kk[j] : x;
          }
          const uint32_t at2 = atomicAdd(&sm_base, 1u);
          if (at2 < (uint32_t)kRankMax) cl[at2] = x;
        }
      }
      __syncthreads();
      const uint32_t nb = sm_base;
      valid = k1 != 0u && nb <= (uint32_t)kRankMax;
      if (valid) {
        // x is T when fewer than k1 of the bin's keys exceed it and k1 reach it
        if (nb <= 64u) {  // one wave, the keys broadcast from its lanes
          if (wave == 0) {
            const uint32_t x = (uint32_t)lane < nb ? cl[lane] : 0u;
            uint32_t gt = 0, ge = 0;
            for (uint32_t i = 0; i < nb; ++i) {
              const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)i);
              gt += y > x ? 1u : 0u;
              ge += y >= x ? 1u : 0u;
            }
            if ((uint32_t)lane < nb && gt < k1 && k1 <= ge) {  // lanes holding the same x agree
              sm_digit = x;
              sm_krem = k1 - gt;
            }
          }
        } else if ((uint32_t)tid < nb) {
          const uint32_t x = cl[tid];
          uint32_t gt = 0, ge = 0;
          for (uint32_t i = 0; i < nb; ++i) {
            const uint32_t y = cl[i];
            gt += y > x ? 1u : 0u;
            ge += y >= x ? 1u : 0u;
          }
          if (gt < k1 && k1 <= ge) {
            sm_digit = x;
            sm_krem = k1 - gt;
          }
        }
        __syncthreads();
        T = sm_digit;
        take = sm_krem;
      }
    }
    if (valid) {
      // published keys of the chunks before this one, above T and equal to T
      // (summed over the workgroup with the kept-row scan)
      // (a word's four keys come from one chunk: pub_cap is a multiple of 4)
      const uint32_t e_end = (uint32_t)(c * mcap);
#pragma unroll
      for (int i = 0; i < kPubW; ++i) {
        const uint32_t kk[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ngt += kk[j] > T ? 1u : 0u;
          neq += kk[j] == T ? 1u : 0u;
        }
        const bool before = 4u * (uint32_t)(tid + kT * i) < e_end;
        pre_gt += before ? ngt : 0u;
        pre_eq += before ? neq : 0u;
      }
      pub_path = true;
    } else {
      // Radix levels over the head's global histograms: bits 31..20, 19..9,
      // 8..0, then every chunk's counts above and equal to T.
      for (int i = tid; i < kBins1; i += kT) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if ((cand >> u) & 1u) atomicAdd(&hist[key[u] >> 20], 1u);
      __syncthreads();
      for (int i = tid; i < kBins1; i += kT) {
        const uint32_t x = hist[i];
        if (x) atomicAdd(w.tot1 + (int64_t)h * kBins1 + i, x);
      }
      head_sync(ctr, (kSb + 2u) * P, a.err);
      pick_bin<kBins1>(w.tot1 + (int64_t)h * kBins1, (uint32_t)K, sm_w, &sm_digit, &sm_krem);
      const uint32_t d1 = sm_digit, krem1 = sm_krem;
      for (int i = tid; i < kBins2; i += kT) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (((cand >> u) & 1u) && (key[u] >> 20) == d1) atomicAdd(&hist[(key[u] >> 9) & (kBins2 - 1)], 1u);
      __syncthreads();
      for (int i = tid; i < kBins2; i += kT) {
        const uint32_t x = hist[i];
        if (x) atomicAdd(w.tot2 + (int64_t)h * kBins2 + i, x);
      }
      head_sync(ctr, (kSb + 3u) * P, a.err);
      pick_bin<kBins2>(w.tot2 + (int64_t)h * kBins2, krem1, sm_w, &sm_digit, &sm_krem);
      const uint32_t q2 = (d1 << 11) | sm_digit, krem2 = sm_krem;
      for (int i = tid; i < kBins3; i += kT) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (((cand >> u) & 1u) && (key[u] >> 9) == q2) atomicAdd(&hist[key[u] & (kBins3 - 1)], 1u);
      __syncthreads();
      for (int i = tid; i < kBins3; i += kT) {
        const uint32_t x = hist[i];
        if (x) atomicAdd(w.tot3 + (int64_t)h * kBins3 + i, x);
      }
      head_sync(ctr, (kSb + 4u) * P, a.err);
      pick_bin<kBins3>(w.tot3 + (int64_t)h * kBins3, krem2, sm_w, &sm_digit, &sm_krem);
      T = (q2 << 9) | sm_digit;
      take = sm_krem;
      uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const bool cu = (cand >> u) & 1u;
        n_gt += (cu && key[u] > T) ? 1u : 0u;
        n_eq += (cu && key[u] == T) ? 1u : 0u;
      }
      uint32_t tot;  // both counts below 2^16: one scan
      wg_excl_scan((n_eq << 16) | n_gt, sm_w, &tot);
      if (tid == 0) {
        st_dev(w.cnts + ((int64_t)h * P + c) * 2, tot & 0xFFFFu);
        st_dev(w.cnts + ((int64_t)h * P + c) * 2 + 1, tot >> 16);
      }
      head_sync(ctr, (kSb + 5u) * P, a.err);
      nb = kSb + 5u;
      // chunks before this one: selected keys and keys equal to T
      uint32_t sb = 0, eq_before = 0;
      for (int c0 = 0; c0 < c; c0 += kT) {
        const int cc = c0 + tid;
        const uint32_t g_ = cc < c ? ld_dev(w.cnts + ((int64_t)h * P + cc) * 2) : 0u;
        const uint32_t e_ = cc < c ? ld_dev(w.cnts + ((int64_t)h * P + cc) * 2 + 1) : 0u;
        uint32_t eq_all;
        const uint32_t eq_ex = wg_excl_scan(e_, sm_w, &eq_all);
        const uint32_t e0 = eq_before + eq_ex;
        const uint32_t tk = e0 >= take ? 0u : (take - e0 < e_ ? take - e0 : e_);
        uint32_t sel_all;
        wg_excl_scan(g_ + tk, sm_w, &sel_all);
        sb += sel_all;
        eq_before += eq_all;
      }
      sel_before = sb;
      my_take = eq_before >= take ? 0u : take - eq_before;
    }
  }

  // ---- E: kept indices, attention partial, merge -----------------------------
  {
    // Positions from one scan: this thread's selected keys start at (keys
    // above T before it) + min(keys equal to T before it, my_take) in the
    // chunk's selection, its kept rows there plus the forced rows (sinks,
    // recent run) before it.  The same exchange sums the published keys of
    // earlier chunks (the selection before this chunk).
    // the forced rows of this thread: sinks and the recent run
    const uint32_t forcedm = interior ? 0u : (run_mask(-r0, nsink - r0) | run_mask(tail - r0, rows));
    // The selection alone: this workgroup's final arrival goes out now (every
    // barrier of the head is behind it), its answer is read at the end, and
    // the scan below takes an LDS-only barrier so that nothing waits for it
    // meanwhile.  The head's last arrival clears its counters.
    // (set in thread 0 only: no value for the other lanes to merge with, so
    // nothing waits for the answer before its use)
    uint32_t arrived;
    if constexpr (SEL)
      if (tid == 0) arrived = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t n_gt = 0, n_eq = 0;
    const uint32_t n_f = (uint32_t)__builtin_popcount(forcedm);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool cu = (cand >> u) & 1u;
      n_gt += (cu && key[u] > T) ? 1u : 0u;
      n_eq += (cu && key[u] == T) ? 1u : 0u;
    }
    uint32_t ex_gf, ex_eq, tot_gf, tot_eq, tot_pre;
    {
      const uint32_t v0 = (n_f << 16) | n_gt, v2 = (pre_eq << 16) | pre_gt;
      const uint32_t x0 = wave_incl_scan(v0), x1 = wave_incl_scan(n_eq), x2 = wave_incl_scan(v2);
      if (lane == 63) {
        sm_w2[wave] = x0;
        sm_w2[kW + wave] = x1;
        sm_w[wave] = x2;
      }
      if constexpr (SEL) {
        wait_lgkm0();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      } else {
        __syncthreads();
      }
      uint32_t b0 = 0, b1 = 0, t0 = 0, t1 = 0, t2 = 0;
#pragma unroll
      for (int v = 0; v < kW; ++v) {
        const uint32_t c0 = sm_w2[v], c1 = sm_w2[kW + v];
        b0 += v < wave ? c0 : 0u;
        b1 += v < wave ? c1 : 0u;
        t0 += c0;
        t1 += c1;
        t2 += sm_w[v];
      }
      ex_gf = b0 + x0 - v0;
      ex_eq = b1 + x1 - n_eq;
      tot_gf = t0;  // counts below 2^16
      tot_eq = t1;
      tot_pre = t2;  // counts up to 2^14
    }
    if (pub_path) {
      const uint32_t eq_b = tot_pre >> 16;
      sel_before = (tot_pre & 0xFFFFu) + (eq_b < take ? eq_b : take);
      my_take = eq_b >= take ? 0u : take - eq_b;
    }
    const uint32_t eq_sel = ex_eq < my_take ? ex_eq : my_take;
    uint32_t s_at = (uint32_t)nsink + sel_before + (ex_gf & 0xFFFFu) + eq_sel;
    uint32_t k_at = (ex_gf & 0xFFFFu) + eq_sel + (ex_gf >> 16);
    const uint32_t nkeep = (tot_gf & 0xFFFFu) + (tot_eq < my_take ? tot_eq : my_take) + (tot_gf >> 16);
    uint32_t eq_rank = ex_eq;
    uint32_t selm = 0, keepm = 0;  // bit u: row rb0 + u selected / attended (selected, sink, recent)
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool cu = (cand >> u) & 1u;
      const bool eq = cu && key[u] == T;
      const bool s_ = cu && (key[u] > T || (eq && eq_rank < my_take));
      eq_rank += eq ? 1u : 0u;
      selm |= (s_ ? 1u : 0u) << u;
    }
    keepm = selm | forcedm;
    if constexpr (SEL) {  // the selection alone: indices, count, and the counters' reset
      (void)k_at;
      (void)nkeep;
      int32_t* orow = a.idx + (int64_t)h * a.idx_stride;
      for (uint32_t m = selm; m; m &= m - 1u) {
        if (s_at < (uint64_t)a.idx_stride) orow[s_at] = (int32_t)(r0 + rb0 + __builtin_ctz(m));
        ++s_at;
      }
      if (c == 0) {
        for (int64_t i = tid; i < nsink; i += kT) orow[i] = (int32_t)i;
        if (tid == 0) a.count[h] = (int32_t)(nsink + K);
      }
      if (tid == 0 && arrived == (nb + 1u) * (uint32_t)P - 1u) {
        st_dev(ctr, 0u);
        st_dev(ctr + 16, 0u);
      }
      return;
    }
    uint32_t* kept = hist;  // the chunk's kept rows (the ring is free again)
    for (uint32_t m = keepm; m; m &= m - 1u) kept[k_at++] = (uint32_t)(rb0 + __builtin_ctz(m));
    __syncthreads();
    // sum_e 2^(l - m) v over the kept rows: LPR lanes per V row, RSL rows per
    // step, kU per slot in flight; acc[g][x] holds channels 8 (lane % LPR) +
    // x; m is the wave's running maximum (rescaled when a batch raises it).
    const int slot = tid / LPR, piece = tid - slot * LPR;
    const char* vb = a.v + (int64_t)h * a.head_stride_b + piece * 16;
    constexpr int kU = G <= 4 ? 8 : (G <= 8 ? 4 : 2);  // rows per slot in flight
    uint4 vr[kU];
    uint32_t rr[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t e = slot + u * RSL;
      rr[u] = e < nkeep ? kept[e] : 0xFFFFFFFFu;
      vr[u] = e < nkeep ? ld16(vb + (r0 + rr[u]) * a.pos_stride_b) : make_uint4(0u, 0u, 0u, 0u);
    }
    // the selected indices go out while the V rows are in flight (ascending)
    int32_t* orow = a.idx + (int64_t)h * a.idx_stride;
    for (uint32_t m = selm; m; m &= m - 1u) {
      if (s_at < (uint64_t)a.idx_stride) orow[s_at] = (int32_t)(r0 + rb0 + __builtin_ctz(m));  // never past the row
      ++s_at;
    }
    if (c == 0) {
      for (int64_t i = tid; i < nsink; i += kT) orow[i] = (int32_t)i;
      if (tid == 0) a.count[h] = (int32_t)(nsink + K);
    }
    float acc[G][8], lsum[G], mg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mg[g] = kNegInf;
      lsum[g] = 0.0f;
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[g][x] = 0.0f;
    }
    // (the batch loop runs the same trips in every lane of a wave: the
    // wave-wide maxima need all its lanes)
    const uint32_t wave_slot0 = (uint32_t)(wave * (64 / LPR));
    for (uint32_t b = 0;;) {
      float lg[kU][G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float bm = kNegInf;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          lg[u][g] = rr[u] == 0xFFFFFFFFu ? kNegInf : sm_lg[g * lg_stride + (rr[u] == 0xFFFFFFFFu ? 0u : rr[u])];
          bm = fmaxf(bm, lg[u][g]);
        }
        bm = wave_max(bm);
        if (bm > mg[g]) {  // wave-uniform
          const float f = mg[g] == kNegInf ? 0.0f : fast_exp2(mg[g] - bm);
          lsum[g] *= f;
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[g][x] *= f;
          mg[g] = bm;
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (rr[u] == 0xFFFFFFFFu) continue;
        float vf[8];
        vf[0] = bf16lo(vr[u].x); vf[1] = bf16hi(vr[u].x);
        vf[2] = bf16lo(vr[u].y); vf[3] = bf16hi(vr[u].y);
        vf[4] = bf16lo(vr[u].z); vf[5] = bf16hi(vr[u].z);
        vf[6] = bf16lo(vr[u].w); vf[7] = bf16hi(vr[u].w);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = fast_exp2(lg[u][g] - mg[g]);
          lsum[g] += p;
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[g][x] = fmaf(p, vf[x], acc[g][x]);
        }
      }
      b += kU * RSL;
      if (wave_slot0 + b >= nkeep) break;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t e = slot + b + u * RSL;
        rr[u] = e < nkeep ? kept[e] : 0xFFFFFFFFu;
        vr[u] = e < nkeep ? ld16(vb + (r0 + rr[u]) * a.pos_stride_b) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // fold the slots of a wave (lanes piece, piece + LPR, ...), then the
    // waves, each weighted by 2^(m_wave - M)
    __syncthreads();  // every wave is done with its kept list
    float* red = reinterpret_cast<float*>(&ring[0][0][0]);  // [kW][G][D + 1]
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[g][x] = slot_sum<LPR>(acc[g][x]);
      lsum[g] = slot_sum<LPR>(lsum[g]);
      if (lane < LPR) {
#pragma unroll
        for (int x = 0; x < 8; ++x) red[(wave * G + g) * (D + 1) + 8 * piece + x] = acc[g][x];
        if (piece == 0) red[(wave * G + g) * (D + 1) + D] = lsum[g];
      }
      if (lane == 0) sm_m[wave][g] = mg[g];
    }
    __syncthreads();
    float* pml = w.part_ml + ((int64_t)h * P + c) * G * 2;
    float* pac = w.part_acc + ((int64_t)h * P + c) * G * D;
    for (int e = tid; e < G * (D + 1); e += kT) {
      const int g = e / (D + 1), x = e - g * (D + 1);
      float M = kNegInf;
#pragma unroll
      for (int v = 0; v < kW; ++v) M = fmaxf(M, sm_m[v][g]);
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < kW; ++v) {
        const float mv = sm_m[v][g];
        s += mv == kNegInf ? 0.0f : red[(v * G + g) * (D + 1) + x] * fast_exp2(mv - M);
      }
      if (x < D) pac[g * D + x] = s;
      else {
        pml[g * 2] = M;
        pml[g * 2 + 1] = s;
      }
    }
  }
}

template <int D, int G>
hipError_t launch_dg(const TopkArgs& a, void* scratch, hipStream_t s) {
  if (a.chunks_per_head > kMaxP || a.chunks_per_head < 1) return hipErrorInvalidValue;
  TopkArgs b = a;
  // each chunk publishes up to pub_cap keys
  const int P = a.chunks_per_head;
  b.pub_cap = (kPubKeys / P) & ~3;
  b.k_per_head = nullptr;
  TopkWs w = topk_ws_layout(b, scratch, G, D);
  hipLaunchKernelGGL((topk_step_kernel<D, G, false>), dim3((unsigned)(a.n_kv_heads * P)), dim3(kT), 0, s, b, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the P partials of each kv head merged by the split-K merge kernel, which
  // also clears the step's counters for its next call
  MergeArgs m{};
  m.part_ml = w.part_ml;
  m.part_acc = w.part_acc;
  m.nch = nullptr;
  m.n_kv_heads = a.n_kv_heads;
  m.cph = P;
  m.rows_per_head = G;
  m.group = G;
  m.out = a.out;
  m.lse = a.lse;
  m.clear_ctr = a.ctr;
  m.clear_heads = a.n_kv_heads;
  return launch_merge(D, m, s);
}

template <int D>
hipError_t launch_d(int g, const TopkArgs& a, void* scratch, hipStream_t s) {
  switch (g) {
    case 1: return launch_dg<D, 1>(a, scratch, s);
    case 2: return launch_dg<D, 2>(a, scratch, s);
    case 3: return launch_dg<D, 3>(a, scratch, s);
    case 4: return launch_dg<D, 4>(a, scratch, s);
    case 5: return launch_dg<D, 5>(a, scratch, s);
    case 6: return launch_dg<D, 6>(a, scratch, s);
    case 7: return launch_dg<D, 7>(a, scratch, s);
    case 8: return launch_dg<D, 8>(a, scratch, s);
    case 16: return launch_dg<D, 16>(a, scratch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

template <int D>
int max_chunk_d(int g) {
  switch (g) {
    case 1: return Chunk<D, 1>::kMax;
    case 2: return Chunk<D, 2>::kMax;
    case 3: return Chunk<D, 3>::kMax;
    case 4: return Chunk<D, 4>::kMax;
    case 5: return Chunk<D, 5>::kMax;
    case 6: return Chunk<D, 6>::kMax;
    case 7: return Chunk<D, 7>::kMax;
    case 8: return Chunk<D, 8>::kMax;
    case 16: return Chunk<D, 16>::kMax;
    default: return 0;
  }
}
int topk_step_max_chunk(int g, int d) { return d == 128 ? max_chunk_d<128>(g) : (d == 64 ? max_chunk_d<64>(g) : 0); }
int topk_step_granule() { return kGranule; }

size_t topk_step_scratch(int hkv, int p, int g, int d) {
  size_t off[10];
  topk_offsets(hkv, p, g, d, off);
  return off[9];
}

hipError_t launch_topk_select(const TopkArgs& a, void* scratch, hipStream_t s) {
  if (a.chunks_per_head > kMaxP || a.chunks_per_head < 1 || a.chunk > kSelKpt * kT) return hipErrorInvalidValue;
  TopkArgs b = a;
  const int P = a.chunks_per_head;
  b.pub_cap = (kPubKeys / P) & ~3;
  TopkWs w = topk_ws_layout(b, scratch, 1, 128);
  hipLaunchKernelGGL((topk_step_kernel<128, 1, true>), dim3((unsigned)(a.n_kv_heads * P)), dim3(kT), 0, s, b, w);
  return hipGetLastError();
}
int topk_select_max_chunk() { return kSelKpt * kT; }
int topk_publish_budget() { return kPubKeys; }
size_t topk_select_scratch(int hkv, int p) { return topk_step_scratch(hkv, p, 1, 128); }

hipError_t launch_topk_step(int d, int g, const TopkArgs& a, void* scratch, hipStream_t s) {
  if (d == 128) return launch_d<128>(g, a, scratch, s);
  if (d == 64) return launch_d<64>(g, a, scratch, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
