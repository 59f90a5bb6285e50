// score_obs.hip -- observation-window score on MFMA.
//
// Method: the kept entries of each kv head are chosen by the attention that
// the last W queries give every key, averaged over the window and summed over
// the query heads of a GQA group ("Sparse-to-Dense ..." Sec. 3.2 equation for
// Cache_s[l] and its GQA rule; the observation window of the last 32 queries
// in the SparseMM blog; the cache scored once by the last prompt queries in
// "Where Activation Sparsity and KV-Cache Sparsity Cross ...").  Window query i
// sits at position n - W + i and sees keys j <= n - W + i:
//   s_h(j) = (1/W) sum_{g in group(h)} sum_i exp(l_{g,i}(j) - lse_{g,i}).
//
// The W x G query rows of a kv head against its keys form a real dense
// contraction, so S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16: a wave keeps
// 64 keys (4 tiles) as A operands in registers and streams 16-row tiles of Q
// as B operands.  A row's probabilities need its normaliser over all keys, so
// pass 1 writes per-(row, 256-key block) (max, sum), a small kernel merges
// them into lse per row, and pass 2 recomputes S and accumulates exp(l - lse)
// per key over the rows (DPP sum over the 16 row lanes at the end).
#include "skv_kernels.h"
#include "skv_mfma.h"
#include "skv_tile.h"

namespace skv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 256;
constexpr int kKT = 4;                      // 16-key tiles of K per wave (A operands in registers)
constexpr int kBlockKeys = 16 * kKT * kWaves;  // keys per workgroup

struct RowInfo {
  bool ok;
  int64_t qoff;     // element offset of the row's query
  int64_t last;     // last visible key
};

__device__ __forceinline__ RowInfo row_info(const ScoreObsArgs& a, int h, int row, int D) {
  const int G = a.group, R = a.n_obs * G, Hq = a.n_kv_heads * G;
  RowInfo ri;
  ri.ok = row < R;
  const int i = ri.ok ? row / G : 0;
  const int g = ri.ok ? row - i * G : 0;
  ri.qoff = ((int64_t)i * Hq + h * G + g) * D;
  ri.last = a.n - a.n_obs + i;
  return ri;
}

template <int D>
__device__ __forceinline__ void load_k_tiles(const ScoreObsArgs& a, int h, int64_t kw0, int q4, int i16,
                                             bf16x8_t (&kf)[kKT][D / 32]) {
  const char* kb = a.k + (int64_t)h * a.head_stride_b;
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
    int64_t key = kw0 + kt * 16 + i16;
    key = key < a.n ? key : a.n - 1;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      kf[kt][ks] = as_bf16x8(ld16(kb + key * a.pos_stride_b + (ks * 32 + q4 * 8) * 2));
  }
}

// Query rows reach the waves through LDS: a workgroup stages kChunk 16-row
// tiles of Q at a time (double-buffered), so the four waves share one copy.
// The next chunk is loaded into registers while the current one is used and
// written to LDS after it, so one barrier per chunk both publishes a chunk and
// frees the buffer it replaces.  Rows are XOR-swizzled by row (swz_q) so the
// B-operand reads (16 rows x one 16-byte piece per 16 lanes) are free of bank
// conflicts.
constexpr int kChunk = 8;  // Q tiles per chunk

// Workgroup barrier after this wave's LDS writes have completed; outstanding
// global loads (the next chunk) and statistics stores stay in flight across
// it.  The signal fences keep the compiler from moving memory operations
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D>
struct QGeom {
  static constexpr int kRB = D * 2;                  // bytes per query row
  static constexpr int kPPR = kRB / 16;              // 16-byte pieces per row
  static constexpr int kTileB = 16 * kRB;            // bytes per 16-row tile
  static constexpr int kChunkB = kChunk * kTileB;
  static constexpr int kPPT = kChunkB / 16 / kThreads;  // pieces per thread per chunk
};

// This thread's pieces of chunk c: piece e = tid + kThreads j is piece e % kPPR
// of chunk row e / kPPR (rows past the window repeat a valid row).
template <int D>
__device__ __forceinline__ void load_q_chunk(const ScoreObsArgs& a, int h, int c, int tid,
                                             uint4 (&v)[QGeom<D>::kPPT]) {
  using QG = QGeom<D>;
  const int R = a.n_obs * a.group;
#pragma unroll
  for (int j = 0; j < QG::kPPT; ++j) {
    const int e = tid + kThreads * j;
    int row = c * kChunk * 16 + e / QG::kPPR;
    row = row < R ? row : R - 1;
    const RowInfo ri = row_info(a, h, row, D);
    v[j] = ld16(a.q + ri.qoff + (e % QG::kPPR) * 8);
  }
}

template <int D>
__device__ __forceinline__ void store_q_chunk(char* dst, int tid, const uint4 (&v)[QGeom<D>::kPPT]) {
  using QG = QGeom<D>;
#pragma unroll
  for (int j = 0; j < QG::kPPT; ++j) {
    const int e = tid + kThreads * j;
    const int rloc = e / QG::kPPR, piece = e % QG::kPPR;
    *reinterpret_cast<uint4*>(dst + rloc * QG::kRB + ((piece ^ swz_q<D>(rloc & 15)) * 16)) = v[j];
  }
}

// B operand of tile tt of a staged chunk: row i16, channels [32 ks + 8 q4, +8).
template <int D>
__device__ __forceinline__ void read_q_tile(const char* chunk, int tt, int q4, int i16, bf16x8_t (&qb)[D / 32]) {
  using QG = QGeom<D>;
  const char* row = chunk + tt * QG::kTileB + i16 * QG::kRB;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(row + (((4 * ks + q4) ^ swz_q<D>(i16)) * 16)));
}

template <int D>
__device__ __forceinline__ void s_tiles(const bf16x8_t (&kf)[kKT][D / 32], const bf16x8_t (&qb)[D / 32],
                                        floatx4_t (&s)[kKT]) {
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) acc = mfma_bf16(kf[kt][ks], qb[ks], acc);
    s[kt] = acc;
  }
}

// Workgroup -> (kv head h, key block kb, row group g) and the range of query
// chunks [c0, c0 + nch) the group covers.  Workgroups are dealt to the eight
// XCDs in turn (block b to XCD b mod 8), and each XCD has its own L2: the row
// groups of one (kv head, key block) tile take blocks b, b + 8, b + 16, ...,
// so they run on one XCD and the tile's keys come from HBM once and from that
// L2 for the other groups.  The grid is padded to whole tiles per XCD; a
// workgroup past the last tile is not live.
constexpr int kXcds = 8;
struct ObsTile {
  int h, kb, g, c0, nch;
  bool live;
};
__device__ __forceinline__ ObsTile obs_tile(const ScoreObsArgs& a, int NCH) {
  ObsTile t;
  const int rg = a.row_groups;
  const int xcd = (int)(blockIdx.x % kXcds), local = (int)(blockIdx.x / kXcds);
  const int tl = local / rg;
  const int g = local - tl * rg;
  t.g = g;
  const int hk = tl * kXcds + xcd;
  t.live = hk < a.n_kv_heads * a.n_kblocks;
  t.h = t.live ? hk / a.n_kblocks : 0;
  t.kb = t.live ? hk - t.h * a.n_kblocks : 0;
  const int per = (NCH + rg - 1) / rg;
  t.c0 = g * per;
  t.nch = NCH - t.c0 < per ? NCH - t.c0 : per;
  if (t.nch < 0) t.nch = 0;
  return t;
}

// NBUF: query-chunk buffers in LDS.  A workgroup that walks one chunk (at
// most 128 window rows per row group) needs one, which halves the LDS of the
// kernel and the registers of the prefetch, so more workgroups share a CU.
template <int D, int NBUF>
__global__ __launch_bounds__(kThreads) void obs_pass1_kernel(const ScoreObsArgs a) {
  using QG = QGeom<D>;
  __shared__ __attribute__((aligned(16))) char qc[NBUF][QG::kChunkB];
  __shared__ float sm_ml[NBUF][kChunk][kWaves][16][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int n = (int)a.n;
  const int R = a.n_obs * a.group;
  const int RT = (R + 15) / 16;
  const int NCH_ALL = (RT + kChunk - 1) / kChunk;
  const ObsTile tl = obs_tile(a, NCH_ALL);
  const int h = tl.h, kb = tl.kb, NCH = NBUF == 1 && tl.nch > 1 ? 1 : tl.nch;  // the host picks NBUF
  if (!tl.live || NCH == 0) return;  // padding, or a row group past the last chunk: nothing to do
  auto buf = [](int c) { return NBUF == 1 ? 0 : (c & 1); };
  const int kw0 = kb * kBlockKeys + wave * 16 * kKT;  // keys are below 2^31
  // every window row sees keys <= n - W: no masks for a wave below that
  const bool all_vis = kw0 + 16 * kKT - 1 <= n - a.n_obs;
  // the workgroups of a kv head walk the query chunks from different starting
  // points, so they do not all fetch the same chunk at the same time
  const int rot = kb % NCH;
  auto cid = [&](int c) { return tl.c0 + (c + rot < NCH ? c + rot : c + rot - NCH); };

  bf16x8_t kf[kKT][D / 32];
  load_k_tiles<D>(a, h, kw0, q4, i16, kf);
  {
    uint4 v[QG::kPPT];
    load_q_chunk<D>(a, h, cid(0), tid, v);
    store_q_chunk<D>(qc[0], tid, v);
  }
  // K and the first chunk have landed: inside the loop only the next chunk's
  // loads are in flight, and the matrix work never waits for them
  wait_vm<0>();
  // per-row (max, sum) of the workgroup's keys for the tiles of chunk cc
  auto combine = [&](int c) {
    const int cc = cid(c);
    const int nt = RT - cc * kChunk < kChunk ? RT - cc * kChunk : kChunk;
    if (tid < nt * 16) {
      const int tt = tid >> 4, rr = tid & 15;
      const int row = (cc * kChunk + tt) * 16 + rr;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[buf(c)][tt][w][rr][0]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw2 = sm_ml[buf(c)][tt][w][rr][0];
        L += mw2 == kNegInf ? 0.0f : sm_ml[buf(c)][tt][w][rr][1] * fast_exp2(mw2 - M);
      }
      if (row < R) {
        float* ml = a.part_ml + (((int64_t)h * a.n_kblocks + kb) * R + row) * 2;
        ml[0] = M;
        ml[1] = L;
      }
    }
  };

  for (int c = 0; c < NCH; ++c) {
    uint4 nxt[QG::kPPT];
    if (NBUF > 1 && c + 1 < NCH) load_q_chunk<D>(a, h, cid(c + 1), tid, nxt);
    lds_barrier();  // chunk c and the statistics of chunk c - 1 are in LDS
    if (c > 0) combine(c - 1);
    const char* qchunk = qc[buf(c)];
    const int ci = cid(c);
    const int nt = RT - ci * kChunk < kChunk ? RT - ci * kChunk : kChunk;
    const float c2 = a.scale_log2;
#pragma unroll
    for (int tt = 0; tt < kChunk; ++tt) {
      if (tt >= nt) break;  // uniform
      bf16x8_t qb[D / 32];
      read_q_tile<D>(qchunk, tt, q4, i16, qb);
      floatx4_t s[kKT];
      s_tiles<D>(kf, qb, s);
      // S^T = K Q^T: lane (q4, i16) holds keys 16 kt + 4 q4 + r of query row
      // 16 rt + i16.  The scale (> 0) is applied after the max, inside the
      // exponent's fused multiply-add.
      float mw = kNegInf;
      if (!all_vis) {
        const int last = (int)row_info(a, h, (ci * kChunk + tt) * 16 + i16, D).last;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kw0 + kt * 16 + q4 * 4 + r;
            if (!(key < n && key <= last)) s[kt][r] = kNegInf;
          }
        }
      }
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
        mw = fmaxf(mw, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
      mw = xor16_max(mw);
      mw = xor32_max(mw);
      const float mu = mw == kNegInf ? 0.0f : mw * c2;
      float lw = 0.0f;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) lw += fast_exp2(fmaf(s[kt][r], c2, -mu));
      }
      lw = xor16_sum(lw);
      lw = xor32_sum(lw);
      if (q4 == 0) {
        sm_ml[buf(c)][tt][wave][i16][0] = mw == kNegInf ? kNegInf : mu;
        sm_ml[buf(c)][tt][wave][i16][1] = lw;
      }
    }
    // the buffer of chunk c + 1 was last read in iteration c - 1, before the
    // barrier above
    if (NBUF > 1 && c + 1 < NCH) store_q_chunk<D>(qc[buf(c + 1)], tid, nxt);
  }
  lds_barrier();
  combine(NCH - 1);
}

// lse of every window row from its per-block statistics: one wave per row,
// lanes over the key blocks.
__global__ __launch_bounds__(kThreads) void obs_lse_kernel(const ScoreObsArgs a, int rblocks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.x / rblocks;
  const int row = (blockIdx.x - h * rblocks) * kWaves + wave;
  const int R = a.n_obs * a.group;
  if (row >= R) return;
  const float* ml = a.part_ml + (int64_t)h * a.n_kblocks * R * 2;
  // statistics of the row's key blocks, loaded once (blocks lane, lane+64, ...)
  constexpr int kPer = 8;  // up to 512 key blocks (131072 keys) in one round
  float bm[kPer], bl[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int kb = lane + 64 * i;
    const int kc = kb < a.n_kblocks ? kb : a.n_kblocks - 1;
    bm[i] = kb < a.n_kblocks ? ml[((int64_t)kc * R + row) * 2] : kNegInf;
    bl[i] = ml[((int64_t)kc * R + row) * 2 + 1];
  }
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < kPer; ++i) M = fmaxf(M, bm[i]);
  for (int kb = lane + 64 * kPer; kb < a.n_kblocks; kb += 64) M = fmaxf(M, ml[((int64_t)kb * R + row) * 2]);
  M = wave_max(M);
  float L = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) L += bm[i] == kNegInf ? 0.0f : bl[i] * fast_exp2(bm[i] - M);
  for (int kb = lane + 64 * kPer; kb < a.n_kblocks; kb += 64) {
    const float m = ml[((int64_t)kb * R + row) * 2];
    L += m == kNegInf ? 0.0f : ml[((int64_t)kb * R + row) * 2 + 1] * fast_exp2(m - M);
  }
  L = wave_sum(L);
  if (lane == 0) a.row_lse2[(int64_t)h * R + row] = M + __log2f(L);
}

template <int D, int NBUF>
__global__ __launch_bounds__(kThreads) void obs_pass2_kernel(const ScoreObsArgs a) {
  using QG = QGeom<D>;
  constexpr int kL2 = kChunk * 16;  // row normalisers per chunk
  __shared__ __attribute__((aligned(16))) char qc[NBUF][QG::kChunkB];
  __shared__ float l2c[NBUF][kL2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int n = (int)a.n;
  const int R = a.n_obs * a.group;
  const int RT = (R + 15) / 16;
  const int NCH_ALL = (RT + kChunk - 1) / kChunk;
  const ObsTile tl = obs_tile(a, NCH_ALL);
  if (!tl.live) return;  // padding of the grid
  const int h = tl.h, kb = tl.kb, NCH = NBUF == 1 && tl.nch > 1 ? 1 : tl.nch;  // the host picks NBUF
  auto buf = [](int c) { return NBUF == 1 ? 0 : (c & 1); };
  const int kw0 = kb * kBlockKeys + wave * 16 * kKT;  // keys are below 2^31
  // every window row sees keys <= n - W: no masks for a wave below that
  const bool all_vis = kw0 + 16 * kKT - 1 <= n - a.n_obs;
  const int rot = NCH > 0 ? kb % NCH : 0;  // staggered chunk order, as in pass 1
  auto cid = [&](int c) { return tl.c0 + (c + rot < NCH ? c + rot : c + rot - NCH); };
  // where this workgroup's key sums go: the score itself, or its row group's
  // partial row
  float* dst = a.row_groups == 1 ? a.score + (int64_t)h * a.score_stride
                                 : a.part_score + ((int64_t)tl.g * a.n_kv_heads + h) * a.n;
  if (NCH == 0) {  // a row group past the last chunk: zero partial sums
    if (tid < 16 * kKT * kWaves) {
      const int key = kb * kBlockKeys + tid;
      if (key < n) dst[key] = 0.0f;
    }
    return;
  }
  auto load_l2 = [&](int c) -> float {
    int row = c * kL2 + tid;
    row = row < R ? row : R - 1;
    return tid < kL2 ? a.row_lse2[(int64_t)h * R + row] : 0.0f;
  };

  bf16x8_t kf[kKT][D / 32];
  load_k_tiles<D>(a, h, kw0, q4, i16, kf);
  {
    uint4 v[QG::kPPT];
    load_q_chunk<D>(a, h, cid(0), tid, v);
    const float l = load_l2(cid(0));
    store_q_chunk<D>(qc[0], tid, v);
    if (tid < kL2) l2c[0][tid] = l;
  }
  wait_vm<0>();  // K and the first chunk have landed (see pass 1)

  float acc[kKT][4];
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[kt][r] = 0.0f;

  for (int c = 0; c < NCH; ++c) {
    uint4 nxt[QG::kPPT];
    float l2n = 0.0f;
    if (NBUF > 1 && c + 1 < NCH) {
      load_q_chunk<D>(a, h, cid(c + 1), tid, nxt);
      l2n = load_l2(cid(c + 1));
    }
    lds_barrier();  // chunk c is in LDS
    const char* qchunk = qc[buf(c)];
    const float* l2s = l2c[buf(c)];
    const int ci = cid(c);
    const int nt = RT - ci * kChunk < kChunk ? RT - ci * kChunk : kChunk;
    const float c2 = a.scale_log2;
#pragma unroll
    for (int tt = 0; tt < kChunk; ++tt) {
      if (tt >= nt) break;  // uniform
      bf16x8_t qb[D / 32];
      read_q_tile<D>(qchunk, tt, q4, i16, qb);
      const float cur_l2 = l2s[tt * 16 + i16];
      floatx4_t s[kKT];
      s_tiles<D>(kf, qb, s);
      const int row = (ci * kChunk + tt) * 16 + i16;
      if (row >= R) continue;
      if (all_vis) {
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[kt][r] += fast_exp2(fmaf(s[kt][r], c2, -cur_l2));
        }
      } else {
        const int last = (int)row_info(a, h, row, D).last;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kw0 + kt * 16 + q4 * 4 + r;
            const bool vis = key < n && key <= last;
            acc[kt][r] += vis ? fast_exp2(fmaf(s[kt][r], c2, -cur_l2)) : 0.0f;
          }
        }
      }
    }
    // the buffers of chunk c + 1 were last read in iteration c - 1
    if (NBUF > 1 && c + 1 < NCH) {
      store_q_chunk<D>(qc[buf(c + 1)], tid, nxt);
      if (tid < kL2) l2c[buf(c + 1)][tid] = l2n;
    }
  }
  if (kw0 >= n) return;
  const float inv_w = 1.0f / (float)a.n_obs;
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float tot = group_sum<16>(acc[kt][r]);
      const int key = kw0 + kt * 16 + q4 * 4 + r;
      if (i16 == 0 && key < n) dst[key] = tot * inv_w;
    }
  }
}

// score = the row groups' partial key sums, added in group order.
__global__ __launch_bounds__(kThreads) void obs_reduce_kernel(const ScoreObsArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // (head, key)
  if (e >= (int64_t)a.n_kv_heads * a.n) return;
  const int h = (int)(e / a.n);
  const int64_t key = e - (int64_t)h * a.n;
  const int64_t plane = (int64_t)a.n_kv_heads * a.n;
  float t = a.part_score[e];
  for (int g = 1; g < a.row_groups; ++g) t += a.part_score[g * plane + e];
  a.score[(int64_t)h * a.score_stride + key] = t;
}

template <int D>
hipError_t launch_d(const ScoreObsArgs& a, hipStream_t s) {
  const int64_t tiles = (int64_t)a.n_kv_heads * a.n_kblocks;
  const dim3 grid((unsigned)((tiles + kXcds - 1) / kXcds * kXcds * a.row_groups));
  const int R = a.n_obs * a.group;
  const int nch_all = ((R + 15) / 16 + kChunk - 1) / kChunk;
  const bool one = (nch_all + a.row_groups - 1) / a.row_groups <= 1;  // chunks per row group
  if (one)
    hipLaunchKernelGGL((obs_pass1_kernel<D, 1>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((obs_pass1_kernel<D, 2>), grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rblocks = (R + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(obs_lse_kernel, dim3((unsigned)(a.n_kv_heads * rblocks)), dim3(kThreads), 0, s, a,
                     rblocks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (one)
    hipLaunchKernelGGL((obs_pass2_kernel<D, 1>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((obs_pass2_kernel<D, 2>), grid, dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.row_groups == 1) return e;
  const int64_t total = (int64_t)a.n_kv_heads * a.n;
  hipLaunchKernelGGL(obs_reduce_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

int score_obs_block_keys() { return kBlockKeys; }
int score_obs_chunk_rows() { return kChunk * 16; }

hipError_t launch_score_obs(int d, const ScoreObsArgs& a, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, s);
  if (d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
