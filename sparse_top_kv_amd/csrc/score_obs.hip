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

namespace skv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 256;
constexpr int kBlockKeys = 64 * kWaves;  // keys per workgroup

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
                                             bf16x8_t (&kf)[4][D / 32]) {
  const char* kb = a.k + (int64_t)h * a.head_stride_b;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    int64_t key = kw0 + kt * 16 + i16;
    key = key < a.n ? key : a.n - 1;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      kf[kt][ks] = as_bf16x8(ld16(kb + key * a.pos_stride_b + (ks * 32 + q4 * 8) * 2));
  }
}

template <int D>
__device__ __forceinline__ void load_q_tile(const ScoreObsArgs& a, const RowInfo& ri, int q4,
                                            bf16x8_t (&qb)[D / 32]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (ri.ok) u = ld16(a.q + ri.qoff + ks * 32 + q4 * 8);
    qb[ks] = as_bf16x8(u);
  }
}

template <int D>
__device__ __forceinline__ void s_tiles(const bf16x8_t (&kf)[4][D / 32], const bf16x8_t (&qb)[D / 32],
                                        floatx4_t (&s)[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) acc = mfma_bf16(kf[kt][ks], qb[ks], acc);
    s[kt] = acc;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void obs_pass1_kernel(const ScoreObsArgs a) {
  __shared__ float sm_ml[2][kWaves][16][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int h = blockIdx.x / a.n_kblocks;
  const int kb = blockIdx.x - h * a.n_kblocks;
  const int64_t kw0 = (int64_t)kb * kBlockKeys + wave * 64;
  const int R = a.n_obs * a.group;
  const int RT = (R + 15) / 16;

  bf16x8_t kf[4][D / 32];
  load_k_tiles<D>(a, h, kw0, q4, i16, kf);
  bf16x8_t qb[D / 32];
  RowInfo ri = row_info(a, h, i16, D);
  load_q_tile<D>(a, ri, q4, qb);

  for (int rt = 0; rt < RT; ++rt) {
    floatx4_t s[4];
    s_tiles<D>(kf, qb, s);
    const RowInfo cur = ri;
    if (rt + 1 < RT) {  // next row tile's queries in flight during the softmax work
      ri = row_info(a, h, (rt + 1) * 16 + i16, D);
      load_q_tile<D>(a, ri, q4, qb);
    }
    float mw = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = kw0 + kt * 16 + q4 * 4 + r;
        const float x = (key < a.n && key <= cur.last) ? s[kt][r] * a.scale_log2 : kNegInf;
        s[kt][r] = x;
        mw = fmaxf(mw, x);
      }
    }
    mw = fmaxf(mw, __shfl_xor(mw, 16, 64));
    mw = fmaxf(mw, __shfl_xor(mw, 32, 64));
    const float mu = mw == kNegInf ? 0.0f : mw;
    float lw = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) lw += fast_exp2(s[kt][r] - mu);
    }
    lw += __shfl_xor(lw, 16, 64);
    lw += __shfl_xor(lw, 32, 64);
    const int buf = rt & 1;
    if (q4 == 0) {
      sm_ml[buf][wave][i16][0] = mw;
      sm_ml[buf][wave][i16][1] = lw;
    }
    __syncthreads();
    if (tid < 16) {
      const int row = rt * 16 + tid;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[buf][w][tid][0]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw2 = sm_ml[buf][w][tid][0];
        L += mw2 == kNegInf ? 0.0f : sm_ml[buf][w][tid][1] * fast_exp2(mw2 - M);
      }
      if (row < R) {
        float* ml = a.part_ml + (((int64_t)h * a.n_kblocks + kb) * R + row) * 2;
        ml[0] = M;
        ml[1] = L;
      }
    }
  }
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

template <int D>
__global__ __launch_bounds__(kThreads) void obs_pass2_kernel(const ScoreObsArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int h = blockIdx.x / a.n_kblocks;
  const int kb = blockIdx.x - h * a.n_kblocks;
  const int64_t kw0 = (int64_t)kb * kBlockKeys + wave * 64;
  if (kw0 >= a.n) return;
  const int R = a.n_obs * a.group;
  const int RT = (R + 15) / 16;
  const float* lse2 = a.row_lse2 + (int64_t)h * R;

  bf16x8_t kf[4][D / 32];
  load_k_tiles<D>(a, h, kw0, q4, i16, kf);
  bf16x8_t qb[D / 32];
  RowInfo ri = row_info(a, h, i16, D);
  load_q_tile<D>(a, ri, q4, qb);
  float l2 = ri.ok ? lse2[i16] : 0.0f;

  float acc[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[kt][r] = 0.0f;

  for (int rt = 0; rt < RT; ++rt) {
    floatx4_t s[4];
    s_tiles<D>(kf, qb, s);
    const RowInfo cur = ri;
    const float cur_l2 = l2;
    if (rt + 1 < RT) {
      const int row = (rt + 1) * 16 + i16;
      ri = row_info(a, h, row, D);
      load_q_tile<D>(a, ri, q4, qb);
      l2 = ri.ok ? lse2[row] : 0.0f;
    }
    if (!cur.ok) continue;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = kw0 + kt * 16 + q4 * 4 + r;
        const bool vis = key < a.n && key <= cur.last;
        acc[kt][r] += vis ? fast_exp2(s[kt][r] * a.scale_log2 - cur_l2) : 0.0f;
      }
    }
  }
  const float inv_w = 1.0f / (float)a.n_obs;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float tot = group_sum<16>(acc[kt][r]);
      const int64_t key = kw0 + kt * 16 + q4 * 4 + r;
      if (i16 == 0 && key < a.n) a.score[(int64_t)h * a.score_stride + key] = tot * inv_w;
    }
  }
}

template <int D>
hipError_t launch_d(const ScoreObsArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_kv_heads * a.n_kblocks));
  hipLaunchKernelGGL(obs_pass1_kernel<D>, grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int R = a.n_obs * a.group;
  const int rblocks = (R + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(obs_lse_kernel, dim3((unsigned)(a.n_kv_heads * rblocks)), dim3(kThreads), 0, s, a,
                     rblocks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(obs_pass2_kernel<D>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int score_obs_block_keys() { return kBlockKeys; }

hipError_t launch_score_obs(int d, const ScoreObsArgs& a, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, s);
  if (d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
