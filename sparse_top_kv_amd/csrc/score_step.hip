// score_step.hip -- per-step score of one decode query (window of one).
//
// Method: the score of key j for kv head h is the attention probability of
// j summed over the query heads of h's group ("Sparse-to-Dense ..." Sec. 3.2:
// attention scores of a GQA group are summed; top-K attention picks keys by
// attention score):
//   s_h(j) = sum_{g in group(h)} exp(l_g(j) - lse_g),  l = scale q.k.
// A softmax row needs its normaliser before any probability, so the K stream
// runs once and stores log2-domain logits plus per-chunk (max, sum) of every
// query head (phase 1, same lane layout as the attention kernel, no V); phase
// 2 merges the chunk statistics into lse_g and writes the group sums.
#include "skv_common.h"
#include "skv_kernels.h"
#include "skv_tile.h"

namespace skv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerIter = 4;
constexpr float kRescaleSlack = 8.0f;
constexpr int kFinalizeKeys = 2048;  // keys per phase-2 workgroup

template <int DT, int D, int G>
__global__ __launch_bounds__(kThreads) void score_logits_kernel(const ScoreStepArgs a) {
  using RG = RowGeom<DT, D>;
  constexpr int LPR = RG::kLanesPerRow;
  constexpr int RPL = RG::kRowsPerLoad;
  constexpr int U = kLoadsPerIter;
  constexpr int RI = U * RPL;
  static_assert(G <= LPR, "one writer lane per query head");

  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cph = a.chunks_per_head;
  const int h = blockIdx.x % a.n_kv_heads;  // a kv head's chunks on one XCD
  const int c = blockIdx.x / a.n_kv_heads;
  const int64_t r0 = (int64_t)c * a.chunk;
  const int64_t rem = a.n - r0;
  const int rows = (int)(rem < 0 ? 0 : (rem > a.chunk ? a.chunk : rem));
  const int part = lane % LPR, rgrp = lane / LPR;

  uint32_t qr[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 t = ld16(reinterpret_cast<const char*>(a.q) +
                         ((int64_t)(h * G + g) * D) * RG::kElem + part * 16);
    qr[g][0] = t.x; qr[g][1] = t.y; qr[g][2] = t.z; qr[g][3] = t.w;
  }
  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = kNegInf; l[g] = 0.0f; }

  const char* kb = a.k + (int64_t)h * a.head_stride_b + part * 16;
  float* lg_out = a.logits + (int64_t)(h * G + (part < G ? part : 0)) * a.logits_stride + r0;
  const int nit_total = (rows + RI - 1) / RI;
  const int per = (nit_total + kWaves - 1) / kWaves;
  const int it0 = wave * per;
  const int it1 = (it0 + per < nit_total) ? it0 + per : nit_total;

  auto issue = [&](int it, uint4 (&kr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = it * RI + u * RPL + rgrp;
      const int rr = r < rows ? r : rows - 1;
      kr[u] = ld16(kb + (r0 + rr) * a.pos_stride_b);
    }
  };
  auto compute = [&](int it, const uint4 (&kr)[U]) {
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = it * RI + u * RPL + rgrp;
      const bool valid = r < rows;
      float mine = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float x = group_sum<LPR>(slice_dot<DT>(qr[g], kr[u])) * a.scale_log2;
        s[u][g] = valid ? x : kNegInf;
        mine = part == g ? x : mine;
      }
      if (valid && part < G) lg_out[r] = mine;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u][g]);
      if (mb > m[g] + kRescaleSlack) {
        l[g] *= fast_exp2(m[g] - mb);
        m[g] = mb;
      }
      const float mu = (m[g] == kNegInf) ? 0.0f : m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) l[g] += fast_exp2(s[u][g] - mu);
    }
  };

  if (it0 < it1) {
    uint4 ka[U], kc[U];
    issue(it0, ka);
    for (int it = it0; it < it1; it += 2) {
      if (it + 1 < it1) issue(it + 1, kc);
      compute(it, ka);
      if (it + 1 >= it1) break;
      if (it + 2 < it1) issue(it + 2, ka);
      compute(it + 1, kc);
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = m[g];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float x = (m[g] == kNegInf) ? 0.0f : l[g] * fast_exp2(m[g] - M);
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    if (lane == 0) { sm_m[wave][g] = M; sm_l[wave][g] = x; }
  }
  __syncthreads();
  if (tid < G) {
    const int g = tid;
    float M = sm_m[0][g];
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.0f;
    for (int w = 0; w < kWaves; ++w)
      L += (sm_m[w][g] == kNegInf) ? 0.0f : sm_l[w][g] * fast_exp2(sm_m[w][g] - M);
    float* ml = a.part_ml + (((int64_t)h * cph + c) * G + g) * 2;
    ml[0] = M;
    ml[1] = L;
  }
}

// Phase 2: lse of each query head from the chunk statistics, then the group
// sum of probabilities for kFinalizeKeys keys.
template <int G>
__global__ __launch_bounds__(kThreads) void score_finalize_kernel(const ScoreStepArgs a, int nblk) {
  static_assert(kFinalizeKeys == kThreads * 8, "eight keys per thread");
  __shared__ float sm_lse2[G];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x % a.n_kv_heads;  // on the XCD that ran the head's chunks
  const int b = blockIdx.x / a.n_kv_heads;
  const int cph = a.chunks_per_head;
  const int64_t nchunks = (a.n + a.chunk - 1) / a.chunk;
  // this thread's eight keys of every head of the group, loaded first (the
  // logits rows are padded to a multiple of four keys)
  const int64_t jb = (int64_t)b * kFinalizeKeys + (int64_t)tid * 8;
  float4 lg[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* row = a.logits + (int64_t)(h * G + g) * a.logits_stride;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      lg[g][u] = jb + 4 * u < a.logits_stride ? *reinterpret_cast<const float4*>(row + jb + 4 * u)
                                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  const float* ml = a.part_ml + (int64_t)h * cph * G * 2;
  for (int g = wave; g < G; g += kWaves) {
    // the first 64 chunks' statistics in one round of loads, any others after
    const float2 st0 = lane < nchunks ? *reinterpret_cast<const float2*>(ml + ((int64_t)lane * G + g) * 2)
                                      : make_float2(kNegInf, 0.0f);
    float M = st0.x;
    for (int64_t cc = lane + 64; cc < nchunks; cc += 64) M = fmaxf(M, ml[(cc * G + g) * 2]);
    M = wave_max(M);
    float L = (st0.x == kNegInf) ? 0.0f : st0.y * fast_exp2(st0.x - M);
    for (int64_t cc = lane + 64; cc < nchunks; cc += 64) {
      const float mc = ml[(cc * G + g) * 2];
      L += (mc == kNegInf) ? 0.0f : ml[(cc * G + g) * 2 + 1] * fast_exp2(mc - M);
    }
    L = wave_sum(L);
    if (lane == 0) sm_lse2[g] = M + __log2f(L);
  }
  __syncthreads();
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l2 = sm_lse2[g];
    const float v[8] = {lg[g][0].x, lg[g][0].y, lg[g][0].z, lg[g][0].w,
                        lg[g][1].x, lg[g][1].y, lg[g][1].z, lg[g][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += fast_exp2(v[e] - l2);
  }
  float* out = a.score + (int64_t)h * a.score_stride;
  if (jb + 8 <= a.n && (reinterpret_cast<uintptr_t>(out + jb) & 15) == 0) {
    *reinterpret_cast<float4*>(out + jb) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4*>(out + jb + 4) = make_float4(s[4], s[5], s[6], s[7]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (jb + e < a.n) out[jb + e] = s[e];
  }
}

// bf16 caches: phase 1 on the matrix cores.  K streams through a per-wave
// ring of 16-key LDS tiles (direct-to-LDS copies, as in the attention kernel);
// q.K^T is one 16x16x32 MFMA per 32 channels with the G query heads padded to
// 16.  Lane (q4, li) holds the logits of keys 4 q4 .. 4 q4 + 3 for head li: it
// keeps a running (max, sum) of its head and puts them into the workgroup's
// LDS copy of its chunk's logits, which goes to memory in one coalesced pass
// after the last tile (interleaving the logit writes with the K stream cost
// about 7 us of the 55 at 128K).  Chunks hold at most kLgFloats / G keys.
constexpr int kLgFloats = 16384;  // logits of one chunk, all heads of the group (64 KB)

template <int D, int W, int S>
__global__ __launch_bounds__(64 * W) void score_mfma_kernel(const ScoreStepArgs a, int G) {
  using TG = TileGeom<D>;
  constexpr int NI = TG::kNI, TB = TG::kTB, PPR = TG::kPPR, KS = TG::kKS;
  __shared__ __attribute__((aligned(1024))) char st0[W][TB];
  __shared__ __attribute__((aligned(1024))) char st1[W][TB];
  __shared__ __attribute__((aligned(1024))) char st2[W][TB];
  __shared__ __attribute__((aligned(1024))) char st3[W][TB];
  __shared__ float sm_m[W][16], sm_l[W][16];
  // chunk logits, head-major; each head's row padded by 4 floats so the heads
  // of one store sit in different banks
  __shared__ __attribute__((aligned(16))) float sm_lg[kLgFloats + 4 * 16];
  static_assert(S >= 2 && S <= 4, "ring of two to four stages");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, li = lane & 15;
  const int cph = a.chunks_per_head;
  const int h = blockIdx.x % a.n_kv_heads;  // a kv head's chunks on one XCD
  const int c = blockIdx.x / a.n_kv_heads;
  const int64_t r0 = (int64_t)c * a.chunk;
  const int64_t rem = a.n - r0;
  const int rows = (int)(rem < 0 ? 0 : (rem > a.chunk ? a.chunk : rem));
  const uint32_t stride = (uint32_t)a.pos_stride_b;

  bf16x8_t qb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (li < G)
      v = ld16(reinterpret_cast<const char*>(a.q) + ((int64_t)(h * G + li) * D + 32 * s + 8 * q4) * 2);
    qb[s] = as_bf16x8(v);
  }
  const uint32_t span = (uint32_t)(a.n * a.pos_stride_b);
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
  const int nst = wave < nsteps ? (nsteps - 1 - wave) / W + 1 : 0;
  const float c2 = a.scale_log2;
  const int lg_stride = a.chunk + 4;  // floats per head row in sm_lg
  float* lg_row = sm_lg + (li < G ? li : 0) * lg_stride;

  auto issue = [&](char (*stg)[TB], int k) {
    const int j = wave + W * k;
    char* dst = &stg[wave][0];
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(r0 + (int64_t)j * kStep) * stride);
#pragma unroll
    for (int u = 0; u < NI; ++u) copy_to_lds(rk, dst + u * 1024, pk[u], soff);
  };
  auto ring = [&](int u) -> char (*)[TB] {
    if (S > 3 && u == 3) return st3;
    if (S > 2 && u == 2) return st2;
    return u == 1 ? st1 : st0;
  };
  auto newer_than = [&](int k) { return (nst - 1 - k) < (S - 1) ? (nst - 1 - k) : (S - 1); };

  float m = kNegInf, l = 0.0f;  // running max and sum of head li over this lane's keys
  auto step = [&](char (*cur)[TB], char (*nxt)[TB], int k) {
    if (k + S - 1 < nst) {
      wait_lgkm0();
      issue(nxt, k + S - 1);
    }
    wait_newer<S - 1, NI>(newer_than(k));
    const char* base = &cur[0][0];
    floatx4_t cs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      cs = mfma_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(base + koff[s])), qb[s], cs);
    const int j = wave + W * k;
    const int rb = j * kStep + 4 * q4;  // chunk row of key r = 0
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = cs[r] * c2;
    const bool full = (j + 1) * kStep <= rows;  // wave-uniform
    if (full) {
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
#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (u < nst) issue(ring(u), u);
  for (int k = 0; k < nst;) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      if (k < nst) step(ring(u), ring((u + S - 1) % S), k);
      ++k;
    }
  }

  // (max, sum) of head li: the four q4 lanes, then the waves
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
  // the chunk's logits to memory: rows of G heads, 16 bytes per thread and step
  // (the logits rows are padded to a multiple of four keys, so a chunk's last
  // four-key group is always in bounds)
  {
    const int q_per_head = (rows + 3) / 4;
    for (int e = tid; e < G * q_per_head; e += 64 * W) {
      const int g = e / q_per_head, r = 4 * (e - g * q_per_head);
      const float4 v = *reinterpret_cast<const float4*>(sm_lg + g * lg_stride + r);
      *reinterpret_cast<float4*>(a.logits + (int64_t)(h * G + g) * a.logits_stride + r0 + r) = v;
    }
  }
  if (tid < G) {
    const int g = tid;
    float Mw = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < W; ++w) Mw = fmaxf(Mw, sm_m[w][g]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w)
      L += (sm_m[w][g] == kNegInf) ? 0.0f : sm_l[w][g] * fast_exp2(sm_m[w][g] - Mw);
    float* ml = a.part_ml + (((int64_t)h * cph + c) * G + g) * 2;
    ml[0] = Mw;
    ml[1] = L;
  }
}

template <int G>
hipError_t launch_finalize(const ScoreStepArgs& a, hipStream_t s) {
  const int nblk = (int)((a.n + kFinalizeKeys - 1) / kFinalizeKeys);
  hipLaunchKernelGGL((score_finalize_kernel<G>), dim3((unsigned)(a.n_kv_heads * nblk)), dim3(kThreads),
                     0, s, a, nblk);
  return hipGetLastError();
}

hipError_t launch_finalize_g(int g, const ScoreStepArgs& a, hipStream_t s) {
  switch (g) {
    case 1: return launch_finalize<1>(a, s);
    case 2: return launch_finalize<2>(a, s);
    case 3: return launch_finalize<3>(a, s);
    case 4: return launch_finalize<4>(a, s);
    case 5: return launch_finalize<5>(a, s);
    case 6: return launch_finalize<6>(a, s);
    case 7: return launch_finalize<7>(a, s);
    case 8: return launch_finalize<8>(a, s);
    case 16: return launch_finalize<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

constexpr int kScoreWaves = 8;
constexpr int kScoreStages = 2;

template <int D>
hipError_t launch_mfma(int g, const ScoreStepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((score_mfma_kernel<D, kScoreWaves, kScoreStages>),
                     dim3((unsigned)(a.n_kv_heads * a.chunks_per_head)), dim3(64 * kScoreWaves), 0, s,
                     a, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_finalize_g(g, a, s);
}

template <int DT, int D, int G>
hipError_t launch_g(const ScoreStepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((score_logits_kernel<DT, D, G>), dim3((unsigned)(a.n_kv_heads * a.chunks_per_head)),
                     dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = (int)((a.n + kFinalizeKeys - 1) / kFinalizeKeys);
  hipLaunchKernelGGL((score_finalize_kernel<G>), dim3((unsigned)(a.n_kv_heads * nblk)), dim3(kThreads),
                     0, s, a, nblk);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_d(int g, const ScoreStepArgs& a, hipStream_t s) {
  switch (g) {
    case 1: return launch_g<DT, D, 1>(a, s);
    case 2: return launch_g<DT, D, 2>(a, s);
    case 3: return launch_g<DT, D, 3>(a, s);
    case 4: return launch_g<DT, D, 4>(a, s);
    case 5: return launch_g<DT, D, 5>(a, s);
    case 6: return launch_g<DT, D, 6>(a, s);
    case 7: return launch_g<DT, D, 7>(a, s);
    case 8: return launch_g<DT, D, 8>(a, s);
    case 16: return launch_g<DT, D, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int score_step_mfma_granule() { return kScoreWaves * kStep; }
int score_step_mfma_max_chunk(int g) {
  const int gr = score_step_mfma_granule();
  return g < 1 ? gr : (kLgFloats / g) / gr * gr;
}

hipError_t launch_score_step(int dtype, int d, int g, const ScoreStepArgs& a, hipStream_t s) {
  if (dtype == 1 && d == 128) return launch_mfma<128>(g, a, s);
  if (dtype == 1 && d == 64) return launch_mfma<64>(g, a, s);
  if (dtype == 0 && d == 128) return launch_d<0, 128>(g, a, s);
  if (dtype == 0 && d == 64) return launch_d<0, 64>(g, a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
