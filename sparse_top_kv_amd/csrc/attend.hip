// attend.hip -- split-K decode attention over a dense or index-gathered row
// list, with the log-sum-exp merge of the per-chunk partials done in-kernel by
// the last workgroup of each kv head.
//
// Method: exact softmax attention restricted to a key set (top-K attention,
// "Sparse-to-Dense ..." Sec. 3.2; the kept set plus the recent tail read by a
// split-K decoding kernel, "Where Activation Sparsity and KV-Cache Sparsity
// Cross ..." sections "Speedup Across Context" and "The Attention Baseline").
//
// Layout on gfx950 (64-lane waves): one K or V row is split into 16-byte lane
// slices, so a wave load moves 1 KB = RowsPerLoad consecutive rows; the G
// query heads of the kv head ride along, so every K/V byte is read once for
// the whole group.  Logits use packed bf16 dot products (v_dot2c_f32_bf16) and
// a DPP reduction over the lanes of a row; softmax runs in the log2 domain in
// fp32 with a lazily refreshed running max.  Each workgroup owns `chunk` rows
// of one kv head, folds its 4 waves into one (max, sum, acc[d]) partial per
// query head, and the last workgroup of the head (completion counter with
// device-scope fences) merges all partials:
//   M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  out = sum_c acc_c 2^(m_c - M) / L,
//   lse = (M + log2 L) ln 2.
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerIter = 4;
constexpr int kMaxChunk = 2048;        // rows per workgroup (LDS position list)
constexpr int kMaxMergeSlots = 2048;   // chunks_per_head * G
constexpr float kRescaleSlack = 8.0f;  // running max may trail the true max by this (log2)

template <int DT, int D, int G, bool SPARSE>
__global__ __launch_bounds__(kThreads) void attend_kernel(const AttendArgs a) {
  using RG = RowGeom<DT, D>;
  constexpr int LPR = RG::kLanesPerRow;
  constexpr int EPL = RG::kElemsPerLane;
  constexpr int RPL = RG::kRowsPerLoad;
  constexpr int U = kLoadsPerIter;
  constexpr int RI = U * RPL;

  __shared__ int32_t sm_pos[kMaxChunk];  // row positions; reused as merge weights
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float4 sm_red[kThreads];
  __shared__ int sm_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cph = a.chunks_per_head;
  const int h = blockIdx.x / cph;
  const int c = blockIdx.x - h * cph;

  int32_t cnt = 0;
  int64_t rows_h;
  if constexpr (SPARSE) {
    cnt = a.count[h];
    cnt = cnt < 0 ? 0 : (cnt > (int32_t)a.count_max ? (int32_t)a.count_max : cnt);
    rows_h = (int64_t)cnt + (a.n - a.tail_start);
  } else {
    rows_h = a.n;
  }
  int nch = (int)((rows_h + a.chunk - 1) / a.chunk);
  nch = nch < 1 ? 1 : (nch > cph ? cph : nch);
  if (c >= nch) return;
  const int64_t r0 = (int64_t)c * a.chunk;
  int64_t rem = rows_h - r0;
  const int rows = (int)(rem < 0 ? 0 : (rem > a.chunk ? a.chunk : rem));

  if constexpr (SPARSE) {
    const int32_t* ih = a.idx + (int64_t)h * a.idx_stride;
    const int32_t last = (int32_t)(a.n - 1);
    for (int i = tid; i < rows; i += kThreads) {
      const int64_t r = r0 + i;
      int32_t p = r < cnt ? ih[r] : (int32_t)(a.tail_start + (r - cnt));
      p = p < 0 ? 0 : (p > last ? last : p);  // keep out-of-contract indices in bounds
      sm_pos[i] = p;
    }
    __syncthreads();
  }

  // this lane's slice of each query head of the group
  const int part = lane % LPR;
  const int rgrp = lane / LPR;
  uint32_t qr[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 t = ld16(reinterpret_cast<const char*>(a.q) +
                         ((int64_t)(h * G + g) * D) * RG::kElem + part * 16);
    qr[g][0] = t.x; qr[g][1] = t.y; qr[g][2] = t.z; qr[g][3] = t.w;
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
  }

  const char* kb = a.k + (int64_t)h * a.head_stride_b + part * 16;
  const char* vb = a.v + (int64_t)h * a.head_stride_b + part * 16;
  const int nit_total = (rows + RI - 1) / RI;
  const int per = (nit_total + kWaves - 1) / kWaves;
  const int it0 = wave * per;
  const int it1 = (it0 + per < nit_total) ? it0 + per : nit_total;

  auto issue = [&](int it, uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = it * RI + u * RPL + rgrp;
      const int rr = r < rows ? r : rows - 1;
      int64_t pos;
      if constexpr (SPARSE) pos = sm_pos[rr];
      else pos = r0 + rr;
      kr[u] = ld16(kb + pos * a.pos_stride_b);
      vr[u] = ld16(vb + pos * a.pos_stride_b);
    }
  };

  auto compute = [&](int it, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = it * RI + u * RPL + rgrp < rows;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float dsum = group_sum<LPR>(slice_dot<DT>(qr[g], kr[u]));
        s[u][g] = valid ? dsum * a.scale_log2 : kNegInf;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u][g]);
      if (mb > m[g] + kRescaleSlack) {
        const float alpha = fast_exp2(m[g] - mb);
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        m[g] = mb;
      }
    }
    float vf[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) slice_to_f32<DT>(vr[u], vf[u]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mu = (m[g] == kNegInf) ? 0.0f : m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(s[u][g] - mu);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[u][e], acc[g][e]);
      }
    }
  };

  if (it0 < it1) {
    uint4 ka[U], va[U], kc[U], vc[U];
    issue(it0, ka, va);
    for (int it = it0; it < it1; it += 2) {
      if (it + 1 < it1) issue(it + 1, kc, vc);
      compute(it, ka, va);
      if (it + 1 >= it1) break;
      if (it + 2 < it1) issue(it + 2, ka, va);
      compute(it + 1, kc, vc);
    }
  }

  // fold the RPL row groups of this wave
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = m[g];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float sc = (m[g] == kNegInf) ? 0.0f : fast_exp2(m[g] - M);
    float lg = l[g] * sc;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) lg += __shfl_xor(lg, off, 64);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[g][e] * sc;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      acc[g][e] = x;
    }
    if (rgrp == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][g][part * EPL + e] = acc[g][e];
      if (part == 0) {
        sm_m[wave][g] = M;
        sm_l[wave][g] = lg;
      }
    }
  }
  __syncthreads();

  // fold the waves into this chunk's partial
  const int64_t slot = (int64_t)h * cph + c;
  for (int o = tid; o < G * D; o += kThreads) {
    const int g = o / D, dd = o - g * D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = (sm_m[w][g] == kNegInf) ? 0.0f : fast_exp2(sm_m[w][g] - M);
      L += sm_l[w][g] * sc;
      A += sm_acc[w][g][dd] * sc;
    }
    a.part_acc[(slot * G + g) * D + dd] = A;
    if (dd == 0) {
      a.part_ml[(slot * G + g) * 2 + 0] = M;
      a.part_ml[(slot * G + g) * 2 + 1] = L;
    }
  }

  // completion count; the last workgroup of this kv head merges
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned t = atomicAdd(&a.counters[h], 1u);
    sm_last = (t == (unsigned)(nch - 1));
  }
  __syncthreads();
  if (!sm_last) return;
  __threadfence();
  if (tid == 0) a.counters[h] = 0u;

  float* sm_w = reinterpret_cast<float*>(sm_pos);
  const float* ml = a.part_ml + (int64_t)h * cph * G * 2;
  for (int g = wave; g < G; g += kWaves) {
    float M = kNegInf;
    for (int cc = lane; cc < nch; cc += 64) M = fmaxf(M, ml[(cc * G + g) * 2]);
    M = wave_max(M);
    float L = 0.0f;
    for (int cc = lane; cc < nch; cc += 64) {
      const float mc = ml[(cc * G + g) * 2];
      L += (mc == kNegInf) ? 0.0f : ml[(cc * G + g) * 2 + 1] * fast_exp2(mc - M);
    }
    L = wave_sum(L);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int cc = lane; cc < nch; cc += 64) {
      const float mc = ml[(cc * G + g) * 2];
      sm_w[cc * G + g] = (mc == kNegInf) ? 0.0f : fast_exp2(mc - M) * inv;
    }
    if (lane == 0 && a.lse) a.lse[h * G + g] = L > 0.0f ? (M + log2f(L)) * kLn2 : kNegInf;
  }
  __syncthreads();

  constexpr int NO4 = G * D / 4;  // float4 outputs of this kv head
  const float* pa = a.part_acc + (int64_t)h * cph * G * D;
  auto accumulate = [&](int o4, int first, int step) {
    const int g = (o4 * 4) / D, d0 = o4 * 4 - g * D;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int cc = first; cc < nch; cc += step) {
      const float w = sm_w[cc * G + g];
      const float4 x = *reinterpret_cast<const float4*>(pa + ((int64_t)cc * G + g) * D + d0);
      A.x = fmaf(w, x.x, A.x); A.y = fmaf(w, x.y, A.y);
      A.z = fmaf(w, x.z, A.z); A.w = fmaf(w, x.w, A.w);
    }
    return A;
  };
  if constexpr (NO4 >= kThreads) {
    for (int o4 = tid; o4 < NO4; o4 += kThreads) {
      const int g = (o4 * 4) / D, d0 = o4 * 4 - g * D;
      *reinterpret_cast<float4*>(a.out + ((int64_t)h * G + g) * D + d0) = accumulate(o4, 0, 1);
    }
  } else {
    constexpr int NS = kThreads / NO4;  // chunk-parallel splits per output
    const int sp = tid / NO4, o4 = tid - sp * NO4;
    if (sp < NS) sm_red[sp * NO4 + o4] = accumulate(o4, sp, NS);
    __syncthreads();
    if (tid < NO4) {
      float4 A = sm_red[tid];
      for (int k = 1; k < NS; ++k) {
        const float4 x = sm_red[k * NO4 + tid];
        A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
      }
      const int g = (tid * 4) / D, d0 = tid * 4 - g * D;
      *reinterpret_cast<float4*>(a.out + ((int64_t)h * G + g) * D + d0) = A;
    }
  }
}

template <int DT, int D, int G>
hipError_t launch3(bool sparse, const AttendArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_kv_heads * a.chunks_per_head));
  if (sparse)
    hipLaunchKernelGGL((attend_kernel<DT, D, G, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attend_kernel<DT, D, G, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch2(int g, bool sparse, const AttendArgs& a, hipStream_t s) {
  switch (g) {
    case 1: return launch3<DT, D, 1>(sparse, a, s);
    case 2: return launch3<DT, D, 2>(sparse, a, s);
    case 4: return launch3<DT, D, 4>(sparse, a, s);
    case 7: return launch3<DT, D, 7>(sparse, a, s);
    case 8: return launch3<DT, D, 8>(sparse, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int attend_rows_per_iter(int dtype, int d) {
  const int elem = dtype == 1 ? 2 : 4;
  const int lpr = d * elem / 16;
  return kLoadsPerIter * (64 / lpr);
}

int attend_max_chunk() { return kMaxChunk; }
int attend_max_merge_slots() { return kMaxMergeSlots; }

hipError_t launch_attend(int dtype, int d, int g, bool sparse, const AttendArgs& a,
                         hipStream_t s) {
  if (dtype == 1 && d == 128) return launch2<1, 128>(g, sparse, a, s);
  if (dtype == 1 && d == 64) return launch2<1, 64>(g, sparse, a, s);
  if (dtype == 0 && d == 128) return launch2<0, 128>(g, sparse, a, s);
  if (dtype == 0 && d == 64) return launch2<0, 64>(g, sparse, a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
