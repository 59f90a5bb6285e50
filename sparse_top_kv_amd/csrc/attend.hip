// attend.hip -- split-K decode attention over a dense or index-gathered row
// list; each workgroup leaves one (max, sum, acc[d]) partial per query head and
// the log-sum-exp merge kernel (merge.hip) combines them.
//
// Method: exact softmax attention restricted to a key set (top-K attention,
// "Sparse-to-Dense ..." Sec. 3.2; the kept set plus the recent tail read by a
// split-K decoding kernel, "Where Activation Sparsity and KV-Cache Sparsity
// Cross ..." sections "Speedup Across Context" and "The Attention Baseline").
//
// Layout on gfx950 (64-lane waves): one K or V row is split into 16-byte lane
// slices, so a wave load moves 1 KB = RowsPerLoad consecutive rows; the G
// query heads of the kv head ride along, so every K/V byte is read once for
// the whole group.  Loads go through buffer descriptors of the head's K and V
// (SGPRs) with 32-bit lane offsets: dense rows need no per-load address
// arithmetic (the row step sits in the scalar offset), gathered rows one
// LDS read.  The library runs it on fp32 caches (bf16 caches take the
// matrix-core kernel, attend_mfma.hip; the template also reads bf16 rows with
// packed dot products).  Logits are lane-slice dot products and a DPP
// reduction over the lanes of a row; softmax runs in the log2 domain in fp32
// against a reference max fixed from each wave's first block (no rescaling
// in the steady state); only the last iteration of a chunk pays for masking.
// Each workgroup owns `chunk` rows of one kv head and folds its waves into
// one partial per query head.  The merge runs as a
// second kernel: a completion counter inside this kernel would need a
// device-scope release per workgroup, which on gfx950 is an L2 write-back plus
// invalidate that serialises across the workgroups of an XCD.
#include <type_traits>

#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
// Loads per lane per iteration for each of K and V (fewer for large groups,
// whose accumulators take the registers).
constexpr int loads_per_iter(int g) { return g >= 16 ? 1 : (g >= 7 ? 2 : 4); }
constexpr int kMaxChunk = 2048;        // rows per workgroup (LDS offset list)
// Probabilities are 2^(logit - reference); the fast loop keeps one reference
// per wave and query head and leaves for a rescaling loop only when a logit
// passes it by this many log2 units (so p <= 2^30 and sums stay far from
// fp32 overflow).
constexpr float kRefSlack = 30.0f;

template <int DT, int D, int G, bool SPARSE>
__global__ __launch_bounds__(kThreads) void attend_kernel(const AttendArgs a) {
  using RG = RowGeom<DT, D>;
  constexpr int LPR = RG::kLanesPerRow;
  constexpr int EPL = RG::kElemsPerLane;
  constexpr int RPL = RG::kRowsPerLoad;
  constexpr int U = loads_per_iter(G);
  constexpr int RI = U * RPL;

  __shared__ uint32_t sm_off[SPARSE ? kMaxChunk : 1];  // byte offsets of this chunk's rows
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  __shared__ float sm_acc[kWaves][G][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int cph = a.chunks_per_head;
  const int h = blockIdx.x % a.n_kv_heads;  // a kv head's chunks on one XCD (as the merge)
  const int c = blockIdx.x / a.n_kv_heads;

  // Sparse: the index entries this chunk may use are read in the same round
  // trip as the head's count (entries below idx_stride are always allocated).
  int32_t cnt = 0;
  int64_t rows_h;
  int32_t spec[SPARSE ? (kMaxChunk + kThreads - 1) / kThreads : 1];
  if constexpr (SPARSE) {
    const int32_t* ih = a.idx + (int64_t)h * a.idx_stride;
    const int64_t rs0 = (int64_t)c * a.chunk;
#pragma unroll
    for (int k = 0; k < (kMaxChunk + kThreads - 1) / kThreads; ++k) spec[k] = 0;
    if (a.count_max > 0) {  // uniform: idx may be null when no entry is usable
#pragma unroll
      for (int k = 0; k < (kMaxChunk + kThreads - 1) / kThreads; ++k) {
        const int64_t r = rs0 + tid + k * kThreads;
        spec[k] = ih[r < a.count_max ? r : a.count_max - 1];  // clamped, all loads in flight
      }
    }
    cnt = a.count[h];
    cnt = cnt < 0 ? 0 : (cnt > (int32_t)a.count_max ? (int32_t)a.count_max : cnt);
    rows_h = (int64_t)cnt + (a.n - a.tail_start);
  } else {
    rows_h = a.n;
  }
  // this lane's slice of each query head of the group (in flight with the
  // index loads above)
  const int part = lane % LPR;
  const int rgrp = lane / LPR;
  uint32_t qr[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 t = ld16(reinterpret_cast<const char*>(a.q) +
                         ((int64_t)(h * G + g) * D) * RG::kElem + part * 16);
    qr[g][0] = t.x; qr[g][1] = t.y; qr[g][2] = t.z; qr[g][3] = t.w;
  }
  int nch = (int)((rows_h + a.chunk - 1) / a.chunk);
  nch = nch < 1 ? 1 : (nch > cph ? cph : nch);
  if (c >= nch) return;
  const int64_t r0 = (int64_t)c * a.chunk;
  const int64_t rem = rows_h - r0;
  const int rows = (int)(rem < 0 ? 0 : (rem > a.chunk ? a.chunk : rem));
  const uint32_t stride = (uint32_t)a.pos_stride_b;

  if constexpr (SPARSE) {
    const int32_t last = (int32_t)(a.n - 1);
#pragma unroll
    for (int k = 0; k < (kMaxChunk + kThreads - 1) / kThreads; ++k) {
      const int i = tid + k * kThreads;
      if (i < a.chunk) {
        const int64_t r = r0 + i;
        int32_t p = 0;
        if (i < rows) p = r < cnt ? spec[k] : (int32_t)(a.tail_start + (r - cnt));
        p = p < 0 ? 0 : (p > last ? last : p);  // keep out-of-contract indices in bounds
        sm_off[i] = (uint32_t)p * stride;
      }
    }
  }

  if constexpr (SPARSE) __syncthreads();

  // the host keeps n * pos_stride below 2^32 so row offsets fit the descriptor
  const uint32_t span = (uint32_t)(a.n * a.pos_stride_b);
  const BufRsrc rk = make_rsrc(a.k + (int64_t)h * a.head_stride_b, span);
  const BufRsrc rv = make_rsrc(a.v + (int64_t)h * a.head_stride_b, span);
  const uint32_t lane_off = (uint32_t)part * 16u;

  // Per query head: reference max m (log2 units) the probabilities are taken
  // against, sum l and acc[d] of this lane's row group.
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
  }

  const int nit_total = (rows + RI - 1) / RI;
  const int per = (nit_total + kWaves - 1) / kWaves;
  const int it0 = wave * per;
  const int it1 = (it0 + per < nit_total) ? it0 + per : nit_total;
  const int full_end = rows / RI;  // iterations below this index need no mask
  // dense: lane offset of row (r0 + rgrp); iteration and load steps ride in the scalar offset
  const uint32_t dense_voff = (uint32_t)(r0 + rgrp) * stride + lane_off;
  const float c2 = a.scale_log2;  // log2-domain logit = dot * c2 (c2 > 0)

  auto issue = [&](int it, uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (SPARSE) {
        const uint32_t off = sm_off[it * RI + u * RPL + rgrp] + lane_off;
        kr[u] = buf_load16_stream(rk, off, 0);
        vr[u] = buf_load16_stream(rv, off, 0);
      } else {
        const uint32_t soff = (uint32_t)(it * RI + u * RPL) * stride;
        kr[u] = buf_load16_stream(rk, dense_voff, soff);
        vr[u] = buf_load16_stream(rv, dense_voff, soff);
      }
    }
  };

  // raw dot products of the iteration's rows, summed over the LPR lanes of a
  // row (the U*G DPP chains interleaved); -inf for rows past the chunk
  auto logits = [&](int it, const uint4 (&kr)[U], float (&s)[U][G]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g) s[u][g] = slice_dot<DT>(qr[g], kr[u]);
    if constexpr (LPR >= 2) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) s[u][g] += dpp<kDppXor1>(s[u][g]);
    }
    if constexpr (LPR >= 4) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) s[u][g] += dpp<kDppXor2>(s[u][g]);
    }
    if constexpr (LPR >= 8) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) s[u][g] += dpp<kDppHalfMirror>(s[u][g]);
    }
    if constexpr (LPR >= 16) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) s[u][g] += dpp<kDppMirror>(s[u][g]);
    }
    if constexpr (LPR >= 32) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) s[u][g] += __shfl_xor(s[u][g], 16, 64);
    }
    if (it >= full_end) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool valid = it * RI + u * RPL + rgrp < rows;
#pragma unroll
        for (int g = 0; g < G; ++g) s[u][g] = valid ? s[u][g] : kNegInf;
      }
    }
  };

  // true if some row of the iteration exceeds its reference by the slack
  auto overflows = [&](const float (&s)[U][G]) {
    bool over = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) x = fmaxf(x, s[u][g]);
      over = over || (x * c2 > m[g] + kRefSlack);
    }
    return __builtin_amdgcn_ballot_w64(over) != 0;
  };

  auto accumulate = [&](const float (&s)[U][G], const uint4 (&vr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      slice_to_f32<DT>(vr[u], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = fast_exp2(fmaf(s[u][g], c2, -m[g]));
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
      }
    }
  };

  if (it0 < it1) {
    uint4 ka[U], va[U], kc[U], vc[U];
    float s[U][G];
    issue(it0, ka, va);
    logits(it0, ka, s);
    // wave-uniform reference: the first block's max (0 if it has no valid row)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) x = fmaxf(x, s[u][g]);
      x = wave_max(x) * c2;
      m[g] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x == kNegInf ? 0.0f : x)));
    }
    // fast path: fixed reference, no rescaling; leaves at the first iteration
    // whose logits pass the reference by kRefSlack (then `it` is redone below)
    int it = it0;
    bool fell_back = false;
    for (;;) {
      if (it + 1 < it1) issue(it + 1, kc, vc);
      if (overflows(s)) { fell_back = true; break; }
      accumulate(s, va);
      if (++it >= it1) break;
      logits(it, kc, s);
      if (it + 1 < it1) issue(it + 1, ka, va);
      if (overflows(s)) { fell_back = true; break; }
      accumulate(s, vc);
      if (++it >= it1) break;
      logits(it, ka, s);
    }
    if (fell_back) {
      // rare: online softmax with rescaling from iteration `it` on
      for (; it < it1; ++it) {
        issue(it, ka, va);
        logits(it, ka, s);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float x = s[0][g];
#pragma unroll
          for (int u = 1; u < U; ++u) x = fmaxf(x, s[u][g]);
          x *= c2;
          if (x > m[g]) {
            const float alpha = fast_exp2(m[g] - x);
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
            m[g] = x;
          }
        }
        accumulate(s, va);
      }
    }
  }
  // from here m is this lane's reference (possibly per lane after a fall-back)

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
  if (c == 0 && tid == 0) a.nch[h] = nch;
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
    case 3: return launch3<DT, D, 3>(sparse, a, s);
    case 4: return launch3<DT, D, 4>(sparse, a, s);
    case 5: return launch3<DT, D, 5>(sparse, a, s);
    case 6: return launch3<DT, D, 6>(sparse, a, s);
    case 7: return launch3<DT, D, 7>(sparse, a, s);
    case 8: return launch3<DT, D, 8>(sparse, a, s);
    case 16: return launch3<DT, D, 16>(sparse, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int attend_rows_per_iter(int dtype, int d) {
  const int elem = dtype == 1 ? 2 : 4;
  const int lpr = d * elem / 16;
  return loads_per_iter(1) * (64 / lpr);  // the largest; chunks are multiples of 4x this
}

int attend_max_chunk() { return kMaxChunk; }
int attend_waves() { return kWaves; }

hipError_t launch_attend(int dtype, int d, int g, bool sparse, const AttendArgs& a,
                         hipStream_t s) {
  // fp32 caches only: bf16 caches run the matrix-core kernel (attend_mfma.hip)
  if (dtype == 0 && d == 128) return launch2<0, 128>(g, sparse, a, s);
  if (dtype == 0 && d == 64) return launch2<0, 64>(g, sparse, a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
