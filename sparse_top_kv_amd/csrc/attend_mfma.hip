// attend_mfma.hip -- split-K decode attention for bf16 caches: K/V tiles
// streamed into LDS by direct-to-LDS buffer loads, q.k and p.v on the matrix
// cores.  Same contract and partial format as attend.hip (which keeps the fp32
// caches); the log-sum-exp merge kernel combines the partials.
//
// Method: exact softmax attention restricted to a key set (top-K attention,
// "Sparse-to-Dense ..." Sec. 3.2; the kept set plus the recent tail read by a
// split-K decoding kernel, "Where Activation Sparsity and KV-Cache Sparsity
// Cross ..." sections "Speedup Across Context" and "The Attention Baseline").
//
// Why this shape on gfx950.  A decode step is HBM-bound: the job is to keep
// enough bytes in flight per CU and to keep the arithmetic off the critical
// path.  With G query heads per kv head the per-key arithmetic is two small
// contractions (q.K^T over d, P.V over keys) that the vector ALUs only do at
// ~30 instructions per key; here they run as MFMAs with the query heads padded
// to the 16-wide tile, and the vector ALUs keep only the softmax.
//   - Each wave owns a private ring of kStages tiles of 16 keys (K and V,
//     4 KB each at d=128) in LDS, filled by buffer_load ... lds, so up to
//     (kStages-1) tiles per wave are in flight without holding registers.
//     Waits are explicit vmcnt counts; the stages are distinct LDS objects so
//     the compiler can tell which outstanding copies a read depends on.
//   - q.K^T: v_mfma_f32_16x16x32_bf16 with A = 16 keys (one 16-byte LDS read
//     per lane) and B = the padded query heads (registers).  The result holds,
//     in lane (q, i), keys 4q..4q+3 of head i: exactly the A operand layout of
//     v_mfma_f32_16x16x16_bf16 for P.V, so probabilities never leave their lanes.
//   - P.V: B = V tile read with ds_read_b64_tr_b16 (a transposing LDS read:
//     four keys of one column per lane); P is split into bf16 hi + lo and
//     both are applied, so the product keeps ~16 bits of P.
//   - LDS tiles are XOR-swizzled per row so the K reads and the transposing V
//     reads are free of bank conflicts; the direct-to-LDS copy writes whole
//     1 KB runs, and each lane fetches the 16-byte piece that belongs at its
//     slot, so the swizzle costs nothing on the copy side.
//   - Softmax in the log2 domain against a per-head reference fixed from the
//     wave's first tile; a tile whose logits pass the reference by kSlack
//     rescales the accumulators (rare, wave-uniform branch).
#include "skv_common.h"
#include "skv_kernels.h"
#include "skv_mfma.h"

namespace skv {
namespace {

constexpr int kW = 4;                     // waves per workgroup
constexpr int kT = 64 * kW;
constexpr int kStep = 16;                 // keys per wave step (one tile)
constexpr int kStages = 4;                // tiles per wave ring
constexpr int kSparseMaxChunk = 512;      // rows per workgroup (LDS offset list)
constexpr float kSlack = 30.0f;

#define SKV_LDS __attribute__((address_space(3)))
typedef short short4_t __attribute__((ext_vector_type(4)));

template <int D>
struct TileGeom {
  static constexpr int kRB = D * 2;              // bytes per bf16 row
  static constexpr int kPPR = kRB / 16;          // 16-byte pieces per row
  static constexpr int kRPI = 1024 / kRB;        // rows per direct-to-LDS copy (1 KB)
  static constexpr int kNI = kStep / kRPI;       // copies per tile (each of K and V)
  static constexpr int kTB = kStep * kRB;        // bytes per tile
  static constexpr int kKS = D / 32;             // k-steps of the q.K^T MFMA
  static constexpr int kNT = D / 16;             // 16-column tiles of the P.V MFMA
};

// Piece swizzles (XOR on the 16-byte piece index) of tile row t.  K rows are
// read 16 rows x one piece per 16 lanes; V is read transposed, 4 rows x two
// pieces per 16 lanes (8 rows per 32 lanes).  Both make those groups hit
// distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int t) {
  return D == 128 ? (t & 15) : ((((t >> 2) << 1) | (t & 1)) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int t) {
  return D == 128 ? 2 * (t & 7) : 2 * ((t & 1) | (((t >> 2) & 1) << 1));
}
// LDS byte of piece slot `pos` of tile row t: copy u = t % NI writes 1 KB
// holding rows u, u + NI, u + 2 NI, ...
template <int D>
__device__ __forceinline__ int tile_byte(int t, int pos) {
  using TG = TileGeom<D>;
  return (t % TG::kNI) * 1024 + (t / TG::kNI) * TG::kRB + pos * 16;
}

// s_waitcnt with vmcnt <= N and the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ floatx4_t mfma16(const short4_t& a, const short4_t& b, const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS: the wave's 64 pieces land
// contiguously (1 KB) at the wave-uniform LDS address `lds` (non-temporal).
__device__ __forceinline__ void copy_to_lds(BufRsrc r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SKV_LDS void*)lds, 16, voff, soff, 0, 2);
}
// Transposing LDS read: within each 16 lanes, lane j receives element j % 4 of
// the 8-byte pieces addressed by lanes 4k + j / 4, k = 0..3.
__device__ __forceinline__ short4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SKV_LDS short4_t*)p);
}

// Two floats to packed bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return f32_to_bf16_bits(x) | (f32_to_bf16_bits(y) << 16);
}

template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(kT) void attend_mfma_kernel(const AttendArgs a) {
  using TG = TileGeom<D>;
  constexpr int NI = TG::kNI, TB = TG::kTB, PPR = TG::kPPR, KS = TG::kKS, NT = TG::kNT;

  // per wave: [K tile | V tile]; one LDS object per stage
  __shared__ __attribute__((aligned(1024))) char st0[kW][2 * TB];
  __shared__ __attribute__((aligned(1024))) char st1[kW][2 * TB];
  __shared__ __attribute__((aligned(1024))) char st2[kW][2 * TB];
  __shared__ __attribute__((aligned(1024))) char st3[kW][2 * TB];
  __shared__ __attribute__((aligned(16))) uint32_t sm_off[SPARSE ? kSparseMaxChunk : 1];
  __shared__ float sm_m[kW][G], sm_l[kW][G];
  __shared__ float sm_acc[kW][G][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, li = lane & 15;
  const int cph = a.chunks_per_head;
  const int h = blockIdx.x / cph;
  const int c = blockIdx.x - h * cph;

  int32_t cnt = 0;
  int64_t rows_h;
  constexpr int kSpec = (kSparseMaxChunk + kT - 1) / kT;
  int32_t spec[SPARSE ? kSpec : 1];
  if constexpr (SPARSE) {
    const int32_t* ih = a.idx + (int64_t)h * a.idx_stride;
    const int64_t rs0 = (int64_t)c * a.chunk;
#pragma unroll
    for (int k = 0; k < kSpec; ++k) spec[k] = 0;
    if (a.count_max > 0) {  // uniform: idx may be null when no entry is usable
#pragma unroll
      for (int k = 0; k < kSpec; ++k) {
        const int64_t r = rs0 + tid + k * kT;
        spec[k] = ih[r < a.count_max ? r : a.count_max - 1];
      }
    }
    cnt = a.count[h];
    cnt = cnt < 0 ? 0 : (cnt > (int32_t)a.count_max ? (int32_t)a.count_max : cnt);
    rows_h = (int64_t)cnt + (a.n - a.tail_start);
  } else {
    rows_h = a.n;
  }
  // q as the B operand of q.K^T: lane (q4, li) holds head li's channels
  // [32 s + 8 q4, +8); heads past G are zero
  bf16x8_t qb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint4 t = make_uint4(0u, 0u, 0u, 0u);
    if (li < G)
      t = ld16(reinterpret_cast<const char*>(a.q) + ((int64_t)(h * G + li) * D + 32 * s + 8 * q4) * 2);
    qb[s] = as_bf16x8(t);
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
    for (int k = 0; k < kSpec; ++k) {
      const int i = tid + k * kT;
      if (i < kSparseMaxChunk) {
        const int64_t r = r0 + i;
        int32_t p = 0;
        if (i < rows) p = r < cnt ? spec[k] : (int32_t)(a.tail_start + (r - cnt));
        p = p < 0 ? 0 : (p > last ? last : p);  // keep out-of-contract indices in bounds
        sm_off[i] = (uint32_t)p * stride;
      }
    }
    __syncthreads();
  }

  const uint32_t span = (uint32_t)(a.n * a.pos_stride_b);
  const BufRsrc rk = make_rsrc(a.k + (int64_t)h * a.head_stride_b, span);
  const BufRsrc rv = make_rsrc(a.v + (int64_t)h * a.head_stride_b, span);

  // copy side: lane -> (row group, piece slot); copy u moves row t = grp*NI + u
  const int grp = lane / PPR, pos = lane % PPR;
  uint32_t pk[NI], pv[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int t = grp * NI + u;
    pk[u] = (uint32_t)((pos ^ swz_k<D>(t)) * 16);
    pv[u] = (uint32_t)((pos ^ swz_v<D>(t)) * 16);
    if constexpr (!SPARSE) {
      pk[u] += (uint32_t)t * stride;
      pv[u] += (uint32_t)t * stride;
    }
  }
  // read side: K rows for the A operand, V columns for the transposed reads
  const int wbase = wave * 2 * TB;
  int koff[KS], voff[NT];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = wbase + tile_byte<D>(li, (4 * s + q4) ^ swz_k<D>(li));
  {
    const int kk = (lane & 15) >> 2, m = lane & 3;
    const int t = 4 * q4 + kk;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      voff[n] = wbase + TB + tile_byte<D>(t, (2 * n + (m >> 1)) ^ swz_v<D>(t)) + (m & 1) * 8;
  }

  const int nsteps = (rows + kStep - 1) / kStep;
  const int nst = wave < nsteps ? (nsteps - 1 - wave) / kW + 1 : 0;  // this wave's steps
  const float c2 = a.scale_log2;

  // copies of local step k (global step wave + kW k) into a stage
  auto issue = [&](char (*stg)[2 * TB], int k) {
    const int j = wave + kW * k;
    char* dst = &stg[wave][0];
    if constexpr (SPARSE) {
      uint32_t ro[NI];
      if constexpr (NI == 4) {
        const uint4 o4 = *reinterpret_cast<const uint4*>(&sm_off[j * kStep + grp * NI]);
        ro[0] = o4.x; ro[1] = o4.y; ro[2] = o4.z; ro[3] = o4.w;
      } else {
        const uint2 o2 = *reinterpret_cast<const uint2*>(&sm_off[j * kStep + grp * NI]);
        ro[0] = o2.x; ro[1] = o2.y;
      }
#pragma unroll
      for (int u = 0; u < NI; ++u)
        copy_to_lds(rk, dst + u * 1024, ro[u] + pk[u], 0);
#pragma unroll
      for (int u = 0; u < NI; ++u)
        copy_to_lds(rv, dst + TB + u * 1024, ro[u] + pv[u], 0);
    } else {
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(r0 + (int64_t)j * kStep) * stride);
#pragma unroll
      for (int u = 0; u < NI; ++u)
        copy_to_lds(rk, dst + u * 1024, pk[u], soff);
#pragma unroll
      for (int u = 0; u < NI; ++u)
        copy_to_lds(rv, dst + TB + u * 1024, pv[u], soff);
    }
  };

  float m = kNegInf;   // reference of head li (log2 units)
  float l = 0.0f;      // this lane's share of head li's sum
  floatx4_t o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // log2-domain logits of the tile of local step k (already in LDS): key
  // 4 q4 + r of head li; -inf past the chunk
  auto logits = [&](const char* base, int k, float (&sv)[4]) {
    floatx4_t cs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 kv = *reinterpret_cast<const uint4*>(base + koff[s]);
      cs = mfma_bf16(as_bf16x8(kv), qb[s], cs);
    }
    const int rb = (wave + kW * k) * kStep + 4 * q4;
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = rb + r < rows ? cs[r] * c2 : kNegInf;
  };
  // max over the tile's keys of head li (all four q4 lanes agree)
  auto head_max = [&](const float (&sv)[4]) {
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    return fmaxf(mx, __shfl_xor(mx, 32, 64));
  };
  // probabilities against the reference, into the sum and the P.V MFMAs
  auto accumulate = [&](const char* base, const float (&sv)[4]) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(sv[r] - m);
      l += p[r];
    }
    const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
    const uint32_t l01 = pack_bf16(p[0] - bf16lo(h01), p[1] - bf16hi(h01));
    const uint32_t l23 = pack_bf16(p[2] - bf16lo(h23), p[3] - bf16hi(h23));
    const short4_t ahi = __builtin_bit_cast(short4_t, make_uint2(h01, h23));
    const short4_t alo = __builtin_bit_cast(short4_t, make_uint2(l01, l23));
    short4_t vb[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
      vb[n] = lds_read_tr16(base + voff[n]);
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = mfma16(ahi, vb[n], o[n]);
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = mfma16(alo, vb[n], o[n]);
  };

  // wait until the copies of local step k have landed (newer = steps issued after k)
  auto wait_step = [&](int newer) {
    if (newer >= kStages - 1) wait_vm<(kStages - 1) * 2 * NI>();
    else if (newer == 2) wait_vm<2 * 2 * NI>();
    else if (newer == 1) wait_vm<2 * NI>();
    else wait_vm<0>();
  };
  auto newer_than = [&](int k) { return (nst - 1 - k) < (kStages - 1) ? (nst - 1 - k) : (kStages - 1); };

  // steady state: refill the stage freed by the previous step, wait for step
  // k, and accumulate it against the fixed reference.  Returns false, with
  // nothing accumulated, if a logit passes the reference by kSlack.
  auto fast_step = [&](char (*cur)[2 * TB], char (*nxt)[2 * TB], int k) {
    if (k + kStages - 1 < nst) {
      wait_lgkm0();  // reads of the stage being refilled are done
      issue(nxt, k + kStages - 1);
    }
    wait_step(newer_than(k));
    float sv[4];
    logits(&cur[0][0], k, sv);
    const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    if (__builtin_amdgcn_ballot_w64(li < G && mx > m + kSlack) != 0) return false;
    accumulate(&cur[0][0], sv);
    return true;
  };

  static_assert(kStages == 4, "the ring below is written for four stages");
  if (nst > 0) issue(st0, 0);
  if (nst > 1) issue(st1, 1);
  if (nst > 2) issue(st2, 2);
  int k = 0;
  bool slow = false;
  if (nst > 0) {
    // reference: the first tile's max per head (0 for a head with no valid key)
    wait_step(newer_than(0));
    float sv[4];
    logits(&st0[0][0], 0, sv);
    const float mx = head_max(sv);
    m = mx == kNegInf ? 0.0f : mx;
    while (k < nst) {
      if (!fast_step(st0, st3, k)) { slow = true; break; }
      if (++k >= nst) break;
      if (!fast_step(st1, st0, k)) { slow = true; break; }
      if (++k >= nst) break;
      if (!fast_step(st2, st1, k)) { slow = true; break; }
      if (++k >= nst) break;
      if (!fast_step(st3, st2, k)) { slow = true; break; }
      ++k;
    }
  }
  if (slow) {
    // rare: online rescaling from step k on; steps up to `issued` are in
    // flight in their stages, later ones are copied one at a time
    int issued = k + kStages - 1 < nst ? k + kStages - 1 : nst - 1;
    for (; k < nst; ++k) {
      const int sel = k & 3;
      char (*cur)[2 * TB] = sel == 0 ? st0 : (sel == 1 ? st1 : (sel == 2 ? st2 : st3));
      if (k > issued) {
        wait_lgkm0();
        issue(cur, k);
        issued = k;
      }
      wait_vm<0>();
      float sv[4];
      logits(&cur[0][0], k, sv);
      const float mn = fmaxf(m, head_max(sv));
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
      m = mn;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * q4 + r, 64);  // head 4 q4 + r
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[n][r] *= ar[r];
      accumulate(&cur[0][0], sv);
    }
  }

  // fold the four lanes of each head (q4 groups) and park the wave's partial
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (nst == 0) {
    m = kNegInf;
    l = 0.0f;
  }
  if (lane < G) {
    sm_m[wave][lane] = m;
    sm_l[wave][lane] = l;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = 4 * q4 + r;
    if (g < G) {
#pragma unroll
      for (int n = 0; n < NT; ++n) sm_acc[wave][g][16 * n + li] = o[n][r];
    }
  }
  __syncthreads();

  const int64_t slot = (int64_t)h * cph + c;
  for (int e = tid; e < G * D; e += kT) {
    const int g = e / D, dd = e - g * D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kW; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
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

template <int D, int G>
hipError_t launch_g(bool sparse, const AttendArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_kv_heads * a.chunks_per_head));
  if (sparse)
    hipLaunchKernelGGL((attend_mfma_kernel<D, G, true>), grid, dim3(kT), 0, s, a);
  else
    hipLaunchKernelGGL((attend_mfma_kernel<D, G, false>), grid, dim3(kT), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int g, bool sparse, const AttendArgs& a, hipStream_t s) {
  switch (g) {
    case 1: return launch_g<D, 1>(sparse, a, s);
    case 2: return launch_g<D, 2>(sparse, a, s);
    case 4: return launch_g<D, 4>(sparse, a, s);
    case 7: return launch_g<D, 7>(sparse, a, s);
    case 8: return launch_g<D, 8>(sparse, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int attend_mfma_granule() { return kW * kStep; }
int attend_mfma_sparse_max_chunk() { return kSparseMaxChunk; }

hipError_t launch_attend_mfma(int d, int g, bool sparse, const AttendArgs& a, hipStream_t s) {
  if (d == 128) return launch_d<128>(g, sparse, a, s);
  if (d == 64) return launch_d<64>(g, sparse, a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
