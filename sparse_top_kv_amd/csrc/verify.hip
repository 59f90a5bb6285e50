// verify.hip -- causal verify of gamma drafted tokens in one pass over the
// cache, on MFMA ("Sparse-to-Dense ..." Sec. 3.1: the dense model checks all
// gamma proposals in parallel with a single read of the full KV cache).
//
// Query t (t < gamma) of query head g sits at position n - gamma + t and sees
// keys [0, n - gamma + t].  Per kv head the gamma x G query rows share every
// K/V byte: rows r = t * G + g_in (R = gamma * G <= 64) form up to four
// 16-row tiles, one per wave.  A workgroup owns `chunk` keys of one kv head
// and walks them in 64-key sub-blocks staged through LDS:
//   S^T[key][row] = K Q^T      (A = K rows from LDS, B = Q rows in registers)
//   online softmax per row in fp32 (log2 domain)
//   O^T[dim][row] += V^T P^T  (B = P split into bf16 hi + lo, two MFMAs, so the
//                              probabilities keep ~16 bits; A = V^T from LDS)
// The P^T operand is used with a permuted key order (keys 4q..4q+3 of two
// 16-key tiles) that matches the C layout of the S MFMA, so P never leaves the
// lane; V^T is read from LDS in the same order.  Chunk partials go through the
// same log-sum-exp merge kernel as the decode attention.
#include "skv_kernels.h"
#include "skv_mfma.h"

namespace skv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 256;
constexpr int kSub = 64;                 // keys per LDS sub-block
constexpr int kMaxRows = 16 * kWaves;    // gamma * G

template <int D>
__global__ __launch_bounds__(kThreads) void verify_kernel(const VerifyArgs a) {
  constexpr int KS = D / 32;        // MFMA k-steps over the head dim
  constexpr int DT = D / 16;        // 16-dim tiles of the output
  constexpr int PITCH = D * 2 + 16; // LDS row pitch in bytes (bank spread)
  constexpr int PIECES = kSub * D / 8;         // 16-byte pieces per tensor sub-block
  constexpr int PPT = PIECES / kThreads;       // pieces per thread
  static_assert(PPT * kThreads == PIECES, "sub-block must tile the workgroup");
  constexpr int kStageBytes = 2 * kSub * PITCH;

  __shared__ __align__(16) unsigned char sm_stage[kStageBytes];
  unsigned char* sK = sm_stage;
  unsigned char* sV = sm_stage + kSub * PITCH;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int G = a.group;
  const int R = a.gamma * G;
  const int Hq = a.n_kv_heads * G;
  const int cph = a.chunks_per_head;
  const int h = blockIdx.x / cph;
  const int c = blockIdx.x - h * cph;
  const int64_t n = a.n;
  const int64_t k0 = (int64_t)c * a.chunk;
  const int64_t k1 = (k0 + a.chunk < n) ? k0 + a.chunk : n;
  const int nsub = (int)((k1 - k0 + kSub - 1) / kSub);

  // this wave's row tile: B operand (Q rows) for every k-step
  const int row = wave * 16 + i16;
  const bool row_ok = row < R;
  const int t_row = row_ok ? row / G : 0;
  const int g_row = row_ok ? row - t_row * G : 0;
  const int64_t last_key = n - a.gamma + t_row;  // causal limit of this row
  bf16x8_t qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (row_ok)
      u = ld16(a.q + ((int64_t)t_row * Hq + h * G + g_row) * D + ks * 32 + q4 * 8);
    qb[ks] = as_bf16x8(u);
  }
  const bool wave_active = wave * 16 < R;

  float m = kNegInf, lsum = 0.0f;
  floatx4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const char* kbase = a.k + (int64_t)h * a.head_stride_b;
  const char* vbase = a.v + (int64_t)h * a.head_stride_b;
  uint4 pk[PPT], pv[PPT];
  auto prefetch = [&](int sb) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = tid + i * kThreads;
      const int r = piece / (D / 8), col = piece - r * (D / 8);
      int64_t key = k0 + (int64_t)sb * kSub + r;
      key = key < k1 ? key : k1 - 1;
      pk[i] = ld16(kbase + key * a.pos_stride_b + col * 16);
      pv[i] = ld16(vbase + key * a.pos_stride_b + col * 16);
    }
  };
  if (nsub > 0) prefetch(0);

  for (int sb = 0; sb < nsub; ++sb) {
    __syncthreads();  // previous sub-block fully consumed
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int piece = tid + i * kThreads;
      const int r = piece / (D / 8), col = piece - r * (D / 8);
      *reinterpret_cast<uint4*>(sK + r * PITCH + col * 16) = pk[i];
      *reinterpret_cast<uint4*>(sV + r * PITCH + col * 16) = pv[i];
    }
    __syncthreads();
    if (sb + 1 < nsub) prefetch(sb + 1);
    if (!wave_active) continue;

    // S^T for 4 key tiles of 16
    const int64_t kb0 = k0 + (int64_t)sb * kSub;
    floatx4_t s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 ka = *reinterpret_cast<const uint4*>(sK + (kt * 16 + i16) * PITCH + ks * 64 + q4 * 16);
        acc = mfma_bf16(as_bf16x8(ka), qb[ks], acc);
      }
      s[kt] = acc;
    }
    float mb = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = kb0 + kt * 16 + q4 * 4 + r;
        const float x = (key < k1 && key <= last_key) ? s[kt][r] * a.scale_log2 : kNegInf;
        s[kt][r] = x;
        mb = fmaxf(mb, x);
      }
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mnew = fmaxf(m, mb);
    const float alpha = (m == kNegInf) ? 0.0f : fast_exp2(m - mnew);
    m = mnew;
    const float mu = (m == kNegInf) ? 0.0f : m;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

    // probabilities, split into bf16 hi + lo, packed as the P^T operand
    uint32_t phi[4][2], plo[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(s[kt][r] - mu);
        lsum += p;
        hb[r] = f32_to_bf16_bits(p);
        lb[r] = f32_to_bf16_bits(p - __uint_as_float(hb[r] << 16));
      }
      phi[kt][0] = hb[0] | (hb[1] << 16); phi[kt][1] = hb[2] | (hb[3] << 16);
      plo[kt][0] = lb[0] | (lb[1] << 16); plo[kt][1] = lb[2] | (lb[3] << 16);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ta = 2 * half, tb = 2 * half + 1;  // key tiles joined in one k-step
      const bf16x8_t bhi = as_bf16x8(make_uint4(phi[ta][0], phi[ta][1], phi[tb][0], phi[tb][1]));
      const bf16x8_t blo = as_bf16x8(make_uint4(plo[ta][0], plo[ta][1], plo[tb][0], plo[tb][1]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int dim = dt * 16 + i16;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ka = (e < 2 ? ta : tb) * 16 + q4 * 4 + (e & 1) * 2;
          const uint32_t lo16 = *reinterpret_cast<const uint16_t*>(sV + ka * PITCH + dim * 2);
          const uint32_t hi16 = *reinterpret_cast<const uint16_t*>(sV + (ka + 1) * PITCH + dim * 2);
          w[e] = lo16 | (hi16 << 16);
        }
        const bf16x8_t va = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
        o[dt] = mfma_bf16(va, bhi, o[dt]);
        o[dt] = mfma_bf16(va, blo, o[dt]);
      }
    }
  }

  // chunk partial of this wave's rows
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const int64_t slot = (int64_t)h * cph + c;
  if (wave_active && row_ok) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.part_acc[(slot * R + row) * D + dt * 16 + q4 * 4 + r] = o[dt][r];
    }
    if (q4 == 0) {
      a.part_ml[(slot * R + row) * 2 + 0] = m;
      a.part_ml[(slot * R + row) * 2 + 1] = lsum;
    }
  }

  if (c == 0 && tid == 0) a.nch[h] = (int32_t)((n + a.chunk - 1) / a.chunk);
}

}  // namespace

int verify_max_rows() { return kMaxRows; }
int verify_chunk_granule() { return kSub; }

hipError_t launch_verify(int d, const VerifyArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_kv_heads * a.chunks_per_head));
  if (d == 128)
    hipLaunchKernelGGL(verify_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else if (d == 64)
    hipLaunchKernelGGL(verify_kernel<64>, grid, dim3(kThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace skv
