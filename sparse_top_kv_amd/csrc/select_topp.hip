// select_topp.hip -- verifier-guided two-stage selection (SpecVLM blog, "The
// SpecVLM Method": Stage I top-P retention, Stage II spatially uniform
// reduction).
//
// One 1024-thread workgroup per selection: a score row (kv head), or, pooled,
// the per-token sum over all rows (the blog averages the verifier's attention
// over layers and heads; the constant factor does not change the selection).
//
// Mass is exact fixed point: u_j = floor(a_j 2^S) for a score a_j >= 0, with
// S = 62 - E - ceil(log2 N), 2^(E-1) <= max a < 2^E and N the number of terms
// in one total, so every sum is an exact 64-bit integer below 2^62 and the
// threshold test cannot depend on the order of additions.
//
//   1. max score -> S; total mass U; theta = ceil(lambda U) (128-bit product)
//   2. radix passes over the 62-bit masses, 8-bit digits from the top, with
//      per-bin count and mass histograms: the pass finds the bin where the
//      running mass (largest first) reaches theta.  The last pass fixes the
//      mass v* of the entry that crosses; `take` entries equal to v* are kept,
//      lowest index first.  c = |V_R| entries in all.
//   3. one pass in index order: V_R membership (u > v*, or u == v* within the
//      first `take` ties), the leftover rank of every other candidate, the
//      uniform picks at leftover ranks floor(i L / n_U), and the ascending
//      output -- three workgroup ballots per 1024 candidates.
//
// Digit 0 of a pass is not counted with atomics: it is the group's count and
// mass minus the other bins (most masses are tiny, so most entries land there
// in the top digits).
#include "skv_block.h"
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

constexpr int kToppBins = 256;

__device__ __forceinline__ uint32_t pos_bits(float x) { return x > 0.0f ? __float_as_uint(x) : 0u; }

// floor(x 2^S) for x > 0 (0 otherwise), exactly, from the fp32 bits.
__device__ __forceinline__ uint64_t fixed_mass(float x, int S) {
  const uint32_t b = pos_bits(x);
  if (b == 0u) return 0u;
  const uint32_t be = b >> 23;
  uint64_t m = b & 0x7fffffu;
  int ex = -149;
  if (be) {
    m |= 0x800000u;
    ex = (int)be - 150;
  }
  const int sh = ex + S;
  if (sh >= 0) return m << sh;  // below 2^62 by the choice of S
  return -sh >= 64 ? 0u : (m >> -sh);
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Inclusive prefix sum over the wave of values below 2^62, on DPP: three
// 25-bit limbs scanned separately (64 limbs sum below 2^31), recombined in
// 64-bit arithmetic (exact: every true prefix is below 2^64).
__device__ __forceinline__ uint64_t wave_incl_scan_u62(uint64_t x) {
  const uint32_t s0 = wave_incl_scan((uint32_t)(x & 0x1FFFFFFu));
  const uint32_t s1 = wave_incl_scan((uint32_t)((x >> 25) & 0x1FFFFFFu));
  const uint32_t s2 = wave_incl_scan((uint32_t)(x >> 50));
  return (uint64_t)s0 + ((uint64_t)s1 << 25) + ((uint64_t)s2 << 50);
}

__global__ __launch_bounds__(kSelThreads) void topp_kernel(const ToppArgs a) {
  __shared__ uint32_t h_cnt[kToppBins];
  __shared__ uint64_t h_mass[kToppBins];
  __shared__ uint32_t sm_w[kSelWaves + 1];
  __shared__ uint64_t sm_q[kSelWaves];
  __shared__ uint32_t sm_c[kSelWaves];
  __shared__ uint64_t sm_need, sm_gmass, sm_theta;
  __shared__ uint32_t sm_digit, sm_gcnt, sm_above;
  __shared__ int sm_S;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = a.pooled ? 0 : blockIdx.x;
  const int h1 = a.pooled ? a.rows : h0 + 1;
  const int64_t n = a.n;
  const int64_t tail = n - a.n_recent > 0 ? n - a.n_recent : 0;
  const int64_t nsink = a.n_sink < tail ? a.n_sink : tail;
  const int64_t c_lo = a.n_sink, c_hi = n - a.n_recent;
  const int64_t ncand = c_lo < c_hi ? c_hi - c_lo : 0;

  for (int h = h0; h < h1; ++h)
    for (int64_t i = tid; i < nsink; i += kSelThreads) a.idx[(int64_t)h * a.idx_stride + i] = (int32_t)i;

  // ---- 1. scale, fixed-point masses, total, threshold ---------------------
  uint32_t mb = 0;
  for (int h = h0; h < h1; ++h) {
    const float* s = a.score + (int64_t)h * a.score_stride;
    for (int64_t j = c_lo + tid; j < c_hi; j += kSelThreads) mb = max(mb, pos_bits(s[j]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off, 64));
  if (lane == 0) sm_w[wave] = mb;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = 0;
    for (int w = 0; w < kSelWaves; ++w) m = max(m, sm_w[w]);
    const int64_t terms = (int64_t)(h1 - h0) * ncand;
    const int lg = terms <= 1 ? 0 : 64 - __clzll((unsigned long long)(terms - 1));
    int E = 0;
    if (m >> 23) E = (int)(m >> 23) - 126;
    else if (m) E = (31 - __clz((int)m)) - 148;
    sm_S = 62 - E - lg;
  }
  __syncthreads();
  const int S = sm_S;
  auto mass_of = [&](int64_t j) -> uint64_t {  // candidate position j
    if (a.pooled) return a.mass[j - c_lo];
    return fixed_mass(a.score[(int64_t)h0 * a.score_stride + j], S);
  };
  uint64_t part = 0;
  for (int64_t j = c_lo + tid; j < c_hi; j += kSelThreads) {
    uint64_t u;
    if (a.pooled) {
      u = 0;
      for (int h = 0; h < a.rows; ++h) u += fixed_mass(a.score[(int64_t)h * a.score_stride + j], S);
      a.mass[j - c_lo] = u;
    } else {
      u = fixed_mass(a.score[(int64_t)h0 * a.score_stride + j], S);
    }
    part += u;
  }
  part = wave_sum_u64(part);
  if (lane == 0) sm_q[wave] = part;
  __syncthreads();
  if (tid == 0) {
    uint64_t U = 0;
    for (int w = 0; w < kSelWaves; ++w) U += sm_q[w];
    const unsigned __int128 prod = (unsigned __int128)a.lam_m * U;
    uint64_t theta;
    if (a.lam_sh >= 128) {
      theta = prod != 0;
    } else {
      const unsigned __int128 low = prod & ((((unsigned __int128)1) << a.lam_sh) - 1);
      theta = (uint64_t)(prod >> a.lam_sh) + (low != 0);
    }
    sm_theta = theta;
    sm_need = theta;
    sm_gmass = U;
    sm_gcnt = (uint32_t)ncand;
    sm_above = 0;
  }
  __syncthreads();  // the pooled masses written above are read back by other threads below

  // ---- 2. radix passes on the masses --------------------------------------
  uint64_t vstar = ~0ull;  // nothing is retained when theta == 0
  uint32_t take = 0, c = 0;
  if (sm_theta > 0) {
    // masses are below 2^(62 - lg) per row, times the rows summed when pooled
    const int64_t terms = (int64_t)(h1 - h0) * ncand;
    const int lg = terms <= 1 ? 0 : 64 - __clzll((unsigned long long)(terms - 1));
    const int lgr = h1 - h0 <= 1 ? 0 : 32 - __clz(h1 - h0 - 1);
    const int kb = 62 - lg + lgr < 62 ? 62 - lg + lgr : 62;
    const int passes = (kb + 7) / 8;
    uint64_t prefix = 0;
#pragma unroll 1
    for (int pass = 0; pass < passes; ++pass) {
      const int shift = 8 * (passes - 1 - pass);
      for (int b = tid; b < kToppBins; b += kSelThreads) {
        h_cnt[b] = 0u;
        h_mass[b] = 0u;
      }
      __syncthreads();
      for (int64_t j = c_lo + tid; j < c_hi; j += kSelThreads) {
        const uint64_t u = mass_of(j);
        const bool in_group = pass == 0 || (u >> (shift + 8)) == (prefix >> (shift + 8));
        const uint32_t dg = (uint32_t)(u >> shift) & 255u;
        if (in_group && dg != 0u) {
          atomicAdd(&h_cnt[dg], 1u);
          atomicAdd((unsigned long long*)&h_mass[dg], (unsigned long long)u);
        }
      }
      __syncthreads();
      // bins from the top: thread t < 256 owns bin 255 - t; bin 0 (t = 255) is
      // the group minus the others
      // read before the barrier below: the crossing thread rewrites them after it
      const uint64_t need = sm_need, gmass = sm_gmass;
      const uint32_t gcnt = sm_gcnt;
      uint64_t q = 0, qx = 0;
      uint32_t k = 0, kx = 0;
      if (wave < 4) {
        const int b = 255 - tid;
        q = b ? h_mass[b] : 0u;
        k = b ? h_cnt[b] : 0u;
        const uint64_t qs = wave_incl_scan_u62(q);
        const uint32_t ks = wave_incl_scan(k);
        if (lane == 63) {
          sm_q[wave] = qs;
          sm_c[wave] = ks;
        }
        qx = qs - q;
        kx = ks - k;
      }
      __syncthreads();
      if (wave < 4) {
        for (int w = 0; w < wave; ++w) {
          qx += sm_q[w];
          kx += sm_c[w];
        }
        if (tid == 255) {
          q = gmass - qx;
          k = gcnt - kx;
        }
        if (q > 0 && qx < need && need - qx <= q) {
          sm_digit = (uint32_t)(255 - tid);
          sm_need = need - qx;
          sm_above += kx;
          sm_gmass = q;
          sm_gcnt = k;
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sm_digit << shift;
      __syncthreads();
    }
    vstar = prefix;  // > 0: the crossing group carries mass
    const uint64_t need = sm_need;
    take = (uint32_t)((need + vstar - 1) / vstar);
    c = sm_above + take;
  }

  // ---- 3. V_R, uniform picks, ascending output ----------------------------
  const int64_t left = ncand - c;
  int64_t n_u = a.fill_mode == 0 ? a.budget - (int64_t)c : a.budget;
  n_u = n_u < 0 ? 0 : (n_u > left ? left : n_u);
  uint32_t base = (uint32_t)nsink, tie_seen = 0, left_seen = 0;
#pragma unroll 1
  for (int64_t t0 = c_lo; t0 < c_hi; t0 += kSelThreads) {
    const int64_t j = t0 + tid;
    const bool valid = j < c_hi;
    const uint64_t u = valid ? mass_of(j) : 0u;
    const bool tie = valid && u == vstar;
    uint32_t n_tie, n_left, n_out;
    const uint32_t tie_rank = tie_seen + block_flag_rank(tie, sm_w, &n_tie);
    const bool in_r = valid && (u > vstar || (tie && tie_rank < take));
    const uint32_t lr = left_seen + block_flag_rank(valid && !in_r, sm_w, &n_left);
    bool pick = false;
    if (valid && !in_r && n_u > 0) {
      const int64_t kk = ((int64_t)lr * n_u + left - 1) / left;
      pick = kk < n_u && (kk * left) / n_u == (int64_t)lr;
    }
    const bool out = in_r || pick;
    const uint32_t pos = base + block_flag_rank(out, sm_w, &n_out);
    if (out && pos < (uint64_t)a.idx_stride)
      for (int h = h0; h < h1; ++h) a.idx[(int64_t)h * a.idx_stride + pos] = (int32_t)j;
    base += n_out;
    tie_seen += n_tie;
    left_seen += n_left;
  }
  if (tid == 0)
    for (int h = h0; h < h1; ++h) {
      a.count[h] = (int32_t)base;
      if (a.count_r) a.count_r[h] = (int32_t)c;
    }
}

// Same selection for up to kRunMax candidates (Qwen2-7B video scores, 25,088
// candidates: 121 -> 55 us per row, 119 -> 77 us pooled), with every mass in
// registers:
// thread t holds candidates t, t + 1024, t + 2048, ... (coalesced loads), so
// the radix passes touch no global memory.  Index-order ranks (ties before a
// candidate, leftovers before it, outputs before it) come from one ballot per
// register slot and wave and one workgroup scan over the (slot, wave) counts
// in slot-major order, instead of three ballots and barriers per 1024
// candidates; the pick test runs in 32-bit arithmetic (every operand < 2^30).
constexpr int kRunPer = 32;
constexpr int kRunMax = kSelThreads * kRunPer;

__global__ __launch_bounds__(kSelThreads) void topp_run_kernel(const ToppArgs a) {
  __shared__ uint32_t h_cnt[kToppBins];
  __shared__ uint64_t h_mass[kToppBins];
  __shared__ uint32_t sm_w[kSelWaves + 1];
  __shared__ uint64_t sm_q[kSelWaves];
  __shared__ uint32_t sm_c[kSelWaves];
  __shared__ uint64_t sm_need, sm_gmass, sm_theta;
  __shared__ uint32_t sm_digit, sm_gcnt, sm_above;
  __shared__ int sm_S;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = a.pooled ? 0 : blockIdx.x;
  const int h1 = a.pooled ? a.rows : h0 + 1;
  const int64_t n = a.n;
  const int64_t tail = n - a.n_recent > 0 ? n - a.n_recent : 0;
  const int64_t nsink = a.n_sink < tail ? a.n_sink : tail;
  const int64_t c_lo = a.n_sink, c_hi = n - a.n_recent;
  const int ncand = c_lo < c_hi ? (int)(c_hi - c_lo) : 0;  // <= kRunMax
  const int R = (ncand + kSelThreads - 1) / kSelThreads;  // register slots in use
  // slot u holds candidate tid + 1024 u (position c_lo + that), if below ncand
  auto valid = [&](int u) { return u < R && tid + kSelThreads * u < ncand; };

  for (int h = h0; h < h1; ++h)
    for (int64_t i = tid; i < nsink; i += kSelThreads) a.idx[(int64_t)h * a.idx_stride + i] = (int32_t)i;

  // ---- 1. scale, fixed-point masses, total, threshold ---------------------
  uint32_t mb = 0;
  for (int h = h0; h < h1; ++h) {
    const float* s = a.score + (int64_t)h * a.score_stride + c_lo + tid;
#pragma unroll
    for (int u = 0; u < kRunPer; ++u)
      if (valid(u)) mb = max(mb, pos_bits(s[kSelThreads * u]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off, 64));
  if (lane == 0) sm_w[wave] = mb;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = 0;
    for (int w = 0; w < kSelWaves; ++w) m = max(m, sm_w[w]);
    const int64_t terms = (int64_t)(h1 - h0) * ncand;
    const int lg = terms <= 1 ? 0 : 64 - __clzll((unsigned long long)(terms - 1));
    int E = 0;
    if (m >> 23) E = (int)(m >> 23) - 126;
    else if (m) E = (31 - __clz((int)m)) - 148;
    sm_S = 62 - E - lg;
  }
  __syncthreads();
  const int S = sm_S;
  uint64_t mass[kRunPer];
#pragma unroll
  for (int u = 0; u < kRunPer; ++u) mass[u] = 0u;
  for (int h = h0; h < h1; ++h) {
    const float* s = a.score + (int64_t)h * a.score_stride + c_lo + tid;
#pragma unroll
    for (int u = 0; u < kRunPer; ++u)
      if (valid(u)) mass[u] += fixed_mass(s[kSelThreads * u], S);
  }
  uint64_t part = 0;
#pragma unroll
  for (int u = 0; u < kRunPer; ++u) part += mass[u];
  part = wave_sum_u64(part);
  if (lane == 0) sm_q[wave] = part;
  __syncthreads();
  if (tid == 0) {
    uint64_t U = 0;
    for (int w = 0; w < kSelWaves; ++w) U += sm_q[w];
    const unsigned __int128 prod = (unsigned __int128)a.lam_m * U;
    uint64_t theta;
    if (a.lam_sh >= 128) {
      theta = prod != 0;
    } else {
      const unsigned __int128 low = prod & ((((unsigned __int128)1) << a.lam_sh) - 1);
      theta = (uint64_t)(prod >> a.lam_sh) + (low != 0);
    }
    sm_theta = theta;
    sm_need = theta;
    sm_gmass = U;
    sm_gcnt = (uint32_t)ncand;
    sm_above = 0;
  }
  __syncthreads();

  // ---- 2. radix passes on the masses (in registers) -------------------------
  uint64_t vstar = ~0ull;  // nothing is retained when theta == 0
  uint32_t take = 0, c = 0;
  if (sm_theta > 0) {
    const int64_t terms = (int64_t)(h1 - h0) * ncand;
    const int lg = terms <= 1 ? 0 : 64 - __clzll((unsigned long long)(terms - 1));
    const int lgr = h1 - h0 <= 1 ? 0 : 32 - __clz(h1 - h0 - 1);
    const int kb = 62 - lg + lgr < 62 ? 62 - lg + lgr : 62;
    const int passes = (kb + 7) / 8;
    uint64_t prefix = 0;
#pragma unroll 1
    for (int pass = 0; pass < passes; ++pass) {
      const int shift = 8 * (passes - 1 - pass);
      for (int b = tid; b < kToppBins; b += kSelThreads) {
        h_cnt[b] = 0u;
        h_mass[b] = 0u;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kRunPer; ++u) {
        const uint64_t m = mass[u];
        const bool in_group = pass == 0 || (m >> (shift + 8)) == (prefix >> (shift + 8));
        const uint32_t dg = (uint32_t)(m >> shift) & 255u;
        if (valid(u) && in_group && dg != 0u) {
          atomicAdd(&h_cnt[dg], 1u);
          atomicAdd((unsigned long long*)&h_mass[dg], (unsigned long long)m);
        }
      }
      __syncthreads();
      // bins from the top: thread t < 256 owns bin 255 - t; bin 0 (t = 255) is
      // the group minus the others; read before the barrier below (the
      // crossing thread rewrites them after it)
      const uint64_t need = sm_need, gmass = sm_gmass;
      const uint32_t gcnt = sm_gcnt;
      uint64_t q = 0, qx = 0;
      uint32_t k = 0, kx = 0;
      if (wave < 4) {
        const int b = 255 - tid;
        q = b ? h_mass[b] : 0u;
        k = b ? h_cnt[b] : 0u;
        const uint64_t qs = wave_incl_scan_u62(q);
        const uint32_t ks = wave_incl_scan(k);
        if (lane == 63) {
          sm_q[wave] = qs;
          sm_c[wave] = ks;
        }
        qx = qs - q;
        kx = ks - k;
      }
      __syncthreads();
      if (wave < 4) {
        for (int w = 0; w < wave; ++w) {
          qx += sm_q[w];
          kx += sm_c[w];
        }
        if (tid == 255) {
          q = gmass - qx;
          k = gcnt - kx;
        }
        if (q > 0 && qx < need && need - qx <= q) {
          sm_digit = (uint32_t)(255 - tid);
          sm_need = need - qx;
          sm_above += kx;
          sm_gmass = q;
          sm_gcnt = k;
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sm_digit << shift;
      __syncthreads();
    }
    vstar = prefix;  // > 0: the crossing group carries mass
    const uint64_t need = sm_need;
    take = (uint32_t)((need + vstar - 1) / vstar);
    c = sm_above + take;
  }

  // ---- 3. V_R, uniform picks, ascending output ----------------------------
  // exclusive index-order rank of every slot's flag: one ballot per slot and
  // wave, one scan over the (slot, wave) counts in slot-major order into tab;
  // a slot's rank is then tab[slot][wave] plus its lanes below in the ballot
  __shared__ uint32_t tab[kRunPer * kSelWaves];
  auto flag_scan = [&](uint32_t bits) -> uint32_t {
    __syncthreads();  // the previous scan's tab is no longer read
#pragma unroll
    for (int u = 0; u < kRunPer; ++u) {
      if (u < R) {  // uniform
        const uint64_t bb = __ballot((bits >> u) & 1u);
        if (lane == 0) tab[u * kSelWaves + wave] = (uint32_t)__popcll(bb);
      }
    }
    __syncthreads();
    const uint32_t v = tid < R * kSelWaves ? tab[tid] : 0u;
    uint32_t total;
    const uint32_t ex = block_excl_scan(v, sm_w, &total);  // ends with a barrier
    if (tid < R * kSelWaves) tab[tid] = ex;
    __syncthreads();
    return total;
  };
  auto slot_rank = [&](uint32_t bits, int u) -> uint32_t {
    const uint64_t bb = __ballot((bits >> u) & 1u);
    return tab[u * kSelWaves + wave] +
           __builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0u));
  };
  uint32_t tie_bits = 0;
#pragma unroll
  for (int u = 0; u < kRunPer; ++u)
    if (valid(u) && mass[u] == vstar) tie_bits |= 1u << u;
  flag_scan(tie_bits);
  uint32_t in_bits = 0;
#pragma unroll
  for (int u = 0; u < kRunPer; ++u) {
    if (u < R) {  // uniform: every lane takes part in the ballot
      const uint32_t r = slot_rank(tie_bits, u);
      if (valid(u) && (mass[u] > vstar || (((tie_bits >> u) & 1u) && r < take))) in_bits |= 1u << u;
    }
  }
  uint32_t left_bits = 0;
#pragma unroll
  for (int u = 0; u < kRunPer; ++u)
    if (valid(u) && !((in_bits >> u) & 1u)) left_bits |= 1u << u;
  const uint32_t left = (uint32_t)ncand - c;
  int64_t n_u64 = a.fill_mode == 0 ? a.budget - (int64_t)c : a.budget;
  n_u64 = n_u64 < 0 ? 0 : (n_u64 > (int64_t)left ? (int64_t)left : n_u64);
  const uint32_t n_u = (uint32_t)n_u64;
  uint32_t out_bits = in_bits;
  if (n_u > 0) {
    flag_scan(left_bits);
    // leftover rank lr is picked when kk = ceil(lr n_u / left) < n_u and
    // kk left < (lr + 1) n_u (i.e. floor(kk left / n_u) == lr); every product
    // is below 2^30.  The quotient comes from a double reciprocal and is made
    // exact by one correction each way.
    const double inv_left = 1.0 / (double)left;
#pragma unroll
    for (int u = 0; u < kRunPer; ++u) {
      if (u < R) {
        const uint32_t lr = slot_rank(left_bits, u);
        if ((left_bits >> u) & 1u) {
          const uint32_t t = lr * n_u;
          uint32_t fl = (uint32_t)((double)t * inv_left);  // floor(t / left), maybe off by one
          if ((fl + 1) * left <= t) ++fl;
          if (fl * left > t) --fl;
          const uint32_t kk = fl + (fl * left != t ? 1u : 0u);
          if (kk < n_u && kk * left < (lr + 1) * n_u) out_bits |= 1u << u;
        }
      }
    }
  }
  const uint32_t n_total = flag_scan(out_bits);
#pragma unroll
  for (int u = 0; u < kRunPer; ++u) {
    if (u < R) {
      const uint32_t pos = (uint32_t)nsink + slot_rank(out_bits, u);
      if (((out_bits >> u) & 1u) && pos < (uint64_t)a.idx_stride)
        for (int h = h0; h < h1; ++h)
          a.idx[(int64_t)h * a.idx_stride + pos] = (int32_t)(c_lo + tid + kSelThreads * u);
    }
  }
  if (tid == 0)
    for (int h = h0; h < h1; ++h) {
      a.count[h] = (int32_t)(nsink + n_total);
      if (a.count_r) a.count_r[h] = (int32_t)c;
    }
}

}  // namespace

hipError_t launch_select_topp(const ToppArgs& a, hipStream_t s) {
  const int64_t ncand = a.n - a.n_sink - a.n_recent;
  if (ncand <= kRunMax)
    hipLaunchKernelGGL(topp_run_kernel, dim3(a.pooled ? 1 : a.rows), dim3(kSelThreads), 0, s, a);
  else
    hipLaunchKernelGGL(topp_kernel, dim3(a.pooled ? 1 : a.rows), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace skv
