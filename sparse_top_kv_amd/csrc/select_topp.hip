// select_topp.hip -- verifier-guided two-stage selection (SpecVLM blog, "The
// SpecVLM Method": Stage I top-P retention, Stage II spatially uniform
// reduction).
//
// One 1024-thread workgroup per selection: a score row (kv head), or, pooled,
// one row of per-token sums over all rows (the blog averages the verifier's
// attention over layers and heads; the constant factor is dropped).  Pooled,
// a token's score is its rows added in double in ascending row order and
// rounded to the nearest fp32 (saturating at the largest finite fp32).
//
// Stage I is exact.  Candidates are ordered by the fp32 score a (descending,
// index ascending); c is the smallest count whose prefix mass reaches
// lambda times the total, compared without rounding.  Every fp32 a >= 0 is
// M 2^(e' - 150) with e the biased exponent, e' = max(e, 1) and M the 24-bit
// significand, i.e. an integer multiple M 2^(e' - 1) of the unit 2^-149:
//   1. histogram over the exponent e (bits 30..23 of a): count and sum of M per
//      bin, exact in 64 bits (M < 2^24, at most 2^31 candidates);
//   2. one wave scans the bins from the top in 384-bit integer arithmetic:
//      total U, theta = ceil(lambda U) (lambda = lam_m / 2^lam_sh exactly), the
//      bin e1 where the running mass reaches theta, and what that bin still
//      has to supply, ceil((theta - P) / 2^(e1' - 1)) in units of M;
//   3. three 8-bit radix passes over M inside bin e1, with per-bin count and
//      M-sum histograms, find the significand M* of the entry that crosses;
//      `take` entries equal to it are kept, lowest index first;
//   4. one pass in index order: V_R membership (a > a*, or a == a* within the
//      first `take` ties), the leftover rank of every other candidate, the
//      uniform picks at leftover ranks floor(i L / n_U), and the ascending
//      output.
// Zero scores carry no mass and are left out of every histogram.
#include <float.h>

#include "skv_block.h"
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

constexpr int kToppBins = 256;

__device__ __forceinline__ uint32_t pos_bits(float x) { return x > 0.0f ? __float_as_uint(x) : 0u; }

// Score bits of candidate position j of a pooled selection.
__device__ __forceinline__ uint32_t pooled_bits(const ToppArgs& a, int64_t j) {
  double s = 0.0;
  for (int h = 0; h < a.rows; ++h) s = s + (double)a.score[(int64_t)h * a.score_stride + j];
  float f = (float)s;
  if (f == __builtin_huge_valf()) f = FLT_MAX;
  return pos_bits(f);
}

// 24-bit significand of positive fp32 bits b (no implicit one for subnormals).
__device__ __forceinline__ uint32_t sig_of(uint32_t b) {
  return (b & 0x7fffffu) | ((b >> 23) ? 0x800000u : 0u);
}
// log2 of the unit of exponent bin e's significands, in units of 2^-149.
__device__ __forceinline__ int unit_shift(int e) { return (e ? e : 1) - 1; }

// 384-bit unsigned integer (little-endian 64-bit limbs): holds every total
// (below 2^311) and lambda times it (below 2^365).
struct Wide {
  uint64_t w[6];
};

__device__ __forceinline__ void wide_zero(Wide& x) {
#pragma unroll
  for (int i = 0; i < 6; ++i) x.w[i] = 0u;
}

// x += v 2^sh, 0 <= sh < 320.
__device__ __forceinline__ void wide_add_shl(Wide& x, uint64_t v, int sh) {
  const int li = sh >> 6, bo = sh & 63;
  const uint64_t lo = v << bo, hi = bo ? v >> (64 - bo) : 0u;
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const uint64_t add = i == li ? lo : (i == li + 1 ? hi : 0u);
    const uint64_t t = x.w[i] + add;
    const uint64_t c1 = t < add;
    const uint64_t t2 = t + carry;
    const uint64_t c2 = t2 < carry;
    x.w[i] = t2;
    carry = c1 | c2;
  }
}

__device__ __forceinline__ int wide_cmp(const Wide& a, const Wide& b) {
  for (int i = 5; i >= 0; --i)
    if (a.w[i] != b.w[i]) return a.w[i] < b.w[i] ? -1 : 1;
  return 0;
}

// a - b for a >= b.
__device__ __forceinline__ Wide wide_sub(const Wide& a, const Wide& b) {
  Wide r;
  uint64_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const uint64_t t = a.w[i] - b.w[i];
    const uint64_t b1 = a.w[i] < b.w[i];
    r.w[i] = t - borrow;
    borrow = b1 | (t < borrow);
  }
  return r;
}

// ceil(x / 2^sh) for 0 <= sh < 384 (the caller knows the result fits in the
// returned limbs: all of them for theta, the lowest for a bin's need).
__device__ __forceinline__ Wide wide_shr_ceil(const Wide& x, int sh) {
  Wide r;
  wide_zero(r);
  const int ls = sh >> 6, bs = sh & 63;
  bool rem = false;
  for (int i = 0; i < 6; ++i)
    if (i < ls) rem = rem || x.w[i] != 0u;
  if (bs && ls < 6) rem = rem || (x.w[ls] << (64 - bs)) != 0u;
  for (int i = 0; i < 6; ++i) {
    const int s0 = i + ls;
    const uint64_t lo = s0 < 6 ? x.w[s0] : 0u, hi = s0 + 1 < 6 ? x.w[s0 + 1] : 0u;
    r.w[i] = bs ? (lo >> bs) | (hi << (64 - bs)) : lo;
  }
  if (rem) wide_add_shl(r, 1u, 0);
  return r;
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

constexpr int kSub = 16;  // private copies of every histogram bin

// Shared state of the Stage I passes.
struct ToppShared {
  uint32_t s_cnt[kToppBins * kSub];   // pass histograms, kSub copies per bin
  uint64_t s_mass[kToppBins * kSub];
  uint32_t h_cnt[kToppBins];          // their sums per bin
  uint64_t h_mass[kToppBins];
  uint64_t sq[kSelWaves];
  uint32_t sc[kSelWaves];
  uint64_t need;    // mass still to supply, in units of the current group's significands
  uint32_t above;   // candidates ordered before the current group
  uint32_t digit;
  int e1;           // exponent bin of the crossing entry; -1: nothing is retained
};

__device__ __forceinline__ void topp_clear_hist(ToppShared& sh) {
  for (int i = threadIdx.x; i < kToppBins * kSub; i += blockDim.x) {
    sh.s_cnt[i] = 0u;
    sh.s_mass[i] = 0u;
  }
}
// After a histogram pass (and a barrier): the per-bin sums of the copies.
__device__ __forceinline__ void topp_sum_sub(ToppShared& sh) {
  for (int b = threadIdx.x; b < kToppBins; b += blockDim.x) {
    uint32_t c = 0;
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < kSub; ++k) {
      c += sh.s_cnt[b * kSub + k];
      m += sh.s_mass[b * kSub + k];
    }
    sh.h_cnt[b] = c;
    sh.h_mass[b] = m;
  }
}

__device__ __forceinline__ Wide wide_add(const Wide& a, const Wide& b) {
  Wide r;
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const uint64_t t = a.w[i] + b.w[i];
    const uint64_t c1 = t < a.w[i];
    r.w[i] = t + carry;
    carry = c1 | (r.w[i] < carry);
  }
  return r;
}

// ceil(lam_m U / 2^lam_sh); lam_m < 2^54 keeps the product in 384 bits.
__device__ __forceinline__ Wide topp_theta(const Wide& U, uint64_t lam_m, int lam_sh) {
  Wide prod;
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const unsigned __int128 t = (unsigned __int128)U.w[i] * lam_m + carry;
    prod.w[i] = (uint64_t)t;
    carry = (uint64_t)(t >> 64);
  }
  if (lam_sh < 384) return wide_shr_ceil(prod, lam_sh);
  Wide theta;
  wide_zero(theta);
  bool nz = false;
#pragma unroll
  for (int i = 0; i < 6; ++i) nz = nz || prod.w[i] != 0u;
  theta.w[0] = nz ? 1u : 0u;
  return theta;
}

// Step 2 (after the exponent histogram), on wave 0: lane i owns exponent
// bins 255 - 4 i - k, k = 0..3, so lane order is descending exponent.  Each
// lane adds its bins' masses exactly (384 bits), a six-step shuffle scan
// gives every lane the mass of all bins above and including its own, every
// lane forms theta from the total, and the one lane whose range crosses
// theta walks its four bins.
__device__ __forceinline__ void topp_walk_exponents(ToppShared& sh, uint64_t lam_m, int lam_sh) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  Wide mine;
  wide_zero(mine);
  uint32_t cnt = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = 255 - 4 * lane - k;
    const uint64_t m = sh.h_mass[e];
    if (m) wide_add_shl(mine, m, unit_shift(e));
    cnt += sh.h_cnt[e];
  }
  Wide incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    Wide o;
#pragma unroll
    for (int i = 0; i < 6; ++i) o.w[i] = __shfl_up(incl.w[i], off, 64);
    if (lane >= off) incl = wide_add(incl, o);
  }
  const uint32_t cincl = wave_incl_scan(cnt);
  Wide U;
#pragma unroll
  for (int i = 0; i < 6; ++i) U.w[i] = __shfl(incl.w[i], 63, 64);
  const Wide theta = topp_theta(U, lam_m, lam_sh);
  bool tz = true;
#pragma unroll
  for (int i = 0; i < 6; ++i) tz = tz && theta.w[i] == 0u;
  if (tz) {  // the empty prefix already reaches lambda U: nothing is retained
    if (lane == 0) {
      sh.e1 = -1;
      sh.need = 0;
      sh.above = 0;
    }
    return;
  }
  Wide P = wide_sub(incl, mine);  // mass of every bin above this lane's
  if (!(wide_cmp(P, theta) < 0 && wide_cmp(theta, incl) <= 0)) return;
  uint32_t above = cincl - cnt;
  for (int k = 0; k < 4; ++k) {
    const int e = 255 - 4 * lane - k;
    const uint64_t m = sh.h_mass[e];
    if (!m) continue;
    Wide Pn = P;
    wide_add_shl(Pn, m, unit_shift(e));
    if (wide_cmp(Pn, theta) >= 0) {
      sh.e1 = e;
      sh.need = wide_shr_ceil(wide_sub(theta, P), unit_shift(e)).w[0];
      sh.above = above;
      return;
    }
    P = Pn;
    above += sh.h_cnt[e];
  }
}

// Step 3, the scan of one radix pass over the significands of the current
// group (histograms filled): thread t < 256 owns bin 255 - t; the bin where
// the running mass from the top reaches `need` becomes the next digit.
__device__ __forceinline__ void topp_pick_digit(ToppShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t need = sh.need;  // read before the barrier below: rewritten after it
  uint64_t q = 0, qx = 0;
  uint32_t k = 0, kx = 0;
  if (wave < 4) {
    const int b = 255 - tid;
    q = sh.h_mass[b];
    k = sh.h_cnt[b];
    const uint64_t qs = wave_incl_scan_u62(q);
    const uint32_t ks = wave_incl_scan(k);
    if (lane == 63) {
      sh.sq[wave] = qs;
      sh.sc[wave] = ks;
    }
    qx = qs - q;
    kx = ks - k;
  }
  __syncthreads();
  if (wave < 4) {
    for (int w = 0; w < wave; ++w) {
      qx += sh.sq[w];
      kx += sh.sc[w];
    }
    if (q > 0 && qx < need && need - qx <= q) {
      sh.digit = (uint32_t)(255 - tid);
      sh.need = need - qx;
      sh.above += kx;
    }
  }
  __syncthreads();
}

// Histogram updates.  Scores cluster in a few exponent (and leading-
// significand) bins, and LDS atomics on one address serialise, so every bin
// has kSub private copies (lane bits 0-1 and wave bits 0-1 pick one), stored
// side by side so a bin's copies sit in distinct banks; topp_sum_sub adds
// them up after the pass (integer sums: the result is exact and ordered).
__device__ __forceinline__ int topp_sub() { return (threadIdx.x & 3) | (((threadIdx.x >> 6) & 3) << 2); }
__device__ __forceinline__ void topp_add(ToppShared& sh, uint32_t bin, uint32_t sig) {
  const int i = (int)bin * kSub + topp_sub();
  atomicAdd(&sh.s_cnt[i], 1u);
  atomicAdd((unsigned long long*)&sh.s_mass[i], (unsigned long long)sig);
}
// Exponent histogram: every positive value into its exponent bin.
__device__ __forceinline__ void topp_add_exp(ToppShared& sh, uint32_t b) {
  if (b) topp_add(sh, b >> 23, sig_of(b));
}
// Significand histogram of exponent bin e1: the values whose significand
// matches `prefix` above bit shift + 8, by the significand digit at `shift`.
__device__ __forceinline__ void topp_add_sig(ToppShared& sh, uint32_t b, int e1, int shift, uint32_t prefix) {
  const uint32_t m = sig_of(b);
  if (b && (int)(b >> 23) == e1 && (m >> (shift + 8)) == (prefix >> (shift + 8)))
    topp_add(sh, (m >> shift) & 255u, m);
}

// Rows of any length: the scores are re-read from memory in every pass (the
// pooled row is written once to the scratch a.pooled_row and re-read).
__global__ __launch_bounds__(kSelThreads) void topp_kernel(const ToppArgs a) {
  __shared__ ToppShared sh;
  __shared__ uint32_t sm_w[kSelWaves + 1];

  const int tid = threadIdx.x;
  const int h0 = a.pooled ? 0 : blockIdx.x;
  const int h1 = a.pooled ? a.rows : h0 + 1;
  const int64_t n = a.n;
  const int64_t tail = n - a.n_recent > 0 ? n - a.n_recent : 0;
  const int64_t nsink = a.n_sink < tail ? a.n_sink : tail;
  const int64_t c_lo = a.n_sink, c_hi = n - a.n_recent;
  const int64_t ncand = c_lo < c_hi ? c_hi - c_lo : 0;

  for (int h = h0; h < h1; ++h)
    for (int64_t i = tid; i < nsink; i += kSelThreads) a.idx[(int64_t)h * a.idx_stride + i] = (int32_t)i;

  if (a.pooled) {
    for (int64_t j = c_lo + tid; j < c_hi; j += kSelThreads) a.pooled_row[j - c_lo] = pooled_bits(a, j);
  }
  topp_clear_hist(sh);
  __syncthreads();  // the pooled row written above is read back by other threads
  auto bits_of = [&](int64_t j) -> uint32_t {  // candidate position j
    if (a.pooled) return a.pooled_row[j - c_lo];
    return pos_bits(a.score[(int64_t)h0 * a.score_stride + j]);
  };

  // ---- 1-2. exponent histogram, then the walk over the exponent bins -------
  for (int64_t j = c_lo + tid; j < c_hi; j += kSelThreads) topp_add_exp(sh, bits_of(j));
  __syncthreads();
  topp_sum_sub(sh);
  __syncthreads();
  topp_walk_exponents(sh, a.lam_m, a.lam_sh);
  __syncthreads();

  // ---- 3. radix passes over the significands of bin e1 ---------------------
  const int e1 = sh.e1;
  uint32_t vbits = 0xFFFFFFFFu;  // nothing is retained when e1 < 0
  uint32_t take = 0, c = 0;
  if (e1 >= 0) {
    uint32_t prefix = 0;
#pragma unroll 1
    for (int shift = 16; shift >= 0; shift -= 8) {
      topp_clear_hist(sh);
      __syncthreads();
      for (int64_t j = c_lo + tid; j < c_hi; j += kSelThreads) topp_add_sig(sh, bits_of(j), e1, shift, prefix);
      __syncthreads();
      topp_sum_sub(sh);
      __syncthreads();
      topp_pick_digit(sh);
      prefix |= sh.digit << shift;
    }
    vbits = ((uint32_t)e1 << 23) | (prefix & 0x7fffffu);
    take = (uint32_t)((sh.need + prefix - 1) / prefix);  // prefix = M* > 0
    c = sh.above + take;
  }

  // ---- 4. V_R, uniform picks, ascending output ----------------------------
  const int64_t left = ncand - c;
  int64_t n_u = a.fill_mode == 0 ? a.budget - (int64_t)c : a.budget;
  n_u = n_u < 0 ? 0 : (n_u > left ? left : n_u);
  uint32_t base = (uint32_t)nsink, tie_seen = 0, left_seen = 0;
#pragma unroll 1
  for (int64_t t0 = c_lo; t0 < c_hi; t0 += kSelThreads) {
    const int64_t j = t0 + tid;
    const bool valid = j < c_hi;
    const uint32_t b = valid ? bits_of(j) : 0u;
    const bool tie = valid && b == vbits;
    uint32_t n_tie, n_left, n_out;
    const uint32_t tie_rank = tie_seen + block_flag_rank(tie, sm_w, &n_tie);
    const bool in_r = valid && e1 >= 0 && (b > vbits || (tie && tie_rank < take));
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
// candidates per row) with every score in registers: thread t holds
// candidates t, t + 1024, t + 2048, ... (coalesced loads), so the passes touch
// no global memory.  Index-order ranks (ties before a candidate, leftovers
// before it, outputs before it) come from one ballot per register slot and
// wave and one workgroup scan over the (slot, wave) counts in slot-major
// order; the pick test runs in 32-bit arithmetic (every operand < 2^30).
constexpr int kRunPer = 32;
constexpr int kRunMax = kSelThreads * kRunPer;

__global__ __launch_bounds__(kSelThreads) void topp_run_kernel(const ToppArgs a) {
  __shared__ ToppShared sh;
  __shared__ uint32_t sm_w[kSelWaves + 1];

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

  uint32_t bits[kRunPer];
#pragma unroll
  for (int u = 0; u < kRunPer; ++u) {
    bits[u] = 0u;
    if (valid(u)) {
      const int64_t j = c_lo + tid + (int64_t)kSelThreads * u;
      bits[u] = a.pooled ? pooled_bits(a, j) : pos_bits(a.score[(int64_t)h0 * a.score_stride + j]);
    }
  }
  topp_clear_hist(sh);
  __syncthreads();

  // ---- 1-2. exponent histogram, then the walk over the exponent bins -------
#pragma unroll
  for (int u = 0; u < kRunPer; ++u) topp_add_exp(sh, bits[u]);  // invalid slots hold 0
  __syncthreads();
  topp_sum_sub(sh);
  __syncthreads();
  topp_walk_exponents(sh, a.lam_m, a.lam_sh);
  __syncthreads();

  // ---- 3. radix passes over the significands of bin e1 ---------------------
  const int e1 = sh.e1;
  uint32_t vbits = 0xFFFFFFFFu;  // nothing is retained when e1 < 0
  uint32_t take = 0, c = 0;
  if (e1 >= 0) {
    uint32_t prefix = 0;
#pragma unroll 1
    for (int shift = 16; shift >= 0; shift -= 8) {
      topp_clear_hist(sh);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kRunPer; ++u) topp_add_sig(sh, bits[u], e1, shift, prefix);
      __syncthreads();
      topp_sum_sub(sh);
      __syncthreads();
      topp_pick_digit(sh);
      prefix |= sh.digit << shift;
    }
    vbits = ((uint32_t)e1 << 23) | (prefix & 0x7fffffu);
    take = (uint32_t)((sh.need + prefix - 1) / prefix);  // prefix = M* > 0
    c = sh.above + take;
  }

  // ---- 4. V_R, uniform picks, ascending output ----------------------------
  // exclusive index-order rank of every slot's flag: one ballot per slot and
  // wave, one scan over the (slot, wave) counts in slot-major order into tab;
  // a slot's rank is then tab[slot][wave] plus its lanes below in the ballot
  __shared__ uint32_t tab[kRunPer * kSelWaves];
  auto flag_scan = [&](uint32_t fl) -> uint32_t {
    __syncthreads();  // the previous scan's tab is no longer read
#pragma unroll
    for (int u = 0; u < kRunPer; ++u) {
      if (u < R) {  // uniform
        const uint64_t bb = __ballot((fl >> u) & 1u);
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
  auto slot_rank = [&](uint32_t fl, int u) -> uint32_t {
    const uint64_t bb = __ballot((fl >> u) & 1u);
    return tab[u * kSelWaves + wave] +
           __builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0u));
  };
  uint32_t tie_bits = 0;
#pragma unroll
  for (int u = 0; u < kRunPer; ++u)
    if (valid(u) && bits[u] == vbits) tie_bits |= 1u << u;
  flag_scan(tie_bits);
  uint32_t in_bits = 0;
#pragma unroll
  for (int u = 0; u < kRunPer; ++u) {
    if (u < R) {  // uniform: every lane takes part in the ballot
      const uint32_t r = slot_rank(tie_bits, u);
      if (valid(u) && e1 >= 0 && (bits[u] > vbits || (((tie_bits >> u) & 1u) && r < take)))
        in_bits |= 1u << u;
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
