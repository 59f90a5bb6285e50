// skv_oracle.cpp -- plain fp64 CPU oracle for sparse top-K KV decode attention.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
// this file: only the tests, the smoke check and the bench's CPU-baseline leg do.
// It shares no source, header, helper or table with the HIP library.
//
// Every step below is the plain definition written out in fp64, looping in
// ascending index order.  Sources (web pages, by title and section):
//   [StD]  "Sparse-to-Dense: A Free Lunch for Lossless Acceleration of Video
//          Understanding in LLMs" -- Sec. 3.1 Decoding Procedures, Sec. 3.2 Model
//          with Sparse Attention (the Cache_s[l] equation and the GQA sentence),
//          Sec. 3.3 I/O complexity analysis, App. A Preliminary.
//   [BX]   "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
//          -- "Speedup Across Context" (SnapKV-style scoring, four sinks, split-K
//          decoding) and the header figure (sinks + scored history + recent run).
//   [SMM]  blog on SparseMM ("Head Sparsity Emerges from Visual Concept Responses
//          in MLLMs") -- the method section: Local Window Cache, Uniform-Based
//          Cache, Score-Preferred Cache, and the observation-window top-K.
//
// Numeric contract: bf16 is decoded by placing its 16 bits in the high half of
// an IEEE binary32 word (exact), fp32 is widened exactly, and everything after
// that is fp64.  The only export in fp32 is the score array (round to nearest).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

enum { ORA_F32 = 0, ORA_BF16 = 1 };

struct OraProblem {
  int32_t n_q_heads;   // Hq
  int32_t n_kv_heads;  // Hkv; query head g reads kv head g / (Hq/Hkv)
  int32_t head_dim;    // d
  int32_t dtype;       // ORA_F32 or ORA_BF16 for q, K and V
  float scale;         // softmax scale applied to q.k (used as (double)scale)
  int32_t pad_;
  int64_t kv_head_stride;  // elements between kv heads
  int64_t kv_pos_stride;   // elements between positions
};

double load(int dtype, const void* base, int64_t off) {
  if (dtype == ORA_F32) return (double)((const float*)base)[off];
  uint32_t u = (uint32_t)((const uint16_t*)base)[off] << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Run fn(i) for i in [0, count) on up to nthreads threads, static partition.
template <class Fn>
void parallel_for(int64_t count, int nthreads, Fn fn) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > count) nthreads = (int)std::max<int64_t>(count, 1);
  if (nthreads == 1) {
    for (int64_t i = 0; i < count; ++i) fn(i);
    return;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < nthreads; ++t) {
    pool.emplace_back([=, &fn]() {
      for (int64_t i = t; i < count; i += nthreads) fn(i);
    });
  }
  for (auto& th : pool) th.join();
}

// One query row decoded to fp64.
std::vector<double> query_row(const OraProblem& p, const void* q, int64_t row,
                              int g) {
  std::vector<double> out(p.head_dim);
  const int64_t base = (row * p.n_q_heads + g) * (int64_t)p.head_dim;
  for (int t = 0; t < p.head_dim; ++t) out[t] = load(p.dtype, q, base + t);
  return out;
}

// Logit l(j) = scale * sum_t q_t k_{h,j,t} for the positions in `pos`
// (the scaled dot product of standard attention; the scale is an argument).
// Four keys are evaluated side by side for speed; each dot product is still
// summed over t in ascending order.
void logits(const OraProblem& p, const std::vector<double>& qv, const void* k,
            int h, const int64_t* pos, int64_t npos, double* out) {
  const double sc = (double)p.scale;
  const int d = p.head_dim;
  const int64_t hb = (int64_t)h * p.kv_head_stride;
  int64_t i = 0;
  for (; i + 4 <= npos; i += 4) {
    const int64_t b0 = hb + pos[i] * p.kv_pos_stride;
    const int64_t b1 = hb + pos[i + 1] * p.kv_pos_stride;
    const int64_t b2 = hb + pos[i + 2] * p.kv_pos_stride;
    const int64_t b3 = hb + pos[i + 3] * p.kv_pos_stride;
    double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    for (int t = 0; t < d; ++t) {
      a0 += qv[t] * load(p.dtype, k, b0 + t);
      a1 += qv[t] * load(p.dtype, k, b1 + t);
      a2 += qv[t] * load(p.dtype, k, b2 + t);
      a3 += qv[t] * load(p.dtype, k, b3 + t);
    }
    out[i] = sc * a0;
    out[i + 1] = sc * a1;
    out[i + 2] = sc * a2;
    out[i + 3] = sc * a3;
  }
  for (; i < npos; ++i) {
    const int64_t b0 = hb + pos[i] * p.kv_pos_stride;
    double a0 = 0;
    for (int t = 0; t < d; ++t) a0 += qv[t] * load(p.dtype, k, b0 + t);
    out[i] = sc * a0;
  }
}

// Exact softmax attention of one query row over the ordered key set `pos`:
//   m = max l, Z = sum exp(l - m), o = sum exp(l - m) v / Z, lse = m + ln Z.
// An empty set gives o = 0 and lse = -inf (the identity of the log-sum-exp merge).
void attend_row(const OraProblem& p, const std::vector<double>& qv, const void* k,
                const void* v, int h, const std::vector<int64_t>& pos,
                double* o, double* lse) {
  const int d = p.head_dim;
  const int64_t npos = (int64_t)pos.size();
  if (npos == 0) {
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    *lse = -std::numeric_limits<double>::infinity();
    return;
  }
  std::vector<double> l(npos);
  logits(p, qv, k, h, pos.data(), npos, l.data());
  double m = l[0];
  for (int64_t i = 1; i < npos; ++i) m = std::max(m, l[i]);
  double z = 0.0;
  std::vector<double> acc(d, 0.0);
  const int64_t hb = (int64_t)h * p.kv_head_stride;
  for (int64_t i = 0; i < npos; ++i) {
    const double w = std::exp(l[i] - m);
    z += w;
    const int64_t vb = hb + pos[i] * p.kv_pos_stride;
    for (int t = 0; t < d; ++t) acc[t] += w * load(p.dtype, v, vb + t);
  }
  for (int t = 0; t < d; ++t) o[t] = acc[t] / z;
  *lse = m + std::log(z);
}

bool problem_ok(const OraProblem* p) {
  return p && p->n_q_heads > 0 && p->n_kv_heads > 0 &&
         p->n_q_heads % p->n_kv_heads == 0 && p->head_dim > 0 &&
         (p->dtype == ORA_F32 || p->dtype == ORA_BF16);
}

// Non-negative integers of any size (base 2^32 digits, least significant
// first), for the exact mass sums of the SpecVLM selection below.  Only what
// that rule needs: from an integer-valued double, add, shift left, multiply by
// a 64-bit integer, compare.
struct Nat {
  std::vector<uint32_t> d;
};

void nat_trim(Nat& a) {
  while (!a.d.empty() && a.d.back() == 0) a.d.pop_back();
}

// x >= 0 with no fractional part, exactly.
Nat nat_from_integer_double(double x) {
  Nat r;
  if (x == 0.0) return r;
  int e = 0;
  const double f = std::frexp(x, &e);                  // x = f 2^e, f in [0.5, 1)
  uint64_t m = (uint64_t)std::ldexp(f, 53);            // 53-bit integer, exact
  int sh = e - 53;                                     // x = m 2^sh
  if (sh < 0) {                                        // x is an integer: the dropped
    m >>= -sh;                                         // bits are zeros
    sh = 0;
  }
  r.d = {(uint32_t)m, (uint32_t)(m >> 32)};
  nat_trim(r);
  Nat out;
  out.d.assign((size_t)(sh / 32) + r.d.size() + 1, 0u);
  const int bs = sh % 32;
  for (size_t i = 0; i < r.d.size(); ++i) {
    const uint64_t v = (uint64_t)r.d[i] << bs;
    out.d[i + sh / 32] |= (uint32_t)v;
    out.d[i + sh / 32 + 1] |= (uint32_t)(v >> 32);
  }
  nat_trim(out);
  return out;
}

Nat nat_add(const Nat& a, const Nat& b) {
  Nat r;
  const size_t n = std::max(a.d.size(), b.d.size());
  r.d.assign(n + 1, 0u);
  uint64_t carry = 0;
  for (size_t i = 0; i < n; ++i) {
    const uint64_t t = (uint64_t)(i < a.d.size() ? a.d[i] : 0u) + (i < b.d.size() ? b.d[i] : 0u) + carry;
    r.d[i] = (uint32_t)t;
    carry = t >> 32;
  }
  r.d[n] = (uint32_t)carry;
  nat_trim(r);
  return r;
}

Nat nat_shl(const Nat& a, int sh) {
  Nat r;
  if (a.d.empty()) return r;
  r.d.assign(a.d.size() + (size_t)(sh / 32) + 1, 0u);
  const int bs = sh % 32;
  for (size_t i = 0; i < a.d.size(); ++i) {
    const uint64_t v = (uint64_t)a.d[i] << bs;
    r.d[i + sh / 32] |= (uint32_t)v;
    r.d[i + sh / 32 + 1] |= (uint32_t)(v >> 32);
  }
  nat_trim(r);
  return r;
}

Nat nat_mul_u64(const Nat& a, uint64_t m) {
  const uint32_t ml[2] = {(uint32_t)m, (uint32_t)(m >> 32)};
  Nat r;
  r.d.assign(a.d.size() + 3, 0u);
  for (int j = 0; j < 2; ++j) {
    uint64_t carry = 0;
    for (size_t i = 0; i < a.d.size(); ++i) {
      const uint64_t t = (uint64_t)a.d[i] * ml[j] + r.d[i + j] + carry;
      r.d[i + j] = (uint32_t)t;
      carry = t >> 32;
    }
    for (size_t k = a.d.size() + j; carry; ++k) {
      const uint64_t t = (uint64_t)r.d[k] + carry;
      r.d[k] = (uint32_t)t;
      carry = t >> 32;
    }
  }
  nat_trim(r);
  return r;
}

int nat_cmp(const Nat& a, const Nat& b) {
  if (a.d.size() != b.d.size()) return a.d.size() < b.d.size() ? -1 : 1;
  for (size_t i = a.d.size(); i-- > 0;)
    if (a.d[i] != b.d[i]) return a.d[i] < b.d[i] ? -1 : 1;
  return 0;
}

}  // namespace

extern "C" {

int ora_version(void) { return 1; }

// Score (StD Sec. 3.2 equation; SMM observation window; BX "Speedup Across
// Context" scoring).  W observation queries q[i][g][:], i < W, sit at positions
// n - W + i and see keys j <= n - W + i (causal).  For each visible key:
//   P_{g,i}(j) = exp(l_{g,i}(j) - lse_{g,i}),
// and the kv head's score sums the probabilities of its query group (the GQA
// rule of StD Sec. 3.2) and averages over the W window rows:
//   s_h(j) = (1/W) * sum_{g in group(h)} sum_{i<W} P_{g,i}(j),   0 for unseen j.
// W = 1 is the per-step score of a decode query at position n-1.
// Writes s in fp64 (score64, may be null) and rounded to fp32 (score32).
int ora_score(const OraProblem* p, const void* q, int32_t W, const void* k,
              int64_t n, double* score64, float* score32, int64_t score_stride,
              int32_t nthreads) {
  if (!problem_ok(p) || !q || !k || W < 1 || n < 1 || W > n ||
      score_stride < n || !score32)
    return 1;
  const int G = p->n_q_heads / p->n_kv_heads;
  const int Hkv = p->n_kv_heads;
  // One task per (kv head, query head of its group): the task sums that query
  // head's window rows in ascending i; the group's tasks are then added in
  // ascending g and divided by W.
  const int64_t ntask = (int64_t)Hkv * G;
  std::vector<std::vector<double>> part(ntask);
  parallel_for(ntask, nthreads, [&](int64_t task) {
    const int h = (int)(task / G);
    const int g = h * G + (int)(task % G);
    std::vector<double>& acc = part[task];
    acc.assign(n, 0.0);
    std::vector<int64_t> pos(n);
    for (int64_t j = 0; j < n; ++j) pos[j] = j;
    std::vector<double> l(n);
    for (int i = 0; i < W; ++i) {
      const int64_t visible = n - W + i + 1;  // keys 0 .. n-W+i
      std::vector<double> qv = query_row(*p, q, i, g);
      logits(*p, qv, k, h, pos.data(), visible, l.data());
      double m = l[0];
      for (int64_t j = 1; j < visible; ++j) m = std::max(m, l[j]);
      double z = 0.0;
      for (int64_t j = 0; j < visible; ++j) z += std::exp(l[j] - m);
      const double lse = m + std::log(z);
      for (int64_t j = 0; j < visible; ++j) acc[j] += std::exp(l[j] - lse);
    }
  });
  parallel_for(Hkv, nthreads, [&](int64_t h) {
    for (int64_t j = 0; j < n; ++j) {
      double s = 0.0;
      for (int g_in = 0; g_in < G; ++g_in) s += part[h * G + g_in][j];
      s = s / (double)W;
      if (score64) score64[h * score_stride + j] = s;
      score32[h * score_stride + j] = (float)s;
    }
  });
  return 0;
}

// Selection (BX: four sinks plus the highest-scoring history entries plus the
// recent run; SMM: K = r + b_score picked by observation-window score, with the
// local window kept separately; StD Sec. 3.2: argTopK per kv head).
//   recent window  = [max(n-R,0), n)            -- attended as the tail, not written
//   sinks          = [0, min(S, max(n-R,0)))    -- always kept, written first
//   candidates C   = [S, n-R)                   -- empty when S >= n-R
// Keep the first min(K_h, |C|) candidates ordered by (score descending, index
// ascending); -0.0 compares equal to +0.0.  idx[h][0..count[h]) lists sinks
// and kept candidates in ascending order.
int ora_select(const float* score, int64_t score_stride, int32_t Hkv, int64_t n,
               int32_t S, int32_t R, const int32_t* k_per_head, int32_t* idx,
               int64_t idx_stride, int32_t* count) {
  if (!score || !k_per_head || !idx || !count || Hkv < 1 || n < 1 || S < 0 ||
      R < 0 || score_stride < n)
    return 1;
  const int64_t tail = std::max<int64_t>(n - R, 0);
  const int64_t nsink = std::min<int64_t>(S, tail);
  const int64_t c_lo = S, c_hi = n - R;
  const int64_t ncand = (c_lo < c_hi) ? c_hi - c_lo : 0;
  for (int h = 0; h < Hkv; ++h) {
    const float* s = score + (int64_t)h * score_stride;
    for (int64_t j = c_lo; j < c_lo + ncand; ++j)
      if (!std::isfinite(s[j])) return 2;
    const int64_t kh = std::min<int64_t>(std::max<int32_t>(k_per_head[h], 0), ncand);
    if (nsink + kh > idx_stride) return 1;
    std::vector<int64_t> cand(ncand);
    for (int64_t i = 0; i < ncand; ++i) cand[i] = c_lo + i;
    std::sort(cand.begin(), cand.end(), [&](int64_t a, int64_t b) {
      const float sa = s[a], sb = s[b];
      if (sa != sb) return sa > sb;  // -0.0 == +0.0 here
      return a < b;
    });
    std::vector<int64_t> kept;
    for (int64_t j = 0; j < nsink; ++j) kept.push_back(j);
    for (int64_t i = 0; i < kh; ++i) kept.push_back(cand[i]);
    std::sort(kept.begin(), kept.end());
    for (size_t i = 0; i < kept.size(); ++i)
      idx[(int64_t)h * idx_stride + (int64_t)i] = (int32_t)kept[i];
    count[h] = (int32_t)kept.size();
  }
  return 0;
}

// Verifier-guided selection (SpecVLM blog, "The SpecVLM Method": Stage I
// top-P retention, Stage II spatially uniform reduction).  Candidates, sinks
// and the recent run are split as in ora_select.  One selection per score row,
// or, with pooled != 0, one selection on the per-token sum over all rows that
// every row then receives (the blog averages the verifier's attention over
// layers and heads; the constant factor is dropped).
//
// Readings, in the order the blog gives the steps:
//   a_j      the candidate's score (fp32, finite, >= 0).  Pooled: the sum over
//            rows, added in double in ascending row order and rounded to the
//            nearest fp32 (saturating at the largest finite fp32);
//   order    a descending, index ascending;
//   Stage I  c = the smallest c' whose first c' candidates in that order carry
//            mass sum >= lambda * (sum of every a), in exact arithmetic: every
//            fp32 a is an integer multiple of 2^-149, so the sums are exact
//            integers in that unit, and lambda (a double) is the exact
//            fraction lam_m / 2^lam_sh; V_R = those c candidates;
//   Stage II B = (1 - r) n_cand rounded to nearest in double (ties away from
//            zero: r = 0.9 of 100 candidates gives 10); the L = n_cand - c leftover
//            candidates, in ascending index order, are sampled at ranks
//            floor(i L / n_U), i < n_U, where n_U = clamp(B - c, 0, L)
//            (fill_mode 0: the interval that brings the kept set to B) or
//            n_U = min(B, L) (fill_mode 1: the interval as printed,
//            (|V| - |V_R|) / ((1 - r) |V|)).
// idx[h][0..count[h]) = sinks, V_R and V_U in ascending order; count_r[h] = c.
// Scores must be finite and >= 0 (else 2).
int ora_select_topp(const float* score, int64_t score_stride, int32_t H, int64_t n, int32_t S,
                    int32_t R, double lambda, double prune, int32_t pooled, int32_t fill_mode,
                    int32_t* idx, int64_t idx_stride, int32_t* count, int32_t* count_r) {
  if (!score || !idx || !count || H < 1 || n < 1 || S < 0 || R < 0 || score_stride < n ||
      !(lambda >= 0.0 && lambda <= 1.0) || !(prune >= 0.0 && prune <= 1.0) ||
      (fill_mode != 0 && fill_mode != 1))
    return 1;
  const int64_t tail = std::max<int64_t>(n - R, 0);
  const int64_t nsink = std::min<int64_t>(S, tail);
  const int64_t c_lo = S, ncand = (S < n - R) ? (n - R) - S : 0;
  if (idx_stride < nsink + ncand) return 1;
  for (int h = 0; h < H; ++h)
    for (int64_t j = c_lo; j < c_lo + ncand; ++j) {
      const float x = score[h * score_stride + j];
      if (!std::isfinite(x) || x < 0.0f) return 2;
    }
  const int64_t budget = std::llround((1.0 - prune) * (double)ncand);
  // lambda = lam_m / 2^lam_sh exactly (a double has a 53-bit significand)
  int lexp = 0;
  const double lfrac = std::frexp(lambda, &lexp);
  const uint64_t lam_m = (uint64_t)std::ldexp(lfrac, 53);
  const int lam_sh = 53 - lexp;
  const int n_sel = pooled ? 1 : H;
  for (int sel = 0; sel < n_sel; ++sel) {
    const int h0 = pooled ? 0 : sel, h1 = pooled ? H : sel + 1;
    std::vector<float> a(ncand);
    for (int64_t i = 0; i < ncand; ++i) {
      double sum = 0.0;
      for (int h = h0; h < h1; ++h) sum += (double)score[h * score_stride + c_lo + i];
      float x = (float)sum;
      if (std::isinf(x)) x = std::numeric_limits<float>::max();
      a[i] = x;
    }
    // exact masses in units of 2^-149, and their total
    std::vector<Nat> mass(ncand);
    Nat total;
    for (int64_t i = 0; i < ncand; ++i) {
      mass[i] = nat_from_integer_double(std::ldexp((double)a[i], 149));
      total = nat_add(total, mass[i]);
    }
    // Stage I: sort by score, keep the shortest prefix reaching lambda of the
    // total: prefix >= lambda * total  <=>  prefix * 2^lam_sh >= lam_m * total
    std::vector<int64_t> order(ncand);
    for (int64_t i = 0; i < ncand; ++i) order[i] = i;
    std::sort(order.begin(), order.end(), [&](int64_t x, int64_t y) {
      if (a[x] != a[y]) return a[x] > a[y];
      return x < y;
    });
    const Nat rhs = nat_mul_u64(total, lam_m);
    int64_t c = 0;
    Nat prefix;
    while (nat_cmp(nat_shl(prefix, lam_sh), rhs) < 0) {
      prefix = nat_add(prefix, mass[order[c]]);
      ++c;
    }
    std::vector<char> in_r(ncand, 0);
    for (int64_t i = 0; i < c; ++i) in_r[order[i]] = 1;
    // Stage II: uniform walk through the leftovers in index order
    const int64_t L = ncand - c;
    int64_t n_u = fill_mode == 0 ? std::min(std::max<int64_t>(budget - c, 0), L) : std::min(budget, L);
    std::vector<char> in_u(ncand, 0);
    if (n_u > 0) {
      std::vector<int64_t> left;
      for (int64_t i = 0; i < ncand; ++i)
        if (!in_r[i]) left.push_back(i);
      for (int64_t t = 0; t < n_u; ++t) in_u[left[(t * L) / n_u]] = 1;
    }
    for (int h = h0; h < h1; ++h) {
      int64_t w = 0;
      for (int64_t j = 0; j < nsink; ++j) idx[h * idx_stride + w++] = (int32_t)j;
      for (int64_t i = 0; i < ncand; ++i)
        if (in_r[i] || in_u[i]) idx[h * idx_stride + w++] = (int32_t)(c_lo + i);
      count[h] = (int32_t)w;
      if (count_r) count_r[h] = (int32_t)c;
    }
  }
  return 0;
}

// Dense decode attention (BX "The Attention Baseline": the dense step reads the
// whole cache): one decode query per head at position n-1 over keys [0, n).
// q [Hq][d]; out [Hq][d]; lse [Hq] (natural log of the softmax normaliser).
int ora_attend_dense(const OraProblem* p, const void* q, const void* k,
                     const void* v, int64_t n, double* out, double* lse,
                     int32_t nthreads) {
  if (!problem_ok(p) || !q || !k || !v || n < 0 || !out || !lse) return 1;
  const int G = p->n_q_heads / p->n_kv_heads;
  std::vector<int64_t> pos(n);
  for (int64_t j = 0; j < n; ++j) pos[j] = j;
  parallel_for(p->n_q_heads, nthreads, [&](int64_t g) {
    std::vector<double> qv = query_row(*p, q, 0, (int)g);
    attend_row(*p, qv, k, v, (int)(g / G), pos, out + g * p->head_dim, lse + g);
  });
  return 0;
}

// Sparse decode attention (StD Sec. 3.2 top-K attention; BX kept set read in
// one call; StD Sec. 3.3: the draft reads the selected entries plus the text
// tokens): per kv head h the key set is idx[h][0..count[h]) followed by the
// contiguous tail [tail_start, n).  idx entries must be unique and < tail_start.
int ora_attend_sparse(const OraProblem* p, const void* q, const void* k,
                      const void* v, int64_t n, const int32_t* idx,
                      int64_t idx_stride, const int32_t* count,
                      int64_t tail_start, double* out, double* lse,
                      int32_t nthreads) {
  if (!problem_ok(p) || !q || !k || !v || n < 0 || !idx || !count || !out ||
      !lse || tail_start < 0 || tail_start > n)
    return 1;
  const int G = p->n_q_heads / p->n_kv_heads;
  for (int h = 0; h < p->n_kv_heads; ++h) {
    if (count[h] < 0 || count[h] > idx_stride) return 1;
    std::vector<char> seen(tail_start, 0);
    for (int32_t i = 0; i < count[h]; ++i) {
      const int32_t j = idx[(int64_t)h * idx_stride + i];
      if (j < 0 || j >= tail_start || seen[j]) return 1;
      seen[j] = 1;
    }
  }
  parallel_for(p->n_q_heads, nthreads, [&](int64_t g) {
    const int h = (int)(g / G);
    std::vector<int64_t> pos;
    for (int32_t i = 0; i < count[h]; ++i)
      pos.push_back(idx[(int64_t)h * idx_stride + i]);
    for (int64_t j = tail_start; j < n; ++j) pos.push_back(j);
    std::vector<double> qv = query_row(*p, q, 0, (int)g);
    attend_row(*p, qv, k, v, h, pos, out + g * p->head_dim, lse + g);
  });
  return 0;
}

// Verify pass (StD Sec. 3.1: the dense model checks all gamma drafted tokens in
// one pass over the full cache).  The gamma new entries already occupy
// positions n-gamma .. n-1; query t (q[t][g][:]) sits at n-gamma+t and sees
// keys [0, n-gamma+t] (causal).  out [gamma][Hq][d], lse [gamma][Hq].
int ora_verify(const OraProblem* p, const void* q, int32_t gamma, const void* k,
               const void* v, int64_t n, double* out, double* lse,
               int32_t nthreads) {
  if (!problem_ok(p) || !q || !k || !v || gamma < 1 || n < gamma || !out || !lse)
    return 1;
  const int G = p->n_q_heads / p->n_kv_heads;
  const int64_t rows = (int64_t)gamma * p->n_q_heads;
  parallel_for(rows, nthreads, [&](int64_t r) {
    const int t = (int)(r / p->n_q_heads);
    const int g = (int)(r % p->n_q_heads);
    const int64_t visible = n - gamma + t + 1;
    std::vector<int64_t> pos(visible);
    for (int64_t j = 0; j < visible; ++j) pos[j] = j;
    std::vector<double> qv = query_row(*p, q, t, g);
    attend_row(*p, qv, k, v, g / G, pos, out + r * p->head_dim, lse + r);
  });
  return 0;
}

// Per-head budgets (SMM method section).  N heads, total budget B, local window
// w, uniform share rho:
//   r        = rho * (B - N*w) / N                       (Uniform-Based Cache)
//   B_remain = B - N*w - rho * (B - N*w)
//   b_score  = B_remain * s_i / sum_k s_k                (Score-Preferred Cache)
//   b_i      = w + r + b_score                            (per-head total)
// The observation-window top-K count of head i is K_i = r + b_score (the local
// window is kept separately); here it is floor(r + b_score) clamped to
// [0, n_cand].  b_out (may be null) receives b_i unrounded.
int ora_budgets(const double* s, int32_t N, double B, int32_t w, double rho,
                int64_t n_cand, int32_t* k_out, double* b_out) {
  if (!s || !k_out || N < 1 || w < 0 || rho < 0.0 || rho > 1.0) return 1;
  double sum = 0.0;
  for (int32_t i = 0; i < N; ++i) {
    if (!(s[i] >= 0.0) || !std::isfinite(s[i])) return 1;
    sum += s[i];
  }
  if (!(sum > 0.0)) return 1;
  const double base = B - (double)N * (double)w;
  const double r = rho * base / (double)N;
  const double b_remain = B - (double)N * (double)w - rho * base;
  for (int32_t i = 0; i < N; ++i) {
    const double b_score = b_remain * s[i] / sum;
    double kf = std::floor(r + b_score);
    if (kf < 0.0) kf = 0.0;
    if (kf > (double)n_cand) kf = (double)n_cand;
    k_out[i] = (int32_t)kf;
    if (b_out) b_out[i] = (double)w + r + b_score;
  }
  return 0;
}

}  // extern "C"
