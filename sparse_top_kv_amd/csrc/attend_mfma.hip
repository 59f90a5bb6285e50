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
//   - Each of the eight waves owns a private ring of kStages tiles of 16 keys
//     (K and V, 4 KB each at d=128) in LDS, filled by buffer_load ... lds, so
//     (kStages-1) tiles per wave are in flight without holding registers:
//     64 KB per CU with two stages, one 128 KB workgroup per CU.  (Four waves
//     with three or four stages, or two workgroups per CU, measured slower.)
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
//   - Softmax in the log2 domain against a per-row reference fixed from the
//     wave's first tile; a tile whose logits pass the reference by kSlack
//     rescales the accumulators first (rare, wave-uniform branch, inside the
//     pipelined loop).
#include "skv_common.h"
#include "skv_kernels.h"
#include "skv_mfma.h"
#include "skv_tile.h"
#include "skv_block.h"

namespace skv {
namespace {

constexpr int kSparseMaxChunk = 2048;     // rows per workgroup (LDS offset list)
constexpr float kSlack = 30.0f;

// W waves of 64 lanes, S-tile ring per wave, NG groups of 16 query rows.
// Query rows of kv head h: r = t * G + g for position t < a.n_pos and group
// member g < G (decode: one position).  CAUSAL: row r sees keys
// j <= n - n_pos + t (the verify pass); otherwise every key of the set.
template <int D, int NG, bool SPARSE, bool CAUSAL, int W, int S, bool LIST, bool SPLIT = false>
__global__ __launch_bounds__(64 * W) void attend_mfma_kernel(const AttendArgs a) {
  using TG = TileGeom<D>;
  constexpr int NI = TG::kNI, TB = TG::kTB, PPR = TG::kPPR, KS = TG::kKS, NT = TG::kNT;
  constexpr int kT = 64 * W;

  // per wave: [K tile | V tile]; one LDS object per stage
  __shared__ __attribute__((aligned(1024))) char st0[W][2 * TB];
  __shared__ __attribute__((aligned(1024))) char st1[W][2 * TB];
  __shared__ __attribute__((aligned(1024))) char st2[W][2 * TB];
  __shared__ __attribute__((aligned(1024))) char st3[W][2 * TB];
  __shared__ __attribute__((aligned(16))) uint32_t sm_off[SPARSE ? kSparseMaxChunk : 1];
  // (max, sum) of each wave's rows per parked row group; a third slot for a
  // third group parked beside the ring (the fold below)
  constexpr bool kXQ = NG == 3 && S == 2;
  __shared__ float sm_m[kXQ ? S + 1 : S][W][16];
  __shared__ __attribute__((aligned(16))) float sm_l[kXQ ? S + 1 : S][W][16];
  static_assert(S >= 2 && S <= 4, "ring of two to four stages");
  static_assert(16 * D * 4 <= 2 * TB, "a wave's 16-row partial fits its first stage");
  static_assert(!(SPARSE && CAUSAL), "the causal pass is dense");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, li = lane & 15;
  const int cph = a.chunks_per_head;
  static_assert(!LIST || SPARSE, "the work list serves gathered rows");

  // one (kv head, chunk) pair
  auto body = [&](const int h, const int c) {
  const int G = a.group;
  const int R = G * a.n_pos;  // query rows of this kv head
  const int Hq = a.n_kv_heads * G;

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
        if (k * kT >= a.chunk) break;  // uniform
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
  // q as the B operand of q.K^T: in group gi, lane (q4, li) takes row
  // 16 gi + li, channels [32 s + 8 q4, +8); rows past R are zero.  One row
  // group lives in registers; more are staged in LDS (XOR-swizzled by row)
  // and read per step, which keeps the accumulators of all groups in VGPRs.
  // lim: the last key position the lane's row may see (causal pass only).
  constexpr bool kQInLds = NG > 1;
  __shared__ __attribute__((aligned(16))) char sm_q[kQInLds ? NG * 16 * D * 2 : 16];
  bf16x8_t qb[kQInLds ? 1 : KS];
  bool row_ok[NG];
  int lim[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int r = 16 * gi + li;
    row_ok[gi] = r < R;
    const int t = row_ok[gi] ? r / G : 0;
    lim[gi] = (int)(a.n - a.n_pos) + t;
  }
  // (staged rows: loaded here, written to LDS once the first tiles' copies
  // are issued, so the two loads overlap)
  constexpr int kQIt = kQInLds ? (NG * 16 * (D / 8) + kT - 1) / kT : 1;
  uint4 qv[kQIt];
  if constexpr (kQInLds) {
#pragma unroll
    for (int i = 0; i < kQIt; ++i) {
      const int e = tid + i * kT, r = e / (D / 8), pc = e - r * (D / 8);
      qv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (e < NG * 16 * (D / 8) && r < R) {
        const int t = r / G, g = r - t * G;
        qv[i] = ld16(reinterpret_cast<const char*>(a.q) + (((int64_t)t * Hq + h * G + g) * D + pc * 8) * 2);
      }
    }
  } else {
    const int r = li;
    const int t = row_ok[0] ? r / G : 0;
    const int g = row_ok[0] ? r - t * G : 0;
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)t * Hq + h * G + g) * D * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok[0]) v = ld16(qrow + (32 * s + 8 * q4) * 2);
      qb[s] = as_bf16x8(v);
    }
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
      if (k * kT >= a.chunk) break;  // uniform
      if (i < kSparseMaxChunk) {
        const int64_t r = r0 + i;
        int32_t p = 0;
        if (i < rows) p = r < cnt ? spec[k] : (int32_t)(a.tail_start + (r - cnt));
        p = p < 0 ? 0 : (p > last ? last : p);  // keep out-of-contract indices in bounds
        sm_off[i] = (uint32_t)p * stride;
      }
    }
  }
  if constexpr (SPARSE) __syncthreads();  // the row offsets (staged query rows: after the prologue)

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
  // Tiles are dealt in rounds of kR: the first wave on each SIMD (waves
  // 0..3) takes kA tiles of a round, the second (waves 4..7) kB.  In a
  // one-row-group step the second wave of a SIMD streams more slowly (its
  // copies queue behind the first wave's): with even shares it finished
  // 1.2 us (32K sparse step) to 4.9 us (32K dense step) after the first,
  // with half the CU's copies in flight meanwhile.  SPLIT (chunks of at
  // least two rounds) deals 2:1 (gathered rows) or 3:2 (dense); verify rows
  // measured slower with any uneven split.
  static_assert(!SPLIT || (W == 8 && NG == 1 && !CAUSAL), "uneven shares for one-row-group steps");
  constexpr int kA = SPLIT ? (SPARSE ? 2 : 3) : 1, kB = SPLIT ? (SPARSE ? 1 : 2) : 1;
  constexpr int kR = SPLIT ? 4 * (kA + kB) : W;
  const bool second = SPLIT && wave >= 4;
  const int wl = second ? wave - 4 : wave;      // position within its half
  const int per = second ? kB : kA;             // tiles per round
  const int base = second ? 4 * kA : 0;         // first slot of its half
  constexpr int kHalf = SPLIT ? 4 : W;            // waves per half
  auto tile_of = [&](int k) {  // (constant divisors in either half)
    if constexpr (!SPLIT) return k * W + wave;
    return second ? (k / kB) * kR + 4 * kA + (k % kB) * 4 + wl : (k / kA) * kR + (k % kA) * 4 + wl;
  };
  int nst;  // this wave's steps
  {
    const int full = nsteps / kR, rem = nsteps - full * kR;
    int extra = (rem - base - wl + kHalf - 1) / kHalf;
    extra = extra < 0 ? 0 : (extra > per ? per : extra);
    nst = full * per + extra;
  }
  const float c2 = a.scale_log2;

  // copies of local step k (global step wave + W k) into a stage
  auto issue = [&](char (*stg)[2 * TB], int k) {
    const int j = tile_of(k);
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
      for (int u = 0; u < NI; ++u) copy_to_lds(rk, dst + u * 1024, ro[u] + pk[u], 0);
#pragma unroll
      for (int u = 0; u < NI; ++u) copy_to_lds(rv, dst + TB + u * 1024, ro[u] + pv[u], 0);
    } else {
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(r0 + (int64_t)j * kStep) * stride);
#pragma unroll
      for (int u = 0; u < NI; ++u) copy_to_lds(rk, dst + u * 1024, pk[u], soff);
#pragma unroll
      for (int u = 0; u < NI; ++u) copy_to_lds(rv, dst + TB + u * 1024, pv[u], soff);
    }
  };

  float m[NG];   // reference of row 16 gi + li (log2 units)
  float l[NG];   // this lane's share of that row's sum
  floatx4_t o[NG][NT];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    m[gi] = kNegInf;
    l[gi] = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[gi][n] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // log2-domain logits of the tile of local step k (already in LDS): key
  // 4 q4 + r of row 16 gi + li; -inf past the chunk (and past the row's
  // causal limit)
  auto logits = [&](const char* base, int k, float (&sv)[NG][4]) {
    floatx4_t cs[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) cs[gi] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 kv = *reinterpret_cast<const uint4*>(base + koff[s]);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        bf16x8_t qv;
        if constexpr (kQInLds)
          qv = as_bf16x8(*reinterpret_cast<const uint4*>(
              sm_q + (16 * gi + li) * D * 2 + (((4 * s + q4) ^ swz_q<D>(16 * gi + li)) * 16)));
        else
          qv = qb[s];
        cs[gi] = mfma_bf16(as_bf16x8(kv), qv, cs[gi]);
      }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[gi][r] = cs[gi][r] * c2;
    // masks only on a tile that reaches past the chunk or, in the causal
    // pass, past the first row's last key (wave-uniform test)
    const int j = tile_of(k);
    bool edge = (j + 1) * kStep > rows;
    if constexpr (CAUSAL) edge = edge || r0 + (int64_t)(j + 1) * kStep - 1 > a.n - a.n_pos;
    if (edge) {
      const int rb = j * kStep + 4 * q4;  // chunk row of key r = 0
      const int pb = (int)r0 + rb;        // its position (dense)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bool ok = rb + r < rows;
          if constexpr (CAUSAL) ok = ok & (pb + r <= lim[gi]);
          sv[gi][r] = ok ? sv[gi][r] : kNegInf;
        }
    }
  };
  // max over the tile's keys of the lane's row (all four q4 lanes agree)
  auto row_max = [&](const float (&x)[4]) {
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = xor16_max(mx);
    return xor32_max(mx);
  };
  // probabilities against the reference, into the sums, as bf16 hi + lo
  // (the A operands of P.V), and the tile's V columns (the B operands)
  auto probs = [&](const char* base, const float (&sv)[NG][4], short4_t (&ahi)[NG], short4_t (&alo)[NG],
                   short4_t (&vb)[NT]) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      // a row still without a reference (-inf) has no visible key in this
      // tile either (any would have triggered the rescale), so every sv is
      // -inf and the probabilities are 0
      const float mref = m[gi] == kNegInf ? 0.0f : m[gi];
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(sv[gi][r] - mref);
        l[gi] += p[r];
      }
      const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
      const uint32_t l01 = pack_bf16(p[0] - bf16lo(h01), p[1] - bf16hi(h01));
      const uint32_t l23 = pack_bf16(p[2] - bf16lo(h23), p[3] - bf16hi(h23));
      ahi[gi] = __builtin_bit_cast(short4_t, make_uint2(h01, h23));
      alo[gi] = __builtin_bit_cast(short4_t, make_uint2(l01, l23));
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) vb[n] = lds_read_tr16(base + voff[n]);
  };
  // P.V of one tile on 16-key MFMAs
  auto pv16 = [&](const short4_t (&ahi)[NG], const short4_t (&alo)[NG], const short4_t (&vb)[NT]) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
      for (int n = 0; n < NT; ++n) o[gi][n] = mfma16(ahi[gi], vb[n], o[gi][n]);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[gi][n] = mfma16(alo[gi], vb[n], o[gi][n]);
    }
  };
  // P.V of two tiles on 32-key MFMAs (half the instructions): reduction
  // index 8 q + j is key 4 q + j of the first tile for j < 4 and key
  // 4 q + j - 4 of the second for j >= 4, in both operands
  auto cat8 = [](const short4_t& x, const short4_t& y) {
    const uint2 a = __builtin_bit_cast(uint2, x), b = __builtin_bit_cast(uint2, y);
    return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
  };
  auto pv32 = [&](const short4_t (&ahi0)[NG], const short4_t (&alo0)[NG], const short4_t (&vb0)[NT],
                  const short4_t (&ahi1)[NG], const short4_t (&alo1)[NG], const short4_t (&vb1)[NT]) {
    bf16x8_t vv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) vv[n] = cat8(vb0[n], vb1[n]);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const bf16x8_t ah = cat8(ahi0[gi], ahi1[gi]), al = cat8(alo0[gi], alo1[gi]);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[gi][n] = mfma_bf16(ah, vv[n], o[gi][n]);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[gi][n] = mfma_bf16(al, vv[n], o[gi][n]);
    }
  };
  // several row groups (the verify pass): a tile's P.V waits for the next
  // tile's and both go on 32-key MFMAs (pend: wave-uniform).  A single row
  // group keeps the 16-key form: its step is latency-bound and the extra
  // registers measured slower there.
  constexpr bool kPair = NG >= 2;
  bool pend = false;
  short4_t phi[kPair ? NG : 1], plo[kPair ? NG : 1], pvb[kPair ? NT : 1];

  // steps issued after local step k (their copies may still be in flight)
  auto newer_than = [&](int k) { return (nst - 1 - k) < (S - 1) ? (nst - 1 - k) : (S - 1); };

  // move the references up to cover this tile and rescale what is accumulated
  auto rescale = [&](const float (&sv)[NG][4]) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float mn = fmaxf(m[gi], row_max(sv[gi]));
      // unchanged reference (also -inf to -inf): nothing to rescale
      const float alpha = m[gi] == mn ? 1.0f : fast_exp2(m[gi] - mn);
      l[gi] *= alpha;
      m[gi] = mn;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * q4 + r, 64);  // row 4 q4 + r
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[gi][n][r] *= ar[r];
    }
  };

  // one step: refill the stage freed by the previous step, wait for step k,
  // and accumulate it against the reference; a tile with a logit past the
  // reference by kSlack first rescales (rare, wave-uniform branch)
  auto step = [&](char (*cur)[2 * TB], char (*nxt)[2 * TB], int k) {
    if (k + S - 1 < nst) {
      wait_lgkm0();  // reads of the stage being refilled are done
      issue(nxt, k + S - 1);
    }
    wait_newer<S - 1, 2 * NI>(newer_than(k));
    float sv[NG][4];
    logits(&cur[0][0], k, sv);
    bool over = false;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float mx = fmaxf(fmaxf(sv[gi][0], sv[gi][1]), fmaxf(sv[gi][2], sv[gi][3]));
      over = over || (row_ok[gi] && mx > m[gi] + kSlack);
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      if constexpr (kPair) {
        if (pend) {  // the waiting tile is summed against the old reference first
          pv16(phi, plo, pvb);
          pend = false;
        }
      }
      rescale(sv);
    }
    short4_t ahi[NG], alo[NG], vb[NT];
    probs(&cur[0][0], sv, ahi, alo, vb);
    if constexpr (!kPair) {
      pv16(ahi, alo, vb);
    } else if (pend) {
      pv32(phi, plo, pvb, ahi, alo, vb);
      pend = false;
    } else {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        phi[gi] = ahi[gi];
        plo[gi] = alo[gi];
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) pvb[n] = vb[n];
      pend = true;
    }
  };

  // stage u of the ring
  auto ring = [&](int u) -> char (*)[2 * TB] {
    if (S > 3 && u == 3) return st3;  // stages past S are never referenced
    if (S > 2 && u == 2) return st2;
    return u == 1 ? st1 : st0;
  };
  // (with staged query rows every prologue copy is issued, also past the
  // wave's tiles: their count is then known where the rows are written, so
  // that write waits for the query loads alone; copies past the kv head's
  // rows read zeros, and a wave with fewer tiles never reads those stages)
#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (kQInLds || u < nst) issue(ring(u), u);
  // the query rows staged in LDS, behind a barrier taken once the first
  // tiles' copies are on their way (their addresses need nothing staged), so
  // the two loads overlap
  if constexpr (kQInLds) {
#pragma unroll
    for (int i = 0; i < kQIt; ++i) {
      const int e = tid + i * kT, r = e / (D / 8), pc = e - r * (D / 8);
      if (e < NG * 16 * (D / 8)) *reinterpret_cast<uint4*>(sm_q + r * D * 2 + ((pc ^ swz_q<D>(r)) * 16)) = qv[i];
    }
    // an LDS-only barrier: this wave's rows are written (lgkmcnt 0), the
    // copies keep flying (a full barrier would wait for every wave's tiles)
    wait_lgkm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if (nst > 0) {
    // reference: the first tile's max per row; -inf for a row with no
    // visible key there (causal pass), which the first tile that shows the
    // row a key replaces through the rescale (softmax is shift-invariant, so
    // no fixed stand-in value may be used: logits far below it would
    // underflow).  Only the prologue's copies are in flight here: steps 1 ..
    // min(nst, S - 1) - 1 are newer than step 0.
    wait_newer<S - 2, 2 * NI>(nst - 1 < S - 2 ? nst - 1 : S - 2);
    float sv[NG][4];
    logits(&st0[0][0], 0, sv);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) m[gi] = row_max(sv[gi]);
    for (int k = 0; k < nst;) {
#pragma unroll
      for (int u = 0; u < S; ++u) {
        if (k < nst) step(ring(u), ring((u + S - 1) % S), k);
        ++k;
      }
    }
    if constexpr (kPair)
      if (pend) pv16(phi, plo, pvb);
  }

  // Folding the waves, S row groups per round: each wave parks the partial
  // of group g0 + u in its own stage u (its copies are done); 16 threads per
  // group turn the waves' (max, sum) into the row's max, sum and one weight
  // per wave; then the workgroup folds the waves' accumulators.
  constexpr int GPR = S < NG ? S : NG;  // groups per round
  // (a wave without tiles may still have prologue copies in flight into the
  // stages the fold parks in)
  if constexpr (kQInLds) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // Three row groups on a two-tile ring whose third group holds one row quad
  // or less (35 or 36 rows: five drafts of seven query heads, nine of four)
  // fold in one round: that quad is parked in a 16 KB buffer of its own
  // (items u = GPR below).  Two rounds measured 1 us slower in verify.
  __shared__ __attribute__((aligned(16))) float st_x[kXQ ? W * 4 * D : 4];
  const bool xq = kXQ && R <= 16 * GPR + 4;  // uniform
  const int64_t slot = (int64_t)h * cph + c;
#pragma unroll
  for (int g0 = 0; g0 < NG; g0 += GPR) {
    if (16 * g0 >= R || (xq && g0 > 0)) break;  // uniform
    if constexpr (kXQ) {
      if (xq) {
        float lg = l[GPR];
        lg = xor16_sum(lg);
        lg = xor32_sum(lg);
        if (lane < 16) {
          sm_m[GPR][wave][lane] = nst == 0 ? kNegInf : m[GPR];
          sm_l[GPR][wave][lane] = nst == 0 ? 0.0f : lg;
        }
        if (q4 == 0) {  // rows 16 GPR .. 16 GPR + 3, column-major (4 floats per column)
          float* xw = &st_x[wave * 4 * D];
#pragma unroll
          for (int n = 0; n < NT; ++n) *reinterpret_cast<floatx4_t*>(xw + (16 * n + li) * 4) = o[GPR][n];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < GPR; ++u) {
      const int gi = g0 + u;
      if (gi < NG) {
        float lg = l[gi];
        lg = xor16_sum(lg);
        lg = xor32_sum(lg);
        if (lane < 16) {
          sm_m[u][wave][lane] = nst == 0 ? kNegInf : m[gi];
          sm_l[u][wave][lane] = nst == 0 ? 0.0f : lg;
        }
        // the wave's rows 4 q4 .. 4 q4 + 3 of column 16 n + li as one 16-byte
        // store (column-major, 16 floats per column, the four row quads
        // XOR-swizzled by column so eight lanes hit distinct banks); rows
        // past the kv head's query rows are not staged
        if (16 * gi + 4 * q4 < R) {
          float* acc_w = reinterpret_cast<float*>(&ring(u)[wave][0]);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const int col = 16 * n + li;
            *reinterpret_cast<floatx4_t*>(acc_w + col * 16 + 4 * (q4 ^ ((col >> 1) & 3))) = o[gi][n];
          }
        }
      }
    }
    __syncthreads();
    const int gpr = xq ? GPR + 1 : GPR;  // groups folded in this round
    if (tid < 16 * gpr) {
      const int u = tid >> 4, rr = tid & 15;
      const int row = 16 * (g0 + u) + rr;
      float M = sm_m[u][0][rr];
#pragma unroll
      for (int w = 1; w < W; ++w) M = fmaxf(M, sm_m[u][w][rr]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float sc = (sm_m[u][w][rr] == kNegInf) ? 0.0f : fast_exp2(sm_m[u][w][rr] - M);
        L += sm_l[u][w][rr] * sc;
        sm_l[u][w][rr] = sc;  // now the wave's weight
      }
      if (g0 + u < NG && row < R) {
        a.part_ml[(slot * R + row) * 2 + 0] = M;
        a.part_ml[(slot * R + row) * 2 + 1] = L;
      }
    }
    __syncthreads();
    // item (u, row quad q, column dd), columns fastest: each wave's quad is
    // one 16-byte LDS read, and a wave's stores are whole row segments
    // (the parked third group: items GPR 4 D .. GPR 4 D + D - 1, quad 0)
    for (int e = tid; e < GPR * 4 * D + (xq ? D : 0); e += kT) {
      const int dd = e % D, q = (e / D) % 4, u = e / (4 * D);
      const int gi = g0 + u, r0q = 16 * gi + 4 * q;  // first row of the quad
      if (gi < NG && r0q < R) {
        const bool xu = kXQ && u == GPR;
        const int at = dd * 16 + 4 * (q ^ ((dd >> 1) & 3));
        float A[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const floatx4_t x = xu ? *reinterpret_cast<const floatx4_t*>(&st_x[(w * D + dd) * 4])
                                 : *reinterpret_cast<const floatx4_t*>(reinterpret_cast<const float*>(&ring(u)[w][0]) + at);
          const floatx4_t wt = *reinterpret_cast<const floatx4_t*>(&sm_l[u][w][4 * q]);
#pragma unroll
          for (int i = 0; i < 4; ++i) A[i] += x[i] * wt[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0q + i < R) a.part_acc[(slot * R + r0q + i) * D + dd] = A[i];
      }
    }
    __syncthreads();
  }
  if (c == 0 && tid == 0) a.nch[h] = nch;
  };

  if constexpr (LIST) {
    const int total = *a.n_items;
    for (int it = blockIdx.x; it < total; it += gridDim.x) {
      const int2 hc = a.items[it];
      body(hc.x, hc.y);
    }
  } else {
    // kv head h takes blocks h, h + Hkv, ...: blocks are dealt to the XCDs
    // in turn, so with Hkv a divisor or multiple of 8 one head's chunks run
    // on one XCD (its L2 and TLB serve one head's rows, and the merge blocks
    // of that head land on the same XCD): the 32K sparse and dense steps
    // 12.62 -> 12.17 and 25.63 -> 24.63 us against head-major blocks
    body(blockIdx.x % a.n_kv_heads, blockIdx.x / a.n_kv_heads);
  }
}

// The (kv head, chunk) pairs of a gathered-rows call that hold rows: chunks
// 0 .. nch_h - 1 of head h, nch_h = clamp(ceil(rows_h / chunk), 1,
// chunks_per_head), rows_h = clamp(count[h]) + (n - tail_start).  The full
// chunks of every head come first, in head order, then each head's last
// chunk: workgroup w takes items w, w + grid, ..., so the long items start
// first (1024 heads of ragged budgets: 38.6 -> 37.5 us against head order).
// One 1024-thread workgroup; each thread owns consecutive heads.
__global__ __launch_bounds__(kSelThreads) void attend_items_kernel(const AttendArgs a) {
  __shared__ uint32_t sm_w[kSelWaves + 1];
  const int tid = threadIdx.x;
  const int H = a.n_kv_heads, cph = a.chunks_per_head;
  const int per = (H + kSelThreads - 1) / kSelThreads;
  auto nch_of = [&](int h) {
    int64_t cnt = a.count[h];
    cnt = cnt < 0 ? 0 : (cnt > a.count_max ? a.count_max : cnt);
    const int64_t rows = cnt + (a.n - a.tail_start);
    int64_t nc = (rows + a.chunk - 1) / a.chunk;
    nc = nc < 1 ? 1 : (nc > cph ? cph : nc);
    return (uint32_t)nc;
  };
  uint32_t mine = 0;  // this thread's heads' chunks before their last
  for (int k = 0; k < per; ++k) {
    const int h = tid * per + k;
    if (h < H) mine += nch_of(h) - 1u;
  }
  uint32_t full;
  uint32_t base = block_excl_scan(mine, sm_w, &full);
  for (int k = 0; k < per; ++k) {
    const int h = tid * per + k;
    if (h < H) {
      const uint32_t nc = nch_of(h);
      for (uint32_t c = 0; c + 1 < nc; ++c) a.items[base + c] = make_int2(h, (int)c);
      base += nc - 1u;
      a.items[full + (uint32_t)h] = make_int2(h, (int)nc - 1);
    }
  }
  if (tid == 0) *a.n_items = (int32_t)(full + (uint32_t)H);
}

// Eight waves with a two-tile ring (one 128 KB workgroup per CU), the
// accumulators kept in VGPRs (built with -amdgpu-mfma-vgpr-form): up to three
// row groups fit two waves per SIMD.  Four groups at d = 128 need more than
// 256 registers per wave, so they run four waves with a four-tile ring.
template <int D, int NG>
constexpr int mfma_waves() { return (NG >= 4 && D == 128) ? 4 : 8; }

template <int D, int NG, bool SPARSE, bool CAUSAL>
hipError_t launch_k(const AttendArgs& a, hipStream_t s) {
  constexpr int W = mfma_waves<D, NG>();
  constexpr int S = W == 8 ? 2 : 4;
  if constexpr (SPARSE) {
    if (a.items) {
      hipLaunchKernelGGL(attend_items_kernel, dim3(1), dim3(kSelThreads), 0, s, a);
      // four waves with a two-tile ring (64 KB): two workgroups per CU overlap
      // one item's start and end with the other's streaming
      hipLaunchKernelGGL((attend_mfma_kernel<D, NG, SPARSE, CAUSAL, 4, 2, true>), dim3((unsigned)a.list_grid),
                         dim3(64 * 4), 0, s, a);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)(a.n_kv_heads * a.chunks_per_head));
  if constexpr (NG == 1 && !CAUSAL) {
    if (a.narrow) {
      hipLaunchKernelGGL((attend_mfma_kernel<D, NG, SPARSE, CAUSAL, 4, 2, false>), grid, dim3(64 * 4), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (NG == 1 && !CAUSAL && W == 8) {
    constexpr int kR = SPARSE ? 4 * (2 + 1) : 4 * (3 + 2);  // the uneven split's round of tiles
    if (a.chunk >= 2 * kR * kStep) {
      hipLaunchKernelGGL((attend_mfma_kernel<D, NG, SPARSE, CAUSAL, W, S, false, true>), grid, dim3(64 * W), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attend_mfma_kernel<D, NG, SPARSE, CAUSAL, W, S, false>), grid, dim3(64 * W), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int rows, bool sparse, bool causal, const AttendArgs& a, hipStream_t s) {
  if (sparse) return rows <= 16 ? launch_k<D, 1, true, false>(a, s) : hipErrorInvalidValue;
  if (!causal) return rows <= 16 ? launch_k<D, 1, false, false>(a, s) : hipErrorInvalidValue;
  if (rows <= 16) return launch_k<D, 1, false, true>(a, s);
  if (rows <= 32) return launch_k<D, 2, false, true>(a, s);
  if (rows <= 48) return launch_k<D, 3, false, true>(a, s);
  if (rows <= 64) return launch_k<D, 4, false, true>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

int attend_mfma_granule(int rows, int d) {
  const int w = rows > 48 ? (d == 128 ? mfma_waves<128, 4>() : mfma_waves<64, 4>()) : 8;
  return w * kStep;
}
int attend_mfma_sparse_max_chunk() { return kSparseMaxChunk; }
int attend_mfma_narrow_granule() { return 4 * kStep; }
int attend_mfma_max_rows() { return 64; }

hipError_t launch_attend_mfma(int d, bool sparse, bool causal, const AttendArgs& a, hipStream_t s) {
  const int rows = a.group * a.n_pos;
  if (rows < 1) return hipErrorInvalidValue;
  if (d == 128) return launch_d<128>(rows, sparse, causal, a, s);
  if (d == 64) return launch_d<64>(rows, sparse, causal, a, s);
  return hipErrorInvalidValue;
}

}  // namespace skv
