// skv_kernels.h -- launch descriptors shared by the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

// Split-K decode attention over a per-kv-head row list.
//   dense : rows of head h are positions [0, n)
//   sparse: rows of head h are idx[h][0..count[h]) followed by [tail_start, n)
struct AttendArgs {
  const void* q;            // [n_pos][Hq][d]
  const char* k;            // byte pointer to element (0,0,0)
  const char* v;
  int64_t head_stride_b;    // bytes between kv heads
  int64_t pos_stride_b;     // bytes between positions
  int64_t n;
  const int32_t* idx;       // sparse only
  int64_t idx_stride;
  const int32_t* count;     // sparse only
  int64_t count_max;        // sparse only: counts are clamped to [0, count_max]
  int64_t tail_start;       // sparse only
  int32_t n_kv_heads;
  int32_t chunk;            // rows per workgroup
  int32_t chunks_per_head;  // grid = n_kv_heads * chunks_per_head
  float scale_log2;         // scale * log2(e)
  float* part_ml;           // [Hkv][chunks_per_head][R][2]  (max in log2 units, sum)
  float* part_acc;          // [Hkv][chunks_per_head][R][d]
  int32_t* nch;             // [Hkv] chunks actually used per kv head
  int32_t group;            // G = Hq / Hkv
  int32_t n_pos;            // query positions (1 for a decode step); R = n_pos * G rows
  // Work-list mode (gathered rows, many kv heads with ragged counts): a small
  // kernel lists the (kv head, chunk) pairs that hold rows, and list_grid
  // workgroups walk that list.  items == nullptr: one workgroup per pair.
  int2* items;              // [n_kv_heads * chunks_per_head]
  int32_t* n_items;
  int32_t list_grid;
  // Four-wave workgroups (chunks a multiple of attend_mfma_narrow_granule())
  // for decode calls too small to fill the CUs with eight-wave ones.
  int32_t narrow;
};

hipError_t launch_attend(int dtype, int d, int g, bool sparse, const AttendArgs& a,
                         hipStream_t stream);

// Log-sum-exp merge of split-K partials: for output row r of kv head h,
//   M = max_c m_c, L = sum_c l_c 2^(m_c - M), out = sum_c acc_c 2^(m_c - M) / L,
//   lse = (M + log2 L) ln 2  (-inf and out = 0 when L = 0).
// Row r of head h goes to query row (r / G) * Hq + h * G + r % G.
struct MergeArgs {
  const float* part_ml;     // [Hkv][cph][rows_per_head][2]
  const float* part_acc;    // [Hkv][cph][rows_per_head][d]
  const int32_t* nch;       // [Hkv], or null when every kv head uses cph chunks
  int32_t n_kv_heads, cph, rows_per_head, group;
  float* out;
  float* lse;               // may be null
  uint32_t* clear_ctr;      // may be null: words 32 h and 32 h + 16, h < clear_heads, set to zero
  int32_t clear_heads;
};
hipError_t launch_merge(int d, const MergeArgs& a, hipStream_t stream);
// Rows per wave iteration of the attend kernel (the chunk must be a multiple
// of 4x this).
int attend_rows_per_iter(int dtype, int d);

// bf16 caches: the matrix-core variant of the split-K partial kernel (same
// partial format).  R = n_pos * G <= attend_mfma_max_rows() query rows per kv
// head; causal: row (t, g) sees keys j <= n - n_pos + t (dense only).  Chunks
// are multiples of attend_mfma_granule(R, d); the sparse variant stages at most
// attend_mfma_sparse_max_chunk() row offsets.
hipError_t launch_attend_mfma(int d, bool sparse, bool causal, const AttendArgs& a,
                              hipStream_t stream);
int attend_mfma_granule(int rows, int d);
int attend_mfma_sparse_max_chunk();
int attend_mfma_narrow_granule();
int attend_mfma_max_rows();

// Per-step score (one decode query): phase 1 writes log2-domain logits and
// per-chunk (max, sum) per query head; phase 2 normalises and group-sums.
struct ScoreStepArgs {
  const void* q;            // [Hq][d]
  const char* k;
  int64_t head_stride_b, pos_stride_b;
  int64_t n;
  int32_t n_kv_heads;
  int32_t chunk, chunks_per_head;
  float scale_log2;
  float* logits;            // [Hq][logits_stride] (log2 domain)
  int64_t logits_stride;    // >= n; a multiple of 4 for 16-byte stores
  float* part_ml;           // [Hkv][chunks_per_head][G][2]
  float* score;             // [Hkv][score_stride]
  int64_t score_stride;
};
hipError_t launch_score_step(int dtype, int d, int g, const ScoreStepArgs& a, hipStream_t stream);
// bf16 runs phase 1 on the matrix cores: chunks are multiples of this and
// hold at most score_step_mfma_max_chunk(G) keys (their logits stay in LDS).
int score_step_mfma_granule();
int score_step_mfma_max_chunk(int g);

// Observation-window score on MFMA (bf16 only): W queries x G heads per kv head.
struct ScoreObsArgs {
  const uint16_t* q;        // [W][Hq][d] bf16
  const char* k;
  int64_t head_stride_b, pos_stride_b;
  int64_t n;
  int32_t n_obs;            // W
  int32_t n_kv_heads, group;
  int32_t n_kblocks;        // key blocks of score_obs_block_keys() per head
  float scale_log2;
  float* part_ml;           // [Hkv][n_kblocks][R][2], R = W * G
  float* row_lse2;          // [Hkv][R]
  float* score;
  int64_t score_stride;
  // Query rows split into row_groups workgroups per (kv head, key block) when
  // there are few key blocks; each group's key sums go to part_score
  // [row_groups][Hkv][n] and a last kernel adds them in group order.
  int32_t row_groups;
  float* part_score;
};
hipError_t launch_score_obs(int d, const ScoreObsArgs& a, hipStream_t stream);
// Query rows per staged chunk of the window score (row groups split chunks).
int score_obs_chunk_rows();

// Sinks + top-K selection by radix select on order-preserving score keys.
struct SelectArgs {
  const float* score;
  int64_t score_stride;
  int64_t n;
  int32_t n_sink, n_recent;
  const int32_t* k_per_head;  // device, may be null
  int32_t k_uniform;
  int32_t k_max;              // bound on every K_h (idx row capacity minus sinks)
  int32_t* idx;
  int64_t idx_stride;
  int32_t* count;
  int32_t n_kv_heads;
  void* ws;                   // scratch of the block-parallel path (select_ws_bytes)
  uint32_t* totals;           // block path: first-level head totals, zero on entry, left zero
};
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
// Scratch the block-parallel select needs (0 when the one-workgroup-per-head
// path is used for this shape).
size_t select_ws_bytes(int32_t n_kv_heads, int64_t n);

// Fill count words with zero (a kernel, so it may sit in a captured graph).
hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t stream);
// y[r][j] += w x[r][j] (j < nx) over `rows` rows; `first` writes instead and
// clears j in [nx, ny)
hipError_t launch_add_rows(float* y, int64_t ys, const float* x, int64_t xs, int rows, int64_t nx, int64_t ny,
                           float w, bool first, hipStream_t stream);

// Verifier-guided top-P retention + uniform fill (skv_select_topp).
struct ToppArgs {
  const float* score;
  int64_t score_stride;
  int32_t rows;             // score rows (kv heads)
  int32_t pooled;           // 1: one selection on the sum over rows, given to every row
  int64_t n;
  int32_t n_sink, n_recent;
  uint64_t lam_m;           // lambda = lam_m / 2^lam_sh exactly
  int32_t lam_sh;
  int32_t fill_mode;        // 0: fill up to the budget; 1: budget uniform picks
  int64_t budget;           // round((1 - r) * candidates)
  int32_t* idx;
  int64_t idx_stride;
  int32_t* count;
  int32_t* count_r;         // may be null
  uint32_t* pooled_row;     // pooled, beyond 32K candidates: each candidate's pooled fp32 bits (scratch)
};
hipError_t launch_select_topp(const ToppArgs& a, hipStream_t stream);

// The per-step top-K decode step in one launch (skv_topk_step): score of one
// decode query, sinks + top-K + recent run, attention over the kept set.
// bf16 caches; one workgroup per (kv head, chunk); a kv head's workgroups
// take their chunks in start order from the head's ticket and meet at bounded
// spin barriers (progress needs (P - 1) Hkv + 1 workgroups resident at once).
struct TopkArgs {
  const void* q;            // [Hq][d]
  const char* k;
  const char* v;
  int64_t head_stride_b, pos_stride_b;
  int64_t n;
  int32_t n_sink, n_recent;
  int64_t k_top;            // candidates kept by score (clamped to the candidate count)
  int32_t n_kv_heads;
  int32_t chunk;            // keys per workgroup, a multiple of topk_step_granule()
  int32_t chunks_per_head;  // P
  float scale_log2;
  float* score;             // [Hkv][score_stride], may be null
  int64_t score_stride;
  int32_t* idx;             // [Hkv][idx_stride]: sinks, then the top-K, ascending
  int64_t idx_stride;
  int32_t* count;           // [Hkv]
  float* out;               // [Hq][d]
  float* lse;               // [Hq], may be null
  uint32_t* ctr;            // per kv head 32 words: arrivals (word 0), ticket (word 16); zero on entry, cleared by the merge
  uint32_t* err;            // set to 1 if a barrier spin ran out
  int32_t pub_cap;          // set by the launch
  const int32_t* k_per_head;  // [Hkv] or null (selection alone; the step keeps k_top)
};
hipError_t launch_topk_step(int d, int g, const TopkArgs& a, void* scratch, hipStream_t stream);
int topk_step_max_chunk(int g, int d);
int topk_step_granule();
size_t topk_step_scratch(int hkv, int p, int g, int d);
// The same kernel doing the selection alone (skv_select, long rows with few kv
// heads): `score` is read, q/k/v/out unused; chunks of at most
// topk_select_max_chunk() scores; no merge launch (the last arrival clears
// the counters).
hipError_t launch_topk_select(const TopkArgs& a, void* scratch, hipStream_t stream);
int topk_select_max_chunk();
int topk_publish_budget();  // keys a kv head's chunks may publish in all
size_t topk_select_scratch(int hkv, int p);

// Compaction of a kept set (skv_gather).
struct GatherArgs {
  const char* k;
  const char* v;
  int64_t head_stride_b, pos_stride_b;
  int64_t n;
  const int32_t* idx;
  int64_t idx_stride;
  const int32_t* count;
  int64_t count_max;        // min(idx_stride, tail_start)
  int64_t tail_start;
  char* k_out;
  char* v_out;
  int64_t out_head_stride_b, out_pos_stride_b;
  int64_t rows_max;
  int32_t* rows_out;        // may be null
  int32_t n_kv_heads;
  int32_t row_bytes;        // d * element bytes
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);

}  // namespace skv
