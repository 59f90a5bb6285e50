/* sparsekv.h -- C ABI of libsparsekv: single-sequence decode attention over a
 * long KV cache with sparse top-K KV selection, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [StD] "Sparse-to-Dense: A Free Lunch for Lossless Acceleration of Video
 *         Understanding in LLMs": Sec. 3.1 Decoding Procedures (gamma drafted
 *         tokens verified in one dense pass), Sec. 3.2 Model with Sparse
 *         Attention (Cache_s[l] = argTopK of text-query attention averaged over
 *         the text tokens; GQA scores summed within each group; selection per
 *         kv head), Sec. 3.3 I/O complexity analysis, App. A Preliminary.
 *   [BX]  "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
 *         Decoding": "Speedup Across Context" (cache scored once by the last
 *         prompt queries, four sinks, highest-scoring entries per kv head,
 *         every step read by a split-K decoding kernel), header figure (sinks,
 *         scored history, run of recent entries), "The Attention Baseline".
 *   [SV]  blog "Paper Breakdown: SpecVLM" (verifier-guided token pruning for
 *         video speculative decoding): "The SpecVLM Method" (Stage I top-P
 *         retention, Stage II spatially uniform reduction), "The Numbers".
 *   [SMM] blog on SparseMM, "Head Sparsity Emerges from Visual Concept
 *         Responses in MLLMs": method section (Local Window Cache w,
 *         Uniform-Based Cache rho, Score-Preferred Cache; observation window of
 *         the last 32 queries; K = r + b_score per head).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.  Host pointers are marked (host).
 *   - dtype of q, K and V: SKV_BF16 (raw bf16, 2 bytes) or SKV_F32.  Outputs
 *     (out, lse, score) are always fp32.
 *   - K and V share one layout: element (h, j, t) of kv head h, position j,
 *     channel t is at base[h * kv_head_stride + j * kv_pos_stride + t]
 *     (strides in elements; channels contiguous; base and both strides must be
 *     multiples of 16 bytes).
 *   - Query rows are contiguous [rows][Hq][d]; query head g reads kv head
 *     g / G with G = Hq / Hkv.
 *   - Scratch: a caller-provided device workspace of at least
 *     skv_workspace_size() bytes, 256-byte aligned, holding split-K partials
 *     and other per-call intermediates.  Its first SKV_WS_HEADER_BYTES are
 *     reserved counters (the long-row selection's per-head histogram
 *     totals): skv_workspace_init zero-fills them and every call leaves them
 *     zero.  A call that returns SKV_ERR_HIP may have stopped between its
 *     kernels and left them non-zero: call skv_workspace_init before reusing
 *     the workspace.  Two calls that share one workspace must not overlap in
 *     time (same stream, or ordered by events); apart from the zero header,
 *     nothing in it needs to survive between calls.
 *   - Streams: every call only enqueues work on `stream` (a hipStream_t; NULL
 *     is the null stream) and returns without synchronising.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; on a validation error nothing is enqueued.  A failed launch
 *     returns SKV_ERR_HIP.
 *   - Determinism: identical inputs give bit-identical outputs (fixed
 *     reduction orders, no floating-point atomics).  How a key set is cut
 *     into split-K chunks, hence the summation order, depends only on the
 *     call's shapes, and for skv_topk_step and the one-launch path of
 *     skv_select also on the device's compute-unit count (no environment
 *     variable enters it).
 */
#ifndef SPARSEKV_H
#define SPARSEKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SKV_OK = 0,
  SKV_ERR_INVALID_ARG = 1, /* null pointer, bad size, stride, range or alignment */
  SKV_ERR_UNSUPPORTED = 2, /* head_dim not 64/128, group size not supported */
  SKV_ERR_WORKSPACE = 3,   /* workspace smaller than skv_workspace_size() */
  SKV_ERR_HIP = 4          /* a HIP launch failed */
} skv_status;

typedef enum { SKV_F32 = 0, SKV_BF16 = 1 } skv_dtype;

#define SKV_WS_HEADER_BYTES 1048576

typedef struct {
  int32_t n_q_heads;      /* Hq (layers x heads may be flattened into heads)     */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0; G = Hq / Hkv in 1..8 or 16    */
  int32_t head_dim;       /* d in {64, 128}                                       */
  int32_t dtype;          /* skv_dtype of q, K, V                                 */
  float scale;            /* softmax scale on q.k; <= 0 selects 1/sqrt(d)         */
  int32_t reserved;       /* must be 0                                            */
  int64_t kv_head_stride; /* elements between kv heads (>= n_cap * kv_pos_stride) */
  int64_t kv_pos_stride;  /* elements between positions (>= d)                    */
} skv_problem;

/* Bytes of workspace every call below needs for caches of length <= n_max and
 * at most rows_max query rows per call (n_obs for skv_score, gamma for
 * skv_verify, 1 otherwise).  Returns 0 for an invalid problem. */
size_t skv_workspace_size(const skv_problem* p, int64_t n_max, int32_t rows_max);

/* Zero-fill the workspace's reserved header (enqueued on `stream`, with a
 * fill kernel so it may sit inside a captured graph). */
skv_status skv_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Score ([StD] Sec. 3.2 equation and GQA rule; [SMM] observation window;
 * [BX] scoring by the last prompt queries).  q: [n_obs][Hq][d]; window query i
 * sits at position n - n_obs + i and sees keys j <= n - n_obs + i.  With
 * l = scale * q.k and P the row's softmax over its visible keys,
 *   score[h * score_stride + j] = (1/n_obs) * sum_{g in group h} sum_i P_{g,i}(j)
 * for j < n (0 for keys no window query sees).  n_obs = 1 is the per-step score
 * of the decode query at position n - 1.  Requires 1 <= n_obs <= n,
 * score_stride >= n.  bf16 windows run as one matrix-core pass; fp32 windows
 * as n_obs per-step scores over the rows' prefixes, added in row order. */
skv_status skv_score(const skv_problem* p, const void* q, int32_t n_obs, const void* k,
                     int64_t n, float* score, int64_t score_stride, void* ws,
                     size_t ws_bytes, void* stream);

/* Select ([BX] sinks + highest-scoring entries + recent run; [SMM] top-K by
 * window score with the local window kept apart; [StD] argTopK per kv head).
 *   recent window = [max(n - n_recent, 0), n): not written, attended as the tail
 *   sinks         = [0, min(n_sink, max(n - n_recent, 0)))
 *   candidates    = [n_sink, n - n_recent) (empty if n_sink >= n - n_recent)
 * Keeps K_h = clamp(k_per_head ? k_per_head[h] : k_uniform, 0, #candidates)
 * candidates, ordered by (score descending, index ascending) on the fp32 bits
 * (-0.0 equals +0.0).  Writes idx[h * idx_stride + i], i < count[h], the sinks
 * and kept candidates in ascending order, and count[h] = #sinks + K_h.
 * k_per_head is a device array or NULL; k_max (host) bounds every K_h and
 * idx_stride >= n_sink + k_max.  Scores must be finite.
 * Long rows with few kv heads (n > 16384, n_kv_heads < 64) keep running
 * histogram totals in the workspace header: it must be zero when the call
 * starts (skv_workspace_init once after allocating the workspace; the call
 * leaves it zero again). */
skv_status skv_select(const skv_problem* p, const float* score, int64_t score_stride,
                      int64_t n, int32_t n_sink, int32_t n_recent,
                      const int32_t* k_per_head, int32_t k_uniform, int32_t k_max,
                      int32_t* idx, int64_t idx_stride, int32_t* count, void* ws,
                      size_t ws_bytes, void* stream);

/* Verifier-guided selection ([SV] "The SpecVLM Method": Stage I top-P
 * retention, Stage II spatially uniform reduction).  Sinks, recent window and
 * candidates are split as in skv_select.  Per score row h (or, pooled = 1, once
 * on the per-candidate sum over all n_kv_heads rows, the set then written to
 * every row):
 *   score    a_j = the fp32 score; pooled: the rows' scores added in double in
 *            ascending row order, rounded to the nearest fp32 (saturating at
 *            the largest finite fp32);
 *   Stage I  V_R = the shortest prefix of the candidates ordered by
 *            (a descending, index ascending) whose summed a is >= lambda times
 *            the sum of every candidate's a, in exact arithmetic (every fp32
 *            is an integer multiple of 2^-149; lambda is taken as the exact
 *            value of the double; c = |V_R|);
 *   Stage II B = round((1 - prune_ratio) * #candidates) (double product,
 *            halves away from zero); the L = #candidates - c leftovers, in
 *            index order, are sampled at ranks floor(i L / n_U), i < n_U, with
 *            n_U = clamp(B - c, 0, L) (fill_mode 0: the kept set is brought to
 *            B) or n_U = min(B, L) (fill_mode 1: B uniform picks on top of V_R).
 * Writes idx[h * idx_stride + i], i < count[h]: sinks, V_R and the uniform
 * picks in ascending order; count_r[h] = c (device, may be NULL).  Scores are
 * finite and >= 0 (others count as zero mass).  Requires 0 <= lambda <= 1,
 * 0 <= prune_ratio <= 1, idx_stride >= #sinks + #candidates; pooled = 1 needs
 * a workspace (skv_workspace_size covers it). */
skv_status skv_select_topp(const skv_problem* p, const float* score, int64_t score_stride,
                           int64_t n, int32_t n_sink, int32_t n_recent, double lambda,
                           double prune_ratio, int32_t pooled, int32_t fill_mode, int32_t* idx,
                           int64_t idx_stride, int32_t* count, int32_t* count_r, void* ws,
                           size_t ws_bytes, void* stream);

/* Sparse decode attention ([StD] Sec. 3.2 top-K attention, Sec. 3.3 draft
 * reads K selected entries plus the text run; [BX] kept set read by one
 * split-K kernel call).  The decode query q [Hq][d] attends, per kv head h, to
 * idx[h * idx_stride + i] for i < count[h] followed by the contiguous tail
 * [tail_start, n).  Every idx entry must be unique and < tail_start;
 * 0 <= count[h] <= idx_stride (device values, checked by the kernel only
 * against idx_stride).  Writes out [Hq][d] and lse [Hq] (natural-log
 * normaliser of scale * q.k over the set; -inf and out = 0 for an empty set;
 * lse may be NULL). */
skv_status skv_attend_sparse(const skv_problem* p, const void* q, const void* k,
                             const void* v, int64_t n, const int32_t* idx,
                             int64_t idx_stride, const int32_t* count, int64_t tail_start,
                             float* out, float* lse, void* ws, size_t ws_bytes,
                             void* stream);

/* skv_attend_sparse without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus ws, ws_bytes),
 * validation, kernels and results as skv_attend_sparse.  Its scratch is a
 * fixed array of SKV_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends; the first call on a device looks it up and
 * enqueues a fill kernel on `stream` that clears its header.  A call whose
 * scratch (SKV_WS_HEADER_BYTES plus the partials of its split-K plan, the
 * same amount skv_workspace_size reserves for it) exceeds that size returns
 * SKV_ERR_WORKSPACE and enqueues nothing.  No call allocates or frees
 * memory.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams, or different host threads without
 * ordering) race and give undefined results. */
#define SKV_NOALLOC_SCRATCH_BYTES (16 * 1048576)
skv_status skv_attend_sparse_noalloc(const skv_problem* p, const void* q, const void* k,
                                     const void* v, int64_t n, const int32_t* idx,
                                     int64_t idx_stride, const int32_t* count,
                                     int64_t tail_start, float* out, float* lse, void* stream);

/* Dense decode attention ([BX] "The Attention Baseline": the dense step reads
 * the whole cache through the same split-K kernel): q [Hq][d] over keys
 * [0, n).  out [Hq][d], lse [Hq] (may be NULL). */
skv_status skv_attend_dense(const skv_problem* p, const void* q, const void* k,
                            const void* v, int64_t n, float* out, float* lse, void* ws,
                            size_t ws_bytes, void* stream);

/* Verify ([StD] Sec. 3.1: the dense model checks all gamma drafted tokens in
 * one pass over the full cache).  The gamma new entries already occupy
 * positions n - gamma .. n - 1; query t (q [gamma][Hq][d]) sits at n - gamma + t
 * and sees keys [0, n - gamma + t].  out [gamma][Hq][d], lse [gamma][Hq] (may be
 * NULL).  Requires 1 <= gamma <= min(n, 16).  bf16: a kernel pass holds at
 * most 64 query rows (gamma * G) per kv head; more run as successive passes of
 * floor(64 / G) queries, each over the prefix its queries see.  fp32: one
 * decode step per query over its prefix. */
skv_status skv_verify(const skv_problem* p, const void* q, int32_t gamma, const void* k,
                      const void* v, int64_t n, float* out, float* lse, void* ws,
                      size_t ws_bytes, void* stream);

/* The per-step top-K decode step ([StD] Sec. 3.2 top-K attention: the keys
 * with the largest group-summed attention score of the current query; [BX]
 * "Speedup Across Context": sinks, the selected history and the recent run,
 * read by split-K attention), as one call.  Equivalent to
 *   skv_score (n_obs = 1) -> skv_select (k_uniform = k_max = k_top)
 *   -> skv_attend_sparse (tail_start = max(n - n_recent, 0))
 * with the same arguments: writes score [Hkv][score_stride] (required),
 * idx / count, out [Hq][d] and lse [Hq] (may be NULL).  With bf16 caches, at
 * most 64 kv heads and a cache short enough that each kv head's keys split
 * over CUs / Hkv workgroups keep their logits in LDS (128K context at G = 4
 * on 256 CUs), it runs as one kernel whose workgroups take their work in
 * start order and meet at per-kv-head barriers (see the kernel's
 * description), followed by the split-K merge kernel; otherwise it runs the
 * three calls.  Scores equal
 * skv_score's bit for bit; the selection is skv_select's on those scores;
 * the attention is exact over the same set (its summation order differs
 * from skv_attend_sparse's).  The workspace (skv_workspace_size) also holds
 * the step's counters in the reserved header (zero after
 * skv_workspace_init, cleared again at the end of every step); a word at
 * byte SKV_TOPK_ERROR_OFFSET of the workspace is set non-zero if a workgroup
 * of the one-launch form ever waited too long for the others of its kv head
 * (only when other work holds the device's CUs); that step's results are
 * then unspecified.  Two steps on one workspace must not overlap in time. */
#define SKV_TOPK_ERROR_OFFSET (SKV_WS_HEADER_BYTES - 64 * 128 - 128)
skv_status skv_topk_step(const skv_problem* p, const void* q, const void* k, const void* v,
                         int64_t n, int32_t n_sink, int32_t n_recent, int32_t k_top,
                         float* score, int64_t score_stride, int32_t* idx, int64_t idx_stride,
                         int32_t* count, float* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/* Compaction ([BX] "Speedup Across Context": the kept entries are gathered
 * once into a contiguous buffer that every later step reads with one kernel
 * call).  For each kv head h, copies K and V rows idx[h * idx_stride + i],
 * i < count[h], then the tail [tail_start, n), to rows 0 .. rows_h - 1 of the
 * output cache, rows_h = count[h] + (n - tail_start); row r of head h is at
 * k_out / v_out + h * out_head_stride + r * out_pos_stride (elements of the
 * problem's dtype, same alignment rules as the input cache).  The output must
 * hold rows_max = min(idx_stride, tail_start) + (n - tail_start) rows per
 * head; rows at or beyond rows_h are left untouched.  rows_out (device, may be
 * NULL) receives rows_h.  On the device count[h] is clamped to
 * [0, min(idx_stride, tail_start)] and index entries to [0, n), so every write
 * stays inside rows_max rows; the copy is exact (bytes).  With equal
 * counts on every head the output is an ordinary cache of rows_h positions
 * for skv_attend_dense, which then gives the result of skv_attend_sparse on
 * the same set.  Input and output must not overlap. */
skv_status skv_gather(const skv_problem* p, const void* k, const void* v, int64_t n,
                      const int32_t* idx, int64_t idx_stride, const int32_t* count,
                      int64_t tail_start, void* k_out, void* v_out, int64_t out_head_stride,
                      int64_t out_pos_stride, int32_t* rows_out, void* stream);

/* Per-head budgets ([SMM] method section), host only.  For N heads with
 * visual scores s (host), total budget B, local window w and share rho:
 *   r = rho (B - N w) / N,  B_remain = B - N w - rho (B - N w),
 *   b_score_i = B_remain s_i / sum s,   b_i = w + r + b_score_i.
 * Writes k_out[i] = floor(r + b_score_i) clamped to [0, n_cand] (host) and,
 * if b_out is not NULL, b_i (host). */
skv_status skv_budgets(const double* s, int32_t n_heads, double total_budget, int32_t window,
                       double rho, int64_t n_cand, int32_t* k_out, double* b_out);

const char* skv_status_string(skv_status s);
int32_t skv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEKV_H */
