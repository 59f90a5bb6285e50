// api.hip -- the C ABI of libsparsekv: argument validation (before anything is
// enqueued), workspace carving, launch planning and status mapping.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/sparsekv.h"
#include "skv_kernels.h"

namespace skv {
int attend_max_chunk();
int attend_waves();
int score_obs_block_keys();
}

namespace {

using skv::AttendArgs;

constexpr size_t kAlign = 256;
constexpr int64_t kCounterSlots = SKV_WS_HEADER_BYTES / 4;
// The header's last 8 KB: per-kv-head counters of skv_topk_step (one 128-byte
// line each, up to 64 kv heads: arrivals and the chunk ticket), and just below
// them its error word.  The long-row select uses at most 63 x 16 KB from the
// start of the header.
constexpr size_t kTopkCtrOffset = SKV_WS_HEADER_BYTES - 64 * 128;
constexpr size_t kTopkErrOffset = kTopkCtrOffset - 128;
constexpr int kTopkMaxKvHeads = 64;
static_assert(kTopkErrOffset == SKV_TOPK_ERROR_OFFSET, "documented error word");
static_assert((size_t)63 * 4096 * 4 <= kTopkErrOffset, "select totals and step counters are disjoint");
// Generous bound on the CUs of one device (sizes the step's scratch).
constexpr int kMaxCUs = 1024;
constexpr int kVerifyMaxGamma = 16;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// query heads per kv head: 1 .. 8 and 16 (the kernels are instantiated per size)
bool group_supported(int g) { return (g >= 1 && g <= 8) || g == 16; }

// Workgroup count the split-K attention aims for: one per CU on 256 CUs
// (measured best on MI355X for 32K-128K; more chunks only add merge work).
// A constant, so a plan -- and with it the summation order -- depends on the
// call's shapes alone.
constexpr int target_wgs() { return 256; }

struct ChunkPlan {
  int chunk;  // rows per workgroup
  int cph;    // chunks per kv head
  bool list = false;    // work-list mode (see AttendArgs::items)
  bool narrow = false;  // four-wave workgroups (see AttendArgs::narrow)
};

// Split rows_bound rows per kv head into chunks: about target_wgs() workgroups
// in total, chunk a multiple of `granule`, at most `max_chunk`.
ChunkPlan plan_chunks(int64_t rows_bound, int hkv, int granule, int max_chunk) {
  const int64_t want = (target_wgs() + hkv - 1) / hkv;
  int64_t chunk = (rows_bound + want - 1) / (want < 1 ? 1 : want);
  chunk = (chunk + granule - 1) / granule * granule;
  if (chunk < granule) chunk = granule;
  if (chunk > max_chunk) chunk = max_chunk;
  int64_t cph = (rows_bound + chunk - 1) / chunk;
  if (cph < 1) cph = 1;
  return {(int)chunk, (int)cph};
}

float scale_log2(const skv_problem* p) {
  const float sc = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  return sc * 1.4426950408889634f;
}

int elem_size(const skv_problem* p) { return p->dtype == SKV_BF16 ? 2 : 4; }

skv_status check_problem(const skv_problem* p) {
  if (!p) return SKV_ERR_INVALID_ARG;
  if (p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->n_q_heads % p->n_kv_heads != 0)
    return SKV_ERR_INVALID_ARG;
  if (p->dtype != SKV_F32 && p->dtype != SKV_BF16) return SKV_ERR_INVALID_ARG;
  if (p->reserved != 0) return SKV_ERR_INVALID_ARG;
  if (!(p->scale == p->scale) || isinf(p->scale)) return SKV_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return SKV_ERR_UNSUPPORTED;
  if (!group_supported(p->n_q_heads / p->n_kv_heads)) return SKV_ERR_UNSUPPORTED;
  if (p->n_kv_heads > kCounterSlots) return SKV_ERR_UNSUPPORTED;
  return SKV_OK;
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15u) == 0; }

// Cache pointer, strides and length n: rows of one head must not run into the
// next head, and every 16-byte lane slice must be aligned.
skv_status check_cache(const skv_problem* p, const void* kv, int64_t n) {
  if (!kv || !aligned16(kv)) return SKV_ERR_INVALID_ARG;
  if (p->kv_pos_stride < p->head_dim) return SKV_ERR_INVALID_ARG;
  if ((p->kv_pos_stride * elem_size(p)) % 16 != 0) return SKV_ERR_INVALID_ARG;
  if ((p->kv_head_stride * elem_size(p)) % 16 != 0) return SKV_ERR_INVALID_ARG;
  if (p->n_kv_heads > 1 && p->kv_head_stride < n * p->kv_pos_stride) return SKV_ERR_INVALID_ARG;
  if (p->kv_head_stride < 0) return SKV_ERR_INVALID_ARG;
  // rows of one head (plus one 16-row tile read past the end and masked) are
  // addressed with 32-bit byte offsets
  if ((double)(n + 16) * (double)p->kv_pos_stride * elem_size(p) >= 4294967296.0)
    return SKV_ERR_UNSUPPORTED;
  return SKV_OK;
}

skv_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ((uintptr_t)ws % kAlign) != 0) return SKV_ERR_INVALID_ARG;
  if (ws_bytes < need) return SKV_ERR_WORKSPACE;
  return SKV_OK;
}

skv_status hip_status(hipError_t e) { return e == hipSuccess ? SKV_OK : SKV_ERR_HIP; }

// ---- per-call workspace requirements (reserved header + scratch) -----------

// chunk granule: one iteration of rows for every wave of a workgroup
// bf16 caches run the matrix-core partial kernel, fp32 caches the vector one.
bool attend_uses_mfma(const skv_problem* p) { return p->dtype == SKV_BF16; }

int attend_granule(const skv_problem* p) {
  if (attend_uses_mfma(p)) return skv::attend_mfma_granule(p->n_q_heads / p->n_kv_heads, p->head_dim);
  return skv::attend_waves() * skv::attend_rows_per_iter(p->dtype, p->head_dim);
}

// Gathered rows with many kv heads: counts are device values and may be very
// uneven (per-head budgets), so a grid sized by the largest head would be
// mostly empty workgroups.  Beyond twice the target workgroup count the call
// runs in work-list mode with chunks of kListChunk rows.
constexpr int kListChunk = 512;

ChunkPlan attend_plan(const skv_problem* p, int64_t rows_bound, bool sparse) {
  int max_chunk;
  if (attend_uses_mfma(p))  // dense chunks need no per-row LDS, so they may grow
    max_chunk = sparse ? skv::attend_mfma_sparse_max_chunk() : (1 << 20);
  else
    max_chunk = sparse ? 512 : skv::attend_max_chunk();
  ChunkPlan cp = plan_chunks(rows_bound, p->n_kv_heads, attend_granule(p), max_chunk);
  if (sparse && attend_uses_mfma(p) && (int64_t)p->n_kv_heads * cp.cph > 2 * (int64_t)target_wgs()) {
    cp.chunk = kListChunk;
    cp.cph = (int)((rows_bound + kListChunk - 1) / kListChunk);
    if (cp.cph < 1) cp.cph = 1;
    cp.list = true;
  }
  // Small calls (e.g. a draft step over a few thousand kept rows) leave most
  // CUs idle with eight-wave workgroups: halve the workgroups' width instead.
  const int G = p->n_q_heads / p->n_kv_heads;
  if (!cp.list && attend_uses_mfma(p) && G <= 16 &&
      (int64_t)p->n_kv_heads * cp.cph <= (int64_t)target_wgs() / 2) {
    const ChunkPlan n4 = plan_chunks(rows_bound, p->n_kv_heads, skv::attend_mfma_narrow_granule(), max_chunk);
    if (n4.cph > cp.cph) {
      cp = n4;
      cp.narrow = true;
    }
  }
  return cp;
}

hipError_t launch_attend_any(const skv_problem* p, bool sparse, const skv::AttendArgs& a,
                             hipStream_t s) {
  const int G = p->n_q_heads / p->n_kv_heads;
  if (attend_uses_mfma(p)) return skv::launch_attend_mfma(p->head_dim, sparse, false, a, s);
  return skv::launch_attend(p->dtype, p->head_dim, G, sparse, a, s);
}

// Split-K scratch: partial (max, sum) and acc[d] per (kv head, chunk, row),
// then the chunk count of every kv head.
struct PartLayout {
  size_t ml, acc, nch, items, n_items, end;
};

// ... then the work list of (kv head, chunk) pairs and its length.
PartLayout part_layout(const skv_problem* p, int cph, int rows_per_head) {
  const size_t slots = (size_t)p->n_kv_heads * cph * rows_per_head;
  PartLayout L;
  L.ml = SKV_WS_HEADER_BYTES;
  L.acc = L.ml + align_up(slots * 2 * sizeof(float));
  L.nch = L.acc + align_up(slots * p->head_dim * sizeof(float));
  L.items = L.nch + align_up((size_t)p->n_kv_heads * sizeof(int32_t));
  L.n_items = L.items + align_up((size_t)p->n_kv_heads * cph * 2 * sizeof(int32_t));
  L.end = L.n_items + align_up(sizeof(int32_t));
  return L;
}

// Chunk counts are not monotone in the row count: one row more can round the
// chunk up to the next granule and halve the count (4096 rows of 8 kv heads:
// 32 chunks of 128; 4097 rows: 17 of 256).  Scratch is therefore sized for
// the larger of a plan's count and the target count per kv head; that bound
// never decreases with the rows, so a workspace sized for n_max serves every
// smaller call (a plan's chunks hold at least rows / target rows unless
// capped, and capped counts grow with the rows).
int cph_bound(const skv_problem* p, int cph) {
  const int want = (target_wgs() + p->n_kv_heads - 1) / p->n_kv_heads;
  return cph > want ? cph : want;
}

size_t attend_scratch(const skv_problem* p, const ChunkPlan& cp) {
  const int G = p->n_q_heads / p->n_kv_heads;
  return part_layout(p, cph_bound(p, cp.cph), G).end - SKV_WS_HEADER_BYTES;
}

skv_status launch_partials_merge(const skv_problem* p, char* base, const PartLayout& L, int cph,
                                 int rows_per_head, bool ragged, float* out, float* lse,
                                 hipStream_t s) {
  skv::MergeArgs m{};
  m.part_ml = (const float*)(base + L.ml);
  m.part_acc = (const float*)(base + L.acc);
  m.nch = ragged ? (const int32_t*)(base + L.nch) : nullptr;
  m.n_kv_heads = p->n_kv_heads;
  m.cph = cph;
  m.rows_per_head = rows_per_head;
  m.group = p->n_q_heads / p->n_kv_heads;
  m.out = out;
  m.lse = lse;
  return hip_status(skv::launch_merge(p->head_dim, m, s));
}

ChunkPlan score_step_plan(const skv_problem* p, int64_t n) {
  if (p->dtype == SKV_BF16)
    return plan_chunks(n, p->n_kv_heads, skv::score_step_mfma_granule(),
                       skv::score_step_mfma_max_chunk(p->n_q_heads / p->n_kv_heads));
  return plan_chunks(n, p->n_kv_heads, 4 * skv::attend_rows_per_iter(p->dtype, p->head_dim),
                     skv::attend_max_chunk());
}

// Logits rows are padded to a multiple of 4 keys (16-byte stores).
int64_t logits_stride(int64_t n) { return (n + 3) / 4 * 4; }

size_t score_step_scratch(const skv_problem* p, int64_t n) {
  const ChunkPlan cp = score_step_plan(p, n);
  const int G = p->n_q_heads / p->n_kv_heads;
  return align_up((size_t)p->n_q_heads * logits_stride(n) * sizeof(float)) +
         align_up((size_t)p->n_kv_heads * cph_bound(p, cp.cph) * G * 2 * sizeof(float));
}

// fp32 window score: the per-step scratch plus one row block [Hkv][n] that
// holds each window row's score before it is added in.
size_t score_window_f32_scratch(const skv_problem* p, int64_t n) {
  return score_step_scratch(p, n) + align_up((size_t)p->n_kv_heads * logits_stride(n) * sizeof(float));
}

// Window-score row groups: with few (kv head, key block) workgroups the query
// rows are split so that the grid holds at least 4 x target workgroups (at
// most one group per staged chunk of rows).
int obs_row_groups(const skv_problem* p, int64_t nkb, int64_t R) {
  const int64_t wgs = (int64_t)p->n_kv_heads * nkb;
  const int64_t want = 4 * (int64_t)target_wgs();
  if (wgs >= want) return 1;
  const int64_t nch = (R + skv::score_obs_chunk_rows() - 1) / skv::score_obs_chunk_rows();
  int64_t rg = (want + wgs - 1) / wgs;
  rg = rg > nch ? nch : rg;
  return (int)(rg < 1 ? 1 : rg);
}

size_t score_obs_scratch(const skv_problem* p, int64_t n, int32_t n_obs) {
  const int G = p->n_q_heads / p->n_kv_heads;
  const int64_t R = (int64_t)n_obs * G;
  const int64_t nkb = (n + skv::score_obs_block_keys() - 1) / skv::score_obs_block_keys();
  const int rg = obs_row_groups(p, nkb, R);
  return align_up((size_t)p->n_kv_heads * nkb * R * 2 * sizeof(float)) +
         align_up((size_t)p->n_kv_heads * R * sizeof(float)) +
         (rg > 1 ? align_up((size_t)rg * p->n_kv_heads * n * sizeof(float)) : 0);
}

// The verify pass: dense, causal, gamma * G query rows per kv head.
ChunkPlan verify_plan(const skv_problem* p, int64_t n, int32_t gamma) {
  const int rows = gamma * (p->n_q_heads / p->n_kv_heads);
  return plan_chunks(n, p->n_kv_heads, skv::attend_mfma_granule(rows, p->head_dim), 1 << 20);
}

// Verify queries per pass: one pass of the matrix-core kernel holds at most
// attend_mfma_max_rows() query rows per kv head.
int32_t verify_pass_queries(const skv_problem* p, int32_t gamma) {
  const int qc = skv::attend_mfma_max_rows() / (p->n_q_heads / p->n_kv_heads);
  return gamma < qc ? gamma : qc;
}

// Scratch of one verify pass of g queries over a cache of n entries.
size_t verify_pass_scratch(const skv_problem* p, int64_t n, int32_t g) {
  const ChunkPlan cp = verify_plan(p, n, g);
  const int G = p->n_q_heads / p->n_kv_heads;
  return part_layout(p, cph_bound(p, cp.cph), g * G).end - SKV_WS_HEADER_BYTES;
}

// Scratch of a whole verify call: its passes run one after another on one
// workspace, so the largest pass decides.
size_t verify_scratch(const skv_problem* p, int64_t n, int32_t gamma) {
  const int32_t qc = verify_pass_queries(p, gamma);
  size_t s = 0;
  for (int32_t t0 = 0; t0 < gamma; t0 += qc) {
    const int32_t g = gamma - t0 < qc ? gamma - t0 : qc;
    const size_t t = verify_pass_scratch(p, n - gamma + t0 + g, g);
    s = s > t ? s : t;
  }
  return s;
}

// Pooled top-P selection: one fp32 pooled score per candidate.
size_t topp_scratch(int64_t n) { return ((size_t)n * 4 + kAlign - 1) / kAlign * kAlign; }

// Argument checks of a gathered-rows decode call (nothing is enqueued) and
// its split-K plan.
skv_status check_attend_sparse(const skv_problem* p, const void* q, const void* k, const void* v,
                               int64_t n, const int32_t* idx, int64_t idx_stride,
                               const int32_t* count, int64_t tail_start, const float* out,
                               ChunkPlan* cp) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (n < 1 || !q || !out || !aligned16(q) || !aligned16(out)) return SKV_ERR_INVALID_ARG;
  if (!count || (!idx && idx_stride > 0) || idx_stride < 0) return SKV_ERR_INVALID_ARG;
  if (tail_start < 0 || tail_start > n) return SKV_ERR_INVALID_ARG;
  if (n > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  if ((st = check_cache(p, k, n)) != SKV_OK || (st = check_cache(p, v, n)) != SKV_OK) return st;
  const int64_t idx_rows = idx_stride < tail_start ? idx_stride : tail_start;
  *cp = attend_plan(p, idx_rows + (n - tail_start), true);
  return SKV_OK;
}

// The launches of a checked gathered-rows decode call; `base` is a workspace
// of at least SKV_WS_HEADER_BYTES + attend_scratch(p, cp) bytes.
skv_status run_attend_sparse(const skv_problem* p, const ChunkPlan& cp, const void* q,
                             const void* k, const void* v, int64_t n, const int32_t* idx,
                             int64_t idx_stride, const int32_t* count, int64_t tail_start,
                             float* out, float* lse, char* base, hipStream_t stream) {
  const int G = p->n_q_heads / p->n_kv_heads;
  const int64_t idx_rows = idx_stride < tail_start ? idx_stride : tail_start;
  const PartLayout L = part_layout(p, cp.cph, G);
  AttendArgs a{};
  a.q = q;
  a.k = (const char*)k;
  a.v = (const char*)v;
  a.head_stride_b = p->kv_head_stride * elem_size(p);
  a.pos_stride_b = p->kv_pos_stride * elem_size(p);
  a.n = n;
  a.idx = idx;
  a.idx_stride = idx_stride;
  a.count = count;
  a.count_max = idx_rows;  // unique entries below tail_start: never more than this
  a.tail_start = tail_start;
  a.n_kv_heads = p->n_kv_heads;
  a.chunk = cp.chunk;
  a.chunks_per_head = cp.cph;
  a.scale_log2 = scale_log2(p);
  a.part_ml = (float*)(base + L.ml);
  a.part_acc = (float*)(base + L.acc);
  a.nch = (int32_t*)(base + L.nch);
  a.group = G;
  a.n_pos = 1;
  a.narrow = cp.narrow;
  if (cp.list) {
    a.items = (int2*)(base + L.items);
    a.n_items = (int32_t*)(base + L.n_items);
    // four-wave workgroups, two per CU, walking the list
    const int64_t pairs = (int64_t)p->n_kv_heads * cp.cph, cap = 4 * (int64_t)target_wgs();
    a.list_grid = (int32_t)(pairs < cap ? pairs : cap);
  }
  skv_status st = hip_status(launch_attend_any(p, true, a, stream));
  if (st != SKV_OK) return st;
  return launch_partials_merge(p, base, L, cp.cph, G, true, out, lse, stream);
}

// ---- fixed scratch of skv_attend_sparse_noalloc -----------------------------
// For callers that cannot allocate device memory: one array per GPU that the
// library holds until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it names a stand-in, not device memory):
// its device address is looked up once per device with hipGetSymbolAddress
// and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[SKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch; the first call on a device
// looks it up and clears its header (a fill kernel on `stream`: calls on one
// GPU share the array, and the header must read zero on entry).
skv_status noalloc_scratch(char** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SKV_ERR_HIP;
    if (skv::launch_zero_u32((uint32_t*)ptr, kCounterSlots, stream) != hipSuccess) return SKV_ERR_HIP;
    g_scratch_ptr[dev] = (char*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return SKV_OK;
}

// ---- skv_topk_step planning -------------------------------------------------
std::mutex g_cu_mu;
int g_cus[kMaxDevices];

int device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(g_cu_mu);
  if (!g_cus[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cus[dev] = v;
  }
  return g_cus[dev];
}

struct TopkPlan {
  bool fused = false;
  int chunk = 0, P = 0;
};

// One workgroup per CU: P = CUs / Hkv chunks per kv head, chunks a multiple of
// the granule and small enough for the group's logits to stay in LDS.
TopkPlan topk_plan(const skv_problem* p, int64_t n, int cus) {
  TopkPlan t;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (p->dtype != SKV_BF16 || p->n_kv_heads > kTopkMaxKvHeads || cus < p->n_kv_heads) return t;
  const int pmax = cus / p->n_kv_heads, gr = skv::topk_step_granule();
  int64_t chunk = (n + pmax - 1) / pmax;
  chunk = (chunk + gr - 1) / gr * gr;
  if (chunk > skv::topk_step_max_chunk(G, p->head_dim)) return t;
  t.fused = true;
  t.chunk = (int)chunk;
  t.P = (int)((n + chunk - 1) / chunk);
  return t;
}

// The selection alone in one launch (long rows with few kv heads): chunks of
// at most topk_select_max_chunk() scores, P = ceil(n / chunk) <= CUs / Hkv,
// and K small enough against the chunks that each chunk's publishing rank
// (2 ceil(K / P) + 16) fits the published-key budget: larger K, whose keys
// rarely fit and then take the six-barrier radix levels, stays with the
// three-kernel select.
struct SelPlan {
  bool one = false;
  int chunk = 0, P = 0;
};
SelPlan select_plan(int32_t hkv, int64_t n, int64_t k_max, int cus) {
  SelPlan t;
  if (n <= 16384 || hkv >= kTopkMaxKvHeads || cus < hkv) return t;
  const int pmax = cus / hkv, gr = skv::topk_step_granule();
  int64_t chunk = (n + pmax - 1) / pmax;
  chunk = (chunk + gr - 1) / gr * gr;
  if (chunk > skv::topk_select_max_chunk()) return t;
  const int64_t P = (n + chunk - 1) / chunk;
  const int64_t cap = (skv::topk_publish_budget() / P) & ~3;
  if (2 * ((k_max + P - 1) / P) + 16 > cap * 3 / 4) return t;
  t.one = true;
  t.chunk = (int)chunk;
  t.P = (int)P;
  return t;
}
size_t select_one_scratch_bound(int32_t hkv, int64_t n_max) {
  if (n_max <= 16384 || hkv >= kTopkMaxKvHeads) return 0;
  int64_t P = kMaxCUs / hkv;
  const int64_t pn = (n_max + skv::topk_step_granule() - 1) / skv::topk_step_granule();
  P = P < pn ? P : pn;
  P = P < 1 ? 1 : P;
  return skv::topk_select_scratch(hkv, (int)P);
}

// Scratch of the fused step for any device: P <= kMaxCUs / Hkv and P <= n / granule.
size_t topk_scratch_bound(const skv_problem* p, int64_t n_max) {
  if (p->dtype != SKV_BF16 || p->n_kv_heads > kTopkMaxKvHeads) return 0;
  const int G = p->n_q_heads / p->n_kv_heads;
  int64_t P = kMaxCUs / p->n_kv_heads;
  const int64_t pn = (n_max + skv::topk_step_granule() - 1) / skv::topk_step_granule();
  P = P < pn ? P : pn;
  P = P < 1 ? 1 : P;
  return skv::topk_step_scratch(p->n_kv_heads, (int)P, G, p->head_dim);
}

// The launches of a checked dense decode call; `base` is a workspace of at
// least SKV_WS_HEADER_BYTES + attend_scratch(p, attend_plan(p, n, false)) bytes.
skv_status run_attend_dense(const skv_problem* p, const void* q, const void* k, const void* v, int64_t n,
                            float* out, float* lse, char* base, hipStream_t stream) {
  const ChunkPlan cp = attend_plan(p, n, false);
  const int G = p->n_q_heads / p->n_kv_heads;
  const PartLayout L = part_layout(p, cp.cph, G);
  AttendArgs a{};
  a.q = q;
  a.k = (const char*)k;
  a.v = (const char*)v;
  a.head_stride_b = p->kv_head_stride * elem_size(p);
  a.pos_stride_b = p->kv_pos_stride * elem_size(p);
  a.n = n;
  a.n_kv_heads = p->n_kv_heads;
  a.chunk = cp.chunk;
  a.chunks_per_head = cp.cph;
  a.scale_log2 = scale_log2(p);
  a.part_ml = (float*)(base + L.ml);
  a.part_acc = (float*)(base + L.acc);
  a.nch = (int32_t*)(base + L.nch);
  a.group = G;
  a.n_pos = 1;
  a.narrow = cp.narrow;
  const skv_status st = hip_status(launch_attend_any(p, false, a, stream));
  if (st != SKV_OK) return st;
  return launch_partials_merge(p, base, L, cp.cph, G, false, out, lse, stream);
}

// The launches of a checked per-step score call (one query row per query
// head); `base` is a workspace of at least SKV_WS_HEADER_BYTES +
// score_step_scratch(p, n) bytes.
skv_status run_score_step(const skv_problem* p, const void* q, const void* k, int64_t n, float* score,
                          int64_t score_stride, char* base, hipStream_t stream) {
  const ChunkPlan cp = score_step_plan(p, n);
  const int G = p->n_q_heads / p->n_kv_heads;
  skv::ScoreStepArgs a{};
  a.q = q;
  a.k = (const char*)k;
  a.head_stride_b = p->kv_head_stride * elem_size(p);
  a.pos_stride_b = p->kv_pos_stride * elem_size(p);
  a.n = n;
  a.n_kv_heads = p->n_kv_heads;
  a.chunk = cp.chunk;
  a.chunks_per_head = cp.cph;
  a.scale_log2 = scale_log2(p);
  a.logits = (float*)(base + SKV_WS_HEADER_BYTES);
  a.logits_stride = logits_stride(n);
  a.part_ml = (float*)(base + SKV_WS_HEADER_BYTES +
                       align_up((size_t)p->n_q_heads * a.logits_stride * sizeof(float)));
  a.score = score;
  a.score_stride = score_stride;
  return hip_status(skv::launch_score_step(p->dtype, p->head_dim, G, a, stream));
}

}  // namespace

extern "C" {

int32_t skv_version(void) { return 1; }

const char* skv_status_string(skv_status s) {
  switch (s) {
    case SKV_OK: return "ok";
    case SKV_ERR_INVALID_ARG: return "invalid argument";
    case SKV_ERR_UNSUPPORTED: return "unsupported problem (head_dim or group size)";
    case SKV_ERR_WORKSPACE: return "workspace too small";
    case SKV_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t skv_workspace_size(const skv_problem* p, int64_t n_max, int32_t rows_max) {
  if (check_problem(p) != SKV_OK || n_max < 1 || rows_max < 1) return 0;
  size_t s = attend_scratch(p, attend_plan(p, n_max, false));
  size_t t = attend_scratch(p, attend_plan(p, n_max, true));
  s = s > t ? s : t;
  t = score_step_scratch(p, n_max);
  s = s > t ? s : t;
  t = skv::select_ws_bytes(p->n_kv_heads, n_max);
  s = s > t ? s : t;
  t = select_one_scratch_bound(p->n_kv_heads, n_max);
  s = s > t ? s : t;
  t = topp_scratch(n_max);
  s = s > t ? s : t;
  t = topk_scratch_bound(p, n_max);
  s = s > t ? s : t;
  if (p->dtype == SKV_F32 && rows_max > 1) {  // the composed fp32 window score
    t = score_window_f32_scratch(p, n_max);
    s = s > t ? s : t;
  }
  if (p->dtype == SKV_BF16) {
    const int32_t w = rows_max < n_max ? rows_max : (int32_t)n_max;
    t = score_obs_scratch(p, n_max, w);
    s = s > t ? s : t;
    const int32_t g = w < kVerifyMaxGamma ? w : kVerifyMaxGamma;
    for (int32_t gg = 1; gg <= g; ++gg) {  // every gamma up to the bound
      t = verify_scratch(p, n_max, gg);
      s = s > t ? s : t;
    }
  }
  return SKV_WS_HEADER_BYTES + s;
}

skv_status skv_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ((uintptr_t)ws % kAlign) != 0) return SKV_ERR_INVALID_ARG;
  if (ws_bytes < SKV_WS_HEADER_BYTES) return SKV_ERR_WORKSPACE;
  return hip_status(skv::launch_zero_u32((uint32_t*)ws, kCounterSlots, (hipStream_t)stream));
}

skv_status skv_attend_dense(const skv_problem* p, const void* q, const void* k, const void* v,
                            int64_t n, float* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (n < 1 || !q || !out || !aligned16(q) || !aligned16(out)) return SKV_ERR_INVALID_ARG;
  if ((st = check_cache(p, k, n)) != SKV_OK || (st = check_cache(p, v, n)) != SKV_OK) return st;
  if ((st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + attend_scratch(p, attend_plan(p, n, false)))) != SKV_OK)
    return st;
  return run_attend_dense(p, q, k, v, n, out, lse, (char*)ws, (hipStream_t)stream);
}

skv_status skv_attend_sparse(const skv_problem* p, const void* q, const void* k, const void* v,
                             int64_t n, const int32_t* idx, int64_t idx_stride,
                             const int32_t* count, int64_t tail_start, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream) {
  ChunkPlan cp;
  skv_status st = check_attend_sparse(p, q, k, v, n, idx, idx_stride, count, tail_start, out, &cp);
  if (st != SKV_OK) return st;
  if ((st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + attend_scratch(p, cp))) != SKV_OK)
    return st;
  return run_attend_sparse(p, cp, q, k, v, n, idx, idx_stride, count, tail_start, out, lse,
                           (char*)ws, (hipStream_t)stream);
}

skv_status skv_attend_sparse_noalloc(const skv_problem* p, const void* q, const void* k,
                                     const void* v, int64_t n, const int32_t* idx,
                                     int64_t idx_stride, const int32_t* count, int64_t tail_start,
                                     float* out, float* lse, void* stream) {
  ChunkPlan cp;
  skv_status st = check_attend_sparse(p, q, k, v, n, idx, idx_stride, count, tail_start, out, &cp);
  if (st != SKV_OK) return st;
  if (SKV_WS_HEADER_BYTES + attend_scratch(p, cp) > (size_t)SKV_NOALLOC_SCRATCH_BYTES)
    return SKV_ERR_WORKSPACE;
  char* base = nullptr;
  if ((st = noalloc_scratch(&base, (hipStream_t)stream)) != SKV_OK) return st;
  return run_attend_sparse(p, cp, q, k, v, n, idx, idx_stride, count, tail_start, out, lse, base,
                           (hipStream_t)stream);
}

skv_status skv_score(const skv_problem* p, const void* q, int32_t n_obs, const void* k, int64_t n,
                     float* score, int64_t score_stride, void* ws, size_t ws_bytes, void* stream) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (n < 1 || n_obs < 1 || n_obs > n || !q || !score || score_stride < n || !aligned16(q))
    return SKV_ERR_INVALID_ARG;
  if (n > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  if ((st = check_cache(p, k, n)) != SKV_OK) return st;
  const int G = p->n_q_heads / p->n_kv_heads;
  char* base = (char*)ws;
  if (n_obs == 1) {
    if ((st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + score_step_scratch(p, n))) != SKV_OK)
      return st;
    return run_score_step(p, q, k, n, score, score_stride, base, (hipStream_t)stream);
  }
  if (p->dtype == SKV_F32) {
    // fp32 window: window row i (at position n - n_obs + i) runs as a per-step
    // score over its prefix of n - n_obs + i + 1 keys into a scratch row block;
    // the rows are added in order with weight 1 / n_obs (the vector kernels
    // have no causal window rows)
    if ((st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + score_window_f32_scratch(p, n))) != SKV_OK)
      return st;
    float* rows = (float*)(base + SKV_WS_HEADER_BYTES + score_step_scratch(p, n));
    const int64_t rs = logits_stride(n);
    const size_t qrow = (size_t)p->n_q_heads * p->head_dim * sizeof(float);
    const float w = 1.0f / (float)n_obs;
    for (int32_t i = 0; i < n_obs; ++i) {
      const int64_t ni = n - n_obs + i + 1;
      if ((st = run_score_step(p, (const char*)q + i * qrow, k, ni, rows, rs, base, (hipStream_t)stream)) != SKV_OK)
        return st;
      if ((st = hip_status(skv::launch_add_rows(score, score_stride, rows, rs, p->n_kv_heads, ni, n, w, i == 0,
                                                (hipStream_t)stream))) != SKV_OK)
        return st;
    }
    return SKV_OK;
  }
  if (p->dtype != SKV_BF16) return SKV_ERR_UNSUPPORTED;  // window scoring runs on bf16 MFMA
  if ((st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + score_obs_scratch(p, n, n_obs))) != SKV_OK)
    return st;
  const int64_t R = (int64_t)n_obs * G;
  const int64_t nkb = (n + skv::score_obs_block_keys() - 1) / skv::score_obs_block_keys();
  skv::ScoreObsArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const char*)k;
  a.head_stride_b = p->kv_head_stride * 2;
  a.pos_stride_b = p->kv_pos_stride * 2;
  a.n = n;
  a.n_obs = n_obs;
  a.n_kv_heads = p->n_kv_heads;
  a.group = G;
  a.n_kblocks = (int32_t)nkb;
  a.scale_log2 = scale_log2(p);
  a.part_ml = (float*)(base + SKV_WS_HEADER_BYTES);
  a.row_lse2 = (float*)(base + SKV_WS_HEADER_BYTES +
                        align_up((size_t)p->n_kv_heads * nkb * R * 2 * sizeof(float)));
  a.row_groups = obs_row_groups(p, nkb, R);
  a.part_score = (float*)((char*)a.row_lse2 + align_up((size_t)p->n_kv_heads * R * sizeof(float)));
  a.score = score;
  a.score_stride = score_stride;
  return hip_status(skv::launch_score_obs(p->head_dim, a, (hipStream_t)stream));
}

skv_status skv_select(const skv_problem* p, const float* score, int64_t score_stride, int64_t n,
                      int32_t n_sink, int32_t n_recent, const int32_t* k_per_head,
                      int32_t k_uniform, int32_t k_max, int32_t* idx, int64_t idx_stride,
                      int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (n < 1 || !score || score_stride < n || n_sink < 0 || n_recent < 0 || !count)
    return SKV_ERR_INVALID_ARG;
  if (k_max < 0 || (!k_per_head && (k_uniform < 0 || k_uniform > k_max)))
    return SKV_ERR_INVALID_ARG;
  if (idx_stride < (int64_t)n_sink + k_max || (idx_stride > 0 && !idx)) return SKV_ERR_INVALID_ARG;
  if (n > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  const SelPlan sp = select_plan(p->n_kv_heads, n, k_per_head ? k_max : k_uniform, device_cus());
  if (sp.one) {  // long rows, few kv heads: one launch
    const size_t need = SKV_WS_HEADER_BYTES + skv::topk_select_scratch(p->n_kv_heads, sp.P);
    if ((st = check_ws(ws, ws_bytes, need)) != SKV_OK) return st;
    skv::TopkArgs a{};
    a.score = const_cast<float*>(score);  // read only
    a.score_stride = score_stride;
    a.n = n;
    a.n_sink = n_sink;
    a.n_recent = n_recent;
    a.k_top = k_uniform;
    a.k_per_head = k_per_head;
    a.n_kv_heads = p->n_kv_heads;
    a.chunk = sp.chunk;
    a.chunks_per_head = sp.P;
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.count = count;
    a.ctr = (uint32_t*)((char*)ws + kTopkCtrOffset);
    a.err = (uint32_t*)((char*)ws + kTopkErrOffset);
    return hip_status(skv::launch_topk_select(a, (char*)ws + SKV_WS_HEADER_BYTES, (hipStream_t)stream));
  }
  const size_t sel_ws = skv::select_ws_bytes(p->n_kv_heads, n);
  if (sel_ws > 0 && (st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + sel_ws)) != SKV_OK) return st;
  skv::SelectArgs a{};
  a.ws = sel_ws > 0 ? (char*)ws + SKV_WS_HEADER_BYTES : nullptr;
  a.totals = sel_ws > 0 ? (uint32_t*)ws : nullptr;  // the reserved header
  a.score = score;
  a.score_stride = score_stride;
  a.n = n;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.k_per_head = k_per_head;
  a.k_uniform = k_uniform;
  a.k_max = k_max;
  a.idx = idx;
  a.idx_stride = idx_stride;
  a.count = count;
  a.n_kv_heads = p->n_kv_heads;
  return hip_status(skv::launch_select(a, (hipStream_t)stream));
}

skv_status skv_select_topp(const skv_problem* p, const float* score, int64_t score_stride,
                           int64_t n, int32_t n_sink, int32_t n_recent, double lambda,
                           double prune_ratio, int32_t pooled, int32_t fill_mode, int32_t* idx,
                           int64_t idx_stride, int32_t* count, int32_t* count_r, void* ws,
                           size_t ws_bytes, void* stream) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (n < 1 || !score || score_stride < n || n_sink < 0 || n_recent < 0 || !count || !idx)
    return SKV_ERR_INVALID_ARG;
  if (!(lambda >= 0.0 && lambda <= 1.0) || !(prune_ratio >= 0.0 && prune_ratio <= 1.0) ||
      (pooled != 0 && pooled != 1) || (fill_mode != 0 && fill_mode != 1))
    return SKV_ERR_INVALID_ARG;
  if (n > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  const int64_t tail = n - n_recent > 0 ? n - n_recent : 0;
  const int64_t nsink = n_sink < tail ? n_sink : tail;
  const int64_t ncand = n_sink < n - n_recent ? n - n_recent - n_sink : 0;
  if (idx_stride < nsink + ncand) return SKV_ERR_INVALID_ARG;
  if (pooled && (st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + topp_scratch(n))) != SKV_OK) return st;
  skv::ToppArgs a{};
  a.score = score;
  a.score_stride = score_stride;
  a.rows = p->n_kv_heads;
  a.pooled = pooled;
  a.n = n;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  // lambda = lam_m / 2^lam_sh exactly (53-bit mantissa)
  int e = 0;
  const double f = frexp(lambda, &e);
  a.lam_m = (uint64_t)ldexp(f, 53);
  a.lam_sh = 53 - e;
  a.fill_mode = fill_mode;
  a.budget = llround((1.0 - prune_ratio) * (double)ncand);
  a.idx = idx;
  a.idx_stride = idx_stride;
  a.count = count;
  a.count_r = count_r;
  a.pooled_row = pooled ? (uint32_t*)((char*)ws + SKV_WS_HEADER_BYTES) : nullptr;
  return hip_status(skv::launch_select_topp(a, (hipStream_t)stream));
}

skv_status skv_verify(const skv_problem* p, const void* q, int32_t gamma, const void* k,
                      const void* v, int64_t n, float* out, float* lse, void* ws,
                      size_t ws_bytes, void* stream) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (gamma < 1 || gamma > kVerifyMaxGamma || n < gamma || !q || !out || !aligned16(q) ||
      !aligned16(out))
    return SKV_ERR_INVALID_ARG;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (n > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  if ((st = check_cache(p, k, n)) != SKV_OK || (st = check_cache(p, v, n)) != SKV_OK) return st;
  if (p->dtype == SKV_F32) {
    // fp32 caches: drafted position t runs as a decode step over its prefix of
    // n - gamma + t + 1 entries (the vector kernel has no causal rows); the
    // dense scratch bound is monotone in the rows, so the longest prefix sizes it
    if ((st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + attend_scratch(p, attend_plan(p, n, false)))) != SKV_OK)
      return st;
    const size_t qrow = (size_t)p->n_q_heads * p->head_dim;
    for (int32_t t = 0; t < gamma; ++t)
      if ((st = run_attend_dense(p, (const float*)q + t * qrow, k, v, n - gamma + t + 1, out + t * qrow,
                                 lse ? lse + (size_t)t * p->n_q_heads : nullptr, (char*)ws,
                                 (hipStream_t)stream)) != SKV_OK)
        return st;
    return SKV_OK;
  }
  if ((st = check_ws(ws, ws_bytes, SKV_WS_HEADER_BYTES + verify_scratch(p, n, gamma))) != SKV_OK)
    return st;
  // Passes of at most qc queries: pass [t0, t0 + g) holds queries at positions
  // n - gamma + t0 .. n - gamma + t0 + g - 1, i.e. a verify of g queries over
  // the prefix of n - gamma + t0 + g entries (later entries are masked for it).
  const int32_t qc = verify_pass_queries(p, gamma);
  const size_t qrow = (size_t)p->n_q_heads * p->head_dim;
  char* base = (char*)ws;
  for (int32_t t0 = 0; t0 < gamma; t0 += qc) {
    const int32_t g = gamma - t0 < qc ? gamma - t0 : qc;
    const int64_t np = n - gamma + t0 + g;
    const ChunkPlan cp = verify_plan(p, np, g);
    const PartLayout L = part_layout(p, cp.cph, g * G);
    skv::AttendArgs a{};
    a.q = (const char*)q + (size_t)t0 * qrow * 2;
    a.k = (const char*)k;
    a.v = (const char*)v;
    a.head_stride_b = p->kv_head_stride * 2;
    a.pos_stride_b = p->kv_pos_stride * 2;
    a.n = np;
    a.n_kv_heads = p->n_kv_heads;
    a.chunk = cp.chunk;
    a.chunks_per_head = cp.cph;
    a.scale_log2 = scale_log2(p);
    a.part_ml = (float*)(base + L.ml);
    a.part_acc = (float*)(base + L.acc);
    a.nch = (int32_t*)(base + L.nch);
    a.group = G;
    a.n_pos = g;
    if ((st = hip_status(skv::launch_attend_mfma(p->head_dim, false, true, a, (hipStream_t)stream))) != SKV_OK)
      return st;
    if ((st = launch_partials_merge(p, base, L, cp.cph, g * G, false, out + (size_t)t0 * qrow,
                                    lse ? lse + (size_t)t0 * p->n_q_heads : nullptr,
                                    (hipStream_t)stream)) != SKV_OK)
      return st;
  }
  return SKV_OK;
}

skv_status skv_topk_step(const skv_problem* p, const void* q, const void* k, const void* v,
                         int64_t n, int32_t n_sink, int32_t n_recent, int32_t k_top, float* score,
                         int64_t score_stride, int32_t* idx, int64_t idx_stride, int32_t* count,
                         float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (n < 1 || !q || !out || !aligned16(q) || !aligned16(out) || !score || score_stride < n || !count)
    return SKV_ERR_INVALID_ARG;
  if (n_sink < 0 || n_recent < 0 || k_top < 0) return SKV_ERR_INVALID_ARG;
  if (idx_stride < (int64_t)n_sink + k_top || (idx_stride > 0 && !idx)) return SKV_ERR_INVALID_ARG;
  if (n > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  if ((st = check_cache(p, k, n)) != SKV_OK || (st = check_cache(p, v, n)) != SKV_OK) return st;
  const int64_t tail = n - n_recent > 0 ? n - n_recent : 0;
  const TopkPlan tp = topk_plan(p, n, device_cus());
  if (tp.fused) {
    const int G = p->n_q_heads / p->n_kv_heads;
    const size_t need = SKV_WS_HEADER_BYTES + skv::topk_step_scratch(p->n_kv_heads, tp.P, G, p->head_dim);
    if ((st = check_ws(ws, ws_bytes, need)) != SKV_OK) return st;
    skv::TopkArgs a{};
    a.q = q;
    a.k = (const char*)k;
    a.v = (const char*)v;
    a.head_stride_b = p->kv_head_stride * 2;
    a.pos_stride_b = p->kv_pos_stride * 2;
    a.n = n;
    a.n_sink = n_sink;
    a.n_recent = n_recent;
    a.k_top = k_top;
    a.n_kv_heads = p->n_kv_heads;
    a.chunk = tp.chunk;
    a.chunks_per_head = tp.P;
    a.scale_log2 = scale_log2(p);
    a.score = score;
    a.score_stride = score_stride;
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.count = count;
    a.out = out;
    a.lse = lse;
    a.ctr = (uint32_t*)((char*)ws + kTopkCtrOffset);
    a.err = (uint32_t*)((char*)ws + kTopkErrOffset);
    const hipError_t e = skv::launch_topk_step(p->head_dim, G, a, (char*)ws + SKV_WS_HEADER_BYTES,
                                               (hipStream_t)stream);
    if (e == hipSuccess) return SKV_OK;
    // not launched: clear the error and take the three-call path
    (void)hipGetLastError();
  }
  if ((st = skv_score(p, q, 1, k, n, score, score_stride, ws, ws_bytes, stream)) != SKV_OK) return st;
  if ((st = skv_select(p, score, score_stride, n, n_sink, n_recent, nullptr, k_top, k_top, idx,
                       idx_stride, count, ws, ws_bytes, stream)) != SKV_OK)
    return st;
  return skv_attend_sparse(p, q, k, v, n, idx, idx_stride, count, tail, out, lse, ws, ws_bytes, stream);
}

skv_status skv_gather(const skv_problem* p, const void* k, const void* v, int64_t n,
                      const int32_t* idx, int64_t idx_stride, const int32_t* count,
                      int64_t tail_start, void* k_out, void* v_out, int64_t out_head_stride,
                      int64_t out_pos_stride, int32_t* rows_out, void* stream) {
  skv_status st = check_problem(p);
  if (st != SKV_OK) return st;
  if (n < 1 || !count || (!idx && idx_stride > 0) || idx_stride < 0) return SKV_ERR_INVALID_ARG;
  if (tail_start < 0 || tail_start > n) return SKV_ERR_INVALID_ARG;
  if (n > INT32_MAX) return SKV_ERR_UNSUPPORTED;
  if ((st = check_cache(p, k, n)) != SKV_OK || (st = check_cache(p, v, n)) != SKV_OK) return st;
  const int64_t count_max = idx_stride < tail_start ? idx_stride : tail_start;
  const int64_t rows_max = count_max + (n - tail_start);
  if (rows_max < 1) return SKV_ERR_INVALID_ARG;
  const int es = elem_size(p);
  if (!k_out || !v_out || !aligned16(k_out) || !aligned16(v_out)) return SKV_ERR_INVALID_ARG;
  if (out_pos_stride < p->head_dim || (out_pos_stride * es) % 16 != 0 ||
      (out_head_stride * es) % 16 != 0 || out_head_stride < 0)
    return SKV_ERR_INVALID_ARG;
  if (p->n_kv_heads > 1 && out_head_stride < rows_max * out_pos_stride) return SKV_ERR_INVALID_ARG;
  skv::GatherArgs a{};
  a.k = (const char*)k;
  a.v = (const char*)v;
  a.head_stride_b = p->kv_head_stride * es;
  a.pos_stride_b = p->kv_pos_stride * es;
  a.n = n;
  a.idx = idx;
  a.idx_stride = idx_stride;
  a.count = count;
  a.count_max = count_max;
  a.tail_start = tail_start;
  a.k_out = (char*)k_out;
  a.v_out = (char*)v_out;
  a.out_head_stride_b = out_head_stride * es;
  a.out_pos_stride_b = out_pos_stride * es;
  a.rows_max = rows_max;
  a.rows_out = rows_out;
  a.n_kv_heads = p->n_kv_heads;
  a.row_bytes = p->head_dim * es;
  return hip_status(skv::launch_gather(a, (hipStream_t)stream));
}

skv_status skv_budgets(const double* s, int32_t n_heads, double total_budget, int32_t window,
                       double rho, int64_t n_cand, int32_t* k_out, double* b_out) {
  if (!s || !k_out || n_heads < 1 || window < 0 || !(rho >= 0.0 && rho <= 1.0) || n_cand < 0 ||
      !(total_budget == total_budget))
    return SKV_ERR_INVALID_ARG;
  double total = 0.0;
  for (int32_t i = 0; i < n_heads; ++i) {
    if (!(s[i] >= 0.0) || isinf(s[i])) return SKV_ERR_INVALID_ARG;
    total += s[i];
  }
  if (!(total > 0.0)) return SKV_ERR_INVALID_ARG;
  // Local Window Cache: w per head; Uniform-Based Cache: r per head;
  // Score-Preferred Cache: the remainder in proportion to the head score.
  const double lwc_total = (double)n_heads * (double)window;
  const double ubc_total = rho * (total_budget - lwc_total);
  const double r = ubc_total / (double)n_heads;
  const double spc_total = total_budget - lwc_total - ubc_total;
  for (int32_t i = 0; i < n_heads; ++i) {
    const double share = spc_total * s[i] / total;
    double k = floor(r + share);
    if (k < 0.0) k = 0.0;
    if (k > (double)n_cand) k = (double)n_cand;
    k_out[i] = (int32_t)k;
    if (b_out) b_out[i] = (double)window + r + share;
  }
  return SKV_OK;
}

}  // extern "C"
