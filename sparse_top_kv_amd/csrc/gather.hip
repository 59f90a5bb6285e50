// gather.hip -- compaction of a kept set into a contiguous cache.
//
// Method: the kept entries of each kv head are copied once into a dense
// buffer that later decode steps read with the dense split-K kernel
// ("Where Activation Sparsity and KV-Cache Sparsity Cross ...", section
// "Speedup Across Context").  Row i of head h in the output is idx[h][i] for
// i < count[h], then the tail [tail_start, n).
//
// A plain HBM copy: each lane moves 16-byte pieces of K and V rows; the
// pieces of one row share its index entry (one broadcast load).
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherIt = 4;                                 // pieces per thread
constexpr int kGatherPieces = kGatherThreads * kGatherIt;   // 16-byte pieces per workgroup

// Workgroup b of head h moves pieces [b * kGatherPieces, (b + 1) * kGatherPieces)
// of the head's output (row-major, row_bytes / 16 pieces per row): all loads
// are issued before the first store.
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(const GatherArgs a, int nblk) {
  const int h = blockIdx.x % a.n_kv_heads;  // a kv head's blocks on one XCD
  const int b = blockIdx.x / a.n_kv_heads;
  // clamped to the rows the output holds (entries are unique and below tail_start)
  int64_t cnt = a.count[h];
  cnt = cnt < 0 ? 0 : (cnt > a.count_max ? a.count_max : cnt);
  const int64_t rows_h = cnt + (a.n - a.tail_start);
  const int ppr = a.row_bytes / 16;
  const char* kh = a.k + (int64_t)h * a.head_stride_b;
  const char* vh = a.v + (int64_t)h * a.head_stride_b;
  char* koh = a.k_out + (int64_t)h * a.out_head_stride_b;
  char* voh = a.v_out + (int64_t)h * a.out_head_stride_b;
  const int32_t* ih = a.idx + (int64_t)h * a.idx_stride;
  uint4 kv[kGatherIt], vv[kGatherIt];
  int64_t dst[kGatherIt];
#pragma unroll
  for (int j = 0; j < kGatherIt; ++j) {
    const int64_t e = (int64_t)b * kGatherPieces + j * kGatherThreads + threadIdx.x;
    const int64_t i = e / ppr;
    const int pc = (int)(e - i * ppr);
    dst[j] = i < rows_h ? i * a.out_pos_stride_b + pc * 16 : -1;
    if (dst[j] >= 0) {
      int64_t src = i < cnt ? (int64_t)ih[i] : a.tail_start + (i - cnt);
      src = src < 0 ? 0 : (src >= a.n ? a.n - 1 : src);  // out-of-contract indices stay in bounds
      kv[j] = ld16(kh + src * a.pos_stride_b + pc * 16);
      vv[j] = ld16(vh + src * a.pos_stride_b + pc * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < kGatherIt; ++j) {
    if (dst[j] >= 0) {
      *reinterpret_cast<uint4*>(koh + dst[j]) = kv[j];
      *reinterpret_cast<uint4*>(voh + dst[j]) = vv[j];
    }
  }
  if (b == 0 && threadIdx.x == 0 && a.rows_out) a.rows_out[h] = (int32_t)rows_h;
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int64_t pieces = a.rows_max * (a.row_bytes / 16);
  const int nblk = (int)((pieces + kGatherPieces - 1) / kGatherPieces);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(a.n_kv_heads * nblk)), dim3(kGatherThreads), 0, s, a,
                     nblk);
  return hipGetLastError();
}

}  // namespace skv
