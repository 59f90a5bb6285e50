// probe_read.hip -- the streaming-read ceiling of the GPU the bench runs on
// (a second denominator beside the 8 TB/s HBM peak).  Not part of the
// method and not part of libsparsekv: it is built into libskvprobe.so, which
// only bench.py loads.
//
// Every workgroup reads a contiguous share of the buffer with 16-byte loads,
// four in flight per thread, and folds them into one word per thread; a
// thread writes its word only if it equals a value the data cannot produce
// by chance, so the loads cannot be dropped and almost nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* p, int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b = (int64_t)blockIdx.x * per;
  const int64_t e = b + per < n16 ? b + per : n16;
  uint32_t x = 0;
  for (int64_t i = b + threadIdx.x; i < e; i += (int64_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kThreads;
      v[u] = j < e ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer `p`
// with `grid` workgroups on `stream`; `sink` is a device word array of `grid`
// entries that is written only by chance.  Returns a hipError_t value.
extern "C" int skv_probe_read(const void* p, int64_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!p || !sink || bytes < 16 || (bytes & 15) || grid < 1 || ((uintptr_t)p & 15)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)p, bytes / 16, sink);
  return (int)hipGetLastError();
}
