// util.hip -- small helper kernels.
#include "skv_common.h"
#include "skv_kernels.h"

namespace skv {
namespace {
__global__ void zero_u32_kernel(uint32_t* p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
}  // namespace

// Plain fill kernel (not hipMemsetAsync) so the clear can sit inside a captured graph.
hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t stream) {
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                     stream, p, count);
  return hipGetLastError();
}

}  // namespace skv
