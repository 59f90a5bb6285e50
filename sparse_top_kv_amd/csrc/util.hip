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

// y[r][j] += w x[r][j] for j < nx; with `first`, y[r][j] = w x[r][j] for
// j < nx and 0 for nx <= j < ny.  Grid: (blocks per row, rows).
__global__ void add_rows_kernel(float* y, int64_t ys, const float* x, int64_t xs, int64_t nx, int64_t ny,
                                float w, int first) {
  const int64_t r = blockIdx.y;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < ny; j += (int64_t)gridDim.x * blockDim.x) {
    const float add = j < nx ? w * x[r * xs + j] : 0.0f;
    if (first) y[r * ys + j] = add;
    else if (j < nx) y[r * ys + j] += add;
  }
}
}  // namespace

// Plain fill kernel (not hipMemsetAsync) so the clear can sit inside a captured graph.
hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t stream) {
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                     stream, p, count);
  return hipGetLastError();
}

hipError_t launch_add_rows(float* y, int64_t ys, const float* x, int64_t xs, int rows, int64_t nx, int64_t ny,
                           float w, bool first, hipStream_t stream) {
  const int64_t blocks = (ny + 255) / 256;
  hipLaunchKernelGGL(add_rows_kernel, dim3((unsigned)(blocks < 256 ? blocks : 256), (unsigned)rows), dim3(256), 0,
                     stream, y, ys, x, xs, nx, ny, w, first ? 1 : 0);
  return hipGetLastError();
}

}  // namespace skv
