// Block copies, fills and sums for the convolution with mixed per-l multiplicities: repacking
// between the mixed node-tensor layout, the uniform channel slices the convolution kernels take
// and the padded path-output rows the mixing GEMM takes.  Plain HBM-bound kernels, 16-byte
// accesses, one thread per four floats.
#include <hip/hip_runtime.h>

#include "common.h"
#include "mixed.h"

namespace equitp {
namespace {

__device__ __forceinline__ float* row_ptr(const RowMap& m, int r) {
  return m.base + (long long)(r / m.d) * m.stride_node + m.off + (long long)(r % m.d) * m.stride_m;
}

__global__ void __launch_bounds__(256) copy_rows_kernel(RowMap dst, RowMap src, int rows, int c4s,
                                                        int accumulate) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)rows * c4s) return;
  const int r = (int)(i / c4s), c = 4 * (int)(i % c4s);
  const f4 v = ld4(row_ptr(src, r) + c);
  float* o = row_ptr(dst, r) + c;
  st4(o, accumulate ? ld4(o) + v : v);
}

__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void __launch_bounds__(256) add_kernel(float* y, const float* x, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] += x[i];
}

}  // namespace

hipError_t launch_copy_rows(RowMap dst, RowMap src, int rows, int cols, bool accumulate,
                            hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 4 != 0 || dst.d <= 0 || src.d <= 0) return hipErrorInvalidValue;
  const long long items = (long long)rows * (cols / 4);
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st,
                     dst, src, rows, cols / 4, accumulate ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_add(float* y, const float* x, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, y, x, n);
  return hipGetLastError();
}

}  // namespace equitp
