// Block copies, fills and sums for the convolution with mixed per-l multiplicities: repacking
// between the mixed node-tensor layout, the uniform channel slices the convolution kernels take
// and the padded path-output rows the mixing GEMM takes.  Plain HBM-bound kernels, 16-byte
// accesses, one thread per four floats.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "mixed.h"

namespace equitp {
namespace {

__device__ __forceinline__ float* row_ptr(const RowMap& m, int r) {
  return m.base + (long long)(r / m.d) * m.stride_node + m.off + (long long)(r % m.d) * m.stride_m;
}

struct CopyBatch {
  CopyJob job[kCopyBatch];
};

// blockIdx.y = job; the x blocks stride over the job's rows x (cols / 4) items
__global__ void __launch_bounds__(256) copy_batch_kernel(CopyBatch b) {
  const CopyJob& j = b.job[blockIdx.y];
  const int c4s = j.cols / 4;
  const long long items = (long long)j.rows * c4s;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < items;
       i += (long long)gridDim.x * 256) {
    const int r = (int)(i / c4s), c = 4 * (int)(i % c4s);
    st4(row_ptr(j.dst, r) + c, ld4(row_ptr(j.src, r) + c));
  }
}

__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void __launch_bounds__(256) iota32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = i;
}

__global__ void __launch_bounds__(256) add_kernel(float* y, const float* x, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] += x[i];
}

}  // namespace

hipError_t launch_copy_batch(const CopyJob* jobs, int n_jobs, hipStream_t st) {
  for (int a = 0; a < n_jobs; a += kCopyBatch) {
    CopyBatch b{};
    const int n = std::min(kCopyBatch, n_jobs - a);
    long long most = 0;
    for (int k = 0; k < n; ++k) {
      const CopyJob& j = jobs[a + k];
      if (j.cols % 4 != 0 || j.dst.d <= 0 || j.src.d <= 0 || j.rows < 0) return hipErrorInvalidValue;
      b.job[k] = j;
      most = std::max(most, (long long)j.rows * (j.cols / 4));
    }
    if (most == 0) continue;
    const unsigned gx = (unsigned)std::min<long long>((most + 255) / 256, 1024);
    hipLaunchKernelGGL(copy_batch_kernel, dim3(gx, n), dim3(256), 0, st, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(iota32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_add(float* y, const float* x, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, y, x, n);
  return hipGetLastError();
}

}  // namespace equitp
