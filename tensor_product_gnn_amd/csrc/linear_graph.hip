// Per-irrep channel-mixing linear on the matrix cores, and the CSR builder for the sender-grouped
// (transpose) edge order.
//
// Linear: for each l, out[n, l*l + m, :] = feat[n, l*l + m, :] W_l, a GEMM with M = n_nodes (2l+1)
// rows (row (n, m) at offset (n F + l*l + m) C), K = N = C.  This is the dense 128 x 128 channel
// mixing that follows a convolution in an interaction block (FlashCart, Fig. 3 caption: linear
// maps that mix paths and channels between steps).  fp32 MFMA 16x16x4 (no reduced-precision
// inputs: "Fast and Accurate Foundation Models for Equivariant MLIPs", Sec. II and VII keep TF32
// off where accuracy matters).  A work-group of 4 waves takes 64 rows; W_l sits in LDS; each
// wave stages its 16 x C row tile in LDS and accumulates 16 x C outputs (C/16 MFMA tiles).
#include <hipcub/hipcub.hpp>

#include "common.h"
#include "params.h"

namespace equitp {
namespace {

constexpr int kLinWaves = 4;

template <int C>
__global__ void __launch_bounds__(kLinWaves * 64)
linear_kernel(int n_nodes, int F, int l, const float* __restrict__ feat,
              const float* __restrict__ W, int transpose_w, float* __restrict__ out) {
  constexpr int NT = C / 16;
  constexpr int AS = C + 4;  // row stride of the staged row tile
  __shared__ float ws[C * C];
  __shared__ float as[kLinWaves * 16 * AS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int es = lane & 15, q = lane >> 4;
  const int dl = 2 * l + 1;
  const int rows = n_nodes * dl;
  // ws[k][j] = W_l[k][j], or W_l[j][k] for the transposed product
  for (int idx = tid; idx < C * C; idx += blockDim.x) {
    const int k = idx / C, j = idx % C;
    ws[idx] = transpose_w ? W[j * C + k] : W[idx];
  }
  float* at = as + wave * 16 * AS;
  const int row0 = blockIdx.x * (kLinWaves * 16) + wave * 16;
  for (int idx = lane; idx < 16 * C; idx += 64) {
    const int rr = idx / C, k = idx % C;
    const int row = row0 + rr;
    float v = 0.0f;
    if (row < rows) {
      const int n = row / dl, m = row % dl;
      v = feat[((size_t)n * F + l * l + m) * C + k];
    }
    at[rr * AS + k] = v;
  }
  __syncthreads();
  f4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  // D[i = row es'][j = col] : A[i][kk] = at[i][4s + kk], B[kk][j] = ws[4s + kk][16 t + j]
#pragma unroll 4
  for (int s = 0; s < C / 4; ++s) {
    const float a = at[es * AS + 4 * s + q];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = mfma_16x16x4(a, ws[(4 * s + q) * C + 16 * t + es], acc[t]);
  }
  // lane holds D[4q + r][es] of column tile t: row row0 + 4q + r, column 16 t + es
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + 4 * q + r;
    if (row < rows) {
      const int n = row / dl, m = row % dl;
      float* op = out + ((size_t)n * F + l * l + m) * C;
#pragma unroll
      for (int t = 0; t < NT; ++t) op[16 * t + es] = acc[t][r];
    }
  }
}

__global__ void iota_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = i;
}

// row_ptr[k] = first position whose sorted key is >= k (binary search), row_ptr[n_keys] = n.
__global__ void row_ptr_kernel(const int32_t* __restrict__ sorted, int n, int n_keys,
                               int32_t* __restrict__ row_ptr) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k > n_keys) return;
  if (k == n_keys) {
    row_ptr[k] = n;
    return;
  }
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sorted[mid] < k) lo = mid + 1;
    else hi = mid;
  }
  row_ptr[k] = lo;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

hipError_t launch_linear(int n_nodes, int lmax, int C, const float* feat, const float* W,
                         int transpose_w, float* out, hipStream_t stream) {
  const int F = (lmax + 1) * (lmax + 1);
  for (int l = 0; l <= lmax; ++l) {
    const int rows = n_nodes * (2 * l + 1);
    const int grid = (rows + kLinWaves * 16 - 1) / (kLinWaves * 16);
    if (grid == 0) continue;
    const float* Wl = W + (size_t)l * C * C;
    switch (C) {
      case 16:
        hipLaunchKernelGGL(linear_kernel<16>, dim3(grid), dim3(kLinWaves * 64), 0, stream, n_nodes, F, l, feat, Wl, transpose_w, out);
        break;
      case 32:
        hipLaunchKernelGGL(linear_kernel<32>, dim3(grid), dim3(kLinWaves * 64), 0, stream, n_nodes, F, l, feat, Wl, transpose_w, out);
        break;
      case 64:
        hipLaunchKernelGGL(linear_kernel<64>, dim3(grid), dim3(kLinWaves * 64), 0, stream, n_nodes, F, l, feat, Wl, transpose_w, out);
        break;
      case 128:
        hipLaunchKernelGGL(linear_kernel<128>, dim3(grid), dim3(kLinWaves * 64), 0, stream, n_nodes, F, l, feat, Wl, transpose_w, out);
        break;
      default:
        return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

size_t csr_workspace_bytes(int n_keys, int n) {
  size_t cub_bytes = 0;
  hipcub::DeviceRadixSort::SortPairs(nullptr, cub_bytes, (const int32_t*)nullptr, (int32_t*)nullptr,
                                     (const int32_t*)nullptr, (int32_t*)nullptr, n);
  (void)n_keys;
  return align256((size_t)n * 4) * 2 + align256(cub_bytes);
}

hipError_t launch_build_csr(int n_keys, int n, const int32_t* key, int32_t* row_ptr, int32_t* perm,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  int32_t* iota = reinterpret_cast<int32_t*>(w);
  int32_t* sorted = reinterpret_cast<int32_t*>(w + align256((size_t)n * 4));
  void* tmp = w + 2 * align256((size_t)n * 4);
  size_t tmp_bytes = ws_bytes - 2 * align256((size_t)n * 4);
  if (n > 0) {
    hipLaunchKernelGGL(iota_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, iota, n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = hipcub::DeviceRadixSort::SortPairs(tmp, tmp_bytes, key, sorted, iota, perm, n, 0,
                                             32, stream);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(row_ptr_kernel, dim3((n_keys + 1 + 255) / 256), dim3(256), 0, stream, sorted,
                     n, n_keys, row_ptr);
  return hipGetLastError();
}

}  // namespace equitp
