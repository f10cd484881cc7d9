// Per-irrep channel-mixing linear on the matrix cores, and the CSR builder for the sender-grouped
// (transpose) edge order.
//
// Linear: for each l, out[n, l*l + m, :] = feat[n, l*l + m, :] W_l, a GEMM with M = n_nodes (2l+1)
// rows (row (n, m) at offset (n F + l*l + m) C), K = N = C.  This is the dense 128 x 128 channel
// mixing that follows a convolution in an interaction block (FlashCart, Fig. 3 caption: linear
// maps that mix paths and channels between steps).  fp32 MFMA 16x16x4 (no reduced-precision
// inputs: "Fast and Accurate Foundation Models for Equivariant MLIPs", Sec. II and VII keep TF32
// off where accuracy matters).  One launch covers every l: a work-group takes 32 rows of one l,
// stages W_l (or its transpose) and the 32 x C row tile in LDS with 16-byte loads, and its four
// waves each compute a 16-row x C/2-column block.
#include <hipcub/hipcub.hpp>

#include "common.h"
#include "params.h"

namespace equitp {
namespace {

constexpr int kLinWaves = 4;
constexpr int kLinRows = 32;

struct LinTiles {
  int first_tile[5];  // work-group index where irrep l starts; first_tile[lmax + 1] = total
};

template <int C>
__global__ void __launch_bounds__(kLinWaves * 64)
linear_kernel(int n_nodes, int F, int lmax, LinTiles tiles, const float* __restrict__ feat,
              const float* __restrict__ W, int transpose_w, float* __restrict__ out) {
  constexpr int WS = C + 4;           // row stride of the staged W_l
  constexpr int AS = C + 4;           // row stride of the staged row tile
  // columns per wave: C/2 (four waves as 2 row blocks x 2 column halves); for C = 16 the two
  // row blocks take all columns and waves 2 and 3 only help staging
  constexpr int CW = C >= 32 ? C / 2 : C;
  constexpr int NT = CW / 16;         // 16-column MFMA tiles per wave
  extern __shared__ float lds[];
  float* ws = lds;                    // [C][WS]: ws[k][j] = W_l[k][j] (or W_l[j][k])
  float* at = lds + C * WS;           // [kLinRows][AS]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int es = lane & 15, q = lane >> 4;
  int l = 0;
  while (l < lmax && (int)blockIdx.x >= tiles.first_tile[l + 1]) ++l;
  const int dl = 2 * l + 1;
  const int rows = n_nodes * dl;
  const int row0 = ((int)blockIdx.x - tiles.first_tile[l]) * kLinRows;
  const float* Wl = W + (size_t)l * C * C;
  // W_l: 16-byte loads along its rows; the transpose goes through registers in 4 x 4 blocks so
  // that LDS is written with 16-byte stores as well
  if (!transpose_w) {
    for (int idx = tid; idx < C * C / 4; idx += kLinWaves * 64) {
      const int r = idx / (C / 4), c4 = (idx % (C / 4)) * 4;
      st4(&ws[r * WS + c4], ld4(Wl + (size_t)r * C + c4));
    }
  } else {
    for (int idx = tid; idx < (C / 4) * (C / 4); idx += kLinWaves * 64) {
      const int r4 = (idx / (C / 4)) * 4, c4 = (idx % (C / 4)) * 4;
      f4 b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = ld4(Wl + (size_t)(r4 + i) * C + c4);
#pragma unroll
      for (int j = 0; j < 4; ++j) st4(&ws[(c4 + j) * WS + r4], f4{b[0][j], b[1][j], b[2][j], b[3][j]});
    }
  }
  // the row tile: row (n, m) of irrep l is a contiguous C-float row of feat
  for (int idx = tid; idx < kLinRows * C / 4; idx += kLinWaves * 64) {
    const int rr = idx / (C / 4), c4 = (idx % (C / 4)) * 4;
    const int row = row0 + rr;
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < rows) {
      const int n = row / dl, m = row % dl;
      v = ld4(feat + ((size_t)n * F + l * l + m) * C + c4);
    }
    st4(&at[rr * AS + c4], v);
  }
  __syncthreads();
  const int rb = C >= 32 ? 16 * (wave >> 1) : 16 * wave;
  const int cb = C >= 32 ? CW * (wave & 1) : 0;
  if (rb >= kLinRows) return;
  f4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  // D[i = row][j = col]: A[i][kk] = at[rb + i][4s + kk], B[kk][j] = ws[4s + kk][cb + 16 t + j]
#pragma unroll 4
  for (int s = 0; s < C / 4; ++s) {
    const float a = at[(rb + es) * AS + 4 * s + q];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = mfma_16x16x4(a, ws[(4 * s + q) * WS + cb + 16 * t + es], acc[t]);
  }
  // lane holds D[4q + r][es] of column tile t
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + rb + 4 * q + r;
    if (row < rows) {
      const int n = row / dl, m = row % dl;
      float* op = out + ((size_t)n * F + l * l + m) * C + cb;
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
  LinTiles tiles{};
  int total = 0;
  for (int l = 0; l <= lmax; ++l) {
    tiles.first_tile[l] = total;
    total += (n_nodes * (2 * l + 1) + kLinRows - 1) / kLinRows;
  }
  tiles.first_tile[lmax + 1] = total;
  if (total == 0) return hipSuccess;
  const size_t lds = (size_t)(C * (C + 4) + kLinRows * (C + 4)) * sizeof(float);
  auto go = [&](auto kern) -> hipError_t {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(total), dim3(kLinWaves * 64), lds, stream, n_nodes, F, lmax, tiles,
                       feat, W, transpose_w, out);
    return hipGetLastError();
  };
  switch (C) {
    case 16: return go(linear_kernel<16>);
    case 32: return go(linear_kernel<32>);
    case 64: return go(linear_kernel<64>);
    case 128: return go(linear_kernel<128>);
    default: return hipErrorInvalidValue;
  }
}

size_t csr_workspace_bytes(int n_keys, int n) {
  size_t cub_bytes = 0;
  hipcub::DeviceRadixSort::SortPairs(nullptr, cub_bytes, (const int32_t*)nullptr, (int32_t*)nullptr,
                                     (const int32_t*)nullptr, (int32_t*)nullptr, n);
  (void)n_keys;
  return align256((size_t)n * 4) * 2 + align256(cub_bytes);
}

// key[t] = 32 - number of paths any edge of tile t needs
__global__ void tile_key_kernel(const uint32_t* __restrict__ mask, int n_edges, int n_tiles,
                                uint32_t* __restrict__ key) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_tiles) return;
  uint32_t m = 0;
  const int e0 = 16 * t, e1 = min(n_edges, e0 + 16);
  for (int e = e0; e < e1; ++e) m |= mask[e];
  key[t] = 32u - (uint32_t)__popc(m);
}

size_t tile_order_workspace_bytes(int n_edges) {
  const int n_tiles = (n_edges + 15) / 16;
  size_t cub_bytes = 0;
  hipcub::DeviceRadixSort::SortPairs(nullptr, cub_bytes, (const uint32_t*)nullptr, (uint32_t*)nullptr,
                                     (const int32_t*)nullptr, (int32_t*)nullptr, n_tiles);
  return align256((size_t)n_tiles * 4) * 3 + align256(cub_bytes);
}

hipError_t launch_tile_order(int n_edges, const uint32_t* path_mask, int32_t* tile_order, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  const int n_tiles = (n_edges + 15) / 16;
  char* w = static_cast<char*>(ws);
  const size_t a = align256((size_t)n_tiles * 4);
  uint32_t* key = reinterpret_cast<uint32_t*>(w);
  uint32_t* key_sorted = reinterpret_cast<uint32_t*>(w + a);
  int32_t* iota = reinterpret_cast<int32_t*>(w + 2 * a);
  void* tmp = w + 3 * a;
  size_t tmp_bytes = ws_bytes - 3 * a;
  if (n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_key_kernel, dim3((n_tiles + 255) / 256), dim3(256), 0, stream, path_mask,
                     n_edges, n_tiles, key);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(iota_kernel, dim3((n_tiles + 255) / 256), dim3(256), 0, stream, iota, n_tiles);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // keys are at most 32: six bits
  return hipcub::DeviceRadixSort::SortPairs(tmp, tmp_bytes, key, key_sorted, iota, tile_order,
                                            n_tiles, 0, 6, stream);
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
