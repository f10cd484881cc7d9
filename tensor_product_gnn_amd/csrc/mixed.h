// Block copies for the convolution with mixed per-l multiplicities (composed from the uniform
// kernels on channel slices; see equitp.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace equitp {

// Row r of a strided view: base + (r / d) * stride_node + off + (r % d) * stride_m (floats).
// Node tensors: d = 2l+1 rows per node; plain matrices: d = 1, stride_node = leading dimension.
struct RowMap {
  float* base;
  int d;
  long long stride_node;
  long long off;
  int stride_m;
};

// dst row r, columns [0, cols) = (accumulate ? dst + : ) src row r, for r < rows.  cols, the row
// starts and the bases must be multiples of 4 floats (16-byte accesses).
hipError_t launch_copy_rows(RowMap dst, RowMap src, int rows, int cols, bool accumulate,
                            hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
// y[i] += x[i]
hipError_t launch_add(float* y, const float* x, size_t n, hipStream_t st);

}  // namespace equitp
