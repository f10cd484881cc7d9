// Block copies for the convolution with mixed per-l multiplicities (composed from the uniform
// kernels on channel slices; see equitp.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "params.h"

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

// Row copies: dst row r, columns [0, cols) = src row r, for r < rows, several jobs per launch
// (any number of jobs; up to kCopyBatch per launch).  cols, the row starts and the bases must be
// multiples of 4 floats (16-byte accesses); the jobs of one call must not overlap.
struct CopyJob {
  RowMap dst, src;
  int rows, cols;
};
constexpr int kCopyBatch = 24;
hipError_t launch_copy_batch(const CopyJob* jobs, int n_jobs, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
// p[i] = i
hipError_t launch_iota(int32_t* p, int n, hipStream_t st);

// The masked backward's path groups (conv_bwd.hip): group of path j at every l <= L, and a launch
// of only some groups (bit g = group g) for masks that keep no path of the others.
int bwd_path_group(int L, int j);
hipError_t launch_bwd_masked_groups(const ConvShape& s, const BwdParams& p, unsigned groups,
                                    hipStream_t st);
// y[i] += x[i]
hipError_t launch_add(float* y, const float* x, size_t n, hipStream_t st);

}  // namespace equitp
