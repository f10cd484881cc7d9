// Kernel argument blocks and launcher declarations shared by the host dispatcher and the
// kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace equitp {

// Static configuration of one convolution: irreps 0..L for input, SH and output, uniform
// multiplicity C per l, radial MLP n_radial -> hidden -> n_paths * C.
struct ConvShape {
  int L_in, L_sh, L_out;
  int C;
  int n_radial;
  int hidden;
  int n_paths;
  float r_cut;
  int mlp_bf16;   // 1: the W2 contractions take bf16 operands (fp32 accumulation)
};

// Segment-sum kernel: forward (segments = receivers, gather x[src]) or the input gradient
// (segments = senders via a permutation, gather G[dst], transpose of each CG block).
struct SegParams {
  int n_seg;
  int C;
  int n_slices;
  int wg_per_slice;
  const int32_t* seg_ptr;    // [n_seg + 1]
  const int32_t* seg_edge;   // nullptr: edge id = position; else edge id = seg_edge[position]
  const int32_t* gather;     // [E] node gathered by each edge
  const float* vec;          // [E][3]
  const float* feat;         // [N][F_gather][C]
  const float* W1;           // [n_radial][hidden]
  const float* W2;           // [hidden][n_paths * C]
  float* out;                // [n_seg][F_scatter][C]
  float inv_r_cut;          // 1 / r_c
  float radial_pref;        // sqrt(2 / r_c), the Bessel-basis prefactor
  const uint32_t* path_mask; // [E] per-edge path bitmask (masked kernels only), by edge id
};

// Fused backward: per channel slice and edge range, dL/dvec partials (one per slice), dL/dW2
// partials (one per work-group, covering its slice's columns) and dL/dW1 partials (one per wave).
struct BwdParams {
  int n_edges;
  int C;
  int n_slices;
  int wg_per_slice;
  const int32_t* src;
  const int32_t* dst;
  const float* vec;
  const float* x;            // [N][F_in][C]
  const float* G;            // [N][F_out][C]
  const float* W1;           // [n_radial][hidden]
  const float* W2;           // [hidden][n_paths * C]
  float* dvec_part;          // [n_slices][E][3] or null (group 0 writes, later groups add)
  float* dW2_part;           // [wg_per_slice][hidden][n_paths * C] or null
  float* dW1_part;           // [gridDim][n_radial][hidden] or null (group 0 writes, later groups add)
  float inv_r_cut;          // 1 / r_c
  float radial_pref;        // sqrt(2 / r_c), the Bessel-basis prefactor
  const uint32_t* path_mask; // [E] per-edge path bitmask (masked kernels only)
  // masked kernels: the 16-edge tiles (tile t = edges 16t .. 16t + 15) in processing order
  int n_tiles;
  const int32_t* tile_order;  // [n_tiles]
};

// Node-local product ladder: lane = (node, channel); a wave task covers cw consecutive channels
// (cw in {16, 32, 64}, dividing C) of 64 / cw consecutive nodes; task t serves channel group
// t % n_groups.  The backward runs n_groups * blocks_per_group work-groups and writes dL/dw
// partials [blocks_per_group][nu-1][n_paths][C].
struct LadderParams {
  int n_nodes;
  int C;
  int cw;
  int n_groups;          // C / cw
  int n_tasks;           // n_groups * ceil(n_nodes / (64 / cw))
  int blocks_per_group;
  const float* A;        // [N][(L+1)^2][C]
  const float* w;        // [nu-1][n_paths][C]
  const float* G;        // [N][(L+1)^2][C] (backward)
  float* out;            // [N][(L+1)^2][C] (forward)
  float* dA;             // [N][(L+1)^2][C] or null
  float* dw_part;        // [blocks_per_group][nu-1][n_paths][C] or null
  float* rungs;          // [nu-2][N][(L+1)^2][C] B_2 .. B_{nu-1}: forward writes, backward reads; or null
};

hipError_t launch_seg_conv(const ConvShape& s, bool transpose, const SegParams& p, int n_cu,
                           hipStream_t stream);
hipError_t launch_seg_conv_masked(const ConvShape& s, bool transpose, const SegParams& p, int n_cu,
                                  hipStream_t stream);
hipError_t launch_bwd(const ConvShape& s, const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_masked(const ConvShape& s, const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_bf16(const ConvShape& s, const BwdParams& p, hipStream_t stream);
int bwd_wg_per_slice(const ConvShape& s, int n_edges, int n_cu);
int bwd_num_groups(const ConvShape& s);
constexpr int kBwdGroups = 4;   // most path groups of the backward (one launch each)
constexpr int kBwdWaves = 8;    // waves per backward work-group (two per SIMD)
hipError_t launch_sum_slices(const float* part, int n_slices, int n, float* out, hipStream_t stream);
hipError_t launch_reduce_rows(const float* part, int rows, int cols, float* out, hipStream_t stream);
hipError_t launch_linear(int n_nodes, int lmax, int C, const float* feat, const float* W,
                         int transpose_w, float* out, hipStream_t stream);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream);
int ladder_num_paths(int lmax);
int ladder_reduce_split();   // rows of the dL/dw reduction's intermediate
// dL/dw rows part [rows][cols] summed into out [cols] in a fixed order, through tmp
// [ladder_reduce_split()][cols]
hipError_t launch_ladder_reduce(const float* part, int rows, int cols, float* tmp, float* out,
                                hipStream_t stream);
hipError_t launch_ladder_fwd(int lmax, int nu, const LadderParams& p, hipStream_t stream);
hipError_t launch_ladder_bwd(int lmax, int nu, const LadderParams& p, bool want_dA, bool want_dw,
                             hipStream_t stream);
size_t csr_workspace_bytes(int n_keys, int n);
// Order of the 16-edge tiles for the masked backward: tiles whose edges need more paths first
// (stable: tiles with equal counts keep their order).
size_t tile_order_workspace_bytes(int n_edges);
hipError_t launch_tile_order(int n_edges, const uint32_t* path_mask, int32_t* tile_order, void* ws,
                             size_t ws_bytes, hipStream_t stream);
hipError_t launch_build_csr(int n_keys, int n, const int32_t* key, int32_t* row_ptr, int32_t* perm,
                            void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace equitp
