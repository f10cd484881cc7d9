// Launchers of the full product ladder (per-path channel-mixing maps between steps).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace equitp {

// Sum of (2 l3 + 1) over the ladder's paths at this lmax: the rows of path outputs per node.
int full_ladder_dsum(int lmax);
// Work-groups (and partial maps) of one step's dL/dW GEMM.
int full_ladder_dw_blocks(int lmax, int n_nodes, int C);
// Whether the kernels take this channel count (32, 64, 128).
bool full_ladder_channels_ok(int C);

// T[p][n][m3][u] = sum C_p[m1, m2, m3] Bp[n, l1 m1, u] A[n, l2 m2, u] for every path p.
hipError_t launch_full_tp(int lmax, int n_nodes, int C, const float* Bp, const float* A, float* T,
                          hipStream_t st);
// B_s[n, l3 m3, v] = sum_{p -> l3} sum_u T[p][n][m3][u] W[p][u][v]; out = / += B_s; bnext = B_s
// (either may be null).
hipError_t launch_mix_fwd(int lmax, int n_nodes, int C, const float* T, const float* W, float* out,
                          bool accumulate, float* bnext, hipStream_t st);
// dT[p][n][m3][u] = sum_v Gs[n, l3 m3, v] W[p][u][v].
hipError_t launch_mix_dt(int lmax, int n_nodes, int C, const float* Gs, const float* W, float* dT,
                         hipStream_t st);
// dW[p] = sum_{n, m3} T[p][n][m3][:]^T Gs[n, l3 m3, :]: partial maps per row range, then their
// sum per path in a fixed order.
hipError_t launch_mix_dw(int lmax, int n_nodes, int C, const float* T, const float* Gs,
                         float* part, float* dW, hipStream_t st);
// From dT (the gradient of every path output) of one step: dB = dL/dBp, dA_step = dL/dA.
// Gs_next = G + dB (if not null); dA = (accumulate ? dA : 0) + dA_step (+ dB when add_dB, the
// last step, where Bp is A).
hipError_t launch_full_tp_bwd(int lmax, int n_nodes, int C, const float* Bp, const float* A,
                              const float* dT, const float* G, float* Gs_next, float* dA,
                              bool accumulate, bool add_dB, hipStream_t st);

}  // namespace equitp
