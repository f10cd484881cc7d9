// Node-local product ladder with path-reduced products ("FlashCart: Fast Cartesian Tensor
// Products for Equivariant Interatomic Potentials", Fig. 3(b) and Fig. E1(b)), per node n and
// channel c, for correlation order nu:
//
//   B_1 = A,   B_s[l3 m3] = sum_p w[s-2][p][c] sum_{m1,m2} C_p[m1,m2,m3] B_{s-1}[l1 m1] A[l2 m2],
//   out = B_2 + ... + B_nu,
//
// over the parity-allowed paths p = (l1, l2, l3) with every l <= L (lexicographic order, the
// same path table as the edge convolution).
//
// Work mapping: one lane owns one (node, channel) pair.  Node tensors are [N][(L+1)^2][C] with
// channels innermost, so a wave covers 64 consecutive channels of one node (or 64/C nodes when
// C < 64) and every load and store is a whole 256-byte row.  Both factors of each product vary
// per channel and the CG blocks are sparse, so there is no dense contraction to give to the
// matrix cores: the products run on the VALU, unrolled over the CG nonzeros with the values as
// instruction literals.  Per product and (node, channel), grouping the entries of each path by
// (m3, m1):  u = sum_m2 C A[l2 m2]  (one FMA per entry),  t[m3] += B[l1 m1] u  (one per group),
// out[l3 m3] += w_p t[m3]  (one per output component).
//
// The backward takes B_2..B_{nu-1} from the forward when the caller kept them (the forward writes
// them as it goes; compute-bound, it has bandwidth to spare), else recomputes them in registers;
// then it walks the steps from nu down to 2
// with the gradient Gh_s = G + (gradient reaching B_s through step s+1):
//   dw[s-2][p][c] += sum_m3 Gh_s[l3 m3] t[m3]
//   dB_{s-1}[l1 m1] += sum_m3 w_p Gh_s[l3 m3] u(m1, m3)
//   dA[l2 m2]       += sum_{m1,m3} C_p[m1,m2,m3] B_{s-1}[l1 m1] w_p Gh_s[l3 m3]
// and finally dA += dB_1 (B_1 is A).  dw is a sum over nodes: the waves of a work-group add each
// step's dL/dw into the work-group's LDS sums in a fixed wave order, the work-group writes one
// partial row per channel group, and a fixed-order row reduction adds the partials (no atomics;
// results are reproducible).  The
// path weights are staged in LDS once per work-group, so a step never waits on L2 for them.
#include <hip/hip_runtime.h>

#include "common.h"
#include "params.h"

namespace equitp {
namespace {

constexpr int kLadWaves = 4;

// Entry k of global path gp and its neighbours: the table lists each path's entries sorted by
// (m3, m1, m2), so the entries sharing (m1, m3) are contiguous.
constexpr bool same_pair(int gp, int a, int b) {
  return cg::kEnt[cg::kPaths[gp].off + a].m1 == cg::kEnt[cg::kPaths[gp].off + b].m1 &&
         cg::kEnt[cg::kPaths[gp].off + a].m3 == cg::kEnt[cg::kPaths[gp].off + b].m3;
}
constexpr bool group_first(int gp, int k) { return k == 0 || !same_pair(gp, k, k - 1); }
constexpr bool group_last(int gp, int k) {
  return k == cg::kPaths[gp].nnz - 1 || !same_pair(gp, k, k + 1);
}
constexpr int group_start(int gp, int k) {
  while (!group_first(gp, k)) --k;
  return k;
}
// Whether entry k (a group's first entry) opens the first group of its m3.
constexpr bool m3_first(int gp, int k) {
  return k == 0 || cg::kEnt[cg::kPaths[gp].off + k - 1].m3 != cg::kEnt[cg::kPaths[gp].off + k].m3;
}
constexpr bool has_m3(int gp, int m3) {
  for (int k = 0; k < cg::kPaths[gp].nnz; ++k)
    if (cg::kEnt[cg::kPaths[gp].off + k].m3 == m3) return true;
  return false;
}

template <int L>
struct Lad {
  using PS = PathSet<L, L, L>;
  static constexpr int P = PS::N;
  static constexpr int F = (L + 1) * (L + 1);
};

// Redefines the values in place through an empty asm statement.  Volatile asm statements keep
// their order, so calling this on a path's operands before it and on its accumulators after it
// pins each path's arithmetic between the two: without it the compiler is free to hoist the
// per-path sums over A of every path (and, across the unrolled steps, to keep them from the first
// step to the last), which needs far more registers than a lane has.
template <int N>
__device__ __forceinline__ void opaque(float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" : "+v"(v[k]));
}

// Path weights of one step for one lane, read from LDS (stride 64 floats between paths).
struct LdsWeights {
  const float* p;
  __device__ __forceinline__ float operator[](int j) const { return p[j * 64]; }
};

// nxt[l3 m3] += sum_p w[p] (B (x)_p A)[m3].  W: a register array or LdsWeights.
template <int L, typename W>
__device__ __forceinline__ void product(float (&B)[Lad<L>::F], float (&A)[Lad<L>::F], const W& w,
                                        float (&nxt)[Lad<L>::F]) {
  static_for<Lad<L>::P>([&](auto j) {
    opaque(A);
    opaque(B);
    constexpr int gp = Lad<L>::PS::id(j);
    constexpr cg::PathDesc pd = cg::kPaths[gp];
    const float wj = w[j];
    float t[2 * pd.l3 + 1];
    float u = 0.0f;
    static_for<pd.nnz>([&](auto k) {
      constexpr cg::Ent e = cg::kEnt[pd.off + k];
      constexpr float v = cg::kVal[pd.off + k];
      const float a = A[pd.l2 * pd.l2 + e.m2];
      if constexpr (group_first(gp, k)) u = v * a;
      else u = __builtin_fmaf(v, a, u);
      if constexpr (group_last(gp, k)) {
        const float b = B[pd.l1 * pd.l1 + e.m1];
        if constexpr (m3_first(gp, group_start(gp, k))) t[e.m3] = b * u;
        else t[e.m3] = __builtin_fmaf(b, u, t[e.m3]);
      }
    });
    static_for<2 * pd.l3 + 1>([&](auto m3) {
      if constexpr (has_m3(gp, m3))
        nxt[pd.l3 * pd.l3 + m3] = __builtin_fmaf(wj, t[m3], nxt[pd.l3 * pd.l3 + m3]);
    });
    opaque(nxt);
  });
}

// Backward of one product with respect to its first factor Bp (dB +=), its second factor A
// (dA +=) and its path weights (dwv +=), for the gradient Gh of its output.
template <int L, typename W>
__device__ __forceinline__ void product_bwd(float (&Bp)[Lad<L>::F], float (&A)[Lad<L>::F],
                                            const W& w, const float (&Gh)[Lad<L>::F],
                                            float (&dB)[Lad<L>::F], float (&dA)[Lad<L>::F],
                                            float (&dwv)[Lad<L>::P]) {
  static_for<Lad<L>::P>([&](auto j) {
    opaque(A);
    opaque(Bp);
    constexpr int gp = Lad<L>::PS::id(j);
    constexpr cg::PathDesc pd = cg::kPaths[gp];
    constexpr int o1 = pd.l1 * pd.l1, o2 = pd.l2 * pd.l2, o3 = pd.l3 * pd.l3;
    const float wj = w[j];
    float gw[2 * pd.l3 + 1];
    static_for<2 * pd.l3 + 1>([&](auto m3) { gw[m3] = wj * Gh[o3 + m3]; });
    float t[2 * pd.l3 + 1];
    float u = 0.0f, bg = 0.0f;
    static_for<pd.nnz>([&](auto k) {
      constexpr cg::Ent e = cg::kEnt[pd.off + k];
      constexpr float v = cg::kVal[pd.off + k];
      const float a = A[o2 + e.m2];
      if constexpr (group_first(gp, k)) {
        u = v * a;
        bg = Bp[o1 + e.m1] * gw[e.m3];
      } else {
        u = __builtin_fmaf(v, a, u);
      }
      dA[o2 + e.m2] = __builtin_fmaf(v, bg, dA[o2 + e.m2]);
      if constexpr (group_last(gp, k)) {
        const float b = Bp[o1 + e.m1];
        if constexpr (m3_first(gp, group_start(gp, k))) t[e.m3] = b * u;
        else t[e.m3] = __builtin_fmaf(b, u, t[e.m3]);
        dB[o1 + e.m1] = __builtin_fmaf(gw[e.m3], u, dB[o1 + e.m1]);
      }
    });
    float d = 0.0f;
    static_for<2 * pd.l3 + 1>([&](auto m3) {
      if constexpr (has_m3(gp, m3)) d = __builtin_fmaf(Gh[o3 + m3], t[m3], d);
    });
    dwv[j] += d;
    opaque(dA);
    opaque(dB);
  });
}

// Lane -> (node, channel) of wave task `task`: channel group cgp = task % n_groups covers
// channels [cgp * cw, cgp * cw + cw), node group task / n_groups covers 64 / cw nodes.
struct LaneItem {
  int node, chan;
};
__device__ __forceinline__ LaneItem lane_item(const LadderParams& p, int task, int lane) {
  const int cgp = task % p.n_groups;
  const int npw = 64 / p.cw;
  return {(task / p.n_groups) * npw + lane / p.cw, cgp * p.cw + lane % p.cw};
}

template <int L>
__device__ __forceinline__ void load_feat(const float* __restrict__ src, const LadderParams& p,
                                          LaneItem it, float (&v)[Lad<L>::F]) {
  // lanes past the last node (only in a partly filled wave when C < 64) read the last node and
  // take zeros: unconditional loads keep the array in plain registers
  const bool ok = it.node < p.n_nodes;
  const float* ptr = src + (size_t)min(it.node, p.n_nodes - 1) * Lad<L>::F * p.C + it.chan;
#pragma unroll
  for (int k = 0; k < Lad<L>::F; ++k) {
    const float x = __builtin_nontemporal_load(ptr + (size_t)k * p.C);
    v[k] = ok ? x : 0.0f;
  }
}

template <int L>
__device__ __forceinline__ void load_w(const LadderParams& p, int step, int chan, float (&w)[Lad<L>::P]) {
  const float* ptr = p.w + (size_t)step * Lad<L>::P * p.C + chan;
#pragma unroll
  for (int j = 0; j < Lad<L>::P; ++j) w[j] = ptr[(size_t)j * p.C];
}

template <int L, int NU>
__global__ void __launch_bounds__(kLadWaves * 64) ladder_fwd_kernel(LadderParams p) {
  constexpr int F = Lad<L>::F, P = Lad<L>::P;
  const int lane = threadIdx.x % 64;
  const int task = blockIdx.x * kLadWaves + threadIdx.x / 64;
  if (task >= p.n_tasks) return;
  const LaneItem it = lane_item(p, task, lane);
  float A[F], B[F], out[F];
  load_feat<L>(p.A, p, it, A);
#pragma unroll
  for (int k = 0; k < F; ++k) {
    B[k] = A[k];
    out[k] = 0.0f;
  }
  // a rolled loop over the steps keeps the next step's weight loads from being hoisted over
  // this step's product (which would hold all steps' weights in registers at once)
#pragma unroll 1
  for (int q = 0; q < NU - 1; ++q) {
    float w[P], nxt[F];
    load_w<L>(p, q, it.chan, w);
#pragma unroll
    for (int k = 0; k < F; ++k) nxt[k] = 0.0f;
    product<L>(B, A, w, nxt);
#pragma unroll
    for (int k = 0; k < F; ++k) {
      out[k] += nxt[k];
      B[k] = nxt[k];
    }
    // B_{q+2} for the backward, when the caller keeps the rungs (q < NU - 2)
    if (p.rungs != nullptr && q < NU - 2 && it.node < p.n_nodes) {
      float* rdst = p.rungs + ((size_t)q * p.n_nodes + it.node) * F * p.C + it.chan;
#pragma unroll
      for (int k = 0; k < F; ++k) __builtin_nontemporal_store(nxt[k], rdst + (size_t)k * p.C);
    }
  }
  if (it.node < p.n_nodes) {
    float* dst = p.out + (size_t)it.node * F * p.C + it.chan;
#pragma unroll
    for (int k = 0; k < F; ++k) __builtin_nontemporal_store(out[k], dst + (size_t)k * p.C);
  }
}

// Work-group g serves channel group g % n_groups and node groups [first, last) of that channel
// group; its waves take those node groups in turn.
// LDS of the backward, in floats: the work-group's dL/dw sums [NS][P][64] (when dL/dw is wanted),
// then every step's path weights for the work-group's channels [NS][P][64].
template <int L, int NU, bool WD>
constexpr size_t bwd_lds_floats() {
  return (size_t)((WD ? 1 : 0) + 1) * (NU - 1) * Lad<L>::P * 64;
}

// Work-group g serves channel group g % n_groups and node groups [first, last) of that channel
// group; its waves take those node groups in turn, all waves running the same number of rounds
// (a node group past `last` contributes zeros), so that they can add their dL/dw of each step
// into the work-group's sums in a fixed wave order between barriers: one set of sums per
// work-group instead of one per wave leaves LDS for two work-groups per CU, and the order keeps
// the results reproducible.
// LB: the rungs B_2 .. B_{NU-1} come from p.rungs (kept by the forward) instead of being
// recomputed.
template <int L, int NU, bool WA, bool WD, bool LB>
__global__ void __launch_bounds__(kLadWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
ladder_bwd_kernel(LadderParams p) {
  constexpr int F = Lad<L>::F, P = Lad<L>::P, NS = NU - 1;
  extern __shared__ float lds[];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int cgp = blockIdx.x % p.n_groups, blk = blockIdx.x / p.n_groups;
  const int n_ng = p.n_tasks / p.n_groups;
  const int per = (n_ng + p.blocks_per_group - 1) / p.blocks_per_group;
  const int first = blk * per, last = min(n_ng, first + per);
  float* sums = lds;                                            // [NS][P][64] when WD
  float* w_lds = lds + (WD ? (size_t)NS * P * 64 : 0);          // [NS][P][64]
  if constexpr (WD) {
    for (int i = threadIdx.x; i < NS * P * 64; i += kLadWaves * 64) sums[i] = 0.0f;
  }
  // every step's path weights for this group's channels, one copy per lane (lanes holding the
  // same channel for different nodes read the same value), staged once
  for (int i = threadIdx.x; i < NS * P * 64; i += kLadWaves * 64) {
    const int l = i % 64, qj = i / 64;
    w_lds[i] = p.w[(size_t)qj * p.C + cgp * p.cw + l % p.cw];
  }
  __syncthreads();
  constexpr int NB = NU > 2 ? NU - 2 : 1;
  const int rounds = last > first ? (last - first + kLadWaves - 1) / kLadWaves : 0;
  for (int r = 0; r < rounds; ++r) {
    const int g = first + wave + r * kLadWaves;
    const bool live = g < last;
    // a node group past `last` reads the last one and contributes nothing (G = 0)
    const LaneItem it = lane_item(p, (live ? g : last - 1) * p.n_groups + cgp, lane);
    float A[F], G[F];
    float Bs[NB][F];
    load_feat<L>(p.A, p, it, A);
    load_feat<L>(p.G, p, it, G);
    if (!live) {
#pragma unroll
      for (int k = 0; k < F; ++k) G[k] = 0.0f;
    }
    if constexpr (LB) {
      static_for<NU - 2>([&](auto q) {
        load_feat<L>(p.rungs + (size_t)q * p.n_nodes * F * p.C, p, it, Bs[q]);
      });
    } else {
      // B_2 .. B_{NU-1}, recomputed
      static_for<NU - 2>([&](auto q) {
        const LdsWeights w{w_lds + q * P * 64 + lane};
#pragma unroll
        for (int k = 0; k < F; ++k) Bs[q][k] = 0.0f;
        if constexpr (q == 0) product<L>(A, A, w, Bs[0]);
        else product<L>(Bs[q - 1], A, w, Bs[q]);
      });
    }
    float Gh[F], dA[F];
#pragma unroll
    for (int k = 0; k < F; ++k) {
      Gh[k] = G[k];
      dA[k] = 0.0f;
    }
    static_for<NS>([&](auto rr) {
      constexpr int q = NS - 1 - rr;      // step s = q + 2, from NU down to 2
      const LdsWeights w{w_lds + q * P * 64 + lane};
      float dB[F], dwv[P];
#pragma unroll
      for (int k = 0; k < F; ++k) dB[k] = 0.0f;
#pragma unroll
      for (int j = 0; j < P; ++j) dwv[j] = 0.0f;
      if constexpr (q == 0) product_bwd<L>(A, A, w, Gh, dB, dA, dwv);
      else product_bwd<L>(Bs[q - 1], A, w, Gh, dB, dA, dwv);
      if constexpr (WD) {
        for (int wv = 0; wv < kLadWaves; ++wv) {
          __syncthreads();
          if (wave == wv) {
#pragma unroll
            for (int j = 0; j < P; ++j) sums[(q * P + j) * 64 + lane] += dwv[j];
          }
        }
      }
      if constexpr (q > 0) {
#pragma unroll
        for (int k = 0; k < F; ++k) Gh[k] = G[k] + dB[k];
      } else {
#pragma unroll
        for (int k = 0; k < F; ++k) dA[k] += dB[k];
      }
    });
    if constexpr (WA) {
      if (live && it.node < p.n_nodes) {
        float* dst = p.dA + (size_t)it.node * F * p.C + it.chan;
#pragma unroll
        for (int k = 0; k < F; ++k) __builtin_nontemporal_store(dA[k], dst + (size_t)k * p.C);
      }
    }
  }
  if constexpr (WD) {
    __syncthreads();
    // partial row blk: [NS][P][C], this group's channels; sum over the lanes that hold the same
    // channel (64 / cw nodes per wave), in a fixed order
    const int npw = 64 / p.cw;
    float* row = p.dw_part + (size_t)blk * NS * P * p.C;
    for (int i = threadIdx.x; i < NS * P * p.cw; i += kLadWaves * 64) {
      const int sp = i / p.cw, c = i % p.cw;
      float sum = 0.0f;
      for (int ns = 0; ns < npw; ++ns) sum += sums[(size_t)sp * 64 + ns * p.cw + c];
      row[(size_t)sp * p.C + cgp * p.cw + c] = sum;
    }
  }
}

// First pass of the dL/dw reduction: part [rows][cols] -> tmp [kSplit][cols], split s summing
// rows s, s + kSplit, ... in order (64 columns x 4 row subsets per work-group, the subsets added
// in a fixed order).  The second pass adds the kSplit rows of tmp.
constexpr int kSplit = 16;
__global__ void __launch_bounds__(256) reduce_split_kernel(const float* __restrict__ part, int rows,
                                                          int cols, float* __restrict__ tmp) {
  __shared__ float buf[4][64];
  const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl, sp = blockIdx.y;
  float a = 0.0f;
  if (c < cols)
    for (int r = sp + kSplit * rg; r < rows; r += 4 * kSplit) a += part[(size_t)r * cols + c];
  buf[rg][cl] = a;
  __syncthreads();
  if (rg == 0 && c < cols) tmp[(size_t)sp * cols + c] = (buf[0][cl] + buf[1][cl]) + (buf[2][cl] + buf[3][cl]);
}

template <int L, int NU>
hipError_t fwd_one(const LadderParams& p, hipStream_t st) {
  const int blocks = (p.n_tasks + kLadWaves - 1) / kLadWaves;
  hipLaunchKernelGGL((ladder_fwd_kernel<L, NU>), dim3(blocks), dim3(kLadWaves * 64), 0, st, p);
  return hipGetLastError();
}

template <int L, int NU, bool LB>
hipError_t bwd_one_lb(const LadderParams& p, bool want_dA, bool want_dw, hipStream_t st) {
  const size_t lds = (want_dw ? bwd_lds_floats<L, NU, true>() : bwd_lds_floats<L, NU, false>()) *
                     sizeof(float);
  auto go = [&](auto kern) -> hipError_t {
    {
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(kern, dim3(p.n_groups * p.blocks_per_group), dim3(kLadWaves * 64), lds, st, p);
    return hipGetLastError();
  };
  if (want_dA && want_dw) return go(ladder_bwd_kernel<L, NU, true, true, LB>);
  if (want_dA) return go(ladder_bwd_kernel<L, NU, true, false, LB>);
  return go(ladder_bwd_kernel<L, NU, false, true, LB>);
}

template <int L, int NU>
hipError_t bwd_one(const LadderParams& p, bool want_dA, bool want_dw, hipStream_t st) {
  if constexpr (NU > 2) {
    if (p.rungs != nullptr) return bwd_one_lb<L, NU, true>(p, want_dA, want_dw, st);
  }
  return bwd_one_lb<L, NU, false>(p, want_dA, want_dw, st);
}

template <int L, typename Fn>
hipError_t dispatch_nu(int nu, Fn&& fn) {
  switch (nu) {
    case 2: return fn(std::integral_constant<int, L>{}, std::integral_constant<int, 2>{});
    case 3: return fn(std::integral_constant<int, L>{}, std::integral_constant<int, 3>{});
    case 4: return fn(std::integral_constant<int, L>{}, std::integral_constant<int, 4>{});
    case 5: return fn(std::integral_constant<int, L>{}, std::integral_constant<int, 5>{});
    default: return hipErrorInvalidValue;
  }
}

template <typename Fn>
hipError_t dispatch(int lmax, int nu, Fn&& fn) {
  switch (lmax) {
    case 0: return dispatch_nu<0>(nu, fn);
    case 1: return dispatch_nu<1>(nu, fn);
    case 2: return dispatch_nu<2>(nu, fn);
    case 3: return dispatch_nu<3>(nu, fn);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_ladder_reduce(const float* part, int rows, int cols, float* tmp, float* out,
                                hipStream_t st) {
  hipLaunchKernelGGL(reduce_split_kernel, dim3((cols + 63) / 64, kSplit), dim3(256), 0, st, part,
                     rows, cols, tmp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_reduce_rows(tmp, kSplit, cols, out, st);
}

int ladder_reduce_split() { return kSplit; }

int ladder_num_paths(int lmax) {
  switch (lmax) {
    case 0: return Lad<0>::P;
    case 1: return Lad<1>::P;
    case 2: return Lad<2>::P;
    case 3: return Lad<3>::P;
    default: return -1;
  }
}

hipError_t launch_ladder_fwd(int lmax, int nu, const LadderParams& p, hipStream_t st) {
  if (p.n_tasks == 0) return hipSuccess;
  return dispatch(lmax, nu, [&](auto l, auto n) { return fwd_one<decltype(l)::value, decltype(n)::value>(p, st); });
}

hipError_t launch_ladder_bwd(int lmax, int nu, const LadderParams& p, bool want_dA, bool want_dw,
                             hipStream_t st) {
  if (p.n_tasks == 0 || !(want_dA || want_dw)) return hipSuccess;
  return dispatch(lmax, nu, [&](auto l, auto n) {
    return bwd_one<decltype(l)::value, decltype(n)::value>(p, want_dA, want_dw, st);
  });
}

}  // namespace equitp
