// Node-local product ladder, full form ("FlashCart: Fast Cartesian Tensor Products for
// Equivariant Interatomic Potentials", Fig. 3(b), dashed curves: linear maps mix paths and
// channels between the products; Fig. E1(b): the products' outputs over the retained coupling
// paths are compressed to d channels per retained rank).  Per step s = 2..nu, with d = C and every
// rank up to lmax kept:
//
//   T_p[n, m3, u] = sum_{m1, m2} C_p[m1, m2, m3] B_{s-1}[n, l1 m1, u] A[n, l2 m2, u]
//   B_s[n, l3 m3, v] = sum_{p -> l3} sum_u T_p[n, m3, u] W[s-2][p][u][v]
//   out = B_2 + ... + B_nu
//
// Two kinds of kernel per step:
//  * the channelwise products (one lane per (node, channel), CG nonzeros unrolled with the values
//    as literals) write every path output T_p to HBM, T_p as [N (2 l3 + 1)][C] row-major;
//  * the mixing is a dense fp32 contraction per l3: rows (n, m3), K = (p -> l3, u), columns v,
//    on the matrix cores (v_mfma_f32_16x16x4f32).  The same GEMM kernel, in three modes, also
//    gives the backward's dT = Gs W^T (per path) and dW = T^T Gs (split over rows, partial maps
//    summed per path in a fixed order: reproducible, no atomics).
// The backward's products take dT and give dL/dB_{s-1} (which plus G is the next step's output
// gradient) and dL/dA.
//
// GEMM tiling: 256 threads as 2 x 2 waves over a TM x C tile (TM = 128 rows, or C for dW), K in
// chunks of 32 (forward) or 16 (backward modes, C >= 64) staged through LDS in two buffers (one
// barrier per chunk; the next chunk's global loads are issued before the current chunk's MFMAs
// and written to the other buffer after them).  An operand whose source rows run along K is
// staged row by row with a stride of KC + 4 floats; one whose source rows run along M (or N) is
// staged k-major with a stride of (tile width + 16) floats.  Either way each group of 16 lanes of
// an operand read touches 64 different banks.
// Measured alternative: loading the operands from global memory straight into registers (no LDS,
// no barriers) ran 4-6 % slower.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "full_ladder.h"

namespace equitp {
namespace {

template <int L>
struct FL {
  using PS = PathSet<L, L, L>;
  static constexpr int P = PS::N;
  static constexpr int F = (L + 1) * (L + 1);
  // first row block of path j within the per-node path outputs (sum of 2 l3 + 1 before it)
  static constexpr int toff(int j) {
    int o = 0;
    for (int i = 0; i < j; ++i) o += 2 * cg::kPaths[PS::id(i)].l3 + 1;
    return o;
  }
  static constexpr int D = toff(P);
};

// ------------------------------------------------------------------ channelwise products
template <int L>
__device__ __forceinline__ void load_node(const float* __restrict__ src, int n, int u, int C,
                                          float (&v)[FL<L>::F]) {
  const float* p = src + (size_t)n * FL<L>::F * C + u;
#pragma unroll
  for (int k = 0; k < FL<L>::F; ++k) v[k] = p[(size_t)k * C];
}

template <int L>
__global__ void __launch_bounds__(256) full_tp_kernel(int n_nodes, int C, const float* __restrict__ Bp,
                                                      const float* __restrict__ A,
                                                      float* __restrict__ T) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)n_nodes * C) return;
  const int n = (int)(t / C), u = (int)(t % C);
  float a[FL<L>::F], b[FL<L>::F];
  load_node<L>(A, n, u, C, a);
  load_node<L>(Bp, n, u, C, b);
  const size_t NC = (size_t)n_nodes * C;
  static_for<FL<L>::P>([&](auto j) {
    constexpr cg::PathDesc pd = cg::kPaths[FL<L>::PS::id(j)];
    constexpr int d3 = 2 * pd.l3 + 1;
    float tt[d3];
#pragma unroll
    for (int m = 0; m < d3; ++m) tt[m] = 0.0f;
    static_for<pd.nnz>([&](auto k) {
      constexpr cg::Ent e = cg::kEnt[pd.off + k];
      constexpr float v = cg::kVal[pd.off + k];
      tt[e.m3] = __builtin_fmaf(v * a[pd.l2 * pd.l2 + e.m2], b[pd.l1 * pd.l1 + e.m1], tt[e.m3]);
    });
    float* dst = T + (size_t)FL<L>::toff(j) * NC + (size_t)n * d3 * C + u;
#pragma unroll
    for (int m = 0; m < d3; ++m) dst[(size_t)m * C] = tt[m];
  });
}

template <int L>
__global__ void __launch_bounds__(256) full_tp_bwd_kernel(int n_nodes, int C, const float* __restrict__ Bp,
                                                          const float* __restrict__ A,
                                                          const float* __restrict__ dT,
                                                          const float* __restrict__ G,
                                                          float* __restrict__ Gs_next,
                                                          float* __restrict__ dA, int accumulate,
                                                          int add_dB) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)n_nodes * C) return;
  const int n = (int)(t / C), u = (int)(t % C);
  constexpr int F = FL<L>::F;
  float a[F], b[F], da[F], db[F];
  load_node<L>(A, n, u, C, a);
  load_node<L>(Bp, n, u, C, b);
#pragma unroll
  for (int k = 0; k < F; ++k) da[k] = db[k] = 0.0f;
  const size_t NC = (size_t)n_nodes * C;
  static_for<FL<L>::P>([&](auto j) {
    constexpr cg::PathDesc pd = cg::kPaths[FL<L>::PS::id(j)];
    constexpr int d3 = 2 * pd.l3 + 1;
    constexpr int o1 = pd.l1 * pd.l1, o2 = pd.l2 * pd.l2;
    // one path's dT at a time: without the fence the compiler issues the loads of every path
    // up front and needs a register per value (occupancy 1 at lmax 3)
    asm volatile("" ::: "memory");
    const float* src = dT + (size_t)FL<L>::toff(j) * NC + (size_t)n * d3 * C + u;
    float g[d3];
#pragma unroll
    for (int m = 0; m < d3; ++m) g[m] = src[(size_t)m * C];
    static_for<pd.nnz>([&](auto k) {
      constexpr cg::Ent e = cg::kEnt[pd.off + k];
      constexpr float v = cg::kVal[pd.off + k];
      const float vg = v * g[e.m3];
      db[o1 + e.m1] = __builtin_fmaf(vg, a[o2 + e.m2], db[o1 + e.m1]);
      da[o2 + e.m2] = __builtin_fmaf(vg, b[o1 + e.m1], da[o2 + e.m2]);
    });
#pragma unroll
    for (int k = 0; k < F; ++k) asm volatile("" : "+v"(da[k]), "+v"(db[k]));
  });
  const size_t base = (size_t)n * F * C + u;
  if (Gs_next != nullptr) {
#pragma unroll
    for (int k = 0; k < F; ++k) Gs_next[base + (size_t)k * C] = G[base + (size_t)k * C] + db[k];
  }
  if (dA != nullptr) {
#pragma unroll
    for (int k = 0; k < F; ++k) {
      float v = da[k] + (add_dB ? db[k] : 0.0f);
      if (accumulate) v += dA[base + (size_t)k * C];
      dA[base + (size_t)k * C] = v;
    }
  }
}

// ------------------------------------------------------------------ mixing GEMM
enum { kMixFwd = 0, kMixDT = 1, kMixDW = 2 };
constexpr int kKC = 32;            // dW row ranges are multiples of this (of either chunk depth)
constexpr int kRowTile = 128;      // rows per work-group (forward, dT)
// dW work-groups: rows of K per work-group sized for about kDWBlocks work-groups in all — one
// round at four work-groups per CU on 256 CUs (416 rows at the 4096-node, lmax-3 size: 160 us,
// against 179 us at 512 rows and 792 work-groups) — a multiple of 32, between 256 and 4096 rows
constexpr int kDWBlocks = 1024;
constexpr int kMaxGroups = 24;

struct MixGroup {
  int l3;
  int path;         // index in the ladder's path list (dT, dW); unused in the forward
  int toff;         // first row block of that path within the per-node path outputs
  int first_block;
};

struct MixArgs {
  int n_nodes, F, n_groups, n_blocks;
  int dw_rows;      // dW: rows of K per work-group
  int ranked;       // dT, dW: one group per l3, blocks ordered (row range, path into the l3)
  int n_paths;
  int red_first[kMaxGroups], red_stride[kMaxGroups], red_count[kMaxGroups];  // dW: path's blocks
  const float* W;   // one step's maps [P][C][C]
  const float* T;   // path outputs (forward, dW)
  float* dT;        // dT output
  const float* Gs;  // gradient of the step's output [N][F][C] (dT, dW)
  float* out;       // forward: running sum (or null)
  float* bnext;     // forward: B_s (or null)
  float* part;      // dW: partial maps [n_blocks][C][C]
  int accumulate;
  int n_seg[4];     // forward: paths into each l3 ...
  int seg_path[4][8];
  int seg_toff[4][8];
  MixGroup g[kMaxGroups];
};

// K consecutive floats in one access (K = 1, 2 or 4; LDS or global).
template <int K>
__device__ __forceinline__ void ld_vec(const float* p, float (&v)[K]) {
  if constexpr (K == 4) {
    const f4 x = *reinterpret_cast<const f4*>(p);
    v[0] = x[0], v[1] = x[1], v[2] = x[2], v[3] = x[3];
  } else if constexpr (K == 2) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 x = *reinterpret_cast<const f2*>(p);
    v[0] = x[0], v[1] = x[1];
  } else {
    v[0] = p[0];
  }
}

template <int K>
__device__ __forceinline__ void st_vec(float* p, const float (&v)[K]) {
  if constexpr (K == 4) {
    *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
  } else if constexpr (K == 2) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<f2*>(p) = f2{v[0], v[1]};
  } else {
    p[0] = v[0];
  }
}

// The K slots of an MFMA step are a free choice as long as both operands agree: step s of a
// chunk of KC takes k = (KC / 4) q + s from lane group q, so an operand staged with K contiguous
// gives a lane its values in 16-byte reads.  Tiles of a k-major operand interleave their rows (or
// columns): tile t, index i -> base + T i + t (T tiles per wave), so one read at a k gives a lane
// all its tiles, and the outputs of a lane's column tiles are contiguous.
template <int C, int MODE>
__global__ void __launch_bounds__(256) mix_kernel(MixArgs a) {
  // K chunk: 32 in the forward (measured faster there), 16 in the backward modes (half the LDS,
  // more waves per CU: measured faster there); 256 threads stage at least one f4 each
  constexpr int KC = MODE == kMixFwd || C < 64 ? 32 : 16;
  constexpr int KQ = KC / 4;                 // K slots per lane group
  constexpr int TM = MODE == kMixDW ? C : kRowTile;
  constexpr int TN = C;
  constexpr bool A_KM = MODE == kMixDW;      // A staged k-major (its source rows run along K)
  constexpr bool B_KM = MODE != kMixDT;
  constexpr int SA = A_KM ? TM + 16 : KC + 4;
  constexpr int SB = B_KM ? TN + 16 : KC + 4;
  constexpr int LA = A_KM ? KC * SA : TM * SA;
  constexpr int LB = B_KM ? KC * SB : TN * SB;
  constexpr int MT = TM / 32, NT = TN / 32;  // 16 x 16 tiles per wave (2 x 2 waves)
  constexpr int NA = TM * KC / 4 / 256, NB = TN * KC / 4 / 256;
  static_assert(NA >= 1 && NB >= 1, "tile too small for 256 threads");
  __shared__ float as[2][LA];                // two chunks: one read while the next is written
  __shared__ float bs[2][LB];

  const int tid = threadIdx.x;
  // Work-groups go round-robin over the 8 XCDs (block b on XCD b % 8).  In the ranked order the
  // blocks of one row range, one per path into the l3, read the same rows of the output gradient:
  // giving each XCD a contiguous run of logical blocks keeps those reads in one L2.
  int bid = (int)blockIdx.x;
  if (a.ranked) {
    const int x = bid % 8;
    int start = 0;
    for (int y = 0; y < x; ++y) start += (a.n_blocks - y + 7) / 8;
    bid = start + bid / 8;
  }
  int gi = 0;
  while (gi + 1 < a.n_groups && bid >= a.g[gi + 1].first_block) ++gi;
  const MixGroup grp = a.g[gi];
  const int l3 = grp.l3, d = 2 * l3 + 1;
  int blk = bid - grp.first_block, path = grp.path, toff = grp.toff;
  if (a.ranked) {
    const int ns = a.n_seg[l3], pj = blk % ns;
    blk /= ns;
    path = a.seg_path[l3][pj];
    toff = a.seg_toff[l3][pj];
  }
  const int M = a.n_nodes * d;
  const size_t NC = (size_t)a.n_nodes * C;
  auto feat_row = [&](int r) -> size_t {
    return ((size_t)(r / d) * a.F + l3 * l3 + r % d) * C;
  };

  int nk, row0 = 0, rend = 0;
  if constexpr (MODE == kMixFwd) {
    row0 = blk * kRowTile;
    nk = a.n_seg[l3] * (C / KC);
  } else if constexpr (MODE == kMixDT) {
    row0 = blk * kRowTile;
    nk = C / KC;
  } else {
    row0 = blk * a.dw_rows;
    rend = min(row0 + a.dw_rows, M);
    nk = (rend - row0 + KC - 1) / KC;
  }

  // Node-tensor rows without a division per load: the dT mode's A rows are fixed per thread; the
  // dW mode's B rows advance by KC per chunk (gload runs for kc = 0, 1, 2, ... in order), so each
  // thread keeps their (node, m3).  Rows past the range read the last valid row (then zeroed).
  size_t arow_off[NA];
  int bn[NB], bm[NB];
  size_t b_last = 0;
  if constexpr (MODE == kMixDT) {
#pragma unroll
    for (int j = 0; j < NA; ++j)
      arow_off[j] = feat_row(min(row0 + (tid + 256 * j) / (KC / 4), M - 1));
  }
  if constexpr (MODE == kMixDW) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = row0 + (tid + 256 * j) / (TN / 4);
      bn[j] = r / d;
      bm[j] = r % d;
    }
    b_last = feat_row(rend - 1);
  }
  const int adv_n = KC / d, adv_m = KC % d;

  f4 ra[NA], rb[NB];
  auto gload = [&](int kc) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + 256 * j;
      const float* src;
      bool ok;
      if constexpr (MODE == kMixFwd) {
        const int row = i / (KC / 4), c4 = i % (KC / 4);
        const int seg = kc / (C / KC), u0 = (kc % (C / KC)) * KC;
        const int r = row0 + row;
        ok = r < M;
        src = a.T + (size_t)a.seg_toff[l3][seg] * NC + (size_t)min(r, M - 1) * C + u0 + 4 * c4;
      } else if constexpr (MODE == kMixDT) {
        const int row = i / (KC / 4), c4 = i % (KC / 4);
        ok = row0 + row < M;
        src = a.Gs + arow_off[j] + kc * KC + 4 * c4;
      } else {
        const int k = i / (TM / 4), c4 = i % (TM / 4);
        const int r = row0 + kc * KC + k;
        ok = r < rend;
        src = a.T + (size_t)toff * NC + (size_t)min(r, rend - 1) * C + 4 * c4;
      }
      const f4 v = ld4(src);
      ra[j] = ok ? v : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = tid + 256 * j;
      const float* src;
      bool ok = true;
      if constexpr (MODE == kMixFwd) {
        const int k = i / (TN / 4), c4 = i % (TN / 4);
        const int seg = kc / (C / KC), u0 = (kc % (C / KC)) * KC;
        src = a.W + ((size_t)a.seg_path[l3][seg] * C + u0 + k) * C + 4 * c4;
      } else if constexpr (MODE == kMixDT) {
        const int col = i / (KC / 4), c4 = i % (KC / 4);
        src = a.W + ((size_t)path * C + col) * C + kc * KC + 4 * c4;
      } else {
        const int k = i / (TN / 4), c4 = i % (TN / 4);
        ok = row0 + kc * KC + k < rend;
        const size_t off = ((size_t)bn[j] * a.F + l3 * l3 + bm[j]) * C;
        src = a.Gs + (ok ? off : b_last) + 4 * c4;
        bm[j] += adv_m;
        bn[j] += adv_n;
        if (bm[j] >= d) {
          bm[j] -= d;
          ++bn[j];
        }
      }
      const f4 v = ld4(src);
      rb[j] = ok ? v : f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + 256 * j;
      if constexpr (A_KM) st4(&as[buf][(i / (TM / 4)) * SA + 4 * (i % (TM / 4))], ra[j]);
      else st4(&as[buf][(i / (KC / 4)) * SA + 4 * (i % (KC / 4))], ra[j]);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = tid + 256 * j;
      if constexpr (B_KM) st4(&bs[buf][(i / (TN / 4)) * SB + 4 * (i % (TN / 4))], rb[j]);
      else st4(&bs[buf][(i / (KC / 4)) * SB + 4 * (i % (KC / 4))], rb[j]);
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int es = lane & 15, q = lane >> 4;
  const int rw = (wave >> 1) * (TM / 2), cw = (wave & 1) * (TN / 2);
  f4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const float* A_ = as[buf];
    const float* B_ = bs[buf];
#pragma unroll
    for (int h = 0; h < KQ / 4; ++h) {
      float av[MT][4], bv[NT][4];            // [tile][k slot 4 h + ss]
      static_assert(KQ % 4 == 0, "slots come in fours");
      if constexpr (A_KM) {
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
          float x[MT];
          ld_vec<MT>(&A_[(KQ * q + 4 * h + ss) * SA + rw + MT * es], x);
#pragma unroll
          for (int t = 0; t < MT; ++t) av[t][ss] = x[t];
        }
      } else {
#pragma unroll
        for (int t = 0; t < MT; ++t) ld_vec<4>(&A_[(rw + 16 * t + es) * SA + KQ * q + 4 * h], av[t]);
      }
      if constexpr (B_KM) {
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
          float x[NT];
          ld_vec<NT>(&B_[(KQ * q + 4 * h + ss) * SB + cw + NT * es], x);
#pragma unroll
          for (int t = 0; t < NT; ++t) bv[t][ss] = x[t];
        }
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) ld_vec<4>(&B_[(cw + 16 * t + es) * SB + KQ * q + 4 * h], bv[t]);
      }
#pragma unroll
      for (int ss = 0; ss < 4; ++ss)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = mfma_16x16x4(av[mt][ss], bv[nt][ss], acc[mt][nt]);
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int cur = kc & 1;
    if (kc + 1 < nk) gload(kc + 1);
    compute(cur);
    // the other buffer was last read in the previous chunk, which every wave finished before
    // the barrier that ended it
    if (kc + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Lane holds D[i = 4 q + r][j = es] of each tile pair (mt, nt).  Row of A index i of tile mt:
  // rw + 16 mt + i (row-staged A) or rw + MT i + mt (k-major A); column of B index j of tile nt:
  // cw + NT j + nt (k-major B: a lane's NT columns are contiguous) or cw + 16 nt + j.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * q + r;
      const int row = A_KM ? rw + MT * i + mt : rw + 16 * mt + i;
      float v[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) v[nt] = acc[mt][nt][r];
      if constexpr (MODE == kMixDW) {
        st_vec<NT>(a.part + (size_t)bid * C * C + (size_t)row * C + cw + NT * es, v);
      } else {
        const int rr = row0 + row;
        if (rr >= M) continue;
        if constexpr (MODE == kMixDT) {
          float* dst = a.dT + (size_t)toff * NC + (size_t)rr * C + cw + es;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) dst[16 * nt] = v[nt];
        } else {
          const size_t o = feat_row(rr) + cw + NT * es;
          if (a.bnext) st_vec<NT>(a.bnext + o, v);
          if (a.out) {
            if (a.accumulate) {
              float old[NT];
              ld_vec<NT>(a.out + o, old);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) v[nt] += old[nt];
            }
            st_vec<NT>(a.out + o, v);
          }
        }
      }
    }
}

// dW[p][e] = sum over path p's work-groups (row ranges in order) of part[b][e]; four consecutive e
// per thread (16-byte loads), the loop unrolled so that loads run ahead of the in-order adds.
template <int C>
__global__ void __launch_bounds__(256) dw_reduce_kernel(MixArgs a, float* __restrict__ dW) {
  const int e = 4 * (blockIdx.x * 256 + threadIdx.x);
  const int j = blockIdx.y;   // path
  if (e >= C * C) return;
  const int b0 = a.red_first[j], bs = a.red_stride[j], nb = a.red_count[j];
  f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int r = 0; r < nb; ++r) s += ld4(a.part + (size_t)(b0 + r * bs) * C * C + e);
  st4(dW + (size_t)j * C * C + e, s);
}

// ------------------------------------------------------------------ host side
struct PathInfo {
  int n;
  int l3[kMaxGroups], toff[kMaxGroups];
};

template <int L>
PathInfo path_info_l() {
  PathInfo pi{};
  pi.n = FL<L>::P;
  int o = 0;
  for (int j = 0; j < FL<L>::P; ++j) {
    pi.l3[j] = cg::kPaths[FL<L>::PS::id(j)].l3;
    pi.toff[j] = o;
    o += 2 * pi.l3[j] + 1;
  }
  return pi;
}

PathInfo path_info(int lmax) {
  switch (lmax) {
    case 0: return path_info_l<0>();
    case 1: return path_info_l<1>();
    case 2: return path_info_l<2>();
    default: return path_info_l<3>();
  }
}

template <typename Fn>
hipError_t with_lmax(int lmax, Fn&& fn) {
  switch (lmax) {
    case 0: return fn(std::integral_constant<int, 0>{});
    case 1: return fn(std::integral_constant<int, 1>{});
    case 2: return fn(std::integral_constant<int, 2>{});
    case 3: return fn(std::integral_constant<int, 3>{});
    default: return hipErrorInvalidValue;
  }
}

template <typename Fn>
hipError_t with_channels(int C, Fn&& fn) {
  switch (C) {
    case 32: return fn(std::integral_constant<int, 32>{});
    case 64: return fn(std::integral_constant<int, 64>{});
    case 128: return fn(std::integral_constant<int, 128>{});
    default: return hipErrorInvalidValue;
  }
}

int full_ladder_dsum_l(int lmax) {
  const PathInfo pi = path_info(lmax);
  int d = 0;
  for (int j = 0; j < pi.n; ++j) d += 2 * pi.l3[j] + 1;
  return d;
}

unsigned grid_for(long long items) { return (unsigned)((items + 255) / 256); }

MixArgs base_args(int lmax, int n_nodes) {
  MixArgs a{};
  a.n_nodes = n_nodes;
  a.F = (lmax + 1) * (lmax + 1);
  return a;
}

int dw_rows(int lmax, int n_nodes) {
  const long long rows = (long long)n_nodes * full_ladder_dsum_l(lmax);
  long long r = (rows + kDWBlocks - 1) / kDWBlocks;
  r = (r + kKC - 1) / kKC * kKC;
  return (int)std::min<long long>(4096, std::max<long long>(256, r));
}

// dT (row tiles of 128) and dW (row ranges of dw_rows): one group per l3, its blocks ordered
// (row range, path into the l3) — the "ranked" order the kernel maps onto the XCDs
MixArgs rank_groups(int lmax, int n_nodes, int rows_per_block) {
  const PathInfo pi = path_info(lmax);
  MixArgs a = base_args(lmax, n_nodes);
  for (int j = 0; j < pi.n; ++j) {
    const int l3 = pi.l3[j];
    a.seg_path[l3][a.n_seg[l3]] = j;
    a.seg_toff[l3][a.n_seg[l3]] = pi.toff[j];
    ++a.n_seg[l3];
  }
  int blocks = 0;
  for (int l3 = 0; l3 <= lmax; ++l3) {
    const long long M = (long long)n_nodes * (2 * l3 + 1);
    const int ranges = (int)((M + rows_per_block - 1) / rows_per_block);
    a.g[l3] = MixGroup{l3, -1, 0, blocks};
    for (int pj = 0; pj < a.n_seg[l3]; ++pj) {
      const int j = a.seg_path[l3][pj];
      a.red_first[j] = blocks + pj;
      a.red_stride[j] = a.n_seg[l3];
      a.red_count[j] = ranges;
    }
    blocks += ranges * a.n_seg[l3];
  }
  a.n_groups = lmax + 1;
  a.n_blocks = blocks;
  a.n_paths = pi.n;
  a.dw_rows = rows_per_block;
  a.ranked = 1;
  return a;
}

}  // namespace

int full_ladder_dsum(int lmax) { return full_ladder_dsum_l(lmax); }

int full_ladder_dw_blocks(int lmax, int n_nodes, int C) {
  (void)C;
  return rank_groups(lmax, n_nodes, dw_rows(lmax, n_nodes)).n_blocks;
}

bool full_ladder_channels_ok(int C) { return C == 32 || C == 64 || C == 128; }

hipError_t launch_full_tp(int lmax, int n_nodes, int C, const float* Bp, const float* A, float* T,
                          hipStream_t st) {
  if (n_nodes == 0) return hipSuccess;
  return with_lmax(lmax, [&](auto l) {
    hipLaunchKernelGGL(full_tp_kernel<decltype(l)::value>, dim3(grid_for((long long)n_nodes * C)),
                       dim3(256), 0, st, n_nodes, C, Bp, A, T);
    return hipGetLastError();
  });
}

hipError_t launch_full_tp_bwd(int lmax, int n_nodes, int C, const float* Bp, const float* A,
                              const float* dT, const float* G, float* Gs_next, float* dA,
                              bool accumulate, bool add_dB, hipStream_t st) {
  if (n_nodes == 0) return hipSuccess;
  return with_lmax(lmax, [&](auto l) {
    hipLaunchKernelGGL(full_tp_bwd_kernel<decltype(l)::value>,
                       dim3(grid_for((long long)n_nodes * C)), dim3(256), 0, st, n_nodes, C, Bp,
                       A, dT, G, Gs_next, dA, accumulate ? 1 : 0, add_dB ? 1 : 0);
    return hipGetLastError();
  });
}

hipError_t launch_mix_fwd(int lmax, int n_nodes, int C, const float* T, const float* W, float* out,
                          bool accumulate, float* bnext, hipStream_t st) {
  if (n_nodes == 0) return hipSuccess;
  const PathInfo pi = path_info(lmax);
  MixArgs a = base_args(lmax, n_nodes);
  for (int j = 0; j < pi.n; ++j) {
    const int l3 = pi.l3[j];
    a.seg_path[l3][a.n_seg[l3]] = j;
    a.seg_toff[l3][a.n_seg[l3]] = pi.toff[j];
    ++a.n_seg[l3];
  }
  int blocks = 0;
  for (int l3 = 0; l3 <= lmax; ++l3) {
    a.g[l3] = MixGroup{l3, -1, 0, blocks};
    blocks += (int)(((long long)n_nodes * (2 * l3 + 1) + kRowTile - 1) / kRowTile);
  }
  a.n_groups = lmax + 1;
  a.n_blocks = blocks;
  a.W = W;
  a.T = T;
  a.out = out;
  a.bnext = bnext;
  a.accumulate = accumulate ? 1 : 0;
  return with_channels(C, [&](auto c) {
    hipLaunchKernelGGL((mix_kernel<decltype(c)::value, kMixFwd>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
  });
}

hipError_t launch_mix_dt(int lmax, int n_nodes, int C, const float* Gs, const float* W, float* dT,
                         hipStream_t st) {
  if (n_nodes == 0) return hipSuccess;
  MixArgs a = rank_groups(lmax, n_nodes, kRowTile);
  a.W = W;
  a.Gs = Gs;
  a.dT = dT;
  return with_channels(C, [&](auto c) {
    hipLaunchKernelGGL((mix_kernel<decltype(c)::value, kMixDT>), dim3(a.n_blocks), dim3(256), 0, st, a);
    return hipGetLastError();
  });
}

hipError_t launch_mix_dw(int lmax, int n_nodes, int C, const float* T, const float* Gs,
                         float* part, float* dW, hipStream_t st) {
  if (n_nodes == 0) return hipSuccess;
  MixArgs a = rank_groups(lmax, n_nodes, dw_rows(lmax, n_nodes));
  a.T = T;
  a.Gs = Gs;
  a.part = part;
  return with_channels(C, [&](auto c) {
    constexpr int CC = decltype(c)::value;
    hipLaunchKernelGGL((mix_kernel<CC, kMixDW>), dim3(a.n_blocks), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dw_reduce_kernel<CC>, dim3((CC * CC / 4 + 255) / 256, a.n_paths), dim3(256),
                       0, st, a, dW);
    return hipGetLastError();
  });
}

}  // namespace equitp
