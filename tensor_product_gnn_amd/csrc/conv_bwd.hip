// Backward of the fused edge convolution (gfx950): the exact vector-Jacobian product for an
// upstream gradient G = dL/dout, giving dL/dvec (the edge vectors: forces follow from them),
// dL/dW1 and dL/dW2 (the radial-MLP weights); dL/dx is the transpose segment kernel in
// conv_seg.hip.  For one edge e = (s -> d), path p = (l1, l2, l3), channel c:
//   t[m3]     = sum_{m1,m2} C[m1,m2,m3] x[s,l1,m1,c] Y_l2[m2]
//   dL/dw     = sum_m3 G[d,l3,m3,c] t[m3]
//   dL/dY[m2] += sum_{m1,m3,c} C[m1,m2,m3] x[s,l1,m1,c] w[p,c] G[d,l3,m3,c]
//   dL/dh     = dL/dw W2^T ,  dL/dW2 = sum_e h^T dL/dw ,  dL/dpre = dL/dh * SiLU'(pre)
//   dL/dW1    = sum_e e^T dL/dpre ,  dL/de = dL/dpre W1^T
//   dL/dvec   = (sum_n dL/de_n de_n/dr) u + (I - u u^T) grad_u(Y . dL/dY) / r
//
// The paths are split into at most kBwdGroups groups and the backward runs as one kernel launch
// per group (in stream order), so each launch holds the code of one group only and stays inside
// the instruction cache.  A work-group of kBwdWaves = 8 waves (two per SIMD, so that one wave's
// latencies are covered by the other's work) owns one 16-channel slice (blockIdx % n_slices: with
// 8 slices every XCD works on one slice, so its L2 keeps that slice of x and G) and a contiguous
// range of edges, cut into 16-edge tiles that the waves take in turn.  Per tile each wave, lane =
// (edge es, channel quad q):
//   * hidden layer on MFMA (A = W1^T in registers, B = radial basis): h and SiLU'(pre) to LDS;
//   * per path of the group: w = MFMA(W2 slice from LDS, h); t, dL/dw, dL/dY on VALU; dL/dh^T
//     += MFMA(W2, dL/dw^T) contracting the slice's channels; dL/dw to LDS;
//   * dL/dW2 += MFMA(h^T, dL/dw) contracting the tile's edges.  Its accumulators (16 registers
//     per path and lane) would not fit beside everything else at two waves per SIMD, so they are
//     spread over the work-group: each wave owns a few (path, 16-row block) pairs and, once per
//     round of tiles (between two barriers), accumulates its blocks over the tiles of all waves;
//   * dL/dpre = dL/dh * SiLU'(pre); dL/de^T = MFMA(W1, dL/dpre^T); dL/dW1 += MFMA(e^T, dL/dpre)
//     (through the wave's LDS);
//   * dL/dvec of its paths and slice, from dL/dY and dL/de (dL/dvec is linear in both, so the
//     partial of each (group, slice) is exact), added to the 3-vector that the previous group's
//     launch left for this edge and slice.
// Each work-group writes one dL/dW2 partial (each launch fills its group's columns) and one dL/dW1
// partial (the waves' accumulators summed in LDS in wave order; the launch of group 0 writes it,
// the later launches add to it).  A small kernel sums the slice partials of dL/dvec; fixed-order
// row sums finish dL/dW1 and dL/dW2.  No atomics anywhere: results are bitwise reproducible run
// to run.
#include "common.h"
#include "params.h"

namespace equitp {
namespace {

// Paths of a configuration split into groups, one launch each (at most kBwdGroups).  For the 23
// paths of l <= 3 the split (6/6/6/5 paths) was chosen by a small offline search to minimise the
// largest number of x and G components a group gathers (18 of 32), which sets its register
// footprint.  The 11 paths of l <= 2 form two contiguous groups of 6 and 5 (13 and 17 gathered
// components, within what the l <= 3 groups hold), and l <= 1 one group: every launch repeats the
// work that does not depend on the paths (geometry, SH, radial basis, hidden layer, dL/de,
// dL/dW1, the dL/dvec epilogue), so fewer groups are cheaper wherever the registers allow.
constexpr int kGroupL3[23] = {2, 3, 1, 3, 0, 2, 1, 0, 2, 1, 0, 0, 2, 2, 0, 0, 2, 3, 1, 3, 3, 1, 1};

template <int NP>
struct Groups {
  static constexpr int n() { return NP == 23 ? 4 : NP == 11 ? 2 : 1; }
  static_assert(n() <= kBwdGroups, "more groups than launches");
  static constexpr int of(int j) { return NP == 23 ? kGroupL3[j] : (j * n()) / NP; }
  static constexpr int count(int g) {
    int n = 0;
    for (int j = 0; j < NP; ++j) n += of(j) == g ? 1 : 0;
    return n;
  }
  // position of path j inside its group
  static constexpr int rank(int j) {
    int n = 0;
    for (int i = 0; i < j; ++i) n += of(i) == of(j) ? 1 : 0;
    return n;
  }
  // path of rank a in group g
  static constexpr int path(int g, int a) {
    for (int j = 0; j < NP; ++j)
      if (of(j) == g && rank(j) == a) return j;
    return -1;
  }
};

// Whether any path of group G (in configuration PS) reads input component block l1 / output l3.
template <typename PS, int G>
constexpr bool group_reads_l1(int l) {
  for (int j = 0; j < PS::N; ++j)
    if (Groups<PS::N>::of(j) == G && cg::kPaths[PS::id(j)].l1 == l) return true;
  return false;
}
template <typename PS, int G>
constexpr bool group_reads_l3(int l) {
  for (int j = 0; j < PS::N; ++j)
    if (Groups<PS::N>::of(j) == G && cg::kPaths[PS::id(j)].l3 == l) return true;
  return false;
}

// Wave-private 16-row tiles in LDS are read both along rows (a lane's own edge, four
// consecutive columns, one ds_read_b128) and along columns (lane (es, q) reads row 4 st + q,
// column es).  An XOR swizzle of the 16-float column block by (row & 3) and of the 4-float group
// by ((row >> 2) & 3) makes both patterns free of bank conflicts on the 64 banks of gfx950 LDS.
__device__ __forceinline__ int swz64(int row, int col) {
  return row * 64 + (col ^ (16 * (row & 3)) ^ (4 * ((row >> 2) & 3)));
}
__device__ __forceinline__ int swz16(int row, int col) {
  return row * 16 + (col ^ (4 * ((row >> 2) & 3)));
}

// LDS of one launch: the group's W2 slice column-major, [rank][channel][CS] with CS = H + 4
// (four consecutive k per ds_read_b128 for the A operand of w; single floats along a column,
// conflict free, for the A operand of dL/dh); the A operands of dL/de = dL/dpre W1^T, [H/4][64]
// (step st, lane: W1[es][16 (st / 4) + 4 q + st % 4], zero for es >= NR), staged once so that the
// tile loop reads them from LDS instead of waiting on one global load per MFMA; then per wave:
// the h tile (later dL/dpre) and the SiLU'(pre) tile, [16][64] swz64 each; the radial basis and
// its derivative, [16][16] each; the dL/dw tiles of the group's paths, [NG][16][16] swz16.
// With bf16 operands (BF) the slice is kept twice as packed bf16 (u2 = four values): column-major
// [rank][channel][H/4 + 1] u2 (four consecutive k: the A operand of w) and row-major
// [rank][k][5] u2 (four consecutive channels: the A operand of dL/dh).
template <int H>
struct BwdLds {
  static constexpr int CS = H + 4;
  static constexpr int ENP = 16;
  static constexpr int CSB = H / 4 + 1;  // u2 per column (BF)
  static constexpr int RSB = 5;          // u2 per row (BF)
  static constexpr int slice_floats(int ng, bool bf) {
    return bf ? ng * (16 * CSB + H * RSB) * 2 : ng * 16 * CS;
  }
  static constexpr int wave_floats(int ng) { return 2 * 16 * 64 + 2 * 16 * ENP + ng * 256; }
  static constexpr int w1_floats() { return 16 * H; }
  static constexpr size_t bytes(int ng, bool bf) {
    return (size_t)(slice_floats(ng, bf) + w1_floats() + kBwdWaves * wave_floats(ng)) * sizeof(float);
  }
};

template <int LIN, int LSH, int LOUT, int H, int NR, int G, bool WW, bool BF, bool MASK = false>
__global__ void __launch_bounds__(kBwdWaves * 64, 1) bwd_kernel(BwdParams p) {
  // WW (compile time) switches the weight-gradient accumulation on: a runtime condition on
  // accumulators makes the compiler copy them between register files every tile.  BF: the three
  // W2 contractions (w, dL/dh, dL/dW2) take bf16 operands (rounded to nearest even) with fp32
  // accumulation on v_mfma_f32_16x16x16_bf16.  MASK: per-edge path subsets (p.path_mask): a path
  // no edge of the tile needs is skipped for the tile (its dL/dw tile is written as zeros for
  // the dL/dW2 pass); for an edge without the path, w and dL/dw are zero.
  using PS = PathSet<LIN, LSH, LOUT>;
  using GR = Groups<PS::N>;
  using LD = BwdLds<H>;
  constexpr int NP = PS::N;
  constexpr int FIN = (LIN + 1) * (LIN + 1);
  constexpr int FSH = (LSH + 1) * (LSH + 1);
  constexpr int FOUT = (LOUT + 1) * (LOUT + 1);
  constexpr int NSTEP = H / 4;
  constexpr int NJ = H / 16;
  constexpr int NG = GR::count(G);
  constexpr int CS = LD::CS;
  constexpr int ENP = LD::ENP;
  constexpr int WF = LD::wave_floats(NG);
  // dL/dW2 blocks (path rank a, rows 16 mt .. 16 mt + 15) owned by each wave: block b = a NJ + mt
  // belongs to wave b % kBwdWaves
  constexpr int NBLK = NG * NJ;
  constexpr int NOWN = (NBLK + kBwdWaves - 1) / kBwdWaves;
  static_assert(NR % 4 == 0 && NR <= 16 && H % 16 == 0 && H <= 64, "unsupported shape");

  extern __shared__ float smem[];
  constexpr int CSB = LD::CSB, RSB = LD::RSB;
  float* w2c = smem;                   // [NG][16][CS], or (BF) the two packed bf16 copies
  u2* w2cb = reinterpret_cast<u2*>(smem);           // BF: [NG][16][CSB]
  u2* w2rb = w2cb + NG * 16 * CSB;                  // BF: [NG][H][RSB]
  float* w1o = smem + LD::slice_floats(NG, BF);     // [NSTEP][64] A operands of dL/de
  float* wbase = w1o + LD::w1_floats();             // kBwdWaves x WF

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int es = lane & 15;
  const int q = lane >> 4;
  const int cs = blockIdx.x % p.n_slices;
  const int wgi = blockIdx.x / p.n_slices;
  const int C = p.C;
  const int PC = NP * C;
  const int chan = cs * 16 + 4 * q;
  const float inv_rc = p.inv_r_cut;
  const float pref = p.radial_pref;
  const bool want_dvec = p.dvec_part != nullptr;

  float* ht = wbase + wave * WF;       // [16][64] h of the tile, later its dL/dpre (swz64)
  float* dsl = ht + 16 * 64;           // [16][64] SiLU'(pre) of the tile (swz64)
  float* ent = dsl + 16 * 64;          // [16][ENP] radial basis of the tile
  float* dent = ent + 16 * ENP;        // [16][ENP] its derivative d e_n / d r
  float* dwt = dent + 16 * ENP;        // [NG][16][16] dL/dw of the group's paths (swz16)

  static_for<NP>([&](auto J) {
    constexpr int j = decltype(J)::value;
    if constexpr (GR::of(j) == G) {
      constexpr int a = GR::rank(j);
      if constexpr (!BF) {
        for (int idx = tid; idx < H * 16; idx += kBwdWaves * 64) {
          const int k = idx >> 4, ch = idx & 15;
          w2c[(a * 16 + ch) * CS + k] = p.W2[(size_t)k * PC + j * C + cs * 16 + ch];
        }
      } else {
        // four consecutive k of one channel, and four consecutive channels of one k
        for (int idx = tid; idx < (H / 4) * 16; idx += kBwdWaves * 64) {
          const int k4 = (idx >> 4) * 4, ch = idx & 15;
          const float* src = p.W2 + (size_t)k4 * PC + j * C + cs * 16 + ch;
          w2cb[(a * 16 + ch) * CSB + k4 / 4] =
              u2{pk_bf16(src[0], src[PC]), pk_bf16(src[2 * (size_t)PC], src[3 * (size_t)PC])};
        }
        for (int idx = tid; idx < H * 4; idx += kBwdWaves * 64) {
          const int k = idx >> 2, c4 = (idx & 3) * 4;
          const f4 v = ld4(p.W2 + (size_t)k * PC + j * C + cs * 16 + c4);
          w2rb[(a * H + k) * RSB + c4 / 4] = pk4_bf16(v);
        }
      }
    }
  });
  for (int idx = tid; idx < NSTEP * 64; idx += kBwdWaves * 64) {
    const int st = idx >> 6, le = idx & 15, lq = (idx >> 4) & 3;
    w1o[idx] = le < NR ? p.W1[le * H + 16 * (st >> 2) + 4 * lq + (st & 3)] : 0.0f;
  }
  // radial-basis tile: columns NR..15 stay zero
  for (int i = lane; i < 16 * ENP; i += 64) ent[i] = 0.0f;
  __syncthreads();

  // loop-invariant MFMA operands and the accumulators
  float w1a[NJ][NR / 4];
  load_w1_operands<H, NR>(p.W1, es, q, w1a);
  f4 own[NOWN > 0 ? NOWN : 1];
  f4 dw1acc[NJ];
#pragma unroll
  for (int b = 0; b < (NOWN > 0 ? NOWN : 1); ++b) own[b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < NJ; ++mt) dw1acc[mt] = f4{0.f, 0.f, 0.f, 0.f};

  // the work-group's edges [lo, hi) in 16-edge tiles; wave w takes tiles w, w + 8, ...; every
  // wave runs the same number of rounds (a tile past the end has no valid edge: its radial basis
  // is zero, so h = 0 and its contributions to dL/dW1 and dL/dW2 are exactly zero)
  // (opaque: otherwise the compiler recomputes the 64-bit divisions inside the loop)
  const int lo = opaque((int)((long long)wgi * p.n_edges / p.wg_per_slice));
  const int hi = opaque((int)((long long)(wgi + 1) * p.n_edges / p.wg_per_slice));
  const int n_tiles = (hi - lo + 15) >> 4;
  const int rounds = (n_tiles + kBwdWaves - 1) / kBwdWaves;
  constexpr int kStride = 16 * kBwdWaves;

  // edge data of a wave's next tile is loaded one round ahead
  // MASK: the 16-edge tiles are taken in the order p.tile_order lists them (tiles that need the
  // most paths first), eight per round, one per wave; work-group g of the slice takes rounds g,
  // g + W, g + 2W, ... of that list (W work-groups per slice), so the tiles of a round need
  // similar work and every work-group gets a similar share of heavy and light rounds.
  const int n_rounds_all = MASK ? (p.n_tiles + kBwdWaves - 1) / kBwdWaves : 0;
  const int my_rounds = !MASK ? rounds
                        : (wgi < n_rounds_all ? (n_rounds_all - 1 - wgi) / p.wg_per_slice + 1 : 0);
  const int limit = MASK ? p.n_edges : hi;
  auto tile_base = [&](int rnd) {
    if constexpr (MASK) {
      const int ti = (wgi + rnd * p.wg_per_slice) * kBwdWaves + wave;
      return ti < p.n_tiles ? 16 * p.tile_order[ti] : p.n_edges;
    } else {
      return lo + 16 * wave + rnd * kStride;
    }
  };
  float nvx = 1.0f, nvy = 0.0f, nvz = 0.0f;
  int ns = 0, nd = 0;
  uint32_t nmask = 0;
  if (my_rounds > 0) {
    const int e = tile_base(0) + es;
    if (e < limit) {
      nvx = p.vec[3 * (size_t)e + 0];
      nvy = p.vec[3 * (size_t)e + 1];
      nvz = p.vec[3 * (size_t)e + 2];
      ns = p.src[e];
      nd = p.dst[e];
      if constexpr (MASK) nmask = p.path_mask[e];
    }
  }
  for (int round = 0; round < my_rounds; ++round) {
    const int base = tile_base(round);
    const int e = base + es;
    const bool valid = e < limit;
    const float vx = nvx, vy = nvy, vz = nvz;
    const int s = ns, d = nd;
    const uint32_t me = nmask;   // MASK: paths computed for this lane's edge
    const int en = MASK ? (round + 1 < my_rounds ? tile_base(round + 1) + es : limit) : e + kStride;
    if (en < limit) {
      nvx = p.vec[3 * (size_t)en + 0];
      nvy = p.vec[3 * (size_t)en + 1];
      nvz = p.vec[3 * (size_t)en + 2];
      ns = p.src[en];
      nd = p.dst[en];
      if constexpr (MASK) nmask = p.path_mask[en];
    } else {
      nvx = 1.0f;
      nvy = 0.0f;
      nvz = 0.0f;
      ns = 0;
      nd = 0;
      nmask = 0;
    }
    const int eid = e;
    // MASK: paths any edge of the tile needs (uniform across the wave)
    uint32_t need = ~0u;
    if constexpr (MASK) {
      uint32_t t = me;
      t |= (uint32_t)__shfl_xor((int)t, 1, 64);
      t |= (uint32_t)__shfl_xor((int)t, 2, 64);
      t |= (uint32_t)__shfl_xor((int)t, 4, 64);
      t |= (uint32_t)__shfl_xor((int)t, 8, 64);
      need = __builtin_amdgcn_readfirstlane(t);
    }
    // x[src] and G[dst] components read by this group's paths (16 bytes per lane each; lanes
    // without an edge read node 0)
    f4 xin[FIN], gin[FOUT];
    const float* xp = p.x + (size_t)s * FIN * C + chan;
    const float* gpp = p.G + (size_t)d * FOUT * C + chan;
    static_for<LIN + 1>([&](auto Lc) {
      constexpr int l = decltype(Lc)::value;
      if constexpr (group_reads_l1<PS, G>(l)) {
#pragma unroll
        for (int m = 0; m < 2 * l + 1; ++m) xin[l * l + m] = ld4(xp + (size_t)(l * l + m) * C);
      }
    });
    static_for<LOUT + 1>([&](auto Lc) {
      constexpr int l = decltype(Lc)::value;
      if constexpr (group_reads_l3<PS, G>(l)) {
#pragma unroll
        for (int m = 0; m < 2 * l + 1; ++m) gin[l * l + m] = ld4(gpp + (size_t)(l * l + m) * C);
      }
    });

    const float r = sqrtf(vx * vx + vy * vy + vz * vz);
    const float inv_r = 1.0f / r;
    const float ux = vx * inv_r, uy = vy * inv_r, uz = vz * inv_r;
    float Y[FSH];
    sh_eval<LSH, float>(ux, uy, uz, Y);
    float eb[NR], deb[NR];
    radial_basis<NR>(r, inv_r, inv_rc, pref, eb, deb);
    if (!valid) {
#pragma unroll
      for (int n = 0; n < NR; ++n) eb[n] = 0.0f;
    }
    {
      // h (B operand of w, and through LDS the A operand of dL/dW2) and SiLU'(pre) of the tile
      float hb[NSTEP], ds[NSTEP];
      hidden_layer<H, NR>(w1a, eb, q, hb, nullptr, ds);
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt) {
        st4(&ht[swz64(es, 16 * mt + 4 * q)], f4{hb[4 * mt], hb[4 * mt + 1], hb[4 * mt + 2], hb[4 * mt + 3]});
        st4(&dsl[swz64(es, 16 * mt + 4 * q)], f4{ds[4 * mt], ds[4 * mt + 1], ds[4 * mt + 2], ds[4 * mt + 3]});
      }
    }
    if (q == 0) {
#pragma unroll
      for (int n = 0; n < NR; ++n) {
        ent[es * ENP + n] = eb[n];
        dent[es * ENP + n] = deb[n];
      }
    }
    // keep the per-path LDS operand reads inside the loop (see opaque())
    const float* w2t = w2c + opaque(0);
    const float* hts = ht + opaque(0);

    float dY[FSH];
#pragma unroll
    for (int i = 0; i < FSH; ++i) dY[i] = 0.0f;
    f4 dh[NJ];
#pragma unroll
    for (int mt = 0; mt < NJ; ++mt) dh[mt] = f4{0.f, 0.f, 0.f, 0.f};
    // BF: h of the lane's edge as the bf16 B operand of w, four K values per group
    u2 hvb[NJ];
    if constexpr (BF) {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) hvb[jj] = pk4_bf16(ld4(&hts[swz64(es, 16 * jj + 4 * q)]));
    }

    static_for<NP>([&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (GR::of(j) == G) {
      constexpr int a = GR::rank(j);
      constexpr int gp = PS::id(j);
      constexpr int l1 = cg::kPaths[gp].l1;
      constexpr int l2 = cg::kPaths[gp].l2;
      constexpr int l3 = cg::kPaths[gp].l3;
      constexpr int off = cg::kPaths[gp].off;
      constexpr int nnz = cg::kPaths[gp].nnz;
      if (!MASK || (need & (1u << j))) {
      // w[channel 4q + i] of edge es = sum_k W2[k][4q + i] h[es][k], k = 16 jj + 4 q + i' in
      // step (jj, i'): A = W2[k][es] (four consecutive k, one ds_read_b128), B = h[es][k]
      f4 w;
      if constexpr (BF) {
        w = f4{0.f, 0.f, 0.f, 0.f};
        const u2* wcol = reinterpret_cast<const u2*>(w2t) + (a * 16 + es) * CSB;
        static_for<NJ>([&](auto JJ) {
          constexpr int jj = decltype(JJ)::value;
          w = mfma_bf16(wcol[4 * jj + q], hvb[jj], w);
        });
      } else {
        w = f4{0.f, 0.f, 0.f, 0.f};
        static_for<NJ>([&](auto JJ) {
          constexpr int jj = decltype(JJ)::value;
          const f4 hv = ld4(&hts[swz64(es, 16 * jj + 4 * q)]);
          const f4 wo = ld4(&w2t[(a * 16 + es) * CS + 16 * jj + 4 * q]);
          static_for<4>([&](auto I) {
            constexpr int i = decltype(I)::value;
            w = mfma_16x16x4(wo[i], hv[i], w);
          });
        });
      }
      const bool on = !MASK || ((me >> j) & 1u);
      if constexpr (MASK) {
        if (!on) w = f4{0.f, 0.f, 0.f, 0.f};
      }
      f4 dw = {0.f, 0.f, 0.f, 0.f};
      static_for<2 * l3 + 1>([&](auto M3) {
        constexpr int m3 = decltype(M3)::value;
        constexpr int fm1 = cg_first_m1(gp, m3);
        if constexpr (fm1 >= 0) {
          float mc[2 * l1 + 1];
          static_for<nnz>([&](auto K) {
            constexpr int k = decltype(K)::value;
            constexpr cg::Ent en = cg::kEnt[off + k];
            if constexpr (en.m3 == m3) {
              const float v = cg::kVal[off + k] * Y[l2 * l2 + en.m2];
              if constexpr (cg_first_in_pair(gp, k)) mc[en.m1] = v;
              else mc[en.m1] += v;
            }
          });
          float wg[4];
          static_for<4>([&](auto I) {
            constexpr int i = decltype(I)::value;
            float t = 0.0f;
            static_for<2 * l1 + 1>([&](auto M1) {
              constexpr int m1 = decltype(M1)::value;
              if constexpr (m1 == fm1) t = mc[m1] * xin[l1 * l1 + m1][i];
              else if constexpr (cg_has(gp, m1, m3)) t += mc[m1] * xin[l1 * l1 + m1][i];
            });
            const float g = gin[l3 * l3 + m3][i];
            dw[i] += g * t;
            wg[i] = w[i] * g;
          });
          static_for<2 * l1 + 1>([&](auto M1) {
            constexpr int m1 = decltype(M1)::value;
            if constexpr (cg_has(gp, m1, m3)) {
              const f4 xv = xin[l1 * l1 + m1];
              const float av = xv[0] * wg[0] + xv[1] * wg[1] + xv[2] * wg[2] + xv[3] * wg[3];
              static_for<nnz>([&](auto K) {
                constexpr int k = decltype(K)::value;
                constexpr cg::Ent en = cg::kEnt[off + k];
                if constexpr (en.m3 == m3 && en.m1 == m1) dY[l2 * l2 + en.m2] += cg::kVal[off + k] * av;
              });
            }
          });
        }
      });
      if constexpr (MASK) {
        if (!on) dw = f4{0.f, 0.f, 0.f, 0.f};
      }
      // dL/dh^T[k = 16 mt + 4q + r][e = es] += sum_{c in slice} W2[k][c] dL/dw[e][c]:
      // A = W2[16 mt + es][4q + r'] (column-major slice, single floats), B = dL/dw[es][4q + r']
      if constexpr (BF) {
        // A = W2[16 mt + es][4q .. 4q + 3] (bf16 row-major copy), B = dL/dw[es][4q .. 4q + 3]
        const u2 dwb = pk4_bf16(dw);
        const u2* wrow = reinterpret_cast<const u2*>(w2t) + NG * 16 * CSB + a * H * RSB;
        static_for<NJ>([&](auto MT) {
          constexpr int mt = decltype(MT)::value;
          dh[mt] = mfma_bf16(wrow[(16 * mt + es) * RSB + q], dwb, dh[mt]);
        });
      } else {
        static_for<NJ>([&](auto MT) {
          constexpr int mt = decltype(MT)::value;
          static_for<4>([&](auto R) {
            constexpr int rr = decltype(R)::value;
            dh[mt] = mfma_16x16x4(w2t[(a * 16 + 4 * q + rr) * CS + 16 * mt + es], dw[rr], dh[mt]);
          });
        });
      }
      // dL/dw of this path for the work-group's dL/dW2 pass
      if constexpr (WW) st4(&dwt[a * 256 + swz16(es, 4 * q)], dw);
      } else {
        if constexpr (WW) st4(&dwt[a * 256 + swz16(es, 4 * q)], f4{0.f, 0.f, 0.f, 0.f});
      }
      }
    });

    if constexpr (WW) {
      // dL/dW2[k = 16 mt + 4q + r][c = es] += sum_{e in tile} h[e][k] dL/dw[e][c] over the tiles of
      // all waves, for the blocks this wave owns: A = h^T[16 mt + es][4 st + q], B =
      // dL/dw[4 st + q][es]
      __syncthreads();
      // sources in the outer loop, the wave's blocks inside it: each source's reads feed NOWN
      // independent accumulation chains, so the MFMAs of one block cover the LDS latency of the
      // next.  The source loop is unrolled four times: the sources' bases then differ by
      // constants that fold into the LDS reads' offset fields (one address add per read for
      // four sources instead of one per source); unrolled fully, the compiler hoists the reads of
      // all eight sources and runs out of registers.
#pragma unroll 4
      for (int src = 0; src < kBwdWaves; ++src) {
        const float* hs = wbase + src * WF;
        static_for<NOWN>([&](auto B) {
          constexpr int ob = decltype(B)::value;
          const int blk = ob * kBwdWaves + wave;
          if (blk < NBLK) {
            const int a = blk / NJ, mt = blk % NJ;
            const float* dws = hs + 2 * 16 * 64 + 2 * 16 * ENP + a * 256;
            if constexpr (BF) {
              // one bf16 MFMA over the 16 edges, taken as e = 4q + st
              own[ob] = mfma_bf16(
                  pk4_bf16(f4{hs[swz64(4 * q, 16 * mt + es)], hs[swz64(4 * q + 1, 16 * mt + es)],
                              hs[swz64(4 * q + 2, 16 * mt + es)], hs[swz64(4 * q + 3, 16 * mt + es)]}),
                  pk4_bf16(f4{dws[swz16(4 * q, es)], dws[swz16(4 * q + 1, es)],
                              dws[swz16(4 * q + 2, es)], dws[swz16(4 * q + 3, es)]}),
                  own[ob]);
            } else {
#pragma unroll
              for (int st = 0; st < 4; ++st)
                own[ob] = mfma_16x16x4(hs[swz64(4 * st + q, 16 * mt + es)],
                                       dws[swz16(4 * st + q, es)], own[ob]);
            }
          }
        });
      }
      __syncthreads();
    }

    // the dL/dvec partial left by the previous group's launch
    float pv0 = 0.0f, pv1 = 0.0f, pv2 = 0.0f;
    float* dvp = want_dvec && valid ? p.dvec_part + ((size_t)cs * p.n_edges + eid) * 3 : nullptr;
    if constexpr (G > 0) {
      if (dvp != nullptr && q == 0) {
        pv0 = dvp[0];
        pv1 = dvp[1];
        pv2 = dvp[2];
      }
    }
    // dL/dpre = dL/dh * SiLU'(pre) for this lane's K set; dL/de^T[n = 4q + r][e = es] =
    // sum_k W1[n][k] dL/dpre[e][k]
    float dpre[NSTEP];
#pragma unroll
    for (int mt = 0; mt < NJ; ++mt) {
      const f4 sl = ld4(&dsl[swz64(es, 16 * mt + 4 * q)]);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) dpre[4 * mt + r4] = dh[mt][r4] * sl[r4];
    }
    f4 de = {0.f, 0.f, 0.f, 0.f};
    {
      // A = W1[n = es][k(st, q)] (rows n >= NR are zero), from LDS (read per tile, not held)
      const float* w1s = w1o + opaque(0);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) de = mfma_16x16x4(w1s[st * 64 + lane], dpre[st], de);
    }

    if constexpr (WW) {
      // dL/dW1[n = 4q + r][k = 16 mt + es] += sum_{e in tile} e_n[e] dL/dpre[e][k]; dL/dpre
      // reuses the h tile (no wave reads it after the barrier above)
      float* ept = ht;
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt)
        st4(&ept[swz64(es, 16 * mt + 4 * q)],
            f4{dpre[4 * mt], dpre[4 * mt + 1], dpre[4 * mt + 2], dpre[4 * mt + 3]});
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float an = ent[(4 * st + q) * ENP + es];
#pragma unroll
        for (int mt = 0; mt < NJ; ++mt)
          dw1acc[mt] = mfma_16x16x4(an, ept[swz64(4 * st + q, 16 * mt + es)], dw1acc[mt]);
      }
    }

    if (want_dvec) {
      // dL/dr = sum_n dL/de_n de_n/dr  (rows n = 4q + r of the dL/de tile)
      float drp = 0.0f;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = 4 * q + r4;
        drp += n < NR ? de[r4] * dent[es * ENP + n] : 0.0f;
      }
      // dL/dvec is linear in dL/dY and dL/dr: each lane forms the contribution of its own
      // channels and rows of dL/de, and only the three components are summed over the quads
      float gx, gy, gz;
      sh_vjp<LSH, float>(ux, uy, uz, dY, gx, gy, gz);
      const float gu = gx * ux + gy * uy + gz * uz;
      const float d0 = cross_row_sum(drp * ux + (gx - gu * ux) * inv_r);
      const float d1 = cross_row_sum(drp * uy + (gy - gu * uy) * inv_r);
      const float d2 = cross_row_sum(drp * uz + (gz - gu * uz) * inv_r);
      if (dvp != nullptr && q == 0) {
        dvp[0] = pv0 + d0;
        dvp[1] = pv1 + d1;
        dvp[2] = pv2 + d2;
      }
    }
  }

  if constexpr (WW) {
    // dL/dW1: the waves' accumulators summed in LDS in wave order; one row per work-group, which
    // the launch of group 0 writes and the later groups' launches add to
    if (p.dW1_part != nullptr) {
      float* acc = smem;  // [NR][H], reuses the W2 slice once every wave is done with it
      for (int wv = 0; wv < kBwdWaves; ++wv) {
        __syncthreads();
        if (wave == wv) {
#pragma unroll
          for (int mt = 0; mt < NJ; ++mt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int n = 4 * q + r4;
              if (n < NR) {
                float* dptr = &acc[n * H + 16 * mt + es];
                *dptr = (wv == 0 ? 0.0f : *dptr) + dw1acc[mt][r4];
              }
            }
        }
      }
      __syncthreads();
      float* op = p.dW1_part + (size_t)blockIdx.x * NR * H;
      for (int idx = tid; idx < NR * H; idx += kBwdWaves * 64)
        op[idx] = (G == 0 ? 0.0f : op[idx]) + acc[idx];
    }
    // dL/dW2: every (k, channel) of the group's paths is owned by exactly one wave, which writes
    // the work-group's partial directly
    if (p.dW2_part != nullptr) {
      static_for<NOWN>([&](auto B) {
        constexpr int ob = decltype(B)::value;
        const int blk = ob * kBwdWaves + wave;
        if (blk < NBLK) {
          const int a = blk / NJ, mt = blk % NJ;
          int j = 0;
          static_for<NG>([&](auto A) {
            constexpr int aa = decltype(A)::value;
            if (a == aa) j = GR::path(G, aa);
          });
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int k = 16 * mt + 4 * q + r4;
            p.dW2_part[((size_t)wgi * H + k) * PC + j * C + cs * 16 + es] = own[ob][r4];
          }
        }
      });
    }
  }
}

#if !EQUITP_BWD_BF16 && !EQUITP_BWD_MASKED
// out[e][c] = sum_s part[s][e][c] over the slices, c < 3 (fixed order).
__global__ void sum_slices_kernel(const float* __restrict__ part, int n_slices, int n,
                                  float* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = 0.0f;
  for (int s = 0; s < n_slices; ++s) v += part[(size_t)s * n + i];
  out[i] = v;
}

// out[c] = sum_r part[r][c].  A block takes 64 columns; its 16 row groups each sum every 16th row
// in order, then the 16 partial sums are added in a fixed tree order (deterministic).
__global__ void __launch_bounds__(1024) reduce_rows_kernel(const float* __restrict__ part, int rows,
                                                           int cols, float* __restrict__ out) {
  __shared__ float buf[16][64];
  const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  float a = 0.0f;
  if (c < cols)
    for (int r = rg; r < rows; r += 16) a += part[(size_t)r * cols + c];
  buf[rg][cl] = a;
  __syncthreads();
  for (int w = 8; w >= 1; w >>= 1) {
    if (rg < w) buf[rg][cl] += buf[rg + w][cl];
    __syncthreads();
  }
  if (rg == 0 && c < cols) out[c] = buf[0][cl];
}

__global__ void fill_zero_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

#endif  // !EQUITP_BWD_BF16 && !EQUITP_BWD_MASKED

template <int L, int H, int G, bool BF, bool MASK = false>
hipError_t bwd_group(const BwdParams& p, hipStream_t st) {
  using PS = PathSet<L, L, L>;
  constexpr int NG = Groups<PS::N>::count(G);
  if constexpr (NG == 0) {
    return hipSuccess;
  } else {
    const bool ww = p.dW1_part != nullptr || p.dW2_part != nullptr;
    auto kern = ww ? bwd_kernel<L, L, L, H, 8, G, true, BF, MASK>
                   : bwd_kernel<L, L, L, H, 8, G, false, BF, MASK>;
    constexpr size_t lds = BwdLds<H>::bytes(NG, BF);
    static_assert(lds <= 160 * 1024, "LDS of a backward work-group exceeds the 160 KiB of a CU");
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(p.wg_per_slice * p.n_slices), dim3(kBwdWaves * 64), lds, st, p);
    return hipGetLastError();
  }
}

template <int L, int H, bool BF = false, bool MASK = false>
hipError_t bwd_one(const BwdParams& p, hipStream_t st) {
  static_assert(kBwdGroups == 4, "bwd_one launches up to four groups (empty groups launch nothing)");
  hipError_t err;
  if ((err = bwd_group<L, H, 0, BF, MASK>(p, st)) != hipSuccess) return err;
  if ((err = bwd_group<L, H, 1, BF, MASK>(p, st)) != hipSuccess) return err;
  if ((err = bwd_group<L, H, 2, BF, MASK>(p, st)) != hipSuccess) return err;
  return bwd_group<L, H, 3, BF, MASK>(p, st);
}

}  // namespace

#if EQUITP_BWD_MASKED
// The per-edge path-subset kernels (fp32, width 64, l = 1..3), a translation unit of their own
// (this file compiled with EQUITP_BWD_MASKED=1).
hipError_t launch_bwd_masked(const ConvShape& s, const BwdParams& p, hipStream_t st) {
  if (s.n_radial != 8 || s.L_in != s.L_sh || s.L_in != s.L_out || s.hidden != 64 || s.mlp_bf16 ||
      p.path_mask == nullptr)
    return hipErrorInvalidValue;
  switch (s.L_in) {
    case 1: return bwd_one<1, 64, false, true>(p, st);
    case 2: return bwd_one<2, 64, false, true>(p, st);
    case 3: return bwd_one<3, 64, false, true>(p, st);
  }
  return hipErrorInvalidValue;
}

namespace {
template <int L>
hipError_t bwd_some(const BwdParams& p, unsigned groups, hipStream_t st) {
  hipError_t err = hipSuccess;
  if ((groups & 1u) && (err = bwd_group<L, 64, 0, false, true>(p, st)) != hipSuccess) return err;
  if ((groups & 2u) && (err = bwd_group<L, 64, 1, false, true>(p, st)) != hipSuccess) return err;
  if ((groups & 4u) && (err = bwd_group<L, 64, 2, false, true>(p, st)) != hipSuccess) return err;
  if ((groups & 8u) && (err = bwd_group<L, 64, 3, false, true>(p, st)) != hipSuccess) return err;
  return err;
}
}  // namespace

// Only the path groups in `groups` (bit g = group g), for masks under which the other groups'
// paths are off for every edge.  The caller zeroes what a skipped group would have written or
// started: the dL/dvec and dL/dW1 partials when group 0 is skipped, and the dL/dW2 partial's
// columns of every skipped group.
hipError_t launch_bwd_masked_groups(const ConvShape& s, const BwdParams& p, unsigned groups,
                                    hipStream_t st) {
  if (s.n_radial != 8 || s.L_in != s.L_sh || s.L_in != s.L_out || s.hidden != 64 || s.mlp_bf16 ||
      p.path_mask == nullptr)
    return hipErrorInvalidValue;
  switch (s.L_in) {
    case 1: return bwd_some<1>(p, groups, st);
    case 2: return bwd_some<2>(p, groups, st);
    case 3: return bwd_some<3>(p, groups, st);
  }
  return hipErrorInvalidValue;
}

// The backward launch group of path j of the configuration with every l <= L.
int bwd_path_group(int L, int j) {
  switch (L) {
    case 1: return Groups<PathSet<1, 1, 1>::N>::of(j);
    case 2: return Groups<PathSet<2, 2, 2>::N>::of(j);
    case 3: return Groups<PathSet<3, 3, 3>::N>::of(j);
  }
  return -1;
}
#elif EQUITP_BWD_BF16
// The bf16-operand kernels, built as a translation unit of their own (this file compiled with
// EQUITP_BWD_BF16=1) so that the two halves compile in parallel.
hipError_t launch_bwd_bf16(const ConvShape& s, const BwdParams& p, hipStream_t st) {
  if (s.n_radial != 8 || s.L_in != s.L_sh || s.L_in != s.L_out || s.hidden != 64)
    return hipErrorInvalidValue;
  switch (s.L_in) {
    case 1: return bwd_one<1, 64, true>(p, st);
    case 2: return bwd_one<2, 64, true>(p, st);
    case 3: return bwd_one<3, 64, true>(p, st);
  }
  return hipErrorInvalidValue;
}
#else
hipError_t launch_bwd(const ConvShape& s, const BwdParams& p, hipStream_t st) {
  if (s.n_radial != 8 || s.L_in != s.L_sh || s.L_in != s.L_out) return hipErrorInvalidValue;
  if (s.mlp_bf16) return launch_bwd_bf16(s, p, st);
  if (s.hidden == 64) {
    switch (s.L_in) {
      case 0: return bwd_one<0, 64>(p, st);
      case 1: return bwd_one<1, 64>(p, st);
      case 2: return bwd_one<2, 64>(p, st);
      case 3: return bwd_one<3, 64>(p, st);
    }
  } else if (s.hidden == 16) {
    switch (s.L_in) {
      case 0: return bwd_one<0, 16>(p, st);
      case 1: return bwd_one<1, 16>(p, st);
      case 2: return bwd_one<2, 16>(p, st);
      case 3: return bwd_one<3, 16>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

int bwd_num_groups(const ConvShape& s) {
  switch (s.L_in) {
    case 0: return Groups<PathSet<0, 0, 0>::N>::n();
    case 1: return Groups<PathSet<1, 1, 1>::N>::n();
    case 2: return Groups<PathSet<2, 2, 2>::N>::n();
    case 3: return Groups<PathSet<3, 3, 3>::N>::n();
  }
  return 0;
}

int bwd_wg_per_slice(const ConvShape& s, int n_edges, int n_cu) {
  const int n_slices = s.C / 16;
  int wps = n_cu / n_slices;  // one work-group per CU (LDS-bound)
  if (wps < 1) wps = 1;
  const int max_by_edges = (n_edges + 255) / 256;  // at least two tiles per wave on average
  if (wps > max_by_edges) wps = max_by_edges;
  return wps < 1 ? 1 : wps;
}

hipError_t launch_sum_slices(const float* part, int n_slices, int n, float* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sum_slices_kernel, dim3((n + 255) / 256), dim3(256), 0, st, part, n_slices, n, out);
  return hipGetLastError();
}

hipError_t launch_reduce_rows(const float* part, int rows, int cols, float* out, hipStream_t st) {
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((cols + 63) / 64), dim3(1024), 0, st, part, rows, cols,
                     out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

#endif  // EQUITP_BWD_BF16

}  // namespace equitp
