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
// The paths are split into kBwdWaves groups and the backward runs as one kernel launch per group
// (in stream order), so each launch holds the code of one group only and stays inside the
// instruction cache.  A work-group owns one 16-channel slice (blockIdx % n_slices: with 8 slices
// every XCD works on one slice, so its L2 keeps that slice of x and G) and a contiguous range of
// edges, split between its waves; every wave runs the same code on its own edges, with no
// synchronisation until the end.  Per 16-edge tile each wave, lane = (edge es, channel quad q):
//   * hidden layer on MFMA (A = W1^T in registers, B = radial basis), h and pre in registers;
//   * per own path: w = MFMA(W2 slice from LDS, h); t, dL/dw, dL/dY on VALU; dL/dh^T +=
//     MFMA(W2 in registers, dL/dw^T) contracting the slice's channels; dL/dW2 += MFMA(h^T,
//     dL/dw) contracting the tile's edges (both operands transposed through a wave-private LDS
//     buffer);
//   * dL/dpre = dL/dh * SiLU'(pre); dL/de^T = MFMA(W1, dL/dpre^T); dL/dW1 += MFMA(e^T, dL/dpre)
//     (again through wave-private LDS);
//   * dL/dvec of its paths and slice, from dL/dY and dL/de (dL/dvec is linear in both, so the
//     partial of each (group, slice) is exact), added to the 3-vector that the previous group's
//     launch left for this edge and slice.
// At the end the waves' dL/dW2 accumulators are summed in LDS and one partial per work-group is
// written (each launch fills its group's columns).  A small kernel sums the slice partials of
// dL/dvec; fixed-order row sums finish dL/dW1 and dL/dW2.  No atomics anywhere: results are
// bitwise reproducible run to run.
#include "common.h"
#include "params.h"

namespace equitp {
namespace {

// Paths of a configuration split into kBwdWaves groups, one per wave.  For the 23 paths of
// l <= 3 the split (6/6/6/5 paths) was chosen by a small offline search to minimise the largest
// number of x and G components a wave gathers (18 of 32), which sets its register footprint;
// smaller path sets use contiguous groups.
constexpr int kGroupL3[23] = {2, 3, 1, 3, 0, 2, 1, 0, 2, 1, 0, 0, 2, 2, 0, 0, 2, 3, 1, 3, 3, 1, 1};

template <int NP>
struct Groups {
  static constexpr int of(int j) { return NP == 23 ? kGroupL3[j] : (j * kBwdWaves) / NP; }
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

// Slots of the wave's LDS gather buffer (one 64-lane x 16-byte row per component): the x
// components of the blocks l1 that group G reads, in order of l, then its G components.
template <typename PS, int G>
constexpr int x_slot(int l) {
  int n = 0;
  for (int k = 0; k < l; ++k) n += group_reads_l1<PS, G>(k) ? 2 * k + 1 : 0;
  return n;
}
template <typename PS, int G>
constexpr int g_slot(int l) {
  int n = x_slot<PS, G>(4);
  for (int k = 0; k < l; ++k) n += group_reads_l3<PS, G>(k) ? 2 * k + 1 : 0;
  return n;
}
template <typename PS, int G>
constexpr int gather_slots() { return g_slot<PS, G>(4); }

// Direct global-to-LDS load of 16 bytes per lane: lane l's bytes land at dst + 16 l.  dst must
// be the same for every lane of the wave.
__device__ __forceinline__ void lds_dma16(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                   (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
}

constexpr int kRS = 20;          // row stride (floats) of the W2 slice in LDS: [path][k][kRS]

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

template <int H>
struct WaveLds {
  static constexpr int ENP = 16;                 // radial-basis tile row stride
  // h (later dL/dpre) tile [16][64] swizzled, radial basis and derivative [16][16] each,
  // dL/dw tile [16][16] swizzled
  static constexpr int floats = 16 * 64 + 2 * 16 * ENP + 16 * 16;
};

template <int LIN, int LSH, int LOUT, int H, int NR, int G, bool WW>
__device__ __forceinline__ void bwd_wave(const BwdParams& p, const float* w2s, const float* w2c,
                                         float* wl,
                                         float* red, int cs, int e_lo, int e_hi) {
  // w2s holds the W2 slice of this group's paths row-major, [rank][k][kRS] (four consecutive
  // channels per ds_read_b128: the A operand of dL/dh); w2c the same slice column-major,
  // [rank][channel][H + 4] (four consecutive k per ds_read_b128: the A operand of w)
  using PS = PathSet<LIN, LSH, LOUT>;
  using GR = Groups<PS::N>;
  constexpr int NP = PS::N;
  constexpr int FIN = (LIN + 1) * (LIN + 1);
  constexpr int FSH = (LSH + 1) * (LSH + 1);
  constexpr int FOUT = (LOUT + 1) * (LOUT + 1);
  constexpr int NSTEP = H / 4;
  constexpr int NJ = H / 16;
  constexpr int NG = GR::count(G);
  constexpr int NGA = NG > 0 ? NG : 1;
  constexpr int ENP = WaveLds<H>::ENP;
  static_assert(NR <= 16 && H <= 64, "unsupported shape");

  float* ht = wl;                      // [16][64] h of the tile, later its dL/dpre (swz64)
  float* ent = wl + 16 * 64;           // [16][ENP] radial basis of the tile
  float* dent = ent + 16 * ENP;        // [16][ENP] its derivative d e_n / d r
  float* dwt = dent + 16 * ENP;        // [16][16] dL/dw of one path (swz16)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int es = lane & 15;
  const int q = lane >> 4;
  const int C = p.C;
  const int PC = NP * C;
  const float r_cut = p.r_cut;
  const float inv_rc = 1.0f / r_cut;
  const int chan = cs * 16 + 4 * q;
  // WW: the weight gradients are accumulated (a compile-time switch: a runtime condition on the
  // accumulators would make the compiler copy them between register files every tile)
  const bool want_dvec = p.dvec_part != nullptr;

  // loop-invariant MFMA operands
  float w1a[NJ][NR / 4];
  load_w1_operands<H, NR>(p.W1, es, q, w1a);
  f4 dw2acc[NGA][NJ];
  f4 dw1acc[NJ];
#pragma unroll
  for (int a = 0; a < NGA; ++a)
#pragma unroll
    for (int mt = 0; mt < NJ; ++mt) dw2acc[a][mt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < NJ; ++mt) dw1acc[mt] = f4{0.f, 0.f, 0.f, 0.f};
  // radial-basis tile: columns NR..15 stay zero
  for (int i = lane; i < 16 * ENP; i += 64) ent[i] = 0.0f;

  // The x and G rows of a tile reach this wave's LDS gather buffer through direct global-to-LDS
  // loads issued one tile ahead; the edge ids those loads need are read two tiles ahead and the
  // edge vectors one tile ahead.  Lanes past the end of the range gather node 0: their radial
  // basis is zeroed, so h = 0 and every contribution of theirs to dL/dW1 and dL/dW2 is exactly
  // zero, and their dL/dvec is not stored.
  float* gbuf = wl + WaveLds<H>::floats;  // [gather_slots][64 lanes][4]
  auto issue_gather = [&](int s_, int d_) {
    const float* xp = p.x + (size_t)s_ * FIN * C + chan;
    const float* gp_ = p.G + (size_t)d_ * FOUT * C + chan;
    static_for<LIN + 1>([&](auto Lc) {
      constexpr int l = decltype(Lc)::value;
      if constexpr (group_reads_l1<PS, G>(l)) {
        static_for<2 * l + 1>([&](auto Mc) {
          constexpr int m = decltype(Mc)::value;
          lds_dma16(xp + (size_t)(l * l + m) * C, gbuf + (x_slot<PS, G>(l) + m) * 256);
        });
      }
    });
    static_for<LOUT + 1>([&](auto Lc) {
      constexpr int l = decltype(Lc)::value;
      if constexpr (group_reads_l3<PS, G>(l)) {
        static_for<2 * l + 1>([&](auto Mc) {
          constexpr int m = decltype(Mc)::value;
          lds_dma16(gp_ + (size_t)(l * l + m) * C, gbuf + (g_slot<PS, G>(l) + m) * 256);
        });
      }
    });
  };
  float nvx = 1.0f, nvy = 0.0f, nvz = 0.0f;
  int ns = 0, nd = 0;
  if (e_lo < e_hi) {
    int s0 = 0, d0 = 0;
    if (e_lo + es < e_hi) {
      const int e = e_lo + es;
      nvx = p.vec[3 * (size_t)e + 0];
      nvy = p.vec[3 * (size_t)e + 1];
      nvz = p.vec[3 * (size_t)e + 2];
      s0 = p.src[e];
      d0 = p.dst[e];
    }
    issue_gather(s0, d0);
    if (e_lo + 16 + es < e_hi) {
      ns = p.src[e_lo + 16 + es];
      nd = p.dst[e_lo + 16 + es];
    }
  }
  // dL/dvec of a tile is stored at the start of the next one, after the wait below, so that the
  // wait (which counts stores too) never waits for it
  float* dv_ptr = nullptr;
  float dv0 = 0.0f, dv1 = 0.0f, dv2 = 0.0f;
  for (int base = e_lo; base < e_hi; base += 16) {
    const int e = base + es;
    const bool valid = e < e_hi;
    const float vx = nvx, vy = nvy, vz = nvz;
    // this tile's gathers (the compiler does not track direct-to-LDS loads), its edge vectors
    // and the next tile's ids have arrived
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (dv_ptr != nullptr) {
      dv_ptr[0] = dv0;
      dv_ptr[1] = dv1;
      dv_ptr[2] = dv2;
    }
    dv_ptr = nullptr;
    f4 xin[FIN], gin[FOUT];
    static_for<LIN + 1>([&](auto Lc) {
      constexpr int l = decltype(Lc)::value;
      if constexpr (group_reads_l1<PS, G>(l)) {
#pragma unroll
        for (int m = 0; m < 2 * l + 1; ++m)
          xin[l * l + m] = ld4(gbuf + (x_slot<PS, G>(l) + m) * 256 + 4 * lane);
      }
    });
    static_for<LOUT + 1>([&](auto Lc) {
      constexpr int l = decltype(Lc)::value;
      if constexpr (group_reads_l3<PS, G>(l)) {
#pragma unroll
        for (int m = 0; m < 2 * l + 1; ++m)
          gin[l * l + m] = ld4(gbuf + (g_slot<PS, G>(l) + m) * 256 + 4 * lane);
      }
    });
    // the buffer is free once these reads have completed: gather the next tile into it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (base + 16 < e_hi) issue_gather(ns, nd);
    if (base + 16 + es < e_hi) {
      const int en = base + 16 + es;
      nvx = p.vec[3 * (size_t)en + 0];
      nvy = p.vec[3 * (size_t)en + 1];
      nvz = p.vec[3 * (size_t)en + 2];
    } else {
      nvx = 1.0f;
      nvy = 0.0f;
      nvz = 0.0f;
    }
    if (base + 32 + es < e_hi) {
      ns = p.src[base + 32 + es];
      nd = p.dst[base + 32 + es];
    } else {
      ns = 0;
      nd = 0;
    }
    const float r = sqrtf(vx * vx + vy * vy + vz * vz);
    const float inv_r = 1.0f / r;
    const float ux = vx * inv_r, uy = vy * inv_r, uz = vz * inv_r;
    float Y[FSH];
    sh_eval<LSH, float>(ux, uy, uz, Y);
    float eb[NR], deb[NR];
    radial_basis<NR>(r, inv_r, r_cut, inv_rc, eb, deb);
    if (!valid) {
#pragma unroll
      for (int n = 0; n < NR; ++n) eb[n] = 0.0f;
    }
    {
      float hb[NSTEP];
      hidden_layer<H, NR>(w1a, eb, q, hb);
      // h of the tile goes to this wave's LDS: the per-path MFMAs read it back as operands
      asm volatile("" ::: "memory");
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt)
        st4(&ht[swz64(es, 16 * mt + 4 * q)], f4{hb[4 * mt], hb[4 * mt + 1], hb[4 * mt + 2], hb[4 * mt + 3]});
    }
    const float* w2t = w2s + opaque(0);
    const float* w2ct = w2c + opaque(0);
    if (q == 0) {
#pragma unroll
      for (int n = 0; n < NR; ++n) {
        ent[es * ENP + n] = eb[n];
        dent[es * ENP + n] = deb[n];
      }
    }

    float dY[FSH];
#pragma unroll
    for (int i = 0; i < FSH; ++i) dY[i] = 0.0f;
    f4 dh[NJ];
#pragma unroll
    for (int mt = 0; mt < NJ; ++mt) dh[mt] = f4{0.f, 0.f, 0.f, 0.f};
    asm volatile("" ::: "memory");
    // tile operands shared by all paths: h of the lane's edge (B of the W2 contraction) and
    // h^T (A of the dL/dW2 contraction)
    f4 hvv[NJ];
    float hAA[4][NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) hvv[jj] = ld4(&ht[swz64(es, 16 * jj + 4 * q)]);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt) hAA[st][mt] = ht[swz64(4 * st + q, 16 * mt + es)];

    // A operands of the w contraction, W2[k = 16 jj + 4 q + i][c = es], read one path ahead
    constexpr int CS = H + 4;
    f4 wop[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) wop[jj] = ld4(&w2ct[es * CS + 16 * jj + 4 * q]);

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
      // w[channel 4q + i] of edge es: A = W2[k(st, q)][es], B = h[es][k(st, q)]
      f4 w = {0.f, 0.f, 0.f, 0.f};
      static_for<NJ>([&](auto JJ) {
        constexpr int jj = decltype(JJ)::value;
        const f4 hv = hvv[jj];
        static_for<4>([&](auto I) {
          constexpr int i = decltype(I)::value;
          w = mfma_16x16x4(wop[jj][i], hv[i], w);
        });
      });
      if constexpr (a + 1 < NG) {
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          wop[jj] = ld4(&w2ct[((a + 1) * 16 + es) * CS + 16 * jj + 4 * q]);
      }
      // A operands of dL/dh: W2[k = 16 mt + es][c = 4q .. 4q + 3]
      f4 dho[NJ];
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt) dho[mt] = ld4(&w2t[(a * H + 16 * mt + es) * kRS + 4 * q]);
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
      // dL/dh^T[k = 16 mt + 4q + r][e = es] += sum_{c in slice} W2[k][c] dL/dw[e][c]
      static_for<NJ>([&](auto MT) {
        constexpr int mt = decltype(MT)::value;
        const f4 b4 = dho[mt];
        dh[mt] = mfma_16x16x4(b4[0], dw[0], dh[mt]);
        dh[mt] = mfma_16x16x4(b4[1], dw[1], dh[mt]);
        dh[mt] = mfma_16x16x4(b4[2], dw[2], dh[mt]);
        dh[mt] = mfma_16x16x4(b4[3], dw[3], dh[mt]);
      });
      // dL/dW2[k = 16 mt + 4q + r][c = es] += sum_{e in tile} h[e][k] dL/dw[e][c]
      if constexpr (WW) {
        asm volatile("" ::: "memory");
        st4(&dwt[swz16(es, 4 * q)], dw);
        asm volatile("" ::: "memory");
        float bv[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) bv[st] = dwt[swz16(4 * st + q, es)];
        asm volatile("" ::: "memory");
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int mt = 0; mt < NJ; ++mt)
            dw2acc[a][mt] = mfma_16x16x4(hAA[st][mt], bv[st], dw2acc[a][mt]);
      }
      }
    });

    // the dL/dvec partial left by the previous group's launch, added at the end of the tile
    float pv0 = 0.0f, pv1 = 0.0f, pv2 = 0.0f;
    float* dvp = want_dvec ? p.dvec_part + ((size_t)cs * p.n_edges + e) * 3 : nullptr;
    if constexpr (G > 0) {
      if (want_dvec && q == 0 && valid) {
        pv0 = dvp[0];
        pv1 = dvp[1];
        pv2 = dvp[2];
      }
    }
    // pre-activations again (from the radial basis kept in LDS), then dL/dpre for this lane's K
    // set; dL/de^T[n = 4q + r][e = es] = sum_k W1[n][k] dL/dpre[e][k]
    float pre[NSTEP];
    {
      float hb[NSTEP];
      float eb2[NR];
#pragma unroll
      for (int n = 0; n < NR; ++n) eb2[n] = ent[es * ENP + n];
      hidden_layer<H, NR>(w1a, eb2, q, hb, pre);
    }
    float dpre[NSTEP];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const float z = pre[st];
      const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
      dpre[st] = dh[st >> 2][st & 3] * sg * (1.0f + z * (1.0f - sg));
    }
    f4 de = {0.f, 0.f, 0.f, 0.f};
    {
      // A = W1[n = es][k(st, q)] (rows n >= NR are zero), read per tile
      const float* w1p = p.W1 + opaque(0);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const float a1 = es < NR ? w1p[es * H + 16 * (st >> 2) + 4 * q + (st & 3)] : 0.0f;
        de = mfma_16x16x4(a1, dpre[st], de);
      }
    }

    if constexpr (WW) {
      // dL/dW1[n = 4q + r][k = 16 mt + es] += sum_{e in tile} e_n[e] dL/dpre[e][k]; dL/dpre
      // reuses the h buffer (h is no longer read in this tile)
      float* ept = ht;
      asm volatile("" ::: "memory");
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt)
        st4(&ept[swz64(es, 16 * mt + 4 * q)],
            f4{dpre[4 * mt], dpre[4 * mt + 1], dpre[4 * mt + 2], dpre[4 * mt + 3]});
      asm volatile("" ::: "memory");
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float an = ent[(4 * st + q) * ENP + es];
#pragma unroll
        for (int mt = 0; mt < NJ; ++mt)
          dw1acc[mt] = mfma_16x16x4(an, ept[swz64(4 * st + q, 16 * mt + es)], dw1acc[mt]);
      }
      asm volatile("" ::: "memory");
    }

    if (want_dvec) {
      // dL/dr = sum_n dL/de_n de_n/dr  (rows n = 4q + r of the dL/de tile)
      float drp = 0.0f;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = 4 * q + r4;
        drp += n < NR ? de[r4] * dent[es * ENP + n] : 0.0f;
      }
      const float dr = cross_row_sum(drp);
#pragma unroll
      for (int i = 0; i < FSH; ++i) dY[i] = cross_row_sum(dY[i]);
      float gx, gy, gz;
      sh_vjp<LSH, float>(ux, uy, uz, dY, gx, gy, gz);
      const float gu = gx * ux + gy * uy + gz * uz;
      if (q == 0 && valid) {
        dv_ptr = dvp;
        dv0 = pv0 + (dr * ux + (gx - gu * ux) * inv_r);
        dv1 = pv1 + (dr * uy + (gy - gu * uy) * inv_r);
        dv2 = pv2 + (dr * uz + (gz - gu * uz) * inv_r);
      }
    }
  }
  if (dv_ptr != nullptr) {
    dv_ptr[0] = dv0;
    dv_ptr[1] = dv1;
    dv_ptr[2] = dv2;
  }

  // dL/dW1: the waves' accumulators summed in LDS in wave order; one row per work-group, which
  // the launch of group 0 writes and the later groups' launches add to
  if (WW && p.dW1_part != nullptr) {
    float* acc = red;  // [NR][H], reuses the W2 slice once every wave is done with it
    for (int wv = 0; wv < kBwdWaves; ++wv) {
      __syncthreads();
      if (wave == wv) {
#pragma unroll
        for (int mt = 0; mt < NJ; ++mt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int n = 4 * q + r4;
            if (n < NR) {
              float* d = &acc[n * H + 16 * mt + es];
              *d = (wv == 0 ? 0.0f : *d) + dw1acc[mt][r4];
            }
          }
      }
    }
    __syncthreads();
    float* op = p.dW1_part + (size_t)blockIdx.x * NR * H;
    for (int idx = threadIdx.x; idx < NR * H; idx += kBwdWaves * 64)
      op[idx] = (G == 0 ? 0.0f : op[idx]) + acc[idx];
    __syncthreads();
  }
  // dL/dW2: the waves' accumulators summed in LDS in wave order, one partial per work-group
  if (WW && p.dW2_part != nullptr) {
    float* acc = red;  // [NG][H][16], reuses the W2 slice once every wave is done with it
    const int wgi = blockIdx.x / p.n_slices;
    for (int wv = 0; wv < kBwdWaves; ++wv) {
      __syncthreads();
      if (wave == wv) {
#pragma unroll
        for (int a = 0; a < NG; ++a)
#pragma unroll
          for (int mt = 0; mt < NJ; ++mt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              float* d = &acc[(a * H + 16 * mt + 4 * q + r4) * 16 + es];
              *d = (wv == 0 ? 0.0f : *d) + dw2acc[a][mt][r4];
            }
      }
    }
    __syncthreads();
    const int tid = threadIdx.x;
    static_for<NP>([&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (GR::of(j) == G) {
        constexpr int a = GR::rank(j);
        for (int idx = tid; idx < H * 16; idx += kBwdWaves * 64) {
          const int k = idx >> 4, ch = idx & 15;
          p.dW2_part[((size_t)wgi * H + k) * PC + j * C + cs * 16 + ch] = acc[(a * H + k) * 16 + ch];
        }
      }
    });
  }
}

template <int LIN, int LSH, int LOUT, int H, int NR, int G, bool WW>
__global__ void __launch_bounds__(kBwdWaves * 64, 1) bwd_kernel(BwdParams p) {
  using PS = PathSet<LIN, LSH, LOUT>;
  using GR = Groups<PS::N>;
  constexpr int NP = PS::N;
  constexpr int NG = GR::count(G);
  static_assert(NR % 4 == 0 && H % 16 == 0, "unsupported shape");
  constexpr int WF = WaveLds<H>::floats + gather_slots<PS, G>() * 256;
  extern __shared__ float smem[];
  constexpr int CS = H + 4;
  float* w2s = smem;                                      // [NG][H][kRS] W2 slice of the group
  float* w2c = w2s + NG * H * kRS;                        // [NG][16][H + 4] the same, transposed
  float* wls = w2c + NG * 16 * CS;                        // per-wave scratch, WF floats each

  const int tid = threadIdx.x;
  const int cs = blockIdx.x % p.n_slices;
  const int wgi = blockIdx.x / p.n_slices;
  const int C = p.C;
  const int PC = NP * C;
  static_for<NP>([&](auto J) {
    constexpr int j = decltype(J)::value;
    if constexpr (GR::of(j) == G) {
      constexpr int a = GR::rank(j);
      for (int idx = tid; idx < H * 16; idx += kBwdWaves * 64) {
        const int k = idx >> 4, ch = idx & 15;
        const float v = p.W2[(size_t)k * PC + j * C + cs * 16 + ch];
        w2s[(a * H + k) * kRS + ch] = v;
        w2c[(a * 16 + ch) * CS + k] = v;
      }
    }
  });
  __syncthreads();
  const int lo = (int)((long long)wgi * p.n_edges / p.wg_per_slice);
  const int hi = (int)((long long)(wgi + 1) * p.n_edges / p.wg_per_slice);
  const int wave = tid >> 6;
  const int e_lo = lo + (int)((long long)(hi - lo) * wave / kBwdWaves);
  const int e_hi = lo + (int)((long long)(hi - lo) * (wave + 1) / kBwdWaves);
  bwd_wave<LIN, LSH, LOUT, H, NR, G, WW>(p, w2s, w2c, wls + wave * WF, w2s, cs, e_lo, e_hi);
}

template <int H>
constexpr size_t bwd_lds_bytes(int ng, int gather_slots) {
  return (size_t)(ng * H * kRS + ng * 16 * (H + 4) +
                  kBwdWaves * (WaveLds<H>::floats + gather_slots * 256)) * sizeof(float);
}

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

template <int L, int H, int G>
hipError_t bwd_group(const BwdParams& p, hipStream_t st) {
  using PS = PathSet<L, L, L>;
  constexpr int NG = Groups<PS::N>::count(G);
  if constexpr (NG == 0) {
    return hipSuccess;
  } else {
    const bool ww = p.dW1_part != nullptr || p.dW2_part != nullptr;
    auto kern = ww ? bwd_kernel<L, L, L, H, 8, G, true> : bwd_kernel<L, L, L, H, 8, G, false>;
    const size_t lds = bwd_lds_bytes<H>(NG, gather_slots<PS, G>());
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(p.wg_per_slice * p.n_slices), dim3(kBwdWaves * 64), lds, st, p);
    return hipGetLastError();
  }
}

template <int L, int H>
hipError_t bwd_one(const BwdParams& p, hipStream_t st) {
  hipError_t err;
  if ((err = bwd_group<L, H, 0>(p, st)) != hipSuccess) return err;
  if ((err = bwd_group<L, H, 1>(p, st)) != hipSuccess) return err;
  if ((err = bwd_group<L, H, 2>(p, st)) != hipSuccess) return err;
  return bwd_group<L, H, 3>(p, st);
}

}  // namespace

hipError_t launch_bwd(const ConvShape& s, const BwdParams& p, hipStream_t st) {
  if (s.n_radial != 8 || s.L_in != s.L_sh || s.L_in != s.L_out) return hipErrorInvalidValue;
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
  const int L = s.L_in;
  const int np = L == 0 ? 1 : L == 1 ? 4 : L == 2 ? 11 : 23;
  return np < kBwdWaves ? np : kBwdWaves;
}

int bwd_wg_per_slice(const ConvShape& s, int n_edges, int n_cu) {
  const int n_slices = s.C / 16;
  int wps = n_cu / n_slices;  // one work-group per CU (LDS-bound)
  if (wps < 1) wps = 1;
  const int max_by_edges = (n_edges + 255) / 256;  // at least four tiles per wave
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

}  // namespace equitp
