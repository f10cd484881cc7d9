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
// Every sum is a register, MFMA or fixed-order tree sum: no atomics, so results are bitwise
// reproducible run to run.
#include "common.h"
#include "params.h"

namespace equitp {
namespace {

// ---------------------------------------------------------------------------------------------
// Kernel 1: per-edge dL/dY and dL/dh.  A wave owns a tile of 16 edges (lane = edge es, channel
// quad q) and walks all channel slices and all paths, so both reductions over channels finish
// in registers.  The work-group's 8 waves share one W2 slice at a time in LDS (row stride 20
// floats keeps both read patterns conflict-free).  Per path: w = MFMA(W2 slice, h) as in the
// forward; then dL/dh^T += MFMA(W2 slice, (dL/dw)^T), contracting over the 16 channels of the
// slice, so dL/dw never leaves registers either.
// ---------------------------------------------------------------------------------------------
constexpr int kEdgeWaves = 8;
constexpr int kRS = 20;

template <int LIN, int LSH, int LOUT, int H, int NR>
__global__ void __launch_bounds__(kEdgeWaves * 64) edge_bwd_kernel(EdgeBwdParams p) {
  using PS = PathSet<LIN, LSH, LOUT>;
  constexpr int NP = PS::N;
  constexpr int FIN = (LIN + 1) * (LIN + 1);
  constexpr int FSH = (LSH + 1) * (LSH + 1);
  constexpr int FOUT = (LOUT + 1) * (LOUT + 1);
  constexpr int NSTEP = H / 4;
  constexpr int NJ = H / 16;
  static_assert(NR % 4 == 0 && H % 16 == 0, "unsupported shape");

  extern __shared__ float smem[];
  float* w2l = smem;  // [NP][H][kRS]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int es = lane & 15;
  const int q = lane >> 4;
  const int C = p.C;
  const int PC = NP * C;
  const float r_cut = p.r_cut;
  const float inv_rc = 1.0f / r_cut;

  float w1a[NJ][NR / 4];
  load_w1_operands<H, NR>(p.W1, es, q, w1a);

  for (int tg = blockIdx.x; tg * (kEdgeWaves * 16) < p.n_edges; tg += gridDim.x) {
    const int e = tg * (kEdgeWaves * 16) + wave * 16 + es;
    const bool valid = e < p.n_edges;
    float vx = 1.0f, vy = 0.0f, vz = 0.0f;
    int s = 0, d = 0;
    if (valid) {
      vx = p.vec[3 * (size_t)e + 0];
      vy = p.vec[3 * (size_t)e + 1];
      vz = p.vec[3 * (size_t)e + 2];
      s = p.src[e];
      d = p.dst[e];
    }
    const float r = sqrtf(vx * vx + vy * vy + vz * vz);
    const float inv_r = 1.0f / r;
    float Y[FSH];
    sh_eval<LSH, float>(vx * inv_r, vy * inv_r, vz * inv_r, Y);
    float eb[NR];
    radial_basis<NR>(r, inv_r, r_cut, inv_rc, eb, nullptr);
    if (!valid) {
#pragma unroll
      for (int n = 0; n < NR; ++n) eb[n] = 0.0f;
    }
    float hb[NSTEP];
    hidden_layer<H, NR>(w1a, eb, q, hb);

    float dY[FSH];
#pragma unroll
    for (int i = 0; i < FSH; ++i) dY[i] = 0.0f;
    f4 dh[NJ];
#pragma unroll
    for (int mt = 0; mt < NJ; ++mt) dh[mt] = f4{0.f, 0.f, 0.f, 0.f};

    for (int cs = 0; cs < p.n_slices; ++cs) {
      __syncthreads();  // the previous slice's readers are done
      for (int idx = tid; idx < NP * H * 16; idx += blockDim.x) {
        const int ch = idx & 15;
        const int k = (idx >> 4) % H;
        const int j = (idx >> 4) / H;
        w2l[(j * H + k) * kRS + ch] = p.W2[(size_t)k * PC + j * C + cs * 16 + ch];
      }
      __syncthreads();
      const int chan = cs * 16 + 4 * q;
      f4 xin[FIN], gin[FOUT];
      const float* xp = p.x + (size_t)s * FIN * C + chan;
      const float* gpp = p.G + (size_t)d * FOUT * C + chan;
#pragma unroll
      for (int c = 0; c < FIN; ++c) xin[c] = valid ? ld4(xp + (size_t)c * C) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < FOUT; ++c) gin[c] = valid ? ld4(gpp + (size_t)c * C) : f4{0.f, 0.f, 0.f, 0.f};
      const float* w2t = w2l + opaque(0);

      static_for<NP>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int gp = PS::id(j);
        constexpr int l1 = cg::kPaths[gp].l1;
        constexpr int l2 = cg::kPaths[gp].l2;
        constexpr int l3 = cg::kPaths[gp].l3;
        constexpr int off = cg::kPaths[gp].off;
        constexpr int nnz = cg::kPaths[gp].nnz;
        // w[channel 4q + i] of edge es: A = W2[k(s, q')][ch = es'] from LDS, B = hb[s]
        f4 w = {0.f, 0.f, 0.f, 0.f};
        static_for<NSTEP>([&](auto S) {
          constexpr int st = decltype(S)::value;
          const int k = 16 * (st >> 2) + 4 * q + (st & 3);
          w = mfma_16x16x4(w2t[(j * H + k) * kRS + es], hb[st], w);
        });
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
            // dL/dY[m2] += C[m1,m2,m3] sum_c x[m1,c] w[c] G[m3,c]
            static_for<2 * l1 + 1>([&](auto M1) {
              constexpr int m1 = decltype(M1)::value;
              if constexpr (cg_has(gp, m1, m3)) {
                const f4 xv = xin[l1 * l1 + m1];
                const float a = xv[0] * wg[0] + xv[1] * wg[1] + xv[2] * wg[2] + xv[3] * wg[3];
                static_for<nnz>([&](auto K) {
                  constexpr int k = decltype(K)::value;
                  constexpr cg::Ent en = cg::kEnt[off + k];
                  if constexpr (en.m3 == m3 && en.m1 == m1) dY[l2 * l2 + en.m2] += cg::kVal[off + k] * a;
                });
              }
            });
          }
        });
        // dL/dh^T[k = 16 mt + 4q + r][e = es] += sum_{c in slice} W2[k][c] dL/dw[e][c]
        static_for<NJ>([&](auto MT) {
          constexpr int mt = decltype(MT)::value;
          const f4 b4 = ld4(&w2t[(j * H + 16 * mt + es) * kRS + 4 * q]);
          dh[mt] = mfma_16x16x4(b4[0], dw[0], dh[mt]);
          dh[mt] = mfma_16x16x4(b4[1], dw[1], dh[mt]);
          dh[mt] = mfma_16x16x4(b4[2], dw[2], dh[mt]);
          dh[mt] = mfma_16x16x4(b4[3], dw[3], dh[mt]);
        });
      });
    }

    // dL/dY: sum over the four channel quads
#pragma unroll
    for (int i = 0; i < FSH; ++i) dY[i] = cross_row_sum(dY[i]);
    if (valid) {
      if (q == 0) {
#pragma unroll
        for (int i = 0; i < FSH; ++i) p.dY[(size_t)e * FSH + i] = dY[i];
      }
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt) st4(p.dh + (size_t)e * H + 16 * mt + 4 * q, dh[mt]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Kernel 2: dL/dW2 = sum_e h_e^T dL/dw_e.  A work-group owns one channel slice and a contiguous
// edge range; its four waves own the paths j with j % 4 == wave, so each wave keeps the dW2
// accumulators of its paths (H x 16 per path) in registers for the whole range.  Per 16-edge
// tile: each wave computes dL/dw of its paths (VALU, lane = edge es, channels 4q..4q+3) and
// writes it to LDS; h of the tile is computed once (one 16-wide K quarter per wave) into LDS;
// then dW2 += h^T dL/dw on MFMA with the 16 edges as the contraction.  One partial per
// work-group goes to the workspace; a fixed-order row reduction sums them.
// ---------------------------------------------------------------------------------------------
constexpr int kDw2Waves = 4;

template <int LIN, int LSH, int LOUT, int H, int NR, int G>
__device__ __forceinline__ void dw2_group(const Dw2Params& p, float* ht, float* dwt, int e_lo,
                                          int e_hi, int cs, int wgi) {
  using PS = PathSet<LIN, LSH, LOUT>;
  constexpr int NP = PS::N;
  constexpr int FIN = (LIN + 1) * (LIN + 1);
  constexpr int FSH = (LSH + 1) * (LSH + 1);
  constexpr int FOUT = (LOUT + 1) * (LOUT + 1);
  constexpr int NJ = H / 16;
  constexpr int NPG = (NP + kDw2Waves - 1) / kDw2Waves;
  constexpr int HP = H + 16;  // h tile row stride
  constexpr int DS = 20;      // dL/dw tile row stride

  const int lane = threadIdx.x & 63;
  const int es = lane & 15;
  const int q = lane >> 4;
  const int C = p.C;
  const int PC = NP * C;
  const float r_cut = p.r_cut;
  const float inv_rc = 1.0f / r_cut;
  const int chan = cs * 16 + 4 * q;

  // This wave's quarter of the hidden layer: h[e][k], k = 16 G + 4 q + r.
  float w1g[NR / 4];
  if constexpr (G < NJ) {
#pragma unroll
    for (int t = 0; t < NR / 4; ++t) w1g[t] = p.W1[(4 * t + q) * H + 16 * G + es];
  }

  f4 acc[NPG][NJ];
#pragma unroll
  for (int a = 0; a < NPG; ++a)
#pragma unroll
    for (int mt = 0; mt < NJ; ++mt) acc[a][mt] = f4{0.f, 0.f, 0.f, 0.f};

  for (int base = e_lo; base < e_hi; base += 16) {
    const int e = base + es;
    const bool valid = e < e_hi;
    float vx = 1.0f, vy = 0.0f, vz = 0.0f;
    int s = 0, d = 0;
    if (valid) {
      vx = p.vec[3 * (size_t)e + 0];
      vy = p.vec[3 * (size_t)e + 1];
      vz = p.vec[3 * (size_t)e + 2];
      s = p.src[e];
      d = p.dst[e];
    }
    const float r = sqrtf(vx * vx + vy * vy + vz * vz);
    const float inv_r = 1.0f / r;
    float Y[FSH];
    sh_eval<LSH, float>(vx * inv_r, vy * inv_r, vz * inv_r, Y);
    if constexpr (G < NJ) {
      float eb[NR];
      radial_basis<NR>(r, inv_r, r_cut, inv_rc, eb, nullptr);
      float ebq[NR / 4];
#pragma unroll
      for (int t = 0; t < NR / 4; ++t) {
        const float v = q == 0 ? eb[4 * t] : q == 1 ? eb[4 * t + 1] : q == 2 ? eb[4 * t + 2] : eb[4 * t + 3];
        ebq[t] = valid ? v : 0.0f;
      }
      f4 pre = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NR / 4; ++t) pre = mfma_16x16x4(w1g[t], ebq[t], pre);
      st4(&ht[es * HP + 16 * G + 4 * q], f4{silu(pre[0]), silu(pre[1]), silu(pre[2]), silu(pre[3])});
    }
    f4 xin[FIN], gin[FOUT];
    const float* xp = p.x + (size_t)s * FIN * C + chan;
    const float* gpp = p.G + (size_t)d * FOUT * C + chan;
#pragma unroll
    for (int c = 0; c < FIN; ++c) xin[c] = valid ? ld4(xp + (size_t)c * C) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < FOUT; ++c) gin[c] = valid ? ld4(gpp + (size_t)c * C) : f4{0.f, 0.f, 0.f, 0.f};

    static_for<NP>([&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (j % kDw2Waves == G) {
        constexpr int gp = PS::id(j);
        constexpr int l1 = cg::kPaths[gp].l1;
        constexpr int l2 = cg::kPaths[gp].l2;
        constexpr int l3 = cg::kPaths[gp].l3;
        constexpr int off = cg::kPaths[gp].off;
        constexpr int nnz = cg::kPaths[gp].nnz;
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
            static_for<4>([&](auto I) {
              constexpr int i = decltype(I)::value;
              float t = 0.0f;
              static_for<2 * l1 + 1>([&](auto M1) {
                constexpr int m1 = decltype(M1)::value;
                if constexpr (m1 == fm1) t = mc[m1] * xin[l1 * l1 + m1][i];
                else if constexpr (cg_has(gp, m1, m3)) t += mc[m1] * xin[l1 * l1 + m1][i];
              });
              dw[i] += gin[l3 * l3 + m3][i] * t;
            });
          }
        });
        st4(&dwt[((j / kDw2Waves) * 16 + es) * DS + 4 * q], dw);
      }
    });
    __syncthreads();
    // dW2[k = 16 mt + 4q + r][c = es] += sum_{e in tile} h[e][k] dL/dw[e][c]
    static_for<NP>([&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (j % kDw2Waves == G) {
        constexpr int a = j / kDw2Waves;
        static_for<4>([&](auto S) {
          constexpr int st = decltype(S)::value;
          const float b = dwt[(a * 16 + 4 * st + q) * DS + es];
          static_for<NJ>([&](auto MT) {
            constexpr int mt = decltype(MT)::value;
            acc[a][mt] = mfma_16x16x4(ht[(4 * st + q) * HP + 16 * mt + es], b, acc[a][mt]);
          });
        });
      }
    });
    __syncthreads();
  }
  static_for<NP>([&](auto J) {
    constexpr int j = decltype(J)::value;
    if constexpr (j % kDw2Waves == G) {
      constexpr int a = j / kDw2Waves;
#pragma unroll
      for (int mt = 0; mt < NJ; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          p.part[((size_t)wgi * H + 16 * mt + 4 * q + r) * PC + j * C + cs * 16 + es] = acc[a][mt][r];
    }
  });
}

template <int LIN, int LSH, int LOUT, int H, int NR>
__global__ void __launch_bounds__(kDw2Waves * 64) dw2_kernel(Dw2Params p) {
  using PS = PathSet<LIN, LSH, LOUT>;
  constexpr int NPG = (PS::N + kDw2Waves - 1) / kDw2Waves;
  __shared__ float ht[16 * (H + 16)];
  __shared__ float dwt[kDw2Waves * NPG * 16 * 20];
  const int cs = blockIdx.x % p.n_slices;
  const int wgi = blockIdx.x / p.n_slices;
  const int e_lo = (int)((long long)wgi * p.n_edges / p.wg_per_slice);
  const int e_hi = (int)((long long)(wgi + 1) * p.n_edges / p.wg_per_slice);
  const int wave = threadIdx.x >> 6;
  float* dw_w = dwt + wave * NPG * 16 * 20;
  if (wave == 0) dw2_group<LIN, LSH, LOUT, H, NR, 0>(p, ht, dw_w, e_lo, e_hi, cs, wgi);
  else if (wave == 1) dw2_group<LIN, LSH, LOUT, H, NR, 1>(p, ht, dw_w, e_lo, e_hi, cs, wgi);
  else if (wave == 2) dw2_group<LIN, LSH, LOUT, H, NR, 2>(p, ht, dw_w, e_lo, e_hi, cs, wgi);
  else dw2_group<LIN, LSH, LOUT, H, NR, 3>(p, ht, dw_w, e_lo, e_hi, cs, wgi);
}

// ---------------------------------------------------------------------------------------------
// Kernel 3: per-edge finish.  Thread = edge: dL/dpre = dL/dh * SiLU'(pre), dL/de = dL/dpre W1^T,
// dL/dr = sum_n dL/de_n de_n/dr, and dL/dvec.  Then the block's 128 edges contribute
// e^T dL/dpre to its dW1 partial (threads switch to (n, k) pairs, fixed summation order).
// ---------------------------------------------------------------------------------------------
constexpr int kPostThreads = 128;

template <int LSH, int H, int NR>
__global__ void __launch_bounds__(kPostThreads) edge_post_kernel(EdgePostParams p) {
  constexpr int FSH = (LSH + 1) * (LSH + 1);
  constexpr int PAIRS = NR * H;
  constexpr int PPT = (PAIRS + kPostThreads - 1) / kPostThreads;
  __shared__ float w1s[NR * H];
  __shared__ float dps[kPostThreads * (H + 1)];
  __shared__ float ebs[kPostThreads * (NR + 1)];
  const int t = threadIdx.x;
  for (int i = t; i < NR * H; i += kPostThreads) w1s[i] = p.W1[i];
  const float r_cut = p.r_cut;
  const float inv_rc = 1.0f / r_cut;
  float accw[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) accw[i] = 0.0f;
  __syncthreads();

  for (int chunk = blockIdx.x; chunk * kPostThreads < p.n_edges; chunk += gridDim.x) {
    const int e = chunk * kPostThreads + t;
    const bool valid = e < p.n_edges;
    if (valid) {
      const float vx = p.vec[3 * (size_t)e + 0];
      const float vy = p.vec[3 * (size_t)e + 1];
      const float vz = p.vec[3 * (size_t)e + 2];
      const float r = sqrtf(vx * vx + vy * vy + vz * vz);
      const float inv_r = 1.0f / r;
      const float ux = vx * inv_r, uy = vy * inv_r, uz = vz * inv_r;
      float eb[NR], deb[NR];
      radial_basis<NR>(r, inv_r, r_cut, inv_rc, eb, deb);
      float de[NR];
#pragma unroll
      for (int n = 0; n < NR; ++n) de[n] = 0.0f;
      const float* dhp = p.dh + (size_t)e * H;
#pragma unroll 4
      for (int k4 = 0; k4 < H; k4 += 4) {
        const f4 dh4 = ld4(dhp + k4);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int k = k4 + r4;
          float pre = 0.0f;
#pragma unroll
          for (int n = 0; n < NR; ++n) pre += eb[n] * w1s[n * H + k];
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-pre));
          const float dpre = dh4[r4] * sg * (1.0f + pre * (1.0f - sg));
          dps[t * (H + 1) + k] = dpre;
#pragma unroll
          for (int n = 0; n < NR; ++n) de[n] += dpre * w1s[n * H + k];
        }
      }
#pragma unroll
      for (int n = 0; n < NR; ++n) ebs[t * (NR + 1) + n] = eb[n];
      if (p.dvec != nullptr) {
        float dr = 0.0f;
#pragma unroll
        for (int n = 0; n < NR; ++n) dr += de[n] * deb[n];
        float dY[FSH];
#pragma unroll
        for (int i = 0; i < FSH; ++i) dY[i] = p.dY[(size_t)e * FSH + i];
        float gx, gy, gz;
        sh_vjp<LSH, float>(ux, uy, uz, dY, gx, gy, gz);
        const float gu = gx * ux + gy * uy + gz * uz;
        p.dvec[3 * (size_t)e + 0] = dr * ux + (gx - gu * ux) * inv_r;
        p.dvec[3 * (size_t)e + 1] = dr * uy + (gy - gu * uy) * inv_r;
        p.dvec[3 * (size_t)e + 2] = dr * uz + (gz - gu * uz) * inv_r;
      }
    } else {
      for (int k = 0; k < H; ++k) dps[t * (H + 1) + k] = 0.0f;
#pragma unroll
      for (int n = 0; n < NR; ++n) ebs[t * (NR + 1) + n] = 0.0f;
    }
    __syncthreads();
    if (p.dW1_part != nullptr) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pr = t + i * kPostThreads;
        if (pr < PAIRS) {
          const int n = pr / H, k = pr % H;
          float a = accw[i];
          for (int tt = 0; tt < kPostThreads; ++tt) a += ebs[tt * (NR + 1) + n] * dps[tt * (H + 1) + k];
          accw[i] = a;
        }
      }
    }
    __syncthreads();
  }
  if (p.dW1_part != nullptr) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pr = t + i * kPostThreads;
      if (pr < PAIRS) p.dW1_part[(size_t)blockIdx.x * PAIRS + pr] = accw[i];
    }
  }
}

// out[c] = sum_r part[r][c], rows summed in order (deterministic).
__global__ void reduce_rows_kernel(const float* __restrict__ part, int rows, int cols,
                                   float* __restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int r = 0;
  for (; r + 4 <= rows; r += 4) {
    a0 += part[(size_t)(r + 0) * cols + c];
    a1 += part[(size_t)(r + 1) * cols + c];
    a2 += part[(size_t)(r + 2) * cols + c];
    a3 += part[(size_t)(r + 3) * cols + c];
  }
  for (; r < rows; ++r) a0 += part[(size_t)r * cols + c];
  out[c] = (a0 + a1) + (a2 + a3);
}

__global__ void fill_zero_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

template <int L, int H>
hipError_t edge_bwd_one(const EdgeBwdParams& p, int n_cu, hipStream_t st) {
  using PS = PathSet<L, L, L>;
  auto kern = edge_bwd_kernel<L, L, L, H, 8>;
  const size_t lds = (size_t)PS::N * H * kRS * sizeof(float);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kEdgeWaves * 64, lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  const int tiles = (p.n_edges + kEdgeWaves * 16 - 1) / (kEdgeWaves * 16);
  int grid = n_cu * per_cu;
  if (grid > tiles) grid = tiles;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kEdgeWaves * 64), lds, st, p);
  return hipGetLastError();
}

template <int L, int H>
hipError_t dw2_one(const Dw2Params& p, hipStream_t st) {
  hipLaunchKernelGGL((dw2_kernel<L, L, L, H, 8>), dim3(p.wg_per_slice * p.n_slices),
                     dim3(kDw2Waves * 64), 0, st, p);
  return hipGetLastError();
}

template <int L, int H>
hipError_t post_one(const EdgePostParams& p, int n_blocks, hipStream_t st) {
  hipLaunchKernelGGL((edge_post_kernel<L, H, 8>), dim3(n_blocks), dim3(kPostThreads), 0, st, p);
  return hipGetLastError();
}

#define EQUITP_DISPATCH_LH(FN, ...)                                     \
  do {                                                                  \
    if (s.n_radial != 8 || s.L_in != s.L_sh || s.L_in != s.L_out)       \
      return hipErrorInvalidValue;                                      \
    if (s.hidden == 64) {                                               \
      switch (s.L_in) {                                                 \
        case 0: return FN<0, 64>(__VA_ARGS__);                          \
        case 1: return FN<1, 64>(__VA_ARGS__);                          \
        case 2: return FN<2, 64>(__VA_ARGS__);                          \
        case 3: return FN<3, 64>(__VA_ARGS__);                          \
      }                                                                 \
    } else if (s.hidden == 16) {                                        \
      switch (s.L_in) {                                                 \
        case 0: return FN<0, 16>(__VA_ARGS__);                          \
        case 1: return FN<1, 16>(__VA_ARGS__);                          \
        case 2: return FN<2, 16>(__VA_ARGS__);                          \
        case 3: return FN<3, 16>(__VA_ARGS__);                          \
      }                                                                 \
    }                                                                   \
    return hipErrorInvalidValue;                                        \
  } while (0)

}  // namespace

hipError_t launch_edge_bwd(const ConvShape& s, const EdgeBwdParams& p, int n_cu, hipStream_t st) {
  EQUITP_DISPATCH_LH(edge_bwd_one, p, n_cu, st);
}

int dw2_wg_per_slice(const ConvShape& s, int n_edges, int n_cu) {
  const int n_slices = s.C / 16;
  int wps = (2 * n_cu) / n_slices;
  if (wps < 1) wps = 1;
  const int max_by_edges = (n_edges + 63) / 64;  // at least four tiles per work-group
  if (wps > max_by_edges) wps = max_by_edges;
  if (wps < 1) wps = 1;
  return wps;
}

hipError_t launch_dw2(const ConvShape& s, const Dw2Params& p, int n_cu, hipStream_t st) {
  (void)n_cu;
  EQUITP_DISPATCH_LH(dw2_one, p, st);
}

int edge_post_blocks(int n_edges, int n_cu) {
  int chunks = (n_edges + kPostThreads - 1) / kPostThreads;
  int b = 2 * n_cu;
  if (b > chunks) b = chunks;
  return b < 1 ? 1 : b;
}

hipError_t launch_edge_post(const ConvShape& s, const EdgePostParams& p, int n_blocks,
                            hipStream_t st) {
  EQUITP_DISPATCH_LH(post_one, p, n_blocks, st);
}

hipError_t launch_reduce_rows(const float* part, int rows, int cols, float* out, hipStream_t st) {
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((cols + 255) / 256), dim3(256), 0, st, part, rows,
                     cols, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace equitp
