// Fused edge-convolution segment kernel (gfx950).
//
// Forward: for every receiver d (one CSR segment of edges sorted by receiver),
//   out[d, l3, m3, c] = sum_{e -> d} sum_paths w_e[p, c] sum_{m1,m2} C_p[m1,m2,m3] x[src_e, l1, m1, c] Y_l2(u_e)[m2]
// with w_e = SiLU(e(r_e) W1) W2: the channelwise ("uvu") tensor product with one radial weight
// per path and channel, paths with the same l3 summed in-kernel (FlashCart, Fig. 3 caption:
// path-reduced products with a scalar weight per path and feature channel), summed over the
// segment in registers and stored once (fp32 throughout: "Fast and Accurate Foundation Models
// for Equivariant MLIPs", Sec. II).
//
// Transpose (gradient w.r.t. x): segments are senders (edge ids through a permutation), the
// gathered tensor is G[dst_e] and every CG block is applied transposed:
//   dx[s, l1, m1, c] = sum_{e: src_e = s} sum_paths w_e[p, c] sum_{m2,m3} C_p[m1,m2,m3] Y_l2[m2] G[dst_e, l3, m3, c].
//
// Work decomposition.  A work-group owns one 16-channel slice (blockIdx % n_slices, so that with
// 8 slices every XCD works on one slice and its L2 holds only that slice of the features) and a
// contiguous range of segments, handed to its waves through an LDS counter.  A wave walks its
// segment in tiles of 16 edges; lane = (edge slot es = lane % 16, channel quad q = lane / 16).
// For each path, the radial weights w[e, p, 16 channels] of the tile come from H/4 MFMA
// 16x16x4 f32 steps: A = W2 slice (staged once per work-group in LDS, laid out so each lane
// reads its four K values with one ds_read_b128), B = the lane's own hidden activations.  The
// MFMA result lands exactly where the tensor product needs it (lane = edge es, channels
// 4q..4q+3), so w never leaves registers.  The tensor product is fp32 VALU with the CG sparsity
// unrolled at compile time and the CG values compiled in as instruction literals (no loads).  At
// the end of a segment the 16 edge slots are summed with DPP row reductions (no atomics) and
// one float4 per lane and component is stored.
#include "common.h"
#include "params.h"

namespace equitp {
namespace {

// Waves per work-group: as many as the registers allow at two (l = 3), three (l = 2: at most 168
// VGPRs per wave) or four (l <= 1: at most 128) waves per SIMD, so that one wave's gather and LDS
// latencies are covered by the others' work.  (The work-group size is the whole occupancy: one
// work-group per CU.)
template <int L>
constexpr int seg_waves() { return L >= 3 ? 8 : L == 2 ? 12 : 16; }

// BF: the W2 contraction takes bf16 operands (W2 and h rounded to nearest even) with fp32
// accumulation, on v_mfma_f32_16x16x16_bf16 (four K steps of 16 instead of sixteen of 4).
// MASK: per-edge path subsets (p.path_mask, bit j = path j is computed for the edge): a path no
// edge of the tile needs is skipped for the whole tile (radial-weight MFMAs and tensor product),
// and for an edge without the path its radial weights are zero.  The paths then run one after
// another instead of software-pipelined, since each may be skipped.
template <int LIN, int LSH, int LOUT, int H, int NR, bool TRANS, bool BF, bool MASK>
__global__ void __launch_bounds__(seg_waves<LIN>() * 64) seg_conv_kernel(SegParams p) {
  using PS = PathSet<LIN, LSH, LOUT>;
  constexpr int NP = PS::N;
  constexpr int FIN = (LIN + 1) * (LIN + 1);
  constexpr int FSH = (LSH + 1) * (LSH + 1);
  constexpr int FOUT = (LOUT + 1) * (LOUT + 1);
  constexpr int FG = TRANS ? FOUT : FIN;   // components gathered per edge
  constexpr int FS = TRANS ? FIN : FOUT;   // components accumulated per segment
  constexpr int NSTEP = H / 4;             // MFMA K steps
  constexpr int NJ = H / 16;               // groups of four K steps (one ds_read_b128 each)
  static_assert(H % 16 == 0 && FS <= 16, "unsupported shape");

  static_assert(NR % 4 == 0, "n_radial must be a multiple of 4");
  extern __shared__ float smem[];
  float* w2s = smem;                   // [NP][NJ][64 lanes][4] fp32, or (BF) [NP][NJ][64 lanes] u2
  __shared__ int next_seg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int es = lane & 15;
  const int q = lane >> 4;
  const int cs = blockIdx.x % p.n_slices;
  const int wgi = blockIdx.x / p.n_slices;
  const int C = p.C;
  const int PC = NP * C;

  // W2 slice: element i of w2s[j][jj][kk*16 + ch] = W2[k = 16 jj + 4 kk + i][j*C + cs*16 + ch]
  if constexpr (!BF) {
    for (int idx = tid; idx < NP * H * 16; idx += blockDim.x) {
      const int ch = idx & 15;
      const int k = (idx >> 4) % H;
      const int j = (idx >> 4) / H;
      const float v = p.W2[(size_t)k * PC + j * C + cs * 16 + ch];
      const int jj = k >> 4, kk = (k >> 2) & 3, i = k & 3;
      w2s[((j * NJ + jj) * 64 + kk * 16 + ch) * 4 + i] = v;
    }
  } else {
    u2* w2b = reinterpret_cast<u2*>(smem);
    for (int idx = tid; idx < NP * NJ * 64; idx += blockDim.x) {
      const int ln = idx & 63, ch = ln & 15, kk = ln >> 4;
      const int jj = (idx >> 6) % NJ, j = (idx >> 6) / NJ;
      const float* src = p.W2 + (size_t)(16 * jj + 4 * kk) * PC + j * C + cs * 16 + ch;
      w2b[idx] = u2{pk_bf16(src[0], src[PC]), pk_bf16(src[2 * (size_t)PC], src[3 * (size_t)PC])};
    }
  }
  float w1a[NJ][NR / 4];
  load_w1_operands<H, NR>(p.W1, es, q, w1a);
  const int seg_lo = (int)((long long)wgi * p.n_seg / p.wg_per_slice);
  const int seg_hi = (int)((long long)(wgi + 1) * p.n_seg / p.wg_per_slice);
  if (tid == 0) next_seg = seg_lo;
  __syncthreads();

  const float inv_rc = p.inv_r_cut;
  const float pref = p.radial_pref;
  const int chan = cs * 16 + 4 * q;

  for (;;) {
    int seg = 0;
    if (lane == 0) seg = atomicAdd(&next_seg, 1);
    seg = __shfl(seg, 0, 64);
    if (seg >= seg_hi) break;

    f4 acc[FS];
#pragma unroll
    for (int c = 0; c < FS; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};

    const int e_beg = p.seg_ptr[seg];
    const int e_end = p.seg_ptr[seg + 1];
    for (int base = e_beg; base < e_end; base += 16) {
      const int pos = base + es;
      const bool valid = pos < e_end;
      float vx = 1.0f, vy = 0.0f, vz = 0.0f;
      int g = 0;
      uint32_t me = 0;   // MASK: paths computed for this lane's edge
      if (valid) {
        const int e = p.seg_edge ? p.seg_edge[pos] : pos;
        vx = p.vec[3 * (size_t)e + 0];
        vy = p.vec[3 * (size_t)e + 1];
        vz = p.vec[3 * (size_t)e + 2];
        g = p.gather[e];
        if constexpr (MASK) me = p.path_mask[e];
      }
      // MASK: paths any edge of the tile needs (the 16 edge slots; the four channel quads hold
      // the same edges)
      uint32_t need = 0;
      if constexpr (MASK) {
        uint32_t t = me;
        t |= (uint32_t)__shfl_xor((int)t, 1, 64);
        t |= (uint32_t)__shfl_xor((int)t, 2, 64);
        t |= (uint32_t)__shfl_xor((int)t, 4, 64);
        t |= (uint32_t)__shfl_xor((int)t, 8, 64);
        need = __builtin_amdgcn_readfirstlane(t);
      }
      const float r = sqrtf(vx * vx + vy * vy + vz * vz);
      const float inv_r = 1.0f / r;
      float Y[FSH];
      sh_eval<LSH, float>(vx * inv_r, vy * inv_r, vz * inv_r, Y);
      float eb[NR];
      radial_basis<NR>(r, inv_r, inv_rc, pref, eb, nullptr);
      if (!valid) {
#pragma unroll
        for (int n = 0; n < NR; ++n) eb[n] = 0.0f;
      }
      // hidden activations for this lane's K indices k(s) = 16 (s/4) + 4 q + s % 4
      float hb[NSTEP];
      hidden_layer<H, NR>(w1a, eb, q, hb);
      // keep the per-path W2 operand reads inside this loop (see opaque())
      const float* w2t = w2s + opaque(0);
      f4 xin[FG];
      const float* fp = p.feat + (size_t)g * FG * C + chan;
#pragma unroll
      for (int c = 0; c < FG; ++c) xin[c] = valid ? ld4(fp + (size_t)c * C) : f4{0.f, 0.f, 0.f, 0.f};

      // bf16 B operands: the lane's four K values per group of four steps
      u2 hbf[NJ];
      if constexpr (BF) {
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          hbf[jj] = pk4_bf16(f4{hb[4 * jj], hb[4 * jj + 1], hb[4 * jj + 2], hb[4 * jj + 3]});
      }
      // W2 operands of path j (NJ ds_read_b128, or NJ ds_read_b64 of bf16) and the radial
      // weights of path j for this tile (w[channel 4q + i] of edge es: H/4 MFMA 16x16x4 steps,
      // or H/16 bf16 16x16x16 steps).
      auto aload = [&](auto Jc, f4 (&ops)[NJ], u2 (&opb)[NJ]) {
        constexpr int jn = decltype(Jc)::value;
        static_for<NJ>([&](auto JJ) {
          constexpr int jj = decltype(JJ)::value;
          if constexpr (BF)
            opb[jj] = *reinterpret_cast<const u2*>(&w2t[((jn * NJ + jj) * 64 + lane) * 2]);
          else
            ops[jj] = ld4(&w2t[((jn * NJ + jj) * 64 + lane) * 4]);
        });
      };
      auto wchain = [&](const f4 (&ops)[NJ], const u2 (&opb)[NJ]) {
        f4 acc;
        if constexpr (BF) {
          acc = f4{0.f, 0.f, 0.f, 0.f};
          static_for<NJ>([&](auto JJ) {
            constexpr int jj = decltype(JJ)::value;
            acc = mfma_bf16(opb[jj], hbf[jj], acc);
          });
        } else {
          acc = f4{0.f, 0.f, 0.f, 0.f};
          static_for<NJ>([&](auto JJ) {
            constexpr int jj = decltype(JJ)::value;
            acc = mfma_16x16x4(ops[jj][0], hb[4 * jj + 0], acc);
            acc = mfma_16x16x4(ops[jj][1], hb[4 * jj + 1], acc);
            acc = mfma_16x16x4(ops[jj][2], hb[4 * jj + 2], acc);
            acc = mfma_16x16x4(ops[jj][3], hb[4 * jj + 3], acc);
          });
        }
        return acc;
      };
      // Tensor product of path J with radial weights w (lane: edge es, channels 4q..4q+3),
      // accumulated into acc.
      auto tp_path = [&](auto J, const f4 w) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        constexpr int gp = PS::id(j);
        constexpr int l1 = cg::kPaths[gp].l1;
        constexpr int l2 = cg::kPaths[gp].l2;
        constexpr int l3 = cg::kPaths[gp].l3;
        constexpr int off = cg::kPaths[gp].off;
        constexpr int nnz = cg::kPaths[gp].nnz;
        if constexpr (!TRANS) {
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
                acc[l3 * l3 + m3][i] += w[i] * t;
              });
            }
          });
        } else {
          static_for<2 * l1 + 1>([&](auto M1) {
            constexpr int m1 = decltype(M1)::value;
            constexpr int fm3 = cg_first_m3(gp, m1);
            if constexpr (fm3 >= 0) {
              float mr[2 * l3 + 1];
              static_for<nnz>([&](auto K) {
                constexpr int k = decltype(K)::value;
                constexpr cg::Ent en = cg::kEnt[off + k];
                if constexpr (en.m1 == m1) {
                  const float v = cg::kVal[off + k] * Y[l2 * l2 + en.m2];
                  if constexpr (cg_first_in_pair(gp, k)) mr[en.m3] = v;
                  else mr[en.m3] += v;
                }
              });
              static_for<4>([&](auto I) {
                constexpr int i = decltype(I)::value;
                float t = 0.0f;
                static_for<2 * l3 + 1>([&](auto M3) {
                  constexpr int m3 = decltype(M3)::value;
                  if constexpr (m3 == fm3) t = mr[m3] * xin[l3 * l3 + m3][i];
                  else if constexpr (cg_has(gp, m1, m3)) t += mr[m3] * xin[l3 * l3 + m3][i];
                });
                acc[l1 * l1 + m1][i] += w[i] * t;
              });
            }
          });
        }
      };
      if constexpr (MASK) {
        static_for<NP>([&](auto J) {
          constexpr int j = decltype(J)::value;
          if (need & (1u << j)) {
            f4 ops1[NJ];
            u2 opb1[NJ];
            aload(J, ops1, opb1);
            f4 w = wchain(ops1, opb1);
            if (!((me >> j) & 1u)) w = f4{0.f, 0.f, 0.f, 0.f};
            tp_path(J, w);
          }
        });
      } else {
      // Software pipeline over paths.  In the scheduling region of path j: the MFMA chain of path
      // j + 1 (its W2 operands were read one region earlier, so no LDS wait), the LDS reads of
      // path j + 2's operands, and the VALU tensor product of path j, interleaved so that the
      // matrix cores, the LDS and the vector ALU work at the same time within one wave.
      f4 ops[2][NJ];
      u2 opb[2][NJ];
      f4 wbuf[2];
      aload(std::integral_constant<int, 0>{}, ops[0], opb[0]);
      wbuf[0] = wchain(ops[0], opb[0]);
      if constexpr (NP > 1) aload(std::integral_constant<int, 1>{}, ops[1], opb[1]);
      static_for<NP>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int gp = PS::id(j);
        constexpr int l3 = cg::kPaths[gp].l3;
        constexpr int nnz = cg::kPaths[gp].nnz;
        if constexpr (j + 1 < NP) wbuf[(j + 1) & 1] = wchain(ops[(j + 1) & 1], opb[(j + 1) & 1]);
        if constexpr (j + 2 < NP) aload(std::integral_constant<int, j + 2>{}, ops[j & 1], opb[j & 1]);
        tp_path(J, wbuf[j & 1]);
        if constexpr (j + 1 < NP) {
          // one MFMA of the next path's chain, then a share of this path's VALU work
          constexpr int npairs = [] {
            int n = 0;
            for (int a = 0; a < 2 * cg::kPaths[gp].l1 + 1; ++a)
              for (int b = 0; b < 2 * cg::kPaths[gp].l3 + 1; ++b) n += cg_has(gp, a, b) ? 1 : 0;
            return n;
          }();
          constexpr int nvalu = 4 * (npairs + 2 * l3 + 1) + nnz;
          constexpr int NMF = BF ? NJ : NSTEP;  // MFMAs in a chain
          constexpr int per = (nvalu + NMF - 1) / NMF;
          __builtin_amdgcn_sched_group_barrier(0x100, NJ, 0);
          static_for<NMF>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, per, 0);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      }
    }

    // Sum the 16 edge slots of each channel quad; lane es stores component es.
    float* op = p.out + (size_t)seg * FS * C + chan;
    static_for<FS>([&](auto Cc) {
      constexpr int c = decltype(Cc)::value;
      f4 v = acc[c];
      v[0] = row16_sum(v[0]);
      v[1] = row16_sum(v[1]);
      v[2] = row16_sum(v[2]);
      v[3] = row16_sum(v[3]);
      if (es == c) st4(op + (size_t)c * C, v);
    });
  }
}

template <int LIN, int LSH, int LOUT, int H, int NR, bool TRANS, bool BF, bool MASK = false>
hipError_t launch_one(const SegParams& p0, int n_cu, hipStream_t stream) {
  using PS = PathSet<LIN, LSH, LOUT>;
  auto kern = seg_conv_kernel<LIN, LSH, LOUT, H, NR, TRANS, BF, MASK>;
  const size_t lds = (size_t)(PS::N * H * 16) * (BF ? 2 : 4);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  constexpr int threads = seg_waves<LIN>() * 64;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  SegParams p = p0;
  const int total = n_cu * per_cu;
  int wps = total / p.n_slices;
  if (wps < 1) wps = 1;
  if (wps > p.n_seg) wps = p.n_seg;
  if (wps < 1) return hipSuccess;  // no segments
  p.wg_per_slice = wps;
  hipLaunchKernelGGL(kern, dim3(wps * p.n_slices), dim3(threads), lds, stream, p);
  return hipGetLastError();
}

#if !EQUITP_MASKED
template <bool TRANS>
hipError_t dispatch(const ConvShape& s, const SegParams& p, int n_cu, hipStream_t st) {
  const int L = s.L_in;
  if (s.n_radial != 8) return hipErrorInvalidValue;
  if (s.mlp_bf16) {
    // bf16 operands for the radial-MLP contraction: width 64, l = 1..3
    if (s.hidden != 64) return hipErrorInvalidValue;
    switch (L) {
      case 1: return launch_one<1, 1, 1, 64, 8, TRANS, true>(p, n_cu, st);
      case 2: return launch_one<2, 2, 2, 64, 8, TRANS, true>(p, n_cu, st);
      case 3: return launch_one<3, 3, 3, 64, 8, TRANS, true>(p, n_cu, st);
    }
    return hipErrorInvalidValue;
  }
  if (s.hidden == 64) {
    switch (L) {
      case 0: return launch_one<0, 0, 0, 64, 8, TRANS, false>(p, n_cu, st);
      case 1: return launch_one<1, 1, 1, 64, 8, TRANS, false>(p, n_cu, st);
      case 2: return launch_one<2, 2, 2, 64, 8, TRANS, false>(p, n_cu, st);
      case 3: return launch_one<3, 3, 3, 64, 8, TRANS, false>(p, n_cu, st);
    }
  } else if (s.hidden == 16) {
    switch (L) {
      case 0: return launch_one<0, 0, 0, 16, 8, TRANS, false>(p, n_cu, st);
      case 1: return launch_one<1, 1, 1, 16, 8, TRANS, false>(p, n_cu, st);
      case 2: return launch_one<2, 2, 2, 16, 8, TRANS, false>(p, n_cu, st);
      case 3: return launch_one<3, 3, 3, 16, 8, TRANS, false>(p, n_cu, st);
    }
  }
  return hipErrorInvalidValue;
}
#else
// per-edge path subsets: fp32, hidden width 64, l = 1..3
template <bool TRANS>
hipError_t dispatch_masked(const ConvShape& s, const SegParams& p, int n_cu, hipStream_t st) {
  if (s.n_radial != 8 || s.hidden != 64 || s.mlp_bf16) return hipErrorInvalidValue;
  switch (s.L_in) {
    case 1: return launch_one<1, 1, 1, 64, 8, TRANS, false, true>(p, n_cu, st);
    case 2: return launch_one<2, 2, 2, 64, 8, TRANS, false, true>(p, n_cu, st);
    case 3: return launch_one<3, 3, 3, 64, 8, TRANS, false, true>(p, n_cu, st);
  }
  return hipErrorInvalidValue;
}
#endif

}  // namespace

#if !EQUITP_MASKED
hipError_t launch_seg_conv(const ConvShape& s, bool transpose, const SegParams& p, int n_cu,
                           hipStream_t stream) {
  if (s.L_in != s.L_sh || s.L_in != s.L_out) return hipErrorInvalidValue;
  return transpose ? dispatch<true>(s, p, n_cu, stream) : dispatch<false>(s, p, n_cu, stream);
}
#else
hipError_t launch_seg_conv_masked(const ConvShape& s, bool transpose, const SegParams& p, int n_cu,
                                  hipStream_t stream) {
  if (s.L_in != s.L_sh || s.L_in != s.L_out || p.path_mask == nullptr) return hipErrorInvalidValue;
  return transpose ? dispatch_masked<true>(s, p, n_cu, stream)
                   : dispatch_masked<false>(s, p, n_cu, stream);
}
#endif

}  // namespace equitp
