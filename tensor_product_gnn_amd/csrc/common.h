// Device-side helpers shared by the edge-convolution kernels: compile-time path sets, the
// radial basis, SiLU, MFMA and cross-lane wrappers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "cg_table.h"
#include "sh.h"

namespace equitp {

typedef float f4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ compile-time iteration
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------------ path sets
// Paths of a configuration: every global path (cg_table.h, lexicographic) with l1 <= LIN,
// l2 <= LSH, l3 <= LOUT, in the same order.  W2 columns are p * C + channel in this order.
template <int LIN, int LSH, int LOUT>
struct PathSet {
  static constexpr bool in(int gp) {
    return cg::kPaths[gp].l1 <= LIN && cg::kPaths[gp].l2 <= LSH && cg::kPaths[gp].l3 <= LOUT;
  }
  static constexpr int count() {
    int n = 0;
    for (int i = 0; i < cg::kNumPaths; ++i) n += in(i) ? 1 : 0;
    return n;
  }
  static constexpr int N = count();
  static constexpr int id(int j) {
    int n = 0;
    for (int i = 0; i < cg::kNumPaths; ++i)
      if (in(i)) {
        if (n == j) return i;
        ++n;
      }
    return -1;
  }
};

// Whether path gp has an entry with this (m1, m3); whether entry k is the first of its
// (m1, m3) group; the first m1 of column m3; the first m3 of row m1.
constexpr bool cg_has(int gp, int m1, int m3) {
  for (int k = 0; k < cg::kPaths[gp].nnz; ++k) {
    const cg::Ent e = cg::kEnt[cg::kPaths[gp].off + k];
    if (e.m1 == m1 && e.m3 == m3) return true;
  }
  return false;
}
constexpr bool cg_first_in_pair(int gp, int k) {
  const cg::Ent e = cg::kEnt[cg::kPaths[gp].off + k];
  for (int j = 0; j < k; ++j) {
    const cg::Ent f = cg::kEnt[cg::kPaths[gp].off + j];
    if (f.m1 == e.m1 && f.m3 == e.m3) return false;
  }
  return true;
}
constexpr int cg_first_m1(int gp, int m3) {
  for (int m1 = 0; m1 < 2 * cg::kPaths[gp].l1 + 1; ++m1)
    if (cg_has(gp, m1, m3)) return m1;
  return -1;
}
constexpr int cg_first_m3(int gp, int m1) {
  for (int m3 = 0; m3 < 2 * cg::kPaths[gp].l3 + 1; ++m3)
    if (cg_has(gp, m1, m3)) return m3;
  return -1;
}

// ------------------------------------------------------------------ math helpers
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Bessel radial basis times the polynomial envelope:
//   e_n(r) = sqrt(2 / r_c) * sin(n pi r / r_c) / r * f(r / r_c),  n = 1..NR,
//   f(t) = 1 - 28 t^6 + 48 t^7 - 21 t^8 for t < 1, else 0.
// sin(pi t) and cos(pi t) for t in [0, 1]; t is clamped to that range (beyond the cutoff the
// envelope is zero and the value is unused).  With y = pi min(t, 1 - t) in [0, pi/2]:
// sin(pi t) = sin y and cos(pi t) = +-cos y, both from their Taylor series (the first omitted terms
// are below 6e-8 on [0, pi/2]); about twenty FMAs instead of a general range-reduced sincos.
__device__ __forceinline__ void sincos_pi01(float t, float& s, float& c) {
  t = fminf(fmaxf(t, 0.0f), 1.0f);
  const bool upper = t > 0.5f;
  const float y = 3.14159265358979f * (upper ? 1.0f - t : t);
  const float y2 = y * y;
  float sp = -1.0f / 39916800.0f;            // sin y = y (1 - y^2/3! + ... - y^10/11!)
  sp = sp * y2 + 1.0f / 362880.0f;
  sp = sp * y2 - 1.0f / 5040.0f;
  sp = sp * y2 + 1.0f / 120.0f;
  sp = sp * y2 - 1.0f / 6.0f;
  sp = sp * y2 + 1.0f;
  float cp = 1.0f / 479001600.0f;            // cos y = 1 - y^2/2! + ... + y^12/12!
  cp = cp * y2 - 1.0f / 3628800.0f;
  cp = cp * y2 + 1.0f / 40320.0f;
  cp = cp * y2 - 1.0f / 720.0f;
  cp = cp * y2 + 1.0f / 24.0f;
  cp = cp * y2 - 0.5f;
  cp = cp * y2 + 1.0f;
  s = sp * y;
  c = upper ? -cp : cp;
}

// sin(n theta), cos(n theta) by the angle-addition recurrence from sin(theta), cos(theta).  If
// de != nullptr also returns d e_n / d r.
// inv_r_cut = 1 / r_c and pref = sqrt(2 / r_c) come precomputed (kernel arguments).
template <int NR>
__device__ __forceinline__ void radial_basis(float r, float inv_r, float inv_r_cut, float pref,
                                             float* e, float* de) {
  const float t = r * inv_r_cut;
  float sn[NR], cn[NR];
  float s1, c1;
  sincos_pi01(t, s1, c1);
  sn[0] = s1;
  cn[0] = c1;
#pragma unroll
  for (int n = 1; n < NR; ++n) {
    // sin((n+1)x) = sin(nx) cos x + cos(nx) sin x ; cos((n+1)x) = cos(nx) cos x - sin(nx) sin x
    sn[n] = sn[n - 1] * c1 + cn[n - 1] * s1;
    cn[n] = cn[n - 1] * c1 - sn[n - 1] * s1;
  }
  const float t2 = t * t, t3 = t2 * t, t5 = t2 * t3, t6 = t3 * t3;
  const bool inside = t < 1.0f;
  const float f = inside ? 1.0f + t6 * (-28.0f + t * (48.0f - 21.0f * t)) : 0.0f;
#pragma unroll
  for (int n = 0; n < NR; ++n) e[n] = pref * sn[n] * inv_r * f;
  if (de != nullptr) {
    const float df = inside ? t5 * (-168.0f + t * (336.0f - 168.0f * t)) * inv_r_cut : 0.0f;
    const float kscale = 3.14159265358979f * inv_r_cut;
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      const float k = kscale * float(n + 1);
      const float B = pref * sn[n] * inv_r;
      const float dB = pref * (k * cn[n] * inv_r - sn[n] * inv_r * inv_r);
      de[n] = dB * f + B * df;
    }
  }
}

// ------------------------------------------------------------------ bf16 operands
// Four bf16 values in two registers: element t of an MFMA 16x16x16 operand is bits 16 t .. 16 t + 15.
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef short s4v __attribute__((ext_vector_type(4)));

// (a, b) rounded to bf16 (round to nearest even), a in the low half.  One instruction (the
// compiler's own conversion takes three per pair).  The compiler does not count an inline-asm
// VALU write when it pads the wait states an MFMA operand read needs after a VALU write (two on
// gfx950; an operand read one instruction after this convert was measured to get stale data),
// so the asm pads them itself.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2\n\ts_nop 2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ u2 pk4_bf16(f4 v) { return u2{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])}; }

// D = A B + C with A[i][k] from lane i + 16 (k / 4), B[k][j] from lane j + 16 (k / 4), element
// k % 4 of the lane's four bf16 values; D as for mfma_16x16x4 (layout checked on the GPU).
__device__ __forceinline__ f4 mfma_bf16(u2 a, u2 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4v, a),
                                                   __builtin_bit_cast(s4v, b), c, 0, 0, 0);
}

__device__ __forceinline__ f4 mfma_16x16x4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Sum over the four lanes {l, l^16, l^32, l^48}.
__device__ __forceinline__ float cross_row_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Hide a value from the optimiser, so that loads whose address depends on it stay inside the
// loop that issues them instead of being hoisted (and kept live in registers) ahead of it.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Hidden layer of the radial MLP for one 16-edge tile on the matrix cores:
//   pre[e, k] = sum_n e_n(r_e) W1[n, k],   h = SiLU(pre)
// as h^T = W1^T e^T with MFMA 16x16x4: A = W1^T (lane holds W1[4t + q][16 mt + es] in
// w1a[mt][t]), B = the lane's radial basis values e[n = 4t + q].  The output of m-tile mt lands in
// lane (edge es, quad q) as k = 16 mt + 4 q + r, i.e. hb[4 mt + r]: exactly the K index the lane
// supplies to the W2 contraction.
// Optionally also returns pre (pre_out) and SiLU'(pre) = s (1 + pre (1 - s)), s = sigmoid(pre)
// (dsilu_out).
template <int H, int NR>
__device__ __forceinline__ void hidden_layer(const float (&w1a)[H / 16][NR / 4], const float* eb,
                                             int q, float* hb, float* pre_out = nullptr,
                                             float* dsilu_out = nullptr) {
  float ebq[NR / 4];
#pragma unroll
  for (int t = 0; t < NR / 4; ++t)
    ebq[t] = q == 0 ? eb[4 * t] : q == 1 ? eb[4 * t + 1] : q == 2 ? eb[4 * t + 2] : eb[4 * t + 3];
#pragma unroll
  for (int mt = 0; mt < H / 16; ++mt) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NR / 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w1a[mt][t], ebq[t], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float z = acc[r];
      const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
      hb[4 * mt + r] = z * sg;
      if (pre_out != nullptr) pre_out[4 * mt + r] = z;
      if (dsilu_out != nullptr) dsilu_out[4 * mt + r] = sg * (1.0f + z * (1.0f - sg));
    }
  }
}

template <int H, int NR>
__device__ __forceinline__ void load_w1_operands(const float* W1, int es, int q,
                                                 float (&w1a)[H / 16][NR / 4]) {
#pragma unroll
  for (int mt = 0; mt < H / 16; ++mt)
#pragma unroll
    for (int t = 0; t < NR / 4; ++t) w1a[mt][t] = W1[(4 * t + q) * H + 16 * mt + es];
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }

}  // namespace equitp
