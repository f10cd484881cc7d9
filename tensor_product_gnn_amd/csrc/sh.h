// Real spherical harmonics for l <= 3, component normalisation (sum_m Y_lm^2 = 2l + 1,
// Y_0 = 1), m = -l..l, hand-expanded as polynomials of the unit vector (x, y, z).
//
// The pages this library follows ("Fast and Accurate Foundation Models for Equivariant MLIPs",
// Sec. VII; "FlashCart", Fig. 3) use spherical-harmonic edge features but print no formulas;
// the convention here is the standard real form with positive cos(m phi) / sin(|m| phi)
// prefactors, so that Y_1 = sqrt(3) (y, z, x).
//
// Shared by the device kernels (float) and the host CG-table generator (double).
#pragma once

#ifndef EQUITP_HD
#if defined(__HIPCC__)
#define EQUITP_HD __host__ __device__ __forceinline__
#else
#define EQUITP_HD inline
#endif
#endif

namespace equitp {

// Y[(l*l) + (m + l)] for l = 0..L.
template <int L, typename T>
EQUITP_HD void sh_eval(T x, T y, T z, T* Y) {
  Y[0] = T(1);
  if constexpr (L >= 1) {
    const T s3 = T(1.7320508075688772);  // sqrt(3)
    Y[1] = s3 * y;
    Y[2] = s3 * z;
    Y[3] = s3 * x;
  }
  if constexpr (L >= 2) {
    const T s15 = T(3.872983346207417);     // sqrt(15)
    const T s5h = T(1.118033988749895);     // sqrt(5) / 2
    const T s15h = T(1.9364916731037085);   // sqrt(15) / 2
    Y[4] = s15 * x * y;
    Y[5] = s15 * y * z;
    Y[6] = s5h * (T(3) * z * z - T(1));
    Y[7] = s15 * x * z;
    Y[8] = s15h * (x * x - y * y);
  }
  if constexpr (L >= 3) {
    const T a = T(2.091650066335189);   // sqrt(70) / 4
    const T b = T(10.246950765959598);  // sqrt(105)
    const T c = T(1.6201851746019651);  // sqrt(42) / 4
    const T d = T(1.3228756555322954);  // sqrt(7) / 2
    const T e = T(5.123475382979799);   // sqrt(105) / 2
    const T z2 = z * z;
    Y[9] = a * y * (T(3) * x * x - y * y);
    Y[10] = b * x * y * z;
    Y[11] = c * y * (T(5) * z2 - T(1));
    Y[12] = d * z * (T(5) * z2 - T(3));
    Y[13] = c * x * (T(5) * z2 - T(1));
    Y[14] = e * z * (x * x - y * y);
    Y[15] = a * x * (x * x - T(3) * y * y);
  }
}

// g = sum_i dY[i] * grad P_i(x, y, z), where P_i is the polynomial of sh_eval.  The caller
// projects g onto the tangent plane and divides by |v| to get dL/dv (any extension of Y off the
// sphere gives the same tangential part).
template <int L, typename T>
EQUITP_HD void sh_vjp(T x, T y, T z, const T* dY, T& gx, T& gy, T& gz) {
  gx = T(0);
  gy = T(0);
  gz = T(0);
  if constexpr (L >= 1) {
    const T s3 = T(1.7320508075688772);
    gy += s3 * dY[1];
    gz += s3 * dY[2];
    gx += s3 * dY[3];
  }
  if constexpr (L >= 2) {
    const T s15 = T(3.872983346207417);
    const T s5x3 = T(6.708203932499369);  // 3 sqrt(5)
    // xy
    gx += s15 * y * dY[4];
    gy += s15 * x * dY[4];
    // yz
    gy += s15 * z * dY[5];
    gz += s15 * y * dY[5];
    // (sqrt5/2)(3z^2 - 1)
    gz += s5x3 * z * dY[6];
    // xz
    gx += s15 * z * dY[7];
    gz += s15 * x * dY[7];
    // (sqrt15/2)(x^2 - y^2)
    gx += s15 * x * dY[8];
    gy -= s15 * y * dY[8];
  }
  if constexpr (L >= 3) {
    const T a = T(2.091650066335189);
    const T b = T(10.246950765959598);
    const T c = T(1.6201851746019651);
    const T d = T(1.3228756555322954);
    const T e = T(5.123475382979799);
    const T z2 = z * z;
    // a y (3x^2 - y^2)
    gx += a * T(6) * x * y * dY[9];
    gy += a * T(3) * (x * x - y * y) * dY[9];
    // b xyz
    gx += b * y * z * dY[10];
    gy += b * x * z * dY[10];
    gz += b * x * y * dY[10];
    // c y (5z^2 - 1)
    gy += c * (T(5) * z2 - T(1)) * dY[11];
    gz += c * T(10) * y * z * dY[11];
    // d z (5z^2 - 3)
    gz += d * (T(15) * z2 - T(3)) * dY[12];
    // c x (5z^2 - 1)
    gx += c * (T(5) * z2 - T(1)) * dY[13];
    gz += c * T(10) * x * z * dY[13];
    // e z (x^2 - y^2)
    gx += e * T(2) * x * z * dY[14];
    gy -= e * T(2) * y * z * dY[14];
    gz += e * (x * x - y * y) * dY[14];
    // a x (x^2 - 3y^2)
    gx += a * T(3) * (x * x - y * y) * dY[15];
    gy -= a * T(6) * x * y * dY[15];
  }
}

}  // namespace equitp
