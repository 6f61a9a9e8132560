// Real spherical harmonics from Cartesian recurrences, fp64.
//
// Convention (the pages leave it open): component normalisation (Y_0 = 1,
// sum_m Y_lm^2 = 2l+1 on the unit sphere) in the real basis whose l = 1 block is
// sqrt(3) (y, z, x):
//   Y_{l,0}  = sqrt(2l+1) Q_l^0(z)
//   Y_{l,+m} = sqrt(2) sqrt((2l+1)(l-m)!/(l+m)!) Q_l^m(z) Re[(x + i y)^m]
//   Y_{l,-m} = sqrt(2) sqrt((2l+1)(l-m)!/(l+m)!) Q_l^m(z) Im[(x + i y)^m]
// where Q_l^m = P_l^m / sin^m(theta) is the associated Legendre function without the
// Condon-Shortley phase divided by sin^m, a polynomial in z obtained from
//   Q_m^m = (2m-1)!!,  Q_{m+1}^m = (2m+1) z Q_m^m,
//   (l-m) Q_l^m = (2l-1) z Q_{l-1}^m - (l+m-1) Q_{l-2}^m,
// and (x + i y)^m = sin^m(theta) e^{i m phi} by complex multiplication.  No
// trigonometric or inverse-trigonometric function is evaluated.
#pragma once

#include "cg_real.hpp"

namespace cgtp {

struct ShConst {
  double norm[kMaxL + 1][kMaxL + 1];  // [l][m], m >= 0
  double qmm[kMaxL + 1];              // (2m-1)!!
  constexpr ShConst() : norm(), qmm() {
    for (int l = 0; l <= kMaxL; ++l)
      for (int m = 0; m <= l; ++m)
        norm[l][m] = (m == 0) ? cgdetail::csqrt(double(2 * l + 1))
                              : cgdetail::csqrt(2.0 * double(2 * l + 1) * cgdetail::fact(l - m) /
                                                cgdetail::fact(l + m));
    for (int m = 0; m <= kMaxL; ++m) {
      double r = 1.0;
      for (int k = 2 * m - 1; k > 1; k -= 2) r *= double(k);
      qmm[m] = r;
    }
  }
};

// A value and its derivatives with respect to the three components of an edge vector
// (forward-mode differentiation): running the harmonics' recurrence on these gives
// dY/dr exactly, through the same polynomial arithmetic as Y itself.
struct Dual3 {
  double v, d[3];
  __host__ __device__ Dual3() : v(0.0), d{0.0, 0.0, 0.0} {}
  __host__ __device__ Dual3(double c) : v(c), d{0.0, 0.0, 0.0} {}
};
__host__ __device__ inline Dual3 operator+(const Dual3& a, const Dual3& b) {
  Dual3 r(a.v + b.v);
  for (int k = 0; k < 3; ++k) r.d[k] = a.d[k] + b.d[k];
  return r;
}
__host__ __device__ inline Dual3 operator-(const Dual3& a, const Dual3& b) {
  Dual3 r(a.v - b.v);
  for (int k = 0; k < 3; ++k) r.d[k] = a.d[k] - b.d[k];
  return r;
}
__host__ __device__ inline Dual3 operator*(const Dual3& a, const Dual3& b) {
  Dual3 r(a.v * b.v);
  for (int k = 0; k < 3; ++k) r.d[k] = a.d[k] * b.v + a.v * b.d[k];
  return r;
}
__host__ __device__ inline Dual3 operator*(double c, const Dual3& a) {
  Dual3 r(c * a.v);
  for (int k = 0; k < 3; ++k) r.d[k] = c * a.d[k];
  return r;
}
__host__ __device__ inline Dual3 operator/(const Dual3& a, double c) {
  Dual3 r(a.v / c);
  for (int k = 0; k < 3; ++k) r.d[k] = a.d[k] / c;
  return r;
}

// Y[(L+1)^2], index l*l + l + m, for the unit vector (x, y, z); S = double, or Dual3
// for the harmonics together with their derivatives.
template <int L, typename S = double>
__host__ __device__ inline void sh_unit(S x, S y, S z, S* Y) {
  constexpr ShConst K{};
  S C[L + 1], Sn[L + 1];
  C[0] = S(1.0);
  Sn[0] = S(0.0);
#pragma unroll
  for (int m = 1; m <= L; ++m) {
    C[m] = x * C[m - 1] - y * Sn[m - 1];
    Sn[m] = x * Sn[m - 1] + y * C[m - 1];
  }
#pragma unroll
  for (int m = 0; m <= L; ++m) {
    S q2(0.0), q1(0.0);
#pragma unroll
    for (int l = m; l <= L; ++l) {
      S q;
      if (l == m)
        q = S(K.qmm[m]);
      else if (l == m + 1)
        q = double(2 * m + 1) * z * q1;
      else
        q = (double(2 * l - 1) * z * q1 - double(l + m - 1) * q2) / double(l - m);
      q2 = q1;
      q1 = q;
      if (m == 0) {
        Y[l * l + l] = K.norm[l][0] * q;
      } else {
        Y[l * l + l + m] = K.norm[l][m] * q * C[m];
        Y[l * l + l - m] = K.norm[l][m] * q * Sn[m];
      }
    }
  }
}

}  // namespace cgtp
