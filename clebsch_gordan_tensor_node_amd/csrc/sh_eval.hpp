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

// Y[(L+1)^2], index l*l + l + m, for the unit vector (x, y, z).
template <int L>
__host__ __device__ inline void sh_unit(double x, double y, double z, double* Y) {
  constexpr ShConst K{};
  double C[L + 1], S[L + 1];
  C[0] = 1.0;
  S[0] = 0.0;
#pragma unroll
  for (int m = 1; m <= L; ++m) {
    C[m] = x * C[m - 1] - y * S[m - 1];
    S[m] = x * S[m - 1] + y * C[m - 1];
  }
#pragma unroll
  for (int m = 0; m <= L; ++m) {
    double q2 = 0.0, q1 = 0.0;
#pragma unroll
    for (int l = m; l <= L; ++l) {
      double q;
      if (l == m)
        q = K.qmm[m];
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
        Y[l * l + l - m] = K.norm[l][m] * q * S[m];
      }
    }
  }
}

}  // namespace cgtp
