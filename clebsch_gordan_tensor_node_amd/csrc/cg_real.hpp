// Real-basis Clebsch-Gordan coefficients, evaluated at compile time or at run time.
//
// The pages (LunaTP abstract; spec definition of the uvu CGTP) couple an input
// irrep l1 with the edge spherical harmonics l2 into l3 through "sparse CG
// coefficients" but print no convention.  This library uses:
//   * complex CG by Racah's closed form (Condon-Shortley phase), factorials in double
//     (exact up to 22!, far above the l <= 6 supported here);
//   * the unitary U_l from complex to real spherical harmonics,
//       m < 0: U[m,m] = i/sqrt2, U[m,-m] = -i(-1)^m/sqrt2;  m = 0: 1;
//       m > 0: U[m,-m] = 1/sqrt2, U[m,m] = (-1)^m/sqrt2;
//   * C_real[m1,m2,m3] = sum conj(U1[m1,a]) conj(U2[m2,b]) U3[m3,c] CG[a,b,c], keeping the
//     real part when l1+l2+l3 is even and the imaginary part when it is odd (the other
//     part vanishes identically).
// Every function here is constexpr so that kernels specialised on (l1,l2,l3) carry the
// coefficients and their sparsity pattern as compile-time constants (LunaTP Table 10
// shows compile-time specialisation of the coupling code).
#pragma once

namespace cgtp {

constexpr int kMaxL = 6;

namespace cgdetail {

constexpr double fact(int n) {
  double r = 1.0;
  for (int i = 2; i <= n; ++i) r *= double(i);
  return r;
}

constexpr double csqrt(double x) {
  if (!(x > 0.0)) return 0.0;
  double r = x > 1.0 ? x : 1.0;  // Newton from above converges monotonically
  for (int it = 0; it < 200; ++it) {
    double n = 0.5 * (r + x / r);
    if (!(n < r)) break;
    r = n;
  }
  return r;
}

constexpr int iabs(int a) { return a < 0 ? -a : a; }
constexpr int imin(int a, int b) { return a < b ? a : b; }
constexpr int imax(int a, int b) { return a > b ? a : b; }
constexpr double sgn_pow(int k) { return (k % 2 == 0) ? 1.0 : -1.0; }  // (-1)^k, k may be < 0

// <j1 m1 j2 m2 | J M>, Racah's formula.
constexpr double cg_complex(int j1, int m1, int j2, int m2, int J, int M) {
  if (M != m1 + m2) return 0.0;
  if (J < iabs(j1 - j2) || J > j1 + j2) return 0.0;
  if (iabs(m1) > j1 || iabs(m2) > j2 || iabs(M) > J) return 0.0;
  double pre = double(2 * J + 1) * fact(J + j1 - j2) * fact(J - j1 + j2) * fact(j1 + j2 - J) /
               fact(j1 + j2 + J + 1);
  pre *= fact(J + M) * fact(J - M) * fact(j1 - m1) * fact(j1 + m1) * fact(j2 - m2) * fact(j2 + m2);
  double s = 0.0;
  const int kmin = imax(0, imax(j2 - J - m1, j1 - J + m2));
  const int kmax = imin(j1 + j2 - J, imin(j1 - m1, j2 + m2));
  for (int k = kmin; k <= kmax; ++k) {
    double den = fact(k) * fact(j1 + j2 - J - k) * fact(j1 - m1 - k) * fact(j2 + m2 - k) *
                 fact(J - j2 + m1 + k) * fact(J - j1 - m2 + k);
    s += sgn_pow(k) / den;
  }
  return csqrt(pre) * s;
}

struct cplx {
  double re, im;
};
constexpr cplx cmul(cplx a, cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
constexpr cplx conj(cplx a) { return {a.re, -a.im}; }

// U_l[m, mu]
constexpr cplx u_entry(int m, int mu) {
  const double r = 0.70710678118654752440;
  if (m < 0) {
    if (mu == m) return {0.0, r};
    if (mu == -m) return {0.0, -r * sgn_pow(m)};
    return {0.0, 0.0};
  }
  if (m == 0) return (mu == 0) ? cplx{1.0, 0.0} : cplx{0.0, 0.0};
  if (mu == -m) return {r, 0.0};
  if (mu == m) return {r * sgn_pow(m), 0.0};
  return {0.0, 0.0};
}

}  // namespace cgdetail

// Real CG coefficient C[m1,m2,m3] (m's in -l..l).
constexpr double real_cg(int l1, int l2, int l3, int m1, int m2, int m3) {
  using namespace cgdetail;
  cplx acc{0.0, 0.0};
  const int a_opts[2] = {m1, -m1};
  const int b_opts[2] = {m2, -m2};
  const int na = (m1 == 0) ? 1 : 2;
  const int nb = (m2 == 0) ? 1 : 2;
  for (int ia = 0; ia < na; ++ia) {
    for (int ib = 0; ib < nb; ++ib) {
      const int a = a_opts[ia], b = b_opts[ib], c = a + b;
      if (c != m3 && c != -m3) continue;
      const double v = cg_complex(l1, a, l2, b, l3, c);
      if (v == 0.0) continue;
      cplx t = cmul(cmul(conj(u_entry(m1, a)), conj(u_entry(m2, b))), u_entry(m3, c));
      acc.re += t.re * v;
      acc.im += t.im * v;
    }
  }
  return ((l1 + l2 + l3) % 2 == 0) ? acc.re : acc.im;
}

// Dense table for one path, fp32 and fp64, index
// ((m1+l1)*(2l2+1) + (m2+l2))*(2l3+1) + (m3+l3).
template <int L1, int L2, int L3>
struct RealCG {
  static constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
  float v[N1 * N2 * N3];
  double vd[N1 * N2 * N3];
  int nnz;
  constexpr RealCG() : v(), vd(), nnz(0) {
    for (int a = 0; a < N1; ++a)
      for (int b = 0; b < N2; ++b)
        for (int c = 0; c < N3; ++c) {
          double x = real_cg(L1, L2, L3, a - L1, b - L2, c - L3);
          // |values| are >= 1e-3 or exactly zero for l <= 6; snap round-off to zero
          if (x < 1e-12 && x > -1e-12) x = 0.0;
          v[(a * N2 + b) * N3 + c] = float(x);
          vd[(a * N2 + b) * N3 + c] = x;
          nnz += (x != 0.0);
        }
  }
  constexpr float at(int a, int b, int c) const { return v[(a * N2 + b) * N3 + c]; }
  // the coefficient in the arithmetic type of a kernel (float or double)
  template <typename T>
  constexpr T coef(int a, int b, int c) const {
    if constexpr (sizeof(T) == 4)
      return v[(a * N2 + b) * N3 + c];
    else
      return vd[(a * N2 + b) * N3 + c];
  }
  // A[m1,m3] = sum_m2 C[m1,m2,m3] Y[m2] is structurally nonzero
  constexpr bool a_nonzero(int a, int c) const {
    for (int b = 0; b < N2; ++b)
      if (v[(a * N2 + b) * N3 + c] != 0.0f) return true;
    return false;
  }
};

}  // namespace cgtp
