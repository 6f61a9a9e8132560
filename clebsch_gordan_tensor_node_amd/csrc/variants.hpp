// Registry of the compiled path specialisations.
//
// A variant is one (l1, l2, l3, K) combination: the coupling of an input irrep l1 with
// the edge harmonic l2 into l3, with K channels per lane.  Every triangle-allowed
// triple with l <= 6 is compiled for K = 4 (16-byte vector loads and stores) and
// K = 1 (any alignment).
#pragma once

#include "cg_real.hpp"

namespace cgtp {

constexpr int kNumK = 2;
constexpr int k_of(int kidx) { return kidx == 0 ? 4 : 1; }

constexpr int count_triples() {
  int n = 0;
  for (int a = 0; a <= kMaxL; ++a)
    for (int b = 0; b <= kMaxL; ++b)
      for (int c = (a > b ? a - b : b - a); c <= (a + b < kMaxL ? a + b : kMaxL); ++c) ++n;
  return n;
}
constexpr int kNumTriples = count_triples();
constexpr int kNumVariants = kNumTriples * kNumK;

struct VariantDesc {
  int l1, l2, l3, k;
};

constexpr VariantDesc variant_desc(int v) {
  const int t = v / kNumK, kidx = v % kNumK;
  int n = 0;
  for (int a = 0; a <= kMaxL; ++a)
    for (int b = 0; b <= kMaxL; ++b)
      for (int c = (a > b ? a - b : b - a); c <= (a + b < kMaxL ? a + b : kMaxL); ++c) {
        if (n == t) return VariantDesc{a, b, c, k_of(kidx)};
        ++n;
      }
  return VariantDesc{-1, -1, -1, 0};
}

constexpr int variant_index(int l1, int l2, int l3, int k) {
  int n = 0;
  for (int a = 0; a <= kMaxL; ++a)
    for (int b = 0; b <= kMaxL; ++b)
      for (int c = (a > b ? a - b : b - a); c <= (a + b < kMaxL ? a + b : kMaxL); ++c) {
        if (a == l1 && b == l2 && c == l3) return n * kNumK + (k == 4 ? 0 : 1);
        ++n;
      }
  return -1;
}

constexpr int variant_lmax(int v) {
  const VariantDesc d = variant_desc(v);
  const int m = d.l1 > d.l2 ? d.l1 : d.l2;
  return m > d.l3 ? m : d.l3;
}

// Kernel classes, each a separate kernel built in its own translation unit (so that
// the register budget of small-l code is not set by large-l code, and the classes
// compile in parallel):
//   0: every variant with l <= 2        (plans whose largest l is 2 or less)
//   1: every variant with l <= 3        (l <= 3 jobs of plans that reach l = 3 or more)
//   2 + l1: variants with some l >= 4 and that l1
constexpr int kNumClasses = 2 + kMaxL + 1;
constexpr bool class_contains(int c, int v) {
  const int m = variant_lmax(v);
  if (c == 0) return m <= 2;
  if (c == 1) return m <= 3;
  return m >= 4 && variant_desc(v).l1 == c - 2;
}
// Largest l1 among the variants of class c (it sizes the class's LDS staging).
constexpr int class_max_l1(int c) { return c == 0 ? 2 : c == 1 ? 3 : c - 2; }
// class of a variant inside a plan whose largest l is plan_lmax
constexpr int job_class(int v, int plan_lmax) {
  const int m = variant_lmax(v);
  if (m >= 4) return 2 + variant_desc(v).l1;
  return plan_lmax <= 2 ? 0 : 1;
}

}  // namespace cgtp
