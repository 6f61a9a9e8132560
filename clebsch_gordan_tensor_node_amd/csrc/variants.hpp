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

constexpr int kSmallLMax = 3;
// Kernel class: 0 = every l <= 3; 1 + l1 otherwise.  Each class is a separate kernel
// built in its own translation unit, so the register budget of small-l code is not set
// by large-l code and the classes compile in parallel.
constexpr int variant_class(int v) {
  const VariantDesc d = variant_desc(v);
  const int m = d.l1 > d.l2 ? (d.l1 > d.l3 ? d.l1 : d.l3) : (d.l2 > d.l3 ? d.l2 : d.l3);
  return m <= kSmallLMax ? 0 : 1 + d.l1;
}
constexpr int kNumClasses = 2 + kMaxL;

}  // namespace cgtp
