// Compile-time tables of the symmetric monomial basis.
//
// The basis of "Expanding Attention: A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States" ("Higher orders":
// width C(d+m-1, m) per order): one feature per non-decreasing index tuple
// i_1 <= ... <= i_m over {0..d-1}; orders ascending, tuples lexicographic.
// The feature value is sqrt(m! / prod_i c_i!) * prod_j x[i_j], so that
// phi_m(x).phi_m(y) = (x.y)^m (multinomial theorem).
#pragma once

#include <stdint.h>

#include "rank.hpp"

namespace tl {

constexpr int kMaxOrder = 4;  // highest degree instantiated (n_terms <= 5)

constexpr long long binom(int n, int k) {
  if (k < 0 || k > n) return 0;
  long long r = 1;
  for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
  return r;
}

constexpr int feature_count(int d, int n_terms) {
  long long f = 0;
  for (int m = 0; m < n_terms; ++m) f += binom(d + m - 1, m);
  return static_cast<int>(f);
}

constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }

constexpr long long factorial(int m) {
  long long r = 1;
  for (int i = 2; i <= m; ++i) r *= i;
  return r;
}

// Newton iteration for sqrt in double, exact to the last bit for the small
// integers used here (multinomial coefficients up to 24).
constexpr double csqrt(double x) {
  if (x <= 0) return 0;
  double r = x < 1 ? 1.0 : x;
  for (int it = 0; it < 64; ++it) r = 0.5 * (r + x / r);
  return r;
}

struct Monomial {
  int m;              // degree
  int idx[kMaxOrder]; // indices, non-decreasing; unused slots = 0
  long long mult;     // m! / prod c_i!
};

// Number of ordered sequences sorting to the tuple.
constexpr long long multinomial_of(const int* idx, int m) {
  long long den = 1;
  int run = 1;
  for (int j = 1; j <= m; ++j) {
    if (j < m && idx[j] == idx[j - 1]) {
      ++run;
    } else {
      den *= factorial(run);
      run = 1;
    }
  }
  return factorial(m) / den;
}

template <int D, int NT>
struct BasisTable {
  static constexpr int F = feature_count(D, NT);
  Monomial e[F];
  int order_begin[NT + 1];
};

template <int D, int NT>
constexpr BasisTable<D, NT> make_basis() {
  BasisTable<D, NT> t{};
  int f = 0;
  for (int m = 0; m < NT; ++m) {
    t.order_begin[m] = f;
    int idx[kMaxOrder] = {0, 0, 0, 0};
    // enumerate non-decreasing tuples of length m in lexicographic order
    while (true) {
      Monomial& e = t.e[f++];
      e.m = m;
      for (int j = 0; j < kMaxOrder; ++j) e.idx[j] = j < m ? idx[j] : 0;
      e.mult = multinomial_of(idx, m);
      if (m == 0) break;
      int p = m - 1;
      while (p >= 0 && idx[p] == D - 1) --p;
      if (p < 0) break;
      ++idx[p];
      for (int j = p + 1; j < m; ++j) idx[j] = idx[p];
    }
  }
  t.order_begin[NT] = f;
  return t;
}

template <int D, int NT>
inline constexpr BasisTable<D, NT> kBasis = make_basis<D, NT>();

// Device-side record for table-driven (runtime-indexed) kernels:
// 4 packed 8-bit indices, degree, and sqrt(multinomial).
struct PackedFeature {
  uint32_t idx;  // idx[j] in bits 8j..8j+7
  uint32_t m;
  float w;       // sqrt(m! / prod c_i!)
  float inv_mfact;  // 1 / m!
};

template <int D, int NT>
struct PackedTable {
  static constexpr int F = feature_count(D, NT);
  PackedFeature e[F];
};

template <int D, int NT>
constexpr PackedTable<D, NT> make_packed() {
  PackedTable<D, NT> p{};
  constexpr auto& b = kBasis<D, NT>;
  for (int f = 0; f < PackedTable<D, NT>::F; ++f) {
    uint32_t packed = 0;
    for (int j = 0; j < kMaxOrder; ++j) packed |= static_cast<uint32_t>(b.e[f].idx[j]) << (8 * j);
    p.e[f].idx = packed;
    p.e[f].m = static_cast<uint32_t>(b.e[f].m);
    p.e[f].w = static_cast<float>(csqrt(static_cast<double>(b.e[f].mult)));
    p.e[f].inv_mfact = static_cast<float>(1.0 / static_cast<double>(factorial(b.e[f].m)));
  }
  return p;
}

// Per-feature constants for the unrolled generators. For feature f with
// tuple (i_1..i_m), value = G * prod_{j<m} x[i_j] * x[i_m] * R, where G is
// shared by every feature with the same prefix (i_1..i_{m-1}) whose last
// index is new (i_m > i_{m-1}), and R = 1 for those; a repeated last index
// (i_m == i_{m-1}) takes R = weight / G. Writing G * prefix the same way for
// every such feature lets the compiler share the prefix products.
struct GenConst {
  int m;
  int idx[kMaxOrder];
  double G;  // group constant (includes `scale_m`)
  double R;  // correction for a repeated last index
};

// scale_m: extra per-order factor folded into G (1/m! for the query side).
template <int D, int NT, bool QSIDE>
constexpr GenConst gen_const(int f) {
  const Monomial& e = kBasis<D, NT>.e[f];
  GenConst g{};
  g.m = e.m;
  for (int j = 0; j < kMaxOrder; ++j) g.idx[j] = e.idx[j];
  const double w = csqrt(static_cast<double>(e.mult));
  const double s = QSIDE ? 1.0 / static_cast<double>(factorial(e.m)) : 1.0;
  if (e.m <= 1) {
    g.G = w * s;
    g.R = 1.0;
    return g;
  }
  // weight of a feature with this prefix and a new last index
  int tmp[kMaxOrder] = {0, 0, 0, 0};
  for (int j = 0; j < e.m - 1; ++j) tmp[j] = e.idx[j];
  tmp[e.m - 1] = D + 1;  // strictly larger than any index: "new"
  const double wnew = csqrt(static_cast<double>(multinomial_of(tmp, e.m)));
  g.G = wnew * s;
  g.R = (e.idx[e.m - 1] == e.idx[e.m - 2]) ? w / wnew : 1.0;
  return g;
}

}  // namespace tl
