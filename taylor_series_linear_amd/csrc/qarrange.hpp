// Internal feature order of the per-token query generator (order 4, d = 16),
// with no HIP dependency so that a CPU test can check it.
//
// Rotating every index of a tuple by d/2 (mod d) and sorting gives another
// tuple of the same order with the same multiplicities, hence the same
// sqrt-multinomial weight ("Expanding Attention: A Taylor-Series Route to
// Linear-Time Transformers with a Fixed Number of Recurrent States", "Higher
// orders": one feature per non-decreasing tuple). The rotation is an
// involution, so the basis splits into pairs {f, rot(f)} and fixed points.
// The internal order lays the basis out in ranges of 2 HALF positions: HALF
// representatives (one per pair, canonical order, then the fixed points),
// followed by the rotated images of the same HALF representatives (no
// feature where the representative is a fixed point or missing). Lanes that
// run the generator on rotated coordinates then produce the second half of a
// range with the same instructions as the first.
#pragma once

#include "features.hpp"

namespace tl {

// Canonical index of the non-decreasing m-tuple idx (orders ascending, tuples
// lexicographic within an order).
constexpr int tuple_rank(int D, const int* idx, int m) {
  long long r = 0;
  for (int mm = 0; mm < m; ++mm) r += binom(D + mm - 1, mm);
  int lo = 0;
  for (int p = 0; p < m; ++p) {
    // tuples with the same prefix and a smaller index u at position p (lo <=
    // u < idx[p]): the other L = m-p-1 positions are non-decreasing over
    // {u..D-1}, C(D-u+L-1, L) of them; summed over u, C(D-lo+L, L+1) -
    // C(D-idx[p]+L, L+1)
    const int L = m - p - 1;
    r += binom(D - lo + L, L + 1) - binom(D - idx[p] + L, L + 1);
    lo = idx[p];
  }
  return static_cast<int>(r);
}

// Canonical index of the rotation of feature f by D/2.
template <int D, int NT>
constexpr int rotated_feature(int f) {
  const Monomial& e = kBasis<D, NT>.e[f];
  int t[kMaxOrder] = {0, 0, 0, 0};
  for (int j = 0; j < e.m; ++j) t[j] = (e.idx[j] + D / 2) % D;
  for (int a = 1; a < e.m; ++a)  // insertion sort
    for (int b = a; b > 0 && t[b - 1] > t[b]; --b) {
      const int x = t[b];
      t[b] = t[b - 1];
      t[b - 1] = x;
    }
  return tuple_rank(D, t, e.m);
}

template <int D, int NT, int HALF>
struct QArrange {
  static constexpr int F = feature_count(D, NT);
  static constexpr int CAP = 2 * F + 2 * HALF;
  int nA = 0;       // representatives (paired ones, then fixed points)
  int a[F] = {};    // canonical index of representative i
  bool paired[F] = {};
  int npos = 0;     // positions used: whole ranges of 2 HALF
  int perm[CAP] = {};  // position -> canonical index, or -1 (no feature)
};

template <int D, int NT, int HALF>
constexpr QArrange<D, NT, HALF> make_qarrange() {
  QArrange<D, NT, HALF> q{};
  constexpr int F = QArrange<D, NT, HALF>::F;
  int rot[F] = {};
  for (int f = 0; f < F; ++f) rot[f] = rotated_feature<D, NT>(f);
  for (int f = 0; f < F; ++f) {
    if (rot[f] > f) {
      q.a[q.nA] = f;
      q.paired[q.nA] = true;
      ++q.nA;
    }
  }
  for (int f = 0; f < F; ++f) {
    if (rot[f] == f) {
      q.a[q.nA] = f;
      q.paired[q.nA] = false;
      ++q.nA;
    }
  }
  const int ranges = (q.nA + HALF - 1) / HALF;
  q.npos = ranges * 2 * HALF;
  for (int i = 0; i < QArrange<D, NT, HALF>::CAP; ++i) q.perm[i] = -1;
  for (int i = 0; i < ranges * HALF; ++i) {
    const int r = i / HALF, k = i % HALF;
    const int pa = 2 * HALF * r + k;
    if (i < q.nA) {
      q.perm[pa] = q.a[i];
      if (q.paired[i]) q.perm[pa + HALF] = rot[q.a[i]];
    }
  }
  return q;
}

}  // namespace tl
