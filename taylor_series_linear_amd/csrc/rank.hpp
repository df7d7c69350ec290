// Runtime decoding of a canonical feature index into its monomial, with no
// HIP dependency: the kernels call it for bases too wide for a compile-time
// table (order 6 at d = 16 has 74,613 features), and a CPU test checks it
// against an enumeration of the basis.
#pragma once

#include <stdint.h>

#ifndef TL_HD
#ifdef __HIPCC__
#define TL_HD __host__ __device__
#else
#define TL_HD
#endif
#endif

// Loops over the kMaxOrderRank tuple positions are fully unrolled with a
// guard, so that a decoded tuple stays in registers on the GPU.
#ifdef __HIPCC__
#define TL_UNROLL _Pragma("unroll")
#else
#define TL_UNROLL
#endif

namespace tl {

constexpr int kMaxOrderRank = 6;  // highest degree the decoder handles (n_terms <= 7)

// Degree, indices and sqrt-multinomial weight of canonical feature f of the
// basis (d, n_terms): orders ascending; within order m the non-decreasing
// tuples in lexicographic order. The rank r inside the order is decoded one
// position at a time: with the first free index i, the tuples that remain
// after position j are the non-decreasing (m-j-1)-tuples over {i..d-1}, of
// which there are C(d-i+m-j-2, m-j-1).
struct RankedFeature {
  int m;
  int idx[kMaxOrderRank];
  float w;  // sqrt(m! / prod_i c_i!)
};

// C(n, k) for the small k of a feature decoder (products divided by a
// constant k!, which compiles to multiplications on the GPU)
TL_HD inline long long rank_binom(int n, int k) {
  if (k < 0 || k > n) return 0;
  const long long x = n;
  switch (k) {
    case 0: return 1;
    case 1: return x;
    case 2: return x * (x - 1) / 2;
    case 3: return x * (x - 1) * (x - 2) / 6;
    case 4: return x * (x - 1) * (x - 2) * (x - 3) / 24;
    case 5: return x * (x - 1) * (x - 2) * (x - 3) * (x - 4) / 120;
    case 6: return x * (x - 1) * (x - 2) * (x - 3) * (x - 4) * (x - 5) / 720;
    default: {
      long long r = 1;
      for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
      return r;
    }
  }
}

// sqrt(m! / prod of factorials of the run lengths) of a sorted tuple
TL_HD inline float rank_weight(const int (&idx)[kMaxOrderRank], int m) {
  int num = 1, den = 1, run = 1;
  TL_UNROLL
  for (int j = 1; j < kMaxOrderRank; ++j) {
    if (j < m) {
      num *= j + 1;
      run = idx[j] == idx[j - 1] ? run + 1 : 1;
      den *= run;
    }
  }
  return __builtin_sqrtf(static_cast<float>(num / den));
}

TL_HD inline RankedFeature rank_decode(int d, int n_terms, long long f) {
  RankedFeature out{};
  int m = 0;
  long long width = 1;  // C(d+m-1, m)
  while (m + 1 < n_terms && f >= width) {
    f -= width;
    ++m;
    width = rank_binom(d + m - 1, m);
  }
  out.m = m;
  int lo = 0;
  TL_UNROLL
  for (int j = 0; j < kMaxOrderRank; ++j) {
    if (j < m) {
      const int rem = m - j - 1;
      int i = lo;
      for (; i < d - 1; ++i) {
        const long long cnt = rank_binom(d - i + rem - 1, rem);
        if (f < cnt) break;
        f -= cnt;
      }
      out.idx[j] = i;
      lo = i;
    }
  }
  out.w = rank_weight(out.idx, m);
  return out;
}

// The feature after e in canonical order (the next non-decreasing tuple of
// the same degree, or the first tuple (0, ..., 0) of the next degree). Past
// the highest degree the decoder handles, e is left unchanged.
TL_HD inline void rank_next(int d, RankedFeature& e) {
  // last position that can still grow
  int p = -1;
  TL_UNROLL
  for (int j = 0; j < kMaxOrderRank; ++j)
    if (j < e.m && e.idx[j] < d - 1) p = j;
  if (p < 0) {
    if (e.m >= kMaxOrderRank) return;
    ++e.m;
    TL_UNROLL
    for (int j = 0; j < kMaxOrderRank; ++j) e.idx[j] = 0;
  } else {
    int v = 0;
    TL_UNROLL
    for (int j = 0; j < kMaxOrderRank; ++j) {
      if (j == p) v = e.idx[j] + 1;
      if (j >= p && j < e.m) e.idx[j] = v;
    }
  }
  e.w = rank_weight(e.idx, e.m);
}

}  // namespace tl
