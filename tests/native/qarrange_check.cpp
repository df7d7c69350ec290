// Prints the internal feature order of the per-token query generator
// (taylor_series_linear_amd/csrc/qarrange.hpp) for d = 16, n_terms = 5 and
// 40 representatives per range: first "nA npos", then one line per position,
// "pos canonical_index" (-1 where no feature sits), then one line per
// representative, "i canonical_index paired". The Python test checks it
// against an enumeration of the basis and of the index rotation.
#include <cstdio>

#include "qarrange.hpp"

static constexpr auto kQ = tl::make_qarrange<16, 5, 40>();

int main() {
  std::printf("%d %d\n", kQ.nA, kQ.npos);
  for (int p = 0; p < kQ.npos; ++p) std::printf("%d %d\n", p, kQ.perm[p]);
  for (int i = 0; i < kQ.nA; ++i) std::printf("%d %d %d\n", i, kQ.a[i], kQ.paired[i] ? 1 : 0);
  return 0;
}
