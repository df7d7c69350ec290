// Prints the decoding of every feature index of the basis (d, n_terms) given
// on the command line, one line per feature: "f m w i_1 ... i_m", using the
// library's HIP-free decoder (taylor_series_linear_amd/csrc/rank.hpp): with a
// fourth argument "step", feature 0 is decoded and every later one reached
// with rank_next; otherwise each index is decoded on its own. The Python test
// compares the lines with an enumeration of the basis.
#include <cstdio>
#include <cstdlib>

#include "rank.hpp"

int main(int argc, char** argv) {
  if (argc != 4 && argc != 5) return 2;
  const bool step = argc == 5;
  const int d = std::atoi(argv[1]), n = std::atoi(argv[2]);
  const long long F = std::atoll(argv[3]);
  for (long long f = 0; f < F; ++f) {
    static tl::RankedFeature cur = tl::rank_decode(d, n, 0);
    if (step && f > 0) tl::rank_next(d, cur);
    const tl::RankedFeature e = step ? cur : tl::rank_decode(d, n, f);
    std::printf("%lld %d %.9g", f, e.m, static_cast<double>(e.w));
    for (int j = 0; j < e.m; ++j) std::printf(" %d", e.idx[j]);
    std::printf("\n");
  }
  return 0;
}
