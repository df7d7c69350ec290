// Prints the generic prefill's segment choice (csrc/sched.hpp,
// choose_segments) for the cases given as arguments, one line per case:
// "units nchunks slots minp maxp -> P prefix". The Python test checks the
// choice against the cost it is meant to minimise.
#include <cstdio>
#include <cstdlib>

#include "sched.hpp"

int main(int argc, char** argv) {
  if ((argc - 1) % 5 != 0) return 2;
  for (int i = 1; i + 4 < argc; i += 5) {
    const long long units = std::atoll(argv[i]), nch = std::atoll(argv[i + 1]), slots = std::atoll(argv[i + 2]);
    const long long minp = std::atoll(argv[i + 3]), maxp = std::atoll(argv[i + 4]);
    const tl::SegChoice c = tl::choose_segments(units, nch, slots, minp, maxp, 0.6, 0.45, 0.4);
    std::printf("%lld %lld %lld %lld %lld -> %d %d\n", units, nch, slots, minp, maxp, c.P, c.prefix ? 1 : 0);
  }
  return 0;
}
