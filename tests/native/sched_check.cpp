// CPU check of the prefill segment split and of the single-pass order-2
// kernel's work-ticket mapping (taylor_series_linear_amd/csrc/sched.hpp).
//
// Forward progress of the single-pass kernel rests on three facts checked
// here for many (B*H, N):
//  1. the split covers the sequence: P segments of L tokens (L a multiple of
//     the chunk), the last one non-empty, each within a 32-bit buffer range;
//  2. with grouped tickets, (group, ticket) -> unit is a bijection onto the
//     B*H*P units, and group g receives exactly the workgroups
//     blockIdx % 8 == g of a grid of B*H*P;
//  3. every unit waits only on units of its own head with a lower segment
//     index, and those hold lower tickets of the same counter. Workgroups
//     take tickets in the order they start, so a waited-on unit belongs to a
//     workgroup that is already running and that waits only on lower
//     tickets itself: by induction every wait ends.
// Prints "ok <cases>" and exits 0, or prints the first failure and exits 1.
#include <cstdio>
#include <vector>

#include "sched.hpp"

using namespace tl;

static int fail(const char* what, int BH, long long N, int P, int L) {
  std::printf("FAIL %s: BH=%d N=%lld P=%d L=%d\n", what, BH, N, P, L);
  return 1;
}

int main() {
  const int C = 32, DV = 64;
  const long long ns[] = {1, 2, 31, 32, 33, 255, 256, 257, 1000, 1100, 3000, 4096, 8192, 65536, 100003,
                          1 << 20, (1LL << 24) + 7};
  long long cases = 0;
  for (int BH = 1; BH <= 1100; BH += (BH < 80 ? 1 : 37)) {
    for (long long N : ns) {
      if (static_cast<long long>(BH) * N > (1LL << 31)) continue;
      const Split sp = split_segments(BH, N, C, 512, 1, 8, DV * 2);
      const int P = sp.P, L = sp.L;
      ++cases;
      // 1. coverage
      if (P < 1 || L < 1 || L % C != 0) return fail("L not a positive multiple of the chunk", BH, N, P, L);
      if (static_cast<long long>(P) * L < N) return fail("segments do not cover N", BH, N, P, L);
      if (static_cast<long long>(P - 1) * L >= N) return fail("empty last segment", BH, N, P, L);
      if (static_cast<long long>(L) * DV * 2 >= (1LL << 31)) return fail("segment beyond a buffer range", BH, N, P, L);
      if (!o2s::grouped(BH, P)) continue;
      // 2. bijection, and group sizes equal to the grid's blockIdx % 8 classes
      const int units = BH * P;
      std::vector<int> owner(units, -1), tick(units, -1);
      for (int g = 0; g < o2s::kGroups; ++g) {
        int in_group = 0;
        for (int b = 0; b < units; ++b) in_group += (b % o2s::kGroups == g);
        for (int t = 0; t < in_group; ++t) {
          const int u = o2s::ticket_unit(t, g, P);
          if (u < 0 || u >= units) return fail("ticket maps outside the units", BH, N, P, L);
          if (owner[u] != -1) return fail("two tickets map to one unit", BH, N, P, L);
          owner[u] = g;
          tick[u] = t;
        }
      }
      for (int u = 0; u < units; ++u)
        if (owner[u] == -1) return fail("a unit has no ticket", BH, N, P, L);
      // 3. waits only on lower tickets of the same counter
      for (int u = 0; u < units; ++u) {
        const int bh = u / P, p = u % P;
        for (int q = 0; q < p; ++q) {
          const int v = bh * P + q;
          if (owner[v] != owner[u] || tick[v] >= tick[u]) return fail("wait on a later ticket", BH, N, P, L);
        }
      }
    }
  }
  std::printf("ok %lld\n", cases);
  return 0;
}
