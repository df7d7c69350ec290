// Segment split and work-ticket mapping of the prefill kernels, as plain
// functions with no HIP dependency: the kernels and the host planner call
// them, and a CPU test checks the forward-progress argument of the
// single-pass order-2 kernel with them (every wait is on lower tickets).
#pragma once

#include <stdint.h>

#ifndef TL_HD
#ifdef __HIPCC__
#define TL_HD __host__ __device__
#else
#define TL_HD
#endif
#endif

namespace tl {

// Smallest segment count that keeps every segment's rows below 2^31 bytes,
// the range of a 32-bit buffer resource: rows per segment * row_bytes < 2^31.
TL_HD inline int64_t min_segments(int64_t nchunks, int chunk, int64_t row_bytes) {
  const int64_t max_chunks = (((int64_t{1} << 31) - 1) / row_bytes) / chunk;
  return (nchunks + max_chunks - 1) / max_chunks;
}

// Split of N tokens into P segments of L tokens (L a multiple of `chunk`; the
// last segment may be shorter): about `target` workgroups over the BH heads
// (`per_head` workgroups per segment of a head), at least `min_chunks` chunks
// per segment, and every segment's rows within a 32-bit buffer range.
struct Split {
  int P;
  int L;
};
TL_HD inline Split split_segments(int BH, int64_t N, int chunk, int64_t target, int per_head, int64_t min_chunks,
                                  int64_t row_bytes) {
  const int64_t nch = (N + chunk - 1) / chunk;
  if (BH <= 0 || nch == 0) return Split{1, static_cast<int>(N)};
  const int64_t units = static_cast<int64_t>(BH) * per_head;
  const int64_t want = (target + units - 1) / units;
  const int64_t maxp = nch / min_chunks > 1 ? nch / min_chunks : 1;
  int64_t P = want < 1 ? 1 : (want > maxp ? maxp : want);
  const int64_t minp = min_segments(nch, chunk, row_bytes);
  if (P < minp) P = minp;
  const int64_t cps = (nch + P - 1) / P;
  return Split{static_cast<int>((nch + cps - 1) / cps), static_cast<int>(cps * chunk)};
}

// Segments per head for the generic prefill kernels: the P that minimises
// an estimate of the call's time in units of one read-out chunk on one
// workgroup slot. `units` workgroups run per segment (heads x feature
// slices), `slots` are resident at once. P = 1: one round of
// ceil(units / slots) over all chunks. P = 2 with a prefix pass (segment 1
// first runs segment 0's keys without read-out, at rho_pre of a read-out
// chunk each): segment 0 takes nchunks / (2 - rho_pre) chunks and sets the
// time. P >= 2 with segment sums: a sum launch over P - 1 segments (rho_sum
// per chunk) then the main launch over P, each in ceil(workgroups / slots)
// rounds of ceil(nchunks / P) chunks, a main-launch workgroup also reading up
// to P - 1 earlier sums (rho_read each). Ties keep the smaller P; P stays
// within [minp, maxp] and the prefix pass needs minp == 1 (all rows of the
// head in one 32-bit buffer range).
struct SegChoice {
  int P;
  bool prefix;  // two segments with a prefix pass (no segment sums)
};
TL_HD inline SegChoice choose_segments(int64_t units, int64_t nchunks, int64_t slots, int64_t minp, int64_t maxp,
                                       double rho_pre, double rho_sum, double rho_read) {
  auto rounds = [&](int64_t w) { return static_cast<double>((w + slots - 1) / slots); };
  if (maxp < minp) maxp = minp;
  SegChoice best{static_cast<int>(minp), false};
  double best_cost = 1e300;
  for (int64_t P = minp; P <= maxp && P <= 256; ++P) {
    const double cps = static_cast<double>((nchunks + P - 1) / P);
    double cost;
    bool prefix = false;
    if (P == 1) {
      cost = rounds(units) * static_cast<double>(nchunks);
    } else if (P == 2 && minp <= 1) {
      cost = rounds(2 * units) * static_cast<double>(nchunks) / (2.0 - rho_pre);
      prefix = true;
    } else {
      cost = rounds(units * P) * (cps + static_cast<double>(P - 1) * rho_read) + rounds(units * (P - 1)) * cps * rho_sum;
    }
    if (cost < best_cost * (1.0 - 1e-9)) {
      best_cost = cost;
      best = SegChoice{static_cast<int>(P), prefix};
    }
  }
  return best;
}

namespace o2s {

// Workgroups of the single-pass order-2 kernel are dispatched to the 8 XCDs
// round-robin by blockIdx; with B*H a multiple of kGroups each group
// blockIdx % kGroups has its own ticket counter and serves heads g, g + 8, ...
constexpr int kGroups = 8;

TL_HD inline bool grouped(int BH, int P) { return P > 1 && BH % kGroups == 0; }

// Unit (head * P + segment) of the `ticket`-th workgroup of group `group`.
TL_HD inline int ticket_unit(int ticket, int group, int P) {
  return ((ticket / P) * kGroups + group) * P + ticket % P;
}

}  // namespace o2s
}  // namespace tl
