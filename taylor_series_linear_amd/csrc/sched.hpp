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
