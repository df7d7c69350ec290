// Host-side interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sched.hpp"

namespace tl {

// Sequence split and workspace layout of one prefill call.
struct PrefillPlan {
  int P = 1;             // segments per head
  int L = 0;             // tokens per segment (multiple of the chunk length)
  int L0 = 0;            // generic kernels, two segments [0, L0) and [L0, N)
                         // with a prefix pass instead of segment sums (0: off)
  size_t seg_off = 0;    // byte offsets into the workspace
  size_t fin_off = 0;
  size_t part_off = 0;
  size_t sync_off = 0;   // flags and tickets of single-pass kernels
  size_t bytes = 0;      // workspace size
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* S0;
  const float* z0;
  void* o;
  int out_bf16;
  float* S;
  float* z;
  float* seg;   // per-segment state sums (layout private to the kernel family)
  float* fin;   // final-state staging for in-place continuation (defer_state)
  float* part;  // partial outputs of feature-sliced kernels
  int* sync;    // flags and work tickets of single-pass kernels (cleared by the launch)
  int wait_spins;  // bound of a single-pass kernel's wait for earlier segments (polls)
  int BH;
  int N;
  int P;        // segments per head
  int L;        // tokens per segment (multiple of C)
  int L0;       // see PrefillPlan::L0
  float inv_a;
  int defer_state;  // final state goes through `fin`, then a copy kernel
  // extended options (generic kernel family only)
  int decay;        // extended kernels: decay and query/key preprocessing
  float log2g;      // log2(gamma) (0: no decay)
  int qk_norm;      // divide q and k rows by their l2 norm
  float q_scale;    // then multiply q by q_scale * q_head_scale[h], k by k_scale
  float k_scale;
  const float* q_head_scale;  // device [H] or null
  int H;
};

// Plans a prefill of BH heads x N tokens. Returns false when
// (d, dv, n_terms, bf16) is not instantiated. `decay` selects the kernel
// family that supports a decayed state (the generic one).
bool prefill_plan(int d, int dv, int n_terms, bool bf16, bool decay, int BH, int N, PrefillPlan* plan);

// Enqueue the whole prefill for one instantiation. Returns hipSuccess or the
// launch error.
hipError_t prefill_launch(int d, int dv, int n_terms, bool bf16, const PrefillArgs& a,
                          hipStream_t stream);

hipError_t state_init_launch(const float* S0, const float* z0, float* S, float* z,
                             int64_t BH, int F, int dv, hipStream_t stream);

// Order-2, d = 16, dv = 64, bf16 prefill (prefill_o2.hip).
namespace o2 {
bool plan(int BH, int N, PrefillPlan* plan);
hipError_t launch(const PrefillArgs& a, hipStream_t stream);
}  // namespace o2

// Order-2, d = 64, dv = 64, bf16 prefill (prefill_w2.hip).
namespace w2 {
bool plan(int BH, int N, PrefillPlan* plan);
hipError_t launch(const PrefillArgs& a, hipStream_t stream);
}  // namespace w2

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* S;
  float* z;
  void* o;
  int out_bf16;
  int BH;
  float inv_a;
  float gamma;  // decay of the state before the write (1: none)
  int qk_norm;  // query/key preprocessing, as for prefill
  float q_scale;
  float k_scale;
  const float* q_head_scale;
  int H;
};

hipError_t decode_launch(int d, int dv, int n_terms, bool bf16, const DecodeArgs& a,
                         hipStream_t stream);

// Per-order factor applied by the feature map (1, or (m! a^m)^(-1/2)).
struct OrderScale {
  float s[8];
};

hipError_t feature_map_launch(int d, int n_terms, bool bf16, const void* x, int64_t rows,
                              float* phi, const OrderScale& sc, hipStream_t stream);

}  // namespace tl
