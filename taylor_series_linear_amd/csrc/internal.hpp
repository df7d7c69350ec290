// Host-side interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tl {

// Launch geometry of one prefill instantiation, known to the host.
struct PrefillTraits {
  int F;    // features
  int FS;   // features per slice (one workgroup's share of the state)
  int G;    // slices
  int C;    // tokens per chunk
  int NW;   // waves per workgroup (dv tiles incl. the denominator tile)
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
  float* seg;   // segment sums, [BH][P-1][G][NW][FS/16][64] x float4
  float* fin;   // final state staging, [BH][G][NW][FS/16][64] x float4 (defer_state)
  float* part;  // partial outputs, [G][BH][N][DV+4] (G > 1 only)
  int BH;
  int N;
  int P;        // segments per head
  int L;        // tokens per segment (multiple of C)
  float inv_a;
  int defer_state;  // final state goes through `fin`, then a copy kernel
};

// Returns false when (d, dv, n_terms, bf16) is not instantiated.
bool prefill_traits(int d, int dv, int n_terms, bool bf16, PrefillTraits* t);

// Enqueue the whole prefill for one instantiation. Returns hipSuccess or the
// launch error.
hipError_t prefill_launch(int d, int dv, int n_terms, bool bf16, const PrefillArgs& a,
                          hipStream_t stream);

hipError_t state_init_launch(const float* S0, const float* z0, float* S, float* z,
                             int64_t BH, int F, int dv, hipStream_t stream);

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
