// gfx950 matrix-core (MFMA) operand policies.
//
// Every contraction here uses 16x16 output tiles. A "k-step" is 32 deep: each
// lane supplies 8 values ("slots") of its A row / B column. For bf16 one
// v_mfma_f32_16x16x32_bf16 consumes all 8 slots; for fp32 eight
// v_mfma_f32_16x16x4_f32 consume one slot each. The product is a sum over k,
// so any assignment of k values to (lane group, slot) works as long as A and
// B use the same one.
//
// Output (accumulator) layout of a 16x16 tile: lane l holds rows
// 4*(l/16) + i, i = 0..3, of column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <bool BF16>
struct Mma;

template <>
struct Mma<true> {
  using elem = __bf16;
  using frag = bf16x8;  // one 32-deep k-step
  using half = bf16x4;  // one 16-deep k-step (d = 16 score tiles)
  static __device__ __forceinline__ f32x4 step(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 hstep(half a, half b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ elem cvt(float x) { return static_cast<__bf16>(x); }
};

template <>
struct Mma<false> {
  using elem = float;
  using frag = f32x8;
  using half = f32x4;
  static __device__ __forceinline__ f32x4 step(frag a, frag b, f32x4 c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4 hstep(half a, half b, f32x4 c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ elem cvt(float x) { return x; }
};

// Load 8 consecutive elements (a natural-order k-step slice) from LDS. Only
// 16-byte alignment is assumed.
template <typename E>
__device__ __forceinline__ typename Mma<sizeof(E) == 2>::frag lds_frag8(const E* p) {
  if constexpr (sizeof(E) == 2) {
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = lo[j];
      r[j + 4] = hi[j];
    }
    return r;
  }
}

// Load 4 + 4 elements at p[0..3] and p[16..19]: the k-step slice that matches
// the accumulator layout (lane group g owns rows 4g..4g+3 of two stacked
// 16-row tiles).
template <typename E>
__device__ __forceinline__ typename Mma<sizeof(E) == 2>::frag lds_frag_split(const E* p) {
  using F = typename Mma<sizeof(E) == 2>::frag;
  using H = typename Mma<sizeof(E) == 2>::half;
  H lo = *reinterpret_cast<const H*>(p);
  H hi = *reinterpret_cast<const H*>(p + 16);
  F r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = lo[j];
    r[j + 4] = hi[j];
  }
  return r;
}

}  // namespace tl
