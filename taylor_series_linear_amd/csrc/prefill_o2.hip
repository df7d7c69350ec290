// Order-2 causal prefill for d = 16, dv = 64, bf16 inputs (n_terms = 3),
// written for gfx950's 32x32x16 bf16 matrix cores.
//
// What is computed ("Expanding Attention: A Taylor-Series Route to
// Linear-Time Transformers with a Fixed Number of Recurrent States"; the
// order-2 weight is the posfloor README's 1 + t + t^2/2):
//   o_t = sum_{s<=t} w(q_t.k_s/a) v_s / sum_{s<=t} w(q_t.k_s/a),
//   w(x) = 1 + x + x^2/2,
// chunked as on that page ("Time": a state part plus diagonal blocks):
//   O_c   = phi~(Q_c) S_<c + P_c V_c          (P_c = w(Q_c K_c^T / a), causal)
//   den_c = Q'_c Z~_<c Q'_c^T (diag) + P_c 1
//   S    += phi(K_c)^T V_c,   Z += K'_c^T K'_c
//
// Internal feature basis. The 153 monomials of degree <= 2 over 16
// coordinates (plus 7 zero slots, 160 in all) are ordered so that both
// MFMA operand layouts can be produced with compile-time register
// indices (see feat() below). The key side carries plain products
// (k_i k_j, k_i, 1); the query side carries every weight (1/a^2 for i != j,
// 1/(2a^2) on the diagonal, 1/a on the linear terms). The state in this
// basis differs from the canonical one of the C ABI (sqrt-multinomial
// weights on both sides, lexicographic order) by a permutation and a
// per-row factor sqrt(2) on the off-diagonal monomials; the conversion
// happens when S0/z0 are read and S/z are written.
//
// Denominator. For order 2 the denominator state z (153 numbers) is the
// Gram matrix Z = K'^T K' of K' = [k, 1] (17 x 17): z_0 = Z[16][16],
// z_1 = Z[i][16], z_2 = Z[i][j]. The read-out q'^T Z~ q' with q' = [q, 1]
// and Z~ = Z scaled by 1/(2a^2), 1/(2a), 1 on its blocks equals
// sum_m alpha_m phi_m(q).z_m. Z is 32x32 in the MFMA (rows/cols 17..31 are
// zero). Its read-out adds the count z_0 in fp32, outside the bf16
// contraction of the other entries, so the count is not rounded to 8 bits.
//
// Precision: scores and the read-out use bf16 operands; the state update,
// the intra-chunk term and Z use fp16 operands (keys, values, key products
// and weights are exact or better than bf16 in fp16 within its range), all
// with fp32 accumulation and fp32 states.
//
// Work decomposition: one workgroup of 4 waves per (head, segment).
//  * waves 0, 1 ("M"): state columns [32m, 32m+32) of S (5 tiles of
//    32x32 fp32 in registers); per chunk: score tile, polynomial and causal
//    mask in registers, read-out, intra-chunk term, normalisation, update.
//  * wave 2 ("Q"): stages Q, builds phi~(Q) tiles, owns Z, computes the
//    inter-chunk denominator, stores the normalised output rows.
//  * wave 3 ("K"): stages K, K'^T and V^T (fp16), builds phi(K)^T tiles
//    with packed fp16 products.
// The Q and K waves prepare chunk c+1 in one LDS buffer while the M waves
// consume chunk c from the other; one barrier per chunk. Global loads run
// PD chunks ahead in registers.
//
// Segments, in one launch. Segments of a head are independent given the sum
// of the earlier segments' states (additivity, closing paragraph of the same
// page). Each workgroup takes a work ticket from an atomic counter (tickets
// follow dispatch order), so it only ever waits for segments of lower
// tickets, whose workgroups are already running. Unless it holds the head's
// last segment it first sums its own segment (phase 1), publishes the sum
// with device-scope stores and sets a flag; it then waits for the flags of
// the head's earlier segments, adds their published sums and S0 (phase 2),
// and runs the output pass over its segment (phase 3). The wait is bounded;
// a timed-out wait makes the unit's outputs and final state NaN.
#include "internal.hpp"
#include "mma.hpp"

#include <stdint.h>

#include <type_traits>

namespace tl {
namespace o2 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int C = 32;        // tokens per chunk
constexpr int D = 16;
constexpr int DV = 64;
constexpr int FI = 160;      // internal features (153 monomials + 7 zero slots)
constexpr int NFT = 5;       // 32-feature tiles
constexpr int NTHR = 256;
constexpr int PD = 2;        // chunks of global loads in flight ahead of use
constexpr float kSqrt2 = 1.41421356237309515f;

// LDS layout (bf16 elements per row, 16 bytes of padding per row).
constexpr int QP_P = 40;     // Q' rows: q[0..15], 1, zeros
constexpr int K_P = 24;      // K rows
constexpr int KF_P = 40;     // K'^T rows 0..17 in fp16 (16 = valid-key indicator, 17 = 0)
constexpr int VT_P = 40;     // V^T rows, fp16
constexpr int FQ_P = 168;    // phi~(Q), operand order
constexpr int FK_P = 40;     // phi(K)^T rows
constexpr int OFF_QP = 0;
constexpr int OFF_K = OFF_QP + C * QP_P * 2;
constexpr int OFF_KT = OFF_K + C * K_P * 2;
constexpr int OFF_VT = OFF_KT + 18 * KF_P * 2;
constexpr int OFF_FQ = OFF_VT + DV * VT_P * 2;
constexpr int OFF_FK = OFF_FQ + C * FQ_P * 2;
constexpr int BUF = OFF_FK + FI * FK_P * 2;
constexpr int OFF_DEN = 2 * BUF;
constexpr int OFF_O = OFF_DEN + 2 * C * 4;
// Output transpose area of each M wave: 32 query rows x 32 dv columns.
template <bool OBF>
struct OStage {
  static constexpr int P = OBF ? 40 : 36;           // row pitch in elements
  static constexpr int BYTES = C * P * (OBF ? 2 : 4);
};
template <bool OBF>
constexpr int lds_bytes() {
  return OFF_O + 2 * OStage<OBF>::BYTES;
}
static_assert(lds_bytes<true>() <= 80 * 1024, "two workgroups per CU");
static_assert(lds_bytes<false>() <= 80 * 1024, "two workgroups per CU");
static_assert(OFF_K % 16 == 0 && OFF_KT % 16 == 0 && (KF_P * 2) % 16 == 0 && OFF_VT % 16 == 0 && OFF_FQ % 16 == 0 &&
                  OFF_FK % 16 == 0 && BUF % 16 == 0 && OFF_O % 16 == 0,
              "16-byte aligned regions");

// State sums of one (head, segment) in the accumulator layout: S of the two
// M waves ([wave][tile][4 x float4][64 lanes]) then Z ([4 x float4][64 lanes]).
constexpr int UNIT_F4 = 2 * NFT * 4 * 64 + 4 * 64;   // float4 count
constexpr size_t UNIT_BYTES = static_cast<size_t>(UNIT_F4) * 16;

// Segment-sum pass (phase 1 of the kernel below): chunks of 128 tokens staged
// by all four waves into its own LDS layout (K'^T rows 0..17 and V^T rows,
// fp16, 272-byte rows so consecutive rows start 4 banks apart).
namespace s1 {
constexpr int C = 128;
constexpr int P = C + 8;                 // row pitch in halves
constexpr int KROWS = 18;
constexpr int BUF = (KROWS + DV) * P * 2;
constexpr int NV = C * DV / 8 / NTHR;    // 16-byte V items per thread (K: one)
static_assert(C * D / 8 == NTHR && (C * DV / 8) % NTHR == 0, "whole items per thread");
static_assert(2 * BUF <= lds_bytes<true>() && 2 * BUF <= lds_bytes<false>(), "fits the kernel's LDS");
static_assert(BUF % 16 == 0 && (P * 2) % 16 == 0, "16-byte aligned rows");
}  // namespace s1

// ---------------------------------------------------------------------------
// internal feature basis
// ---------------------------------------------------------------------------

struct Feat {
  int i, j;      // rows of K'^T / columns of Q' multiplied (16 = one, 17 = zero)
  float wq;      // query-side weight before the 1/a powers
  int deg;       // degree of the monomial
  int can;       // canonical feature index, -1 for a zero slot
  float wcan;    // canonical = wcan * internal (key-side sqrt-multinomial)
};

// Internal feature f = 32 ft + 16 u + 8 v + 4 h + r. With K = 2 ft + u,
// s = 4 v + r and a = 8 h + s: K <= 7 (and K = 8 for h = 0) is the pair
// (a, a + K mod 16); K = 8, h = 1 holds the constant (s = 0) and zeros;
// K = 9 is the linear term k_a. Every pair i <= j occurs exactly once.
__host__ __device__ constexpr Feat feat(int f) {
  const int ft = f >> 5, m = f & 31;
  const int u = m >> 4, v = (m >> 3) & 1, h = (m >> 2) & 1, r = m & 3;
  const int K = 2 * ft + u, s = 4 * v + r, a = 8 * h + s;
  Feat e{0, 0, 0.f, 0, -1, 0.f};
  if (K == 9) {
    e = Feat{a, 16, 1.f, 1, 1 + a, 1.f};
  } else if (K == 8 && h == 1) {
    if (s == 0)
      e = Feat{16, 16, 1.f, 0, 0, 1.f};
    else
      e = Feat{17, 17, 0.f, 0, -1, 0.f};
  } else {
    const int b = (a + K) & 15;
    const int lo = a < b ? a : b, hi = a < b ? b : a;
    e = Feat{a, b, K == 0 ? 0.5f : 1.f, 2, 17 + lo * 16 - lo * (lo - 1) / 2 + (hi - lo),
             K == 0 ? 1.f : kSqrt2};
  }
  return e;
}

// Each canonical index 0..152 is produced by exactly one internal slot.
constexpr bool basis_is_bijective() {
  int hits[153] = {};
  for (int f = 0; f < FI; ++f) {
    const Feat e = feat(f);
    if (e.can < -1 || e.can >= 153) return false;
    if (e.can >= 0) ++hits[e.can];
  }
  for (int c = 0; c < 153; ++c)
    if (hits[c] != 1) return false;
  return true;
}
static_assert(basis_is_bijective(), "internal basis covers the canonical one once");

// Z~ = Z scaled blockwise so that q'^T Z~ q' = sum_m alpha_m phi_m(q).z_m.
__device__ __forceinline__ float zscale(int r, int c, float inv_a) {
  if (r > 16 || c > 16) return 0.f;
  if (r == 16 && c == 16) return 1.f;
  if (r == 16 || c == 16) return 0.5f * inv_a;
  return 0.5f * inv_a * inv_a;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 ldh8(const _Float16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ f16x4 ldh4(const _Float16* p) { return *reinterpret_cast<const f16x4*>(p); }
__device__ __forceinline__ f16x8 cath44(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// bf16 -> fp16 (exact for magnitudes in fp16's normal range)
__device__ __forceinline__ f16x8 to_h8(bf16x8 v) {
  f16x8 r;
#pragma unroll
  for (int u = 0; u < 8; ++u) r[u] = static_cast<_Float16>(static_cast<float>(v[u]));
  return r;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 ld4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ f32x8 ldf8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void st8(__bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// cache-policy operand of buffer accesses: device scope (sc1)
constexpr int kDeviceScope = 16;

// Raw buffer resource over `bytes` bytes at p (gfx9 descriptor word 3);
// loads outside the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 a, bf16x4 b) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = a[j];
    r[j + 4] = b[j];
  }
  return r;
}

// Accumulator row of register j for lane half h (32x32 tile layout).
__device__ __forceinline__ constexpr int acc_row(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

struct Smem {
  char* base;
  __device__ __bf16* qp(int b) const { return reinterpret_cast<__bf16*>(base + b * BUF + OFF_QP); }
  __device__ __bf16* kr(int b) const { return reinterpret_cast<__bf16*>(base + b * BUF + OFF_K); }
  __device__ _Float16* kt(int b) const { return reinterpret_cast<_Float16*>(base + b * BUF + OFF_KT); }
  __device__ _Float16* vt(int b) const { return reinterpret_cast<_Float16*>(base + b * BUF + OFF_VT); }
  __device__ __bf16* fq(int b) const { return reinterpret_cast<__bf16*>(base + b * BUF + OFF_FQ); }
  __device__ _Float16* fk(int b) const { return reinterpret_cast<_Float16*>(base + b * BUF + OFF_FK); }
  __device__ float* den(int b) const { return reinterpret_cast<float*>(base + OFF_DEN) + b * C; }
  __device__ char* ostage(int m, int bytes) const { return base + OFF_O + m * bytes; }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Sync area of the single-pass launch (ints): one flag per (head, segment),
// then the work-ticket counter and one counter per workgroup group, each
// counter in a 128-byte line of its own: every workgroup of a call takes a
// ticket at its start, and atomics on one line are served one at a time.
// o2_reset clears the area at the start of a call.
constexpr int kGroups = o2s::kGroups;
constexpr int kCtrStride = 32;  // ints per counter line
__host__ __device__ constexpr int ctr_base(int units) { return (units + kCtrStride - 1) / kCtrStride * kCtrStride; }
__host__ __device__ constexpr int sync_ints(int units) { return ctr_base(units) + kCtrStride * (kGroups + 1); }

__global__ __launch_bounds__(256) void o2_reset(int* sync, int n) {
  for (int i = threadIdx.x; i < n; i += 256) sync[i] = 0;
}

template <bool OBF>
__global__ __launch_bounds__(NTHR, 2) void o2_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem_raw[lds_bytes<OBF>()];
  __shared__ int s_unit;
  __shared__ int s_wait_failed;
  const Smem sm{smem_raw};
  constexpr int OP = OStage<OBF>::P;
  constexpr int OB = OStage<OBF>::BYTES;

  const int tid = threadIdx.x;
  // Role of this wave (a scalar, so role branches are uniform). Workgroups
  // of the second round on a compute unit take the roles rotated by two
  // SIMDs, so two co-resident workgroups put an MFMA wave and a staging wave
  // on every SIMD.
  const int w = __builtin_amdgcn_readfirstlane(((tid >> 6) + 2 * ((blockIdx.x >> 8) & 1)) & 3);
  const int l = tid & 63;
  const int lc = l & 31;
  const int lh = l >> 5;

  const int P = a.P;
  const int units = a.BH * P;
  int* const flags = a.sync;
  // Work unit. With several segments the unit comes from a ticket counter,
  // so tickets follow dispatch order: a workgroup only ever waits for
  // segments of lower tickets, whose workgroups are already running and
  // publish their sums without waiting themselves. When the heads split
  // evenly, workgroups are grouped by blockIdx % 8 (the XCD a workgroup
  // is dispatched to) with one counter per group, and group g serves heads
  // g, g + 8, ...: all segments of a head then share one XCD, and the
  // ticket argument holds within each group.
  if (tid == 0) {
    s_wait_failed = 0;
    if (P == 1) {
      s_unit = static_cast<int>(blockIdx.x);
    } else if (o2s::grouped(a.BH, P)) {
      const int g = static_cast<int>(blockIdx.x % kGroups);
      const int t = atomicAdd(flags + ctr_base(units) + kCtrStride * (1 + g), 1);
      s_unit = o2s::ticket_unit(t, g, P);
    } else {
      s_unit = atomicAdd(flags + ctr_base(units), 1);
    }
  }
  __syncthreads();
  const int unit = __builtin_amdgcn_readfirstlane(s_unit);
  if (unit >= units) return;
  const int bh = unit / P;
  const int p = unit - bh * P;
  const bool want_out = a.o != nullptr;
  const bool want_state = a.S != nullptr && p == P - 1;
  const bool publish = p < P - 1;  // later segments of the head read this one's sum
  if (!want_out && !want_state && !publish) return;
  const int N = a.N;
  const int t0 = p * a.L;
  const int t1 = min(N, t0 + a.L);
  const int nch = (t1 - t0 + C - 1) / C;
  const float inv_a = a.inv_a;

  const __bf16* qh = reinterpret_cast<const __bf16*>(a.q) + static_cast<size_t>(bh) * N * D;
  const __bf16* kh = reinterpret_cast<const __bf16*>(a.k) + static_cast<size_t>(bh) * N * D;
  const __bf16* vh = reinterpret_cast<const __bf16*>(a.v) + static_cast<size_t>(bh) * N * DV;

  // ---------------------------------------------------------------- roles
  // M waves: state S[ft] (rows 32 ft + acc_row, column 32 w + lc).
  f32x16 S[NFT];
  // Q wave: Z (row acc_row, column lc).
  f32x16 Z;
  // prefetch registers of the staging waves
  uint4 pq[PD];
  uint4 pk[PD];
  uint4 pv[PD][4];

  // staging helpers ---------------------------------------------------------
  // Loads go through buffer resources bounded by the segment: rows past its
  // end (and chunks past the last) read as zero in hardware, so every call
  // issues its loads unconditionally and the wait counts stay exact.
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);
  const auto rq = make_rsrc(qh + static_cast<size_t>(t0) * D, seg_rows * D * 2);
  const auto rk = make_rsrc(kh + static_cast<size_t>(t0) * D, seg_rows * D * 2);
  const auto rv = make_rsrc(vh + static_cast<size_t>(t0) * DV, seg_rows * DV * 2);
  // row index of chunk c, clamped so the byte offset cannot wrap
  auto crow = [&](int c, int row) __attribute__((always_inline)) -> uint32_t {
    const int r = c * C + row;
    return static_cast<uint32_t>(r < static_cast<int>(seg_rows) ? r : static_cast<int>(seg_rows));
  };
  // Q wave: lane l loads row l>>1, half l&1 (16 bytes) of the chunk's Q.
  auto load_q = [&](int c) __attribute__((always_inline)) -> uint4 {
    return bload16(rq, (crow(c, l >> 1) * D + 8 * (l & 1)) * 2);
  };
  // K wave: K the same way; V item k covers rows 8k..8k+7, lane l holds
  // row 8k + (l&7), columns 8 (l>>3) .. +8.
  auto load_k = [&](int c) __attribute__((always_inline)) -> uint4 {
    return bload16(rk, (crow(c, l >> 1) * D + 8 * (l & 1)) * 2);
  };
  auto load_v = [&](int c, int k) __attribute__((always_inline)) -> uint4 {
    return bload16(rv, (crow(c, 8 * k + (l & 7)) * DV + 8 * (l >> 3)) * 2);
  };

  // Q wave: write chunk c's Q rows (ring slot SL) to buffer b, refill the
  // slot with chunk c + PD, then build phi~(Q) in operand order.
  auto produce_q = [&](int c, int b, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    {
      const int row = l >> 1, half = l & 1;
      *reinterpret_cast<uint4*>(sm.qp(b) + row * QP_P + 8 * half) = pq[SL];
      pq[SL] = load_q(c + PD);
    }
    const bf16x8 qa = ld8(sm.qp(b) + lc * QP_P + 8 * lh);
    const bf16x8 qb = ld8(sm.qp(b) + lc * QP_P + 8 * (1 - lh));
    float qr[16];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qr[s] = static_cast<float>(qa[s]) * inv_a;
      qr[8 + s] = static_cast<float>(qb[s]) * inv_a;
    }
    __bf16* dst = sm.fq(b) + lc * FQ_P + 8 * lh;
#pragma unroll
    for (int K = 0; K < 10; ++K) {
      bf16x8 out;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float x;
        if (K == 9)
          x = qr[s];
        else if (K == 8)
          x = lh ? (s == 0 ? 1.f : 0.f) : qr[s] * qr[s + 8];
        else if (K == 0)
          x = 0.5f * qr[s] * qr[s];
        else
          x = qr[s] * qr[(s + K) & 15];
        out[s] = static_cast<__bf16>(x);
      }
      st8(dst + 16 * K, out);
    }
  };

  // K wave: write chunk c's K, K'^T (with the valid-key row) and V^T to
  // buffer b, advance the ring, then build phi(K)^T.
  int fk_i[NFT], fk_j[NFT];
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft) {
    const Feat e = feat(32 * ft + lc);
    fk_i[ft] = e.i;
    fk_j[ft] = e.j;
  }
  auto produce_k = [&](int c, int b, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    {
      const int row = l >> 1, half = l & 1;
      *reinterpret_cast<uint4*>(sm.kr(b) + row * K_P + 8 * half) = pk[SL];
      const bf16x8 e = __builtin_bit_cast(bf16x8, pk[SL]);
      const f16x8 eh = to_h8(e);
      _Float16* kt = sm.kt(b);
#pragma unroll
      for (int u = 0; u < 8; ++u) kt[(8 * half + u) * KF_P + row] = eh[u];
      if (half == 0) kt[16 * KF_P + row] = static_cast<_Float16>(t0 + c * C + row < t1 ? 1.f : 0.f);
      _Float16* vt = sm.vt(b);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int vrow = 8 * k + (l & 7), c8 = l >> 3;
        const f16x8 ev = to_h8(__builtin_bit_cast(bf16x8, pv[SL][k]));
#pragma unroll
        for (int u = 0; u < 8; ++u) vt[(8 * c8 + u) * VT_P + vrow] = ev[u];
      }
      pk[SL] = load_k(c + PD);
#pragma unroll
      for (int k = 0; k < 4; ++k) pv[SL][k] = load_v(c + PD, k);
    }
    const _Float16* kt = sm.kt(b);
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f16x8 x = ldh8(kt + fk_i[ft] * KF_P + 16 * u + 8 * lh);
        const f16x8 y = ldh8(kt + fk_j[ft] * KF_P + 16 * u + 8 * lh);
        *reinterpret_cast<f16x8*>(sm.fk(b) + (32 * ft + lc) * FK_P + 16 * u + 8 * lh) = x * y;
      }
    }
  };

  // Q wave: Z += K'_c^T K'_c from buffer b.
  auto z_update = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // rows 18..31 of K' are zero
      const f16x8 x = ldh8(sm.kt(b) + (lc < 18 ? lc : 17) * KF_P + 16 * u + 8 * lh);
      Z = mfma32h(x, x, Z);
    }
  };

  // Q wave: inter-chunk denominator of the queries in buffer b from Z.
  // The count of earlier keys, Z[16][16] (weight 1), stays outside the bf16
  // contraction: lane 16 holds it in element 8 (row acc_row(8, 0) = 16), in
  // fp32 and exact; every other entry of Z~ is rounded to bf16 once, as the
  // state is in the read-out.
  auto den_inter = [&](int b) __attribute__((always_inline)) {
    const float z00 = __shfl(Z[8], 16);
    f32x16 dq = f32x16{};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 hi;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = 8 * u + s;
        const float x = Z[j] * zscale(lc, acc_row(j, lh), inv_a);
        hi[s] = static_cast<__bf16>(j == 8 && l == 16 ? 0.f : x);
      }
      const __bf16* qrow = sm.qp(b) + lc * QP_P;
      const bf16x8 bq = cat44(ld4(qrow + 16 * u + 4 * lh), ld4(qrow + 16 * u + 8 + 4 * lh));
      dq = mfma32(hi, bq, dq);
    }
    const __bf16* qrow = sm.qp(b) + lc * QP_P;
    float part = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const bf16x4 qv = ld4(qrow + 8 * bb + 4 * lh);
#pragma unroll
      for (int r = 0; r < 4; ++r) part += dq[4 * bb + r] * static_cast<float>(qv[r]);
    }
    part += __shfl_xor(part, 32);
    if (lh == 0) sm.den(b)[lc] = part + z00;
  };

  // M wave: constants of the intra-chunk weights, evaluated two at a time in
  // packed fp16 (the precision P has in its MFMA), and per lane the causal
  // mask of accumulator elements 2j, 2j + 1 as a bit mask of the packed pair
  // (key after query: all bits clear). The mask is applied with a bitwise
  // AND, so a masked weight is exactly 0 even where the weight itself would
  // overflow fp16 (a multiply by 0 would turn inf into NaN).
  const f16x2 one_h = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  const f16x2 half_h = {static_cast<_Float16>(0.5f), static_cast<_Float16>(0.5f)};
  uint32_t cmask[8];
#pragma unroll
  for (int j2 = 0; j2 < 8; ++j2)
    cmask[j2] = (acc_row(2 * j2, lh) > lc ? 0u : 0xFFFFu) | (acc_row(2 * j2 + 1, lh) > lc ? 0u : 0xFFFF0000u);

  // M wave: one chunk from buffer b. OUT: read out and store the chunk's
  // outputs; UPD: fold the chunk into S.
  auto m_chunk = [&](int i, bool out, bool upd) __attribute__((always_inline)) {
    const int b = i & 1;
    const int m = w;
    if (out) {
      // score tile D[key][query] = K Q^T (both raw), weights and mask
      const bf16x8 kf = ld8(sm.kr(b) + lc * K_P + 8 * lh);
      const bf16x8 qf = ld8(sm.qp(b) + lc * QP_P + 8 * lh);
      const f32x16 sc = mfma32(kf, qf, f32x16{});
      // weights 1 + t + t^2/2 of t = y/a for the raw scores y = q.k: t is
      // formed in fp32 (so any y whose t fits fp16 is fine, and 1/a is not
      // rounded), then the polynomial runs two per packed fp16 instruction;
      // the denominator sums the same fp16 weights the P V product uses, in
      // fp32
      f16x8 P0, P1;
      float den = 0.f;
#pragma unroll
      for (int j2 = 0; j2 < 8; ++j2) {
        const f16x2 t = __builtin_convertvector(f32x2{sc[2 * j2] * inv_a, sc[2 * j2 + 1] * inv_a}, f16x2);
        const f16x2 wv = __builtin_bit_cast(
            f16x2, __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_elementwise_fma(half_h, t, one_h),
                                                                          t, one_h)) &
                       cmask[j2]);
        den = __builtin_amdgcn_fdot2(wv, one_h, den, false);
        if (j2 < 4) {
          P0[2 * j2] = wv[0];
          P0[2 * j2 + 1] = wv[1];
        } else {
          P1[2 * j2 - 8] = wv[0];
          P1[2 * j2 - 7] = wv[1];
        }
      }
      // read-out: O^T[dv][query] = S^T phi~(Q)^T over 10 k-steps
      f32x16 O = f32x16{};
      const __bf16* fq = sm.fq(b) + lc * FQ_P + 8 * lh;
#pragma unroll
      for (int K = 0; K < 10; ++K) {
        const int ft = K >> 1, u = K & 1;
        bf16x8 sa;
#pragma unroll
        for (int s = 0; s < 8; ++s) sa[s] = static_cast<__bf16>(S[ft][8 * u + s]);
        O = mfma32(sa, ld8(fq + 16 * K), O);
      }
      // intra-chunk term: O^T += V^T P^T, keys in the accumulator order
      const _Float16* vrow = sm.vt(b) + (32 * m + lc) * VT_P;
      O = mfma32h(cath44(ldh4(vrow + 4 * lh), ldh4(vrow + 8 + 4 * lh)), P0, O);
      O = mfma32h(cath44(ldh4(vrow + 16 + 4 * lh), ldh4(vrow + 24 + 4 * lh)), P1, O);
      den += __shfl_xor(den, 32);
      den += sm.den(b)[lc];
      const float rd = __builtin_amdgcn_rcpf(den);
      // normalise, transpose through this wave's LDS area, store rows
      char* st = sm.ostage(m, OB);
      const int rows = min(C, t1 - (t0 + i * C));
      const size_t orow0 = static_cast<size_t>(bh) * N + t0 + i * C;
      if constexpr (OBF) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          bf16x4 ov;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = static_cast<__bf16>(O[4 * bb + r] * rd);
          *reinterpret_cast<bf16x4*>(st + (lc * OP + 8 * bb + 4 * lh) * 2) = ov;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int e = l + 64 * k, row = e >> 2, c4 = e & 3;
          const uint4 x = *reinterpret_cast<const uint4*>(st + (row * OP + 8 * c4) * 2);
          if (row < rows)
            *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(a.o) + (orow0 + row) * DV + 32 * m + 8 * c4) = x;
        }
      } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          f32x4 ov;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = O[4 * bb + r] * rd;
          *reinterpret_cast<f32x4*>(st + (lc * OP + 8 * bb + 4 * lh) * 4) = ov;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = l + 64 * k, row = e >> 3, c8 = e & 7;
          const uint4 x = *reinterpret_cast<const uint4*>(st + (row * OP + 4 * c8) * 4);
          if (row < rows)
            *reinterpret_cast<uint4*>(reinterpret_cast<float*>(a.o) + (orow0 + row) * DV + 32 * m + 4 * c8) = x;
        }
      }
    }
    if (upd) {
      const _Float16* vrow = sm.vt(b) + (32 * m + lc) * VT_P;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f16x8 bv = ldh8(vrow + 16 * u + 8 * lh);
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
          S[ft] = mfma32h(ldh8(sm.fk(b) + (32 * ft + lc) * FK_P + 16 * u + 8 * lh), bv, S[ft]);
      }
    }
  };

  // One pass over the segment's chunks. Chunk i is consumed by the M waves
  // from buffer i&1 while the Q and K waves prepare chunk i+1 in the other
  // buffer; one barrier per chunk. Each role runs its own loop so the
  // compiler's wait counts see only that role's memory operations. OUT
  // selects the output pass (read-out, outputs, Q staging); without it the
  // pass only sums the segment's state (S and Z).
  static_assert(PD == 2, "the chunk loops below are unrolled for two ring slots");
  using S0_ = std::integral_constant<int, 0>;
  using S1_ = std::integral_constant<int, 1>;
  auto pass = [&](auto out_tag) __attribute__((always_inline)) {
    constexpr bool OUT = decltype(out_tag)::value;
    const bool qout = OUT && want_out;
    // prologue: fill the prefetch rings and prepare chunk 0
    if (w == 2 && qout) {
      pq[0] = load_q(0);
      pq[1] = load_q(1);
      produce_q(0, 0, S0_{});
    }
    if (w == 3) {
      pk[0] = load_k(0);
      pk[1] = load_k(1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pv[0][k] = load_v(0, k);
        pv[1][k] = load_v(1, k);
      }
      produce_k(0, 0, S0_{});
    }
    __syncthreads();
    if (w == 2 && qout) den_inter(0);
    __syncthreads();
    // On its last iteration each staging loop loads and builds an empty
    // chunk into the idle buffer, which keeps its loads per iteration fixed.
    if (w < 2) {
      for (int i = 0; i < nch; ++i) {
        const bool last = i + 1 == nch;
        m_chunk(i, qout, !OUT || !last || want_state);
        __syncthreads();
      }
    } else if (w == 2) {
      if (qout) {
        auto q_it = [&](int i, auto slot) __attribute__((always_inline)) {
          const int b = i & 1, nb = b ^ 1;
          produce_q(i + 1, nb, slot);
          z_update(b);
          den_inter(nb);
        };
        int i = 0;
        for (; i + 2 <= nch; i += 2) {
          q_it(i, S1_{});
          __syncthreads();
          q_it(i + 1, S0_{});
          __syncthreads();
        }
        if (i < nch) {
          q_it(i, S1_{});
          __syncthreads();
        }
      } else {
        for (int i = 0; i < nch; ++i) {
          z_update(i & 1);
          __syncthreads();
        }
      }
    } else {
      auto k_it = [&](int i, auto slot) __attribute__((always_inline)) { produce_k(i + 1, (i & 1) ^ 1, slot); };
      int i = 0;
      for (; i + 2 <= nch; i += 2) {
        k_it(i, S1_{});
        __syncthreads();
        k_it(i + 1, S0_{});
        __syncthreads();
      }
      if (i < nch) {
        k_it(i, S1_{});
        __syncthreads();
      }
    }
  };

  float4* const segu = reinterpret_cast<float4*>(a.seg);
  auto unit_ptr = [&](int q) __attribute__((always_inline)) {
    return segu + (static_cast<size_t>(bh) * (P - 1) + q) * UNIT_F4;
  };
  // float4 index of (value half h, feature tile ft, register quad q4, lane)
  auto unit_idx = [&](int h, int ft, int q4) __attribute__((always_inline)) { return ((h * NFT + ft) * 4 + q4) * 64 + l; };
  constexpr int ZIDX = 2 * NFT * 4 * 64;
  // Published sums are written and read with device-scope (sc1) buffer
  // accesses, so the flag needs only the stores' completion before it and
  // no cache write-back or invalidation around it.
  auto st_dev = [&](__amdgpu_buffer_rsrc_t r, int idx, const f32x16& x, int q4) __attribute__((always_inline)) {
    const f32x4 v{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, idx * 16, 0, kDeviceScope);
  };
  auto ld_dev = [&](__amdgpu_buffer_rsrc_t r, int idx) __attribute__((always_inline)) -> f32x4 {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, idx * 16, 0, kDeviceScope));
  };

  // phase 1: this segment's own sum, published for the later segments ------
  if (publish) {
    constexpr int C1 = s1::C, P1 = s1::P, NV = s1::NV;
    auto kt1 = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem_raw + b * s1::BUF); };
    auto vt1 = [&](int b) __attribute__((always_inline)) {
      return reinterpret_cast<_Float16*>(smem_raw + b * s1::BUF + s1::KROWS * P1 * 2);
    };
    // V^T row r keeps its 8-token groups XOR-swizzled by r's group of eight,
    // which spreads the transposing 2-byte writes over the banks.
    auto vpos = [&](int r, int t) __attribute__((always_inline)) { return t ^ (8 * ((r >> 3) & 7)); };
    for (int i = tid; i < 2 * C1; i += NTHR) kt1(i / C1)[17 * P1 + i % C1] = static_cast<_Float16>(0.f);
    auto crow1 = [&](int c, int row) __attribute__((always_inline)) -> uint32_t {
      const int r = c * C1 + row;
      return static_cast<uint32_t>(r < static_cast<int>(seg_rows) ? r : static_cast<int>(seg_rows));
    };
    uint4 r1[2][1 + NV];
    auto load1 = [&](int c, uint4* dst) __attribute__((always_inline)) {
      dst[0] = bload16(rk, (crow1(c, tid >> 1) * D + 8 * (tid & 1)) * 2);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int j = tid + NTHR * k;
        dst[1 + k] = bload16(rv, (crow1(c, j >> 3) * DV + 8 * (j & 7)) * 2);
      }
    };
    auto stage1 = [&](int c, int b, auto slot) __attribute__((always_inline)) {
      constexpr int SL = decltype(slot)::value;
      {
        const int row = tid >> 1, half = tid & 1;
        const f16x8 e = to_h8(__builtin_bit_cast(bf16x8, r1[SL][0]));
        _Float16* kt = kt1(b);
#pragma unroll
        for (int u = 0; u < 8; ++u) kt[(8 * half + u) * P1 + row] = e[u];
        if (half == 0) kt[16 * P1 + row] = static_cast<_Float16>(c * C1 + row < static_cast<int>(seg_rows) ? 1.f : 0.f);
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int j = tid + NTHR * k, row = j >> 3, c8 = j & 7;
        const f16x8 e = to_h8(__builtin_bit_cast(bf16x8, r1[SL][1 + k]));
        _Float16* vt = vt1(b);
#pragma unroll
        for (int u = 0; u < 8; ++u) vt[(8 * c8 + u) * P1 + vpos(8 * c8 + u, row)] = e[u];
      }
      load1(c + 2, r1[SL]);
    };
    // Accumulators: wave w owns feature tile w for both value halves (A0,
    // A1); the third one (A2) is tile 4 for value half w on waves 0 and 1,
    // Z on wave 2 (K'^T row r times the valid-key row, i.e. K' itself), and
    // unused on wave 3. The rows are chosen per lane so that every wave runs
    // the same instructions.
    const int ftw = w;
    const Feat fw = feat(32 * ftw + lc), f4 = feat(32 * 4 + lc);
    const int ra = w < 2 ? f4.i : (w == 2 ? (lc < 18 ? lc : 17) : 17);
    const int rb = w < 2 ? f4.j : (w == 2 ? 16 : 17);
    // B operand of A2: V^T row 32w + lc (waves 0, 1) or K'^T row ra (wave 2)
    const int xrow = w < 2 ? 32 * w + lc : ra;
    const int xoff = w < 2 ? s1::KROWS * P1 + xrow * P1 : xrow * P1;
    const int xsw = w < 2 ? 8 * ((xrow >> 3) & 7) : 0;
    f32x16 A0 = f32x16{}, A1 = f32x16{}, A2 = f32x16{};
    auto compute1 = [&](int b) __attribute__((always_inline)) {
      const _Float16* kt = kt1(b);
      const _Float16* vt = vt1(b);
#pragma unroll
      for (int u = 0; u < C1 / 16; ++u) {
        const int tk = 16 * u + 8 * lh;
        const f16x8 af = ldh8(kt + fw.i * P1 + tk) * ldh8(kt + fw.j * P1 + tk);
        const f16x8 b0 = ldh8(vt + lc * P1 + vpos(lc, tk));
        const f16x8 b1 = ldh8(vt + (32 + lc) * P1 + vpos(32 + lc, tk));
        const f16x8 xa = ldh8(kt + ra * P1 + tk) * ldh8(kt + rb * P1 + tk);
        const f16x8 xb = ldh8(kt + xoff + (tk ^ xsw));
        A0 = mfma32h(af, b0, A0);
        A1 = mfma32h(af, b1, A1);
        A2 = mfma32h(xa, xb, A2);
      }
    };
    using T0_ = std::integral_constant<int, 0>;
    using T1_ = std::integral_constant<int, 1>;
    const int nch1 = (static_cast<int>(seg_rows) + C1 - 1) / C1;
    load1(0, r1[0]);
    load1(1, r1[1]);
    stage1(0, 0, T0_{});
    __syncthreads();
    int i = 0;
    for (; i + 2 <= nch1; i += 2) {
      stage1(i + 1, 1, T1_{});
      compute1(0);
      __syncthreads();
      stage1(i + 2, 0, T0_{});
      compute1(1);
      __syncthreads();
    }
    if (i < nch1) {
      stage1(i + 1, 1, T1_{});
      compute1(0);
      __syncthreads();
    }
    const auto ru = make_rsrc(unit_ptr(p), static_cast<uint32_t>(UNIT_BYTES));
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      st_dev(ru, unit_idx(0, ftw, q4), A0, q4);
      st_dev(ru, unit_idx(1, ftw, q4), A1, q4);
      if (w < 2) st_dev(ru, unit_idx(w, 4, q4), A2, q4);
      if (w == 2) st_dev(ru, ZIDX + q4 * 64 + l, A2, q4);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flags + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!want_out) return;
  }

  // phase 2: initial state = S0 + the sums of segments 0..p-1 ---------------
  if (p > 0 && tid < 64) {
    // The first 64 threads poll up to 64 flags at once (one device-scope
    // load each; a flag read costs a memory round trip) until a wave vote
    // finds them all set. The wait is bounded (about a second): if it ends
    // with a flag still clear, the unit's initial state is set to NaN below,
    // so every output row of the unit (and, for the last segment, the final
    // state) comes out NaN instead of silently wrong, and the workgroup
    // still ends.
    int spins = 0;
    bool all_set = true;
    for (int q0 = 0; q0 < p; q0 += 64) {
      const int q = q0 + tid;
      while (true) {
        const int f = q < p ? __hip_atomic_load(flags + bh * P + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
        if (__all(f != 0)) break;
        if (++spins >= a.wait_spins) {
          all_set = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (tid == 0) s_wait_failed = all_set ? 0 : 1;
  }
  __syncthreads();
  if (p == 0) {
    if (w < 2) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) S[ft] = f32x16{};
    } else if (w == 2) {
      Z = f32x16{};
    }
  } else {
    // All four waves add up the earlier sums: wave w takes float4 items
    // [w RQ, (w+1) RQ) of every sum, with two sums' loads in flight at a
    // time, and leaves the total in LDS (free until phase 3) in the unit
    // layout, from which the owning waves read their accumulators.
    constexpr int RQ = UNIT_F4 / 4;
    constexpr int RJ = RQ / 64;
    static_assert(RQ % 64 == 0 && UNIT_BYTES <= static_cast<size_t>(lds_bytes<true>()) &&
                      UNIT_BYTES <= static_cast<size_t>(lds_bytes<false>()),
                  "whole float4 items per lane; the total fits the kernel's LDS");
    f32x4 acc[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int i0 = w * RQ + l;
    int q = 0;
    for (; q + 2 <= p; q += 2) {
      const auto r0 = make_rsrc(unit_ptr(q), static_cast<uint32_t>(UNIT_BYTES));
      const auto r1 = make_rsrc(unit_ptr(q + 1), static_cast<uint32_t>(UNIT_BYTES));
      f32x4 x0[RJ], x1[RJ];
#pragma unroll
      for (int j = 0; j < RJ; ++j) x0[j] = ld_dev(r0, i0 + 64 * j);
#pragma unroll
      for (int j = 0; j < RJ; ++j) x1[j] = ld_dev(r1, i0 + 64 * j);
#pragma unroll
      for (int j = 0; j < RJ; ++j) acc[j] += x0[j] + x1[j];
    }
    if (q < p) {
      const auto r0 = make_rsrc(unit_ptr(q), static_cast<uint32_t>(UNIT_BYTES));
#pragma unroll
      for (int j = 0; j < RJ; ++j) acc[j] += ld_dev(r0, i0 + 64 * j);
    }
    f32x4* const tot = reinterpret_cast<f32x4*>(smem_raw);
#pragma unroll
    for (int j = 0; j < RJ; ++j) tot[i0 + 64 * j] = acc[j];
    __syncthreads();
    if (w < 2) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 x = tot[unit_idx(w, ft, q4)];
#pragma unroll
          for (int r = 0; r < 4; ++r) S[ft][4 * q4 + r] = x[r];
        }
    } else if (w == 2) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 x = tot[ZIDX + q4 * 64 + l];
#pragma unroll
        for (int r = 0; r < 4; ++r) Z[4 * q4 + r] = x[r];
      }
    }
    __syncthreads();  // the area is reused below
  }
  if (w < 2 && a.S0 != nullptr) {
    const int col = 32 * w + lc;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const Feat e = feat(32 * ft + acc_row(j, lh));
        if (e.can >= 0) S[ft][j] += a.S0[(static_cast<size_t>(bh) * 153 + e.can) * DV + col] / e.wcan;
      }
  } else if (w == 2 && a.z0 != nullptr) {
    const float* z0 = a.z0 + static_cast<size_t>(bh) * 153;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = acc_row(j, lh), c = lc;
      float x = 0.f;
      if (r < 16 && c < 16) {
        const int lo = r < c ? r : c, hi = r < c ? c : r;
        x = z0[17 + lo * 16 - lo * (lo - 1) / 2 + (hi - lo)] / (r == c ? 1.f : kSqrt2);
      } else if ((r < 16 && c == 16) || (r == 16 && c < 16)) {
        x = z0[1 + (r < c ? r : c)];
      } else if (r == 16 && c == 16) {
        x = z0[0];
      }
      Z[j] += x;
    }
  }

  // a timed-out wait poisons the unit (see the wait above)
  if (s_wait_failed) {
    const float nan = __builtin_nanf("");
    if (w < 2) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int j = 0; j < 16; ++j) S[ft][j] = nan;
    } else if (w == 2) {
#pragma unroll
      for (int j = 0; j < 16; ++j) Z[j] = nan;
    }
  }

  // constant parts of both phase-3 buffers: Q' columns 16..31 = (1, 0, ...);
  // K'^T row 17 = 0.
  for (int i = tid; i < 2 * C * 16; i += NTHR) {
    const int b = i / (C * 16), rest = i % (C * 16), row = rest / 16, col = 16 + rest % 16;
    sm.qp(b)[row * QP_P + col] = static_cast<__bf16>(col == 16 ? 1.f : 0.f);
  }
  for (int i = tid; i < 2 * KF_P; i += NTHR) sm.kt(i / KF_P)[17 * KF_P + i % KF_P] = static_cast<_Float16>(0.f);
  __syncthreads();  // the K wave reads row 17 while building chunk 0

  // phase 3: outputs (and, for the last segment, the final state) -----------
  pass(std::true_type{});

  if (!want_state) return;
  if (a.defer_state) {
    float4* dst = reinterpret_cast<float4*>(a.fin) + static_cast<size_t>(bh) * UNIT_F4;
    if (w < 2) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dst[unit_idx(w, ft, q4)] = float4{S[ft][4 * q4], S[ft][4 * q4 + 1], S[ft][4 * q4 + 2], S[ft][4 * q4 + 3]};
    } else if (w == 2) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        dst[ZIDX + q4 * 64 + l] = float4{Z[4 * q4], Z[4 * q4 + 1], Z[4 * q4 + 2], Z[4 * q4 + 3]};
    }
  } else if (w < 2) {
    const int col = 32 * w + lc;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const Feat e = feat(32 * ft + acc_row(j, lh));
        if (e.can >= 0) a.S[(static_cast<size_t>(bh) * 153 + e.can) * DV + col] = e.wcan * S[ft][j];
      }
  } else if (w == 2) {
    float* z = a.z + static_cast<size_t>(bh) * 153;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = acc_row(j, lh), c = lc;
      if (r < 16 && c < 16 && r <= c)
        z[17 + r * 16 - r * (r - 1) / 2 + (c - r)] = (r == c ? 1.f : kSqrt2) * Z[j];
      else if (r < 16 && c == 16)
        z[1 + r] = Z[j];
      else if (r == 16 && c == 16)
        z[0] = Z[j];
    }
  }
}

// Final state from the staging area (internal layout) to S, z (canonical).
__global__ __launch_bounds__(192) void o2_state_store(const float4* fin, float* S, float* z) {
  const int bh = blockIdx.x;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lc = l & 31, lh = l >> 5;
  const float4* src = fin + static_cast<size_t>(bh) * UNIT_F4;
  if (w < 2) {
    const int col = 32 * w + lc;
    for (int ft = 0; ft < NFT; ++ft)
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = src[((w * NFT + ft) * 4 + q4) * 64 + l];
        const float v[4] = {x.x, x.y, x.z, x.w};
        for (int r = 0; r < 4; ++r) {
          const Feat e = feat(32 * ft + acc_row(4 * q4 + r, lh));
          if (e.can >= 0) S[(static_cast<size_t>(bh) * 153 + e.can) * DV + col] = e.wcan * v[r];
        }
      }
  } else {
    float* zz = z + static_cast<size_t>(bh) * 153;
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x = src[(2 * NFT * 4 + q4) * 64 + l];
      const float v[4] = {x.x, x.y, x.z, x.w};
      for (int rr = 0; rr < 4; ++rr) {
        const int r = acc_row(4 * q4 + rr, lh), c = lc;
        if (r < 16 && c < 16 && r <= c)
          zz[17 + r * 16 - r * (r - 1) / 2 + (c - r)] = (r == c ? 1.f : kSqrt2) * v[rr];
        else if (r < 16 && c == 16)
          zz[1 + r] = v[rr];
        else if (r == 16 && c == 16)
          zz[0] = v[rr];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool plan(int BH, int N, PrefillPlan* pl) {
  *pl = PrefillPlan{};
  // about two workgroups per compute unit, at least 8 chunks per segment,
  // 32-bit buffer ranges per segment
  const Split sp = split_segments(BH, N, C, 512, 1, 8, DV * 2);
  pl->P = sp.P;
  pl->L = sp.L;
  if (BH <= 0 || N == 0) return true;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  pl->seg_off = off;
  if (pl->P > 1) off += al(static_cast<size_t>(BH) * (pl->P - 1) * UNIT_BYTES);
  pl->fin_off = off;
  if (pl->P > 1) off += al(static_cast<size_t>(BH) * UNIT_BYTES);
  pl->part_off = off;
  if (pl->P > 1) {
    pl->sync_off = off;
    off += al(static_cast<size_t>(sync_ints(static_cast<int>(BH * pl->P))) * sizeof(int));
  }
  pl->bytes = off;
  return true;
}

hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  hipError_t e;
  const int units = a.BH * a.P;
  if (a.P > 1) {
    hipLaunchKernelGGL(o2_reset, dim3(1), dim3(256), 0, stream, a.sync, sync_ints(units));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.o == nullptr || a.out_bf16)
    hipLaunchKernelGGL((o2_kernel<true>), dim3(units), dim3(NTHR), 0, stream, a);
  else
    hipLaunchKernelGGL((o2_kernel<false>), dim3(units), dim3(NTHR), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.defer_state && a.S != nullptr) {
    hipLaunchKernelGGL(o2_state_store, dim3(a.BH), dim3(192), 0, stream,
                       reinterpret_cast<const float4*>(a.fin), a.S, a.z);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace o2
}  // namespace tl
