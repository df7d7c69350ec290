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
// zero) and its read-out uses a hi/lo bf16 split so the count z_0 is not
// rounded to 8 bits.
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
// PD chunks ahead in registers. Segments of a head are independent given
// the sum of the earlier segments' states (additivity, closing paragraph of
// the same page): a first launch computes per-segment sums, a second turns
// them into inclusive prefixes, the main launch reads one prefix each.
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

enum { SEGSUM = 0, MAIN = 1 };

template <int MODE, bool OBF>
__global__ __launch_bounds__(NTHR, 2) void o2_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem_raw[lds_bytes<OBF>()];
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

  const int PL = MODE == MAIN ? a.P : a.P - 1;
  const int unit = blockIdx.x;
  if (unit >= a.BH * PL) return;
  const int bh = unit / PL;
  const int p = unit - bh * PL;
  const bool want_out = MODE == MAIN && a.o != nullptr;
  const bool want_state = MODE == MAIN && a.S != nullptr && p == a.P - 1;
  if (MODE == MAIN && !want_out && !want_state) return;
  const int N = a.N;
  const int t0 = p * a.L;
  const int t1 = min(N, t0 + a.L);
  const int nch = (t1 - t0 + C - 1) / C;
  const float inv_a = a.inv_a;

  const __bf16* qh = reinterpret_cast<const __bf16*>(a.q) + static_cast<size_t>(bh) * N * D;
  const __bf16* kh = reinterpret_cast<const __bf16*>(a.k) + static_cast<size_t>(bh) * N * D;
  const __bf16* vh = reinterpret_cast<const __bf16*>(a.v) + static_cast<size_t>(bh) * N * DV;

  // constant parts of both buffers: Q' columns 16..31 = (1, 0, ...);
  // K'^T row 17 = 0.
  for (int i = tid; i < 2 * C * 16; i += NTHR) {
    const int b = i / (C * 16), rest = i % (C * 16), row = rest / 16, col = 16 + rest % 16;
    sm.qp(b)[row * QP_P + col] = static_cast<__bf16>(col == 16 ? 1.f : 0.f);
  }
  for (int i = tid; i < 2 * KF_P; i += NTHR) sm.kt(i / KF_P)[17 * KF_P + i % KF_P] = static_cast<_Float16>(0.f);
  __syncthreads();

  // ---------------------------------------------------------------- roles
  // M waves: state S[ft] (rows 32 ft + acc_row, column 32 w + lc).
  f32x16 S[NFT];
  // Q wave: Z (row acc_row, column lc).
  f32x16 Z;
  // prefetch registers of the staging waves
  uint4 pq[PD];
  uint4 pk[PD];
  uint4 pv[PD][4];

  const float4* segp = reinterpret_cast<const float4*>(a.seg);

  // initial state ----------------------------------------------------------
  if (w < 2) {
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) S[ft] = f32x16{};
    if (MODE == MAIN) {
      if (p > 0) {
        const float4* src = segp + (static_cast<size_t>(bh) * (a.P - 1) + (p - 1)) * UNIT_F4 +
                            (static_cast<size_t>(w) * NFT) * 4 * 64 + l;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 x = src[(ft * 4 + q4) * 64];
            S[ft][4 * q4 + 0] = x.x;
            S[ft][4 * q4 + 1] = x.y;
            S[ft][4 * q4 + 2] = x.z;
            S[ft][4 * q4 + 3] = x.w;
          }
      }
      if (a.S0 != nullptr) {
        const int col = 32 * w + lc;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const Feat e = feat(32 * ft + acc_row(j, lh));
            if (e.can >= 0)
              S[ft][j] += a.S0[(static_cast<size_t>(bh) * 153 + e.can) * DV + col] / e.wcan;
          }
      }
    }
  } else if (w == 2) {
    Z = f32x16{};
    if (MODE == MAIN) {
      if (p > 0) {
        const float4* src = segp + (static_cast<size_t>(bh) * (a.P - 1) + (p - 1)) * UNIT_F4 +
                            2 * NFT * 4 * 64 + l;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = src[q4 * 64];
          Z[4 * q4 + 0] = x.x;
          Z[4 * q4 + 1] = x.y;
          Z[4 * q4 + 2] = x.z;
          Z[4 * q4 + 3] = x.w;
        }
      }
      if (a.z0 != nullptr) {
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
    }
  }

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
  auto den_inter = [&](int b) __attribute__((always_inline)) {
    f32x16 dq = f32x16{};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 hi, lo;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = 8 * u + s;
        const float x = Z[j] * zscale(lc, acc_row(j, lh), inv_a);
        hi[s] = static_cast<__bf16>(x);
        lo[s] = static_cast<__bf16>(x - static_cast<float>(hi[s]));
      }
      const __bf16* qrow = sm.qp(b) + lc * QP_P;
      const bf16x8 bq = cat44(ld4(qrow + 16 * u + 4 * lh), ld4(qrow + 16 * u + 8 + 4 * lh));
      dq = mfma32(hi, bq, dq);
      dq = mfma32(lo, bq, dq);
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
    if (lh == 0) sm.den(b)[lc] = part;
  };

  // prologue: fill the prefetch ring and prepare chunk 0 ------------------
  static_assert(PD == 2, "the chunk loop below is unrolled for two ring slots");
  using S0_ = std::integral_constant<int, 0>;
  using S1_ = std::integral_constant<int, 1>;
  if (w == 2 && want_out) {
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
  if (w == 2 && want_out) den_inter(0);
  __syncthreads();

  // chunk loop ---------------------------------------------------------------
  // Iteration i: the M waves consume chunk i from buffer i&1 while the Q and
  // K waves prepare chunk i+1 (ring slot (i+1)&1) in the other buffer.
  // Each role runs its own loop (one barrier per chunk in each), so the
  // compiler's wait counts see only that role's memory operations.
  auto m_iteration = [&](int i) __attribute__((always_inline)) {
    const int b = i & 1;
    const bool last = i + 1 == nch;
    {
      const int m = w;
      const bool update = MODE == SEGSUM || !last || want_state;
      if (want_out) {
        // score tile D[key][query] = K Q^T (both raw), weights and mask
        const bf16x8 kf = ld8(sm.kr(b) + lc * K_P + 8 * lh);
        const bf16x8 qf = ld8(sm.qp(b) + lc * QP_P + 8 * lh);
        const f32x16 sc = mfma32(kf, qf, f32x16{});
        f16x8 P0, P1;
        float den = 0.f;
        const float c2 = 0.5f * inv_a * inv_a;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = acc_row(j, lh);
          // 1 + y/a + y^2/(2a^2) for the raw score y = q.k
          float wv = __builtin_fmaf(__builtin_fmaf(c2, sc[j], inv_a), sc[j], 1.f);
          if (key > lc) wv = 0.f;  // causal mask (key after query)
          const _Float16 pb = static_cast<_Float16>(wv);
          den += wv;
          if (j < 8)
            P0[j] = pb;
          else
            P1[j - 8] = pb;
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
        const float rd = 1.f / den;
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
      if (update) {
        const _Float16* vrow = sm.vt(b) + (32 * m + lc) * VT_P;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f16x8 bv = ldh8(vrow + 16 * u + 8 * lh);
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
            S[ft] = mfma32h(ldh8(sm.fk(b) + (32 * ft + lc) * FK_P + 16 * u + 8 * lh), bv, S[ft]);
        }
      }
    }
  };
  // Q and K waves: prepare chunk i+1 (on the last iteration this loads and
  // builds an empty chunk into the idle buffer, which keeps the number of
  // loads per iteration constant).
  auto q_iteration = [&](int i, auto slot) __attribute__((always_inline)) {
    const int b = i & 1, nb = b ^ 1;
    produce_q(i + 1, nb, slot);
    z_update(b);
    den_inter(nb);
  };
  auto k_iteration = [&](int i, auto slot) __attribute__((always_inline)) { produce_k(i + 1, (i & 1) ^ 1, slot); };
  if (w < 2) {
    for (int i = 0; i < nch; ++i) {
      m_iteration(i);
      __syncthreads();
    }
  } else if (w == 2) {
    if (want_out) {
      int i = 0;
      for (; i + 2 <= nch; i += 2) {
        q_iteration(i, S1_{});
        __syncthreads();
        q_iteration(i + 1, S0_{});
        __syncthreads();
      }
      if (i < nch) {
        q_iteration(i, S1_{});
        __syncthreads();
      }
    } else {
      for (int i = 0; i < nch; ++i) {
        z_update(i & 1);
        __syncthreads();
      }
    }
  } else {
    int i = 0;
    for (; i + 2 <= nch; i += 2) {
      k_iteration(i, S1_{});
      __syncthreads();
      k_iteration(i + 1, S0_{});
      __syncthreads();
    }
    if (i < nch) {
      k_iteration(i, S1_{});
      __syncthreads();
    }
  }

  // results ------------------------------------------------------------------
  float4* dstu = nullptr;
  if (MODE == SEGSUM) {
    dstu = reinterpret_cast<float4*>(a.seg) + (static_cast<size_t>(bh) * (a.P - 1) + p) * UNIT_F4;
  } else if (want_state && a.defer_state) {
    dstu = reinterpret_cast<float4*>(a.fin) + static_cast<size_t>(bh) * UNIT_F4;
  }
  if (dstu != nullptr) {
    if (w < 2) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dstu[((w * NFT + ft) * 4 + q4) * 64 + l] =
              float4{S[ft][4 * q4], S[ft][4 * q4 + 1], S[ft][4 * q4 + 2], S[ft][4 * q4 + 3]};
    } else if (w == 2) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        dstu[(2 * NFT * 4 + q4) * 64 + l] = float4{Z[4 * q4], Z[4 * q4 + 1], Z[4 * q4 + 2], Z[4 * q4 + 3]};
    }
  } else if (want_state) {
    if (w < 2) {
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
}

// Per-segment state sums (segments 0..P-2), update only: S += phi(K)^T V and
// Z += K'^T K' over the segment. Five symmetric waves; wave w owns feature
// tile w (32 features) for all 64 value columns and builds its own phi(K)^T
// fragments from an fp32 K'^T in LDS, so the work per wave is a handful of
// fragments and MFMAs per chunk and the pass runs at the speed of streaming
// K and V. Chunks of 64 tokens, two LDS buffers, loads two chunks ahead.
namespace ss {
constexpr int C = 64;
constexpr int NW = NFT;                   // one wave per 32-feature tile
constexpr int NTHR = NW * 64;
constexpr int KF_P = 72;                  // fp16 K'^T rows 0..17, 64 keys + pad
constexpr int VT_P = 72;                  // fp16 V^T rows, 64 keys + pad
constexpr int OFF_KF = 0;
constexpr int OFF_VT = 18 * KF_P * 2;
constexpr int BUF = OFF_VT + DV * VT_P * 2;
constexpr int KITEMS = C * D / 8;         // 16-byte items of K per chunk
constexpr int ITEMS = KITEMS + C * DV / 8;
constexpr int PER_T = ITEMS / NTHR;       // items per thread
static_assert(ITEMS % NTHR == 0, "whole items per thread");
static_assert(KITEMS % 64 == 0, "K items fill whole waves");
static_assert(OFF_VT % 16 == 0 && BUF % 16 == 0 && (KF_P * 2) % 16 == 0 && (VT_P * 2) % 16 == 0,
              "16-byte aligned rows");
}  // namespace ss

__global__ __launch_bounds__(ss::NTHR) void o2_segsum(PrefillArgs a) {
  constexpr int C = ss::C, NTHR = ss::NTHR, KF_P = ss::KF_P, VT_P = ss::VT_P, BUF = ss::BUF;
  constexpr int OFF_KF = ss::OFF_KF, OFF_VT = ss::OFF_VT, KITEMS = ss::KITEMS, PER_T = ss::PER_T;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lc = l & 31, lh = l >> 5;
  const int PS = a.P - 1;
  const int unit = blockIdx.x;
  if (unit >= a.BH * PS) return;
  const int bh = unit / PS;
  const int p = unit - bh * PS;
  const int N = a.N;
  const int t0 = p * a.L;
  const int t1 = min(N, t0 + a.L);
  const int nch = (t1 - t0 + C - 1) / C;
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);
  const auto rk = make_rsrc(reinterpret_cast<const __bf16*>(a.k) + (static_cast<size_t>(bh) * N + t0) * D,
                            seg_rows * D * 2);
  const auto rv = make_rsrc(reinterpret_cast<const __bf16*>(a.v) + (static_cast<size_t>(bh) * N + t0) * DV,
                            seg_rows * DV * 2);
  auto kf = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem + b * BUF + OFF_KF); };
  auto vt = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem + b * BUF + OFF_VT); };
  for (int i = tid; i < 2 * KF_P; i += NTHR) kf(i / KF_P)[17 * KF_P + i % KF_P] = static_cast<_Float16>(0.f);

  auto crow = [&](int c, int row) __attribute__((always_inline)) -> uint32_t {
    const int r = c * C + row;
    return static_cast<uint32_t>(r < static_cast<int>(seg_rows) ? r : static_cast<int>(seg_rows));
  };
  // Item e of a chunk: K rows (two 16-byte items per key) first, then V rows
  // (eight per key). Thread tid holds items tid + k*NTHR; the K items are
  // exactly slot 0 of the first KITEMS/64 waves, so the choice between the
  // two buffers is uniform per wave.
  auto is_k = [&](int k) __attribute__((always_inline)) { return k == 0 && w < KITEMS / 64; };
  auto load_item = [&](int c, int k) __attribute__((always_inline)) -> uint4 {
    const int e = tid + k * NTHR;
    if (is_k(k)) return bload16(rk, (crow(c, e >> 1) * D + 8 * (e & 1)) * 2);
    const int j = e - KITEMS;
    return bload16(rv, (crow(c, j >> 3) * DV + 8 * (j & 7)) * 2);
  };
  auto store_item = [&](int c, int b, int k, uint4 x) __attribute__((always_inline)) {
    const int e = tid + k * NTHR;
    const f16x8 v = to_h8(__builtin_bit_cast(bf16x8, x));
    if (is_k(k)) {
      const int row = e >> 1, half = e & 1;
      _Float16* kk = kf(b);
#pragma unroll
      for (int u = 0; u < 8; ++u) kk[(8 * half + u) * KF_P + row] = v[u];
      if (half == 0) kk[16 * KF_P + row] = static_cast<_Float16>(c * C + row < static_cast<int>(seg_rows) ? 1.f : 0.f);
    } else {
      const int j = e - KITEMS, row = j >> 3, c8 = j & 7;
      _Float16* t = vt(b);
#pragma unroll
      for (int u = 0; u < 8; ++u) t[(8 * c8 + u) * VT_P + row] = v[u];
    }
  };

  uint4 pf[2][PER_T];
  auto stage = [&](int c, int b, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      store_item(c, b, k, pf[SL][k]);
      pf[SL][k] = load_item(c + 2, k);
    }
  };

  const Feat fe = feat(32 * w + lc);
  f32x16 S0 = f32x16{}, S1 = f32x16{}, Z = f32x16{};
  auto compute = [&](int b) __attribute__((always_inline)) {
    const _Float16* k = kf(b);
    const _Float16* v = vt(b);
#pragma unroll
    for (int u = 0; u < C / 16; ++u) {
      const f16x8 af = ldh8(k + fe.i * KF_P + 16 * u + 8 * lh) * ldh8(k + fe.j * KF_P + 16 * u + 8 * lh);
      S0 = mfma32h(af, ldh8(v + lc * VT_P + 16 * u + 8 * lh), S0);
      S1 = mfma32h(af, ldh8(v + (32 + lc) * VT_P + 16 * u + 8 * lh), S1);
      if (w == 0) {
        // rows 18..31 of K' are zero
        const f16x8 zf = ldh8(k + (lc < 18 ? lc : 17) * KF_P + 16 * u + 8 * lh);
        Z = mfma32h(zf, zf, Z);
      }
    }
  };

  using S0_ = std::integral_constant<int, 0>;
  using S1_ = std::integral_constant<int, 1>;
#pragma unroll
  for (int k = 0; k < PER_T; ++k) {
    pf[0][k] = load_item(0, k);
    pf[1][k] = load_item(1, k);
  }
  stage(0, 0, S0_{});
  __syncthreads();
  int i = 0;
  for (; i + 2 <= nch; i += 2) {
    stage(i + 1, 1, S1_{});
    compute(0);
    __syncthreads();
    stage(i + 2, 0, S0_{});
    compute(1);
    __syncthreads();
  }
  if (i < nch) {
    stage(i + 1, 1, S1_{});
    compute(0);
    __syncthreads();
  }

  // sums in the accumulator layout of the main kernel's state waves
  float4* dst = reinterpret_cast<float4*>(a.seg) + (static_cast<size_t>(bh) * PS + p) * UNIT_F4;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    dst[((0 * NFT + w) * 4 + q4) * 64 + l] = float4{S0[4 * q4], S0[4 * q4 + 1], S0[4 * q4 + 2], S0[4 * q4 + 3]};
    dst[((1 * NFT + w) * 4 + q4) * 64 + l] = float4{S1[4 * q4], S1[4 * q4 + 1], S1[4 * q4 + 2], S1[4 * q4 + 3]};
  }
  if (w == 0) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      dst[(2 * NFT * 4 + q4) * 64 + l] = float4{Z[4 * q4], Z[4 * q4 + 1], Z[4 * q4 + 2], Z[4 * q4 + 3]};
  }
}

// Inclusive prefix over the segments of each head, in place.
__global__ __launch_bounds__(256) void o2_scan(float4* seg, int BH, int PS) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(BH) * UNIT_F4) return;
  const int64_t bh = e / UNIT_F4, pos = e - bh * UNIT_F4;
  float4* base = seg + bh * PS * static_cast<int64_t>(UNIT_F4) + pos;
  float4 acc = base[0];
  constexpr int B8 = 8;
  for (int p0 = 1; p0 < PS; p0 += B8) {
    float4 x[B8];
#pragma unroll
    for (int j = 0; j < B8; ++j) x[j] = p0 + j < PS ? base[static_cast<int64_t>(p0 + j) * UNIT_F4] : float4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < B8; ++j) {
      if (p0 + j < PS) {
        acc.x += x[j].x;
        acc.y += x[j].y;
        acc.z += x[j].z;
        acc.w += x[j].w;
        base[static_cast<int64_t>(p0 + j) * UNIT_F4] = acc;
      }
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
  const int64_t nch = (static_cast<int64_t>(N) + C - 1) / C;
  if (BH <= 0 || nch == 0) {
    pl->P = 1;
    pl->L = N;
    return true;
  }
  // about two workgroups per compute unit, at least 8 chunks per segment
  const int64_t target = 512;
  const int64_t want = (target + BH - 1) / BH;
  const int64_t maxp = nch / 8 > 1 ? nch / 8 : 1;
  const int64_t P = want < 1 ? 1 : (want > maxp ? maxp : want);
  const int64_t cps = (nch + P - 1) / P;
  pl->L = static_cast<int>(cps * C);
  pl->P = static_cast<int>((nch + cps - 1) / cps);
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  pl->seg_off = off;
  if (pl->P > 1) off += al(static_cast<size_t>(BH) * (pl->P - 1) * UNIT_BYTES);
  pl->fin_off = off;
  if (pl->P > 1) off += al(static_cast<size_t>(BH) * UNIT_BYTES);
  pl->part_off = off;
  pl->bytes = off;
  return true;
}

hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  hipError_t e;
  if (a.P > 1) {
    hipLaunchKernelGGL(o2_segsum, dim3(a.BH * (a.P - 1)), dim3(ss::NTHR), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.P > 2) {
      const int64_t n = static_cast<int64_t>(a.BH) * UNIT_F4;
      hipLaunchKernelGGL(o2_scan, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                         reinterpret_cast<float4*>(a.seg), a.BH, a.P - 1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (a.o == nullptr || a.out_bf16)
    hipLaunchKernelGGL((o2_kernel<MAIN, true>), dim3(a.BH * a.P), dim3(NTHR), 0, stream, a);
  else
    hipLaunchKernelGGL((o2_kernel<MAIN, false>), dim3(a.BH * a.P), dim3(NTHR), 0, stream, a);
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
