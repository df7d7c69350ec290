// Order-2 causal prefill for d = 64, dv = 64, bf16 inputs (n_terms = 3),
// on gfx950's 32x32x16 matrix cores.
//
// What is computed ("Expanding Attention: A Taylor-Series Route to
// Linear-Time Transformers with a Fixed Number of Recurrent States"; order-2
// weight 1 + t + t^2/2 as in the posfloor README):
//   o_t = sum_{s<=t} w(q_t.k_s/a) v_s / sum_{s<=t} w(q_t.k_s/a),
// chunked as on that page ("Time": a state part plus diagonal blocks):
//   O_c   = phi~(Q_c) S_<c + P_c V_c,    S += phi(K_c)^T V_c
//   den_c = q'^T Z~_<c q' + P_c 1,       Z += K'^T K'   (K' = [k, 1])
//
// Internal feature basis. The 2145 monomials of degree <= 2 over 64
// coordinates sit in 68 tiles of 32 (2176 slots, 31 zero):
//   tiles 0..63  pairs (a, a+K mod 64), K = tile % 32, a = 32 (tile / 32) + r
//   tile  64     pairs (r, r+32)
//   tiles 65, 66 linear terms k_a, a = 32 (tile - 65) + r
//   tile  67     the constant (r = 0) and zeros
// so every pair a <= b occurs exactly once (a static_assert checks it) and
// both operand fragments come from contiguous LDS rows. The key side carries
// plain products; the query side carries every weight (q/a is staged, so
// products are q_a q_b / a^2, halved on the diagonal class, q_a / a on the
// linear tiles). Canonical (sqrt-multinomial, lexicographic) states differ
// by a permutation and sqrt(2) on the off-diagonal rows.
//
// Denominator: z is the Gram matrix of K' = [k, 1] (65 x 65; order 2,
// linear and constant blocks), held as six 32x32 tiles of a 96x96 matrix
// (block 2 = the ones coordinate and zeros); the inter-chunk part is the
// bilinear form q'^T Z~ q' with Z~ scaled by 1/(2a^2), 1/(2a) and 1 on its
// blocks, off-diagonal tiles counted twice.
//
// Work decomposition: one workgroup of 8 waves per (head, value half of 32
// columns, segment). The 74 tiles (68 state, 6 Gram) are split over the
// waves, 9 or 10 each, as fp32 accumulators. Per 32-token chunk every wave
// reads out its state tiles into a partial output, updates them, and (for
// Gram tiles) updates Z and adds its part of the denominator; wave 0 also
// computes the diagonal block (scores, weights, causal mask, P V). Partial
// outputs meet in double-buffered LDS and all threads normalise and store
// the previous chunk. Feature fragments are built with packed fp16
// products: keys from an fp16 K'^T, queries from an fp16 q/a row that
// carries duplicated, one and zero regions so every fragment is two
// contiguous reads.
//
// Segments (states are additive, closing paragraph of the same page): a
// first launch sums segments 0..P-2, a scan makes inclusive prefixes, the
// main launch starts each segment from its prefix.
#include "internal.hpp"
#include "mma.hpp"

#include <stdint.h>

#include <type_traits>
#include <utility>

namespace tl {
namespace w2 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int D = 64, DV = 64, DH = 32;  // value columns per workgroup
constexpr int C = 32;                     // tokens per chunk
constexpr int NW = 8, NTHR = NW * 64;
constexpr int F = 2145;
constexpr int NS = 68, NZ = 3, NSLOT = NS + NZ;
constexpr int W_Z1 = 0;                   // wave that keeps z1 = sum of keys
constexpr int W_DIAG = NW - 1;            // wave that computes the diagonal block
constexpr float kSqrt2 = 1.41421356237309515f;

// slots [slot_begin(w), slot_begin(w+1)) belong to wave w. The diagonal
// block costs its wave about three slots' time, so that wave holds 6 slots
// and two others hold 10 (measured: with 9 slots everywhere but 8 on it,
// the diagonal wave reached the chunk barrier last every time, 1.75 us
// after the first of 8 us).
__host__ __device__ constexpr int slot_begin(int w) {
  constexpr int t[NW + 1] = {0, 9, 18, 28, 38, 47, 56, 65, NSLOT};
  return w < NW ? t[w] : NSLOT;
}
static_assert(slot_begin(W_DIAG + 1) - slot_begin(W_DIAG) == 6, "the diagonal wave holds six slots");
static_assert(slot_begin(NW) == NSLOT, "all slots assigned");

enum { S_CLASS = 0, S_LIN = 1, S_CONST = 2, S_Z = 3 };
struct Slot {
  int kind;
  int abase;  // first coordinate of the tile's a range
  int koff;   // b = a + koff (classes)
  int zr, zc; // Gram block of the key coordinates (rows, columns)
};
__host__ __device__ constexpr Slot slot_info(int s) {
  if (s < 64) return Slot{S_CLASS, 32 * (s / 32), s % 32, 0, 0};
  if (s == 64) return Slot{S_CLASS, 0, 32, 0, 0};
  if (s < 67) return Slot{S_LIN, 32 * (s - 65), 0, 0, 0};
  if (s == 67) return Slot{S_CONST, 0, 0, 0, 0};
  const int i = s - 68;  // (0,0), (0,1), (1,1)
  return Slot{S_Z, 0, 0, i == 2 ? 1 : 0, i == 0 ? 0 : 1};
}

// a range shared by every state slot of wave w (all of them pair classes),
// or -1
__host__ __device__ constexpr int uniform_abase(int w) {
  int ab = -1;
  for (int s = slot_begin(w); s < slot_begin(w + 1); ++s) {
    const Slot t = slot_info(s);
    if (t.kind == S_Z) continue;
    if (t.kind != S_CLASS) return -1;
    if (ab >= 0 && t.abase != ab) return -1;
    ab = t.abase;
  }
  return ab;
}

// Canonical index and weight of state row r of state slot s.
struct Feat {
  int can;      // canonical feature, -1 for a zero slot
  float wcan;   // canonical = wcan * internal
};
__host__ __device__ constexpr int pair_index(int lo, int hi) { return lo * D - lo * (lo - 1) / 2 + (hi - lo); }
__host__ __device__ constexpr Feat feat(int s, int r) {
  const Slot t = slot_info(s);
  if (t.kind == S_CLASS) {
    const int a = t.abase + r, b = (a + t.koff) % D;
    const int lo = a < b ? a : b, hi = a < b ? b : a;
    return Feat{1 + D + pair_index(lo, hi), a == b ? 1.f : kSqrt2};
  }
  if (t.kind == S_LIN) return Feat{1 + t.abase + r, 1.f};
  if (t.kind == S_CONST) return Feat{r == 0 ? 0 : -1, 1.f};
  return Feat{-1, 0.f};
}
constexpr bool basis_is_bijective() {
  int hits[F] = {};
  for (int s = 0; s < NS; ++s)
    for (int r = 0; r < 32; ++r) {
      const Feat e = feat(s, r);
      if (e.can < -1 || e.can >= F) return false;
      if (e.can >= 0) ++hits[e.can];
    }
  for (int c = 0; c < F; ++c)
    if (hits[c] != 1) return false;
  return true;
}
static_assert(basis_is_bijective(), "internal basis covers the canonical one once");

// LDS layout of one chunk buffer (bytes). Row pitches keep 16-byte alignment
// and put consecutive rows on different banks.
constexpr int QRP = 104;   // raw q (bf16): q[0..63], 1, zeros (Gram block 2)
constexpr int QFP = 164;   // q/a (fp16): q/a[0..63], q/a[0..31], ones x32, zeros x32;
                           // 82-dword rows: 8-byte reads of 32 rows hit 64 banks
constexpr int KRP = 72;    // raw k rows (bf16)
constexpr int KTP = 40;    // K'^T rows (fp16): 0..63 coordinates, 64..95 = 0..31, 96 valid, 97 zero
constexpr int VTP = 40;    // V^T rows (fp16), this workgroup's 32 columns
constexpr int KT_ROWS = 98;
constexpr int ROW_VALID = 96, ROW_ZERO = 97;
constexpr int QF_ONES = 96, QF_ONE_THEN_ZEROS = 127;
constexpr int OFF_QR = 0;
constexpr int OFF_QF = OFF_QR + C * QRP * 2;
constexpr int OFF_KR = OFF_QF + C * QFP * 2;
constexpr int OFF_KT = OFF_KR + C * KRP * 2;
constexpr int OFF_VT = OFF_KT + KT_ROWS * KTP * 2;
constexpr int BUF = OFF_VT + DH * VTP * 2;
// partial outputs [buffer][wave][query][32 + 4 pad] fp32, then partial
// denominators [buffer][wave][query]
constexpr int PP = DH + 4;
constexpr int OFF_PART = 2 * BUF;
constexpr int PART = NW * C * PP * 4;
constexpr int OFF_PDEN = OFF_PART + 2 * PART;
constexpr int OFF_Z1 = OFF_PDEN + 2 * NW * C * 4;  // z1 as bf16, 64 entries
constexpr int LDS = OFF_Z1 + 64 * 2;
static_assert(LDS <= 160 * 1024, "one workgroup per CU");
static_assert(OFF_QF % 16 == 0 && OFF_KR % 16 == 0 && OFF_KT % 16 == 0 && OFF_VT % 16 == 0 && BUF % 16 == 0 &&
                  OFF_PART % 16 == 0 && OFF_PDEN % 16 == 0,
              "16-byte aligned regions");

// Published per-segment sums: [slot][4 x float4][64 lanes] per (head, half),
// then z1 (64 floats) and the token count z0.
constexpr int Z1_F4 = NSLOT * 4 * 64;
constexpr int Z0_F4 = Z1_F4 + 16;          // token count (first float)
constexpr int UNIT_F4 = Z0_F4 + 1;
constexpr size_t UNIT_BYTES = static_cast<size_t>(UNIT_F4) * 16;

__device__ __forceinline__ constexpr int acc_row(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
template <class T>
__device__ __forceinline__ T lds(const void* p) {
  return *reinterpret_cast<const T*>(p);
}
__device__ __forceinline__ f16x8 cat(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x8 catb(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x8 h2b(f16x8 x) {
  bf16x8 r;
#pragma unroll
  for (int u = 0; u < 8; ++u) r[u] = static_cast<__bf16>(static_cast<float>(x[u]));
  return r;
}
__device__ __forceinline__ f16x8 b2h(bf16x8 x, float scale) {
  f16x8 r;
#pragma unroll
  for (int u = 0; u < 8; ++u) r[u] = static_cast<_Float16>(static_cast<float>(x[u]) * scale);
  return r;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}


template <int B, class Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& fn, std::integer_sequence<int, Is...>) {
  (fn(std::integral_constant<int, B + Is>{}), ...);
}
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (E > B) static_for_impl<B>(fn, std::make_integer_sequence<int, E - B>{});
}

enum { SEGSUM = 0, MAIN = 1 };

template <int MODE, bool OBF>
__global__ __launch_bounds__(NTHR, 1) void w2_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lc = l & 31, lh = l >> 5;

  const int PL = MODE == MAIN ? a.P : a.P - 1;
  const int unit = blockIdx.x;
  if (unit >= a.BH * 2 * PL) return;
  const int bhh = unit / PL;  // head * 2 + value half
  const int p = unit - bhh * PL;
  const int bh = bhh >> 1, hv = bhh & 1;
  const bool want_out = MODE == MAIN && a.o != nullptr;
  const bool want_state = MODE == MAIN && a.S != nullptr && p == a.P - 1;
  if (MODE == MAIN && !want_out && !want_state) return;
  const int N = a.N;
  const int t0 = p * a.L;
  const int t1 = min(N, t0 + a.L);
  const int nch = (t1 - t0 + C - 1) / C;
  const float inv_a = a.inv_a;
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);

  auto qr = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<__bf16*>(smem + b * BUF + OFF_QR); };
  auto qf = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem + b * BUF + OFF_QF); };
  auto kr = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<__bf16*>(smem + b * BUF + OFF_KR); };
  auto kt = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem + b * BUF + OFF_KT); };
  auto vt = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem + b * BUF + OFF_VT); };
  auto part = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<float*>(smem + OFF_PART + b * PART); };
  auto pden = [&](int b) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(smem + OFF_PDEN) + b * NW * C;
  };

  // constant regions of both buffers
  for (int i = tid; i < 2 * C; i += NTHR) {
    const int b = i / C, row = i % C;
    _Float16* f = qf(b) + row * QFP;
    for (int c = 96; c < 160; ++c) f[c] = static_cast<_Float16>(c < 128 ? 1.f : 0.f);
    __bf16* r = qr(b) + row * QRP;
    for (int c = 64; c < 96; ++c) r[c] = static_cast<__bf16>(c == 64 ? 1.f : 0.f);
    kt(b)[ROW_ZERO * KTP + row] = static_cast<_Float16>(0.f);
  }

  // staging -----------------------------------------------------------------
  const __bf16* qh = reinterpret_cast<const __bf16*>(a.q) + (static_cast<size_t>(bh) * N + t0) * D;
  const __bf16* kh = reinterpret_cast<const __bf16*>(a.k) + (static_cast<size_t>(bh) * N + t0) * D;
  const __bf16* vh = reinterpret_cast<const __bf16*>(a.v) + (static_cast<size_t>(bh) * N + t0) * DV;
  const auto rq = make_rsrc(qh, seg_rows * D * 2);
  const auto rk = make_rsrc(kh, seg_rows * D * 2);
  const auto rv = make_rsrc(vh, seg_rows * DV * 2);
  auto crow = [&](int c, int row) __attribute__((always_inline)) -> uint32_t {
    const int r = c * C + row;
    return static_cast<uint32_t>(r < static_cast<int>(seg_rows) ? r : static_cast<int>(seg_rows));
  };
  // item of this thread: threads 0..255 a Q item, 256..511 a K item (row
  // it >> 3, coordinates 8 (it & 7) .. +8); threads 0..127 also a V item
  // (row tid >> 2, this half's columns 8 (tid & 3) .. +8)
  const bool is_q = __builtin_amdgcn_readfirstlane(tid) < 256;
  const int it = is_q ? tid : tid - 256;
  const int irow = it >> 3, ic8 = it & 7;
  const bool has_v = tid < 128;
  const int vrow = tid >> 2, vc4 = tid & 3;
  auto load_a = [&](int c) __attribute__((always_inline)) -> uint4 {
    return bload16(is_q ? rq : rk, (crow(c, irow) * D + 8 * ic8) * 2);
  };
  auto load_v = [&](int c) __attribute__((always_inline)) -> uint4 {
    return bload16(rv, (crow(c, vrow) * DV + DH * hv + 8 * vc4) * 2);
  };
  uint4 ra[1], rvv[1];  // one chunk ahead: the chunk's compute covers the load latency
  auto stage = [&](int c, int b, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    static_assert(SL == 0, "one ring slot");
    const bf16x8 x = __builtin_bit_cast(bf16x8, ra[SL]);
    if (MODE == MAIN && is_q) {
      *reinterpret_cast<bf16x8*>(qr(b) + irow * QRP + 8 * ic8) = x;
      const f16x8 h = b2h(x, inv_a);
      const f16x4 h0{h[0], h[1], h[2], h[3]}, h1{h[4], h[5], h[6], h[7]};
      *reinterpret_cast<f16x4*>(qf(b) + irow * QFP + 8 * ic8) = h0;
      *reinterpret_cast<f16x4*>(qf(b) + irow * QFP + 8 * ic8 + 4) = h1;
      if (ic8 < 4) {
        *reinterpret_cast<f16x4*>(qf(b) + irow * QFP + D + 8 * ic8) = h0;
        *reinterpret_cast<f16x4*>(qf(b) + irow * QFP + D + 8 * ic8 + 4) = h1;
      }
    } else if (!is_q) {
      if (MODE == MAIN) *reinterpret_cast<bf16x8*>(kr(b) + irow * KRP + 8 * ic8) = x;
      const f16x8 h = b2h(x, 1.f);
      _Float16* t = kt(b);
#pragma unroll
      for (int u = 0; u < 8; ++u) t[(8 * ic8 + u) * KTP + irow] = h[u];
      if (ic8 < 4) {
#pragma unroll
        for (int u = 0; u < 8; ++u) t[(D + 8 * ic8 + u) * KTP + irow] = h[u];
      }
      if (ic8 == 0) t[ROW_VALID * KTP + irow] = static_cast<_Float16>(c * C + irow < static_cast<int>(seg_rows) ? 1.f : 0.f);
    }
    if (has_v) {
      const f16x8 h = b2h(__builtin_bit_cast(bf16x8, rvv[SL]), 1.f);
      _Float16* t = vt(b);
#pragma unroll
      for (int u = 0; u < 8; ++u) t[(8 * vc4 + u) * VTP + vrow] = h[u];
    }
    ra[SL] = load_a(c + 1);
    if (has_v) rvv[SL] = load_v(c + 1);
  };

  // per-chunk compute ---------------------------------------------------------
  const float c2 = 0.5f * inv_a * inv_a;
  const f16x8 halfh = f16x8{0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f};
  // K'^T row of Gram block `blk` for lane lc
  const float c2z = 0.5f * inv_a * inv_a;  // Z~ = Z / (2 a^2) on the key-coordinate blocks
  // One chunk for wave W (compile-time slot list).
  auto compute_w = [&](auto wtag, auto& acc, float& z1r, int i, int b, bool out) __attribute__((always_inline)) {
    constexpr int W = decltype(wtag)::value;
    constexpr int SB = slot_begin(W), NSW = slot_begin(W + 1) - SB;
    const _Float16* K = kt(b);
    const _Float16* V = vt(b);
    const _Float16* QF = qf(b) + lc * QFP;
    const __bf16* QR = qr(b) + lc * QRP;
    f32x16 O = f32x16{};
    float dpart = 0.f;
    // operands shared by the chunk: V^T fragments; and, when every state
    // slot of the wave covers the same a range, the a-side rows of both
    // feature fragments
    constexpr int UAB = uniform_abase(W);
    f16x8 bv[2], aq[2], kx[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bv[ks] = lds<f16x8>(V + lc * VTP + 16 * ks + 8 * lh);
      if constexpr (UAB >= 0) {
        const int o = UAB + 16 * ks + 4 * lh;
        aq[ks] = cat(lds<f16x4>(QF + o), lds<f16x4>(QF + o + 8));
        kx[ks] = lds<f16x8>(K + (UAB + lc) * KTP + 16 * ks + 8 * lh);
      }
    }
    static_for<0, NSW>([&](auto sli) {
      constexpr int sl = decltype(sli)::value;
      constexpr Slot t = slot_info(SB + sl);
      if constexpr (t.kind != S_Z) {
        if (out) {
          // read-out: O^T[dv][query] += S^T phi~(Q)^T, features in the
          // accumulator order (rows 16ks + 4lh + 0..3 and 16ks + 8 + 4lh + 0..3)
          constexpr int acol = t.kind == S_CONST ? QF_ONE_THEN_ZEROS : t.abase;
          constexpr int bcol = t.kind == S_CLASS ? t.abase + t.koff : QF_ONES;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int o = 16 * ks + 4 * lh;
            f16x8 qa;
            if constexpr (UAB >= 0)
              qa = aq[ks];
            else
              qa = cat(lds<f16x4>(QF + acol + o), lds<f16x4>(QF + acol + o + 8));
            f16x8 ph = qa * cat(lds<f16x4>(QF + bcol + o), lds<f16x4>(QF + bcol + o + 8));
            if constexpr (t.kind == S_CLASS && t.koff == 0) ph = ph * halfh;
            bf16x8 sa;
#pragma unroll
            for (int s = 0; s < 8; ++s) sa[s] = static_cast<__bf16>(acc[sl][8 * ks + s]);
            O = mfma32(sa, h2b(ph), O);
          }
        }
        // update: S += phi(K)^T V
        const int arow = t.kind == S_CONST ? (lc == 0 ? ROW_VALID : ROW_ZERO) : t.abase + lc;
        const int brow = t.kind == S_CLASS ? t.abase + lc + t.koff : ROW_VALID;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f16x8 x;
          if constexpr (UAB >= 0)
            x = kx[ks];
          else
            x = lds<f16x8>(K + arow * KTP + 16 * ks + 8 * lh);
          acc[sl] = mfma32h(x * lds<f16x8>(K + brow * KTP + 16 * ks + 8 * lh), bv[ks], acc[sl]);
        }
      } else {
        if (out) {
          // denominator part: sum_{i in zr, j in zc} q_i Z~_ij q_j (x2 off
          // the diagonal), as U = Z~^T q_zr then q_zc . U
          f32x16 U = f32x16{};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 za;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int j = 8 * ks + s;
              za[s] = static_cast<__bf16>(acc[sl][j] * c2z);
            }
            const int o = 32 * t.zr + 16 * ks + 4 * lh;
            U = mfma32(za, catb(lds<bf16x4>(QR + o), lds<bf16x4>(QR + o + 8)), U);
          }
          float bil = 0.f;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const bf16x4 qv = lds<bf16x4>(QR + 32 * t.zc + 8 * g + 4 * lh);
#pragma unroll
            for (int e = 0; e < 4; ++e) bil += U[4 * g + e] * static_cast<float>(qv[e]);
          }
          dpart += (t.zr == t.zc ? 1.f : 2.f) * bil;
        }
        const int ar = 32 * t.zr + lc, br = 32 * t.zc + lc;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          acc[sl] = mfma32h(lds<f16x8>(K + ar * KTP + 16 * ks + 8 * lh), lds<f16x8>(K + br * KTP + 16 * ks + 8 * lh),
                            acc[sl]);
      }
    });
    if constexpr (W == W_Z1) {
      // linear part of the denominator, (q . z1) / a with z1 of the earlier
      // chunks (every row of the product equals q . z1), then z1 += keys
      if (out) {
        __bf16* zb = reinterpret_cast<__bf16*>(smem + OFF_Z1);
        zb[l] = static_cast<__bf16>(z1r);
        f32x16 U = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          U = mfma32(lds<bf16x8>(zb + 16 * ks + 8 * lh), lds<bf16x8>(QR + 16 * ks + 8 * lh), U);
        if (lh == 0) dpart += inv_a * U[0];
      }
      const _Float16* kr0 = K + l * KTP;
      float zs = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f16x8 x = lds<f16x8>(kr0 + 8 * u);
#pragma unroll
        for (int e = 0; e < 8; ++e) zs += static_cast<float>(x[e]);
      }
      z1r += zs;
    }
    if (!out) return;
    if constexpr (W == W_DIAG) {
      // diagonal block: scores D[key][query] = K Q^T (raw), weights, causal
      // mask, then O^T += V^T P^T with keys in the accumulator order
      const __bf16* KR = kr(b) + lc * KRP;
      f32x16 sc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sc = mfma32(lds<bf16x8>(KR + 16 * ks + 8 * lh), lds<bf16x8>(QR + 16 * ks + 8 * lh), sc);
      f16x8 P0, P1;
      float den = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float wv = __builtin_fmaf(__builtin_fmaf(c2, sc[j], inv_a), sc[j], 1.f);
        if (acc_row(j, lh) > lc) wv = 0.f;
        den += wv;
        if (j < 8)
          P0[j] = static_cast<_Float16>(wv);
        else
          P1[j - 8] = static_cast<_Float16>(wv);
      }
      const _Float16* vr = V + lc * VTP;
      O = mfma32h(cat(lds<f16x4>(vr + 4 * lh), lds<f16x4>(vr + 8 + 4 * lh)), P0, O);
      O = mfma32h(cat(lds<f16x4>(vr + 16 + 4 * lh), lds<f16x4>(vr + 24 + 4 * lh)), P1, O);
      dpart += den;
    }
    dpart += __shfl_xor(dpart, 32);
    // partial outputs: [wave][query lc][dv rows 8g + 4lh + 0..3]
    float* pt = part(i & 1) + (W * C + lc) * PP;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4*>(pt + 8 * g + 4 * lh) = f32x4{O[4 * g], O[4 * g + 1], O[4 * g + 2], O[4 * g + 3]};
    if (lh == 0) pden(i & 1)[W * C + lc] = dpart;
  };
  // z0 (the constant term of the denominator) before this segment: the
  // tokens of the earlier segments plus z0 of the initial state
  const float4* segp = reinterpret_cast<const float4*>(a.seg);
  // units [head * 2 + half][P]: after the scan, unit p is the state before
  // segment p (unit 0 holds S0/z0, unit q + 1 the sum of segment q)
  auto unit_at = [&](int q) __attribute__((always_inline)) {
    return segp + (static_cast<size_t>(bhh) * a.P + q) * UNIT_F4;
  };
  const float z0base = MODE == MAIN ? unit_at(p)[Z0_F4].x : 0.f;

  // sum the partials of chunk i, normalise, store rows
  auto finalize = [&](int i) __attribute__((always_inline)) {
    const int q = tid >> 4, pc = tid & 15;
    const float* pt = part(i & 1) + q * PP + 2 * pc;
    float o0 = 0.f, o1 = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float2 x = *reinterpret_cast<const float2*>(pt + ww * C * PP);
      o0 += x.x;
      o1 += x.y;
      den += pden(i & 1)[ww * C + q];
    }
    den += z0base + static_cast<float>(i * C);  // constant term: tokens before this chunk
    const float rd = __builtin_amdgcn_rcpf(den);
    if (i * C + q < static_cast<int>(seg_rows)) {
      const size_t off = (static_cast<size_t>(bh) * N + t0 + i * C + q) * DV + DH * hv + 2 * pc;
      if constexpr (OBF) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<bf16x2*>(reinterpret_cast<__bf16*>(a.o) + off) =
            bf16x2{static_cast<__bf16>(o0 * rd), static_cast<__bf16>(o1 * rd)};
      } else {
        *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.o) + off) = float2{o0 * rd, o1 * rd};
      }
    }
  };

  // everything that depends on the wave's slot list, per wave ---------------
  using S0_ = std::integral_constant<int, 0>;
  using S1_ = std::integral_constant<int, 1>;
  auto wave_body = [&](auto wtag) __attribute__((always_inline)) {
    constexpr int W = decltype(wtag)::value;
    constexpr int SB = slot_begin(W), NSW = slot_begin(W + 1) - SB;
    f32x16 acc[NSW];
#pragma unroll
    for (int i = 0; i < NSW; ++i) acc[i] = f32x16{};
    float z1r = 0.f;  // wave W_Z1: z1 of coordinate l

    // initial state: unit p
    if (MODE == MAIN) {
      const float4* src = unit_at(p) + l;
#pragma unroll
      for (int i = 0; i < NSW; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = src[((SB + i) * 4 + q4) * 64];
          acc[i][4 * q4 + 0] = x.x;
          acc[i][4 * q4 + 1] = x.y;
          acc[i][4 * q4 + 2] = x.z;
          acc[i][4 * q4 + 3] = x.w;
        }
      if (W == W_Z1) z1r = reinterpret_cast<const float*>(unit_at(p) + Z1_F4)[l];
    }

    // chunk loop: iteration i stages chunk i+1, computes chunk i and
    // finishes chunk i-1
    ra[0] = load_a(0);
    if (has_v) rvv[0] = load_v(0);
    stage(0, 0, S0_{});
    __syncthreads();
    auto iter = [&](int i, auto slot) __attribute__((always_inline)) {
      stage(i + 1, (i + 1) & 1, slot);
      compute_w(wtag, acc, z1r, i, i & 1, want_out);
      if (want_out && i > 0) finalize(i - 1);
      __syncthreads();
    };
    int i = 0;
    for (; i + 2 <= nch; i += 2) {
      iter(i, S0_{});
      iter(i + 1, S0_{});
    }
    if (i < nch) iter(i, S0_{});
    if (want_out && nch > 0) finalize(nch - 1);

    // results
    float4* dstu = nullptr;
    if (MODE == SEGSUM) {
      dstu = reinterpret_cast<float4*>(a.seg) + (static_cast<size_t>(bhh) * a.P + p + 1) * UNIT_F4;
    } else if (want_state && a.defer_state) {
      dstu = reinterpret_cast<float4*>(a.fin) + static_cast<size_t>(bhh) * UNIT_F4;
    }
    const float count = (MODE == MAIN ? z0base : 0.f) + static_cast<float>(t1 - t0);
    if (dstu != nullptr) {
#pragma unroll
      for (int sl = 0; sl < NSW; ++sl)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dstu[((SB + sl) * 4 + q4) * 64 + l] =
              float4{acc[sl][4 * q4], acc[sl][4 * q4 + 1], acc[sl][4 * q4 + 2], acc[sl][4 * q4 + 3]};
      if (W == W_Z1) {
        reinterpret_cast<float*>(dstu + Z1_F4)[l] = z1r;
        if (l == 0) dstu[Z0_F4] = float4{count, 0.f, 0.f, 0.f};
      }
    } else if (want_state) {
      if (W == W_Z1 && hv == 0) {
        float* z = a.z + static_cast<size_t>(bh) * F;
        z[1 + l] = z1r;
        if (l == 0) z[0] = count;
      }
      const int col = DH * hv + lc;
      static_for<0, NSW>([&](auto sli) {
        constexpr int sl = decltype(sli)::value;
        constexpr int s = SB + sl;
        constexpr Slot t = slot_info(s);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = acc_row(j, lh);
          if constexpr (t.kind != S_Z) {
            const Feat e = feat(s, r);
            if (e.can >= 0) a.S[(static_cast<size_t>(bh) * F + e.can) * DV + col] = e.wcan * acc[sl][j];
          } else {
            if (hv != 0) continue;
            const int ti = 32 * t.zr + r, tj = 32 * t.zc + lc;
            if (ti <= tj) a.z[static_cast<size_t>(bh) * F + 1 + D + pair_index(ti, tj)] = (ti == tj ? 1.f : kSqrt2) * acc[sl][j];
          }
        }
      });
    }
  };
  switch (w) {
    case 0: wave_body(std::integral_constant<int, 0>{}); break;
    case 1: wave_body(std::integral_constant<int, 1>{}); break;
    case 2: wave_body(std::integral_constant<int, 2>{}); break;
    case 3: wave_body(std::integral_constant<int, 3>{}); break;
    case 4: wave_body(std::integral_constant<int, 4>{}); break;
    case 5: wave_body(std::integral_constant<int, 5>{}); break;
    case 6: wave_body(std::integral_constant<int, 6>{}); break;
    default: wave_body(std::integral_constant<int, 7>{}); break;
  }
}

// Unit 0 of each (head, half): S0/z0 in the internal layout (zeros without
// an initial state). One workgroup of 64 threads per (head, half, slot), plus
// one per (head, half) for z1 and z0.
__global__ __launch_bounds__(64) void w2_s0_unit(const float* S0, const float* z0, float4* seg, int P) {
  const int u = blockIdx.x / (NSLOT + 1), s = blockIdx.x % (NSLOT + 1);
  const int bh = u >> 1, hv = u & 1;
  const int l = threadIdx.x, lc = l & 31, lh = l >> 5;
  float4* dst = seg + static_cast<size_t>(u) * P * UNIT_F4;
  if (s == NSLOT) {
    reinterpret_cast<float*>(dst + Z1_F4)[l] = S0 != nullptr ? z0[static_cast<size_t>(bh) * F + 1 + l] : 0.f;
    if (l == 0) dst[Z0_F4] = float4{S0 != nullptr ? z0[static_cast<size_t>(bh) * F] : 0.f, 0.f, 0.f, 0.f};
    return;
  }
  const Slot t = slot_info(s);
  for (int q4 = 0; q4 < 4; ++q4) {
    float v[4];
    for (int rr = 0; rr < 4; ++rr) {
      const int r = acc_row(4 * q4 + rr, lh);
      float x = 0.f;
      if (S0 != nullptr) {
        if (t.kind != S_Z) {
          const Feat e = feat(s, r);
          if (e.can >= 0) x = S0[(static_cast<size_t>(bh) * F + e.can) * DV + DH * hv + lc] / e.wcan;
        } else {
          const int ti = 32 * t.zr + r, tj = 32 * t.zc + lc;
          const int lo = ti < tj ? ti : tj, hi = ti < tj ? tj : ti;
          x = z0[static_cast<size_t>(bh) * F + 1 + D + pair_index(lo, hi)] / (lo == hi ? 1.f : kSqrt2);
        }
      }
      v[rr] = x;
    }
    dst[(s * 4 + q4) * 64 + l] = float4{v[0], v[1], v[2], v[3]};
  }
}

// Inclusive prefix over the segments of each (head, half), in place.
__global__ __launch_bounds__(256) void w2_scan(float4* seg, int BHH, int PS) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(BHH) * UNIT_F4) return;
  const int64_t u = e / UNIT_F4, pos = e - u * UNIT_F4;
  float4* base = seg + u * PS * static_cast<int64_t>(UNIT_F4) + pos;
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
// One workgroup of 64 threads per (head, half, slot), plus one per (head,
// half) for z1 and z0.
__global__ __launch_bounds__(64) void w2_state_store(const float4* fin, float* S, float* z) {
  const int u = blockIdx.x / (NSLOT + 1), s = blockIdx.x % (NSLOT + 1);
  const int bh = u >> 1, hv = u & 1;
  const int l = threadIdx.x, lc = l & 31, lh = l >> 5;
  const float4* src = fin + static_cast<size_t>(u) * UNIT_F4;
  if (s == NSLOT) {
    if (hv == 0) {
      z[static_cast<size_t>(bh) * F + 1 + l] = reinterpret_cast<const float*>(src + Z1_F4)[l];
      if (l == 0) z[static_cast<size_t>(bh) * F] = src[Z0_F4].x;
    }
    return;
  }
  const Slot t = slot_info(s);
  for (int q4 = 0; q4 < 4; ++q4) {
    const float4 x = src[(s * 4 + q4) * 64 + l];
    const float v[4] = {x.x, x.y, x.z, x.w};
    for (int rr = 0; rr < 4; ++rr) {
      const int j = 4 * q4 + rr, r = acc_row(j, lh);
      if (t.kind != S_Z) {
        const Feat e = feat(s, r);
        if (e.can >= 0) S[(static_cast<size_t>(bh) * F + e.can) * DV + DH * hv + lc] = e.wcan * v[rr];
      } else if (hv == 0) {
        const int ti = 32 * t.zr + r, tj = 32 * t.zc + lc;
        if (ti <= tj) z[static_cast<size_t>(bh) * F + 1 + D + pair_index(ti, tj)] = (ti == tj ? 1.f : kSqrt2) * v[rr];
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
  // about one workgroup per compute unit (two value halves per head), at
  // least 8 chunks per segment
  const int64_t target = 256;
  const int64_t want = (target + 2 * BH - 1) / (2 * BH);
  const int64_t maxp = nch / 8 > 1 ? nch / 8 : 1;
  int64_t P = want < 1 ? 1 : (want > maxp ? maxp : want);
  const int64_t minp = min_segments(nch, C, D * 2);  // 32-bit buffer ranges per segment
  if (P < minp) P = minp;
  const int64_t cps = (nch + P - 1) / P;
  pl->L = static_cast<int>(cps * C);
  pl->P = static_cast<int>((nch + cps - 1) / cps);
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  pl->seg_off = off;
  off += al(static_cast<size_t>(BH) * 2 * pl->P * UNIT_BYTES);
  pl->fin_off = off;
  if (pl->P > 1) off += al(static_cast<size_t>(BH) * 2 * UNIT_BYTES);
  pl->part_off = off;
  pl->bytes = off;
  return true;
}

hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  hipError_t e;
  float4* seg = reinterpret_cast<float4*>(a.seg);
  hipLaunchKernelGGL(w2_s0_unit, dim3(a.BH * 2 * (NSLOT + 1)), dim3(64), 0, stream, a.S0, a.z0, seg, a.P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.P > 1) {
    hipLaunchKernelGGL((w2_kernel<SEGSUM, true>), dim3(a.BH * 2 * (a.P - 1)), dim3(NTHR), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = static_cast<int64_t>(a.BH) * 2 * UNIT_F4;
    hipLaunchKernelGGL(w2_scan, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, seg, a.BH * 2,
                       a.P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.o == nullptr || a.out_bf16)
    hipLaunchKernelGGL((w2_kernel<MAIN, true>), dim3(a.BH * 2 * a.P), dim3(NTHR), 0, stream, a);
  else
    hipLaunchKernelGGL((w2_kernel<MAIN, false>), dim3(a.BH * 2 * a.P), dim3(NTHR), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.defer_state && a.S != nullptr) {
    hipLaunchKernelGGL(w2_state_store, dim3(a.BH * 2 * (NSLOT + 1)), dim3(64), 0, stream,
                       reinterpret_cast<const float4*>(a.fin), a.S, a.z);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace w2
}  // namespace tl
