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
// columns, segment). The 71 slots (68 state tiles, 3 Gram tiles) are spread
// over the waves as fp32 accumulators: seven waves hold 9 pair-class tiles
// each, grouped so that one wave's tiles share their first coordinate range
// (at most two such groups per wave); wave 3 holds the linear, constant and
// Gram tiles and the diagonal block (scores, weights, causal mask, P V),
// wave 1 the key sum z1. Per 32-token chunk every wave reads its tiles out
// into a partial output, then updates them. Partial outputs meet in
// double-buffered LDS, and waves 0..3 normalise and store the previous chunk.
//
// Feature fragments. Key side (update, fp16 MFMA): packed fp16 products of
// two rows of an fp16 K'^T tile. Query side (read-out, bf16 MFMA against the
// state rounded to bf16): each lane holds, per 16-deep k-step, the q/a values
// its tiles need in fp32 registers (one contiguous block per group, loaded
// once per chunk from an fp32 q/a row that repeats its 64 coordinates), and
// forms every feature with one fp32 multiply; pairs are rounded to bf16 with
// one conversion. No LDS read per tile on the query side.
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
constexpr int W_AUX = 3;                  // linear, constant and Gram slots, diagonal block
constexpr int W_Z1 = 1;                   // key sum z1 and its read-out (1% faster than on W_AUX)
constexpr float kSqrt2 = 1.41421356237309515f;

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

// Slots of each wave. Pair classes of one first-coordinate range (abase)
// and consecutive offsets K stay together, so a wave's query features come
// from at most two register blocks. The auxiliary wave (linear, constant
// and Gram tiles, diagonal block) also takes two pair classes: per chunk
// it then issues about as many VALU instructions as a wave of nine classes,
// but its work has more dependent steps. Waves w and w + 4 share a SIMD and
// the older one (w < 4) gets issue priority. With the auxiliary slots on
// wave 7, per-chunk timestamps showed that wave arriving last at the barrier
// in every chunk; on wave 3 the main launch runs about 2.5% faster.
constexpr int MAXSL = 10;
struct SlotList {
  int n;
  int s[MAXSL];
};
__host__ __device__ constexpr SlotList wave_slots(int w) {
  switch (w) {
    case 0: return SlotList{9, {0, 1, 2, 3, 4, 5, 6, 7, 8}};
    case 1: return SlotList{9, {9, 10, 11, 12, 13, 14, 15, 16, 17}};
    case 2: return SlotList{9, {18, 19, 20, 21, 22, 23, 24, 25, 26}};
    case 3: return SlotList{8, {62, 63, 65, 66, 67, 68, 69, 70}};
    case 4: return SlotList{9, {35, 36, 37, 38, 39, 40, 41, 42, 43}};
    case 5: return SlotList{9, {44, 45, 46, 47, 48, 49, 50, 51, 52}};
    case 6: return SlotList{9, {53, 54, 55, 56, 57, 58, 59, 60, 61}};
    default: return SlotList{9, {27, 28, 29, 30, 31, 64, 32, 33, 34}};
  }
}
constexpr bool slots_partitioned() {
  int hits[NSLOT] = {};
  for (int w = 0; w < NW; ++w) {
    const SlotList L = wave_slots(w);
    for (int i = 0; i < L.n; ++i) {
      if (L.s[i] < 0 || L.s[i] >= NSLOT) return false;
      ++hits[L.s[i]];
    }
  }
  for (int s = 0; s < NSLOT; ++s)
    if (hits[s] != 1) return false;
  for (int w = 0; w < NW; ++w) {
    if (w == W_AUX) continue;
    const SlotList L = wave_slots(w);
    for (int i = 0; i < L.n; ++i)
      if (slot_info(L.s[i]).kind != S_CLASS) return false;
  }
  // the auxiliary wave's pair classes share the range of its second linear
  // tile (abase 32), so its two key rows serve both
  for (int i = 0; i < wave_slots(W_AUX).n; ++i) {
    const Slot t = slot_info(wave_slots(W_AUX).s[i]);
    if (t.kind == S_CLASS && t.abase != 32) return false;
  }
  return true;
}
static_assert(slots_partitioned(), "every slot on exactly one wave; the waves other than W_AUX hold pair classes only");

// Query-side register blocks of a wave: one per first-coordinate range of
// its pair classes. A block holds, for one k-step, q/a at coordinates
// abase + 16 ks + 4 lh + kb + [0, nb) (kb = smallest offset K rounded down to
// a multiple of 4; nb covers the largest K plus the 12-wide span of a
// lane's eight features).
struct Group {
  int abase, kb, nb;
};
__host__ __device__ constexpr int n_groups(int w) {
  const SlotList L = wave_slots(w);
  int ab0 = -1, n = 0;
  for (int i = 0; i < L.n; ++i) {
    const Slot t = slot_info(L.s[i]);
    if (t.kind != S_CLASS) continue;
    if (n == 0) {
      ab0 = t.abase;
      n = 1;
    } else if (t.abase != ab0) {
      n = 2;
    }
  }
  return n;
}
__host__ __device__ constexpr int group_abase(int w, int g) {
  const SlotList L = wave_slots(w);
  int seen = -1, k = -1;
  for (int i = 0; i < L.n; ++i) {
    const Slot t = slot_info(L.s[i]);
    if (t.kind != S_CLASS || t.abase == seen) continue;
    seen = t.abase;
    if (++k == g) return t.abase;
  }
  return -1;
}
__host__ __device__ constexpr Group group_of(int w, int g) {
  const SlotList L = wave_slots(w);
  const int ab = group_abase(w, g);
  int kmin = 1 << 20, kmax = -1;
  for (int i = 0; i < L.n; ++i) {
    const Slot t = slot_info(L.s[i]);
    if (t.kind != S_CLASS || t.abase != ab) continue;
    kmin = t.koff < kmin ? t.koff : kmin;
    kmax = t.koff > kmax ? t.koff : kmax;
  }
  const int kb = kmin & ~3;
  return Group{ab, kb, ((kmax + 12 - kb) + 3) & ~3};
}
// Block of the pair classes of wave w with first-coordinate range ab (nb = 0
// when the wave has none).
__host__ __device__ constexpr Group group_for(int w, int ab) {
  return group_abase(w, 0) == ab ? group_of(w, 0) : (group_abase(w, 1) == ab ? group_of(w, 1) : Group{ab, 0, 0});
}
// The two key-row / first-coordinate ranges a wave works with: its class
// groups, or for the auxiliary wave the ranges of its linear and Gram tiles.
__host__ __device__ constexpr int row_base(int w, int g) {
  if (w == W_AUX) return 32 * g;
  return g < n_groups(w) ? group_abase(w, g) : -1;
}
constexpr bool groups_fit() {
  for (int w = 0; w < NW; ++w) {
    if (n_groups(w) < 1 || n_groups(w) > 2) return false;
    for (int g = 0; g < 2; ++g) {
      const Group G = group_for(w, row_base(w, g));
      // the block stays inside the repeated 128-float q/a row
      if (G.abase + 16 + 4 + G.kb + G.nb > 128 || G.nb > 24) return false;
    }
    // every class tile of the wave belongs to one of its two ranges
    const SlotList L = wave_slots(w);
    for (int i = 0; i < L.n; ++i) {
      const Slot t = slot_info(L.s[i]);
      if (t.kind == S_CLASS && t.abase != row_base(w, 0) && t.abase != row_base(w, 1)) return false;
    }
  }
  return true;
}
static_assert(groups_fit(), "query register blocks fit the repeated q/a row");

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
constexpr int QAP = 132;   // q/a (fp32): q/a[0..63], q/a[0..63] again; 4 pad
constexpr int KRP = 72;    // raw k rows (bf16)
constexpr int KTP = 40;    // K'^T rows (fp16): coordinates 0..63, then 0..31 again
constexpr int VTP = 40;    // V^T rows (fp16), this workgroup's 32 columns
constexpr int KT_ROWS = 96;
constexpr int OFF_QR = 0;
constexpr int OFF_QA = OFF_QR + C * QRP * 2;
constexpr int OFF_KR = OFF_QA + C * QAP * 4;
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
static_assert(OFF_QA % 16 == 0 && OFF_KR % 16 == 0 && OFF_KT % 16 == 0 && OFF_VT % 16 == 0 && BUF % 16 == 0 &&
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
__device__ __forceinline__ f16x8 b2h(bf16x8 x) {
  return __builtin_convertvector(__builtin_convertvector(x, f32x8), f16x8);
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

// position, within a lane's eight features of a k-step, of element s: the
// accumulator rows 16 ks + 4 lh + {0..3} and 16 ks + 8 + 4 lh + {0..3}
__device__ __forceinline__ constexpr int fpos(int s) { return s < 4 ? s : s + 4; }

// Main launch: every segment from its inclusive prefix; outputs and, for the
// last segment, the final state.
template <bool OBF>
__global__ __launch_bounds__(NTHR, 1) void w2_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lc = l & 31, lh = l >> 5;

  const int PL = a.P;
  const int unit = blockIdx.x;
  if (unit >= a.BH * 2 * PL) return;
  const int bhh = unit / PL;  // head * 2 + value half
  const int p = unit - bhh * PL;
  const int bh = bhh >> 1, hv = bhh & 1;
  const bool want_out = a.o != nullptr;
  const bool want_state = a.S != nullptr && p == a.P - 1;
  if (!want_out && !want_state) return;
  const int N = a.N;
  const int t0 = p * a.L;
  const int t1 = min(N, t0 + a.L);
  const int nch = (t1 - t0 + C - 1) / C;
  const float inv_a = a.inv_a;
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);

  auto qr = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<__bf16*>(smem + b * BUF + OFF_QR); };
  auto qa = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<float*>(smem + b * BUF + OFF_QA); };
  auto kr = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<__bf16*>(smem + b * BUF + OFF_KR); };
  auto kt = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem + b * BUF + OFF_KT); };
  auto vt = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<_Float16*>(smem + b * BUF + OFF_VT); };
  auto part = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<float*>(smem + OFF_PART + b * PART); };
  auto pden = [&](int b) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(smem + OFF_PDEN) + b * NW * C;
  };

  // constant region of both buffers: Q' columns 64..95 = (1, 0, ...)
  for (int i = tid; i < 2 * C; i += NTHR) {
    __bf16* r = qr(i / C) + (i % C) * QRP;
    for (int c = 64; c < 96; ++c) r[c] = static_cast<__bf16>(c == 64 ? 1.f : 0.f);
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
  // item of this thread: threads 0..255 a Q item (row it >> 3, coordinates
  // 8 (it & 7) .. +8), 256..511 a K item; threads 0..127 also a V item (this
  // half's columns 8 vc4 .. +8). K and V are written transposed, 2 bytes per
  // element: their items put the 32 rows of a chunk on the lanes of each half
  // wave (row it & 31, coordinates 8 (2 (it >> 6) + bit 5 of it), columns 8
  // (tid >> 5)), so a wave's stores spread over 32 banks (with eight rows per
  // wave four lanes shared a bank; the call is 1.4% faster this way). Rows
  // past the segment's end load as zero (buffer range), so they add nothing.
  const bool is_q = __builtin_amdgcn_readfirstlane(tid) < 256;
  const int it = is_q ? tid : tid - 256;
  const int irow = is_q ? it >> 3 : (it & 31), ic8 = is_q ? it & 7 : 2 * (it >> 6) + ((it >> 5) & 1);
  const bool has_v = tid < 128;
  const int vrow = tid & 31, vc4 = tid >> 5;
  auto load_a = [&](int c) __attribute__((always_inline)) -> uint4 {
    return bload16(is_q ? rq : rk, (crow(c, irow) * D + 8 * ic8) * 2);
  };
  auto load_v = [&](int c) __attribute__((always_inline)) -> uint4 {
    return bload16(rv, (crow(c, vrow) * DV + DH * hv + 8 * vc4) * 2);
  };
  uint4 ra, rvv;  // one chunk ahead: the chunk's compute covers the load latency
  auto stage = [&](int c, int b) __attribute__((always_inline)) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, ra);
    if (is_q) {
      *reinterpret_cast<bf16x8*>(qr(b) + irow * QRP + 8 * ic8) = x;
      f32x4 lo, hi;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lo[u] = static_cast<float>(x[u]) * inv_a;
        hi[u] = static_cast<float>(x[u + 4]) * inv_a;
      }
      float* row = qa(b) + irow * QAP + 8 * ic8;
      *reinterpret_cast<f32x4*>(row) = lo;
      *reinterpret_cast<f32x4*>(row + 4) = hi;
      *reinterpret_cast<f32x4*>(row + D) = lo;
      *reinterpret_cast<f32x4*>(row + D + 4) = hi;
    } else if (!is_q) {
      *reinterpret_cast<bf16x8*>(kr(b) + irow * KRP + 8 * ic8) = x;
      const f16x8 h = b2h(x);
      _Float16* t = kt(b);
#pragma unroll
      for (int u = 0; u < 8; ++u) t[(8 * ic8 + u) * KTP + irow] = h[u];
      if (ic8 < 4) {
#pragma unroll
        for (int u = 0; u < 8; ++u) t[(D + 8 * ic8 + u) * KTP + irow] = h[u];
      }
    }
    if (has_v) {
      const f16x8 h = b2h(__builtin_bit_cast(bf16x8, rvv));
      _Float16* t = vt(b);
#pragma unroll
      for (int u = 0; u < 8; ++u) t[(8 * vc4 + u) * VTP + vrow] = h[u];
    }
    ra = load_a(c + 1);
    if (has_v) rvv = load_v(c + 1);
  };

  // per-chunk compute ---------------------------------------------------------
  const float c2 = 0.5f * inv_a * inv_a;
  const float c2z = 0.5f * inv_a * inv_a;  // Z~ = Z / (2 a^2) on the key-coordinate blocks
  // One chunk for wave W (compile-time slot list): read out every slot into
  // a partial output (before its update), then update every slot.
  auto compute_w = [&](auto wtag, auto& acc, float& z1r, int i, int b, bool out) __attribute__((always_inline)) {
    constexpr int W = decltype(wtag)::value;
    constexpr SlotList SL = wave_slots(W);
    constexpr int NSW = SL.n;
    const _Float16* K = kt(b);
    const _Float16* V = vt(b);
    const float* QA = qa(b) + lc * QAP;
    const __bf16* QR = qr(b) + lc * QRP;
    f32x16 O = f32x16{};
    float dpart = 0.f;
    // the wave's two first-coordinate ranges and their query blocks
    constexpr int NG = W == W_AUX ? 2 : n_groups(W);
    constexpr int AB0 = row_base(W, 0);
    constexpr int AB1 = NG > 1 ? row_base(W, 1) : AB0;
    constexpr Group G0 = group_for(W, AB0);
    constexpr Group G1 = group_for(W, AB1);
    constexpr int NB0 = G0.nb > 0 ? G0.nb : 4, NB1 = G1.nb > 0 ? G1.nb : 4;

    if (out) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // q/a of the lane's query at its eight features' first coordinates,
        // per range, and each range's block of second coordinates
        float av[NG][8];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const float* base = QA + (g == 0 ? AB0 : AB1) + 16 * ks + 4 * lh;
          const f32x4 x0 = lds<f32x4>(base), x1 = lds<f32x4>(base + 8);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            av[g][u] = x0[u];
            av[g][u + 4] = x1[u];
          }
        }
        float blk0[NB0], blk1[NB1];
        if constexpr (G0.nb > 0) {
#pragma unroll
          for (int u = 0; u < NB0 / 4; ++u) {
            const f32x4 x = lds<f32x4>(QA + AB0 + 16 * ks + 4 * lh + G0.kb + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) blk0[4 * u + e] = x[e];
          }
        }
        if constexpr (NG > 1 && G1.nb > 0) {
#pragma unroll
          for (int u = 0; u < NB1 / 4; ++u) {
            const f32x4 x = lds<f32x4>(QA + AB1 + 16 * ks + 4 * lh + G1.kb + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) blk1[4 * u + e] = x[e];
          }
        }
        static_for<0, NSW>([&](auto sli) {
          constexpr int sl = decltype(sli)::value;
          constexpr Slot t = slot_info(SL.s[sl]);
          if constexpr (t.kind != S_Z) {
            // read-out: O^T[dv][query] += S^T phi~(Q)^T, features in the
            // accumulator order
            bf16x8 ph;
            if constexpr (t.kind == S_CLASS) {
              constexpr int g = t.abase == AB0 ? 0 : 1;
              constexpr int kb = g == 0 ? G0.kb : G1.kb;
#pragma unroll
              for (int s = 0; s < 8; ++s) {
                const float y = (g == 0 ? blk0 : blk1)[fpos(s) + t.koff - kb];
                const float x = t.koff == 0 ? 0.5f * av[g][s] : av[g][s];
                ph[s] = static_cast<__bf16>(x * y);
              }
            } else if constexpr (t.kind == S_LIN) {
              constexpr int g = t.abase == AB0 ? 0 : 1;
#pragma unroll
              for (int s = 0; s < 8; ++s) ph[s] = static_cast<__bf16>(av[g][s]);
            } else {  // the constant: feature 0 only
#pragma unroll
              for (int s = 0; s < 8; ++s) ph[s] = static_cast<__bf16>(ks == 0 && s == 0 && lh == 0 ? 1.f : 0.f);
            }
            bf16x8 sa;
#pragma unroll
            for (int s = 0; s < 8; ++s) sa[s] = static_cast<__bf16>(acc[sl][8 * ks + s]);
            O = mfma32(sa, ph, O);
          } else if (ks == 0) {
            // denominator part: sum_{i in zr, j in zc} q_i Z~_ij q_j (x2 off
            // the diagonal), as U = Z~^T q_zr then q_zc . U
            f32x16 U = f32x16{};
#pragma unroll
            for (int kz = 0; kz < 2; ++kz) {
              bf16x8 za;
#pragma unroll
              for (int s = 0; s < 8; ++s) za[s] = static_cast<__bf16>(acc[sl][8 * kz + s] * c2z);
              const int o = 32 * t.zr + 16 * kz + 4 * lh;
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
        });
      }
    }
    // update: S += phi(K)^T V (key products in fp16; rows past the segment's
    // end are zero in K and V, so they add nothing). Operands shared by the
    // wave's tiles: the V^T fragments and the key rows of its two ranges
    // (every tile of a range multiplies by the same row of K'^T).
    f16x8 bv[2], kx[NG][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bv[ks] = lds<f16x8>(V + lc * VTP + 16 * ks + 8 * lh);
#pragma unroll
      for (int g = 0; g < NG; ++g) kx[g][ks] = lds<f16x8>(K + ((g == 0 ? AB0 : AB1) + lc) * KTP + 16 * ks + 8 * lh);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      static_for<0, NSW>([&](auto sli) {
        constexpr int sl = decltype(sli)::value;
        constexpr Slot t = slot_info(SL.s[sl]);
        if constexpr (t.kind == S_CLASS) {
          constexpr int g = t.abase == AB0 ? 0 : 1;
          acc[sl] = mfma32h(kx[g][ks] * lds<f16x8>(K + (t.abase + t.koff + lc) * KTP + 16 * ks + 8 * lh), bv[ks],
                            acc[sl]);
        } else if constexpr (t.kind == S_LIN) {
          acc[sl] = mfma32h(kx[t.abase == AB0 ? 0 : 1][ks], bv[ks], acc[sl]);
        } else if constexpr (t.kind == S_CONST) {
          const _Float16 one = static_cast<_Float16>(lc == 0 ? 1.f : 0.f);
          acc[sl] = mfma32h(f16x8{one, one, one, one, one, one, one, one}, bv[ks], acc[sl]);
        } else {
          acc[sl] = mfma32h(kx[t.zr][ks], kx[t.zc][ks], acc[sl]);
        }
      });
    }
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
      typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
      const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
      const _Float16* kr0 = K + l * KTP;
      float zs = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f16x8 x = lds<f16x8>(kr0 + 8 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) zs = __builtin_amdgcn_fdot2(f16x2{x[2 * e], x[2 * e + 1]}, ones, zs, false);
      }
      z1r += zs;
    }
    if constexpr (W == W_AUX) {
      if (out) {
        // diagonal block: scores D[key][query] = K Q^T (raw), weights,
        // causal mask, then O^T += V^T P^T with keys in the accumulator order
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
    }
    if (!out) return;
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
  // unit 0 is written only when there is an initial state (zero otherwise)
  const bool from_unit = p > 0 || a.S0 != nullptr;
  const float z0base = from_unit ? unit_at(p)[Z0_F4].x : 0.f;

  // sum the partials of chunk i, normalise, store rows: waves 0..3 only,
  // which have issue priority on their SIMDs and finish the chunk's compute
  // first (four columns per thread)
  auto finalize = [&](int i) __attribute__((always_inline)) {
    if (w >= 4) return;
    const int q = tid >> 3, pc = tid & 7;
    const float* pt = part(i & 1) + q * PP + 4 * pc;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      o += *reinterpret_cast<const f32x4*>(pt + ww * C * PP);
      den += pden(i & 1)[ww * C + q];
    }
    den += z0base + static_cast<float>(i * C);  // constant term: tokens before this chunk
    const float rd = __builtin_amdgcn_rcpf(den);
    if (i * C + q < static_cast<int>(seg_rows)) {
      const size_t off = (static_cast<size_t>(bh) * N + t0 + i * C + q) * DV + DH * hv + 4 * pc;
      if constexpr (OBF) {
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + off) =
            bf16x4{static_cast<__bf16>(o[0] * rd), static_cast<__bf16>(o[1] * rd), static_cast<__bf16>(o[2] * rd),
                   static_cast<__bf16>(o[3] * rd)};
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + off) = o * rd;
      }
    }
  };


  // everything that depends on the wave's slot list, per wave ---------------
  auto wave_body = [&](auto wtag) __attribute__((always_inline)) {
    constexpr int W = decltype(wtag)::value;
    constexpr SlotList SL = wave_slots(W);
    constexpr int NSW = SL.n;
    f32x16 acc[NSW];
#pragma unroll
    for (int i = 0; i < NSW; ++i) acc[i] = f32x16{};
    float z1r = 0.f;  // wave W_Z1: z1 of coordinate l

    // initial state: unit p
    if (from_unit) {
      const float4* src = unit_at(p) + l;
#pragma unroll
      for (int i = 0; i < NSW; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = src[(SL.s[i] * 4 + q4) * 64];
          acc[i][4 * q4 + 0] = x.x;
          acc[i][4 * q4 + 1] = x.y;
          acc[i][4 * q4 + 2] = x.z;
          acc[i][4 * q4 + 3] = x.w;
        }
      if (W == W_Z1) z1r = reinterpret_cast<const float*>(unit_at(p) + Z1_F4)[l];
    }

    // chunk loop: iteration i stages chunk i+1, computes chunk i and
    // finishes chunk i-1
    ra = load_a(0);
    if (has_v) rvv = load_v(0);
    stage(0, 0);
    __syncthreads();
    for (int i = 0; i < nch; ++i) {
      stage(i + 1, (i + 1) & 1);
      compute_w(wtag, acc, z1r, i, i & 1, want_out);
      if (want_out && i > 0) finalize(i - 1);
      __syncthreads();
    }
    if (want_out && nch > 0) finalize(nch - 1);

    // results
    float4* dstu = nullptr;
    if (want_state && a.defer_state) {
      dstu = reinterpret_cast<float4*>(a.fin) + static_cast<size_t>(bhh) * UNIT_F4;
    }
    const float count = z0base + static_cast<float>(t1 - t0);
    if (dstu != nullptr) {
#pragma unroll
      for (int sl = 0; sl < NSW; ++sl)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dstu[(SL.s[sl] * 4 + q4) * 64 + l] =
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
        constexpr int s = SL.s[sl];
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

// Segment sums (update only) of segments 0..P-2, written to unit p + 1 of
// both value halves of the head. Here the features, not the value columns,
// are split over the two workgroups of a (head, segment): each holds its
// state tiles for all 64 value columns, so every key-product fragment feeds
// two matrix-core products (one per value half) and the key rows are read
// once per pair of tiles. 64 tokens are staged per barrier.
namespace fs {
constexpr int C = 64;                    // tokens per stage
constexpr int KTP = C + 8;               // K'^T rows (fp16): coordinates 0..63, then 0..31 again
constexpr int VTP = C + 8;               // V^T rows (fp16), all 64 value columns
constexpr int KT = 0;
constexpr int VT = KT + 96 * KTP * 2;
constexpr int BUF = VT + DV * VTP * 2;
static_assert(2 * BUF <= 160 * 1024 && VT % 16 == 0 && BUF % 16 == 0 && (KTP * 2) % 16 == 0, "LDS layout");

// Work of wave w of the workgroup holding feature half f: up to five state
// slots (each a tile per value half; key rows of first range AB = 32 f),
// at most one Gram tile, and (one wave) the key sums z1.
constexpr int MAXC = 5;
struct Work {
  int nc;
  int cls[MAXC];  // state slots 0..67
  int gram;       // Gram slot 68..70, or -1
  bool z1;
};
__host__ __device__ constexpr Work work(int f, int w) {
  if (f == 0) {
    // pair classes of the first range 0..31 and the linear tile of range 0
    if (w == NW - 1) return Work{5, {4 * w, 4 * w + 1, 4 * w + 2, 4 * w + 3, 65}, -1, false};
    return Work{4, {4 * w, 4 * w + 1, 4 * w + 2, 4 * w + 3, -1}, -1, false};
  }
  // pair classes of the range 32..63; the (r, r + 32) class, the second
  // linear tile, the constant, the Gram tiles and z1 on top
  const int b = 32 + 4 * w;
  if (w < 3) return Work{5, {b, b + 1, b + 2, b + 3, w == 0 ? 64 : (w == 1 ? 66 : 67)}, -1, false};
  if (w < 6) return Work{4, {b, b + 1, b + 2, b + 3, -1}, 68 + (w - 3), false};
  return Work{4, {b, b + 1, b + 2, b + 3, -1}, -1, w == 6};
}
constexpr bool work_partitioned() {
  int hits[NSLOT] = {};
  int z1 = 0;
  for (int f = 0; f < 2; ++f)
    for (int w = 0; w < NW; ++w) {
      const Work k = work(f, w);
      for (int i = 0; i < k.nc; ++i) {
        const int s = k.cls[i];
        if (s < 0 || s >= NS) return false;
        ++hits[s];
        const Slot t = slot_info(s);
        // pair classes and linear tiles use the workgroup's key range
        if ((t.kind == S_CLASS && s != 64) || t.kind == S_LIN)
          if (t.abase != 32 * f) return false;
      }
      if (k.gram >= 0) {
        if (k.gram < NS || k.gram >= NSLOT) return false;
        ++hits[k.gram];
      }
      z1 += k.z1 ? 1 : 0;
    }
  for (int s = 0; s < NSLOT; ++s)
    if (hits[s] != 1) return false;
  return z1 == 1;
}
static_assert(work_partitioned(), "every slot on exactly one wave of one feature half; z1 once");
}  // namespace fs

__global__ __launch_bounds__(NTHR, 1) void w2_segsum_fs(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * fs::BUF];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lc = l & 31, lh = l >> 5;
  const int PL = a.P - 1;
  // blocks of 16 workgroups: eight (head, segment) pairs with feature half 0,
  // then the same eight with half 1, so that the two halves of a pair are 8
  // apart in dispatch order (workgroups go to the 8 XCDs round-robin) and
  // share an L2 for the keys and values they both read
  const int grp = blockIdx.x >> 4, r16 = blockIdx.x & 15;
  const int f = r16 >> 3, hs = 8 * grp + (r16 & 7);  // (head, segment) index
  if (hs >= a.BH * PL) return;
  const int bh = hs / PL, p = hs - bh * PL;
  const int N = a.N;
  const int t0 = p * a.L;
  const int t1 = min(N, t0 + a.L);
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);
  const int nst = (t1 - t0 + fs::C - 1) / fs::C;

  auto kt = [&](int b) __attribute__((always_inline)) {
    return reinterpret_cast<_Float16*>(smem + b * fs::BUF + fs::KT);
  };
  auto vt = [&](int b) __attribute__((always_inline)) {
    return reinterpret_cast<_Float16*>(smem + b * fs::BUF + fs::VT);
  };
  const __bf16* kh = reinterpret_cast<const __bf16*>(a.k) + (static_cast<size_t>(bh) * N + t0) * D;
  const __bf16* vh = reinterpret_cast<const __bf16*>(a.v) + (static_cast<size_t>(bh) * N + t0) * DV;
  const auto rk = make_rsrc(kh, seg_rows * D * 2);
  const auto rv = make_rsrc(vh, seg_rows * DV * 2);

  // Staging: threads 0..255 hold a K item, 256..511 a V item: coordinates
  // (or columns) 8 ic8 .. + 8 of the token pair 2 tp, 2 tp + 1. The pair is
  // written to the transposed tile as one dword per coordinate. Rows past
  // the segment's end load as zero (buffer range), so they add nothing.
  const bool is_k = __builtin_amdgcn_readfirstlane(tid) < 256;
  const int it = tid & 255, ic8 = it >> 5, tp = it & 31;
  const auto rsrc = is_k ? rk : rv;
  uint4 r0, r1;
  auto load = [&](int c) __attribute__((always_inline)) {
    const int row = c * fs::C + 2 * tp;
    const uint32_t ra = static_cast<uint32_t>(row < static_cast<int>(seg_rows) ? row : static_cast<int>(seg_rows));
    const uint32_t rb =
        static_cast<uint32_t>(row + 1 < static_cast<int>(seg_rows) ? row + 1 : static_cast<int>(seg_rows));
    r0 = bload16(rsrc, (ra * 64 + 8 * ic8) * 2);  // D == DV == 64
    r1 = bload16(rsrc, (rb * 64 + 8 * ic8) * 2);
  };
  auto stage = [&](int b) __attribute__((always_inline)) {
    const f16x8 x0 = b2h(__builtin_bit_cast(bf16x8, r0));
    const f16x8 x1 = b2h(__builtin_bit_cast(bf16x8, r1));
    _Float16* t = is_k ? kt(b) : vt(b);
    const int pitch = is_k ? fs::KTP : fs::VTP;
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<f16x2*>(t + (8 * ic8 + u) * pitch + 2 * tp) = f16x2{x0[u], x1[u]};
    if (is_k && ic8 < 4) {
#pragma unroll
      for (int u = 0; u < 8; ++u) *reinterpret_cast<f16x2*>(t + (D + 8 * ic8 + u) * pitch + 2 * tp) = f16x2{x0[u], x1[u]};
    }
  };

  auto wave_body = [&](auto ftag, auto wtag) __attribute__((always_inline)) {
    constexpr int FH = decltype(ftag)::value;
    constexpr int W = decltype(wtag)::value;
    constexpr fs::Work WK = fs::work(FH, W);
    constexpr int NC = WK.nc;
    constexpr int AB = 32 * FH;  // first key range of the workgroup
    constexpr bool HAS_G = WK.gram >= 0;
    // the auxiliary key range (coordinates 32 (1 - FH) + lc) is needed by the
    // (r, r + 32) class and by Gram tiles that touch it
    constexpr bool NEED_OTHER = [] {
      for (int i = 0; i < WK.nc; ++i)
        if (WK.cls[i] == 64) return true;
      if (WK.gram >= 0) {
        const Slot g = slot_info(WK.gram);
        if (32 * g.zr != 32 * FH || 32 * g.zc != 32 * FH) return true;
      }
      return false;
    }();
    f32x16 acc[2 * NC + (HAS_G ? 1 : 0)];
#pragma unroll
    for (int i = 0; i < 2 * NC + (HAS_G ? 1 : 0); ++i) acc[i] = f32x16{};
    float z1r = 0.f;
    auto chunk = [&](int b) __attribute__((always_inline)) {
      const _Float16* K = kt(b);
      const _Float16* V = vt(b);
#pragma unroll
      for (int ks = 0; ks < fs::C / 16; ++ks) {
        const int col = 16 * ks + 8 * lh;
        const f16x8 bv0 = lds<f16x8>(V + lc * fs::VTP + col);
        const f16x8 bv1 = lds<f16x8>(V + (32 + lc) * fs::VTP + col);
        const f16x8 kx = lds<f16x8>(K + (AB + lc) * fs::KTP + col);
        f16x8 ko = kx;
        if constexpr (NEED_OTHER) ko = lds<f16x8>(K + (32 - AB + lc) * fs::KTP + col);
        static_for<0, NC>([&](auto ci) {
          constexpr int i = decltype(ci)::value;
          constexpr int s = WK.cls[i];
          constexpr Slot t = slot_info(s);
          f16x8 x;
          if constexpr (s == 64) {
            x = FH == 0 ? kx * ko : ko * kx;  // rows r and r + 32
          } else if constexpr (t.kind == S_CLASS) {
            x = kx * lds<f16x8>(K + (AB + t.koff + lc) * fs::KTP + col);
          } else if constexpr (t.kind == S_LIN) {
            x = kx;
          } else {  // the constant
            const _Float16 one = static_cast<_Float16>(lc == 0 ? 1.f : 0.f);
            x = f16x8{one, one, one, one, one, one, one, one};
          }
          acc[2 * i] = mfma32h(x, bv0, acc[2 * i]);
          acc[2 * i + 1] = mfma32h(x, bv1, acc[2 * i + 1]);
        });
        if constexpr (HAS_G) {
          constexpr Slot g = slot_info(WK.gram);
          const f16x8 xr = 32 * g.zr == AB ? kx : ko;
          const f16x8 xc = 32 * g.zc == AB ? kx : ko;
          acc[2 * NC] = mfma32h(xr, xc, acc[2 * NC]);
        }
      }
      if constexpr (WK.z1) {
        // z1 += keys (lane l = coordinate l), summed with fp16 dot2
        const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
        const _Float16* kr0 = K + l * fs::KTP;
        float zs = 0.f;
#pragma unroll
        for (int u = 0; u < fs::C / 8; ++u) {
          const f16x8 x = lds<f16x8>(kr0 + 8 * u);
#pragma unroll
          for (int e = 0; e < 4; ++e) zs = __builtin_amdgcn_fdot2(f16x2{x[2 * e], x[2 * e + 1]}, ones, zs, false);
        }
        z1r += zs;
      }
    };
    load(0);
    stage(0);
    load(1);
    __syncthreads();
    for (int c = 0; c < nst; ++c) {
      if (c + 1 < nst) stage((c + 1) & 1);
      load(c + 2);
      chunk(c & 1);
      __syncthreads();
    }
    // results: unit p + 1 of both value halves
    float4* dst[2];
#pragma unroll
    for (int hv = 0; hv < 2; ++hv)
      dst[hv] = reinterpret_cast<float4*>(a.seg) + (static_cast<size_t>(bh * 2 + hv) * a.P + p + 1) * UNIT_F4;
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int hv = 0; hv < 2; ++hv)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dst[hv][(WK.cls[i] * 4 + q4) * 64 + l] = float4{acc[2 * i + hv][4 * q4], acc[2 * i + hv][4 * q4 + 1],
                                                           acc[2 * i + hv][4 * q4 + 2], acc[2 * i + hv][4 * q4 + 3]};
    if constexpr (HAS_G) {
#pragma unroll
      for (int hv = 0; hv < 2; ++hv)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dst[hv][(WK.gram * 4 + q4) * 64 + l] = float4{acc[2 * NC][4 * q4], acc[2 * NC][4 * q4 + 1],
                                                         acc[2 * NC][4 * q4 + 2], acc[2 * NC][4 * q4 + 3]};
    }
    if constexpr (WK.z1) {
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        reinterpret_cast<float*>(dst[hv] + Z1_F4)[l] = z1r;
        if (l == 0) dst[hv][Z0_F4] = float4{static_cast<float>(t1 - t0), 0.f, 0.f, 0.f};
      }
    }
  };
  auto per_wave = [&](auto ftag) __attribute__((always_inline)) {
    switch (w) {
      case 0: wave_body(ftag, std::integral_constant<int, 0>{}); break;
      case 1: wave_body(ftag, std::integral_constant<int, 1>{}); break;
      case 2: wave_body(ftag, std::integral_constant<int, 2>{}); break;
      case 3: wave_body(ftag, std::integral_constant<int, 3>{}); break;
      case 4: wave_body(ftag, std::integral_constant<int, 4>{}); break;
      case 5: wave_body(ftag, std::integral_constant<int, 5>{}); break;
      case 6: wave_body(ftag, std::integral_constant<int, 6>{}); break;
      default: wave_body(ftag, std::integral_constant<int, 7>{}); break;
    }
  };
  if (f == 0)
    per_wave(std::integral_constant<int, 0>{});
  else
    per_wave(std::integral_constant<int, 1>{});
}

// Unit 0 of each (head, half): S0/z0 in the internal layout (launched only
// with an initial state; without one the scan and the main launch take unit
// 0 as zero and never read it). One workgroup of 64 threads per (head, half,
// slot), plus one per (head, half) for z1 and z0.
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
__global__ __launch_bounds__(256) void w2_scan(float4* seg, int BHH, int PS, int has_s0) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(BHH) * UNIT_F4) return;
  const int64_t u = e / UNIT_F4, pos = e - u * UNIT_F4;
  float4* base = seg + u * PS * static_cast<int64_t>(UNIT_F4) + pos;
  float4 acc = has_s0 ? base[0] : float4{0.f, 0.f, 0.f, 0.f};  // unit 0: S0 (zero without one)
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
  if (a.S0 != nullptr) {
    hipLaunchKernelGGL(w2_s0_unit, dim3(a.BH * 2 * (NSLOT + 1)), dim3(64), 0, stream, a.S0, a.z0, seg, a.P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.P > 1) {
    hipLaunchKernelGGL(w2_segsum_fs, dim3(16 * ((a.BH * (a.P - 1) + 7) / 8)), dim3(NTHR), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = static_cast<int64_t>(a.BH) * 2 * UNIT_F4;
    hipLaunchKernelGGL(w2_scan, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, seg, a.BH * 2,
                       a.P, a.S0 != nullptr ? 1 : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.o == nullptr || a.out_bf16)
    hipLaunchKernelGGL((w2_kernel<true>), dim3(a.BH * 2 * a.P), dim3(NTHR), 0, stream, a);
  else
    hipLaunchKernelGGL((w2_kernel<false>), dim3(a.BH * 2 * a.P), dim3(NTHR), 0, stream, a);
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
