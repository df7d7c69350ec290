// Chunked causal prefill of Taylor-series linear attention on gfx950.
//
// Method ("Expanding Attention: A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States"):
//   o_t = sum_{s<=t} w(q_t.k_s/a) v_s / sum_{s<=t} w(q_t.k_s/a),
//   w(x) = sum_{m<n} x^m/m!.
// "Time" on that page splits prefill into a state part and diagonal blocks
// of size c: for a chunk of c tokens,
//   O  = phi~(Q_c) S_<c   (read-out of the state of all earlier tokens)
//      + P V_c            (P_ij = w(q_i.k_j/a), j <= i inside the chunk)
//   S += phi(K_c)^T [V_c, 1]   (per-order states, "Memory")
// with phi~ = phi with alpha_m = 1/(m! a^m) folded in. The trailing column
// of ones carries the denominator through the same contractions. States are
// additive (closing paragraph of the page), which gives the sequence split
// below.
//
// Work decomposition on the chip:
//  * A workgroup owns one (head, segment, feature slice). Segment sums of
//    earlier segments arrive from a first pass (MODE_SEGSUM); the state slice
//    [FS x (dv+16)] lives in the accumulator registers of NW = dv/16 + 1
//    waves, wave w holding dv columns 16w..16w+15 (the last wave holds the
//    ones column, i.e. the denominator state z).
//  * Per chunk: stage Q, K and V^T (+ ones row) in LDS; generate phi~(Q)
//    [C x FS] and phi(K) [FS x C] in LDS; score tiles K Q^T on MFMA with the
//    polynomial and causal mask applied in registers; read-out, intra-chunk
//    and update contractions on MFMA.
//  * With one slice (small feature widths) the workgroup normalises and
//    writes o itself; with several slices each writes a partial
//    (numerator, denominator) and a small kernel sums and divides.
#include "features.hpp"
#include "qarrange.hpp"
#include "internal.hpp"
#include "mma.hpp"

#include <type_traits>
#include <utility>

namespace tl {

// ---------------------------------------------------------------------------
// compile-time helpers
// ---------------------------------------------------------------------------

template <int B, class Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& fn, std::integer_sequence<int, Is...>) {
  (fn(std::integral_constant<int, B + Is>{}), ...);
}
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (E > B) static_for_impl<B>(fn, std::make_integer_sequence<int, E - B>{});
}

// 1/m! as float, m < n (Horner coefficients of the truncated exponential).
template <int NT>
__device__ __forceinline__ float taylor_poly(float t) {
  // w(t) = sum_{m<NT} t^m/m!, Horner from the highest term down.
  float p = static_cast<float>(1.0 / static_cast<double>(factorial(NT - 1)));
  static_for<0, NT - 1>([&](auto jj) {
    constexpr int m = NT - 2 - decltype(jj)::value;
    p = __builtin_fmaf(p, t, static_cast<float>(1.0 / static_cast<double>(factorial(m))));
  });
  return p;
}

// ---------------------------------------------------------------------------
// configuration of one instantiation
// ---------------------------------------------------------------------------

template <int D_, int DV_, int NT_, bool BF16_, int FS_, int C_, bool UNROLL_>
struct PCfg {
  static constexpr bool ZS_() { return !UNROLL_ && DV_ == 64; }
  static constexpr int D = D_, DV = DV_, NT = NT_, FS = FS_, C = C_;
  static constexpr bool BF16 = BF16_, UNROLL = UNROLL_;
  using M = Mma<BF16>;
  using E = typename M::elem;
  static constexpr int ES = sizeof(E);
  static constexpr int F = feature_count(D, NT);
  static constexpr int G = (F + FS - 1) / FS;
  // Denominator state z (the state of the ones column of [V, 1]). With the
  // table-driven generator at dv = 64 ("split z") eight waves, two per SIMD,
  // hold the state: wave w the value tiles 2 (w % 2) and 2 (w % 2) + 1 of
  // feature group w / 2 (a quarter of the slice), and z for a share of that
  // group's read-out k-steps, so that every phi fragment read from LDS feeds
  // two or three MFMAs. Otherwise one wave per value tile holds all of the
  // slice's features and a last wave holds z as a sixteen-column tile.
  static constexpr bool ZS = ZS_();
  // wide split-z slices (one workgroup per compute unit in any case): the
  // read-out partials of every feature group go through LDS and all waves
  // sum, normalise and store the chunk's output; narrower ones keep to the
  // LDS budget of two workgroups per compute unit (group 0 sums)
  static constexpr bool WIDE = ZS && FS >= 512;
  static constexpr int NDT = ZS ? 2 : 1;  // value tiles per wave
  static constexpr int NFG = ZS ? 4 : 1;  // feature groups
  static constexpr int NW = ZS ? (DV / 16 / NDT) * NFG : DV / 16 + 1;
  static constexpr int NTHR = NW * 64;
  static constexpr int DVP = (DV / 16 + 1) * 16;  // V^T rows: values, the ones row, zero padding
  static constexpr int FT = FS / 16;    // 16-feature tiles per slice
  static constexpr int KSF = FS / 32;   // read-out k-steps
  static constexpr int FTG = FT / NFG;  // feature tiles per group
  static constexpr int KSG = KSF / NFG; // read-out k-steps per group
  // split z: in each feature group the wave of dv pair 0 holds z for the
  // group's k-steps [0, KZ0), the wave of dv pair 1 for [KZ0, KSG)
  static constexpr int KZ0 = KSG / 2;
  static constexpr int ZT = ZS ? 2 * (KSG - KZ0) : 0;  // z tiles per wave (at most)
  // per-(unit, slice) state in the accumulator layout: NW waves x (NDT FTG
  // value tiles + ZT z tiles) x 64 lanes of float4
  static constexpr int TPW = NDT * FTG + ZT;
  static constexpr size_t SLICE_F4 = static_cast<size_t>(NW) * TPW * 64;
  static constexpr int NDEN = 1;  // denominator columns of a partial-output row
  static constexpr int QT = C / 16;    // query tiles per chunk
  static constexpr int KSC = C / 32;   // key k-steps per chunk
  static constexpr int PADE = 16 / ES; // 16 bytes of padding, in elements
  static constexpr int XP = D + PADE;  // Q/K tile pitch
  static constexpr int PQ = FS + PADE; // phi~(Q) pitch (query-major)
  // phi(K)^T, V^T pitch (key-contiguous); wide bf16 slices pad by 48 bytes
  // (order 4: 1.2% faster than 16, same bank-conflict count)
  static constexpr int PK = C + (WIDE && ES == 2 ? 24 : PADE);
  static constexpr int PP = C + PADE;  // P^T pitch (query-major, keys contiguous)
  static constexpr int PPITCH = DV + 4;  // partial-output row pitch (floats)
  // LDS layout (bytes)
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + C * XP * ES;
  static constexpr int OFF_V = OFF_K + C * XP * ES;
  static constexpr int OFF_PQ = OFF_V + DVP * PK * ES;
  static constexpr int OFF_PK = OFF_PQ + C * PQ * ES;
  static constexpr int OFF_P = OFF_PK + FS * PK * ES;
  static constexpr int OFF_DEN = OFF_P + C * PP * ES;
  // table-driven generator: per-token factor tables T^T [TE][TP] fp32 for the
  // query and the key side (1, the coordinates, and for orders above 2 the
  // pair products), token-contiguous
  static constexpr bool PAIRS = NT > 3;
  // orders 5 and 6 are products of three table entries; their features are
  // decoded at run time (no compile-time basis table) and the key side
  // carries the sqrt-multinomial weight, so that internal and canonical
  // state rows differ by KS^m only
  static constexpr bool TRIPLE = NT > 5;
  // order 4 at d = 16 with bf16 inputs: the query features are generated
  // per token with compile-time indices (one code path per slice and wave)
  // and only the key side keeps a factor table
  static constexpr bool QGEN = BF16 && !UNROLL && D == 16 && NT == 5 && C == 32 && DV == 64;
  static constexpr bool TAB = !UNROLL;  // factor tables (key side; query side unless QGEN)
  static constexpr int TE = TAB ? 1 + D + (PAIRS ? D * (D + 1) / 2 : 0) : 0;
  static constexpr int TQE = QGEN ? 0 : TE;  // query table rows
  static constexpr int TP = C + 4;
  // key side of the table-driven generator: bf16 inputs keep the key table,
  // phi(K)^T and the update contraction in fp16 (keys scaled by KS, so
  // features of order m carry KS^m), fp32 inputs in fp32
  static constexpr bool KH = BF16 && !UNROLL;
  static constexpr float KS = KH ? 0.5f : 1.f;
  static constexpr int KES = KH ? 2 : ES;
  static constexpr int TPK = KH ? C + 8 : C + 4;
  // (split z: the denominator shares of all waves, [NW][C])
  static constexpr int OFF_TQ = OFF_DEN + (ZS_() ? NW : 1) * C * 4;
  static constexpr int OFF_TK = OFF_TQ + TQE * TP * 4;
  static constexpr int TAB_END = OFF_TK + TE * TPK * KES;
  // split z: the read-out partials of the feature groups (all of them, or
  // 1 .. NFG-1 when group 0 sums; [C][DV] each, f32x4 per lane and tile)
  // reuse the factor tables, which are dead from the feature generation to
  // the next chunk's staging
  static constexpr int OFF_RED = OFF_TQ;
  static constexpr int RED_END = OFF_RED + (ZS_() ? (WIDE ? NFG : NFG - 1) * C * DV * 4 : 0);
  static constexpr int LDS = TAB_END > RED_END ? TAB_END : RED_END;
  static_assert(NT <= 7, "features are products of at most three table entries (order 6)");
  static_assert(!TRIPLE || (PAIRS && !UNROLL), "orders 5 and 6 use the table-driven generator with pairs");
  static_assert(FS % 32 == 0 && C % 32 == 0 && DV % 16 == 0, "tile multiples");
  static_assert(D % 16 == 0, "head dim multiple of 16");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(DV + NDEN <= PPITCH, "partial-output row holds the values and the denominator columns");
  static_assert(!ZS || (FS % (32 * NFG) == 0 && DV == 16 * NDT * (NW / NFG)), "split z: whole k-steps per group");
  static_assert(!WIDE || (C / 16) * (DV / 16) * 64 == NTHR, "wide split z: one output item of the chunk per thread");
  static_assert(!QGEN || (ZS && FS % (8 * NW) == 0), "per-token generator: whole 8-feature packs per wave");
  // score tiles (kt, qt) needed per chunk: key tiles up to the end of the
  // 32-key step that contains the diagonal tile
  static constexpr int NTILES = [] {
    int n = 0;
    for (int qt = 0; qt < C / 16; ++qt) n += 2 * (qt / 2) + 2;
    return n;
  }();
};

template <class Cfg>
struct TileList {
  int kt[Cfg::NTILES];
  int qt[Cfg::NTILES];
};
template <class Cfg>
constexpr TileList<Cfg> make_tiles() {
  TileList<Cfg> t{};
  int n = 0;
  for (int qt = 0; qt < Cfg::QT; ++qt)
    for (int kt = 0; kt < 2 * (qt / 2) + 2; ++kt) {
      t.kt[n] = kt;
      t.qt[n] = qt;
      ++n;
    }
  return t;
}

// ---------------------------------------------------------------------------
// feature generation, unrolled (whole basis in one slice; small widths)
// ---------------------------------------------------------------------------

// Value of feature f for a row x (query side: x already divided by a and the
// 1/m! folded into the constants).
template <int D, int NT, bool QSIDE, int f>
__device__ __forceinline__ float feat_val(const float (&x)[D]) {
  if constexpr (f >= feature_count(D, NT)) {
    return 0.f;
  } else {
    constexpr GenConst gc = gen_const<D, NT, QSIDE>(f);
    if constexpr (gc.m == 0) {
      return static_cast<float>(gc.G);
    } else {
      float p = static_cast<float>(gc.G);
      static_for<0, gc.m - 1>([&](auto jj) { p = p * x[gc.idx[decltype(jj)::value]]; });
      float v = p * x[gc.idx[gc.m - 1]];
      if constexpr (gc.R != 1.0) v = v * static_cast<float>(gc.R);
      return v;
    }
  }
}

// phi~(q) for features [8*PB, 8*PE) of one token, written as 8-wide packs
// into its row of the query-major tile.
template <class Cfg, int PB, int PE>
__device__ __forceinline__ void gen_q_packs(const float (&x)[Cfg::D], typename Cfg::E* row) {
  using E = typename Cfg::E;
  static_for<PB, PE>([&](auto pi) {
    constexpr int p = decltype(pi)::value;
    E vals[8];
    static_for<0, 8>([&](auto ji) {
      constexpr int f = 8 * p + decltype(ji)::value;
      vals[decltype(ji)::value] = Cfg::M::cvt(feat_val<Cfg::D, Cfg::NT, true, f>(x));
    });
    if constexpr (Cfg::BF16) {
      bf16x8 pk;
#pragma unroll
      for (int j = 0; j < 8; ++j) pk[j] = vals[j];
      *reinterpret_cast<bf16x8*>(row + 8 * p) = pk;
    } else {
      f32x4 a = {vals[0], vals[1], vals[2], vals[3]};
      f32x4 b = {vals[4], vals[5], vals[6], vals[7]};
      *reinterpret_cast<f32x4*>(row + 8 * p) = a;
      *reinterpret_cast<f32x4*>(row + 8 * p + 4) = b;
    }
  });
}

// phi(k) for features [8*PB, 8*PE) of one token, into its column of the
// feature-major tile.
template <class Cfg, int PB, int PE>
__device__ __forceinline__ void gen_k_packs(const float (&x)[Cfg::D], typename Cfg::E* col) {
  static_for<8 * PB, 8 * PE>([&](auto fi) {
    constexpr int f = decltype(fi)::value;
    col[f * Cfg::PK] = Cfg::M::cvt(feat_val<Cfg::D, Cfg::NT, false, f>(x));
  });
}

template <class Cfg, bool QSIDE>
__device__ __forceinline__ void gen_unrolled(int w, const float (&x)[Cfg::D], typename Cfg::E* dst) {
  constexpr int NP = Cfg::FS / 8;
  static_for<0, Cfg::NW>([&](auto wi) {
    constexpr int W = decltype(wi)::value;
    constexpr int PB = W * NP / Cfg::NW;
    constexpr int PE = (W + 1) * NP / Cfg::NW;
    if (w == W) {
      if constexpr (QSIDE)
        gen_q_packs<Cfg, PB, PE>(x, dst);
      else
        gen_k_packs<Cfg, PB, PE>(x, dst);
    }
  });
}

// ---------------------------------------------------------------------------
// query features per token with compile-time indices (order 4, d = 16)
// ---------------------------------------------------------------------------
// Features sit in the internal order of qarrange.hpp: per wave range of FW
// positions, HALF = FW / 2 representatives, then their images under the
// rotation of the coordinates by d/2. Lane t < 32 of a wave computes the
// representatives for token t of the chunk from q / (a KS) in registers,
// lane 32 + t the same instructions on the rotated coordinates, i.e. the
// images; each stores 16-byte packs into the token's row of phi~(Q). Code is
// straight-line with compile-time feature indices, one path per slice and
// wave. The query features are plain products; the key side (table path)
// carries the weight w^2 / m! = 1 / prod_i c_i! (c_i the multiplicities of
// the tuple), one packed multiply per eight keys.

template <class Cfg>
inline constexpr auto kQArr = make_qarrange<Cfg::D, Cfg::NT, Cfg::FS / Cfg::NW / 2>();
template <class Cfg>
__device__ const auto g_qarr = kQArr<Cfg>;

// Canonical feature of slice position f (-1: no feature there).
template <class Cfg>
__device__ __forceinline__ int canon_feat(int f) {
  if constexpr (Cfg::QGEN) {
    return f < kQArr<Cfg>.npos ? g_qarr<Cfg>.perm[f] : -1;
  } else {
    return f < Cfg::F ? f : -1;
  }
}

template <int D, int NT, int f>
__device__ __forceinline__ float qfeat_val(const float (&x)[D]) {
  constexpr Monomial e = kBasis<D, NT>.e[f];
  if constexpr (e.m == 0) {
    return 1.f;
  } else {
    // left-to-right products: features that share a prefix share its
    // product after value numbering
    float p = x[e.idx[0]];
    static_for<1, e.m>([&](auto jj) { p = p * x[e.idx[decltype(jj)::value]]; });
    return p;
  }
}

template <class Cfg, int SL, int W>
__device__ __forceinline__ void gen_q_wave(const float (&x)[Cfg::D], bool rot, typename Cfg::E* dq) {
  constexpr int HALF = Cfg::FS / Cfg::NW / 2;
  static_for<0, HALF / 8>([&](auto pi) {
    constexpr int p = decltype(pi)::value;
    bf16x8 pk;
    static_for<0, 8>([&](auto ji) {
      constexpr int j = decltype(ji)::value;
      constexpr int i = (SL * Cfg::NW + W) * HALF + 8 * p + j;  // representative
      float v = 0.f;
      if constexpr (i < kQArr<Cfg>.nA) {
        v = qfeat_val<Cfg::D, Cfg::NT, kQArr<Cfg>.a[i]>(x);
        // a fixed point has no image: the rotated lanes store zero
        if constexpr (!kQArr<Cfg>.paired[i]) v = rot ? 0.f : v;
      }
      pk[j] = static_cast<__bf16>(v);
    });
    *reinterpret_cast<bf16x8*>(dq + 8 * p) = pk;
  });
}

// phi~(Q) of the slice for one chunk (query-major). The slice and the wave
// pick one of G x NW straight-line code paths (scalar branches).
template <class Cfg>
__device__ __forceinline__ void gen_q_token(int gsl, int w, int lane, const typename Cfg::E* sQ,
                                            typename Cfg::E* sPQ, float inv_a) {
  constexpr int D = Cfg::D, FW = Cfg::FS / Cfg::NW;
  static_assert(Cfg::C == 32 && D == 16 && Cfg::ES == 2, "one token per lane pair, two 16-byte halves per row");
  static_assert(kQArr<Cfg>.npos <= Cfg::G * Cfg::FS, "internal order fits the slices");
  const int t = lane & 31;
  const bool rot = lane >= 32;
  // rotation by d/2: the rotated lanes read the two halves of the row swapped
  const typename Cfg::E* xr = sQ + t * Cfg::XP;
  const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(xr + (rot ? 8 : 0));
  const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(xr + (rot ? 0 : 8));
  const float sc = inv_a / Cfg::KS;
  float x[D];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = static_cast<float>(h0[j]) * sc;
    x[8 + j] = static_cast<float>(h1[j]) * sc;
  }
  typename Cfg::E* row = sPQ + t * Cfg::PQ + (rot ? FW / 2 : 0);
  static_for<0, Cfg::G>([&](auto si) {
    constexpr int SL = decltype(si)::value;
    if (gsl == SL) {
      static_for<0, Cfg::NW>([&](auto wi) {
        constexpr int W = decltype(wi)::value;
        if (w == W) gen_q_wave<Cfg, SL, W>(x, rot, row + W * FW);
      });
    }
  });
}

// ---------------------------------------------------------------------------
// feature generation, table-driven (large widths; one slice of the basis)
// ---------------------------------------------------------------------------

template <int D, int NT>
__device__ const PackedTable<D, NT> g_ptab = make_packed<D, NT>();

// Table-driven generation. Every feature of order m <= 4 is the product of
// two entries of a per-token factor table T = [1, x_0..x_{d-1}, x_i x_j
// (i <= j, lexicographic; orders above 2 only)] times a constant:
//   m = 0: T[0] T[0],  m = 1: T[0] T[1+i],  m = 2: T[0] T[pair(i,j)] (or
//   T[1+i] T[1+j] without pairs),  m = 3: T[pair(i,j)] T[1+k],
//   m = 4: T[pair(i,j)] T[pair(k,l)],
// and with a third entry (bases up to order 6)
//   m = 5: T[pair(i,j)] T[pair(k,l)] T[1+p],  m = 6: three pairs,
// the third entry being T[0] = 1 for lower orders.
// The tables are built once per chunk; each lane owns a feature and reads
// its rows 16 bytes at a time.
template <int D>
__host__ __device__ constexpr int tab_pair(int i, int j) {
  return 1 + D + i * D - i * (i - 1) / 2 + (j - i);
}

// The key side carries plain products of the scaled keys, u(KS k); the
// query side carries every weight, w^2 alpha_m / KS^m with w the
// sqrt-multinomial and alpha_m = 1 / (m! a^m), so that the read-out equals
// the canonical one. Internal states relate to canonical ones by
// canonical = (w / KS^m) internal.
struct TabFeat {
  int oa, ob, oc;  // offsets (elements) of the table rows, query table (oc: third entry)
  int ka, kb, kc;  // the same rows in the key table
  float cq;        // query-side weight
  float ck;        // key-side weight (bases with three-entry features; 1 otherwise)
};

template <class Cfg>
__device__ __forceinline__ TabFeat tab_feat(int f, float inv_a) {
  constexpr int D = Cfg::D, TP = Cfg::TP;
  TabFeat t{0, 0, 0, 0, 0, 0, 0.f, 0.f};
  f = canon_feat<Cfg>(f);  // slice position -> canonical feature
  if (f < 0) return t;
  int m, i0, i1, i2, i3, i4 = 0, i5 = 0;
  float w, inv_mfact;
  if constexpr (Cfg::TRIPLE) {
    const RankedFeature e = rank_decode(D, Cfg::NT, f);
    m = e.m;
    i0 = e.idx[0], i1 = e.idx[1], i2 = e.idx[2], i3 = e.idx[3], i4 = e.idx[4], i5 = e.idx[5];
    w = e.w;
    inv_mfact = 1.f;
    for (int j = 2; j <= m; ++j) inv_mfact *= 1.f / static_cast<float>(j);
  } else {
    const PackedFeature e = g_ptab<D, Cfg::NT>.e[f];
    m = static_cast<int>(e.m);
    i0 = e.idx & 255, i1 = (e.idx >> 8) & 255, i2 = (e.idx >> 16) & 255, i3 = e.idx >> 24;
    w = e.w;
    inv_mfact = e.inv_mfact;
  }
  int a = 0, b = 0, c = 0;
  if (m == 1) {
    b = 1 + i0;
  } else if (m == 2) {
    if constexpr (Cfg::PAIRS) {
      b = tab_pair<D>(i0, i1);
    } else {
      a = 1 + i0;
      b = 1 + i1;
    }
  } else if (m == 3) {
    a = tab_pair<D>(i0, i1);
    b = 1 + i2;
  } else if (m == 4) {
    a = tab_pair<D>(i0, i1);
    b = tab_pair<D>(i2, i3);
  } else if (m == 5) {
    a = tab_pair<D>(i0, i1);
    b = tab_pair<D>(i2, i3);
    c = 1 + i4;
  } else if (m == 6) {
    a = tab_pair<D>(i0, i1);
    b = tab_pair<D>(i2, i3);
    c = tab_pair<D>(i4, i5);
  }
  t.oa = a * TP;
  t.ob = b * TP;
  t.oc = c * TP;
  t.ka = a * Cfg::TPK;
  t.kb = b * Cfg::TPK;
  t.kc = c * Cfg::TPK;
  // three-entry bases: key side w u(KS k), query side w alpha_m / KS^m;
  // per-token query features (their own generator): key side
  // (w^2 / m!) u(KS k); otherwise key side u(KS k), query side
  // w^2 alpha_m / KS^m
  float cq = (Cfg::TRIPLE ? w : w * w) * inv_mfact;
  for (int j = 0; j < m; ++j) cq *= inv_a / Cfg::KS;
  t.cq = cq;
  t.ck = Cfg::TRIPLE ? w : (Cfg::QGEN ? w * w * inv_mfact : 1.f);
  return t;
}

// canonical / internal state row scale of feature f (1 for the unrolled
// generators, which weight both sides)
template <class Cfg>
__device__ __forceinline__ float state_scale(int f) {
  if constexpr (Cfg::UNROLL) {
    return 1.f;
  } else if constexpr (Cfg::TRIPLE) {
    // internal rows carry w KS^m: canonical = internal / KS^m
    int m = 0;
    long long end = 1;
    while (m + 1 < Cfg::NT && f >= end) {
      ++m;
      end += rank_binom(Cfg::D + m - 1, m);
    }
    float sc = 1.f;
    for (int j = 0; j < m; ++j) sc *= 1.f / Cfg::KS;
    return sc;
  } else {
    // internal rows carry KS^m (and with per-token query features w^2 / m!):
    // canonical = w / KS^m internal (m! / (w KS^m) internal)
    const PackedFeature e = g_ptab<Cfg::D, Cfg::NT>.e[f];
    float sc = Cfg::QGEN ? 1.f / (e.w * e.inv_mfact) : e.w;
    for (int j = 0; j < static_cast<int>(e.m); ++j) sc *= 1.f / Cfg::KS;
    return sc;
  }
}

// Pair rows of both tables from their coordinate rows (rows 1..D, written
// while staging): T[pair(i,j)][t] = T[1+i][t] T[1+j][t], 16 bytes at a time.
// Thread tid handles pairs tid, tid + NTHR, ... of the query pairs and then
// the key pairs (key pairs only with per-token query features), so the jobs
// sit on the first waves, which have issue priority on their SIMDs; their
// coordinates are decoded once per kernel.
template <class Cfg>
struct PairJobs {
  static constexpr int NPAIR = Cfg::D * (Cfg::D + 1) / 2;
  static constexpr int NQP = Cfg::QGEN ? 0 : NPAIR;  // query-side pair jobs
  static constexpr int N = Cfg::PAIRS ? (NQP + NPAIR + Cfg::NTHR - 1) / Cfg::NTHR : 0;
  int ij[N > 0 ? N : 1];  // i | j << 8, or -1
};
template <class Cfg>
__device__ __forceinline__ PairJobs<Cfg> pair_jobs(int tid) {
  constexpr int D = Cfg::D, NPAIR = PairJobs<Cfg>::NPAIR, NQP = PairJobs<Cfg>::NQP;
  PairJobs<Cfg> pj;
#pragma unroll
  for (int n = 0; n < PairJobs<Cfg>::N; ++n) {
    const int k = tid + n * Cfg::NTHR;
    pj.ij[n] = -1;
    if (k < NQP + NPAIR) {
      int r = k < NQP ? k : k - NQP, pi = 0;
      while (r >= D - pi) {
        r -= D - pi;
        ++pi;
      }
      pj.ij[n] = pi | (pi + r) << 8;
    }
  }
  return pj;
}
template <class Cfg, class KE>
__device__ __forceinline__ void build_pairs(int tid, const PairJobs<Cfg>& pj, float* __restrict__ TQ,
                                            KE* __restrict__ TK, bool qside) {
  constexpr int D = Cfg::D, C = Cfg::C, NQP = PairJobs<Cfg>::NQP;
#pragma unroll
  for (int n = 0; n < PairJobs<Cfg>::N; ++n) {
    const int k = tid + n * Cfg::NTHR;
    const int ij = pj.ij[n];
    if (ij < 0) continue;
    const int pi = ij & 255, pjj = ij >> 8;
    if (k < NQP) {
      if (!qside) continue;
      const f32x4* xi = reinterpret_cast<const f32x4*>(TQ + (1 + pi) * Cfg::TP);
      const f32x4* xj = reinterpret_cast<const f32x4*>(TQ + (1 + pjj) * Cfg::TP);
      f32x4* dst = reinterpret_cast<f32x4*>(TQ + tab_pair<D>(pi, pjj) * Cfg::TP);
      // all reads of a half row before its writes (same table: no reordering)
#pragma unroll
      for (int h = 0; h < C / 4; h += 4) {
        f32x4 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[u] = xi[h + u];
          b[u] = xj[h + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[h + u] = a[u] * b[u];
      }
    } else if constexpr (Cfg::KH) {
      const f16x8* xi = reinterpret_cast<const f16x8*>(TK + (1 + pi) * Cfg::TPK);
      const f16x8* xj = reinterpret_cast<const f16x8*>(TK + (1 + pjj) * Cfg::TPK);
      f16x8* dst = reinterpret_cast<f16x8*>(TK + tab_pair<D>(pi, pjj) * Cfg::TPK);
      f16x8 a[C / 8], b[C / 8];
#pragma unroll
      for (int u = 0; u < C / 8; ++u) {
        a[u] = xi[u];
        b[u] = xj[u];
      }
#pragma unroll
      for (int u = 0; u < C / 8; ++u) dst[u] = a[u] * b[u];
    } else {
      const f32x4* xi = reinterpret_cast<const f32x4*>(TK + (1 + pi) * Cfg::TPK);
      const f32x4* xj = reinterpret_cast<const f32x4*>(TK + (1 + pjj) * Cfg::TPK);
      f32x4* dst = reinterpret_cast<f32x4*>(TK + tab_pair<D>(pi, pjj) * Cfg::TPK);
#pragma unroll
      for (int u = 0; u < C / 4; ++u) dst[u] = xi[u] * xj[u];
    }
  }
}

// Blocks of 64 features of the table-driven generators, per wave: entry j
// of wave w is block w + NW j, except that when the blocks beyond one per
// wave (R of them) divide the first half of the waves, each of them is split
// by tokens over NW / (2 R) of those waves (a 640-feature slice on eight
// waves: one block each, and half a block more on waves 0..3). Waves w and
// w + 4 share a SIMD and the older one, w < 4, gets issue priority: the same
// work takes longer on waves 4..7, so the first half takes the extra.
template <class Cfg>
struct TabSplit {
  static constexpr int NB = (Cfg::FS + 63) / 64, NW = Cfg::NW, R = NB - NW, HW = NW / 2;
  static constexpr bool BAL = R > 0 && R <= HW && HW % R == 0 && (Cfg::C / (HW / R)) % 8 == 0;
  static constexpr int P = BAL ? HW / R : 1;     // token pieces per left-over block
  static constexpr int NBW = (NB + NW - 1) / NW;  // entries per wave
  __device__ static int block(int w, int j) { return BAL ? (j == 0 ? w : (w < HW ? NW + w / P : NB)) : w + NW * j; }
  __device__ static int tok0(int w, int j) { return BAL && j > 0 ? (w % P) * (Cfg::C / P) : 0; }
  template <int J>
  static constexpr int ntok() { return BAL && J > 0 ? Cfg::C / P : Cfg::C; }
};

// Query side: phi~(Q) [C x FS], query-major. Key side: u(KS K)^T [FS x C].
template <class Cfg, bool QSIDE, class TE_, class DE>
__device__ __forceinline__ void gen_tab(int w, int lane, const TabFeat* tf, const TE_* __restrict__ T,
                                        DE* __restrict__ dst) {
  using TS = TabSplit<Cfg>;
  static_for<0, TS::NBW>([&](auto ji) {
    constexpr int j = decltype(ji)::value;
    constexpr int NTOK = TS::template ntok<j>();
    const int blk = TS::block(w, j);
    const int fl = 64 * blk + lane;
    if (blk >= TS::NB || fl >= Cfg::FS) return;
    const int tbase = TS::tok0(w, j);
    if constexpr (QSIDE) {
      const float* __restrict__ ta = T + tf[j].oa;
      const float* __restrict__ tb = T + tf[j].ob;
      const float* __restrict__ tc = T + tf[j].oc;
      const float cf = tf[j].cq;
#pragma unroll
      for (int tt = 0; tt < NTOK; tt += 4) {
        const int t0 = tbase + tt;
        const f32x4 va = *reinterpret_cast<const f32x4*>(ta + t0);
        f32x4 vb = *reinterpret_cast<const f32x4*>(tb + t0);
        if constexpr (Cfg::TRIPLE) vb *= *reinterpret_cast<const f32x4*>(tc + t0);
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[(t0 + u) * Cfg::PQ + fl] = Cfg::M::cvt(va[u] * vb[u] * cf);
      }
    } else if constexpr (Cfg::KH) {
      const TE_* ta = T + tf[j].ka;
      const TE_* tb = T + tf[j].kb;
      const TE_* tc = T + tf[j].kc;
      const _Float16 ck = static_cast<_Float16>(tf[j].ck);
#pragma unroll
      for (int tt = 0; tt < NTOK; tt += 8) {
        const int t0 = tbase + tt;
        f16x8 v = *reinterpret_cast<const f16x8*>(ta + t0) * *reinterpret_cast<const f16x8*>(tb + t0);
        if constexpr (Cfg::TRIPLE) v = v * (*reinterpret_cast<const f16x8*>(tc + t0) * ck);
        if constexpr (Cfg::QGEN) v = v * ck;
        *reinterpret_cast<f16x8*>(dst + fl * Cfg::PK + t0) = v;
      }
    } else {
      const TE_* ta = T + tf[j].ka;
      const TE_* tb = T + tf[j].kb;
      const TE_* tc = T + tf[j].kc;
      const float ck = tf[j].ck;
#pragma unroll
      for (int tt = 0; tt < NTOK; tt += 4) {
        const int t0 = tbase + tt;
        f32x4 v = *reinterpret_cast<const f32x4*>(ta + t0) * *reinterpret_cast<const f32x4*>(tb + t0);
        if constexpr (Cfg::TRIPLE) v = v * (*reinterpret_cast<const f32x4*>(tc + t0) * ck);
        *reinterpret_cast<f32x4*>(dst + fl * Cfg::PK + t0) = v;
      }
    }
  });
}

// Score tiles of one chunk handled by wave R (tiles R, R+NW, ...): all
// operand fragments are fetched first, then the MFMAs run, then the
// polynomial and the causal mask are applied in registers and the P^T tile
// (query-major, keys contiguous) is written to LDS. Tiles above the diagonal
// inside the last 32-key step are written as zeros.
template <class Cfg, int R>
__device__ __forceinline__ void score_tiles(const typename Cfg::E* sK, const typename Cfg::E* sQ,
                                            typename Cfg::E* sP, int c, int g4, float inv_a, bool decay,
                                            float log2g) {
  using M = typename Cfg::M;
  using frag = typename M::frag;
  using half = typename M::half;
  constexpr int NW = Cfg::NW, XP = Cfg::XP, D = Cfg::D;
  constexpr TileList<Cfg> tiles = make_tiles<Cfg>();
  constexpr int NTR = (Cfg::NTILES - R + NW - 1) / NW;
  constexpr int KU = D == 16 ? 1 : D / 32;
  using opnd = std::conditional_t<D == 16, half, frag>;
  opnd ak[NTR > 0 ? NTR : 1][KU], bq[NTR > 0 ? NTR : 1][KU];
  static_for<0, NTR>([&](auto ji) {
    constexpr int j = decltype(ji)::value;
    constexpr int kt = tiles.kt[R + j * NW], qt = tiles.qt[R + j * NW];
    if constexpr (kt <= qt) {
      static_for<0, KU>([&](auto ui) {
        constexpr int u = decltype(ui)::value;
        if constexpr (D == 16) {
          ak[j][u] = *reinterpret_cast<const half*>(sK + (16 * kt + c) * XP + 4 * g4);
          bq[j][u] = *reinterpret_cast<const half*>(sQ + (16 * qt + c) * XP + 4 * g4);
        } else {
          ak[j][u] = lds_frag8(sK + (16 * kt + c) * XP + 32 * u + 8 * g4);
          bq[j][u] = lds_frag8(sQ + (16 * qt + c) * XP + 32 * u + 8 * g4);
        }
      });
    }
  });
  f32x4 acc[NTR > 0 ? NTR : 1];
  static_for<0, NTR>([&](auto ji) {
    constexpr int j = decltype(ji)::value;
    constexpr int kt = tiles.kt[R + j * NW], qt = tiles.qt[R + j * NW];
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kt <= qt) {
      static_for<0, KU>([&](auto ui) {
        constexpr int u = decltype(ui)::value;
        if constexpr (D == 16)
          acc[j] = M::hstep(ak[j][u], bq[j][u], acc[j]);
        else
          acc[j] = M::step(ak[j][u], bq[j][u], acc[j]);
      });
    }
  });
  static_for<0, NTR>([&](auto ji) {
    constexpr int j = decltype(ji)::value;
    constexpr int kt = tiles.kt[R + j * NW], qt = tiles.qt[R + j * NW];
    typename Cfg::E* dst = sP + (16 * qt + c) * Cfg::PP + 16 * kt + 4 * g4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float wv = 0.f;
      if constexpr (kt <= qt) {
        wv = taylor_poly<Cfg::NT>(acc[j][i] * inv_a);
        const int lag = 16 * (qt - kt) + c - 4 * g4 - i;  // query - key
        if (kt == qt && lag < 0) wv = 0.f;                // causal mask (key > query)
        if (decay && lag > 0) wv *= exp2f(static_cast<float>(lag) * log2g);
      }
      dst[i] = M::cvt(wv);
    }
  });
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Raw buffer resource over `bytes` bytes at p (loads past the end return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}

enum { MODE_SEGSUM = 0, MODE_MAIN = 1 };

template <class Cfg, int MODE, bool EXT>
__global__ __launch_bounds__(Cfg::NTHR) void prefill_kernel(PrefillArgs a) {
  using M = typename Cfg::M;
  using E = typename Cfg::E;
  using frag = typename M::frag;
  constexpr int D = Cfg::D, DV = Cfg::DV, C = Cfg::C, NW = Cfg::NW, G = Cfg::G;
  constexpr int QT = Cfg::QT, KSC = Cfg::KSC, NDT = Cfg::NDT, FTG = Cfg::FTG, KSG = Cfg::KSG, KZ0 = Cfg::KZ0;
  constexpr bool MAIN = MODE == MODE_MAIN;

  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
  E* sQ = reinterpret_cast<E*>(smem + Cfg::OFF_Q);
  E* sK = reinterpret_cast<E*>(smem + Cfg::OFF_K);
  E* sV = reinterpret_cast<E*>(smem + Cfg::OFF_V);
  E* sPQ = reinterpret_cast<E*>(smem + Cfg::OFF_PQ);
  using KE = std::conditional_t<Cfg::KH, _Float16, E>;  // phi(K)^T and key-table element
  KE* sPK = reinterpret_cast<KE*>(smem + Cfg::OFF_PK);
  E* sP = reinterpret_cast<E*>(smem + Cfg::OFF_P);
  float* sDen = reinterpret_cast<float*>(smem + Cfg::OFF_DEN);
  f32x4* sRed = reinterpret_cast<f32x4*>(smem + Cfg::OFF_RED);

  const int tid = threadIdx.x;
  // wave index in a scalar register: branches on it around MFMAs must be
  // scalar branches (an MFMA ignores the exec mask)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // split z: dv pair dg (value tiles 2 dg, 2 dg + 1) of feature group fg
  const int dg = Cfg::ZS ? (w & 1) : 0;
  const int fg = Cfg::ZS ? (w >> 1) : 0;
  const int vt0 = Cfg::ZS ? NDT * dg : w;  // first value tile (16 columns of dv)
  const int ftg0 = fg * FTG;               // first feature tile of the group
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int c = lane & 15;

  // block -> (unit, slice); the G slices of a unit share an XCD (b % 8).
  const int PL = MAIN ? a.P : a.P - 1;  // segments handled by this launch
  const int nunits = a.BH * PL;
  const int b = blockIdx.x;
  const int gsl = (b >> 3) % G;
  const int unit = (b & 7) + 8 * ((b >> 3) / G);
  if (unit >= nunits) return;
  const int bh = unit / PL;
  const int p = unit - bh * PL;
  const int f0 = gsl * Cfg::FS;
  const int N = a.N;
  const bool want_out = MAIN && a.o != nullptr;
  const bool want_state = MAIN && a.S != nullptr && p == a.P - 1;
  if (MAIN && !want_out && !want_state) return;

  // Segment p holds tokens [t0, t1). With a prefix pass (two segments of
  // lengths L0 and N - L0) the main launch runs segment 1 from token 0,
  // updating the state without read-out up to t0: there are no segment sums.
  const bool prefix_pass = a.L0 > 0;
  const int t0 = prefix_pass ? (p == 0 ? 0 : a.L0) : p * a.L;
  const int t1 = prefix_pass ? (p == 0 ? a.L0 : N) : min(N, t0 + a.L);
  const int lo = (MAIN && prefix_pass) ? 0 : t0;  // first token of the chunk loop

  const E* qh = reinterpret_cast<const E*>(a.q) + static_cast<size_t>(bh) * N * D;
  const E* kh = reinterpret_cast<const E*>(a.k) + static_cast<size_t>(bh) * N * D;
  const E* vh = reinterpret_cast<const E*>(a.v) + static_cast<size_t>(bh) * N * DV;

  // constant part of V^T: padding rows below the ones row
  for (int i = tid; i < (Cfg::DVP - DV - 1) * Cfg::PK; i += Cfg::NTHR)
    sV[(DV + 1) * Cfg::PK + i] = M::cvt(0.f);

  // ---- initial state of this slice ------------------------------------------
  // S[j][ft]: value tile vt0 + j (without split z, on the last wave: the
  // ones column) of feature tile ftg0 + ft. Z (split z): the ones column of
  // the slice's feature tiles zlo .. zlo + nzt - 1.
  constexpr int ZT = Cfg::ZT, TPW = Cfg::TPW;
  const int zlo = Cfg::ZS ? 2 * (fg * KSG + (dg == 0 ? 0 : KZ0)) : 0;
  const int nzt = Cfg::ZS ? 2 * (dg == 0 ? KZ0 : KSG - KZ0) : 0;
  f32x4 S[NDT][FTG];
  f32x4 Z[ZT > 0 ? ZT : 1];
#pragma unroll
  for (int j = 0; j < NDT; ++j)
#pragma unroll
    for (int ft = 0; ft < FTG; ++ft) S[j][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < (ZT > 0 ? ZT : 1); ++j) Z[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (MAIN) {
    if (a.S0 != nullptr) {
#pragma unroll
      for (int j = 0; j < NDT; ++j)
#pragma unroll
        for (int ft = 0; ft < FTG; ++ft)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int f = canon_feat<Cfg>(f0 + 16 * (ftg0 + ft) + 4 * g4 + i);
            float val = 0.f;
            if (f >= 0) {
              if (Cfg::ZS || w < NW - 1)
                val = a.S0[(static_cast<size_t>(bh) * Cfg::F + f) * DV + 16 * (vt0 + j) + c];
              else if (c == 0)
                val = a.z0[static_cast<size_t>(bh) * Cfg::F + f];
              if constexpr (!Cfg::UNROLL) val /= state_scale<Cfg>(f);
            }
            S[j][ft][i] = val;
          }
      if constexpr (Cfg::ZS) {
#pragma unroll
        for (int jz = 0; jz < ZT; ++jz)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int f = canon_feat<Cfg>(f0 + 16 * (zlo + jz) + 4 * g4 + i);
            Z[jz][i] = (c == 0 && jz < nzt && f >= 0)
                           ? a.z0[static_cast<size_t>(bh) * Cfg::F + f] / state_scale<Cfg>(f)
                           : 0.f;
          }
      }
      if (EXT && lo > 0) {
        // S0 is the state just before token 0; the chunk loop starts at lo
        const float g0 = exp2f(static_cast<float>(lo) * a.log2g);
#pragma unroll
        for (int j = 0; j < NDT; ++j)
#pragma unroll
          for (int ft = 0; ft < FTG; ++ft) S[j][ft] *= g0;
#pragma unroll
        for (int jz = 0; jz < ZT; ++jz) Z[jz] *= g0;
      }
    }
    // sum of the earlier segments' states, PB segments' loads in flight at once
    const int PS = a.P - 1;
    constexpr int PB = TPW <= 10 ? 4 : (TPW <= 20 ? 2 : 1);
    for (int pp = 0; pp < (prefix_pass ? 0 : p); pp += PB) {
      f32x4 t[PB][TPW];
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        // segments past p - 1 re-read segment pp (in bounds) and are dropped
        const int ps = pp + j < p ? pp + j : pp;
        const f32x4* src = reinterpret_cast<const f32x4*>(a.seg) +
                           ((((static_cast<size_t>(bh) * PS + ps) * G + gsl) * NW + w) * TPW) * 64 + lane;
#pragma unroll
        for (int ft = 0; ft < TPW; ++ft) t[j][ft] = src[ft * 64];
      }
#pragma unroll
      for (int j = 0; j < PB; ++j)
        if (pp + j < p) {
          // segment q = pp + j ends L (p - 1 - q) tokens before this one starts
          const float gq = EXT ? exp2f(static_cast<float>(p - 1 - pp - j) * static_cast<float>(a.L) * a.log2g)
                                   : 1.f;
#pragma unroll
          for (int jj = 0; jj < NDT; ++jj)
#pragma unroll
            for (int ft = 0; ft < FTG; ++ft) S[jj][ft] += gq * t[j][jj * FTG + ft];
#pragma unroll
          for (int zj = 0; zj < ZT; ++zj) Z[zj] += gq * t[j][NDT * FTG + zj];
        }
    }
  }

  const float inv_a = a.inv_a;

  // table-driven generator: this lane's features (fixed for the kernel)
  constexpr int NBW = TabSplit<Cfg>::NBW;
  TabFeat tf[NBW];
  float* sTQ = reinterpret_cast<float*>(smem + Cfg::OFF_TQ);
  KE* sTK = reinterpret_cast<KE*>(smem + Cfg::OFF_TK);
  const PairJobs<Cfg> pj = pair_jobs<Cfg>(tid);
  if constexpr (Cfg::TAB) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) tf[j] = tab_feat<Cfg>(f0 + 64 * TabSplit<Cfg>::block(w, j) + lane, inv_a);
    // row 0 of both tables is the constant 1 (also for rows past the end of
    // the sequence: their values and ones-row entries are zero)
    for (int t = tid; t < Cfg::C; t += Cfg::NTHR) {
      if constexpr (!Cfg::QGEN) sTQ[t] = 1.f;
      sTK[t] = static_cast<KE>(1.f);
    }
  }

  // ---- chunk loop ------------------------------------------------------------
  // Global loads run one chunk ahead: the next chunk's Q, K and V rows are
  // fetched into registers (16 bytes per item) while the current chunk is in
  // compute, then written to LDS at the top of the next iteration.
  constexpr int EV = 16 / Cfg::ES;         // elements per 16-byte item
  constexpr int NQI = C * D / EV;          // items of Q (and of K)
  constexpr int NVI = C * DV / EV;         // items of V
  constexpr int QB = MAIN ? NQI : 0;       // Q items exist only when reading out
  constexpr int NIT = QB + NQI + NVI;
  constexpr int NSLOT = (NIT + Cfg::NTHR - 1) / Cfg::NTHR;
  static_assert(QB % 64 == 0 && NQI % 64 == 0 && NIT % 64 == 0, "staging items: whole waves per kind");
  uint4 pf[NSLOT];

  // Buffer resources over this segment's rows (base and size in scalar
  // registers): rows past the segment, and Q when no output is wanted, read
  // as zero without branches.
  // (queries from t0, keys and values from the first token of the loop)
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0), loop_rows = static_cast<uint32_t>(t1 - lo);
  const E* const qb = qh + static_cast<size_t>(t0) * D;
  const E* const kb = kh + static_cast<size_t>(lo) * D;
  const E* const vb = vh + static_cast<size_t>(lo) * DV;
  const uint32_t qbytes = want_out ? seg_rows * D * Cfg::ES : 0u, kbytes = loop_rows * D * Cfg::ES,
                 vbytes = loop_rows * DV * Cfg::ES;
  // V items (16 bytes each). V is written transposed, one element per
  // store: in wide slices consecutive lanes take consecutive rows (tokens)
  // of one 16-byte column group, so that the stores of a wave spread over
  // the banks (in the row-major order of a row's items, four different
  // dwords of a wave's store shared a bank at dv = 64; order 4 runs 1%
  // faster); the narrower instantiations keep the row-major order, which
  // coalesces their global loads better
  auto v_row = [](int j) { return Cfg::WIDE ? j % C : j / (DV / EV); };
  auto v_col = [](int j) { return Cfg::WIDE ? (j / C) * EV : (j % (DV / EV)) * EV; };
  auto fetch = [&](int cc0) {
    const uint32_t r0 = static_cast<uint32_t>(cc0 - lo);
    const bool qrows = cc0 >= t0;  // prefix-pass chunks read no queries
    constexpr uint32_t kNone = 0x7ffffff0u;  // past every buffer range: loads zeros
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
      const int i = tid + s * Cfg::NTHR;
      // Every thread issues exactly one load per slot, straight into pf[s];
      // items it does not have read zeros from past the range. (With
      // conditional loads the compiler merged the loaded value into pf under
      // an exec mask and waited for the load at once, stalling each loading
      // wave for the load's latency.) The item kind is the same on all lanes
      // of a wave (its boundaries are multiples of 64), so the buffer base
      // and size are chosen in scalar registers.
      const int kind = __builtin_amdgcn_readfirstlane(i < QB ? 0 : (i < QB + NQI ? 1 : (i < NIT ? 2 : 3)));
      const E* bp = kb;
      uint32_t nb = 0u, off = kNone;
      if (kind == 0) {
        const int row = i / (D / EV), col = (i % (D / EV)) * EV;
        bp = qb;
        nb = qrows ? qbytes : 0u;
        off = ((static_cast<uint32_t>(cc0 - t0) + row) * D + col) * Cfg::ES;
      } else if (kind == 1) {
        const int j = i - QB;
        const int row = j / (D / EV), col = (j % (D / EV)) * EV;
        nb = kbytes;
        off = ((r0 + row) * D + col) * Cfg::ES;
      } else if (kind == 2) {
        const int j = i - QB - NQI;
        const int row = v_row(j), col = v_col(j);
        bp = vb;
        nb = vbytes;
        off = ((r0 + row) * DV + col) * Cfg::ES;
      }
      pf[s] = bload16(make_rsrc(bp, nb), off);
    }
  };



  // Q, K row-major (and, for the table-driven generator, transposed into the
  // coordinate rows of the factor tables); V transposed (key-contiguous) with
  // the ones row below it. Extended kernels first preprocess the Q and K
  // rows: the D / EV consecutive lanes that hold one row sum its squares
  // with lane exchanges, then scale their items.
  const float qhead = (EXT && a.q_head_scale != nullptr) ? a.q_head_scale[bh % a.H] : 1.f;
  auto stage = [&](int nvv, bool ro) {
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
      const int i = tid + s * Cfg::NTHR;
      uint4 val = pf[s];
      if constexpr (EXT) {
        E* e = reinterpret_cast<E*>(&val);
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < EV; ++u) ss += static_cast<float>(e[u]) * static_cast<float>(e[u]);
#pragma unroll
        for (int m = 1; m < D / EV; m <<= 1) ss += __shfl_xor(ss, m);
        float f = i < QB ? a.q_scale * qhead : a.k_scale;
        if (a.qk_norm) f = ss > 0.f ? f / __builtin_sqrtf(ss) : 0.f;
        if (i < QB + NQI && f != 1.f) {
#pragma unroll
          for (int u = 0; u < EV; ++u) e[u] = M::cvt(static_cast<float>(e[u]) * f);
        }
      }
      if (i < QB) {
        const int row = i / (D / EV), col = (i % (D / EV)) * EV;
        if (ro) {
          *reinterpret_cast<uint4*>(sQ + row * Cfg::XP + col) = val;
          if constexpr (Cfg::TAB && !Cfg::QGEN) {
            const E* e = reinterpret_cast<const E*>(&val);
#pragma unroll
            for (int u = 0; u < EV; ++u) sTQ[(1 + col + u) * Cfg::TP + row] = static_cast<float>(e[u]);
          }
        }
      } else if (i < QB + NQI) {
        const int j = i - QB;
        const int row = j / (D / EV), col = (j % (D / EV)) * EV;
        *reinterpret_cast<uint4*>(sK + row * Cfg::XP + col) = val;
        if constexpr (Cfg::TAB) {
          const E* e = reinterpret_cast<const E*>(&val);
#pragma unroll
          for (int u = 0; u < EV; ++u) sTK[(1 + col + u) * Cfg::TPK + row] = static_cast<KE>(static_cast<float>(e[u]) * Cfg::KS);
        }
      } else if (i < NIT) {
        const int j = i - QB - NQI;
        const int row = v_row(j), col = v_col(j);
        const E* e = reinterpret_cast<const E*>(&pf[s]);
#pragma unroll
        for (int u = 0; u < EV; ++u) sV[(col + u) * Cfg::PK + row] = e[u];
      }
    }
    for (int i = tid; i < C; i += Cfg::NTHR) sV[DV * Cfg::PK + i] = M::cvt(i < nvv ? 1.f : 0.f);
    if constexpr (Cfg::ZS && Cfg::TAB) {
      // row 0 of the factor tables, again for every chunk: their space holds
      // the read-out partials from the feature generation to the chunk's end
      for (int t = tid; t < C; t += Cfg::NTHR) {
        if constexpr (!Cfg::QGEN) sTQ[t] = 1.f;
        sTK[t] = static_cast<KE>(1.f);
      }
    }
  };

  if (lo < t1) fetch(lo);
  for (int c0 = lo; c0 < t1; c0 += C) {
    const int nv = min(C, t1 - c0);
    const bool last_chunk = c0 + C >= t1;
    const bool do_update = !MAIN || !last_chunk || want_state;
    const bool ro = want_out && c0 >= t0;  // read-out wanted for this chunk

    stage(nv, ro);
    __syncthreads();
    // the next chunk's loads stay in flight through this chunk's work (a
    // barrier waits for LDS operations only; the next staging waits for them)
    if (!last_chunk) fetch(c0 + C);

    // features and score tiles
    if constexpr (Cfg::UNROLL) {
      if (lane < C) {
        float x[D];
        if (ro) {
#pragma unroll
          for (int j = 0; j < D; ++j) x[j] = static_cast<float>(sQ[lane * Cfg::XP + j]) * inv_a;
          gen_unrolled<Cfg, true>(w, x, sPQ + lane * Cfg::PQ);
        }
        if (do_update) {
#pragma unroll
          for (int j = 0; j < D; ++j) x[j] = static_cast<float>(sK[lane * Cfg::XP + j]);
          gen_unrolled<Cfg, false>(w, x, sPK + lane);
        }
      }
    } else {
      // (per-token query features: before the pair rows' barrier, which they
      // do not need)
      if constexpr (Cfg::PAIRS) build_pairs<Cfg>(tid, pj, sTQ, sTK, ro && !Cfg::QGEN);
      if constexpr (Cfg::QGEN) {
        if (ro) gen_q_token<Cfg>(gsl, w, lane, sQ, sPQ, inv_a);
      }
      if constexpr (Cfg::PAIRS) __syncthreads();
      if constexpr (!Cfg::QGEN) {
        if (ro) gen_tab<Cfg, true>(w, lane, tf, sTQ, sPQ);
      }
      if (do_update) gen_tab<Cfg, false>(w, lane, tf, sTK, sPK);
    }
    if (ro && gsl == 0) {
      static_for<0, NW>([&](auto ri) {
        if (w == decltype(ri)::value)
          score_tiles<Cfg, decltype(ri)::value>(sK, sQ, sP, c, g4, inv_a, EXT, a.log2g);
      });
    }
    __syncthreads();

    // [V,1]^T fragments of the wave's value tiles (A operand of the
    // intra-chunk term, B operand of the state update)
    frag bv[NDT][KSC];
#pragma unroll
    for (int j = 0; j < NDT; ++j)
#pragma unroll
      for (int u = 0; u < KSC; ++u) bv[j][u] = lds_frag8(sV + (16 * (vt0 + j) + c) * Cfg::PK + 32 * u + 8 * g4);
    // split z: the ones row of [V,1]^T (and zero rows below it), the B
    // operand of the z update and the A operand of the intra-chunk
    // denominator
    frag bo[KSC];
    if constexpr (Cfg::ZS) {
#pragma unroll
      for (int u = 0; u < KSC; ++u) bo[u] = lds_frag8(sV + (DV + c) * Cfg::PK + 32 * u + 8 * g4);
    }

    if (ro) {
      // read-out of the state over the wave's feature group: O^T[value tile]
      // = S^T phi~(Q)^T. Each phi~(Q) fragment feeds the wave's NDT value
      // tiles and, on the wave's z k-steps, the z tile (row 0 of accZ is
      // the denominator); the fragments of k-step t+1 are fetched before
      // the MFMAs of k-step t.
      f32x4 acc[NDT][QT], accZ[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int j = 0; j < NDT; ++j) acc[j][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accZ[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const E* pq = sPQ + 32 * fg * KSG + 4 * g4;
      frag bq[2][QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) bq[0][qt] = lds_frag_split(pq + (16 * qt + c) * Cfg::PQ);
#pragma unroll
      for (int t = 0; t < KSG; ++t) {
        if (t + 1 < KSG) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            bq[(t + 1) & 1][qt] = lds_frag_split(pq + (16 * qt + c) * Cfg::PQ + 32 * (t + 1));
        }
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
          frag sa;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sa[i] = M::cvt(S[j][2 * t][i]);
            sa[i + 4] = M::cvt(S[j][2 * t + 1][i]);
          }
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) acc[j][qt] = M::step(sa, bq[t & 1][qt], acc[j][qt]);
        }
        if constexpr (Cfg::ZS) {
          // k-step t of the group: z of dv pair 0 if t < KZ0, else of pair 1
          if ((t < KZ0) == (dg == 0)) {
            const int jz = 2 * (t < KZ0 ? t : t - KZ0);
            frag za;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              za[i] = M::cvt(Z[jz][i]);
              za[i + 4] = M::cvt(Z[jz + 1][i]);
            }
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) accZ[qt] = M::step(za, bq[t & 1][qt], accZ[qt]);
          }
        }
      }
      if constexpr (EXT) {
        // the state read out by query i of the chunk is i + 1 steps old
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float gq = exp2f(static_cast<float>(16 * qt + c + 1) * a.log2g);
#pragma unroll
          for (int j = 0; j < NDT; ++j) acc[j][qt] *= gq;
          accZ[qt] *= gq;
        }
      }
      // intra-chunk term: O^T += [V,1]^T P^T (first slice, first feature
      // group); all P^T fragments are fetched before the MFMAs.
      if (gsl == 0 && fg == 0) {
        constexpr int NPF = [] {
          int n = 0;
          for (int qt = 0; qt < QT; ++qt) n += qt / 2 + 1;
          return n;
        }();
        frag bp[NPF];
        static_for<0, QT>([&](auto qi) {
          constexpr int qt = decltype(qi)::value;
          constexpr int base = [] { int n = 0; for (int q2 = 0; q2 < qt; ++q2) n += q2 / 2 + 1; return n; }();
          static_for<0, qt / 2 + 1>([&](auto ui) {
            constexpr int u = decltype(ui)::value;
            bp[base + u] = lds_frag8(sP + (16 * qt + c) * Cfg::PP + 32 * u + 8 * g4);
          });
        });
        static_for<0, QT>([&](auto qi) {
          constexpr int qt = decltype(qi)::value;
          constexpr int base = [] { int n = 0; for (int q2 = 0; q2 < qt; ++q2) n += q2 / 2 + 1; return n; }();
          static_for<0, qt / 2 + 1>([&](auto ui) {
            constexpr int u = decltype(ui)::value;
#pragma unroll
            for (int j = 0; j < NDT; ++j) acc[j][qt] = M::step(bv[j][u], bp[base + u], acc[j][qt]);
            // split z: wave 0 adds the intra-chunk denominator (ones row)
            if (Cfg::ZS && w == 0) accZ[qt] = M::step(bo[u], bp[base + u], accZ[qt]);
          });
        });
      }
      if constexpr (Cfg::ZS) {
        if constexpr (Cfg::WIDE) {
          // every feature group hands its value partials, every wave its
          // share of the denominator, to LDS; then each thread sums one output
          // item of the chunk (query tile iqt, value tile ivt, accumulator lane
          // il: four values of one query), so that the sums, the normalisation
          // and the stores are spread over all waves
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int j = 0; j < NDT; ++j) sRed[((fg * QT + qt) * (DV / 16) + vt0 + j) * 64 + lane] = acc[j][qt];
          if (g4 == 0) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) sDen[w * C + 16 * qt + c] = accZ[qt][0];
          }
          __syncthreads();
          const int il = tid & 63, ivt = (tid >> 6) % (DV / 16), iqt = tid / (64 * (DV / 16));
          f32x4 o = sRed[(iqt * (DV / 16) + ivt) * 64 + il];
#pragma unroll
          for (int g = 1; g < Cfg::NFG; ++g) o += sRed[((g * QT + iqt) * (DV / 16) + ivt) * 64 + il];
          const int qi = 16 * iqt + (il & 15), col = 16 * ivt + 4 * (il >> 4);
          float dsum = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) dsum += sDen[ww * C + qi];
          if (qi < nv) {
            if constexpr (G == 1) {
              const float r = 1.f / dsum;
              const size_t off = (static_cast<size_t>(bh) * N + c0 + qi) * DV + col;
              if (a.out_bf16) {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(o[i] * r);
                *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + off) = ov;
              } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + off) = o * r;
              }
            } else {
              // partial row: the values, and the denominator in column DV
              float* pr = a.part + ((static_cast<size_t>(gsl) * a.BH + bh) * N + c0 + qi) * Cfg::PPITCH;
              *reinterpret_cast<f32x4*>(pr + col) = o;
              if (col == 0) pr[DV] = dsum;
            }
          }
        } else {
          // feature groups 1 .. NFG-1 hand their value partials to group 0,
          // every wave its share of the denominator
          if (fg > 0) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
              for (int j = 0; j < NDT; ++j)
                sRed[(((fg - 1) * QT + qt) * (DV / 16) + vt0 + j) * 64 + lane] = acc[j][qt];
          }
          if (g4 == 0) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) sDen[w * C + 16 * qt + c] = accZ[qt][0];
          }
          __syncthreads();
          if (fg == 0) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
              for (int g = 0; g < Cfg::NFG - 1; ++g)
#pragma unroll
                for (int j = 0; j < NDT; ++j) acc[j][qt] += sRed[((g * QT + qt) * (DV / 16) + vt0 + j) * 64 + lane];
              float dsum = 0.f;
#pragma unroll
              for (int ww = 0; ww < NW; ++ww) dsum += sDen[ww * C + 16 * qt + c];
              accZ[qt][0] = dsum;
            }
          }        }

      } else if constexpr (G == 1) {
        // denominator: row DV of O^T (wave NW-1, lane group 0, element 0)
        if (w == NW - 1 && g4 == 0) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) sDen[16 * qt + c] = acc[0][qt][0];
        }
        __syncthreads();
        if (w < NW - 1) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) accZ[qt][0] = sDen[16 * qt + c];
        }
      }
      if (Cfg::ZS ? (!Cfg::WIDE && fg == 0) : (w < NW - 1 || G > 1)) {
        if constexpr (G == 1) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const int qi = 16 * qt + c;
            if (qi < nv) {
              const float r = 1.f / accZ[qt][0];
#pragma unroll
              for (int j = 0; j < NDT; ++j) {
                const size_t off = (static_cast<size_t>(bh) * N + c0 + qi) * DV + 16 * (vt0 + j) + 4 * g4;
                if (a.out_bf16) {
                  bf16x4 ov;
#pragma unroll
                  for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(acc[j][qt][i] * r);
                  *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + off) = ov;
                } else {
                  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + off) = acc[j][qt] * r;
                }
              }
            }
          }
        } else {
          // partial rows: the value tiles, and the denominator in column DV
          float* pp = a.part + ((static_cast<size_t>(gsl) * a.BH + bh) * N + c0) * Cfg::PPITCH;
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const int qi = 16 * qt + c;
            if (qi < nv) {
              if (Cfg::ZS || w < NW - 1) {
#pragma unroll
                for (int j = 0; j < NDT; ++j)
                  *reinterpret_cast<f32x4*>(pp + qi * Cfg::PPITCH + 16 * (vt0 + j) + 4 * g4) = acc[j][qt];
              }
              if (Cfg::ZS ? (w == 0 && g4 == 0) : (w == NW - 1 && g4 == 0))
                pp[qi * Cfg::PPITCH + DV] = Cfg::ZS ? accZ[qt][0] : acc[0][qt][0];
            }
          }
        }
      }
    }

    if (do_update) {
      // S[value tile, feature tile] += phi(K)^T [V,1]: each phi(K)^T fragment
      // feeds the wave's NDT value tiles and, on the wave's z tiles, the z
      // tile; the fragments of feature tile ft+1 are fetched before the
      // MFMAs of ft. With a decay: S = g^nv S + sum_j g^(nv-1-j) phi(k_j) [v_j, 1].
      frag bu[NDT][KSC], buo[KSC];
#pragma unroll
      for (int u = 0; u < KSC; ++u) {
#pragma unroll
        for (int j = 0; j < NDT; ++j) bu[j][u] = bv[j][u];
        if constexpr (Cfg::ZS) buo[u] = bo[u];
      }
      if constexpr (EXT) {
        const float gs = exp2f(static_cast<float>(nv) * a.log2g);
#pragma unroll
        for (int j = 0; j < NDT; ++j)
#pragma unroll
          for (int ft = 0; ft < FTG; ++ft) S[j][ft] *= gs;
#pragma unroll
        for (int jz = 0; jz < ZT; ++jz) Z[jz] *= gs;
#pragma unroll
        for (int u = 0; u < KSC; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int key = 32 * u + 8 * g4 + i;
            const float f = key < nv ? exp2f(static_cast<float>(nv - 1 - key) * a.log2g) : 0.f;
#pragma unroll
            for (int j = 0; j < NDT; ++j) bu[j][u][i] = M::cvt(static_cast<float>(bv[j][u][i]) * f);
            if constexpr (Cfg::ZS) buo[u][i] = M::cvt(static_cast<float>(bo[u][i]) * f);
          }
      }
      // k-steps of the z update: feature tile ft of the group is a z tile of
      // dv pair 0 if ft < 2 KZ0, else of pair 1
      auto zmine = [&](int ft) { return (ft < 2 * KZ0) == (dg == 0); };
      auto zidx = [&](int ft) { return ft < 2 * KZ0 ? ft : ft - 2 * KZ0; };
      if constexpr (Cfg::KH) {
        // fp16 contraction: u(KS K)^T from the key table, [V,1] converted
        f16x8 bvh[NDT][KSC], boh[KSC], ak[2][KSC];
#pragma unroll
        for (int u = 0; u < KSC; ++u) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < NDT; ++j) bvh[j][u][i] = static_cast<_Float16>(static_cast<float>(bu[j][u][i]));
            if constexpr (Cfg::ZS) boh[u][i] = static_cast<_Float16>(static_cast<float>(buo[u][i]));
          }
        }
        const KE* pk = sPK + (16 * ftg0 + c) * Cfg::PK + 8 * g4;
#pragma unroll
        for (int u = 0; u < KSC; ++u) ak[0][u] = *reinterpret_cast<const f16x8*>(pk + 32 * u);
#pragma unroll
        for (int ft = 0; ft < FTG; ++ft) {
          if (ft + 1 < FTG) {
#pragma unroll
            for (int u = 0; u < KSC; ++u)
              ak[(ft + 1) & 1][u] = *reinterpret_cast<const f16x8*>(pk + 16 * (ft + 1) * Cfg::PK + 32 * u);
          }
#pragma unroll
          for (int j = 0; j < NDT; ++j)
#pragma unroll
            for (int u = 0; u < KSC; ++u)
              S[j][ft] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[ft & 1][u], bvh[j][u], S[j][ft], 0, 0, 0);
          if constexpr (Cfg::ZS) {
            if (zmine(ft)) {
#pragma unroll
              for (int u = 0; u < KSC; ++u)
                Z[zidx(ft)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[ft & 1][u], boh[u], Z[zidx(ft)], 0, 0, 0);
            }
          }
        }
      } else {
        frag ak[2][KSC];
        const KE* pk = sPK + (16 * ftg0 + c) * Cfg::PK + 8 * g4;
#pragma unroll
        for (int u = 0; u < KSC; ++u) ak[0][u] = lds_frag8(pk + 32 * u);
#pragma unroll
        for (int ft = 0; ft < FTG; ++ft) {
          if (ft + 1 < FTG) {
#pragma unroll
            for (int u = 0; u < KSC; ++u) ak[(ft + 1) & 1][u] = lds_frag8(pk + 16 * (ft + 1) * Cfg::PK + 32 * u);
          }
#pragma unroll
          for (int j = 0; j < NDT; ++j)
#pragma unroll
            for (int u = 0; u < KSC; ++u) S[j][ft] = M::step(ak[ft & 1][u], bu[j][u], S[j][ft]);
          if constexpr (Cfg::ZS) {
            if (zmine(ft)) {
#pragma unroll
              for (int u = 0; u < KSC; ++u) Z[zidx(ft)] = M::step(ak[ft & 1][u], buo[u], Z[zidx(ft)]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- results ---------------------------------------------------------------
  // staged states (segment sums, deferred final state): per (unit, slice)
  // and wave, TPW tiles of 64 lanes: the NDT x FTG value tiles, then the ZT
  // z tiles
  auto store_tiles = [&](f32x4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDT; ++j)
#pragma unroll
      for (int ft = 0; ft < FTG; ++ft) dst[(j * FTG + ft) * 64] = S[j][ft];
#pragma unroll
    for (int jz = 0; jz < ZT; ++jz) dst[(NDT * FTG + jz) * 64] = Z[jz];
  };
  if constexpr (MAIN) {
    if (want_state && a.defer_state) {
      store_tiles(reinterpret_cast<f32x4*>(a.fin) + (((static_cast<size_t>(bh) * G + gsl) * NW + w) * TPW) * 64 + lane);
    } else if (want_state) {
#pragma unroll
      for (int j = 0; j < NDT; ++j)
#pragma unroll
        for (int ft = 0; ft < FTG; ++ft)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int f = canon_feat<Cfg>(f0 + 16 * (ftg0 + ft) + 4 * g4 + i);
            if (f >= 0) {
              const float sc = state_scale<Cfg>(f);
              if (Cfg::ZS || w < NW - 1)
                a.S[(static_cast<size_t>(bh) * Cfg::F + f) * DV + 16 * (vt0 + j) + c] = sc * S[j][ft][i];
              else if (c == 0)
                a.z[static_cast<size_t>(bh) * Cfg::F + f] = sc * S[j][ft][i];
            }
          }
      if constexpr (Cfg::ZS) {
#pragma unroll
        for (int jz = 0; jz < ZT; ++jz)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int f = canon_feat<Cfg>(f0 + 16 * (zlo + jz) + 4 * g4 + i);
            if (c == 0 && jz < nzt && f >= 0)
              a.z[static_cast<size_t>(bh) * Cfg::F + f] = state_scale<Cfg>(f) * Z[jz][i];
          }
      }
    }
  } else {
    const int PS = a.P - 1;
    store_tiles(reinterpret_cast<f32x4*>(a.seg) +
                ((((static_cast<size_t>(bh) * PS + p) * G + gsl) * NW + w) * TPW) * 64 + lane);
  }
}

// Sum the per-slice partial (numerator, denominator) rows and divide.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int G,
                                                      int64_t rows, int dv, int pitch, int nden, void* o,
                                                      int out_bf16) {
  const int nq = dv / 4;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= rows * nq) return;
  const int64_t r = e / nq;
  const int dq = static_cast<int>(e - r * nq);
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int g = 0; g < G; ++g) {
    const float* src = part + (static_cast<int64_t>(g) * rows + r) * pitch;
    num += *reinterpret_cast<const f32x4*>(src + 4 * dq);
    for (int j = 0; j < nden; ++j) den += src[dv + j];  // denominator shares of the waves
  }
  const float rcp = 1.f / den;
  const int64_t off = r * dv + 4 * dq;
  if (out_bf16) {
    bf16x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(num[i] * rcp);
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(o) + off) = ov;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + off) = num * rcp;
  }
}

// S = S0 (or zero), z = z0 (or zero): the state after zero tokens.
__global__ __launch_bounds__(256) void state_init_kernel(const float* S0, const float* z0, float* S,
                                                         float* z, int64_t nS, int64_t nz) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < nS) S[i] = S0 ? S0[i] : 0.f;
  if (i < nz) z[i] = z0 ? z0[i] : 0.f;
}

// Scatter the staged final state (accumulator layout) into S [F, dv] and z [F].
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHR) void state_store_kernel(const float* fin, float* S, float* z,
                                                                int BH) {
  constexpr int NW = Cfg::NW, NDT = Cfg::NDT, FTG = Cfg::FTG, KSG = Cfg::KSG, KZ0 = Cfg::KZ0, G = Cfg::G;
  constexpr int DV = Cfg::DV, TPW = Cfg::TPW;
  const int bh = blockIdx.x / G, gsl = blockIdx.x % G;
  if (bh >= BH) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g4 = lane >> 4, c = lane & 15;
  const int dg = Cfg::ZS ? (w & 1) : 0, fg = Cfg::ZS ? (w >> 1) : 0;
  const int vt0 = Cfg::ZS ? NDT * dg : w, ftg0 = fg * FTG;
  const f32x4* src = reinterpret_cast<const f32x4*>(fin) +
                     (((static_cast<size_t>(bh) * G + gsl) * NW + w) * TPW) * 64 + lane;
  for (int j = 0; j < NDT; ++j)
    for (int ft = 0; ft < FTG; ++ft) {
      const f32x4 val = src[(j * FTG + ft) * 64];
      for (int i = 0; i < 4; ++i) {
        const int f = canon_feat<Cfg>(gsl * Cfg::FS + 16 * (ftg0 + ft) + 4 * g4 + i);
        if (f >= 0) {
          const float sc = state_scale<Cfg>(f);
          if (Cfg::ZS || w < NW - 1)
            S[(static_cast<size_t>(bh) * Cfg::F + f) * DV + 16 * (vt0 + j) + c] = sc * val[i];
          else if (c == 0)
            z[static_cast<size_t>(bh) * Cfg::F + f] = sc * val[i];
        }
      }
    }
  if constexpr (Cfg::ZS) {
    // split z: the wave's z tiles (column 0 of each)
    const int zlo = 2 * (fg * KSG + (dg == 0 ? 0 : KZ0)), nzt = 2 * (dg == 0 ? KZ0 : KSG - KZ0);
    for (int jz = 0; jz < nzt; ++jz) {
      const f32x4 val = src[(NDT * FTG + jz) * 64];
      for (int i = 0; i < 4; ++i) {
        const int f = canon_feat<Cfg>(gsl * Cfg::FS + 16 * (zlo + jz) + 4 * g4 + i);
        if (c == 0 && f >= 0) z[static_cast<size_t>(bh) * Cfg::F + f] = state_scale<Cfg>(f) * val[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <class Cfg>
static hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream) {
  constexpr int G = Cfg::G;
  auto blocks_for = [](int units) { return 8 * G * ((units + 7) / 8); };
  if (a.P > 1 && a.L0 == 0) {
    const int units = a.BH * (a.P - 1);
    if (a.decay)
      hipLaunchKernelGGL((prefill_kernel<Cfg, MODE_SEGSUM, true>), dim3(blocks_for(units)), dim3(Cfg::NTHR), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<Cfg, MODE_SEGSUM, false>), dim3(blocks_for(units)), dim3(Cfg::NTHR), 0,
                         stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.decay)
    hipLaunchKernelGGL((prefill_kernel<Cfg, MODE_MAIN, true>), dim3(blocks_for(a.BH * a.P)), dim3(Cfg::NTHR), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<Cfg, MODE_MAIN, false>), dim3(blocks_for(a.BH * a.P)), dim3(Cfg::NTHR), 0,
                       stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.defer_state) {
    hipLaunchKernelGGL((state_store_kernel<Cfg>), dim3(a.BH * G), dim3(Cfg::NTHR), 0, stream, a.fin, a.S,
                       a.z, a.BH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (G > 1 && a.o != nullptr) {
    const int64_t rows = static_cast<int64_t>(a.BH) * a.N;
    const int64_t n = rows * (Cfg::DV / 4);
    hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                       a.part, G, rows, Cfg::DV, Cfg::PPITCH, Cfg::NDEN, a.o, a.out_bf16);
    e = hipGetLastError();
  }
  return e;
}

// Instantiation table: (d, dv, n_terms, bf16) -> slice width, chunk, generator.
#define TL_PREFILL_CFGS(X)                  \
  X(16, 16, 1, true, 32, 64, true)          \
  X(16, 16, 1, false, 32, 64, true)         \
  X(16, 64, 1, true, 32, 64, true)          \
  X(16, 64, 1, false, 32, 64, true)         \
  X(16, 16, 3, true, 160, 64, true)         \
  X(16, 16, 3, false, 160, 64, true)        \
  X(16, 64, 3, true, 160, 64, true)         \
  X(16, 64, 3, false, 160, 64, true)        \
  X(16, 16, 5, true, 608, 32, false)        \
  X(16, 16, 5, false, 256, 32, false)       \
  X(16, 64, 5, true, 640, 32, false)        \
  X(16, 64, 5, false, 256, 32, false)       \
  X(16, 64, 7, true, 640, 32, false)        \
  X(16, 64, 7, false, 256, 32, false)       \
  X(32, 16, 1, true, 32, 64, true)          \
  X(32, 16, 1, false, 32, 64, true)         \
  X(32, 64, 1, true, 32, 64, true)          \
  X(32, 64, 1, false, 32, 64, true)         \
  X(32, 16, 3, true, 576, 32, false)        \
  X(32, 16, 3, false, 128, 32, false)       \
  X(32, 64, 3, true, 640, 32, false)        \
  X(32, 64, 3, false, 128, 32, false)       \
  X(64, 16, 1, true, 32, 64, true)          \
  X(64, 16, 1, false, 32, 64, true)         \
  X(64, 64, 1, true, 32, 64, true)          \
  X(64, 64, 1, false, 32, 64, true)         \
  X(64, 16, 3, true, 544, 32, false)        \
  X(64, 16, 3, false, 128, 32, false)       \
  X(64, 64, 3, false, 128, 32, false)       \
  X(64, 64, 3, true, 256, 32, false)

// Sequence split for the generic kernels: enough workgroups (heads x
// segments x slices) to give each compute unit about two, and at least 4
// chunks per segment.
template <class Cfg>
static void plan_cfg(int BH, int N, PrefillPlan* p) {
  constexpr int C = Cfg::C;
  const int64_t nchunks = (static_cast<int64_t>(N) + C - 1) / C;
  *p = PrefillPlan{};
  if (BH <= 0 || nchunks == 0) {
    p->P = 1;
    p->L = N;
    return;
  }
  // Eight-wave workgroups (split z) run one per compute unit, the others
  // two. An update-only chunk of the prefix pass costs about 0.6 of a
  // read-out chunk (measured for order 4), one of the segment-sum launch
  // about 0.45, and reading one earlier segment's staged sum about 0.4.
  const int64_t slots = Cfg::ZS ? 256 : 512;
  const int64_t maxp = nchunks / 4 > 1 ? nchunks / 4 : 1;
  const int64_t minp = min_segments(nchunks, C, static_cast<int64_t>(Cfg::D > Cfg::DV ? Cfg::D : Cfg::DV) * Cfg::ES);
  const SegChoice sc = choose_segments(static_cast<int64_t>(BH) * Cfg::G, nchunks, slots, minp, maxp, 0.6, 0.45, 0.4);
  if (sc.prefix) {
    // segment 0 takes the larger share, L0 ~ N / (2 - 0.6), so that both
    // workgroups of a (head, slice) finish together
    int64_t c0 = static_cast<int64_t>(static_cast<double>(nchunks) / (2.0 - 0.6) + 0.5);
    if (c0 > nchunks - 1) c0 = nchunks - 1;
    if (c0 < 1) c0 = 1;
    p->P = 2;
    p->L0 = static_cast<int>(c0 * C);
    p->L = p->L0;
  } else {
    const int64_t cps = (nchunks + sc.P - 1) / sc.P;
    p->L = static_cast<int>(cps * C);
    p->P = static_cast<int>((nchunks + cps - 1) / cps);
  }
  // staged states: G slices x SLICE_F4 float4s per (head, segment)
  const size_t UB = static_cast<size_t>(Cfg::G) * Cfg::SLICE_F4 * 16;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  p->seg_off = off;
  if (p->P > 1 && p->L0 == 0) off += al(static_cast<size_t>(BH) * (p->P - 1) * UB);
  p->fin_off = off;
  if (p->P > 1) off += al(static_cast<size_t>(BH) * UB);
  p->part_off = off;
  if (Cfg::G > 1) off += al(static_cast<size_t>(Cfg::G) * BH * static_cast<size_t>(N) * Cfg::PPITCH * 4);
  p->bytes = off;
}

static bool is_w2(int d, int dv, int n_terms, bool bf16) { return d == 64 && dv == 64 && n_terms == 3 && bf16; }

static bool is_o2(int d, int dv, int n_terms, bool bf16) {
  return d == 16 && dv == 64 && n_terms == 3 && bf16;
}

bool prefill_plan(int d, int dv, int n_terms, bool bf16, bool decay, int BH, int N, PrefillPlan* plan) {
  if (!decay && is_o2(d, dv, n_terms, bf16)) return o2::plan(BH, N, plan);
  if (!decay && is_w2(d, dv, n_terms, bf16)) return w2::plan(BH, N, plan);
#define X(D_, DV_, NT_, BF_, FS_, C_, UN_)                                 \
  if (d == D_ && dv == DV_ && n_terms == NT_ && bf16 == BF_) {             \
    plan_cfg<PCfg<D_, DV_, NT_, BF_, FS_, C_, UN_>>(BH, N, plan);          \
    return true;                                                           \
  }
  TL_PREFILL_CFGS(X)
#undef X
  return false;
}

hipError_t prefill_launch(int d, int dv, int n_terms, bool bf16, const PrefillArgs& a,
                          hipStream_t stream) {
  if (!a.decay && is_o2(d, dv, n_terms, bf16)) return o2::launch(a, stream);
  if (!a.decay && is_w2(d, dv, n_terms, bf16)) return w2::launch(a, stream);
#define X(D_, DV_, NT_, BF_, FS_, C_, UN_)                                 \
  if (d == D_ && dv == DV_ && n_terms == NT_ && bf16 == BF_)               \
    return launch_cfg<PCfg<D_, DV_, NT_, BF_, FS_, C_, UN_>>(a, stream);
  TL_PREFILL_CFGS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t state_init_launch(const float* S0, const float* z0, float* S, float* z, int64_t BH,
                             int F, int dv, hipStream_t stream) {
  const int64_t nS = BH * F * dv, nz = BH * F;
  if (nS == 0) return hipSuccess;
  hipLaunchKernelGGL(state_init_kernel, dim3(static_cast<unsigned>((nS + 255) / 256)), dim3(256), 0, stream,
                     S0, z0, S, z, nS, nz);
  return hipGetLastError();
}

}  // namespace tl
