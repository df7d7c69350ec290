// Single-token decode step and the standalone feature map.
//
// Decode ("Expanding Attention: A Taylor-Series Route to Linear-Time
// Transformers with a Fixed Number of Recurrent States", "Decoding": one
// token costs sum_m C(d+m-1,m)(dv+1), independent of the context length):
//   S_m = g S_m + phi_m(k) v^T,  z_m = g z_m + phi_m(k)      (update first ...)
//   o = sum_m alpha_m phi_m(q)^T S_m / sum_m alpha_m phi_m(q)^T z_m  (... then read out)
// following the linear-attention recurrence S_t = S_{t-1} + v_t phi(k_t)^T,
// o_t = S_t phi(q_t) (Spanish linear-attention explainer); g is the constant
// decay that the same explainer's superposed-memory paragraph applies to
// S_{t-1} before the write (g = 1: none).
//
// The step streams each head's state once: read, add, write back, and fold
// the new row into the read-out while it is still in registers. It is bound
// by HBM bandwidth (about 0.5 flop per state byte), so the kernel is shaped
// for coalescing: 16 lanes cover one 64-float state row with 16-byte
// accesses, every lane keeps several rows in flight, and the per-feature
// weights phi(k), alpha*phi(q) are computed once per head into LDS. State
// accesses are non-temporal: each byte is touched once per step, and the
// streaming hint lifts the read-modify-write rate above that of a plain copy.
#include <type_traits>

#include "features.hpp"
#include "internal.hpp"
#include "mma.hpp"

namespace tl {

template <int D, int NT>
__device__ const PackedTable<D, NT> g_dtab = make_packed<D, NT>();

template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
  if constexpr (BF16)
    return static_cast<float>(reinterpret_cast<const __bf16*>(p)[i]);
  else
    return reinterpret_cast<const float*>(p)[i];
}

// Sum of the read-out partials of a block of NWV waves: thread tid holds the
// numerator part `acc` of value columns 4 (tid % NQ) .. + 4 and a share
// `dpart` of the denominator. The row groups inside a wave are summed with
// lane exchanges, then the waves' sums meet in LDS: afterwards red[c]
// (c < NQ) holds the numerator of columns 4c .. 4c + 3 and dred[0] the
// denominator, for every thread.
template <int NQ, int NWV = 4>
__device__ __forceinline__ void block_reduce(f32x4 acc, float dpart, f32x4* red, float* dred) {
  static_assert(NQ == 4 || NQ == 16, "row groups tile a 64-lane wave");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int m = NQ; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], m);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) dpart += __shfl_xor(dpart, m);
  if (lane < NQ) red[wv * NQ + lane] = acc;
  if (lane == 0) dred[wv] = dpart;
  __syncthreads();
  if (tid < NQ) {
    f32x4 t = red[tid];
#pragma unroll
    for (int v = 1; v < NWV; ++v) t += red[v * NQ + tid];
    red[tid] = t;
    if (tid == 0) {
      float dd = dred[0];
#pragma unroll
      for (int v = 1; v < NWV; ++v) dd += dred[v];
      dred[0] = dd;
    }
  }
  __syncthreads();
}

template <int D, int DV, int NT, bool BF16>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int F = feature_count(D, NT);
  constexpr int NQ = DV / 4;              // float4 columns per state row
  constexpr int NG = 256 / NQ;            // row groups
  constexpr int RPT = (F + NG - 1) / NG;  // rows per thread (upper bound)
  // rows whose loads are in flight at once; the whole share when it is small
  constexpr int BATCH = RPT <= 12 ? RPT : 8;
  constexpr int ZPT = (F + 255) / 256;    // z entries per thread

  __shared__ float sq[D], sk[D];
  __shared__ __attribute__((aligned(16))) float sv[DV];
  __shared__ float sfk[F], sfq[F];
  __shared__ f32x4 red[4 * NQ];
  __shared__ float dred[4];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const float inv_a = a.inv_a;
  const float g = a.gamma;
  const int dq = tid % NQ;
  const int rg = tid / NQ;
  float* Sh = a.S + static_cast<size_t>(bh) * F * DV;
  float* zh = a.z + static_cast<size_t>(bh) * F;

  // The state rows do not depend on q, k or v: their loads go out first, so
  // the state read overlaps the small input loads and the feature map.
  f32x4 rows[BATCH];
  auto load_batch = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int f = rg + NG * (r0 + j);
      if (r0 + j < RPT && f < F)
        rows[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sh + static_cast<size_t>(f) * DV + 4 * dq));
    }
  };
  load_batch(0);
  float zv[ZPT];
#pragma unroll
  for (int j = 0; j < ZPT; ++j) {
    const int f = tid + 256 * j;
    zv[j] = f < F ? __builtin_nontemporal_load(zh + f) : 0.f;
  }

  if (tid < D) {
    sq[tid] = load_in<BF16>(a.q, static_cast<size_t>(bh) * D + tid);
    sk[tid] = load_in<BF16>(a.k, static_cast<size_t>(bh) * D + tid);
  }
  if (tid < DV) sv[tid] = load_in<BF16>(a.v, static_cast<size_t>(bh) * DV + tid);
  __syncthreads();

  // query/key preprocessing: row l2-normalisation and scales (factors on
  // every coordinate)
  float fq = a.q_scale * (a.q_head_scale != nullptr ? a.q_head_scale[bh % a.H] : 1.f);
  float fk = a.k_scale;
  if (a.qk_norm) {
    float nq = 0.f, nk = 0.f;
    for (int j = 0; j < D; ++j) {
      nq += sq[j] * sq[j];
      nk += sk[j] * sk[j];
    }
    fq = nq > 0.f ? fq / __builtin_sqrtf(nq) : 0.f;
    fk = nk > 0.f ? fk / __builtin_sqrtf(nk) : 0.f;
  }
  const float cq = fq * inv_a;

  const auto& tab = g_dtab<D, NT>;
  for (int f = tid; f < F; f += 256) {
    const PackedFeature e = tab.e[f];
    const int m = static_cast<int>(e.m);
    float pk = e.w, pq = e.w * e.inv_mfact;
    for (int j = 0; j < m; ++j) {
      const int i = (e.idx >> (8 * j)) & 255;
      pk *= sk[i] * fk;
      pq *= sq[i] * cq;
    }
    sfk[f] = pk;
    sfq[f] = pq;
  }
  __syncthreads();

  const f32x4 vv = *reinterpret_cast<const f32x4*>(sv + 4 * dq);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < RPT; r0 += BATCH) {
    if (r0 > 0) load_batch(r0);
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int f = rg + NG * (r0 + j);
      if (r0 + j < RPT && f < F) {
        const f32x4 s = rows[j] * g + sfk[f] * vv;
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(Sh + static_cast<size_t>(f) * DV + 4 * dq));
        acc += sfq[f] * s;
      }
    }
  }
  float dpart = 0.f;
#pragma unroll
  for (int j = 0; j < ZPT; ++j) {
    const int f = tid + 256 * j;
    if (f < F) {
      const float zz = zv[j] * g + sfk[f];
      __builtin_nontemporal_store(zz, zh + f);
      dpart += sfq[f] * zz;
    }
  }
  block_reduce<NQ>(acc, dpart, red, dred);
  if (tid < NQ) {
    const f32x4 num = red[tid];
    const float r = 1.f / dred[0];
    const size_t off = static_cast<size_t>(bh) * DV + 4 * tid;
    if (a.out_bf16) {
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(num[i] * r);
      *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + off) = ov;
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + off) = num * r;
    }
  }
}

// 1/m! for the degrees of a decoded feature
__device__ __forceinline__ float inv_factorial(int m) {
  float r = 1.f;
  for (int j = 2; j <= m; ++j) r *= 1.f / static_cast<float>(j);
  return r;
}

// Decode step for bases too wide to hold phi(k) and alpha*phi(q) in LDS at
// once (order 6 at d = 16: 74,613 features, a 19 MB state per head). The
// state is processed in blocks of FB rows: every thread decodes the first
// feature of its run of the block and steps through the run, writing both
// feature values to LDS; then the block's rows stream exactly as in
// decode_kernel (read, update, write back, fold into the read-out). The
// first rows of a block are requested before its features are generated.
template <int D, int DV, int NT, bool BF16>
__global__ __launch_bounds__(1024) void decode_wide_kernel(DecodeArgs a) {
  constexpr int NT_ = 1024;                // threads: a 19 MB state per head needs many loads in flight
  constexpr int F = feature_count(D, NT);
  constexpr int FB = 4096;                // state rows per block
  constexpr int RUN = FB / NT_;           // features generated per thread and block
  constexpr int NQ = DV / 4;              // float4 columns per state row
  constexpr int NG = NT_ / NQ;            // row groups
  constexpr int RPB = FB / NG;            // rows per row group and block
  constexpr int BATCH = 8;                // rows in flight per thread
  static_assert(RPB % BATCH == 0 && FB % NT_ == 0, "block shape");

  __shared__ float sq[D], sk[D];
  __shared__ __attribute__((aligned(16))) float sv[DV];
  __shared__ float sfk[FB], sfq[FB];
  __shared__ f32x4 red[(NT_ / 64) * NQ];
  __shared__ float dred[NT_ / 64];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const float g = a.gamma;
  const int dq = tid % NQ;
  const int rg = tid / NQ;
  float* Sh = a.S + static_cast<size_t>(bh) * F * DV;
  float* zh = a.z + static_cast<size_t>(bh) * F;

  f32x4 rows[BATCH];
  auto load_batch = [&](int f0, int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int f = f0 + rg + NG * (r0 + j);
      if (f < F)
        rows[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sh + static_cast<size_t>(f) * DV + 4 * dq));
    }
  };
  load_batch(0, 0);

  if (tid < D) {
    sq[tid] = load_in<BF16>(a.q, static_cast<size_t>(bh) * D + tid);
    sk[tid] = load_in<BF16>(a.k, static_cast<size_t>(bh) * D + tid);
  }
  if (tid < DV) sv[tid] = load_in<BF16>(a.v, static_cast<size_t>(bh) * DV + tid);
  __syncthreads();

  // query/key preprocessing, as in decode_kernel
  float fq = a.q_scale * (a.q_head_scale != nullptr ? a.q_head_scale[bh % a.H] : 1.f);
  float fk = a.k_scale;
  if (a.qk_norm) {
    float nq = 0.f, nk = 0.f;
    for (int j = 0; j < D; ++j) {
      nq += sq[j] * sq[j];
      nk += sk[j] * sk[j];
    }
    fq = nq > 0.f ? fq / __builtin_sqrtf(nq) : 0.f;
    fk = nk > 0.f ? fk / __builtin_sqrtf(nk) : 0.f;
  }
  const float cq = fq * a.inv_a;

  const f32x4 vv = *reinterpret_cast<const f32x4*>(sv + 4 * dq);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float dpart = 0.f;
  for (int f0 = 0; f0 < F; f0 += FB) {
    if (f0 > 0) {
      __syncthreads();  // every thread is done with the previous block's features
      load_batch(f0, 0);
    }
    RankedFeature e = rank_decode(D, NT, f0 + RUN * tid);
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      float pk = 0.f, pq = 0.f;
      if (f0 + RUN * tid + j < F) {
        pk = e.w;
        pq = e.w * inv_factorial(e.m);
#pragma unroll
        for (int u = 0; u < kMaxOrderRank; ++u) {
          if (u < e.m) {
            pk *= sk[e.idx[u]] * fk;
            pq *= sq[e.idx[u]] * cq;
          }
        }
      }
      sfk[RUN * tid + j] = pk;
      sfq[RUN * tid + j] = pq;
      if (j + 1 < RUN) rank_next(D, e);
    }
    __syncthreads();
    for (int r0 = 0; r0 < RPB; r0 += BATCH) {
      if (r0 > 0) load_batch(f0, r0);
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int fl = rg + NG * (r0 + j);
        if (f0 + fl < F) {
          const f32x4 s = rows[j] * g + sfk[fl] * vv;
          __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(Sh + static_cast<size_t>(f0 + fl) * DV + 4 * dq));
          acc += sfq[fl] * s;
        }
      }
    }
    float zv[FB / NT_];
#pragma unroll
    for (int j = 0; j < FB / NT_; ++j) {
      const int f = f0 + tid + NT_ * j;
      zv[j] = f < F ? __builtin_nontemporal_load(zh + f) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < FB / NT_; ++j) {
      const int fl = tid + NT_ * j;
      if (f0 + fl < F) {
        const float zz = zv[j] * g + sfk[fl];
        __builtin_nontemporal_store(zz, zh + f0 + fl);
        dpart += sfq[fl] * zz;
      }
    }
  }
  block_reduce<NQ, NT_ / 64>(acc, dpart, red, dred);
  if (tid < NQ) {
    const f32x4 num = red[tid];
    const float r = 1.f / dred[0];
    const size_t off = static_cast<size_t>(bh) * DV + 4 * tid;
    if (a.out_bf16) {
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(num[i] * r);
      *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + off) = ov;
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + off) = num * r;
    }
  }
}

// Feature map, phi[row, f] = w_f * scale[m_f] * prod_j x[row, i_j]. A
// workgroup covers a block of FM_ROWS rows and FM_FB consecutive features;
// the block's input rows are staged in LDS. Every thread decodes the seven
// features around its four (offsets -3 .. +3) once and steps through them
// (no per-element index arithmetic or table lookup). A row's stretch of
// outputs starts at an arbitrary 4-byte offset (F is odd), so per row the
// threads shift their four outputs by the stretch's misalignment s (the
// same for the whole block): thread t writes elements 4t - s .. 4t - s + 3
// of the stretch with one 16-byte store at a 16-byte aligned address, and
// the consecutive stores of a wave cover a contiguous part of the row. Only
// the first and the last thread of a stretch write single elements. When a
// row has at most 253 features a wave covers it and the four waves of the
// workgroup work on four rows at a time; every wave then holds a row's ends,
// so there each thread writes its four features with 4-byte stores instead
// (no shift). The kernel is bound by the HBM write of phi.
constexpr int FM_ROWS = 64;
constexpr int FM_FPT = 4;                       // outputs per thread and row
constexpr int FM_FB = 256 * FM_FPT - FM_FPT;    // features per block: shifted windows of 1024 cover them
constexpr int FM_WIN = FM_FPT + 3;              // features a thread holds
template <int D, int NT, bool BF16>
__global__ __launch_bounds__(256) void feature_map_kernel(const void* x, int64_t rows, float* phi,
                                                          OrderScale sc) {
  constexpr int F = feature_count(D, NT);
  constexpr int TPR = F + 3 <= 64 * FM_FPT ? 64 : 256;  // threads per row
  constexpr int NGR = 256 / TPR;                        // rows at a time
  __shared__ float xs[FM_ROWS * D];
  const int tid = threadIdx.x;
  const int tr = tid % TPR, grp = tid / TPR;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * FM_ROWS;
  const int nr = static_cast<int>(rows - r0 < FM_ROWS ? rows - r0 : FM_ROWS);
  for (int i = tid; i < nr * D; i += 256) xs[i] = load_in<BF16>(x, static_cast<size_t>(r0) * D + i);
  __syncthreads();
  const int fb = static_cast<int>(blockIdx.y) * FM_FB;
  const int nf = F - fb < FM_FB ? F - fb : FM_FB;  // features of this block
  // features f0 - 3 .. f0 + 3 of this thread: coefficient (zero outside the
  // basis) and indices, in registers
  const int fs = fb + FM_FPT * tr - 3;
  float cf[FM_WIN];
  int ix[FM_WIN][kMaxOrderRank];
  int mm[FM_WIN];
  RankedFeature e = rank_decode(D, NT, fs < 0 ? 0 : fs);
#pragma unroll
  for (int k = 0; k < FM_WIN; ++k) {
    const int fk = fs + k;
    cf[k] = fk >= 0 && fk < F ? e.w * sc.s[e.m] : 0.f;
    mm[k] = e.m;
#pragma unroll
    for (int u = 0; u < kMaxOrderRank; ++u) ix[k][u] = e.idx[u];
    if (k + 1 < FM_WIN && fk >= 0) rank_next(D, e);
  }
  // phi's own misalignment in elements
  const int mis = static_cast<int>((reinterpret_cast<uintptr_t>(phi) >> 2) & 3);
  for (int r = grp; r < nr; r += NGR) {
    const float* xr = xs + r * D;
    const int64_t g = (r0 + r) * static_cast<int64_t>(F) + fb;  // first element of the row's stretch
    const int s = TPR == 64 ? 0 : static_cast<int>((g + mis) & 3);
    const int lo = FM_FPT * tr - s;  // this thread's first element within the stretch
    if (lo >= nf) continue;
    auto out = [&](auto stag) __attribute__((always_inline)) {
      constexpr int S = decltype(stag)::value;
      f32x4 v;
#pragma unroll
      for (int j = 0; j < FM_FPT; ++j) {
        const int k = j - S + 3;
        float p = cf[k];
#pragma unroll
        for (int u = 0; u < kMaxOrderRank; ++u)
          if (u < mm[k]) p *= xr[ix[k][u]];
        v[j] = p;
      }
      float* dst = phi + g + lo;
      if (TPR != 64 && lo >= 0 && lo + FM_FPT <= nf) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
#pragma unroll
        for (int j = 0; j < FM_FPT; ++j)
          if (lo + j >= 0 && lo + j < nf) dst[j] = v[j];
      }
    };
    if constexpr (TPR == 64) {
      out(std::integral_constant<int, 0>{});
    } else {
      switch (s) {
        case 0: out(std::integral_constant<int, 0>{}); break;
        case 1: out(std::integral_constant<int, 1>{}); break;
        case 2: out(std::integral_constant<int, 2>{}); break;
        default: out(std::integral_constant<int, 3>{}); break;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

#define TL_DECODE_CFGS(X) \
  X(16, 16, 1)            \
  X(16, 64, 1)            \
  X(16, 16, 3)            \
  X(16, 64, 3)            \
  X(16, 16, 5)            \
  X(16, 64, 5)            \
  X(32, 16, 1)            \
  X(32, 64, 1)            \
  X(32, 16, 3)            \
  X(32, 64, 3)            \
  X(64, 16, 1)            \
  X(64, 64, 1)            \
  X(64, 16, 3)            \
  X(64, 64, 3)

hipError_t decode_launch(int d, int dv, int n_terms, bool bf16, const DecodeArgs& a,
                         hipStream_t stream) {
#define X(D, DV, NT)                                                                        \
  if (d == D && dv == DV && n_terms == NT) {                                                \
    if (bf16)                                                                               \
      hipLaunchKernelGGL((decode_kernel<D, DV, NT, true>), dim3(a.BH), dim3(256), 0, stream, a);  \
    else                                                                                    \
      hipLaunchKernelGGL((decode_kernel<D, DV, NT, false>), dim3(a.BH), dim3(256), 0, stream, a); \
    return hipGetLastError();                                                               \
  }
  TL_DECODE_CFGS(X)
#undef X
  // bases too wide for the LDS-resident features
  if (d == 16 && dv == 64 && n_terms == 7) {
    if (bf16)
      hipLaunchKernelGGL((decode_wide_kernel<16, 64, 7, true>), dim3(a.BH), dim3(1024), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_wide_kernel<16, 64, 7, false>), dim3(a.BH), dim3(1024), 0, stream, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t feature_map_launch(int d, int n_terms, bool bf16, const void* x, int64_t rows,
                              float* phi, const OrderScale& sc, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t rb = (rows + FM_ROWS - 1) / FM_ROWS;
  if (rb > 0x7fffffff) return hipErrorInvalidValue;
#define X(D, NT)                                                                                       \
  if (d == D && n_terms == NT) {                                                                       \
    const dim3 grid(static_cast<unsigned>(rb), (feature_count(D, NT) + FM_FB - 1) / FM_FB);               \
    if (bf16)                                                                                          \
      hipLaunchKernelGGL((feature_map_kernel<D, NT, true>), grid, dim3(256), 0, stream, x, rows, phi, sc); \
    else                                                                                               \
      hipLaunchKernelGGL((feature_map_kernel<D, NT, false>), grid, dim3(256), 0, stream, x, rows, phi, sc); \
    return hipGetLastError();                                                                          \
  }
  X(16, 1) X(16, 3) X(16, 5) X(16, 7) X(32, 1) X(32, 3) X(64, 1) X(64, 3)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace tl
