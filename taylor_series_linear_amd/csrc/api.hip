// C ABI of libtaylor_attn.so: argument checks, segment planning, dispatch.
// The operation itself is documented in include/taylor_attn.h.
#include "../../include/taylor_attn.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "features.hpp"
#include "internal.hpp"

namespace {

thread_local std::string g_last_error;

taylor_status fail(taylor_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool supported_dn(int d, int n_terms) {
  if (d == 16) return n_terms == 1 || n_terms == 3 || n_terms == 5 || n_terms == 7;
  if (d == 32 || d == 64) return n_terms == 1 || n_terms == 3;
  return false;
}

bool supported(int d, int dv, int n_terms) {
  if (dv != 16 && dv != 64) return false;
  if (n_terms == 7) return d == 16 && dv == 64;  // order 6: one instantiation
  return supported_dn(d, n_terms);
}

taylor_status check_dn(int d, int dv, int n_terms, bool with_dv) {
  if (n_terms >= 1 && n_terms % 2 == 0)
    return fail(TAYLOR_ERR_UNSUPPORTED,
                "n_terms must be odd (highest order even, so every weight is positive); got " +
                    std::to_string(n_terms));
  if (with_dv ? !supported(d, dv, n_terms) : !supported_dn(d, n_terms))
    return fail(TAYLOR_ERR_UNSUPPORTED,
                "unsupported configuration d=" + std::to_string(d) +
                    (with_dv ? " dv=" + std::to_string(dv) : std::string()) +
                    " n_terms=" + std::to_string(n_terms) +
                    " (supported: d=16 with n_terms 1,3,5 and dv 16 or 64, or n_terms 7 and dv 64; d=32 or 64 with n_terms"
                    " 1,3 and dv 16 or 64)");
  return TAYLOR_OK;
}

taylor_status check_scale(float a) {
  if (!std::isfinite(a) || !(a > 0.f))
    return fail(TAYLOR_ERR_BAD_SCALE, "scale a must be finite and > 0");
  return TAYLOR_OK;
}

taylor_status check_gamma(float g) {
  if (!std::isfinite(g) || !(g > 0.f) || g > 1.f)
    return fail(TAYLOR_ERR_BAD_SCALE, "decay gamma must satisfy 0 < gamma <= 1");
  return TAYLOR_OK;
}

taylor_status check_ext(const taylor_attn_ext* x) {
  taylor_status s = check_gamma(x->gamma);
  if (s != TAYLOR_OK) return s;
  if (!std::isfinite(x->q_scale) || !(x->q_scale > 0.f) || !std::isfinite(x->k_scale) || !(x->k_scale > 0.f))
    return fail(TAYLOR_ERR_BAD_SCALE, "q_scale and k_scale must be finite and > 0");
  return TAYLOR_OK;
}

// Options of the plain entry points' decayed variants.
taylor_attn_ext decay_only(float gamma) {
  taylor_attn_ext x{};
  x.gamma = gamma;
  x.qk_norm = 0;
  x.q_scale = 1.f;
  x.k_scale = 1.f;
  x.q_head_scale = nullptr;
  return x;
}

taylor_status check_dtype(taylor_dtype t, const char* what) {
  if (t != TAYLOR_F32 && t != TAYLOR_BF16)
    return fail(TAYLOR_ERR_UNSUPPORTED, std::string(what) + " must be TAYLOR_F32 or TAYLOR_BF16");
  return TAYLOR_OK;
}

// a*b*c*... without int64 overflow; -1 on overflow or negative input.
int64_t checked_mul(std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x < 0) return -1;
    if (x != 0 && r > INT64_MAX / x) return -1;
    r *= x;
  }
  return r;
}

// Bound of the single-pass order-2 kernel's wait for earlier segments, in
// polls (about a second by default). TAYLOR_ATTN_WAIT_SPINS overrides it, read
// once per process: a tiny value lets a test force the timed-out path (the
// unit's rows and final state come out NaN) without any kernel hanging.
int wait_spins() {
  static const int v = [] {
    const char* e = std::getenv("TAYLOR_ATTN_WAIT_SPINS");
    if (e != nullptr) {
      const long x = std::strtol(e, nullptr, 10);
      if (x >= 1 && x <= (1L << 30)) return static_cast<int>(x);
    }
    return 1 << 20;
  }();
  return v;
}

taylor_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return TAYLOR_OK;
  return fail(TAYLOR_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// Validation shared by the size query and the call; fills the plan.
taylor_status check_prefill_shape(int B, int H, int N, int d, int dv, int n_terms,
                                  taylor_dtype in_dtype, bool decay, tl::PrefillPlan* plan) {
  taylor_status s = check_dtype(in_dtype, "in_dtype");
  if (s != TAYLOR_OK) return s;
  if (B < 0 || H < 0 || N < 0)
    return fail(TAYLOR_ERR_BAD_SHAPE, "B, H and N must be >= 0");
  if ((s = check_dn(d, dv, n_terms, true)) != TAYLOR_OK) return s;
  if (checked_mul({B, H, N, d > dv ? d : dv}) < 0 || checked_mul({B, H}) > INT32_MAX / 64)
    return fail(TAYLOR_ERR_BAD_SHAPE, "B*H*N*max(d,dv) overflows");
  if (!tl::prefill_plan(d, dv, n_terms, in_dtype == TAYLOR_BF16, decay, B * H, N, plan))
    return fail(TAYLOR_ERR_UNSUPPORTED, "no prefill instantiation for this configuration");
  return TAYLOR_OK;
}

}  // namespace

extern "C" {

int64_t taylor_feature_dim(int d, int n_terms) {
  if (d < 1 || n_terms < 1) return -1;
  // C(d+n-1, n-1) computed incrementally with an overflow guard
  long double f = 0;
  int64_t total = 0;
  for (int m = 0; m < n_terms; ++m) {
    // C(d+m-1, m)
    long double c = 1;
    for (int i = 1; i <= m; ++i) c = c * (d - 1 + i) / i;
    f += c;
    if (f > static_cast<long double>(INT64_MAX) / 2) return -1;
  }
  total = static_cast<int64_t>(std::llround(static_cast<double>(f)));
  return total;
}

int taylor_is_supported(int d, int dv, int n_terms) { return supported(d, dv, n_terms) ? 1 : 0; }

const char* taylor_last_error(void) { return g_last_error.c_str(); }

taylor_status taylor_feature_map(const void* x, taylor_dtype x_dtype, int64_t rows, int d,
                                 int n_terms, float a, int fold_alpha, float* phi,
                                 void* stream) {
  taylor_status s = check_dtype(x_dtype, "x_dtype");
  if (s != TAYLOR_OK) return s;
  if (rows < 0) return fail(TAYLOR_ERR_BAD_SHAPE, "rows must be >= 0");
  if ((s = check_dn(d, 16, n_terms, false)) != TAYLOR_OK) return s;
  if (fold_alpha && (s = check_scale(a)) != TAYLOR_OK) return s;
  const int F = tl::feature_count(d, n_terms);
  if (checked_mul({rows, F}) < 0 || checked_mul({rows, d}) < 0)
    return fail(TAYLOR_ERR_BAD_SHAPE, "rows*F overflows");
  if (rows == 0) return TAYLOR_OK;
  if (x == nullptr || phi == nullptr) return fail(TAYLOR_ERR_NULL_PTR, "x and phi are required");
  tl::OrderScale sc{};
  for (int m = 0; m < 8; ++m) {
    double v = 1.0;
    if (fold_alpha) v = 1.0 / std::sqrt(static_cast<double>(tl::factorial(m)) * std::pow(static_cast<double>(a), m));
    sc.s[m] = static_cast<float>(v);
  }
  return hip_status(tl::feature_map_launch(d, n_terms, x_dtype == TAYLOR_BF16, x, rows, phi, sc,
                                           static_cast<hipStream_t>(stream)),
                    "taylor_feature_map launch");
}

}  // extern "C"

namespace {

// Scratch of the allocation-free prefill (taylor_attn_prefill_noalloc): its
// per-segment state sums, final-state staging and ticket counters live here
// instead of in a caller-provided workspace. Every GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` is a
// host-side stand-in, not a device address: the device address of each
// GPU's copy comes from hipGetSymbolAddress with that device current, once
// per device, and only that address is ever passed to kernels.
constexpr size_t kScratchBytes = TAYLOR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of this GPU's scratch for work enqueued on `stream` (the
// stream's device; the current device for the null stream).
taylor_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1, cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  dev = cur;
  if (stream != nullptr && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess)
    return hip_status(e, "hipStreamGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TAYLOR_ERR_HIP, "device index out of range for the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return TAYLOR_OK;
}

// Shared by the plain and the decayed prefill; `decay` selects the kernel
// family (the decayed one also runs gamma = 1, so its workspace size does not
// depend on gamma).
taylor_status prefill_impl(const void* q, const void* k, const void* v, taylor_dtype in_dtype, int B, int H,
                           int N, int d, int dv, int n_terms, float a, const taylor_attn_ext* ext, const float* S0,
                           const float* z0, void* o, taylor_dtype out_dtype, float* S, float* z,
                           void* workspace, size_t ws_bytes, void* stream, bool use_scratch = false) {
  tl::PrefillPlan p;
  const bool extk = ext != nullptr;
  taylor_status s = check_prefill_shape(B, H, N, d, dv, n_terms, in_dtype, extk, &p);
  if (s != TAYLOR_OK) return s;
  if ((s = check_dtype(out_dtype, "out_dtype")) != TAYLOR_OK) return s;
  if ((s = check_scale(a)) != TAYLOR_OK) return s;
  if (extk && (s = check_ext(ext)) != TAYLOR_OK) return s;
  if ((S0 == nullptr) != (z0 == nullptr))
    return fail(TAYLOR_ERR_NULL_PTR, "S0 and z0 must both be given or both be NULL");
  if ((S == nullptr) != (z == nullptr))
    return fail(TAYLOR_ERR_NULL_PTR, "S and z must both be given or both be NULL");
  const int BH = B * H;
  if (BH > 0 && N > 0 && (q == nullptr || k == nullptr || v == nullptr))
    return fail(TAYLOR_ERR_NULL_PTR, "q, k and v are required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (use_scratch) {
    if (p.bytes > kScratchBytes)
      return fail(TAYLOR_ERR_WORKSPACE, "these sizes need " + std::to_string(p.bytes) +
                                            " bytes of scratch, more than the " + std::to_string(kScratchBytes) +
                                            " bytes of the allocation-free call; use taylor_attn_prefill with a "
                                            "workspace");
    if (BH == 0 || N == 0) {
      workspace = nullptr;
    } else if (p.bytes > 0) {
      if ((s = scratch_address(st, &workspace)) != TAYLOR_OK) return s;
    }
    ws_bytes = kScratchBytes;
  }
  if (p.bytes > 0 && (workspace == nullptr || ws_bytes < p.bytes))
    return fail(TAYLOR_ERR_WORKSPACE, "workspace too small: need " + std::to_string(p.bytes) +
                                          " bytes, got " + std::to_string(ws_bytes));
  if (BH == 0) return TAYLOR_OK;
  (void)hipGetLastError();  // report only errors of the launches below
  if (N == 0) {
    if (S == nullptr) return TAYLOR_OK;
    return hip_status(tl::state_init_launch(S0, z0, S, z, BH, static_cast<int>(taylor_feature_dim(d, n_terms)), dv, st),
                      "state init launch");
  }
  tl::PrefillArgs args{};
  args.q = q;
  args.k = k;
  args.v = v;
  args.S0 = S0;
  args.z0 = z0;
  args.o = o;
  args.out_bf16 = out_dtype == TAYLOR_BF16;
  args.S = S;
  args.z = z;
  char* ws = static_cast<char*>(workspace);
  args.seg = p.fin_off > p.seg_off ? reinterpret_cast<float*>(ws + p.seg_off) : nullptr;
  args.fin = p.P > 1 ? reinterpret_cast<float*>(ws + p.fin_off) : nullptr;
  args.part = p.bytes > p.part_off ? reinterpret_cast<float*>(ws + p.part_off) : nullptr;
  args.sync = p.sync_off > 0 ? reinterpret_cast<int*>(ws + p.sync_off) : nullptr;
  args.BH = BH;
  args.N = N;
  args.P = p.P;
  args.L = p.L;
  args.L0 = p.L0;
  args.inv_a = 1.0f / a;
  args.wait_spins = wait_spins();
  // In-place continuation with several segments: the first segment reads S0
  // while the last one finishes the state, so the final state goes through
  // the workspace and is copied out afterwards.
  args.defer_state = (S != nullptr && p.P > 1 && (S == S0 || z == z0)) ? 1 : 0;
  args.decay = extk ? 1 : 0;
  args.log2g = extk ? std::log2(ext->gamma) : 0.f;
  args.qk_norm = extk ? (ext->qk_norm != 0) : 0;
  args.q_scale = extk ? ext->q_scale : 1.f;
  args.k_scale = extk ? ext->k_scale : 1.f;
  args.q_head_scale = extk ? ext->q_head_scale : nullptr;
  args.H = H;
  return hip_status(tl::prefill_launch(d, dv, n_terms, in_dtype == TAYLOR_BF16, args, st),
                    "taylor_attn_prefill launch");
}

taylor_status decode_impl(const void* q, const void* k, const void* v, taylor_dtype in_dtype, int B, int H,
                          int d, int dv, int n_terms, float a, const taylor_attn_ext& ext, float* S, float* z,
                          void* o, taylor_dtype out_dtype, void* stream) {
  taylor_status s = check_dtype(in_dtype, "in_dtype");
  if (s != TAYLOR_OK) return s;
  if ((s = check_dtype(out_dtype, "out_dtype")) != TAYLOR_OK) return s;
  if (B < 0 || H < 0) return fail(TAYLOR_ERR_BAD_SHAPE, "B and H must be >= 0");
  if ((s = check_dn(d, dv, n_terms, true)) != TAYLOR_OK) return s;
  if ((s = check_scale(a)) != TAYLOR_OK) return s;
  if ((s = check_ext(&ext)) != TAYLOR_OK) return s;
  if (checked_mul({B, H}) > INT32_MAX)
    return fail(TAYLOR_ERR_BAD_SHAPE, "B*H exceeds the grid limit");
  const int BH = B * H;
  if (BH == 0) return TAYLOR_OK;
  if (!q || !k || !v || !S || !z || !o)
    return fail(TAYLOR_ERR_NULL_PTR, "q, k, v, S, z and o are required");
  tl::DecodeArgs args{};
  args.q = q;
  args.k = k;
  args.v = v;
  args.S = S;
  args.z = z;
  args.o = o;
  args.out_bf16 = out_dtype == TAYLOR_BF16;
  args.BH = BH;
  args.inv_a = 1.0f / a;
  args.gamma = ext.gamma;
  args.qk_norm = ext.qk_norm != 0;
  args.q_scale = ext.q_scale;
  args.k_scale = ext.k_scale;
  args.q_head_scale = ext.q_head_scale;
  args.H = H;
  (void)hipGetLastError();
  return hip_status(tl::decode_launch(d, dv, n_terms, in_dtype == TAYLOR_BF16, args,
                                      static_cast<hipStream_t>(stream)),
                    "taylor_attn_decode launch");
}

}  // namespace

extern "C" {

size_t taylor_attn_prefill_workspace(int B, int H, int N, int d, int dv, int n_terms,
                                     taylor_dtype in_dtype) {
  tl::PrefillPlan p;
  if (check_prefill_shape(B, H, N, d, dv, n_terms, in_dtype, false, &p) != TAYLOR_OK)
    return static_cast<size_t>(-1);
  return p.bytes;
}

taylor_status taylor_attn_prefill(const void* q, const void* k, const void* v,
                                  taylor_dtype in_dtype, int B, int H, int N, int d, int dv,
                                  int n_terms, float a, const float* S0, const float* z0,
                                  void* o, taylor_dtype out_dtype, float* S, float* z,
                                  void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(q, k, v, in_dtype, B, H, N, d, dv, n_terms, a, nullptr, S0, z0, o, out_dtype, S, z,
                      workspace, ws_bytes, stream);
}

taylor_status taylor_attn_prefill_noalloc(const void* q, const void* k, const void* v, taylor_dtype in_dtype, int B,
                                          int H, int N, int d, int dv, int n_terms, float a, const float* S0,
                                          const float* z0, void* o, taylor_dtype out_dtype, float* S, float* z,
                                          void* stream) {
  return prefill_impl(q, k, v, in_dtype, B, H, N, d, dv, n_terms, a, nullptr, S0, z0, o, out_dtype, S, z, nullptr,
                      0, stream, true);
}

size_t taylor_attn_prefill_decayed_workspace(int B, int H, int N, int d, int dv, int n_terms,
                                             taylor_dtype in_dtype) {
  tl::PrefillPlan p;
  if (check_prefill_shape(B, H, N, d, dv, n_terms, in_dtype, true, &p) != TAYLOR_OK)
    return static_cast<size_t>(-1);
  return p.bytes;
}

taylor_status taylor_attn_prefill_decayed(const void* q, const void* k, const void* v,
                                          taylor_dtype in_dtype, int B, int H, int N, int d, int dv,
                                          int n_terms, float a, float gamma, const float* S0,
                                          const float* z0, void* o, taylor_dtype out_dtype, float* S,
                                          float* z, void* workspace, size_t ws_bytes, void* stream) {
  const taylor_attn_ext x = decay_only(gamma);
  return prefill_impl(q, k, v, in_dtype, B, H, N, d, dv, n_terms, a, &x, S0, z0, o, out_dtype, S, z, workspace,
                      ws_bytes, stream);
}

size_t taylor_attn_prefill_ext_workspace(int B, int H, int N, int d, int dv, int n_terms, taylor_dtype in_dtype) {
  return taylor_attn_prefill_decayed_workspace(B, H, N, d, dv, n_terms, in_dtype);
}

taylor_status taylor_attn_prefill_ext(const void* q, const void* k, const void* v, taylor_dtype in_dtype, int B,
                                      int H, int N, int d, int dv, int n_terms, float a, const taylor_attn_ext* ext,
                                      const float* S0, const float* z0, void* o, taylor_dtype out_dtype, float* S,
                                      float* z, void* workspace, size_t ws_bytes, void* stream) {
  if (ext == nullptr) return fail(TAYLOR_ERR_NULL_PTR, "ext is required");
  return prefill_impl(q, k, v, in_dtype, B, H, N, d, dv, n_terms, a, ext, S0, z0, o, out_dtype, S, z, workspace,
                      ws_bytes, stream);
}

taylor_status taylor_attn_decode(const void* q, const void* k, const void* v,
                                 taylor_dtype in_dtype, int B, int H, int d, int dv,
                                 int n_terms, float a, float* S, float* z, void* o,
                                 taylor_dtype out_dtype, void* stream) {
  return decode_impl(q, k, v, in_dtype, B, H, d, dv, n_terms, a, decay_only(1.f), S, z, o, out_dtype, stream);
}

taylor_status taylor_attn_decode_decayed(const void* q, const void* k, const void* v,
                                         taylor_dtype in_dtype, int B, int H, int d, int dv,
                                         int n_terms, float a, float gamma, float* S, float* z, void* o,
                                         taylor_dtype out_dtype, void* stream) {
  return decode_impl(q, k, v, in_dtype, B, H, d, dv, n_terms, a, decay_only(gamma), S, z, o, out_dtype, stream);
}

taylor_status taylor_attn_decode_ext(const void* q, const void* k, const void* v, taylor_dtype in_dtype, int B,
                                     int H, int d, int dv, int n_terms, float a, const taylor_attn_ext* ext, float* S,
                                     float* z, void* o, taylor_dtype out_dtype, void* stream) {
  if (ext == nullptr) return fail(TAYLOR_ERR_NULL_PTR, "ext is required");
  return decode_impl(q, k, v, in_dtype, B, H, d, dv, n_terms, a, *ext, S, z, o, out_dtype, stream);
}

}  // extern "C"
