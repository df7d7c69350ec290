// Timing of the C ABI from a plain C++ host, with no Python or torch in the
// process: the library used the way a C or C++ serving loop would use it.
//
// Workloads (inputs iid N(0,1) from a seeded std::mt19937_64; random values
// matter: all-zero states and inputs run the memory-bound decode step about
// 4% faster than random ones on the same shapes):
//  * order-2 decode: 64 sequences x 16 heads, d = 16, dv = 64, n_terms = 3,
//    a = 4, fp32 q, k, v and states. The state is seeded by a 256-token
//    prefill (its size does not depend on the context length), then 1024
//    steps run with fresh q, k, v per step: "cold" over 8 state replicas
//    used round-robin (325 MB, more than the last-level cache), "hot" on one.
//  * Based-style order-2 prefill: B = 4, H = 16, N = 4096, d = 16, dv = 64,
//    bf16 in and out, a = 4; 200 calls over 4 input replicas.
//  * long-context order-2 prefill: B = 1, H = 8, N = 65536, d = 64, dv = 64,
//    bf16 in and out, a = 8; 20 calls over 2 input replicas (3 untimed).
// The decode and the d = 16 prefill run 64 untimed calls first; times come
// from HIP events around the timed calls on the null stream. Prints one JSON
// line.
//
// Usage: bench_native [decode_steps] [prefill_calls]
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/taylor_attn.h"

namespace {

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "bench_native: %s failed: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

void tl_check(taylor_status s, const char* what) {
  if (s != TAYLOR_OK) {
    std::fprintf(stderr, "bench_native: %s failed: %s\n", what, taylor_last_error());
    std::exit(1);
  }
}

std::vector<float> normals(size_t n, uint64_t seed) {
  std::mt19937_64 g(seed);
  std::normal_distribution<double> nd(0.0, 1.0);
  std::vector<float> x(n);
  for (auto& v : x) v = static_cast<float>(nd(g));
  return x;
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite)
std::vector<uint16_t> to_bf16(const std::vector<float>& x) {
  std::vector<uint16_t> y(x.size());
  for (size_t i = 0; i < x.size(); ++i) {
    uint32_t u;
    std::memcpy(&u, &x[i], 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    y[i] = static_cast<uint16_t>(u >> 16);
  }
  return y;
}

template <typename T>
void* upload(const std::vector<T>& h) {
  void* p = nullptr;
  hip_check(hipMalloc(&p, h.size() * sizeof(T)), "hipMalloc");
  hip_check(hipMemcpy(p, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy");
  return p;
}

void* alloc(size_t bytes) {
  void* p = nullptr;
  hip_check(hipMalloc(&p, bytes ? bytes : 1), "hipMalloc");
  return p;
}

// average milliseconds per call over `n` calls of f(i), i = first .. first+n-1
template <typename Fn>
double time_calls(int first, int n, Fn&& f) {
  hipEvent_t e0, e1;
  hip_check(hipEventCreate(&e0), "hipEventCreate");
  hip_check(hipEventCreate(&e1), "hipEventCreate");
  hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");
  hip_check(hipEventRecord(e0, nullptr), "hipEventRecord");
  for (int i = 0; i < n; ++i) f(first + i);
  hip_check(hipEventRecord(e1, nullptr), "hipEventRecord");
  hip_check(hipEventSynchronize(e1), "hipEventSynchronize");
  float ms = 0.f;
  hip_check(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime");
  hip_check(hipEventDestroy(e0), "hipEventDestroy");
  hip_check(hipEventDestroy(e1), "hipEventDestroy");
  return static_cast<double>(ms) / n;
}

}  // namespace

int main(int argc, char** argv) {
  const int steps = argc > 1 ? std::atoi(argv[1]) : 1024;
  const int calls = argc > 2 ? std::atoi(argv[2]) : 200;
  if (steps < 1 || calls < 1) {
    std::fprintf(stderr, "usage: bench_native [decode_steps >= 1] [prefill_calls >= 1]\n");
    return 2;
  }
  int runtime = 0;
  hip_check(hipRuntimeGetVersion(&runtime), "hipRuntimeGetVersion");

  // ---- order-2 decode ----------------------------------------------------
  const int B = 64, H = 16, d = 16, dv = 64, n = 3, R = 8, N0 = 256;
  const float a = 4.f;
  const int64_t F = taylor_feature_dim(d, n);
  const size_t heads = static_cast<size_t>(B) * H;
  const size_t s_elems = heads * F * dv, z_elems = heads * F;
  void* pq = upload(normals(heads * N0 * d, 1004));
  void* pk = upload(normals(heads * N0 * d, 1005));
  void* pv = upload(normals(heads * N0 * dv, 1006));
  const size_t wsb = taylor_attn_prefill_workspace(B, H, N0, d, dv, n, TAYLOR_F32);
  void* ws = alloc(wsb);
  std::vector<float*> S(R), z(R);
  for (int r = 0; r < R; ++r) {
    S[r] = static_cast<float*>(alloc(s_elems * 4));
    z[r] = static_cast<float*>(alloc(z_elems * 4));
  }
  tl_check(taylor_attn_prefill(pq, pk, pv, TAYLOR_F32, B, H, N0, d, dv, n, a, nullptr, nullptr, nullptr,
                               TAYLOR_F32, S[0], z[0], ws, wsb, nullptr),
           "seeding prefill");
  for (int r = 1; r < R; ++r) {
    hip_check(hipMemcpy(S[r], S[0], s_elems * 4, hipMemcpyDeviceToDevice), "hipMemcpy");
    hip_check(hipMemcpy(z[r], z[0], z_elems * 4, hipMemcpyDeviceToDevice), "hipMemcpy");
  }
  const char* dq = static_cast<const char*>(upload(normals(static_cast<size_t>(steps) * heads * d, 1007)));
  const char* dk = static_cast<const char*>(upload(normals(static_cast<size_t>(steps) * heads * d, 1008)));
  const char* dvv = static_cast<const char*>(upload(normals(static_cast<size_t>(steps) * heads * dv, 1009)));
  void* o = alloc(heads * dv * 4);
  auto step = [&](int i, int reps) {
    const size_t s = static_cast<size_t>(i % steps);
    const taylor_status st =
        taylor_attn_decode(dq + s * heads * d * 4, dk + s * heads * d * 4, dvv + s * heads * dv * 4, TAYLOR_F32, B,
                           H, d, dv, n, a, S[i % reps], z[i % reps], o, TAYLOR_F32, nullptr);
    if (st != TAYLOR_OK) tl_check(st, "decode");
  };
  for (int i = 0; i < 64; ++i) step(i, R);
  const double ms_cold = time_calls(0, steps, [&](int i) { step(i, R); });
  for (int i = 0; i < 64; ++i) step(i, 1);
  const double ms_hot = time_calls(0, steps, [&](int i) { step(i, 1); });
  const double state_bytes = 2.0 * F * (dv + 1) * 4 * heads;

  // ---- Based-style order-2 prefill -----------------------------------------
  const int PB = 4, PH = 16, PN = 4096, PR = 4;
  const size_t nqk = static_cast<size_t>(PB) * PH * PN * d, nv = static_cast<size_t>(PB) * PH * PN * dv;
  const auto hq = to_bf16(normals(nqk, 1002)), hk = to_bf16(normals(nqk, 1012)), hv = to_bf16(normals(nv, 1022));
  std::vector<void*> q(PR), k(PR), v(PR), po(PR);
  for (int r = 0; r < PR; ++r) {
    q[r] = upload(hq);
    k[r] = upload(hk);
    v[r] = upload(hv);
    po[r] = alloc(nv * 2);
  }
  const size_t pwsb = taylor_attn_prefill_workspace(PB, PH, PN, d, dv, n, TAYLOR_BF16);
  void* pws = alloc(pwsb);
  auto call = [&](int i) {
    const int r = i % PR;
    const taylor_status st = taylor_attn_prefill(q[r], k[r], v[r], TAYLOR_BF16, PB, PH, PN, d, dv, n, a, nullptr,
                                                 nullptr, po[r], TAYLOR_BF16, nullptr, nullptr, pws, pwsb, nullptr);
    if (st != TAYLOR_OK) tl_check(st, "prefill");
  };
  for (int i = 0; i < 64; ++i) call(i);
  const double ms_pf = time_calls(0, calls, call);
  const double pf_bytes = static_cast<double>(PB) * PH * PN * ((2.0 * d + dv) * 2 + dv * 2);
  hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");

  // ---- long-context order-2 prefill (d = 64) -------------------------------
  const int LB = 1, LH = 8, LN = 65536, LD = 64, LR = 2, LC = calls < 20 ? calls : 20;
  const float la = 8.f;
  const size_t lqk = static_cast<size_t>(LB) * LH * LN * LD;
  const auto lq = to_bf16(normals(lqk, 1005)), lk = to_bf16(normals(lqk, 1015)), lv = to_bf16(normals(lqk, 1025));
  std::vector<void*> q2(LR), k2(LR), v2(LR), o2(LR);
  for (int r = 0; r < LR; ++r) {
    q2[r] = upload(lq);
    k2[r] = upload(lk);
    v2[r] = upload(lv);
    o2[r] = alloc(lqk * 2);
  }
  const size_t lwsb = taylor_attn_prefill_workspace(LB, LH, LN, LD, dv, n, TAYLOR_BF16);
  void* lws = alloc(lwsb);
  auto lcall = [&](int i) {
    const int r = i % LR;
    const taylor_status st = taylor_attn_prefill(q2[r], k2[r], v2[r], TAYLOR_BF16, LB, LH, LN, LD, dv, n, la,
                                                 nullptr, nullptr, o2[r], TAYLOR_BF16, nullptr, nullptr, lws, lwsb,
                                                 nullptr);
    if (st != TAYLOR_OK) tl_check(st, "long prefill");
  };
  for (int i = 0; i < 3; ++i) lcall(i);
  const double ms_long = time_calls(0, LC, lcall);
  const int64_t LF = taylor_feature_dim(LD, n);
  const double long_flops = static_cast<double>(LB) * LH * LN * (4.0 * LF * (dv + 1) + 33.0 * (LD + dv + 1));
  hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");

  std::printf(
      "{\"hip_runtime_version\": %d, "
      "\"decode\": {\"heads\": %zu, \"features\": %lld, \"steps_timed\": %d, \"state_replicas_cold\": %d, "
      "\"us_per_step_cold\": %.3f, \"us_per_step_hot\": %.3f, \"state_GBps_cold\": %.1f, "
      "\"hbm_frac_cold\": %.4f}, "
      "\"prefill\": {\"B\": %d, \"H\": %d, \"N\": %d, \"calls_timed\": %d, \"input_replicas\": %d, "
      "\"us_per_call\": %.3f, \"tokens_per_s\": %.4e, \"algorithmic_GBps\": %.1f, \"hbm_frac\": %.4f}, "
      "\"long_prefill\": {\"B\": %d, \"H\": %d, \"N\": %d, \"d\": %d, \"calls_timed\": %d, \"input_replicas\": %d, "
      "\"ms_per_call\": %.4f, \"tokens_per_s\": %.4e, \"algorithmic_TFLOPs\": %.1f, \"mfma_frac\": %.4f}}\n",
      runtime, heads, static_cast<long long>(F), steps, R, ms_cold * 1e3, ms_hot * 1e3,
      state_bytes / (ms_cold * 1e-3) / 1e9, state_bytes / (ms_cold * 1e-3) / 8e12, PB, PH, PN, calls, PR, ms_pf * 1e3,
      PB * PN / (ms_pf * 1e-3), pf_bytes / (ms_pf * 1e-3) / 1e9, pf_bytes / (ms_pf * 1e-3) / 8e12, LB, LH, LN, LD,
      LC, LR, ms_long, LB * LN / (ms_long * 1e-3), long_flops / (ms_long * 1e-3) / 1e12,
      long_flops / (ms_long * 1e-3) / 1e12 / 2500.0);
  return 0;
}
