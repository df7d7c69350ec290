/*
 * taylor_attn.h -- C ABI of the MI355X (gfx950) causal Taylor-series linear
 * attention library (libtaylor_attn.so).
 *
 * What is computed. For one (batch, head) with queries q_t, keys k_s in R^d
 * and values v_s in R^dv, t = 0..N-1, and n = n_terms:
 *
 *   w(x)  = sum_{m=0}^{n-1} x^m / m!            (truncated exp; coefficient
 *                                               1/(m! a^m) on (q.k)^m)
 *   o_t   = sum_{s<=t} w(q_t.k_s / a) v_s  /  sum_{s<=t} w(q_t.k_s / a)
 *
 * ("Expanding Attention: A Taylor-Series Route to Linear-Time Transformers
 * with a Fixed Number of Recurrent States": the expansion of exp(q.k/a),
 * the causal mask and normalisation of the softmax it replaces.) The library
 * evaluates it through per-order states (same page, "Memory"; the
 * linear-attention recurrence S_t = S_{t-1} + v_t phi(k_t)^T of the Spanish
 * linear-attention explainer):
 *
 *   S_m = sum_s phi_m(k_s) v_s^T   [F_m x dv],   z_m = sum_s phi_m(k_s)   [F_m]
 *   o_t = sum_m alpha_m phi_m(q_t)^T S_m / sum_m alpha_m phi_m(q_t)^T z_m,
 *   alpha_m = 1 / (m! a^m),
 *
 * where phi_m is the symmetric tensor-power feature map of width
 * F_m = C(d+m-1, m) ("Higher orders"): one feature per index tuple
 * i_1 <= ... <= i_m, value sqrt(m! / prod_i c_i!) * prod_j x[i_j] (c_i counts
 * index i in the tuple), so phi_m(x).phi_m(y) = (x.y)^m.
 *
 * Canonical feature order (the F axis of every state buffer): orders
 * m = 0..n-1 ascending; within order m, tuples in lexicographic order.
 * F = sum_m F_m = C(d+n-1, n-1).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller, dense row-major, with the layouts stated per argument. The
 *    library allocates no device memory and never synchronises: work is
 *    enqueued on `stream` (a hipStream_t passed as void*; NULL = the default
 *    stream) and kernel errors surface at the caller's next synchronisation.
 *  - Argument checks are synchronous and happen before anything is enqueued;
 *    on a non-OK status nothing has been launched and no output is touched.
 *  - Inputs are not scanned for NaN or Inf; such values propagate.
 *  - taylor_last_error() returns a message for the last non-OK status on the
 *    calling thread (thread-local; valid until the next call on that thread).
 *  - Supported (d, dv, n_terms): d = 16 with dv in {16, 64} and n_terms in
 *    {1, 3, 5}, and with dv = 64 and n_terms = 7 (order 6, F = 74,613: the
 *    highest even order the positivity-floor README discusses, minimum
 *    weight about 0.15); d = 32 or 64 with dv in {16, 64} and n_terms in
 *    {1, 3}. The feature map supports the same (d, n_terms). n_terms must
 *    be odd so that the highest order is even and every weight is positive
 *    ("Two prerequisites" on the same page; posfloor README, "The 1/2
 *    positivity floor": even truncations are globally positive). Anything
 *    else returns TAYLOR_ERR_UNSUPPORTED.
 */
#ifndef TAYLOR_ATTN_H
#define TAYLOR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TAYLOR_OK = 0,
  TAYLOR_ERR_NULL_PTR = 1,    /* a required pointer is NULL, or only one of a pointer pair is */
  TAYLOR_ERR_BAD_SHAPE = 2,   /* negative size, or a size product overflowing int64 */
  TAYLOR_ERR_UNSUPPORTED = 3, /* (d, dv, n_terms) or dtype not instantiated; even n_terms */
  TAYLOR_ERR_BAD_SCALE = 4,   /* a not finite or a <= 0 */
  TAYLOR_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the size query returned */
  TAYLOR_ERR_HIP = 6          /* a HIP launch failed (message from hipGetErrorString) */
} taylor_status;

typedef enum {
  TAYLOR_F32 = 0,  /* IEEE binary32 */
  TAYLOR_BF16 = 1  /* bfloat16 (upper half of binary32) */
} taylor_dtype;

/* Width F = sum_{m<n} C(d+m-1, m) of the symmetric basis; -1 if d < 1,
 * n_terms < 1 or the result overflows int64. Pure host function. */
int64_t taylor_feature_dim(int d, int n_terms);

/* 1 if (d, dv, n_terms) is an instantiated configuration, else 0. */
int taylor_is_supported(int d, int dv, int n_terms);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* taylor_last_error(void);

/*
 * Symmetric feature map (the basis above).
 *   x    [rows, d]  x_dtype (F32 or BF16), device.
 *   phi  [rows, F]  float32, device, written in full.
 *   fold_alpha = 0: block m holds phi_m(x), so phi_m(x).phi_m(y) = (x.y)^m.
 *   fold_alpha = 1: block m is also scaled by sqrt(alpha_m) = (m! a^m)^(-1/2),
 *                   so phi(x).phi(y) = w(x.y / a).  `a` is ignored when 0.
 * rows = 0 is valid and launches nothing. Same (d, n_terms) support set as the
 * attention calls (dv is not involved).
 */
taylor_status taylor_feature_map(const void* x, taylor_dtype x_dtype, int64_t rows, int d,
                                 int n_terms, float a, int fold_alpha, float* phi,
                                 void* stream);

/*
 * Bytes of device workspace taylor_attn_prefill needs for these sizes (0 if
 * none). Depends only on the arguments, and is the same for any output dtype.
 * Returns (size_t)-1 when the arguments would be rejected by the call.
 */
size_t taylor_attn_prefill_workspace(int B, int H, int N, int d, int dv, int n_terms,
                                     taylor_dtype in_dtype);

/*
 * Causal prefill over N tokens for B x H independent heads.
 *   q, k      [B, H, N, d]   in_dtype (F32 or BF16)
 *   v         [B, H, N, dv]  in_dtype
 *   S0, z0    [B, H, F, dv], [B, H, F] float32: state of earlier tokens to
 *             continue from (both NULL = start from zero). States are
 *             additive (the closing paragraph of the same page), so
 *             prefill(x1) then prefill(x2 | S, z) equals prefill(x1 ++ x2).
 *   o         [B, H, N, dv]  out_dtype (F32 or BF16), or NULL to compute the
 *             state only.
 *   S, z      [B, H, F, dv], [B, H, F] float32: final state after the N
 *             tokens (both NULL = not wanted). S may be the same buffer as
 *             S0 and z the same as z0 (in-place continuation); other
 *             overlaps between inputs and outputs are not allowed.
 *   workspace at least taylor_attn_prefill_workspace(...) bytes of device
 *             memory (may be NULL when that size is 0). Its contents are
 *             scratch: clobbered by the call, never read before written.
 * B, H or N may be 0: then no token is processed; with N = 0 the final state
 * is S0 (or zero). The normalisation divides by a sum of weights that is
 * >= 1/2 per key for n_terms = 3 (>= 0.27 for 5, >= 0.149 for 7), so it never
 * divides by 0.
 * Range: several bf16 instantiations carry operands in fp16 (largest finite
 * magnitude 65504) with fp32 accumulation:
 *  - order 2, d = 16, dv = 64: keys, values, key products k_i k_j, and the
 *    intra-chunk weights w(q.k/a) (t = q.k/a is formed in fp32, so this
 *    holds for |t| up to about 360, whatever a is);
 *  - order 2, d = 64: q/a, the query products q_i q_j / a^2, k_i k_j, values
 *    and the intra-chunk weights;
 *  - the other bf16 instantiations with n_terms > 1 and d > 16, or
 *    n_terms = 5 or 7, use keys halved, so the products of m halved
 *    coordinates must stay below 65504, e.g. |k_i| < 32 for n_terms = 5;
 *    for n_terms = 7 the key features also carry the sqrt-multinomial
 *    weight (at most sqrt(720) ~ 26.8), e.g. |k_i| < 8 suffices.
 * Under the normalisation the method asks for (|q.k/a| of order 1) these
 * always hold. Beyond them results are inf or NaN from the first affected
 * row on; rows of earlier queries stay exact, because the causal mask sets
 * masked weights to exactly zero.
 * Long sequences are split into segments that run concurrently; in the
 * order-2, d = 16, dv = 64 bf16 instantiation a segment waits (boundedly,
 * about a second) for the sums of the earlier segments of its head. If that
 * wait ever times out, the segment's output rows, and for the last segment
 * the final state, are written as NaN rather than silently wrong; the status
 * is still TAYLOR_OK, since kernels run after the call returns. The
 * environment variable TAYLOR_ATTN_WAIT_SPINS (read once per process; polls,
 * default 2^20) lowers the bound, so tests can force that path.
 */
taylor_status taylor_attn_prefill(const void* q, const void* k, const void* v,
                                  taylor_dtype in_dtype, int B, int H, int N, int d, int dv,
                                  int n_terms, float a, const float* S0, const float* z0,
                                  void* o, taylor_dtype out_dtype, float* S, float* z,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Allocation-free prefill, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, results and errors as taylor_attn_prefill,
 * without the workspace: the call's scratch (per-segment state sums,
 * final-state staging, ticket counters) lives in a static device array of
 * TAYLOR_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends. The call allocates and frees nothing.
 *  - Sizes whose workspace (taylor_attn_prefill_workspace) exceeds
 *    TAYLOR_NOALLOC_SCRATCH_BYTES return TAYLOR_ERR_WORKSPACE.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents: calls that overlap on one GPU (other streams, other
 *    threads) race and give wrong results. Serialise them (one stream).
 *  - The first call on a device looks the array's device address up (once
 *    per device, with the stream's device current).
 */
#define TAYLOR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
taylor_status taylor_attn_prefill_noalloc(const void* q, const void* k, const void* v,
                                          taylor_dtype in_dtype, int B, int H, int N, int d, int dv,
                                          int n_terms, float a, const float* S0, const float* z0,
                                          void* o, taylor_dtype out_dtype, float* S, float* z,
                                          void* stream);

/*
 * One generation step for B x H heads: update the state with (k, v), then
 * read out with q (update before read-out, as in S_t = S_{t-1} + v_t phi(k_t)^T,
 * o_t = S_t phi(q_t)).
 *   q, k  [B, H, d]   in_dtype;  v [B, H, dv]  in_dtype
 *   S, z  [B, H, F, dv], [B, H, F] float32, read and updated in place.
 *   o     [B, H, dv]  out_dtype.
 * B or H may be 0 (nothing launched).
 */
taylor_status taylor_attn_decode(const void* q, const void* k, const void* v,
                                 taylor_dtype in_dtype, int B, int H, int d, int dv,
                                 int n_terms, float a, float* S, float* z, void* o,
                                 taylor_dtype out_dtype, void* stream);

/*
 * Decayed state (Spanish linear-attention explainer, paragraph on the
 * superposed memory: forgetting by a decay that multiplies S_{t-1} before
 * each write, the reading of Mamba-2 as linear attention with decay). One
 * constant gamma for every step, head and order, applied to S and z alike:
 *   S_t = gamma S_{t-1} + phi(k_t) v_t^T,  z_t = gamma z_{t-1} + phi(k_t),
 *   o_t = sum_m alpha_m phi_m(q_t).S_m,t / sum_m alpha_m phi_m(q_t).z_m,t,
 * i.e. token s enters o_t with weight gamma^(t-s) w(q_t.k_s/a), and S0/z0
 * (the state just before token 0) with gamma^(t+1). gamma = 1 gives the
 * plain results (up to rounding; the decayed prefill always runs the generic
 * kernel family).
 * Arguments, layouts, ownership and errors are those of taylor_attn_prefill
 * and taylor_attn_decode, plus:
 *   gamma  0 < gamma <= 1 and finite, else TAYLOR_ERR_BAD_SCALE.
 * The workspace of the decayed prefill is sized by
 * taylor_attn_prefill_decayed_workspace (independent of gamma).
 */
size_t taylor_attn_prefill_decayed_workspace(int B, int H, int N, int d, int dv, int n_terms,
                                             taylor_dtype in_dtype);
taylor_status taylor_attn_prefill_decayed(const void* q, const void* k, const void* v,
                                          taylor_dtype in_dtype, int B, int H, int N, int d, int dv,
                                          int n_terms, float a, float gamma, const float* S0,
                                          const float* z0, void* o, taylor_dtype out_dtype, float* S,
                                          float* z, void* workspace, size_t ws_bytes, void* stream);
taylor_status taylor_attn_decode_decayed(const void* q, const void* k, const void* v,
                                         taylor_dtype in_dtype, int B, int H, int d, int dv,
                                         int n_terms, float a, float gamma, float* S, float* z, void* o,
                                         taylor_dtype out_dtype, void* stream);

/*
 * Extended options: the decay above plus query/key preprocessing fused into
 * the kernels. "Expanding Attention" (defaults paragraph, "Two
 * prerequisites") runs on queries and keys normalised to the unit sphere and
 * calls this mandatory; the related work it cites adds a per-head
 * temperature. With qk_norm set, every q and k row is divided by its l2 norm
 * (a zero row stays zero); then q is multiplied by q_scale and, per head h,
 * by q_head_scale[h], and k by k_scale. The method runs on those rows. For
 * bf16 inputs the preprocessed rows are rounded to bf16 inside the kernels.
 *   gamma         0 < gamma <= 1 (1: no decay)
 *   qk_norm       0 or 1
 *   q_scale       finite, > 0 (1: none)
 *   k_scale       finite, > 0 (1: none)
 *   q_head_scale  device pointer to H floats, or NULL (all 1); read by the
 *                 kernels, not checked
 * Invalid gamma or scales return TAYLOR_ERR_BAD_SCALE; a NULL ext returns
 * TAYLOR_ERR_NULL_PTR. Everything else is as for taylor_attn_prefill and
 * taylor_attn_decode; the prefill workspace is sized by
 * taylor_attn_prefill_ext_workspace (the same size as for the decayed call).
 */
typedef struct taylor_attn_ext {
  float gamma;
  int qk_norm;
  float q_scale;
  float k_scale;
  const float* q_head_scale;
} taylor_attn_ext;

size_t taylor_attn_prefill_ext_workspace(int B, int H, int N, int d, int dv, int n_terms,
                                         taylor_dtype in_dtype);
taylor_status taylor_attn_prefill_ext(const void* q, const void* k, const void* v,
                                      taylor_dtype in_dtype, int B, int H, int N, int d, int dv,
                                      int n_terms, float a, const taylor_attn_ext* ext,
                                      const float* S0, const float* z0, void* o, taylor_dtype out_dtype,
                                      float* S, float* z, void* workspace, size_t ws_bytes, void* stream);
taylor_status taylor_attn_decode_ext(const void* q, const void* k, const void* v,
                                     taylor_dtype in_dtype, int B, int H, int d, int dv, int n_terms,
                                     float a, const taylor_attn_ext* ext, float* S, float* z, void* o,
                                     taylor_dtype out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TAYLOR_ATTN_H */
