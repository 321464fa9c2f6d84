// C ABI of libneo: host-side validation, then one launch per call on the caller's
// stream.  Declarations and the contract of each call are in include/neo.h.
#include "neo.h"
#include "neo_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>

namespace {

thread_local char g_err[512];

neo_status fail(neo_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

neo_status ok() {
  g_err[0] = '\0';
  return NEO_OK;
}

neo_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NEO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool finite(float x) { return isfinite(x); }

size_t dtype_size(neo_dtype d) { return d == NEO_BF16 ? 2 : 4; }

// [a, a+na) and [b, b+nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// element count t * h * 128 without int64 overflow
bool rows_fit(int64_t t, int64_t h) {
  return t >= 0 && h >= 1 && t <= (int64_t)(INT64_MAX / 4) / h / neo::kHeadDim;
}

// workgroups x threads within the 32-bit work-item count of one dispatch
bool grid_fits(int64_t blocks, int threads) {
  return blocks >= 0 && blocks <= (int64_t)0xffffffffLL / threads;
}

}  // namespace

extern "C" {

const char* neo_status_string(neo_status s) {
  switch (s) {
    case NEO_OK: return "ok";
    case NEO_ERR_NULL: return "null pointer";
    case NEO_ERR_SHAPE: return "bad shape";
    case NEO_ERR_VALUE: return "bad value";
    case NEO_ERR_UNSUPPORTED: return "unsupported";
    case NEO_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* neo_last_error(void) { return g_err; }

neo_status neo_qknorm_rope3(const void* q_in, const void* k_in, void* q_out, void* k_out,
                            int64_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                            const float* q_norm_w, const float* q_norm_hw_w,
                            const float* k_norm_w, const float* k_norm_hw_w,
                            const int32_t* pos_thw, float rope_theta, float rope_theta_hw,
                            float eps, neo_dtype dtype, void* hip_stream) {
  if (dtype != NEO_F32 && dtype != NEO_BF16)
    return fail(NEO_ERR_UNSUPPORTED, "neo_qknorm_rope3: unknown dtype %d", (int)dtype);
  if (head_dim != NEO_HEAD_DIM)
    return fail(NEO_ERR_SHAPE, "neo_qknorm_rope3: head_dim must be 128, got %d", head_dim);
  if (Hq < 1 || Hkv < 1)
    return fail(NEO_ERR_SHAPE, "neo_qknorm_rope3: Hq=%d Hkv=%d must be >= 1", Hq, Hkv);
  if (T < 0 || !rows_fit(T, Hq) || !rows_fit(T, Hkv))
    return fail(NEO_ERR_SHAPE, "neo_qknorm_rope3: T=%lld out of range", (long long)T);
  if (!finite(rope_theta) || rope_theta <= 0.0f || !finite(rope_theta_hw) ||
      rope_theta_hw <= 0.0f)
    return fail(NEO_ERR_VALUE, "neo_qknorm_rope3: rope bases must be finite and > 0");
  if (!finite(eps) || eps < 0.0f)
    return fail(NEO_ERR_VALUE, "neo_qknorm_rope3: eps must be finite and >= 0");
  if (T == 0) return ok();
  if (!q_in || !k_in || !q_out || !k_out || !q_norm_w || !q_norm_hw_w || !k_norm_w ||
      !k_norm_hw_w || !pos_thw)
    return fail(NEO_ERR_NULL, "neo_qknorm_rope3: a required pointer is NULL");
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q_out) || !aligned16(k_out))
    return fail(NEO_ERR_VALUE, "neo_qknorm_rope3: q/k buffers must be 16-byte aligned");
  const size_t es = dtype_size(dtype);
  const size_t qb = (size_t)T * Hq * NEO_HEAD_DIM * es, kb = (size_t)T * Hkv * NEO_HEAD_DIM * es;
  if ((q_out != q_in && overlap(q_out, qb, q_in, qb)) || overlap(q_out, qb, k_in, kb) ||
      (k_out != k_in && overlap(k_out, kb, k_in, kb)) || overlap(k_out, kb, q_in, qb) ||
      overlap(q_out, qb, k_out, kb))
    return fail(NEO_ERR_VALUE, "neo_qknorm_rope3: outputs overlap inputs other than in place");
  return from_hip(neo::launch_qknorm_rope3(dtype == NEO_BF16, q_in, k_in, q_out, k_out, T, Hq,
                                           Hkv, q_norm_w, q_norm_hw_w, k_norm_w, k_norm_hw_w,
                                           pos_thw, (double)rope_theta, (double)rope_theta_hw,
                                           eps, static_cast<hipStream_t>(hip_stream)),
                  "neo_qknorm_rope3 launch");
}

neo_status neo_gen_attn_fwd(const void* q, const void* k_img, const void* v_img,
                            const void* k_prefix, const void* v_prefix,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_prefix,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                            int64_t total_q, int64_t total_prefix, int32_t max_seqlen_q,
                            int32_t max_seqlen_prefix, float softmax_scale, void* out, float* lse,
                            neo_dtype dtype, void* hip_stream) {
  if (dtype != NEO_F32 && dtype != NEO_BF16)
    return fail(NEO_ERR_UNSUPPORTED, "neo_gen_attn_fwd: unknown dtype %d", (int)dtype);
  if (head_dim != NEO_HEAD_DIM)
    return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: head_dim must be 128, got %d", head_dim);
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: B=%d Hq=%d Hkv=%d must be >= 1", B, Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (max_seqlen_q < 0 || max_seqlen_prefix < 0)
    return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: negative max_seqlen");
  if (!rows_fit(total_q, Hq) || !rows_fit(total_prefix, Hkv))
    return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: total_q=%lld total_prefix=%lld out of range",
                (long long)total_q, (long long)total_prefix);
  if (max_seqlen_q > total_q || max_seqlen_prefix > total_prefix)
    return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: max_seqlen exceeds the tensor's rows");
  // one sample's K or V segment is addressed with 32-bit byte offsets
  if ((int64_t)max_seqlen_q * Hkv * NEO_HEAD_DIM * 4 >= ((int64_t)1 << 31) ||
      (int64_t)max_seqlen_prefix * Hkv * NEO_HEAD_DIM * 4 >= ((int64_t)1 << 31))
    return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: one sample's K/V rows exceed 2 GiB");
  if (!isfinite(softmax_scale))
    return fail(NEO_ERR_VALUE, "neo_gen_attn_fwd: softmax_scale must be finite");
  // grid size: one workgroup per (sample, KV head, 8 chunks of 32 query rows) -- per 4
  // chunks when that launch would have at most 128 workgroups --, or per (sample, KV head,
  // 128 query rows) for fp32; must fit a 32-bit grid
  {
    const int64_t G = Hq / Hkv;
    const int64_t per = dtype == NEO_BF16 ? ((int64_t)G * ((max_seqlen_q + 31) / 32) + 7) / 8
                                          : ((int64_t)max_seqlen_q * G + 127) / 128;
    if (!grid_fits(per * Hkv * B, dtype == NEO_BF16 ? neo::kAttnBf16Threads : neo::kAttnF32Threads))
      return fail(NEO_ERR_SHAPE, "neo_gen_attn_fwd: problem too large for one launch");
  }
  if (max_seqlen_q == 0 || total_q == 0) return ok();
  if (!q || !k_img || !v_img || !cu_seqlens_q || !cu_seqlens_prefix || !out)
    return fail(NEO_ERR_NULL, "neo_gen_attn_fwd: a required pointer is NULL");
  if (total_prefix > 0 && (!k_prefix || !v_prefix))
    return fail(NEO_ERR_NULL, "neo_gen_attn_fwd: k_prefix/v_prefix NULL with total_prefix > 0");
  const void* bufs[5] = {q, k_img, v_img, k_prefix, v_prefix};
  for (const void* p : bufs)
    if (p && !aligned16(p))
      return fail(NEO_ERR_VALUE, "neo_gen_attn_fwd: q/k/v buffers must be 16-byte aligned");
  if (!aligned16(out))
    return fail(NEO_ERR_VALUE, "neo_gen_attn_fwd: out must be 16-byte aligned");
  const size_t es = dtype_size(dtype);
  const size_t ob = (size_t)total_q * Hq * NEO_HEAD_DIM * es;
  const size_t sizes[5] = {ob, (size_t)total_q * Hkv * NEO_HEAD_DIM * es,
                           (size_t)total_q * Hkv * NEO_HEAD_DIM * es,
                           (size_t)total_prefix * Hkv * NEO_HEAD_DIM * es,
                           (size_t)total_prefix * Hkv * NEO_HEAD_DIM * es};
  const size_t lb = lse ? (size_t)total_q * Hq * sizeof(float) : 0;
  for (int i = 0; i < 5; ++i)
    if (bufs[i] && (overlap(out, ob, bufs[i], sizes[i]) || (lse && overlap(lse, lb, bufs[i], sizes[i]))))
      return fail(NEO_ERR_VALUE, "neo_gen_attn_fwd: out/lse overlap an input");
  if (lse && overlap(lse, lb, out, ob))
    return fail(NEO_ERR_VALUE, "neo_gen_attn_fwd: lse overlaps out");
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)NEO_HEAD_DIM);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (dtype == NEO_BF16)
    e = neo::launch_gen_attn_bf16(q, k_img, v_img, k_prefix, v_prefix, cu_seqlens_q,
                                  cu_seqlens_prefix, B, Hq, Hkv, max_seqlen_q, max_seqlen_prefix,
                                  scale, out, lse, total_q, total_prefix, stream);
  else
    e = neo::launch_gen_attn_f32(
        static_cast<const float*>(q), static_cast<const float*>(k_img),
        static_cast<const float*>(v_img), static_cast<const float*>(k_prefix),
        static_cast<const float*>(v_prefix), cu_seqlens_q, cu_seqlens_prefix, B, Hq, Hkv,
        max_seqlen_q, max_seqlen_prefix, scale, static_cast<float*>(out), lse, total_q,
        total_prefix, stream);
  return from_hip(e, "neo_gen_attn_fwd launch");
}

neo_status neo_fm_euler_step(float* z, const float* x0_pred, int64_t n, float t, float t_next,
                             float t_eps, void* hip_stream) {
  if (n < 0 || n > INT64_MAX / 16)
    return fail(NEO_ERR_SHAPE, "neo_fm_euler_step: n=%lld out of range", (long long)n);
  if (!finite(t) || !finite(t_next) || !finite(t_eps))
    return fail(NEO_ERR_VALUE, "neo_fm_euler_step: t, t_next, t_eps must be finite");
  if (t_eps <= 0.0f) return fail(NEO_ERR_VALUE, "neo_fm_euler_step: t_eps must be > 0");
  if (t_next < t) return fail(NEO_ERR_VALUE, "neo_fm_euler_step: t_next < t");
  if (n == 0) return ok();
  if (!z || !x0_pred) return fail(NEO_ERR_NULL, "neo_fm_euler_step: z or x0_pred is NULL");
  const size_t nb = (size_t)n * sizeof(float);
  if (static_cast<const void*>(z) != static_cast<const void*>(x0_pred) &&
      overlap(z, nb, x0_pred, nb))
    return fail(NEO_ERR_VALUE, "neo_fm_euler_step: z and x0_pred partially overlap");
  if ((reinterpret_cast<uintptr_t>(z) | reinterpret_cast<uintptr_t>(x0_pred)) & 3)
    return fail(NEO_ERR_VALUE, "neo_fm_euler_step: buffers must be 4-byte aligned");
  const double denom = fmax(1.0 - (double)t, (double)t_eps);
  const float coef = (float)(((double)t_next - (double)t) / denom);
  return from_hip(neo::launch_euler_step(z, x0_pred, n, coef, static_cast<hipStream_t>(hip_stream)),
                  "neo_fm_euler_step launch");
}

neo_status neo_qkv_proj_norm_rope(const void* x, const void* w_qkv, int64_t N, int32_t hidden,
                                  int32_t Hq, int32_t Hkv, int32_t head_dim, const float* q_norm_w,
                                  const float* q_norm_hw_w, const float* k_norm_w,
                                  const float* k_norm_hw_w, const int32_t* pos_thw,
                                  float rope_theta, float rope_theta_hw, float eps, void* q_out,
                                  void* k_out, void* v_out, neo_dtype dtype, void* hip_stream) {
  const char* fn = "neo_qkv_proj_norm_rope";
  if (dtype != NEO_F32 && dtype != NEO_BF16)
    return fail(NEO_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (dtype != NEO_BF16) return fail(NEO_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (head_dim != NEO_HEAD_DIM)
    return fail(NEO_ERR_SHAPE, "%s: head_dim must be 128, got %d", fn, head_dim);
  if (Hq < 1 || Hkv < 1 || Hq > 4096 || Hkv > 4096)
    return fail(NEO_ERR_SHAPE, "%s: Hq=%d Hkv=%d out of range", fn, Hq, Hkv);
  if (hidden < 64 || hidden % 64 != 0 || hidden > (1 << 20))
    return fail(NEO_ERR_SHAPE, "%s: hidden=%d must be a positive multiple of 64 (<= 2^20)", fn, hidden);
  if (N < 0 || N > (1 << 30)) return fail(NEO_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (!isfinite(rope_theta) || !isfinite(rope_theta_hw) || rope_theta <= 0.0f || rope_theta_hw <= 0.0f)
    return fail(NEO_ERR_VALUE, "%s: rotary bases must be finite and > 0", fn);
  if (!isfinite(eps) || eps < 0.0f) return fail(NEO_ERR_VALUE, "%s: eps must be finite and >= 0", fn);
  {
    const int64_t heads = (int64_t)Hq + 2 * Hkv;
    if (!grid_fits(neo::gemm_max_blocks(heads * 128, N), neo::kGemmThreads))
      return fail(NEO_ERR_SHAPE, "%s: problem too large for one launch", fn);
  }
  if (N == 0) return ok();
  if (!x || !w_qkv || !q_norm_w || !q_norm_hw_w || !k_norm_w || !k_norm_hw_w || !pos_thw ||
      !q_out || !k_out || !v_out)
    return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  const void* bufs[5] = {x, w_qkv, q_out, k_out, v_out};
  for (const void* p : bufs)
    if (!aligned16(p)) return fail(NEO_ERR_VALUE, "%s: x, w_qkv and outputs must be 16-byte aligned", fn);
  const size_t xb = (size_t)N * hidden * 2, wb = ((size_t)Hq + 2 * Hkv) * 128 * hidden * 2;
  const size_t qb = (size_t)N * Hq * 128 * 2, kb = (size_t)N * Hkv * 128 * 2;
  const void* outs[3] = {q_out, k_out, v_out};
  const size_t osz[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], osz[i], x, xb) || overlap(outs[i], osz[i], w_qkv, wb) ||
        overlap(outs[i], osz[i], pos_thw, (size_t)N * 12))
      return fail(NEO_ERR_VALUE, "%s: an output overlaps an input", fn);
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j]))
        return fail(NEO_ERR_VALUE, "%s: outputs overlap", fn);
  }
  return from_hip(neo::launch_qkv_proj_bf16(x, w_qkv, N, hidden, Hq, Hkv, q_norm_w, q_norm_hw_w,
                                            k_norm_w, k_norm_hw_w, pos_thw, rope_theta,
                                            rope_theta_hw, eps, q_out, k_out, v_out,
                                            static_cast<hipStream_t>(hip_stream)),
                  "neo_qkv_proj_norm_rope launch");
}

neo_status neo_prefill_attn_fwd(const void* q, const void* k, const void* v,
                                const int32_t* temporal_idx, const int32_t* cu_seqlens,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                int64_t total, int32_t max_seqlen, float softmax_scale,
                                void* out, float* lse, neo_dtype dtype, void* hip_stream) {
  const char* fn = "neo_prefill_attn_fwd";
  if (dtype != NEO_F32 && dtype != NEO_BF16)
    return fail(NEO_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (dtype != NEO_BF16)
    return fail(NEO_ERR_UNSUPPORTED, "%s: the understanding pass is bf16 only", fn);
  if (head_dim != NEO_HEAD_DIM)
    return fail(NEO_ERR_SHAPE, "%s: head_dim must be 128, got %d", fn, head_dim);
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(NEO_ERR_SHAPE, "%s: B=%d Hq=%d Hkv=%d must be >= 1", fn, B, Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(NEO_ERR_SHAPE, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (max_seqlen < 0) return fail(NEO_ERR_SHAPE, "%s: negative max_seqlen", fn);
  if (!rows_fit(total, Hq))
    return fail(NEO_ERR_SHAPE, "%s: total=%lld out of range", fn, (long long)total);
  if (max_seqlen > total) return fail(NEO_ERR_SHAPE, "%s: max_seqlen exceeds the tensor's rows", fn);
  if ((int64_t)max_seqlen * Hkv * NEO_HEAD_DIM * 4 >= ((int64_t)1 << 31))
    return fail(NEO_ERR_SHAPE, "%s: one sample's K/V rows exceed 2 GiB", fn);
  if (!isfinite(softmax_scale)) return fail(NEO_ERR_VALUE, "%s: softmax_scale must be finite", fn);
  {
    const int64_t G = Hq / Hkv;
    const int64_t per = ((int64_t)G * ((max_seqlen + 31) / 32) + 7) / 8;
    if (!grid_fits(per * Hkv * B, neo::kAttnBf16Threads))
      return fail(NEO_ERR_SHAPE, "%s: problem too large for one launch", fn);
  }
  if (max_seqlen == 0 || total == 0) return ok();
  if (!q || !k || !v || !temporal_idx || !cu_seqlens || !out)
    return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  const void* bufs[3] = {q, k, v};
  for (const void* p : bufs)
    if (!aligned16(p)) return fail(NEO_ERR_VALUE, "%s: q/k/v buffers must be 16-byte aligned", fn);
  if (!aligned16(out)) return fail(NEO_ERR_VALUE, "%s: out must be 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(temporal_idx) & 3)
    return fail(NEO_ERR_VALUE, "%s: temporal_idx must be 4-byte aligned", fn);
  const size_t ob = (size_t)total * Hq * NEO_HEAD_DIM * 2;
  const size_t kb = (size_t)total * Hkv * NEO_HEAD_DIM * 2;
  const size_t sizes[3] = {ob, kb, kb};
  const size_t lb = lse ? (size_t)total * Hq * sizeof(float) : 0;
  for (int i = 0; i < 3; ++i)
    if (overlap(out, ob, bufs[i], sizes[i]) || (lse && overlap(lse, lb, bufs[i], sizes[i])))
      return fail(NEO_ERR_VALUE, "%s: out/lse overlap an input", fn);
  if (lse && overlap(lse, lb, out, ob)) return fail(NEO_ERR_VALUE, "%s: lse overlaps out", fn);
  if (overlap(out, ob, temporal_idx, (size_t)total * 4) ||
      (lse && overlap(lse, lb, temporal_idx, (size_t)total * 4)))
    return fail(NEO_ERR_VALUE, "%s: out/lse overlap temporal_idx", fn);
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)NEO_HEAD_DIM);
  return from_hip(neo::launch_prefill_attn_bf16(q, k, v, temporal_idx, cu_seqlens, B, Hq, Hkv,
                                                max_seqlen, scale, out, lse, total,
                                                static_cast<hipStream_t>(hip_stream)),
                  "neo_prefill_attn_fwd launch");
}

}  // extern "C"

namespace {

// Weights of the three branches' velocities in the guided velocity.  The full three-branch
// guidance of [B] §2.7, v_u + g (v_c - v_tu) + gi (v_tu - v_u), collects to
//     g v_c + (gi - g) v_tu + (1 - gi) v_u,
// and its other code paths are this sum with a vanishing weight dropped.  The weights
// always sum to one.  Guidance acts only for t strictly between the interval's ends, except
// that an interval starting at 0 keeps it on for the whole trajectory; elsewhere the
// conditional branch alone drives the step.  The differences of two floats are exact in
// double, so a weight is zero exactly when its two scales are equal.
struct CfgWeights {
  double c, tu, u;
};

CfgWeights cfg_weights(float t, float g, float gi, float lo, float hi) {
  const bool on = lo == 0.0f || (lo < t && t < hi);
  if (!on) return {1.0, 0.0, 0.0};
  return {(double)g, (double)gi - (double)g, 1.0 - (double)gi};
}

}  // namespace

extern "C" {

int neo_cfg_path(float t, float cfg_scale, float img_cfg_scale, float cfg_interval_lo,
                 float cfg_interval_hi) {
  // a step runs the conditional forward, plus each other branch whose weight is non-zero
  const CfgWeights w = cfg_weights(t, cfg_scale, img_cfg_scale, cfg_interval_lo, cfg_interval_hi);
  return 1 + (w.tu != 0.0 ? 1 : 0) + (w.u != 0.0 ? 2 : 0);
}

neo_status neo_fm_euler_step_cfg(float* z, const float* x0_cond, const float* x0_text_uncond,
                                 const float* x0_uncond, int64_t n, float t, float t_next,
                                 float t_eps, float cfg_scale, float img_cfg_scale,
                                 float cfg_interval_lo, float cfg_interval_hi,
                                 void* hip_stream) {
  const char* fn = "neo_fm_euler_step_cfg";
  if (n < 0 || n > INT64_MAX / 16) return fail(NEO_ERR_SHAPE, "%s: n=%lld out of range", fn, (long long)n);
  if (!finite(t) || !finite(t_next) || !finite(t_eps))
    return fail(NEO_ERR_VALUE, "%s: t, t_next, t_eps must be finite", fn);
  if (!finite(cfg_scale) || !finite(img_cfg_scale) || !finite(cfg_interval_lo) ||
      !finite(cfg_interval_hi))
    return fail(NEO_ERR_VALUE, "%s: guidance scales and interval must be finite", fn);
  if (t_eps <= 0.0f) return fail(NEO_ERR_VALUE, "%s: t_eps must be > 0", fn);
  if (t_next < t) return fail(NEO_ERR_VALUE, "%s: t_next < t", fn);
  const CfgWeights cw = cfg_weights(t, cfg_scale, img_cfg_scale, cfg_interval_lo, cfg_interval_hi);
  const int path = 1 + (cw.tu != 0.0 ? 1 : 0) + (cw.u != 0.0 ? 2 : 0);
  if (n == 0) return ok();
  // the conditional branch, then every branch with a non-zero weight
  const float* x[3] = {x0_cond, nullptr, nullptr};
  double w[3] = {cw.c, 0.0, 0.0};
  int nb = 1;
  if (cw.tu != 0.0) {
    x[nb] = x0_text_uncond;
    w[nb++] = cw.tu;
  }
  if (cw.u != 0.0) {
    x[nb] = x0_uncond;
    w[nb++] = cw.u;
  }
  if (!z) return fail(NEO_ERR_NULL, "%s: z is NULL", fn);
  for (int b = 0; b < nb; ++b)
    if (!x[b]) return fail(NEO_ERR_NULL, "%s: guidance path %d reads a NULL branch", fn, path);
  const size_t bytes = (size_t)n * sizeof(float);
  uintptr_t bits = reinterpret_cast<uintptr_t>(z);
  for (int b = 0; b < nb; ++b) {
    if (static_cast<const void*>(x[b]) != static_cast<const void*>(z) && overlap(z, bytes, x[b], bytes))
      return fail(NEO_ERR_VALUE, "%s: z and a branch input partially overlap", fn);
    bits |= reinterpret_cast<uintptr_t>(x[b]);
  }
  if (bits & 3) return fail(NEO_ERR_VALUE, "%s: buffers must be 4-byte aligned", fn);
  const double denom = fmax(1.0 - (double)t, (double)t_eps);
  const float coef = (float)(((double)t_next - (double)t) / denom);
  const float wf[3] = {(float)w[0], (float)w[1], (float)w[2]};
  return from_hip(neo::launch_euler_step_cfg(z, x, wf, nb, n, coef, static_cast<hipStream_t>(hip_stream)),
                  "neo_fm_euler_step_cfg launch");
}

// ---- generation-branch embedding front end ---------------------------------------------

namespace {

// H and W positive multiples of m and small enough that every count below fits
bool image_ok(int32_t B, int32_t H, int32_t W, int m) {
  return B >= 0 && B <= (1 << 16) && H >= m && W >= m && H % m == 0 && W % m == 0 &&
         H <= (1 << 15) && W <= (1 << 15);
}

bool all16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return false;
  return true;
}

}  // namespace

neo_status neo_gen_patchify(const float* z, int32_t B, int32_t H, int32_t W, void* patches,
                            void* hip_stream) {
  const char* fn = "neo_gen_patchify";
  if (!image_ok(B, H, W, 16))
    return fail(NEO_ERR_SHAPE, "%s: B=%d H=%d W=%d (H, W positive multiples of 16, <= 32768)", fn, B, H, W);
  if (B == 0) return ok();
  if (!z || !patches) return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!all16({z, patches})) return fail(NEO_ERR_VALUE, "%s: buffers must be 16-byte aligned", fn);
  const size_t zb = (size_t)B * 3 * H * W * 4, pb = (size_t)B * 3 * H * W * 2;
  if (overlap(z, zb, patches, pb)) return fail(NEO_ERR_VALUE, "%s: patches overlap z", fn);
  return from_hip(neo::launch_gen_patchify(z, B, H, W, patches, static_cast<hipStream_t>(hip_stream)),
                  "neo_gen_patchify launch");
}

neo_status neo_gen_patch_embed(const void* patches, int32_t B, int32_t H, int32_t W,
                               const void* w1, const float* b1, int32_t C1, float rope_theta,
                               void* h_out, void* hip_stream) {
  const char* fn = "neo_gen_patch_embed";
  if (!image_ok(B, H, W, 16))
    return fail(NEO_ERR_SHAPE, "%s: B=%d H=%d W=%d (H, W positive multiples of 16, <= 32768)", fn, B, H, W);
  if (C1 < 64 || C1 % 64 != 0 || C1 > 16384)
    return fail(NEO_ERR_SHAPE, "%s: C1=%d must be a positive multiple of 64 (<= 16384)", fn, C1);
  if (!finite(rope_theta) || rope_theta <= 1.0f)
    return fail(NEO_ERR_VALUE, "%s: rope_theta must be finite and > 1", fn);
  const int64_t M = (int64_t)B * (H / 16) * (W / 16);
  if (!grid_fits(neo::gemm_max_blocks(C1, M), neo::kGemmThreads))
    return fail(NEO_ERR_SHAPE, "%s: problem too large for one launch", fn);
  if (M == 0) return ok();
  if (!patches || !w1 || !b1 || !h_out) return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!all16({patches, w1, b1, h_out})) return fail(NEO_ERR_VALUE, "%s: buffers must be 16-byte aligned", fn);
  const size_t hb = (size_t)M * C1 * 2;
  if (overlap(h_out, hb, patches, (size_t)M * 768 * 2) || overlap(h_out, hb, w1, (size_t)C1 * 768 * 2) ||
      overlap(h_out, hb, b1, (size_t)C1 * 4))
    return fail(NEO_ERR_VALUE, "%s: h_out overlaps an input", fn);
  return from_hip(neo::launch_gen_patch_embed(patches, B, H, W, w1, b1, C1, (double)rope_theta, h_out,
                                              static_cast<hipStream_t>(hip_stream)),
                  "neo_gen_patch_embed launch");
}

neo_status neo_gen_patch_embed_px(const float* z, int32_t B, int32_t H, int32_t W,
                                  const void* w1, const float* b1, int32_t C1, float rope_theta,
                                  void* h_out, void* hip_stream) {
  const char* fn = "neo_gen_patch_embed_px";
  if (!image_ok(B, H, W, 16))
    return fail(NEO_ERR_SHAPE, "%s: B=%d H=%d W=%d (H, W positive multiples of 16, <= 32768)", fn, B, H, W);
  if (C1 < 64 || C1 % 64 != 0 || C1 > 16384)
    return fail(NEO_ERR_SHAPE, "%s: C1=%d must be a positive multiple of 64 (<= 16384)", fn, C1);
  if (!finite(rope_theta) || rope_theta <= 1.0f)
    return fail(NEO_ERR_VALUE, "%s: rope_theta must be finite and > 1", fn);
  const int64_t M = (int64_t)B * (H / 16) * (W / 16);
  const int64_t zb = (int64_t)B * 3 * H * W * 4;
  if (zb >= ((int64_t)1 << 31))
    return fail(NEO_ERR_SHAPE, "%s: z is %lld bytes (must be below 2 GiB)", fn, (long long)zb);
  if (!grid_fits(neo::gemm_max_blocks(C1, M), neo::kGemmThreads))
    return fail(NEO_ERR_SHAPE, "%s: problem too large for one launch", fn);
  if (M == 0) return ok();
  if (!z || !w1 || !b1 || !h_out) return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!all16({z, w1, b1, h_out})) return fail(NEO_ERR_VALUE, "%s: buffers must be 16-byte aligned", fn);
  const size_t hb = (size_t)M * C1 * 2;
  if (overlap(h_out, hb, z, (size_t)zb) || overlap(h_out, hb, w1, (size_t)C1 * 768 * 2) ||
      overlap(h_out, hb, b1, (size_t)C1 * 4))
    return fail(NEO_ERR_VALUE, "%s: h_out overlaps an input", fn);
  return from_hip(neo::launch_gen_patch_embed_px(z, B, H, W, w1, b1, C1, (double)rope_theta, h_out,
                                                 static_cast<hipStream_t>(hip_stream)),
                  "neo_gen_patch_embed_px launch");
}

neo_status neo_gen_cond_hidden(float t, float noise_scale, float noise_scale_max, int32_t D,
                               const void* wa_t, const float* ba_t, const void* wa_s,
                               const float* ba_s, float* hidden, void* hip_stream) {
  const char* fn = "neo_gen_cond_hidden";
  if (D < 8 || D % 8 != 0 || D > (1 << 20))
    return fail(NEO_ERR_SHAPE, "%s: D=%d must be a positive multiple of 8 (<= 2^20)", fn, D);
  if (!finite(t) || !finite(noise_scale) || !finite(noise_scale_max) || noise_scale_max <= 0.0f)
    return fail(NEO_ERR_VALUE, "%s: t and the noise scale must be finite, its maximum > 0", fn);
  if (!wa_t || !ba_t || !wa_s || !ba_s || !hidden)
    return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!all16({wa_t, ba_t, wa_s, ba_s, hidden}))
    return fail(NEO_ERR_VALUE, "%s: buffers must be 16-byte aligned", fn);
  const size_t hb = (size_t)2 * D * 4, wab = (size_t)D * 256 * 2, bab = (size_t)D * 4;
  if (overlap(hidden, hb, wa_t, wab) || overlap(hidden, hb, wa_s, wab) ||
      overlap(hidden, hb, ba_t, bab) || overlap(hidden, hb, ba_s, bab))
    return fail(NEO_ERR_VALUE, "%s: hidden overlaps an input", fn);
  const float arg_s = (float)((double)noise_scale / (double)noise_scale_max);
  return from_hip(neo::launch_gen_cond_hidden(t, arg_s, D, wa_t, ba_t, wa_s, ba_s, hidden,
                                              static_cast<hipStream_t>(hip_stream)),
                  "neo_gen_cond_hidden launch");
}

neo_status neo_gen_cond_out(int32_t D, const float* hidden, const void* wb_t, const float* bb_t,
                            const void* wb_s, const float* bb_s, float* cond, void* hip_stream) {
  const char* fn = "neo_gen_cond_out";
  if (D < 8 || D % 8 != 0 || D > (1 << 20))
    return fail(NEO_ERR_SHAPE, "%s: D=%d must be a positive multiple of 8 (<= 2^20)", fn, D);
  if (!hidden || !wb_t || !bb_t || !wb_s || !bb_s || !cond)
    return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!all16({hidden, wb_t, bb_t, wb_s, bb_s, cond}))
    return fail(NEO_ERR_VALUE, "%s: buffers must be 16-byte aligned", fn);
  const size_t cb = (size_t)D * 4, wbb = (size_t)D * D * 2;
  if (overlap(cond, cb, hidden, 2 * cb) || overlap(cond, cb, wb_t, wbb) || overlap(cond, cb, wb_s, wbb) ||
      overlap(cond, cb, bb_t, cb) || overlap(cond, cb, bb_s, cb))
    return fail(NEO_ERR_VALUE, "%s: cond overlaps an input", fn);
  return from_hip(neo::launch_gen_cond_out(D, hidden, wb_t, bb_t, wb_s, bb_s, cond,
                                           static_cast<hipStream_t>(hip_stream)),
                  "neo_gen_cond_out launch");
}

neo_status neo_gen_merge_embed(const void* h, int32_t B, int32_t H, int32_t W, int32_t C1,
                               const void* w2, const float* b2, const float* cond, int32_t D,
                               float* tokens, void* hip_stream) {
  const char* fn = "neo_gen_merge_embed";
  if (!image_ok(B, H, W, 32))
    return fail(NEO_ERR_SHAPE, "%s: B=%d H=%d W=%d (H, W positive multiples of 32, <= 32768)", fn, B, H, W);
  if (C1 < 64 || C1 % 64 != 0 || C1 > 16384)
    return fail(NEO_ERR_SHAPE, "%s: C1=%d must be a positive multiple of 64 (<= 16384)", fn, C1);
  if (D < 32 || D % 32 != 0 || D > (1 << 16))
    return fail(NEO_ERR_SHAPE, "%s: D=%d must be a positive multiple of 32 (<= 65536)", fn, D);
  const int64_t P = (int64_t)(H / 16) * (W / 16), Ntot = (int64_t)B * (H / 32) * (W / 32);
  // the gathered input rows are addressed with 32-bit byte offsets
  if ((int64_t)B * P * C1 * 2 >= ((int64_t)1 << 31))
    return fail(NEO_ERR_SHAPE, "%s: the patch features exceed 2 GiB", fn);
  if (!grid_fits(neo::gemm_max_blocks(D, Ntot), neo::kGemmThreads))
    return fail(NEO_ERR_SHAPE, "%s: problem too large for one launch", fn);
  if (Ntot == 0) return ok();
  if (!h || !w2 || !b2 || !cond || !tokens) return fail(NEO_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!all16({h, w2, b2, cond, tokens})) return fail(NEO_ERR_VALUE, "%s: buffers must be 16-byte aligned", fn);
  const size_t tb = (size_t)Ntot * D * 4;
  if (overlap(tokens, tb, h, (size_t)B * P * C1 * 2) || overlap(tokens, tb, w2, (size_t)D * 4 * C1 * 2) ||
      overlap(tokens, tb, b2, (size_t)D * 4) || overlap(tokens, tb, cond, (size_t)D * 4))
    return fail(NEO_ERR_VALUE, "%s: tokens overlap an input", fn);
  return from_hip(neo::launch_gen_merge_embed(h, B, H, W, C1, w2, b2, cond, D, tokens,
                                              static_cast<hipStream_t>(hip_stream)),
                  "neo_gen_merge_embed launch");
}

double neo_shift_time(double t, double shift) {
  const double sigma = 1.0 - t;
  return 1.0 - shift * sigma / (1.0 + (shift - 1.0) * sigma);
}

}  // extern "C"
