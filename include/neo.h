/*
 * neo.h -- C ABI of the NEO-unify generation-pass attention block for MI355X
 * (gfx950).
 *
 * Pages cited:
 *   [A] "SenseNova-U1.5 (NEO-unify) architecture" (Mobius design note)
 *   [B] "SenseNova-U1: Unifying Multimodal Understanding and Generation with
 *        NEO-unify Architecture" (paper notes)
 *
 * The generation pass runs once per flow-matching step: the noisy image tokens,
 * already projected with the generation-branch weights, get split-half
 * QK-RMSNorm and three-axis rotary ([A] §Three rotary axes), then the image
 * queries attend, unmasked and without writing the cache, over the frozen
 * understanding-branch K/V prefix followed by the image block's own K/V
 * ([A] §Mixture of Transformers; §GQA fusion does not apply).  The sampler
 * turns the predicted clean image into a velocity and takes one Euler step
 * ([A] §Flow matching without a VAE).
 *
 * Conventions for every entry point:
 *   - Plain C: no C++ types, no HIP headers are needed to include this file.
 *   - Device pointers are HIP device (or managed) memory on the current
 *     device; the caller owns every buffer.  The library allocates nothing,
 *     keeps no state besides a thread-local error message, and never
 *     synchronises: work is enqueued on `hip_stream` (a hipStream_t; NULL is
 *     the null stream) and outputs are valid once that stream is synchronised.
 *   - Layouts are token-major and contiguous: a [T, H, 128] tensor has row
 *     (t, h) at element offset (t*H + h)*128 ([B] §4.4 KV cache reuse: the
 *     cache is kept as [B, S, H, D], flattened here over the ragged batch).
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns a non-zero neo_status and launches nothing.  neo_last_error()
 *     then describes the failure for the calling thread.
 *   - Only the generation pass is served.  Anything outside it (a mask, a
 *     cache update, another head size) is rejected with NEO_ERR_UNSUPPORTED,
 *     as the upstream code refuses mixed understanding/generation calls
 *     ([A] §Mixture of Transformers).
 */
#ifndef NEO_H
#define NEO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NEO_OK = 0,
    NEO_ERR_NULL = 1,        /* a required pointer is NULL                     */
    NEO_ERR_SHAPE = 2,       /* a size or count is out of range               */
    NEO_ERR_VALUE = 3,       /* a scalar is non-finite or out of its domain   */
    NEO_ERR_UNSUPPORTED = 4, /* outside the generation-pass contract          */
    NEO_ERR_HIP = 5          /* the HIP runtime reported an error at launch   */
} neo_status;

typedef enum {
    NEO_F32 = 0,  /* IEEE binary32                                            */
    NEO_BF16 = 1  /* bfloat16 (upper half of binary32), round-to-nearest-even */
} neo_dtype;

#define NEO_HEAD_DIM 128

/*
 * neo_qknorm_rope3 -- split-half QK-RMSNorm then three-axis rotary on the
 * generation block's queries and keys.
 *
 * Defined by [A] §Three rotary axes: each 128-dim head row is normalised as two
 * independent 64-dim halves, y = x / sqrt(mean(x^2) + eps) * w, with w =
 * q_norm_w (k_norm_w) on dims [0:64) and q_norm_hw_w (k_norm_hw_w) on dims
 * [64:128).  The row is then rotated per slice:
 *     dims [0:64)   by pos_thw[0][t] with base rope_theta     (temporal),
 *     dims [64:96)  by pos_thw[1][t] with base rope_theta_hw  (height),
 *     dims [96:128) by pos_thw[2][t] with base rope_theta_hw  (width),
 * pairing element o+i with o+i+w/2 inside a slice of width w (half-split, as
 * [A] §Vision tower says of the language backbone) at angle
 * pos * base^(-2i/w).  All image tokens of one image carry the same temporal
 * index, the text length ([A] §Three rotary axes).
 *
 *   q_in   [T, Hq, 128]  dtype; device; read.
 *   k_in   [T, Hkv, 128] dtype; device; read.
 *   q_out  [T, Hq, 128]  dtype; device; written.  May equal q_in (in place).
 *   k_out  [T, Hkv, 128] dtype; device; written.  May equal k_in (in place).
 *          Partial overlap of an input and an output is not allowed.
 *   T      tokens, >= 0 (0 is a no-op).  Hq, Hkv >= 1.  head_dim == 128.
 *   q_norm_w, q_norm_hw_w, k_norm_w, k_norm_hw_w   [64] fp32, device.
 *   pos_thw  [3, T] int32, device: temporal, height, width rows.
 *   rope_theta, rope_theta_hw  > 0 and finite (the pages: 5e6 and 1e4).
 *   eps    >= 0 and finite (1e-6 in the workloads).
 *   Arithmetic is fp32; a bf16 output is rounded once, after the rotary.
 */
neo_status neo_qknorm_rope3(const void *q_in, const void *k_in, void *q_out, void *k_out,
                            int64_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                            const float *q_norm_w, const float *q_norm_hw_w,
                            const float *k_norm_w, const float *k_norm_hw_w,
                            const int32_t *pos_thw, float rope_theta, float rope_theta_hw,
                            float eps, neo_dtype dtype, void *hip_stream);

/*
 * neo_gen_attn_fwd -- generation-pass attention of the image queries over
 * [frozen prefix ; image block], no mask, no cache write.
 *
 * Defined by [A] §Mixture of Transformers (the generation branch only reads
 * the cache that the understanding branch filled; it is called with
 * update_cache=False) and §GQA fusion does not apply (the generation graph
 * takes no attention mask at all).  For sample b,
 * query row i in [cu_seqlens_q[b], cu_seqlens_q[b+1]) and query head h, with
 * g = h / (Hq / Hkv):
 *     keys    = k_prefix rows [cu_seqlens_prefix[b], cu_seqlens_prefix[b+1])
 *               followed by k_img rows [cu_seqlens_q[b], cu_seqlens_q[b+1]),
 *     out[i,h] = sum_j softmax_j(softmax_scale * <q[i,h], key_j[g]>) value_j[g],
 *     lse[h,i] = log sum_j exp(softmax_scale * <q[i,h], key_j[g]>).
 *
 *   q        [Tq, Hq, 128]  dtype, device: queries after norm and rotary.
 *   k_img    [Tq, Hkv, 128] dtype, device: the image block's keys (rotated).
 *   v_img    [Tq, Hkv, 128] dtype, device.
 *   k_prefix [Tp, Hkv, 128] dtype, device: the frozen cache, already rotated.
 *   v_prefix [Tp, Hkv, 128] dtype, device.  With Tp == 0 both may be NULL.
 *   cu_seqlens_q      [B+1] int32, device: 0 = c[0] <= c[1] <= ... = Tq.
 *   cu_seqlens_prefix [B+1] int32, device: 0 = c[0] <= ... = Tp.
 *   B >= 1.  Hq, Hkv >= 1 with Hq % Hkv == 0.  head_dim == 128.
 *   total_q (Tq), total_prefix (Tp) >= 0: row counts of the tensors above, on
 *     the host.  The kernels clamp every cu_seqlens entry into [0, Tq] and
 *     [0, Tp], so malformed offsets give wrong numbers, never a stray access.
 *   max_seqlen_q, max_seqlen_prefix: host-side upper bounds of the per-sample
 *     lengths (no device-to-host copy is made), at most total_q and total_prefix
 *     (NEO_ERR_SHAPE otherwise); they size the launch grid and
 *     must not be below the true maxima (a precondition, as in varlen flash
 *     attention: rows and keys beyond the bound are not computed).  One
 *     sample's K or V rows must span less than 2 GiB (max_seqlen * Hkv * 256 B
 *     for bf16, checked at the fp32 size).
 *   softmax_scale: <= 0 selects 1/sqrt(head_dim); otherwise finite.
 *   out      [Tq, Hq, 128] dtype, device: written.  Must not overlap inputs.
 *   lse      [Hq, Tq] fp32, device, natural log, or NULL to skip.
 *   A sample with no keys (P_b + N_b == 0) has no queries either, so no
 *   output row is ever left undefined.
 */
neo_status neo_gen_attn_fwd(const void *q, const void *k_img, const void *v_img,
                            const void *k_prefix, const void *v_prefix,
                            const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_prefix,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                            int64_t total_q, int64_t total_prefix,
                            int32_t max_seqlen_q, int32_t max_seqlen_prefix,
                            float softmax_scale, void *out, float *lse, neo_dtype dtype,
                            void *hip_stream);

/*
 * neo_fm_euler_step -- x0-prediction to velocity and one Euler step of the
 * pixel-space rectified flow, in place:
 *     v = (x0_pred - z) / max(1 - t, t_eps);   z <- z + (t_next - t) * v
 * ([A] §Flow matching without a VAE and §Runtime / metadata status; [B] §2.7).
 * Cutting the image into patches only reorders its elements, so the update is
 * the same elementwise map on any layout.
 *
 *   z        [n] fp32, device: read and written.
 *   x0_pred  [n] fp32, device: read.  May not partially overlap z.
 *   n >= 0 (0 is a no-op).
 *   t, t_next finite with t <= t_next; t_eps > 0 and finite (0.02: the example
 *   scripts keep the function default and never read the config's 0.05, [A]
 *   §Dead or misleading upstream details).
 *   Arithmetic is fp32: z + c*(x0_pred - z) with c = (t_next - t)/max(1-t, t_eps)
 *   formed once in double on the host.
 */
neo_status neo_fm_euler_step(float *z, const float *x0_pred, int64_t n, float t, float t_next,
                             float t_eps, void *hip_stream);

/*
 * neo_qkv_proj_norm_rope -- the generation branch's q/k/v projection of the
 * noisy image tokens fused with the q/k prologue ([A] §Mixture of Transformers:
 * the `_mot_gen` q/k/v projections and q/k norms; §Three rotary axes):
 *     [q | k | v] = x w_qkv^T,  then q, k <- split-half RMSNorm + three-axis
 *     rotary exactly as neo_qknorm_rope3 does,
 * with the projection kept in fp32 on chip (no intermediate rounding) and one
 * rounding to bf16 at the store.
 *
 *   x         [N, hidden] bf16 (the image tokens' hidden states), 16-byte aligned.
 *   w_qkv     [(Hq + 2 Hkv) * 128, hidden] bf16: rows are the Hq query heads,
 *             then the Hkv key heads, then the Hkv value heads (the three
 *             projection matrices stacked; bf16 copies of the branch's weights).
 *   hidden    a positive multiple of 64 (<= 2^20); head_dim must be 128.
 *   q_norm_w, q_norm_hw_w, k_norm_w, k_norm_hw_w  [64] fp32 each.
 *   pos_thw   [3, N] int32 temporal / height / width indices.
 *   rope_theta, rope_theta_hw, eps   as for neo_qknorm_rope3.
 *   q_out [N, Hq, 128], k_out [N, Hkv, 128], v_out [N, Hkv, 128] bf16; may not
 *   overlap any input or each other.
 *   dtype     NEO_BF16 only.
 * Errors: NEO_ERR_SHAPE, NEO_ERR_VALUE, NEO_ERR_NULL, NEO_ERR_UNSUPPORTED, NEO_ERR_HIP.
 */
neo_status neo_qkv_proj_norm_rope(const void *x, const void *w_qkv, int64_t N, int32_t hidden,
                                  int32_t Hq, int32_t Hkv, int32_t head_dim,
                                  const float *q_norm_w, const float *q_norm_hw_w,
                                  const float *k_norm_w, const float *k_norm_hw_w,
                                  const int32_t *pos_thw, float rope_theta, float rope_theta_hw,
                                  float eps, void *q_out, void *k_out, void *v_out,
                                  neo_dtype dtype, void *hip_stream);

/*
 * neo_prefill_attn_fwd -- understanding-pass (prefill) attention with the
 * block-causal mask ([A] §Block-causal attention; [B] §2.5, Fig. 6).  Within
 * each sample, query i attends key j when temporal_idx[j] == temporal_idx[i]
 * or j <= i: tokens sharing a temporal index (one image) see each other both
 * ways, and across different indices the mask is causal.  This produces the
 * frozen K/V prefix's attention outputs; Q, K and V all come from the same
 * sequence (already normed and rotated).
 *
 *   q             [T, Hq, 128] bf16; k, v [T, Hkv, 128] bf16; 16-byte aligned.
 *   temporal_idx  [T] int32, device: each token's temporal index (the first
 *                 rotary axis).  Precondition, not checked: within a sample the
 *                 indices are non-decreasing and tokens sharing an index are
 *                 contiguous, as in every layout the pages describe (text
 *                 tokens count up; an image's tokens share one index).  When
 *                 it is broken the outputs are wrong, but every read stays
 *                 within the sample's rows.
 *   cu_seqlens    [B+1] int32, device: sample s is rows [cu[s], cu[s+1]).
 *   max_seqlen    host-side bound on the sample lengths, at most T (NEO_ERR_SHAPE
 *                 otherwise); total = T.
 *   softmax_scale <= 0 means 1/sqrt(128).
 *   out           [T, Hq, 128] bf16; lse optional [Hq, T] fp32 (natural log).
 *   dtype         NEO_BF16 only (the understanding branch is bf16, [A]
 *                 §Numeric precision); NEO_F32 -> NEO_ERR_UNSUPPORTED.
 * Errors as for neo_gen_attn_fwd; out and lse may not overlap any input.
 */
neo_status neo_prefill_attn_fwd(const void *q, const void *k, const void *v,
                                const int32_t *temporal_idx, const int32_t *cu_seqlens,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                int64_t total, int32_t max_seqlen, float softmax_scale,
                                void *out, float *lse, neo_dtype dtype, void *hip_stream);

/*
 * neo_cfg_path -- which branch forwards a guided flow step needs ([B] §2.7,
 * three-branch guidance).  Written per branch, the guided velocity is
 *     w_c v_c + w_tu v_tu + w_u v_u,
 *     w_c = cfg_scale, w_tu = img_cfg_scale - cfg_scale, w_u = 1 - img_cfg_scale,
 * while guidance is active: for cfg_interval_lo < t < cfg_interval_hi, and for
 * every t when cfg_interval_lo == 0.  Outside it the conditional velocity is
 * used alone (w = 1, 0, 0).  The conditional forward always runs; each other
 * branch runs when its weight is non-zero (scales compared exactly).  Returns
 *   1  conditional only              (w_tu = w_u = 0)
 *   2  plus text-uncond              (w_u = 0: img_cfg_scale == 1)
 *   3  plus full uncond              (w_tu = 0: equal scales)
 *   4  all three branches
 * Pure host function.
 */
int neo_cfg_path(float t, float cfg_scale, float img_cfg_scale, float cfg_interval_lo,
                 float cfg_interval_hi);

/*
 * neo_fm_euler_step_cfg -- classifier-free guidance over the branches' x0
 * predictions fused with the x0-to-velocity Euler step, in place, one pass
 * over the pixels ([B] §2.7: three-branch guidance; [A] §Flow matching without
 * a VAE and §Runtime / metadata status: each branch predicts x0 for the same z
 * from its own frozen prefix).  With v_b = (x0_b - z) / max(1 - t, t_eps) and
 * the weights w_b of neo_cfg_path,
 *     v = sum_b w_b v_b   over the branches with a non-zero weight,
 * and z <- z + (t_next - t) v.  The weights sum to one, so the library forms
 * the guided x0 with them and takes one Euler step: z + c*(sum_b w_b x0_b - z),
 * c and the weights computed once in double on the host, the pass in fp32.
 *
 *   z               [n] fp32, device: read and written.
 *   x0_cond         [n] fp32, device: the conditional branch; always read.
 *   x0_text_uncond  [n] fp32, device: read on paths 2 and 4, else may be NULL.
 *   x0_uncond       [n] fp32, device: read on paths 3 and 4, else may be NULL.
 *   The x0 inputs may alias one another or be exactly z; none may partially
 *   overlap z.  All 4-byte aligned (16-byte alignment takes the vector path).
 *   n >= 0 (0 is a no-op).  t, t_next finite, t <= t_next; t_eps > 0;
 *   cfg_scale, img_cfg_scale and the interval bounds finite.
 * Errors: NEO_ERR_SHAPE (n), NEO_ERR_VALUE (scalars, overlap, alignment),
 * NEO_ERR_NULL (a branch the path reads is NULL), NEO_ERR_HIP (launch).
 */
neo_status neo_fm_euler_step_cfg(float *z, const float *x0_cond, const float *x0_text_uncond,
                                 const float *x0_uncond, int64_t n, float t, float t_next,
                                 float t_eps, float cfg_scale, float img_cfg_scale,
                                 float cfg_interval_lo, float cfg_interval_hi, void *hip_stream);

/* Static English text for a status code; never NULL. */
const char *neo_status_string(neo_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *neo_last_error(void);

/* ---- generation-branch embedding front end -------------------------------------
 *
 * Noisy pixels -> image-token embeddings, in four calls ([A] §Vision tower -- no
 * transformer blocks; [B] §2.1, NEOVisionEmbeddings):
 *   neo_gen_patchify      z -> 16x16 patch rows (bf16);
 *   neo_gen_patch_embed   patch convolution + bias, GELU, interleaved two-axis rotary;
 *   neo_gen_patch_embed_px  the two above in one launch, from the pixels;
 *   neo_gen_cond_hidden / neo_gen_cond_out   the time and noise-scale embedders ([A]
 *                         §Timestep and noise-scale conditioning), summed;
 *   neo_gen_merge_embed   2x2 stride-2 convolution + bias + the conditioning vector.
 * Every intermediate is a caller buffer.  Convolution weights are bf16 (products in
 * fp32), the embedder weights bf16, biases and vectors fp32.  Grids are row-major:
 * patch (py, px) of image b is row b*P + py*(W/16) + px with P = (H/16)*(W/16); token
 * (ty, tx) of image b is row b*(H/32)*(W/32) + ty*(W/32) + tx.  Every buffer is
 * 16-byte aligned; outputs may not overlap inputs.
 * Errors: NEO_ERR_SHAPE, NEO_ERR_VALUE, NEO_ERR_NULL, NEO_ERR_HIP.
 */

/*
 * neo_gen_patchify -- the patch rearrangement of the noisy image ([A] §Flow
 * matching without a VAE: patchify is a permutation), rounded to bf16 for the
 * matrix cores.
 *   z        [B, 3, H, W] fp32; H, W positive multiples of 16 (<= 32768).
 *   patches  [B*P, 768] bf16: row = one 16x16 patch ordered (channel, ky, kx),
 *            the order of a flattened [out, 3, 16, 16] convolution weight.
 */
neo_status neo_gen_patchify(const float *z, int32_t B, int32_t H, int32_t W, void *patches,
                            void *hip_stream);

/*
 * neo_gen_patch_embed -- Conv2d(3, C1, kernel 16, stride 16) + bias, GELU
 * (x * Phi(x), erf form), then the interleaved two-axis rotary of [A] §Vision
 * tower: channels (2i, 2i+1) of the first C1/2 turn by the patch's column
 * index px, those of the last C1/2 by its row index py, pair i of a half by
 * position * rope_theta^(-2i/(C1/2)) (base 1e4 upstream).
 *   patches  [B*P, 768] bf16 (neo_gen_patchify's output).
 *   w1       [C1, 768] bf16: a [C1, 3, 16, 16] convolution weight, flattened.
 *   b1       [C1] fp32.   C1: a positive multiple of 64 (<= 16384).
 *   h_out    [B*P, C1] bf16, the rotated features.
 */
neo_status neo_gen_patch_embed(const void *patches, int32_t B, int32_t H, int32_t W,
                               const void *w1, const float *b1, int32_t C1, float rope_theta,
                               void *h_out, void *hip_stream);

/*
 * neo_gen_patch_embed_px -- neo_gen_patchify and neo_gen_patch_embed in one launch:
 * the same patch convolution, GELU and rotary ([A] §Vision tower), with the patch
 * rows gathered straight from the pixels and rounded to bf16 (RNE) on their way to
 * the matrix cores, so no patch buffer passes through memory.  The result is
 * bit-identical to the two calls.
 *   z        [B, 3, H, W] fp32; H, W positive multiples of 16 (<= 32768); the whole
 *            of z below 2 GiB.
 *   w1, b1, C1, rope_theta, h_out as for neo_gen_patch_embed.
 */
neo_status neo_gen_patch_embed_px(const float *z, int32_t B, int32_t H, int32_t W,
                                  const void *w1, const float *b1, int32_t C1, float rope_theta,
                                  void *h_out, void *hip_stream);

/*
 * neo_gen_cond_hidden -- first layer of the time and noise-scale embedders:
 *   hidden[0] = silu(wa_t e(t) + ba_t),
 *   hidden[1] = silu(wa_s e(noise_scale / noise_scale_max) + ba_s),
 * e(x) the 256-wide sinusoid basis [cos(x f_k), sin(x f_k)], f_k =
 * 10000^(-k/128), k < 128, cosines first ([A] §Timestep and noise-scale
 * conditioning).
 *   wa_t, wa_s  [D, 256] bf16;  ba_t, ba_s [D] fp32;  D a positive multiple of 8.
 *   hidden      [2, D] fp32.
 */
neo_status neo_gen_cond_hidden(float t, float noise_scale, float noise_scale_max, int32_t D,
                               const void *wa_t, const float *ba_t, const void *wa_s,
                               const float *ba_s, float *hidden, void *hip_stream);

/*
 * neo_gen_cond_out -- second layer of both embedders, summed: the vector added
 * to every image token,
 *   cond = wb_t hidden[0] + bb_t + wb_s hidden[1] + bb_s.
 *   hidden [2, D] fp32 (neo_gen_cond_hidden's output); wb_t, wb_s [D, D] bf16;
 *   bb_t, bb_s [D] fp32;  cond [D] fp32.
 */
neo_status neo_gen_cond_out(int32_t D, const float *hidden, const void *wb_t, const float *bb_t,
                            const void *wb_s, const float *bb_s, float *cond, void *hip_stream);

/*
 * neo_gen_merge_embed -- Conv2d(C1, D, kernel 2, stride 2) + bias over the
 * rotated patch features, plus the conditioning vector: the image-token
 * embeddings ([A] §Vision tower's 2x2 merge into the backbone width, one token
 * per 32x32 pixels; §Timestep and noise-scale conditioning).
 *   h       [B*P, C1] bf16 (neo_gen_patch_embed's output); H, W positive
 *           multiples of 32; B*P*C1*2 bytes below 2 GiB.
 *   w2      [D, 2, 2, C1] bf16: a [D, C1, 2, 2] convolution weight with its
 *           axes ordered (out, ky, kx, in), so that each window cell's C1
 *           inputs are contiguous.
 *   b2, cond [D] fp32;  D a positive multiple of 32 (<= 65536).
 *   tokens  [B*(H/32)*(W/32), D] fp32.
 */
neo_status neo_gen_merge_embed(const void *h, int32_t B, int32_t H, int32_t W, int32_t C1,
                               const void *w2, const float *b2, const float *cond, int32_t D,
                               float *tokens, void *hip_stream);

/*
 * neo_shift_time -- the time-grid shift of [A] §Timestep schedule (host only):
 *   sigma = 1 - t;  sigma <- shift sigma / (1 + (shift - 1) sigma);  returns 1 - sigma.
 */
double neo_shift_time(double t, double shift);

#ifdef __cplusplus
}
#endif

#endif /* NEO_H */
