/*
 * fp64 CPU oracle for the NEO-unify generation-pass attention block.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the HIP library links, includes or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It is written to be read against the pages, not to
 * be fast: every step is the plain definition, in fp64, in the pages' order.
 *
 * Sources (cited by page title and section):
 *   [A] "SenseNova-U1.5 (NEO-unify) architecture" (Mobius design note)
 *   [B] "SenseNova-U1: Unifying Multimodal Understanding and Generation with
 *        NEO-unify Architecture" (paper notes)
 *
 * Readings taken where the pages are silent (each one is also listed with its
 * reason in the design notes):
 *   - rotary pairs are half-split inside each slice: (o+i, o+i+w/2);
 *   - the rotary frequency of pair i in a slice of width w is base^(-2i/w);
 *   - RMSNorm is x * 1/sqrt(mean(x^2) + eps) * weight over each 64-dim half;
 *   - softmax scale is 1/sqrt(head_dim); query head h reads KV head h / G with
 *     G = Hq / Hkv (contiguous groups).
 *
 * Pins: every function is checked by the CPU tests against closed forms,
 * special cases and invariants (see tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HEAD_DIM 128
#define HALF_DIM 64

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count for the parallel loops that follow (n >= 1); timing only. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Split-half QK-RMSNorm, [A] §Three rotary axes (last paragraph): dims [0:64)
 * of every head row are normalised with the temporal-half weight (q_norm /
 * k_norm, shape [64]) and dims [64:128) with the spatial-half weight
 * (q_norm_hw / k_norm_hw, shape [64]), each half on its own statistics.
 * x, y: [rows, 128]; y may equal x.
 */
void oracle_split_rmsnorm(const double *x, double *y, int64_t rows,
                          const double *w_t, const double *w_hw, double eps)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * HEAD_DIM;
        double *yr = y + r * HEAD_DIM;
        for (int half = 0; half < 2; ++half) {
            const double *w = half == 0 ? w_t : w_hw;
            double sumsq = 0.0;
            for (int d = 0; d < HALF_DIM; ++d) {
                double v = xr[half * HALF_DIM + d];
                sumsq += v * v;
            }
            double rms = sqrt(sumsq / HALF_DIM + eps);
            for (int d = 0; d < HALF_DIM; ++d)
                yr[half * HALF_DIM + d] = (xr[half * HALF_DIM + d] / rms) * w[d];
        }
    }
}

/*
 * Three-axis rotary embedding, [A] §Three rotary axes (slice table):
 *   [0:64)   temporal axis, base rope_theta,    position row 0
 *   [64:96)  height axis,   base rope_theta_hw, position row 1
 *   [96:128) width axis,    base rope_theta_hw, position row 2
 * Each slice is rotated on its own, half-split ([A] §Vision tower contrasts
 * the vision tower's interleaved pairs with the backbone's half-split ones;
 * [A] §GQA fusion describes three independent axes built from Slice/Mul/Add).
 * y: [T, H, 128] rotated in place; pos: [3, T].
 */
void oracle_rope3(double *y, int64_t T, int64_t H, const int32_t *pos,
                  double theta, double theta_hw)
{
    const int offset[3] = {0, 64, 96};
    const int width[3] = {64, 32, 32};
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double *row = y + (t * H + h) * HEAD_DIM;
            for (int axis = 0; axis < 3; ++axis) {
                double base = axis == 0 ? theta : theta_hw;
                double p = (double)pos[axis * T + t];
                int o = offset[axis], w = width[axis], half = w / 2;
                for (int i = 0; i < half; ++i) {
                    double freq = pow(base, -2.0 * (double)i / (double)w);
                    double phi = p * freq;
                    double c = cos(phi), s = sin(phi);
                    double a = row[o + i];
                    double b = row[o + i + half];
                    row[o + i] = a * c - b * s;
                    row[o + i + half] = b * c + a * s;
                }
            }
        }
    }
}

/*
 * Norm then rotary for one tensor of head rows [T, H, 128]: the step the
 * generation pass applies to the projected queries and to the image block's
 * keys ([A] §Mixture of Transformers weight list; §Three rotary axes).
 */
void oracle_norm_rope(const double *x, double *y, int64_t T, int64_t H,
                      const double *w_t, const double *w_hw, const int32_t *pos,
                      double theta, double theta_hw, double eps)
{
    oracle_split_rmsnorm(x, y, T * H, w_t, w_hw, eps);
    oracle_rope3(y, T, H, pos, theta, theta_hw);
}

/*
 * Generation-pass attention, [A] §Mixture of Transformers (the generation pass
 * reads, and does not update, the frozen understanding-branch cache) and
 * §GQA fusion does not apply (the generation graph takes no attention mask).
 *
 * For sample b, image query i (global row cu_q[b] + i) and query head h,
 * the key/value set is the prefix rows [cu_p[b], cu_p[b+1]) of k_pre/v_pre
 * followed by the image rows [cu_q[b], cu_q[b+1]) of k_img/v_img, all on KV
 * head g = h / (Hq / Hkv):
 *   s_j = scale * <q_ih, k_jg>,  m = max_j s_j,  e_j = exp(s_j - m)
 *   O_ih = sum_j e_j v_jg / sum_j e_j,  lse_ih = m + log(sum_j e_j)
 *
 * tokens: the global query rows to evaluate (ntok of them), or NULL for all
 * Tq = cu_q[B] rows in order.  out: [ntok, Hq, D]; lse: [ntok, Hq] or NULL.
 */
void oracle_gen_attn(const double *q, const double *k_img, const double *v_img,
                     const double *k_pre, const double *v_pre,
                     const int32_t *cu_q, const int32_t *cu_p,
                     int32_t B, int32_t Hq, int32_t Hkv, int32_t D, double scale,
                     const int64_t *tokens, int64_t ntok, double *out, double *lse)
{
    const int32_t G = Hq / Hkv;
    int64_t n = tokens ? ntok : (int64_t)cu_q[B];
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t job = 0; job < n * Hq; ++job) {
        int64_t r = job / Hq;
        int32_t h = (int32_t)(job % Hq);
        int64_t tok = tokens ? tokens[r] : r;
        int32_t b = 0;
        while (b + 1 < B && tok >= cu_q[b + 1])
            ++b;
        int64_t p0 = cu_p[b], np_ = cu_p[b + 1] - cu_p[b];
        int64_t i0 = cu_q[b], ni = cu_q[b + 1] - cu_q[b];
        int64_t nk = np_ + ni;
        int32_t g = h / G;
        const double *qr = q + (tok * Hq + h) * D;
        double *s = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double m = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
            const double *kr = j < np_ ? k_pre + ((p0 + j) * Hkv + g) * D
                                       : k_img + ((i0 + j - np_) * Hkv + g) * D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += qr[d] * kr[d];
            s[j] = scale * dot;
            if (s[j] > m)
                m = s[j];
        }
        double denom = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            s[j] = exp(s[j] - m);
            denom += s[j];
        }
        double *o = out + (r * Hq + h) * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            const double *vr = j < np_ ? v_pre + ((p0 + j) * Hkv + g) * D
                                       : v_img + ((i0 + j - np_) * Hkv + g) * D;
            for (int d = 0; d < D; ++d)
                o[d] += s[j] * vr[d];
        }
        for (int d = 0; d < D; ++d)
            o[d] /= denom;
        if (lse)
            lse[r * Hq + h] = m + log(denom);
        free(s);
    }
}

/*
 * x0-prediction to velocity and one Euler step, [A] §Flow matching without a
 * VAE and §Runtime / metadata status; [B] §2.7 (the Euler update in the main
 * loop):  v = (x0 - z) / max(1 - t, t_eps);  z <- z + (t_next - t) * v.
 * Elementwise, so it holds on patches or on the pixel grid alike.
 */
void oracle_euler_step(double *z, const double *x0, int64_t n,
                       double t, double t_next, double t_eps)
{
    double denom = fmax(1.0 - t, t_eps);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = (x0[i] - z[i]) / denom;
        z[i] = z[i] + (t_next - t) * v;
    }
}

/*
 * Guidance weights, [B] §2.7 (three-branch guidance over the cond, text-uncond
 * and full-uncond forwards).  Its full form
 *     v = v_u + gamma (v_c - v_tu) + gamma_img (v_tu - v_u)
 * is, collected per branch,
 *     v = gamma v_c + (gamma_img - gamma) v_tu + (1 - gamma_img) v_u,
 * and the page's cheaper code paths are exactly this sum with the branches of
 * zero weight left out.  Guidance acts for t strictly inside (lo, hi), and for
 * every t when lo is 0; otherwise the cond velocity is used alone.
 */
static void cfg_weights(double t, double gamma, double gamma_img, double lo, double hi,
                        double w[3])
{
    int active = lo == 0.0 || (lo < t && t < hi);
    w[0] = active ? gamma : 1.0;
    w[1] = active ? gamma_img - gamma : 0.0;
    w[2] = active ? 1.0 - gamma_img : 0.0;
}

/*
 * Which forwards a step needs: the cond branch always, each other branch when
 * its weight is non-zero.  1 = cond only, 2 = + text-uncond, 3 = + full uncond,
 * 4 = all three.
 */
int oracle_cfg_path(double t, double gamma, double gamma_img, double lo, double hi)
{
    double w[3];
    cfg_weights(t, gamma, gamma_img, lo, hi, w);
    return 1 + (w[1] != 0.0) + 2 * (w[2] != 0.0);
}

/*
 * Classifier-free guidance over the conditioning branches, then one Euler step:
 * [B] §2.7 (one forward per needed KV cache and step, combined by the
 * three-branch guidance above) and [A] §Flow matching without a VAE (each
 * branch's head predicts x0, which the sampler turns into a velocity for the
 * shared z).  Per element: each needed branch's velocity
 * v_b = (x0_b - z) / max(1 - t, t_eps), the guided velocity
 * v = sum_b w_b v_b over the branches of non-zero weight, and
 * z <- z + (t_next - t) v.  Branch inputs of zero weight may be NULL.
 */
void oracle_euler_step_cfg(double *z, const double *x0_c, const double *x0_tu,
                           const double *x0_u, int64_t n, double t, double t_next,
                           double t_eps, double gamma, double gamma_img, double lo,
                           double hi)
{
    double denom = fmax(1.0 - t, t_eps);
    double w[3];
    cfg_weights(t, gamma, gamma_img, lo, hi, w);
    const double *x0[3] = {x0_c, x0_tu, x0_u};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = w[0] * ((x0[0][i] - z[i]) / denom);
        for (int br = 1; br < 3; ++br)
            if (w[br] != 0.0)
                v += w[br] * ((x0[br][i] - z[i]) / denom);
        z[i] = z[i] + (t_next - t) * v;
    }
}

/*
 * Understanding-pass (prefill) attention with the block-causal mask,
 * [A] §Block-causal attention: within one sample, query i may attend key j
 * when their temporal indices are equal or j <= i, i.e.
 *     allowed(i, j) = (idx[j] == idx[i]) || (j <= i),
 * evaluated literally for every pair (tokens sharing an index see each other
 * both ways; across different indices the mask is causal).  Q, K and V all
 * come from the same sequence; ragged samples by cu[B+1]; query head h reads
 * KV head h / (Hq / Hkv); scale multiplies q.k.  Softmax in two passes (max,
 * then exp and sum) over the allowed keys only.  Optional `tokens` selects
 * global query rows.
 */
void oracle_prefill_attn(const double *q, const double *k, const double *v,
                         const int32_t *idx, const int32_t *cu, int32_t B, int32_t Hq,
                         int32_t Hkv, int32_t D, double scale, const int64_t *tokens,
                         int64_t ntok, double *out, double *lse)
{
    const int32_t G = Hq / Hkv;
    int64_t n = tokens ? ntok : (int64_t)cu[B];
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t job = 0; job < n * Hq; ++job) {
        int64_t r = job / Hq;
        int32_t h = (int32_t)(job % Hq);
        int64_t tok = tokens ? tokens[r] : r;
        int32_t b = 0;
        while (b + 1 < B && tok >= cu[b + 1])
            ++b;
        int64_t s0 = cu[b], ns = cu[b + 1] - cu[b];
        int64_t i = tok - s0; /* position inside the sample */
        int32_t g = h / G;
        const double *qr = q + (tok * Hq + h) * D;
        double *s = (double *)malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1));
        double m = -INFINITY;
        for (int64_t j = 0; j < ns; ++j) {
            int allowed = idx[s0 + j] == idx[s0 + i] || j <= i;
            if (!allowed) {
                s[j] = -INFINITY;
                continue;
            }
            const double *kr = k + ((s0 + j) * Hkv + g) * D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += qr[d] * kr[d];
            s[j] = scale * dot;
            if (s[j] > m)
                m = s[j];
        }
        double denom = 0.0;
        for (int64_t j = 0; j < ns; ++j) {
            s[j] = s[j] == -INFINITY ? 0.0 : exp(s[j] - m);
            denom += s[j];
        }
        double *o = out + (r * Hq + h) * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int64_t j = 0; j < ns; ++j) {
            if (s[j] == 0.0)
                continue;
            const double *vr = v + ((s0 + j) * Hkv + g) * D;
            for (int d = 0; d < D; ++d)
                o[d] += s[j] * vr[d];
        }
        for (int d = 0; d < D; ++d)
            o[d] /= denom;
        if (lse)
            lse[r * Hq + h] = m + log(denom);
        free(s);
    }
}
