/*
 * CPU oracle for one device's share of a DistriFusion patch layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the product path never calls
 * it.
 *
 * What it follows.  DistriFusion splits the latent into patches, one per
 * device; after the first synchronous step each device reuses the other
 * patches' activations from the previous denoising step as context
 * ("DistriFusion：高分辨率扩散模型的分布式并行推理", the dongaigc.com mirror
 * of the project README, section 概述, figure (c); the meens.ai catalog page
 * on DistriFusion, section 2).  The wrapped layers are Conv2d,
 * self-attention and GroupNorm ("DistriFusion源码探秘：从DistriUNetPP到
 * DistriAttentionTP的模块设计原理", section "Patch Parallelism的实现原理",
 * items 1-3); the default GroupNorm mode is the corrected asynchronous one
 * (README mirror, sections COCO 质量 and 延迟, the --sync_mode flag).
 *
 * The pages print no formula for any layer.  Every function below is the
 * plain definition of the textbook layer applied to the "hybrid map": the
 * previous step's full map with this patch's rows replaced by the fresh
 * local rows.  Readings taken where the pages are silent:
 *   - attention is plain softmax(scale * Q K^T) V with no mask, over all H*W
 *     tokens; K/V rows of the own patch are fresh, all others stale;
 *   - the conv is 3x3, stride 1, pad 1 with zeros at the image edges; the one
 *     halo row above/below the patch comes from the stale map;
 *   - GroupNorm statistics are the raw moments E[x], E[x^2] per (batch,
 *     group) over the whole image, formed as the equal-weight mean of this
 *     patch's fresh moments and the other patches' stale moments; the
 *     variance E[x^2] - E[x]^2 is clamped at zero before adding eps.
 *
 * Precision: every input arrives as double (the exact bf16/fp32 values
 * widened); all arithmetic is double.  Parallel loops (OpenMP) only split
 * independent outputs; no reduction is reordered or blocked.
 *
 * Layouts (row-major, innermost last):
 *   attention tensors  [B, tokens, heads, d]   token = row * W + col
 *   conv / GN maps     [B, rows, W, C]         (NHWC)
 *   conv weight        [Cout, 3, 3, Cin]
 *   moment tables      [B, n, G, 2]            (E[x], E[x^2])
 *
 * All functions return 0 on success and a negative value on a shape error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the following calls use (timing on a given number of host cores);
 * no effect on any result. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Patch self-attention for local query rows [r0, r1) of patch i.
 * out holds (r1 - r0) rows: out[b, r - r0, head, :]. */
int oracle_patch_self_attn(int64_t B, int64_t H, int64_t W, int64_t n, int64_t i,
                           int64_t heads, int64_t d, double scale,
                           const double *q, const double *k_fresh, const double *v_fresh,
                           const double *k_stale, const double *v_stale,
                           int64_t r0, int64_t r1, double *out)
{
    if (n <= 0 || H % n != 0 || i < 0 || i >= n || d <= 0 || heads <= 0)
        return -1;
    const int64_t h = H / n;
    const int64_t Lq = h * W;
    const int64_t L = H * W;
    if (r0 < 0 || r1 > Lq || r0 > r1)
        return -1;
    const int64_t rows = r1 - r0;
    const int64_t own_lo = i * Lq, own_hi = (i + 1) * Lq;

    int64_t task;
#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < B * heads * rows; ++task) {
        const int64_t b = task / (heads * rows);
        const int64_t hd = (task / rows) % heads;
        const int64_t r = r0 + task % rows;
        const double *qrow = q + ((b * Lq + r) * heads + hd) * d;
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        double m = -INFINITY;
        for (int64_t t = 0; t < L; ++t) {
            const double *krow;
            if (t >= own_lo && t < own_hi)
                krow = k_fresh + ((b * Lq + (t - own_lo)) * heads + hd) * d;
            else
                krow = k_stale + ((b * L + t) * heads + hd) * d;
            double dot = 0.0;
            for (int64_t e = 0; e < d; ++e)
                dot += qrow[e] * krow[e];
            s[t] = scale * dot;
            if (s[t] > m)
                m = s[t];
        }
        double denom = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            s[t] = exp(s[t] - m);
            denom += s[t];
        }
        double *orow = out + ((b * rows + (r - r0)) * heads + hd) * d;
        for (int64_t e = 0; e < d; ++e)
            orow[e] = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double *vrow;
            if (t >= own_lo && t < own_hi)
                vrow = v_fresh + ((b * Lq + (t - own_lo)) * heads + hd) * d;
            else
                vrow = v_stale + ((b * L + t) * heads + hd) * d;
            for (int64_t e = 0; e < d; ++e)
                orow[e] += s[t] * vrow[e];
        }
        for (int64_t e = 0; e < d; ++e)
            orow[e] /= denom;
        free(s);
    }
    return 0;
}

/* Pixel (b, local row rr, col cc) of the hybrid map as seen by patch i, or
 * NULL where the conv's zero padding applies. rr runs from -1 to h. */
static const double *hybrid_pixel(const double *x_fresh, const double *x_stale,
                                  int64_t H, int64_t W, int64_t h, int64_t n, int64_t i,
                                  int64_t cin, int64_t b, int64_t rr, int64_t cc)
{
    if (cc < 0 || cc >= W)
        return NULL;
    if (rr >= 0 && rr < h)
        return x_fresh + ((b * h + rr) * W + cc) * cin;
    const int64_t global_row = i * h + rr; /* i*h - 1 above, (i+1)*h below */
    if (global_row < 0 || global_row >= H || (rr == -1 && i == 0) || (rr == h && i == n - 1))
        return NULL;
    return x_stale + ((b * H + global_row) * W + cc) * cin;
}

/* 3x3 conv (stride 1, pad 1) of the hybrid map, output local rows [r0, r1).
 * y holds (r1 - r0) rows: y[b, r - r0, col, cout]. bias may be NULL. */
int oracle_patch_conv3x3_halo(int64_t B, int64_t H, int64_t W, int64_t n, int64_t i,
                              int64_t cin, int64_t cout,
                              const double *x_fresh, const double *x_stale,
                              const double *w, const double *bias,
                              int64_t r0, int64_t r1, double *y)
{
    if (n <= 0 || H % n != 0 || i < 0 || i >= n || cin <= 0 || cout <= 0)
        return -1;
    const int64_t h = H / n;
    if (r0 < 0 || r1 > h || r0 > r1)
        return -1;
    const int64_t rows = r1 - r0;

    int64_t task;
#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < B * rows * W; ++task) {
        const int64_t b = task / (rows * W);
        const int64_t r = r0 + (task / W) % rows;
        const int64_t c = task % W;
        double *yp = y + ((b * rows + (r - r0)) * W + c) * cout;
        for (int64_t o = 0; o < cout; ++o) {
            double acc = bias ? bias[o] : 0.0;
            for (int64_t kh = 0; kh < 3; ++kh) {
                for (int64_t kw = 0; kw < 3; ++kw) {
                    const double *xp = hybrid_pixel(x_fresh, x_stale, H, W, h, n, i, cin,
                                                    b, r + kh - 1, c + kw - 1);
                    if (!xp)
                        continue;
                    const double *wp = w + ((o * 3 + kh) * 3 + kw) * cin;
                    for (int64_t ci = 0; ci < cin; ++ci)
                        acc += wp[ci] * xp[ci];
                }
            }
            yp[o] = acc;
        }
    }
    return 0;
}

/* Raw group moments of a map x[B, rows, W, C]: out[b, g, 0] = E[x],
 * out[b, g, 1] = E[x^2] over rows * W * (C / G) values. */
int oracle_group_moments(int64_t B, int64_t rows, int64_t W, int64_t C, int64_t G,
                         const double *x, double *out)
{
    if (G <= 0 || C % G != 0 || rows * W <= 0)
        return -1;
    const int64_t cg = C / G;
    const double count = (double)(rows * W * cg);
    int64_t task;
#pragma omp parallel for schedule(static)
    for (task = 0; task < B * G; ++task) {
        const int64_t b = task / G, g = task % G;
        double s1 = 0.0, s2 = 0.0;
        for (int64_t p = 0; p < rows * W; ++p) {
            const double *xp = x + (b * rows * W + p) * C + g * cg;
            for (int64_t c = 0; c < cg; ++c) {
                s1 += xp[c];
                s2 += xp[c] * xp[c];
            }
        }
        out[task * 2 + 0] = s1 / count;
        out[task * 2 + 1] = s2 / count;
    }
    return 0;
}

/* Corrected asynchronous GroupNorm on patch i.
 *   x_fresh        [B, h, W, C]   this patch's fresh rows
 *   stale_moments  [B, n, G, 2]   previous step's per-patch moments; slot i
 *                                 is never read
 *   gamma, beta    [C] or NULL (1 and 0)
 *   y              [B, h, W, C]
 *   fresh_moments  [B, G, 2]      this patch's fresh (E[x], E[x^2])
 */
int oracle_async_groupnorm(int64_t B, int64_t H, int64_t W, int64_t n, int64_t i,
                           int64_t C, int64_t G, double eps,
                           const double *x_fresh, const double *stale_moments,
                           const double *gamma, const double *beta,
                           double *y, double *fresh_moments)
{
    if (n <= 0 || H % n != 0 || i < 0 || i >= n || G <= 0 || C % G != 0)
        return -1;
    const int64_t h = H / n;
    const int64_t cg = C / G;
    if (oracle_group_moments(B, h, W, C, G, x_fresh, fresh_moments) != 0)
        return -1;

    double *mean = (double *)malloc(sizeof(double) * (size_t)(B * G));
    double *rstd = (double *)malloc(sizeof(double) * (size_t)(B * G));
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t g = 0; g < G; ++g) {
            double e1 = fresh_moments[(b * G + g) * 2 + 0];
            double e2 = fresh_moments[(b * G + g) * 2 + 1];
            for (int64_t j = 0; j < n; ++j) {
                if (j == i)
                    continue;
                e1 += stale_moments[((b * n + j) * G + g) * 2 + 0];
                e2 += stale_moments[((b * n + j) * G + g) * 2 + 1];
            }
            e1 /= (double)n;
            e2 /= (double)n;
            double var = e2 - e1 * e1;
            if (var < 0.0)
                var = 0.0;
            mean[b * G + g] = e1;
            rstd[b * G + g] = 1.0 / sqrt(var + eps);
        }
    }

    int64_t task;
#pragma omp parallel for schedule(static)
    for (task = 0; task < B * h * W; ++task) {
        const int64_t b = task / (h * W);
        const double *xp = x_fresh + task * C;
        double *yp = y + task * C;
        for (int64_t c = 0; c < C; ++c) {
            const int64_t g = c / cg;
            const double ga = gamma ? gamma[c] : 1.0;
            const double be = beta ? beta[c] : 0.0;
            yp[c] = (xp[c] - mean[b * G + g]) * rstd[b * G + g] * ga + be;
        }
    }
    free(mean);
    free(rstd);
    return 0;
}

/* Stale refresh: rows [i*h, (i+1)*h) of stale[B, H, row_elems] take the fresh
 * slice fresh[B, h, row_elems]; every other row is left as it was. */
int oracle_refresh_stale(int64_t B, int64_t H, int64_t n, int64_t i, int64_t row_elems,
                         const double *fresh, double *stale)
{
    if (n <= 0 || H % n != 0 || i < 0 || i >= n || row_elems < 0)
        return -1;
    const int64_t h = H / n;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t r = 0; r < h; ++r)
            for (int64_t e = 0; e < row_elems; ++e)
                stale[(b * H + i * h + r) * row_elems + e] = fresh[(b * h + r) * row_elems + e];
    return 0;
}

/* Token-wise linear map, the form of the attention layer's Q/K/V and output
 * projections (the modules that the wrapped self-attention holds: source
 * walkthrough, section "Patch Parallelism的实现原理", item 2):
 *   y[m, o] = bias[o] + sum_c w[o, c] * x[m, c]     m < M, o < N
 * x [M, C], w [N, C] (row o holds output o's weights), bias [N] or NULL,
 * y [M, N]. */
int oracle_linear(int64_t M, int64_t C, int64_t N, const double *x, const double *w,
                  const double *bias, double *y)
{
    if (M < 0 || C < 0 || N < 0)
        return -1;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t o = 0; o < N; ++o) {
            double acc = bias ? bias[o] : 0.0;
            for (int64_t c = 0; c < C; ++c)
                acc += w[o * C + c] * x[m * C + c];
            y[m * N + o] = acc;
        }
    }
    return 0;
}

/* Q/K/V projection of patch i with the refresh folded in.  x [B, h, W, C]
 * holds the patch's hidden states (token t = r * W + c of the patch);
 * w_qkv [3C, C] stacks the Q, K and V weights, bias [3C] or NULL:
 *   [q | k | v][b, t, :] = linear(x[b, t, :])       each [B, Lq, C]
 * and, when k_stale / v_stale [B, H*W, C] are given, their rows of patch i
 * take the new k / v (the previous step's stale maps then hold this step's
 * fresh K/V for the next step, as a separate refresh would leave them). */
int oracle_patch_qkv_proj(int64_t B, int64_t H, int64_t W, int64_t n, int64_t i, int64_t C,
                          const double *x, const double *w_qkv, const double *bias, double *q,
                          double *k, double *v, double *k_stale, double *v_stale)
{
    if (n <= 0 || H % n != 0 || i < 0 || i >= n || C <= 0)
        return -1;
    const int64_t Lq = (H / n) * W, L = H * W, M = B * Lq;
    double *y = (double *)malloc(sizeof(double) * (size_t)(M * 3 * C));
    if (!y)
        return -2;
    oracle_linear(M, C, 3 * C, x, w_qkv, bias, y);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < C; ++c) {
            q[m * C + c] = y[m * 3 * C + c];
            k[m * C + c] = y[m * 3 * C + C + c];
            v[m * C + c] = y[m * 3 * C + 2 * C + c];
        }
    free(y);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < Lq; ++t)
            for (int64_t c = 0; c < C; ++c) {
                const int64_t src = (b * Lq + t) * C + c;
                const int64_t dst = (b * L + i * Lq + t) * C + c;
                if (k_stale)
                    k_stale[dst] = k[src];
                if (v_stale)
                    v_stale[dst] = v[src];
            }
    return 0;
}

/* SiLU, the activation that follows GroupNorm in SDXL's ResNet blocks:
 * y = z * sigmoid(z) = z / (1 + exp(-z)), elementwise over n values. */
int oracle_silu(int64_t n, const double *z, double *y)
{
    if (n < 0) return -1;
    for (int64_t k = 0; k < n; ++k) y[k] = z[k] / (1.0 + exp(-z[k]));
    return 0;
}

/* Cross-attention of patch queries over a context that every patch shares
 * (the text encoder's tokens; the wrapped cross-attention of the source
 * walkthrough, section "Patch Parallelism的实现原理", item 2): for each image
 * b, head and query row r,
 *   out[b, r, head, :] = sum_t softmax_t(scale q[b, r, head, :] . k[b, t, head, :]) v[b, t, head, :]
 * over the Lk context tokens.  Nothing is stale: the context is the same on
 * every patch and every step.
 *   q, out [B, Lq, heads, d]     k, v [B, Lk, heads, d] */
int oracle_cross_attn(int64_t B, int64_t Lq, int64_t Lk, int64_t heads, int64_t d, double scale,
                      const double *q, const double *k, const double *v, double *out)
{
    if (B < 0 || Lq < 0 || Lk <= 0 || heads <= 0 || d <= 0)
        return -1;
    int64_t task;
#pragma omp parallel for schedule(dynamic, 16)
    for (task = 0; task < B * heads * Lq; ++task) {
        const int64_t b = task / (heads * Lq);
        const int64_t hd = (task / Lq) % heads;
        const int64_t r = task % Lq;
        const double *qrow = q + ((b * Lq + r) * heads + hd) * d;
        double *s = (double *)malloc(sizeof(double) * (size_t)Lk);
        double m = -INFINITY;
        for (int64_t t = 0; t < Lk; ++t) {
            const double *krow = k + ((b * Lk + t) * heads + hd) * d;
            double dot = 0.0;
            for (int64_t e = 0; e < d; ++e)
                dot += qrow[e] * krow[e];
            s[t] = scale * dot;
            if (s[t] > m)
                m = s[t];
        }
        double denom = 0.0;
        for (int64_t t = 0; t < Lk; ++t) {
            s[t] = exp(s[t] - m);
            denom += s[t];
        }
        double *orow = out + ((b * Lq + r) * heads + hd) * d;
        for (int64_t e = 0; e < d; ++e)
            orow[e] = 0.0;
        for (int64_t t = 0; t < Lk; ++t) {
            const double *vrow = v + ((b * Lk + t) * heads + hd) * d;
            for (int64_t e = 0; e < d; ++e)
                orow[e] += s[t] * vrow[e];
        }
        for (int64_t e = 0; e < d; ++e)
            orow[e] /= denom;
        free(s);
    }
    return 0;
}
