/*
 * c3d_oracle.c - CPU oracle for the 3D convolution / transposed-convolution
 * forward path and its fused epilogues.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path never does.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * Every function is the plain definition written out: nested loops, double
 * accumulation, no tiling, no fusion and no reordering beyond what the
 * definition states.  Inputs are float32 (the same bits the GPU reads);
 * results are float64.
 *
 * Sources ("page" = a POPCORNBENCH agent transcript, named by its title):
 *   [p59] "Kimi-K2.6 l1_p59"  Conv3d with a (k,k,1) kernel, depth-last input
 *   [p72] "Kimi-K2.6 l2_p72"  ConvTranspose3d -> BatchNorm3d -> AvgPool3d x2
 *   [p43] "Kimi-K2.6 l2_p43"  Conv3d -> MaxPool3d -> logsumexp -> ReLU
 *   [p77] "Kimi-K2.6 l1_p77"  ConvTranspose3d with stride, padding, dilation
 *
 * Layouts: x is [N, C, S0, S1, S2] contiguous (S2 fastest).  A depth-last
 * tensor x[N,C,H,W,D] is simply S0=H, S1=W, S2=D: the kernel triple applies
 * to the last three dims in order ([p59], the passage that settles how
 * PyTorch reads the (k,k,1) kernel on an [N,C,H,W,D] tensor).
 * Conv weight: [Cout, Cin/groups, k0, k1, k2].
 * ConvT weight: [Cin, Cout/groups, k0, k1, k2] ([p77], the late passage
 * that corrects the kernel's [oc][ic] weight indexing; [p72], weight shape
 * of ConvTranspose3d).
 *
 * Parity pins: every function here is checked, in the CPU test suite,
 * against closed forms, worked examples from the pages, invariants and
 * library routines (PyTorch CPU in float64).  Nothing is left unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The oracle's own parameter block (deliberately not the HIP library's). */
typedef struct {
    int32_t k[3];     /* kernel extent per spatial dim            */
    int32_t s[3];     /* stride                                   */
    int32_t p[3];     /* zero padding                             */
    int32_t d[3];     /* dilation                                 */
    int32_t op[3];    /* output padding (transposed conv only)     */
    int32_t groups;
} oracle_params;

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ sizes */

/* Direct-conv output length: floor((L + 2p - d(k-1) - 1)/s) + 1.
 * [p43] states this formula for the conv output; [p59] uses it for each
 * spatial dim including the size-1 kernel dim, where stride and padding
 * still apply.  Returns 0 when no window fits. */
int64_t oracle_conv_out_len(int64_t L, int32_t k, int32_t s, int32_t p, int32_t d) {
    int64_t num = L + 2 * (int64_t)p - (int64_t)d * (k - 1) - 1;
    if (num < 0) return 0;
    return num / s + 1;
}

/* Transposed-conv output length: (L-1)s - 2p + d(k-1) + output_padding + 1.
 * [p72] states it for dilation 1; [p77] states it with dilation.  May be
 * <= 0 for degenerate parameters. */
int64_t oracle_convT_out_len(int64_t L, int32_t k, int32_t s, int32_t p, int32_t d, int32_t op) {
    return (L - 1) * s - 2 * (int64_t)p + (int64_t)d * (k - 1) + op + 1;
}

/* Pooling output length with window = stride = w, floor mode, no padding:
 * floor((L - w)/w) + 1, i.e. the trailing L mod w elements are dropped
 * ([p72], the passage noting that input indices 60, 61, 62 are dropped). */
int64_t oracle_pool_out_len(int64_t L, int32_t w) {
    if (L < w) return 0;
    return (L - w) / w + 1;
}

/* ------------------------------------------------------------ conv3d */

static inline int64_t idx5(int64_t a, int64_t b, int64_t c, int64_t d, int64_t e,
                           int64_t B, int64_t C, int64_t D, int64_t E) {
    return (((a * B + b) * C + c) * D + d) * E + e;
}

/* One output of the direct convolution, from its definition ([p59], the
 * opening statement of the output formula summed over the channels of the
 * group; [p43], the per-output sum over c_in and the 3x3x3 window):
 *   y[n,oc,o] = bias[oc] + sum_{icg, k} W[oc,icg,k] * x[n, g*Cin_g+icg, o*s - p + k*d]
 * with g = oc / (Cout/groups) and zero outside the input. */
static double conv3d_one(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                         const oracle_params* P, const float* bias,
                         int64_t n, int64_t oc, int64_t o0, int64_t o1, int64_t o2) {
    const int64_t C = xs[1], S0 = xs[2], S1 = xs[3], S2 = xs[4];
    const int64_t cin_g = C / P->groups, cout_g = cout / P->groups;
    const int64_t g = oc / cout_g;
    double acc = bias ? (double)bias[oc] : 0.0;
    for (int64_t icg = 0; icg < cin_g; ++icg) {
        const int64_t ic = g * cin_g + icg;
        for (int32_t k0 = 0; k0 < P->k[0]; ++k0) {
            const int64_t i0 = o0 * P->s[0] - P->p[0] + (int64_t)k0 * P->d[0];
            if (i0 < 0 || i0 >= S0) continue;
            for (int32_t k1 = 0; k1 < P->k[1]; ++k1) {
                const int64_t i1 = o1 * P->s[1] - P->p[1] + (int64_t)k1 * P->d[1];
                if (i1 < 0 || i1 >= S1) continue;
                for (int32_t k2 = 0; k2 < P->k[2]; ++k2) {
                    const int64_t i2 = o2 * P->s[2] - P->p[2] + (int64_t)k2 * P->d[2];
                    if (i2 < 0 || i2 >= S2) continue;
                    const double wv = w[idx5(oc, icg, k0, k1, k2, cin_g, P->k[0], P->k[1], P->k[2])];
                    const double xv = x[idx5(n, ic, i0, i1, i2, C, S0, S1, S2)];
                    acc += wv * xv;
                }
            }
        }
    }
    return acc;
}

static void conv3d_dims(const int64_t xs[5], int64_t cout, const oracle_params* P, int64_t ys[5]) {
    ys[0] = xs[0];
    ys[1] = cout;
    for (int j = 0; j < 3; ++j) ys[2 + j] = oracle_conv_out_len(xs[2 + j], P->k[j], P->s[j], P->p[j], P->d[j]);
}

/* Full conv3d output y[N,Cout,O0,O1,O2], rows o0 in [o0_begin, o0_end) only
 * (y points at row o0_begin; the whole tensor when the range is [0,O0)). */
void oracle_conv3d_rows(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                        const oracle_params* P, const float* bias,
                        int64_t o0_begin, int64_t o0_end, double* y) {
    int64_t ys[5];
    conv3d_dims(xs, cout, P, ys);
    const int64_t R = o0_end - o0_begin, O1 = ys[3], O2 = ys[4];
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < xs[0]; ++n)
        for (int64_t oc = 0; oc < cout; ++oc)
            for (int64_t r = 0; r < R; ++r)
                for (int64_t o1 = 0; o1 < O1; ++o1)
                    for (int64_t o2 = 0; o2 < O2; ++o2)
                        y[idx5(n, oc, r, o1, o2, cout, R, O1, O2)] =
                            conv3d_one(x, xs, w, cout, P, bias, n, oc, o0_begin + r, o1, o2);
}

void oracle_conv3d(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                   const oracle_params* P, const float* bias, double* y) {
    int64_t ys[5];
    conv3d_dims(xs, cout, P, ys);
    oracle_conv3d_rows(x, xs, w, cout, P, bias, 0, ys[2], y);
}

/* Selected outputs, by flat index into y[N,Cout,O0,O1,O2]. */
void oracle_conv3d_at(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                      const oracle_params* P, const float* bias,
                      const int64_t* flat, int64_t count, double* out) {
    int64_t ys[5];
    conv3d_dims(xs, cout, P, ys);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < count; ++t) {
        int64_t f = flat[t];
        const int64_t o2 = f % ys[4]; f /= ys[4];
        const int64_t o1 = f % ys[3]; f /= ys[3];
        const int64_t o0 = f % ys[2]; f /= ys[2];
        const int64_t oc = f % ys[1]; f /= ys[1];
        out[t] = conv3d_one(x, xs, w, cout, P, bias, f, oc, o0, o1, o2);
    }
}

/* ------------------------------------------------------ conv_transpose3d */

static void convT_dims(const int64_t xs[5], int64_t cout, const oracle_params* P, int64_t ys[5]) {
    ys[0] = xs[0];
    ys[1] = cout;
    for (int j = 0; j < 3; ++j)
        ys[2 + j] = oracle_convT_out_len(xs[2 + j], P->k[j], P->s[j], P->p[j], P->d[j], P->op[j]);
}

/* Scatter definition of the transposed convolution, for output channels
 * [oc_begin, oc_end) of every batch item ([p77], the derivation in which
 * input position i and kernel tap k land at output i*s - p + k*d, and its
 * later corrected weight indexing W[ic][oc]; [p72], the same mapping written
 * od = id*stride - padding + kd):
 *   y[n, g*Cout_g+ocg, :] = bias
 *   y[n, g*Cout_g+ocg, i*s - p + k*d] += x[n, ic, i] * W[ic, ocg, k]
 * for every input channel ic of group g = ic / Cin_g, every input position
 * i and every tap k whose target lies inside the output.  y holds
 * [N, oc_end-oc_begin, O0, O1, O2]. */
void oracle_conv_transpose3d_channels(const float* x, const int64_t xs[5], const float* w,
                                      int64_t cout, const oracle_params* P, const float* bias,
                                      int64_t oc_begin, int64_t oc_end, double* y) {
    int64_t ys[5];
    convT_dims(xs, cout, P, ys);
    const int64_t C = xs[1], S0 = xs[2], S1 = xs[3], S2 = xs[4];
    const int64_t O0 = ys[2], O1 = ys[3], O2 = ys[4];
    const int64_t cin_g = C / P->groups, cout_g = cout / P->groups;
    const int64_t nc = oc_end - oc_begin;
    const int64_t plane = O0 * O1 * O2;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < xs[0]; ++n)
        for (int64_t c = 0; c < nc; ++c) {
            const int64_t oc = oc_begin + c;
            const int64_t g = oc / cout_g, ocg = oc % cout_g;
            double* yp = y + (n * nc + c) * plane;
            const double b = bias ? (double)bias[oc] : 0.0;
            for (int64_t t = 0; t < plane; ++t) yp[t] = b;
            for (int64_t icg = 0; icg < cin_g; ++icg) {
                const int64_t ic = g * cin_g + icg;
                for (int64_t i0 = 0; i0 < S0; ++i0)
                    for (int64_t i1 = 0; i1 < S1; ++i1)
                        for (int64_t i2 = 0; i2 < S2; ++i2) {
                            const double xv = x[idx5(n, ic, i0, i1, i2, C, S0, S1, S2)];
                            for (int32_t k0 = 0; k0 < P->k[0]; ++k0) {
                                const int64_t o0 = i0 * P->s[0] - P->p[0] + (int64_t)k0 * P->d[0];
                                if (o0 < 0 || o0 >= O0) continue;
                                for (int32_t k1 = 0; k1 < P->k[1]; ++k1) {
                                    const int64_t o1 = i1 * P->s[1] - P->p[1] + (int64_t)k1 * P->d[1];
                                    if (o1 < 0 || o1 >= O1) continue;
                                    for (int32_t k2 = 0; k2 < P->k[2]; ++k2) {
                                        const int64_t o2 = i2 * P->s[2] - P->p[2] + (int64_t)k2 * P->d[2];
                                        if (o2 < 0 || o2 >= O2) continue;
                                        const double wv =
                                            w[idx5(ic, ocg, k0, k1, k2, cout_g, P->k[0], P->k[1], P->k[2])];
                                        yp[(o0 * O1 + o1) * O2 + o2] += xv * wv;
                                    }
                                }
                            }
                        }
            }
        }
}

void oracle_conv_transpose3d(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                             const oracle_params* P, const float* bias, double* y) {
    oracle_conv_transpose3d_channels(x, xs, w, cout, P, bias, 0, cout, y);
}

/* Gather form of one transposed-conv output ([p77], the passage solving
 * o = i*s - p + k*d for i: a tap contributes iff (o + p - k*d) is divisible
 * by s and the quotient is a valid input index; [p72], the same test
 * d_in = (d' + padding - kd)/stride).  Equal to the scatter form. */
static double convT_one(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                        const oracle_params* P, const float* bias,
                        int64_t n, int64_t oc, const int64_t o[3]) {
    const int64_t C = xs[1];
    const int64_t cin_g = C / P->groups, cout_g = cout / P->groups;
    const int64_t g = oc / cout_g, ocg = oc % cout_g;
    double acc = bias ? (double)bias[oc] : 0.0;
    for (int64_t icg = 0; icg < cin_g; ++icg) {
        const int64_t ic = g * cin_g + icg;
        for (int32_t k0 = 0; k0 < P->k[0]; ++k0) {
            const int64_t t0 = o[0] + P->p[0] - (int64_t)k0 * P->d[0];
            if (t0 < 0 || t0 % P->s[0] != 0 || t0 / P->s[0] >= xs[2]) continue;
            for (int32_t k1 = 0; k1 < P->k[1]; ++k1) {
                const int64_t t1 = o[1] + P->p[1] - (int64_t)k1 * P->d[1];
                if (t1 < 0 || t1 % P->s[1] != 0 || t1 / P->s[1] >= xs[3]) continue;
                for (int32_t k2 = 0; k2 < P->k[2]; ++k2) {
                    const int64_t t2 = o[2] + P->p[2] - (int64_t)k2 * P->d[2];
                    if (t2 < 0 || t2 % P->s[2] != 0 || t2 / P->s[2] >= xs[4]) continue;
                    const double xv =
                        x[idx5(n, ic, t0 / P->s[0], t1 / P->s[1], t2 / P->s[2], C, xs[2], xs[3], xs[4])];
                    const double wv = w[idx5(ic, ocg, k0, k1, k2, cout_g, P->k[0], P->k[1], P->k[2])];
                    acc += xv * wv;
                }
            }
        }
    }
    return acc;
}

void oracle_conv_transpose3d_at(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                                const oracle_params* P, const float* bias,
                                const int64_t* flat, int64_t count, double* out) {
    int64_t ys[5];
    convT_dims(xs, cout, P, ys);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < count; ++t) {
        int64_t f = flat[t], o[3];
        o[2] = f % ys[4]; f /= ys[4];
        o[1] = f % ys[3]; f /= ys[3];
        o[0] = f % ys[2]; f /= ys[2];
        const int64_t oc = f % ys[1]; f /= ys[1];
        out[t] = convT_one(x, xs, w, cout, P, bias, f, oc, o);
    }
}

/* ------------------------------------------------------------- epilogues */

/* Training-mode BatchNorm3d on y[N,C,S...] (plane = S0*S1*S2), in place:
 * per channel c, mu = mean over (n, spatial), var = mean of (y - mu)^2
 * (biased, two passes), then z = gamma*(y - mu)/sqrt(var + eps) + beta
 * ([p72], the passage on training-mode batch statistics with
 * var(..., unbiased=False)).  mean/var outputs are optional. */
void oracle_batchnorm_train(double* y, int64_t N, int64_t C, int64_t plane,
                            const float* gamma, const float* beta, double eps,
                            double* mean_out, double* var_out) {
    for (int64_t c = 0; c < C; ++c) {
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t t = 0; t < plane; ++t) s += y[(n * C + c) * plane + t];
        const double cnt = (double)(N * plane);
        const double mu = s / cnt;
        double v = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t t = 0; t < plane; ++t) {
                const double e = y[(n * C + c) * plane + t] - mu;
                v += e * e;
            }
        v /= cnt;
        const double inv = 1.0 / sqrt(v + eps);
        const double ga = gamma ? (double)gamma[c] : 1.0, be = beta ? (double)beta[c] : 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t t = 0; t < plane; ++t) {
                double* e = &y[(n * C + c) * plane + t];
                *e = ga * (*e - mu) * inv + be;
            }
        if (mean_out) mean_out[c] = mu;
        if (var_out) var_out[c] = v;
    }
}

/* Average pool, cubic window = stride = w, floor mode, no padding:
 * out[n,c,j] = mean of in[n,c, w*j + u] over u in [0,w)^3.  in is
 * [NC, S0, S1, S2] (NC = N*C planes); out is [NC, P0, P1, P2]. */
void oracle_avgpool3d(const double* in, int64_t NC, const int64_t S[3], int32_t w, double* out) {
    const int64_t P0 = oracle_pool_out_len(S[0], w), P1 = oracle_pool_out_len(S[1], w),
                  P2 = oracle_pool_out_len(S[2], w);
    const double inv = 1.0 / ((double)w * w * w);
    for (int64_t q = 0; q < NC; ++q)
        for (int64_t j0 = 0; j0 < P0; ++j0)
            for (int64_t j1 = 0; j1 < P1; ++j1)
                for (int64_t j2 = 0; j2 < P2; ++j2) {
                    double s = 0.0;
                    for (int32_t u0 = 0; u0 < w; ++u0)
                        for (int32_t u1 = 0; u1 < w; ++u1)
                            for (int32_t u2 = 0; u2 < w; ++u2)
                                s += in[((q * S[0] + j0 * w + u0) * S[1] + j1 * w + u1) * S[2] + j2 * w + u2];
                    out[((q * P0 + j0) * P1 + j1) * P2 + j2] = s * inv;
                }
}

/* Max pool, cubic window = stride = w, floor mode, no padding. */
void oracle_maxpool3d(const double* in, int64_t NC, const int64_t S[3], int32_t w, double* out) {
    const int64_t P0 = oracle_pool_out_len(S[0], w), P1 = oracle_pool_out_len(S[1], w),
                  P2 = oracle_pool_out_len(S[2], w);
    for (int64_t q = 0; q < NC; ++q)
        for (int64_t j0 = 0; j0 < P0; ++j0)
            for (int64_t j1 = 0; j1 < P1; ++j1)
                for (int64_t j2 = 0; j2 < P2; ++j2) {
                    double m = -INFINITY;
                    for (int32_t u0 = 0; u0 < w; ++u0)
                        for (int32_t u1 = 0; u1 < w; ++u1)
                            for (int32_t u2 = 0; u2 < w; ++u2) {
                                const double v =
                                    in[((q * S[0] + j0 * w + u0) * S[1] + j1 * w + u1) * S[2] + j2 * w + u2];
                                if (v > m) m = v;
                            }
                    out[((q * P0 + j0) * P1 + j1) * P2 + j2] = m;
                }
}

/* logsumexp over the channel dim of in[N, C, plane] -> out[N, 1, plane],
 * two passes: M = max_c v_c, then M + log(sum_c exp(v_c - M)) ([p43], the
 * logsumexp(dim=1, keepdim=True) step and its max-shifted evaluation). */
void oracle_logsumexp_channels(const double* in, int64_t N, int64_t C, int64_t plane, double* out) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t t = 0; t < plane; ++t) {
            double m = -INFINITY;
            for (int64_t c = 0; c < C; ++c) {
                const double v = in[(n * C + c) * plane + t];
                if (v > m) m = v;
            }
            double s = 0.0;
            for (int64_t c = 0; c < C; ++c) s += exp(in[(n * C + c) * plane + t] - m);
            out[n * plane + t] = m + log(s);
        }
}

/* ReLU in place: max(v, 0). */
void oracle_relu(double* v, int64_t count) {
    for (int64_t t = 0; t < count; ++t)
        if (!(v[t] > 0.0)) v[t] = 0.0;
}

/* ------------------------------------------------------ fused modules */

/* ConvTranspose3d -> BatchNorm3d (batch statistics) -> AvgPool3d(pool).
 * The module on [p72] applies AvgPool3d(2) twice; the page shows that this
 * equals one AvgPool3d(4, stride 4) (the 1-D proof extended to 3-D), so
 * pool = 4 is that module.  Steps, per output channel, in the module's
 * order: the transposed conv for every batch item (scatter form above), the
 * biased batch statistics over all of that channel's outputs, the affine
 * normalisation, the average pool.  out is [N, Cout, P0, P1, P2]; mean/var
 * (optional) receive the batch mean and biased variance. */
void oracle_convT_bn_avgpool(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                             const oracle_params* P, const float* bias, const float* gamma,
                             const float* beta, double eps, int32_t pool, double* out,
                             double* mean_out, double* var_out) {
    int64_t ys[5];
    convT_dims(xs, cout, P, ys);
    const int64_t N = xs[0];
    const int64_t S[3] = {ys[2], ys[3], ys[4]};
    const int64_t plane = S[0] * S[1] * S[2];
    const int64_t P0 = oracle_pool_out_len(S[0], pool), P1 = oracle_pool_out_len(S[1], pool),
                  P2 = oracle_pool_out_len(S[2], pool);
    const int64_t pplane = P0 * P1 * P2;
    double* y = (double*)malloc(sizeof(double) * (size_t)(N * plane));
    double* pooled = (double*)malloc(sizeof(double) * (size_t)(N * (pplane > 0 ? pplane : 1)));
    for (int64_t c = 0; c < cout; ++c) {
        /* y[n, 0, :] = channel c of the transposed conv, for every n */
        oracle_conv_transpose3d_channels(x, xs, w, cout, P, bias, c, c + 1, y);
        double mu, var;
        oracle_batchnorm_train(y, N, 1, plane, gamma ? gamma + c : NULL, beta ? beta + c : NULL, eps,
                               &mu, &var);
        if (mean_out) mean_out[c] = mu;
        if (var_out) var_out[c] = var;
        oracle_avgpool3d(y, N, S, pool, pooled);
        for (int64_t n = 0; n < N; ++n)
            memcpy(out + (n * cout + c) * pplane, pooled + n * pplane, sizeof(double) * (size_t)pplane);
    }
    free(y);
    free(pooled);
}

/* The same module with BatchNorm3d in eval mode ([p72], the eval-mode
 * kernel the page ships: BN normalises with the running statistics, an
 * affine map per channel).  In the module's order: t = convT(x, w, bias),
 * then u = gamma_c (t - running_mean_c) / sqrt(running_var_c + eps) + beta_c
 * on every element, then the average pool.  out is [N, Cout, P0, P1, P2]. */
void oracle_convT_bn_eval_avgpool(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                                  const oracle_params* P, const float* bias, const float* gamma,
                                  const float* beta, const float* running_mean, const float* running_var,
                                  double eps, int32_t pool, double* out) {
    int64_t ys[5];
    convT_dims(xs, cout, P, ys);
    const int64_t N = xs[0];
    const int64_t S[3] = {ys[2], ys[3], ys[4]};
    const int64_t plane = S[0] * S[1] * S[2];
    const int64_t P0 = oracle_pool_out_len(S[0], pool), P1 = oracle_pool_out_len(S[1], pool),
                  P2 = oracle_pool_out_len(S[2], pool);
    const int64_t pplane = P0 * P1 * P2;
    double* y = (double*)malloc(sizeof(double) * (size_t)(N * plane));
    double* pooled = (double*)malloc(sizeof(double) * (size_t)(N * (pplane > 0 ? pplane : 1)));
    for (int64_t c = 0; c < cout; ++c) {
        oracle_conv_transpose3d_channels(x, xs, w, cout, P, bias, c, c + 1, y);
        const double rm = running_mean[c], rs = sqrt((double)running_var[c] + eps);
        for (int64_t e = 0; e < N * plane; ++e) y[e] = (double)gamma[c] * (y[e] - rm) / rs + (double)beta[c];
        oracle_avgpool3d(y, N, S, pool, pooled);
        for (int64_t n = 0; n < N; ++n)
            memcpy(out + (n * cout + c) * pplane, pooled + n * pplane, sizeof(double) * (size_t)pplane);
    }
    free(y);
    free(pooled);
}

/* Running statistics after one training-mode forward (BatchNorm3d, [p72]'s
 * momentum 0.1 and its training/eval distinction): with count = elements per
 * channel,
 *   running_mean <- (1 - m) running_mean + m * batch_mean
 *   running_var  <- (1 - m) running_var  + m * batch_var * count / (count - 1)
 * i.e. the running variance tracks the unbiased batch variance while the
 * normalisation itself uses the biased one. */
void oracle_bn_running_update(int64_t C, double momentum, int64_t count, const double* batch_mean,
                              const double* batch_var_biased, double* running_mean, double* running_var) {
    for (int64_t c = 0; c < C; ++c) {
        const double unbiased = batch_var_biased[c] * (double)count / (double)(count - 1);
        running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * batch_mean[c];
        running_var[c] = (1.0 - momentum) * running_var[c] + momentum * unbiased;
    }
}

/* Conv3d -> MaxPool3d(pool) -> logsumexp over channels (keepdim) -> ReLU
 * ([p43], the module definition).  Processed one pooled row j0 at a time
 * (the conv rows [pool*j0, pool*j0 + pool) of every channel, then the three
 * epilogue steps on that slab) so the full conv output is never held.
 * out is [N, 1, P0, P1, P2]. */
void oracle_conv_maxpool_lse_relu(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                                  const oracle_params* P, const float* bias, int32_t pool, double* out) {
    int64_t ys[5];
    conv3d_dims(xs, cout, P, ys);
    const int64_t N = xs[0], O1 = ys[3], O2 = ys[4];
    const int64_t P0 = oracle_pool_out_len(ys[2], pool), P1 = oracle_pool_out_len(O1, pool),
                  P2 = oracle_pool_out_len(O2, pool);
    const int64_t slab = (int64_t)pool * O1 * O2, pplane = P1 * P2;
    double* y = (double*)malloc(sizeof(double) * (size_t)(N * cout * slab));
    double* m = (double*)malloc(sizeof(double) * (size_t)(N * cout * (pplane > 0 ? pplane : 1)));
    double* l = (double*)malloc(sizeof(double) * (size_t)(N * (pplane > 0 ? pplane : 1)));
    for (int64_t j0 = 0; j0 < P0; ++j0) {
        oracle_conv3d_rows(x, xs, w, cout, P, bias, j0 * pool, j0 * pool + pool, y);
        const int64_t S[3] = {pool, O1, O2};
        oracle_maxpool3d(y, N * cout, S, pool, m);
        oracle_logsumexp_channels(m, N, cout, pplane, l);
        oracle_relu(l, N * pplane);
        for (int64_t n = 0; n < N; ++n)
            memcpy(out + (n * P0 + j0) * pplane, l + n * pplane, sizeof(double) * (size_t)pplane);
    }
    free(y);
    free(m);
    free(l);
}

/* Selected outputs of conv_maxpool_lse_relu, by flat index into
 * [N, 1, P0, P1, P2]: for each, the pool^3 conv outputs of every channel,
 * their max, the two-pass logsumexp over channels, then ReLU. */
void oracle_conv_maxpool_lse_relu_at(const float* x, const int64_t xs[5], const float* w, int64_t cout,
                                     const oracle_params* P, const float* bias, int32_t pool,
                                     const int64_t* flat, int64_t count, double* out) {
    int64_t ys[5];
    conv3d_dims(xs, cout, P, ys);
    const int64_t P0 = oracle_pool_out_len(ys[2], pool), P1 = oracle_pool_out_len(ys[3], pool),
                  P2 = oracle_pool_out_len(ys[4], pool);
#pragma omp parallel
    {
        double* mc = (double*)malloc(sizeof(double) * (size_t)cout);
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < count; ++t) {
            int64_t f = flat[t];
            const int64_t j2 = f % P2; f /= P2;
            const int64_t j1 = f % P1; f /= P1;
            const int64_t j0 = f % P0; f /= P0;
            const int64_t n = f;
            for (int64_t oc = 0; oc < cout; ++oc) {
                double mx = -INFINITY;
                for (int32_t u0 = 0; u0 < pool; ++u0)
                    for (int32_t u1 = 0; u1 < pool; ++u1)
                        for (int32_t u2 = 0; u2 < pool; ++u2) {
                            const double v = conv3d_one(x, xs, w, cout, P, bias, n, oc, j0 * pool + u0,
                                                        j1 * pool + u1, j2 * pool + u2);
                            if (v > mx) mx = v;
                        }
                mc[oc] = mx;
            }
            double l;
            oracle_logsumexp_channels(mc, 1, cout, 1, &l);
            oracle_relu(&l, 1);
            out[t] = l;
        }
        free(mc);
    }
}
