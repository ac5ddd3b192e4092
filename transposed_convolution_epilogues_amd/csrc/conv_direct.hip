// conv_direct.hip - generic kernels: one thread per output, fp32 FMA, correct
// for every stride / padding / dilation / groups / output_padding.  They are
// the fallback for shapes the MFMA and specialised kernels do not take.
//
// Definitions follow the pages (POPCORNBENCH transcripts, cited by title):
//   direct conv   - "Kimi-K2.6 l1_p59", the output formula summed over the
//                   channels of the group; "Kimi-K2.6 l2_p43", the per-output
//                   sum over c_in and the window
//   transposed    - "Kimi-K2.6 l1_p77", the gather test: tap k reaches output
//                   o from input i = (o + p - k*d)/s when that is an integer
//                   inside the input; weights indexed [ic][oc]
//   fused pools   - "Kimi-K2.6 l2_p72" (batch-statistics BN, folded avg pool)
//                   and "Kimi-K2.6 l2_p43" (max pool, channel logsumexp, ReLU)
#include <float.h>
#include <math.h>

#include "c3d_internal.h"

namespace c3d {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ float conv_one(const float* __restrict__ x, const float* __restrict__ w,
                                          const Geom& g, int64_t n, int64_t oc, int64_t o0, int64_t o1,
                                          int64_t o2) {
    const int64_t grp = oc / g.cout_g;
    float acc = 0.f;
    for (int icg = 0; icg < g.cin_g; ++icg) {
        const float* xc = x + ((n * g.Cin + grp * g.cin_g + icg) * g.S[0]) * g.S[1] * g.S[2];
        const float* wc = w + ((oc * g.cin_g + icg) * g.k[0]) * g.k[1] * g.k[2];
        for (int k0 = 0; k0 < g.k[0]; ++k0) {
            const int64_t i0 = o0 * g.s[0] - g.p[0] + (int64_t)k0 * g.d[0];
            if (i0 < 0 || i0 >= g.S[0]) continue;
            for (int k1 = 0; k1 < g.k[1]; ++k1) {
                const int64_t i1 = o1 * g.s[1] - g.p[1] + (int64_t)k1 * g.d[1];
                if (i1 < 0 || i1 >= g.S[1]) continue;
                const float* xr = xc + (i0 * g.S[1] + i1) * g.S[2];
                const float* wr = wc + (k0 * g.k[1] + k1) * g.k[2];
                for (int k2 = 0; k2 < g.k[2]; ++k2) {
                    const int64_t i2 = o2 * g.s[2] - g.p[2] + (int64_t)k2 * g.d[2];
                    if (i2 < 0 || i2 >= g.S[2]) continue;
                    acc = fmaf(wr[k2], xr[i2], acc);
                }
            }
        }
    }
    return acc;
}

__device__ __forceinline__ float convT_one(const float* __restrict__ x, const float* __restrict__ w,
                                           const Geom& g, int64_t n, int64_t oc, int64_t o0, int64_t o1,
                                           int64_t o2) {
    const int64_t grp = oc / g.cout_g, ocg = oc % g.cout_g;
    float acc = 0.f;
    for (int icg = 0; icg < g.cin_g; ++icg) {
        const int64_t ic = grp * g.cin_g + icg;
        const float* xc = x + ((n * g.Cin + ic) * g.S[0]) * g.S[1] * g.S[2];
        const float* wc = w + ((ic * g.cout_g + ocg) * g.k[0]) * g.k[1] * g.k[2];
        for (int k0 = 0; k0 < g.k[0]; ++k0) {
            const int64_t t0 = o0 + g.p[0] - (int64_t)k0 * g.d[0];
            if (t0 < 0 || t0 % g.s[0] != 0) continue;
            const int64_t i0 = t0 / g.s[0];
            if (i0 >= g.S[0]) continue;
            for (int k1 = 0; k1 < g.k[1]; ++k1) {
                const int64_t t1 = o1 + g.p[1] - (int64_t)k1 * g.d[1];
                if (t1 < 0 || t1 % g.s[1] != 0) continue;
                const int64_t i1 = t1 / g.s[1];
                if (i1 >= g.S[1]) continue;
                for (int k2 = 0; k2 < g.k[2]; ++k2) {
                    const int64_t t2 = o2 + g.p[2] - (int64_t)k2 * g.d[2];
                    if (t2 < 0 || t2 % g.s[2] != 0) continue;
                    const int64_t i2 = t2 / g.s[2];
                    if (i2 >= g.S[2]) continue;
                    acc = fmaf(xc[(i0 * g.S[1] + i1) * g.S[2] + i2], wc[(k0 * g.k[1] + k1) * g.k[2] + k2], acc);
                }
            }
        }
    }
    return acc;
}

__global__ __launch_bounds__(kBlock) void conv3d_direct_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               const float* __restrict__ bias,
                                                               float* __restrict__ y, Geom g, int64_t total) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        int64_t f = idx;
        const int64_t o2 = f % g.O[2]; f /= g.O[2];
        const int64_t o1 = f % g.O[1]; f /= g.O[1];
        const int64_t o0 = f % g.O[0]; f /= g.O[0];
        const int64_t oc = f % g.Cout;
        const int64_t n = f / g.Cout;
        float acc = conv_one(x, w, g, n, oc, o0, o1, o2);
        if (bias) acc += bias[oc];
        y[idx] = acc;
    }
}

// The same for a 3x3x3 kernel: the 27 taps of an input channel are unrolled,
// so their loads issue together (the loop above waits for one weight and one
// input value per tap), and the index arithmetic is 32-bit (the launcher
// checks the sizes).  Taps outside the input are skipped as above, so the
// sum is formed in the same order.
__global__ __launch_bounds__(kBlock) void conv3d_k3_direct_kernel(const float* __restrict__ x,
                                                                  const float* __restrict__ w,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ y, Geom g, int32_t total) {
    const int O0 = (int)g.O[0], O1 = (int)g.O[1], O2 = (int)g.O[2];
    const int S0 = (int)g.S[0], S1 = (int)g.S[1], S2 = (int)g.S[2];
    const int Cout = (int)g.Cout, Cin = (int)g.Cin, cin_g = (int)g.cin_g, cout_g = (int)g.cout_g;
    const int64_t plane = (int64_t)S0 * S1 * S2;
    for (int idx = (int)(blockIdx.x * blockDim.x + threadIdx.x); idx < total; idx += (int)(gridDim.x * blockDim.x)) {
        int f = idx;
        const int o2 = f % O2;
        f /= O2;
        const int o1 = f % O1;
        f /= O1;
        const int o0 = f % O0;
        f /= O0;
        const int oc = f % Cout;
        const int n = f / Cout;
        const int grp = oc / cout_g;
        // the taps' offsets in an input plane, and whether they are inside it
        int off[27];
        bool ok[27];
#pragma unroll
        for (int k0 = 0; k0 < 3; ++k0)
#pragma unroll
            for (int k1 = 0; k1 < 3; ++k1)
#pragma unroll
                for (int k2 = 0; k2 < 3; ++k2) {
                    const int t = (k0 * 3 + k1) * 3 + k2;
                    const int i0 = o0 * g.s[0] - g.p[0] + k0 * g.d[0];
                    const int i1 = o1 * g.s[1] - g.p[1] + k1 * g.d[1];
                    const int i2 = o2 * g.s[2] - g.p[2] + k2 * g.d[2];
                    ok[t] = i0 >= 0 && i0 < S0 && i1 >= 0 && i1 < S1 && i2 >= 0 && i2 < S2;
                    // formed from in-range coordinates only, so it stays below the plane size
                    off[t] = ((ok[t] ? i0 : 0) * S1 + (ok[t] ? i1 : 0)) * S2 + (ok[t] ? i2 : 0);
                }
        float acc = 0.f;
        for (int icg = 0; icg < cin_g; ++icg) {
            const float* xc = x + (int64_t)(n * Cin + grp * cin_g + icg) * plane;
            const float* wc = w + (int64_t)(oc * cin_g + icg) * 27;
            float v[27];
#pragma unroll
            for (int t = 0; t < 27; ++t) v[t] = xc[off[t]];
#pragma unroll
            for (int t = 0; t < 27; ++t) acc = ok[t] ? fmaf(wc[t], v[t], acc) : acc;
        }
        if (bias) acc += bias[oc];
        y[idx] = acc;
    }
}

__global__ __launch_bounds__(kBlock) void convT_gather_kernel(const float* __restrict__ x,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ y, Geom g, int64_t total) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        int64_t f = idx;
        const int64_t o2 = f % g.O[2]; f /= g.O[2];
        const int64_t o1 = f % g.O[1]; f /= g.O[1];
        const int64_t o0 = f % g.O[0]; f /= g.O[0];
        const int64_t oc = f % g.Cout;
        const int64_t n = f / g.Cout;
        float acc = convT_one(x, w, g, n, oc, o0, o1, o2);
        if (bias) acc += bias[oc];
        y[idx] = acc;
    }
}

// Conv -> max pool -> channel logsumexp -> ReLU, one thread per pooled output.
// The logsumexp is evaluated in the streaming form with the running maximum
// started from the first channel, so no -inf - (-inf) can occur ("Kimi-K2.6
// l2_p43", the branchless streaming update and its initialisation caveat).
__global__ __launch_bounds__(kBlock) void conv_pool_lse_relu_direct_kernel(const float* __restrict__ x,
                                                                           const float* __restrict__ w,
                                                                           const float* __restrict__ bias,
                                                                           float* __restrict__ y, PoolGeom pg,
                                                                           int64_t total) {
    const Geom& g = pg.g;
    const int pool = pg.pool;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        int64_t f = idx;
        const int64_t j2 = f % pg.P[2]; f /= pg.P[2];
        const int64_t j1 = f % pg.P[1]; f /= pg.P[1];
        const int64_t j0 = f % pg.P[0];
        const int64_t n = f / pg.P[0];
        float run_max = 0.f, run_sum = 0.f;
        for (int64_t oc = 0; oc < g.Cout; ++oc) {
            float m = -FLT_MAX;
            for (int u0 = 0; u0 < pool; ++u0)
                for (int u1 = 0; u1 < pool; ++u1)
                    for (int u2 = 0; u2 < pool; ++u2) {
                        float v = conv_one(x, w, g, n, oc, j0 * pool + u0, j1 * pool + u1, j2 * pool + u2);
                        if (bias) v += bias[oc];
                        m = fmaxf(m, v);
                    }
            if (oc == 0) {
                run_max = m;
                run_sum = 1.f;
            } else {
                const float nm = fmaxf(run_max, m);
                run_sum = run_sum * expf(run_max - nm) + expf(m - nm);
                run_max = nm;
            }
        }
        const float l = run_max + logf(run_sum);
        y[idx] = l > 0.f ? l : 0.f;
    }
}

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Block-wide sum of two doubles; result valid in thread 0.
__device__ __forceinline__ void block_sum2(double& a, double& b) {
    __shared__ double sa[kBlock / 64], sb[kBlock / 64];
    a = wave_sum(a);
    b = wave_sum(b);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 0) {
        sa[wv] = a;
        sb[wv] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) {
            a += sa[i];
            b += sb[i];
        }
    }
}

// Phase 1 of convT_bn_avgpool, generic: one thread per cell of pool^3
// transposed-conv outputs (cells tile the whole output; the last cell of a
// dim may be partial and is then used for the statistics only).  The bias is
// left out: it shifts every output of a channel and its batch mean equally,
// so it cancels from the normalised result ("Kimi-K2.6 l2_p72": BN on the
// conv output, and the commuting of the per-channel affine map with the
// linear average pool, which lets the affine map act on pooled sums).
// Blocks are ordered channel-major so a channel's partials are contiguous.
__global__ __launch_bounds__(kBlock) void convT_bn_pool_phase1_direct_kernel(const float* __restrict__ x,
                                                                             const float* __restrict__ w,
                                                                             float* __restrict__ y,
                                                                             double* __restrict__ ws,
                                                                             PoolGeom pg, int64_t blocks_per_plane,
                                                                             BnEval ev) {
    const Geom& g = pg.g;
    const int pool = pg.pool;
    const int64_t b = blockIdx.x;
    const int64_t c = b / (g.N * blocks_per_plane);
    const int64_t n = (b / blocks_per_plane) % g.N;
    const int64_t cell = (b % blocks_per_plane) * kBlock + threadIdx.x;
    const int64_t cells = pg.C[0] * pg.C[1] * pg.C[2];
    double s1 = 0.0, s2 = 0.0;
    if (cell < cells) {
        const int64_t c2 = cell % pg.C[2];
        const int64_t c1 = (cell / pg.C[2]) % pg.C[1];
        const int64_t c0 = cell / (pg.C[2] * pg.C[1]);
        float win = 0.f;
        for (int u0 = 0; u0 < pool; ++u0) {
            const int64_t o0 = c0 * pool + u0;
            if (o0 >= g.O[0]) break;
            for (int u1 = 0; u1 < pool; ++u1) {
                const int64_t o1 = c1 * pool + u1;
                if (o1 >= g.O[1]) break;
                for (int u2 = 0; u2 < pool; ++u2) {
                    const int64_t o2 = c2 * pool + u2;
                    if (o2 >= g.O[2]) break;
                    const float t = convT_one(x, w, g, n, c, o0, o1, o2);
                    win += t;
                    s1 += (double)t;
                    s2 += (double)t * (double)t;
                }
            }
        }
        if (c0 < pg.P[0] && c1 < pg.P[1] && c2 < pg.P[2]) {
            const float inv = 1.f / (float)(pool * pool * pool);
            float v = win * inv;
            if (ev.gamma) {  // eval mode: the final output
                float sc, sh;
                bn_eval_affine(ev, c, sc, sh);
                v = fmaf(v, sc, sh);
            }
            y[((n * g.Cout + c) * pg.P[0] + c0) * pg.P[1] * pg.P[2] + c1 * pg.P[2] + c2] = v;
        }
    }
    if (ev.gamma) return;  // workgroup-uniform: eval mode keeps no statistics
    block_sum2(s1, s2);
    if (threadIdx.x == 0) {
        const int64_t part = c * (g.N * blocks_per_plane) + n * blocks_per_plane + (b % blocks_per_plane);
        ws[2 * part] = s1;
        ws[2 * part + 1] = s2;
    }
}

// Phase 2: each block merges its channel's partials in float64 (redundantly
// across the blocks of that channel), forms mean and biased variance, and
// applies gamma*(v - mean)/sqrt(var + eps) + beta to the pooled values of a
// run of samples.  A sample's pooled values of one channel are one contiguous
// plane, so a block reads and writes whole planes with coalesced accesses,
// issuing a batch of loads before their stores.
__global__ __launch_bounds__(kBlock) void bn_pool_phase2_kernel(float* __restrict__ y,
                                                                const double* __restrict__ ws,
                                                                int64_t parts, const float* __restrict__ conv_bias,
                                                                const float* __restrict__ gamma,
                                                                const float* __restrict__ beta, float eps,
                                                                float* __restrict__ mean_out,
                                                                float* __restrict__ var_out, BnRunning run,
                                                                PoolGeom pg, int64_t blocks_per_channel,
                                                                int64_t count) {
    __shared__ float s_scale, s_shift;
    const Geom& g = pg.g;
    const int64_t c = blockIdx.x / blocks_per_channel;
    const int64_t q = blockIdx.x % blocks_per_channel;
    constexpr int kBatch = 16;
    const int64_t pp = pg.P[0] * pg.P[1] * pg.P[2];
    const int64_t spb = ceil_div(g.N, blocks_per_channel);
    const int64_t n0 = q * spb, n1 = n0 + spb < g.N ? n0 + spb : g.N;
    // the first batch of this block's pooled values does not depend on the
    // statistics: its loads are issued before the partials are merged, so the
    // two round trips overlap
    float v0[kBatch];
    if (n0 < n1) {
        const float* yp = y + (n0 * g.Cout + c) * pp;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t j = u * kBlock + threadIdx.x;
            if (j < pp) v0[u] = yp[j];
        }
    }
    double a = 0.0, b2 = 0.0;
    const double* pc = ws + 2 * c * parts;
    for (int64_t i = threadIdx.x; i < parts; i += blockDim.x) {
        a += pc[2 * i];
        b2 += pc[2 * i + 1];
    }
    block_sum2(a, b2);
    if (threadIdx.x == 0) {
        const double mean = a / (double)count;
        double var = b2 / (double)count - mean * mean;
        if (var < 0.0) var = 0.0;
        const double sc = (double)gamma[c] / sqrt(var + (double)eps);
        s_scale = (float)sc;
        s_shift = (float)((double)beta[c] - mean * sc);
        if (q == 0) {
            const double true_mean = mean + (conv_bias ? (double)conv_bias[c] : 0.0);
            if (mean_out) mean_out[c] = (float)true_mean;
            if (var_out) var_out[c] = (float)var;
            if (run.mean) {  // count > 1 is checked on the host
                const double m = (double)run.momentum;
                run.mean[c] = (float)((1.0 - m) * (double)run.mean[c] + m * true_mean);
                run.var[c] = (float)((1.0 - m) * (double)run.var[c] + m * var * (double)count / (double)(count - 1));
            }
        }
    }
    __syncthreads();
    const float sc = s_scale, sh = s_shift;
    for (int64_t n = n0; n < n1; ++n) {
        float* yp = y + (n * g.Cout + c) * pp;  // this sample's plane of channel c
        for (int64_t j0 = 0; j0 < pp; j0 += (int64_t)kBatch * kBlock) {
            float v[kBatch];
            if (n == n0 && j0 == 0) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u) v[u] = v0[u];
            } else {
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int64_t j = j0 + u * kBlock + threadIdx.x;
                    if (j < pp) v[u] = yp[j];
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t j = j0 + u * kBlock + threadIdx.x;
                if (j < pp) yp[j] = fmaf(v[u], sc, sh);
            }
        }
    }
}

inline unsigned grid_for(int64_t total) {
    int64_t b = ceil_div(total, kBlock);
    if (b > (int64_t)1 << 20) b = (int64_t)1 << 20;
    if (b < 1) b = 1;
    return (unsigned)b;
}

}  // namespace

hipError_t launch_conv3d_direct(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                hipStream_t st) {
    const int64_t total = g.N * g.Cout * g.O[0] * g.O[1] * g.O[2];
    const bool k3 = g.k[0] == 3 && g.k[1] == 3 && g.k[2] == 3;
    // 32-bit arithmetic in the 3x3x3 kernel: output index, sample-channel index,
    // weight row, and every input coordinate it forms
    const int64_t reach = 2 * (int64_t)g.d[0] + 2 * (int64_t)g.d[1] + 2 * (int64_t)g.d[2];
    const bool small = total < (1ll << 30) && g.N * g.Cin < (1ll << 31) && g.Cout * g.cin_g < (1ll << 26) &&
                       g.S[0] * g.S[1] * g.S[2] < (1ll << 31) &&
                       (g.O[0] + g.O[1] + g.O[2]) * 4 * (int64_t)(g.s[0] + g.s[1] + g.s[2]) + reach < (1ll << 30);
    if (k3 && small)
        hipLaunchKernelGGL(conv3d_k3_direct_kernel, dim3(grid_for(total)), dim3(kBlock), 0, st, x, w, bias, y, g,
                           (int32_t)total);
    else
        hipLaunchKernelGGL(conv3d_direct_kernel, dim3(grid_for(total)), dim3(kBlock), 0, st, x, w, bias, y, g, total);
    return hipGetLastError();
}

hipError_t launch_convT_gather(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                               hipStream_t st) {
    const int64_t total = g.N * g.Cout * g.O[0] * g.O[1] * g.O[2];
    hipLaunchKernelGGL(convT_gather_kernel, dim3(grid_for(total)), dim3(kBlock), 0, st, x, w, bias, y, g, total);
    return hipGetLastError();
}

hipError_t launch_conv_pool_lse_relu_direct(const float* x, const float* w, const float* bias, float* y,
                                            const PoolGeom& pg, hipStream_t st) {
    const int64_t total = pg.g.N * pg.P[0] * pg.P[1] * pg.P[2];
    hipLaunchKernelGGL(conv_pool_lse_relu_direct_kernel, dim3(grid_for(total)), dim3(kBlock), 0, st, x, w, bias,
                       y, pg, total);
    return hipGetLastError();
}

size_t convT_bn_pool_partials(const PoolGeom& pg, int fast) {
    // partials per channel; the fast phase-1 kernel uses the same block shape
    (void)fast;
    const int64_t cells = pg.C[0] * pg.C[1] * pg.C[2];
    return (size_t)(pg.g.N * ceil_div(cells, kBlock));
}

hipError_t launch_convT_bn_pool_phase1_direct(const float* x, const float* w, float* y, double* ws,
                                              const PoolGeom& pg, const BnEval& ev, hipStream_t st) {
    const int64_t cells = pg.C[0] * pg.C[1] * pg.C[2];
    const int64_t bpp = ceil_div(cells, kBlock);
    const int64_t blocks = pg.g.Cout * pg.g.N * bpp;
    hipLaunchKernelGGL(convT_bn_pool_phase1_direct_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, x, w, y,
                       ws, pg, bpp, ev);
    return hipGetLastError();
}

hipError_t launch_bn_pool_phase2(float* y, const double* ws, int64_t parts_per_channel, const float* conv_bias,
                                 const float* gamma, const float* beta, float eps, float* mean_out,
                                 float* var_out, const BnRunning& run, const PoolGeom& pg, hipStream_t st) {
    // runs of samples of one channel, about 1024 blocks in all (every block
    // also merges its channel's partials)
    int64_t bpc = ceil_div(1024, pg.g.Cout);
    if (bpc > pg.g.N) bpc = pg.g.N;
    bpc = ceil_div(pg.g.N, ceil_div(pg.g.N, bpc));  // no block without a sample
    const int64_t count = pg.g.N * pg.g.O[0] * pg.g.O[1] * pg.g.O[2];
    hipLaunchKernelGGL(bn_pool_phase2_kernel, dim3((unsigned)(bpc * pg.g.Cout)), dim3(kBlock), 0, st, y, ws,
                       parts_per_channel, conv_bias, gamma, beta, eps, mean_out, var_out, run, pg, bpc, count);
    return hipGetLastError();
}

}  // namespace c3d
