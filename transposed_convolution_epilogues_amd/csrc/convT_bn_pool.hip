// convT_bn_pool.hip - phase 1 of convT_bn_avgpool for the page's transposed
// conv (kernel 3, stride 2, padding 1, dilation 1) with pool 4
// ("Kimi-K2.6 l2_p72").
//
// Parity tables (the page's derivation for stride 2, padding 1): output o
// takes tap k from input i = (o + 1 - k)/2, so an even o takes only tap 1
// (i = o/2) and an odd o takes taps 0 and 2 (i = (o+1)/2 and (o-1)/2).  A
// pooled window [4j, 4j+4) per dim therefore reads inputs 2j .. 2j+2 only:
// with u = o - 4j,
//   u = 0: (k=1, i=2j)      u = 1: (k=0, i=2j+1), (k=2, i=2j)
//   u = 2: (k=1, i=2j+1)    u = 3: (k=0, i=2j+2), (k=2, i=2j+1)
// i.e. 1 + 2 + 1 + 2 = 6 taps per dim and 216 MACs per input channel for
// the 64 positions of a window (the page's 648 for 3 channels).
//
// One thread owns one cell of 4x4x4 outputs (cells tile the whole output, the
// last one per dim holding the positions pooling drops) and keeps its
// 3x3x3xCin input patch in registers.  Output channels are a runtime loop, so
// the weights are wave-uniform scalar loads and the code stays small.  Per
// channel the thread forms the window sum (the pooled pre-normalisation mean
// times 64) and the float64 sum of squares of all valid positions; the bias is
// left out (it cancels from batch-statistics BN).  The 64 x 16 x 63^3 conv
// output never leaves registers.
#include "c3d_internal.h"

namespace c3d {
namespace {

constexpr int kThreads = 256;
constexpr int kRedChannels = 16;  // channels whose wave partials wait in LDS for one block reduction

__device__ __forceinline__ double wave_sum_d(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <int CIN>
__global__ __launch_bounds__(kThreads) void convT_bn_pool_phase1_kernel(const float* __restrict__ x,
                                                                        const float* __restrict__ w,
                                                                        float* __restrict__ y,
                                                                        double* __restrict__ ws, PoolGeom pg,
                                                                        int64_t blocks_per_plane, BnEval ev) {
    __shared__ double red[kRedChannels][kThreads / 64][2];
    const Geom& g = pg.g;
    const int64_t cells = pg.C[0] * pg.C[1] * pg.C[2];
    const int64_t n = blockIdx.x / blocks_per_plane;
    const int64_t bip = blockIdx.x % blocks_per_plane;
    const int64_t cell = bip * kThreads + threadIdx.x;
    const bool active = cell < cells;
    const int64_t c2 = active ? cell % pg.C[2] : 0;
    const int64_t c1 = active ? (cell / pg.C[2]) % pg.C[1] : 0;
    const int64_t c0 = active ? cell / (pg.C[2] * pg.C[1]) : 0;

    // input patch: inputs 2c + {0,1,2} per dim, zero outside x
    float p[CIN][3][3][3];
    const int64_t plane = g.S[0] * g.S[1] * g.S[2];
#pragma unroll
    for (int ic = 0; ic < CIN; ++ic)
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b)
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    const int64_t i0 = 2 * c0 + a, i1 = 2 * c1 + b, i2 = 2 * c2 + c;
                    p[ic][a][b][c] = (active && i0 < g.S[0] && i1 < g.S[1] && i2 < g.S[2])
                                         ? x[(n * CIN + ic) * plane + (i0 * g.S[1] + i1) * g.S[2] + i2]
                                         : 0.f;
                }
    // which of the 4 positions per dim lie inside the output
    bool v0[4], v1[4], v2[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        v0[u] = active && 4 * c0 + u < g.O[0];
        v1[u] = active && 4 * c1 + u < g.O[1];
        v2[u] = active && 4 * c2 + u < g.O[2];
    }
    const bool full = active && c0 < pg.P[0] && c1 < pg.P[1] && c2 < pg.P[2];
    const int64_t pplane = pg.P[0] * pg.P[1] * pg.P[2];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t parts = g.N * blocks_per_plane;

    for (int oc = 0; oc < (int)g.Cout; ++oc) {
        const float* wo = w + (int64_t)oc * 27;  // + ic * Cout * 27
        float win = 0.f;
        double sq = 0.0;
#pragma unroll
        for (int u0 = 0; u0 < 4; ++u0)
#pragma unroll
            for (int u1 = 0; u1 < 4; ++u1)
#pragma unroll
                for (int u2 = 0; u2 < 4; ++u2) {
                    // (k, patch index) lists for each dim, from the parity table above
                    const int n0 = (u0 & 1) ? 2 : 1, n1 = (u1 & 1) ? 2 : 1, n2 = (u2 & 1) ? 2 : 1;
                    float t = 0.f;
#pragma unroll
                    for (int e0 = 0; e0 < n0; ++e0)
#pragma unroll
                        for (int e1 = 0; e1 < n1; ++e1)
#pragma unroll
                            for (int e2 = 0; e2 < n2; ++e2) {
                                const int k0 = (u0 & 1) ? 2 * e0 : 1, k1 = (u1 & 1) ? 2 * e1 : 1,
                                          k2 = (u2 & 1) ? 2 * e2 : 1;
                                const int i0 = (u0 + 1 - k0) >> 1, i1 = (u1 + 1 - k1) >> 1,
                                          i2 = (u2 + 1 - k2) >> 1;
#pragma unroll
                                for (int ic = 0; ic < CIN; ++ic)
                                    t = fmaf(wo[(int64_t)ic * g.Cout * 27 + (k0 * 3 + k1) * 3 + k2],
                                             p[ic][i0][i1][i2], t);
                            }
                    if (v0[u0] && v1[u1] && v2[u2]) {
                        win += t;
                        sq = fma((double)t, (double)t, sq);
                    }
                }
        float* yo = y + (n * g.Cout + oc) * pplane + (c0 * pg.P[1] + c1) * pg.P[2] + c2;
        if (ev.gamma) {  // eval mode (workgroup-uniform): final output, no statistics
            float sc, sh;
            bn_eval_affine(ev, oc, sc, sh);
            if (full) *yo = fmaf(win * (1.f / 64.f), sc, sh);
            continue;
        }
        if (full) *yo = win * (1.f / 64.f);
        // wave partial of (sum, sum of squares) for this channel; the block
        // reduction over waves waits until every channel is done
        const double s1 = wave_sum_d((double)win);
        const double s2 = wave_sum_d(sq);
        if (lane == 0) {
            red[oc % kRedChannels][wv][0] = s1;
            red[oc % kRedChannels][wv][1] = s2;
        }
        if (oc % kRedChannels == kRedChannels - 1 || oc == (int)g.Cout - 1) {
            // flush a group of kRedChannels channels (workgroup-uniform)
            __syncthreads();
            const int base = oc - oc % kRedChannels;
            const int cnt = oc - base + 1;
            if (threadIdx.x < 2 * cnt) {
                const int c = threadIdx.x >> 1, k = threadIdx.x & 1;
                double v = 0.0;
                for (int i = 0; i < kThreads / 64; ++i) v += red[c][i][k];
                const int64_t part = (int64_t)(base + c) * parts + n * blocks_per_plane + bip;
                ws[2 * part + k] = v;
            }
            __syncthreads();
        }
    }
}

}  // namespace

bool convT_bn_pool_fast_supported(const PoolGeom& pg, const void*) {
    const Geom& g = pg.g;
    for (int j = 0; j < 3; ++j)
        if (g.k[j] != 3 || g.s[j] != 2 || g.p[j] != 1 || g.d[j] != 1 || g.O[j] != 2 * g.S[j] - 1) return false;
    return g.groups == 1 && pg.pool == 4 && g.Cin >= 1 && g.Cin <= 4 && g.Cout <= 4096;
}

hipError_t launch_convT_bn_pool_phase1_fast(const float* x, const float* w, float* y, double* ws,
                                            const PoolGeom& pg, const BnEval& ev, hipStream_t st) {
    const int64_t cells = pg.C[0] * pg.C[1] * pg.C[2];
    const int64_t bpp = ceil_div(cells, kThreads);
    const int64_t blocks = pg.g.N * bpp;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (pg.g.Cin) {
        case 1: hipLaunchKernelGGL(convT_bn_pool_phase1_kernel<1>, grid, block, 0, st, x, w, y, ws, pg, bpp, ev); break;
        case 2: hipLaunchKernelGGL(convT_bn_pool_phase1_kernel<2>, grid, block, 0, st, x, w, y, ws, pg, bpp, ev); break;
        case 3: hipLaunchKernelGGL(convT_bn_pool_phase1_kernel<3>, grid, block, 0, st, x, w, y, ws, pg, bpp, ev); break;
        default: hipLaunchKernelGGL(convT_bn_pool_phase1_kernel<4>, grid, block, 0, st, x, w, y, ws, pg, bpp, ev); break;
    }
    return hipGetLastError();
}

}  // namespace c3d
