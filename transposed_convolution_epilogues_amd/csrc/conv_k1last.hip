// conv_k1last.hip - Conv3d whose last kernel extent is 1 (the (k,k,1) kernel
// on a depth-last tensor x[N,C,H,W,D], "Kimi-K2.6 l1_p59"), stride 1, no
// padding.
//
// With k2 = 1 the last dim is never mixed, so for fixed (n, c, row i0) the
// (i1, i2) plane is one contiguous run and an output row (n, oc, o0) is the
// contiguous run j = o1*S2 + o2 of O1*S2 floats.  Every tap (ic, k0, k1) reads
// that run shifted by k1*d1*S2 from input row o0 + k0*d0 of channel ic - the
// page's observation that D is the fastest dim, taken to its end: the whole
// (w, d) plane is one 1-D axis and no layout transform is needed.
//
// GEMM per output row: D[oc, j] = sum_k W[oc, k] * B[k, j], K = Cin*k0*k1
// (27 for the (3,3,1) kernel on 3 channels, padded to an even count).  On
// v_mfma_f32_32x32x2f32 the rows are output channels (the weights stay in
// VGPRs for the whole kernel) and the columns are 32 consecutive j, so each
// store instruction writes two full 128-byte runs.  One wave owns one output
// row of 64 channels and walks it in blocks of 64 positions.  The work is
// bound by the 2.6 GB of output stores; the MFMA work runs underneath them.
#include "c3d_internal.h"

namespace c3d {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kMaxSteps = 16;  // K <= 32

struct K1Args {
    const float* x;
    const float* w;
    const float* bias;
    float* y;
    int64_t N, Cin, Cout;
    int64_t S0, S1S2;   // input rows and row length (S1*S2)
    int64_t O0, J;      // output rows and row length (O1*S2)
    int32_t K, k0n, k1n, d0, d1S2;
    int32_t ocb;        // blocks of 64 output channels
};

template <int kSteps, bool kBias>
__global__ __launch_bounds__(kThreads) void conv_k1last_kernel(K1Args a) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, r = lane & 31;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t rows = a.N * a.ocb * a.O0;
    if (row >= rows) return;
    const int64_t o0 = row % a.O0;
    const int64_t ocb = (row / a.O0) % a.ocb;
    const int64_t n = row / (a.O0 * a.ocb);

    // A operand (weights), kept for the whole row: lane holds W[oc][k] with
    // oc = 64*ocb + 32*mt + r and k = 2s + h
    float wa[2][kSteps];
    int boff[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int k = 2 * s + h;
        const bool kv = k < a.K;
        const int k1 = kv ? k % a.k1n : 0;
        const int k0 = kv ? (k / a.k1n) % a.k0n : 0;
        const int ic = kv ? k / (a.k1n * a.k0n) : 0;
        boff[s] = kv ? (int)(((int64_t)ic * a.S0 + (int64_t)k0 * a.d0) * a.S1S2 + (int64_t)k1 * a.d1S2) : -1;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int64_t oc = 64 * ocb + 32 * mt + r;
            wa[mt][s] = (kv && oc < a.Cout) ? a.w[oc * a.K + k] : 0.f;
        }
    }
    // bias of the 32 output channels whose accumulators this lane holds
    float brow[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t oc = 64 * ocb + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
            brow[mt][i] = (kBias && oc < a.Cout) ? a.bias[oc] : 0.f;
        }

    const float* xb = a.x + (n * a.Cin * a.S0 + o0) * a.S1S2;
    float* yb = a.y + ((n * a.Cout + 64 * ocb) * a.O0 + o0) * a.J;
    const int64_t ystride = a.O0 * a.J;  // between output channels

    for (int64_t j0 = 0; j0 < a.J; j0 += 64) {
        float bx[2][kSteps];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int64_t j = j0 + 32 * nt + r;
            const float* p = xb + j;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) bx[nt][s] = (boff[s] >= 0 && j < a.J) ? p[boff[s]] : 0.f;
        }
        f32x16 acc[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[mt][s], bx[nt][s], acc[mt][nt], 0, 0, 0);
        // result: lane holds D[oc = 32mt + 8(i/4) + 4h + i%4][j = j0 + 32nt + r]
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int64_t j = j0 + 32 * nt + r;
            if (j >= a.J) continue;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int oc = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (64 * ocb + oc < a.Cout) yb[oc * ystride + j] = kBias ? acc[mt][nt][i] + brow[mt][i] : acc[mt][nt][i];
                }
        }
    }
}

}  // namespace

bool conv_k1last_supported(const Geom& g, const void*, const void*, const void*) {
    if (g.k[2] != 1 || g.groups != 1) return false;
    for (int j = 0; j < 3; ++j)
        if (g.s[j] != 1 || g.p[j] != 0) return false;
    const int64_t K = g.Cin * g.k[0] * g.k[1];
    // MFMA pays off with many output channels; K must fit the VGPR-resident weights
    return K >= 2 && K <= 2 * kMaxSteps && g.Cout >= 16 && g.S[1] * g.S[2] < (1ll << 30) &&
           g.Cin * g.S[0] * g.S[1] * g.S[2] < (1ll << 31);
}

hipError_t launch_conv_k1last(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                              hipStream_t st) {
    K1Args a{};
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.N = g.N;
    a.Cin = g.Cin;
    a.Cout = g.Cout;
    a.S0 = g.S[0];
    a.S1S2 = g.S[1] * g.S[2];
    a.O0 = g.O[0];
    a.J = g.O[1] * g.S[2];
    a.K = (int32_t)(g.Cin * g.k[0] * g.k[1]);
    a.k0n = g.k[0];
    a.k1n = g.k[1];
    a.d0 = g.d[0];
    a.d1S2 = (int32_t)(g.d[1] * g.S[2]);
    a.ocb = (int32_t)ceil_div(g.Cout, 64);
    const int64_t rows = g.N * a.ocb * g.O[0];
    const int64_t blocks = ceil_div(rows, kThreads / 64);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const int steps = (a.K + 1) / 2;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (steps <= 8) {
        if (bias) hipLaunchKernelGGL((conv_k1last_kernel<8, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((conv_k1last_kernel<8, false>), grid, block, 0, st, a);
    } else if (steps <= 14) {
        if (bias) hipLaunchKernelGGL((conv_k1last_kernel<14, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((conv_k1last_kernel<14, false>), grid, block, 0, st, a);
    } else {
        if (bias) hipLaunchKernelGGL((conv_k1last_kernel<16, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((conv_k1last_kernel<16, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace c3d
