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
// VGPRs for the whole kernel) and the columns are output positions.  One wave
// owns one output row of 64 channels and walks it in blocks of 128 positions
// (four N tiles).  The work is bound by the 2.6 GB of output stores, so the
// column-to-position map is chosen for the store shape (see load_block); the
// MFMA work runs underneath the stores.
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

__device__ __forceinline__ float ld(const float* base, uint32_t idx) {
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + (size_t)(idx * 4u));
}

// Block of 128 output positions.  N tile t's column c is position j0 + 4c + t,
// so after the MFMAs a lane holds 4 consecutive positions of each of its 16
// channels per M tile, and one 16-byte store per channel covers them: lanes
// 0-31 then write 512 contiguous bytes of one channel row and lanes 32-63 of
// another.  Measured on MI355X this store shape runs at ~6.3 TB/s, against
// ~2.2 TB/s for one 4-byte column per lane.
template <int kSteps>
__device__ __forceinline__ void load_block(const float* xb, const uint32_t (&off)[kSteps], int64_t j0, int r,
                                           int64_t J, float (&bx)[4][kSteps]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        int64_t j = j0 + 4 * r + t;
        j = j < J ? j : J - 1;  // positions past the row end are computed but never stored
#pragma unroll
        for (int s = 0; s < kSteps; ++s) bx[t][s] = ld(xb, off[s] + (uint32_t)j);
    }
}

template <bool kBias, bool kVec, bool kFull>
__device__ __forceinline__ void store_block(float* yb, uint32_t ystride, const f32x16 (&acc)[2][4],
                                            const float (&brow)[2][16], int64_t j0, int r, int h, int64_t J,
                                            int64_t Cout, int64_t oc0) {
    const int64_t j = j0 + 4 * r;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int oc = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = kBias ? acc[mt][t][i] + brow[mt][i] : acc[mt][t][i];
            char* dst = reinterpret_cast<char*>(yb) + (size_t)(((uint32_t)oc * ystride + (uint32_t)j) * 4u);
            const bool oc_ok = kFull || oc0 + oc < Cout;
            if (kVec) {
                // J % 4 == 0 and 16-byte aligned rows: a lane's 4 positions are all in or all out
                if (kFull || (oc_ok && j < J)) *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (kFull || (oc_ok && j + t < J)) reinterpret_cast<float*>(dst)[t] = v[t];
            }
        }
}

template <int kSteps, bool kBias, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv_k1last_kernel(
    K1Args a) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, r = lane & 31;
    // the wave index is uniform across the wave: keep the row bases in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    const int64_t rows = a.N * a.ocb * a.O0;
    if (row >= rows) return;
    const int64_t o0 = row % a.O0;
    const int64_t ocb = (row / a.O0) % a.ocb;
    const int64_t n = row / (a.O0 * a.ocb);

    // A operand (weights), kept for the whole row: lane holds W[oc][k] with
    // oc = 64*ocb + 32*mt + r and k = 2s + h.  Padding rows k >= K get a zero
    // weight and read a valid input element, so no load is predicated.
    float wa[2][kSteps];
    uint32_t off[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int k = 2 * s + h;
        const bool kv = k < a.K;
        const int kk = kv ? k : 0;
        const int k1 = kk % a.k1n;
        const int k0 = (kk / a.k1n) % a.k0n;
        const int ic = kk / (a.k1n * a.k0n);
        off[s] = (uint32_t)((ic * a.S0 + k0 * a.d0) * a.S1S2 + k1 * a.d1S2);
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
    const bool all_oc = 64 * (ocb + 1) <= a.Cout;

    const float* xb = a.x + (n * a.Cin * a.S0 + o0) * a.S1S2;
    float* yb = a.y + ((n * a.Cout + 64 * ocb) * a.O0 + o0) * a.J;
    const uint32_t ystride = (uint32_t)(a.O0 * a.J);  // between output channels

    for (int64_t j0 = 0; j0 < a.J; j0 += 128) {
        float bx[4][kSteps];
        load_block<kSteps>(xb, off, j0, r, a.J, bx);
        f32x16 acc[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mt][t][i] = 0.f;
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[mt][s], bx[t][s], acc[mt][t], 0, 0, 0);
        if (all_oc && j0 + 128 <= a.J)
            store_block<kBias, kVec, true>(yb, ystride, acc, brow, j0, r, h, a.J, 0, 0);
        else
            store_block<kBias, kVec, false>(yb, ystride, acc, brow, j0, r, h, a.J, a.Cout, 64 * ocb);
    }
}

}  // namespace

bool conv_k1last_supported(const Geom& g, const void*, const void*, const void*) {
    if (g.k[2] != 1 || g.groups != 1) return false;
    for (int j = 0; j < 3; ++j)
        if (g.s[j] != 1 || g.p[j] != 0) return false;
    const int64_t K = g.Cin * g.k[0] * g.k[1];
    // MFMA pays off with many output channels; K must fit the VGPR-resident weights
    // 32-bit element offsets: within one image's input, and within 64 output channels
    return K >= 2 && K <= 2 * kMaxSteps && g.Cout >= 16 && g.Cin * g.S[0] * g.S[1] * g.S[2] < (1ll << 30) &&
           64 * g.O[0] * g.O[1] * g.S[2] < (1ll << 30);
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
    const bool vec = (a.J % 4 == 0) && ((uintptr_t)y % 16 == 0);
    const dim3 grid((unsigned)blocks), block(kThreads);
#define C3D_K1_LAUNCH(S)                                                                               \
    do {                                                                                               \
        if (bias) {                                                                                    \
            if (vec) hipLaunchKernelGGL((conv_k1last_kernel<S, true, true>), grid, block, 0, st, a);  \
            else hipLaunchKernelGGL((conv_k1last_kernel<S, true, false>), grid, block, 0, st, a);     \
        } else {                                                                                       \
            if (vec) hipLaunchKernelGGL((conv_k1last_kernel<S, false, true>), grid, block, 0, st, a); \
            else hipLaunchKernelGGL((conv_k1last_kernel<S, false, false>), grid, block, 0, st, a);    \
        }                                                                                              \
    } while (0)
    if (steps <= 8) C3D_K1_LAUNCH(8);
    else if (steps <= 14) C3D_K1_LAUNCH(14);
    else C3D_K1_LAUNCH(16);
#undef C3D_K1_LAUNCH
    return hipGetLastError();
}

}  // namespace c3d
