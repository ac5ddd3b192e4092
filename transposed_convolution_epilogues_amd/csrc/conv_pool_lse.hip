// conv_pool_lse.hip - Conv3d(k3, s1, d1) -> MaxPool3d(2) -> logsumexp over
// channels -> ReLU in one kernel ("Kimi-K2.6 l2_p43": the module, and its plan
// to compute the conv tile by tile and reduce it to the pooled logsumexp in
// the epilogue instead of writing the conv output).
//
// The conv runs on the MFMA engine in conv333_mfma.h.  Epilogue per wave:
//   - 2x2x2 max pool: each lane already holds whole windows (4 registers in
//     each of the two M tiles), so the max is lane-local; the bias is added
//     after the max (max(v) + b = max(v + b)).
//   - logsumexp over the 64 channels: a channel lives in lane%32 of one of two
//     N tiles, so each lane first combines its two channels, then the max and
//     the shifted sum are reduced across the 32 lanes of its half (DPP moves
//     and one swizzle, see half_max); the running
//     maximum starts from real values, never from -inf ("Kimi-K2.6 l2_p43",
//     the streaming-logsumexp initialisation caveat).
//   - ReLU and one 4-byte store per pooled voxel.
// The 4 x 64 x 32 x 128 x 128 conv output is never written to memory.
#include "conv333_mfma.h"

namespace c3d {
namespace {

using namespace mfma333;

constexpr int kMT = 4;  // tile depth: two pooled planes per tile

// Lane permutations within each 32-lane half of the wave.  DPP moves stay in
// the ALU: quad_perm [1,0,3,2] and [2,3,0,1] pair lanes 1 and 2 apart,
// row_half_mirror pairs the two quads of each 8 (i <-> 7 - i) and row_mirror
// the two 8s of each 16 (i <-> 15 - i); one ds_swizzle in bitmask mode
// (xor 16 within 32) pairs the two 16s.  Each step pairs every lane with a
// partner from the other subset, so after all five every lane of the half
// holds the reduction over its 32 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float swizzle_xor16(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ float half_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return fmaxf(v, swizzle_xor16(v));
}
__device__ __forceinline__ float half_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v + swizzle_xor16(v);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv_pool_lse_mfma_kernel(Args a) {
    __shared__ __attribute__((aligned(16))) float lds[Geo<kMT>::LDS_MAIN];
    const Tile t = tile_of<kMT>(a);
    f32x16 acc[kMT][2];
    mainloop<kConvWeights, kMT>(a, t, lds, acc);

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int64_t j1 = (t.h0 >> 1) + (wv >> 1);
    float bias_v[2];
    bool valid[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int64_t oc = t.oc0 + nt * 32 + (lane & 31);
        valid[nt] = oc < a.Cout;
        bias_v[nt] = (a.bias && valid[nt]) ? a.bias[oc] : 0.f;
    }
    // pooled plane pd takes M tiles (D planes) 2pd and 2pd + 1.  Window
    // q = 2*(a%2) + b/2 holds registers {a%2 + 2*ay, ...}: x = 8(a%2) + 4h + b,
    // y = a/2 in {0,1}; see acc_voxel in conv333_mfma.h
#pragma unroll
    for (int pd = 0; pd < kMT / 2; ++pd) {
        const int64_t j0 = (t.d0 >> 1) + pd;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ax = q >> 1, bx = (q & 1) * 2;
            float m[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float v = -FLT_MAX;
#pragma unroll
                for (int mt = 2 * pd; mt < 2 * pd + 2; ++mt)
#pragma unroll
                    for (int ay = 0; ay < 2; ++ay)
#pragma unroll
                        for (int u = 0; u < 2; ++u) v = fmaxf(v, acc[mt][nt][(2 * ay + ax) * 4 + bx + u]);
                m[nt] = valid[nt] ? v + bias_v[nt] : -FLT_MAX;
            }
            const float M = half_max(fmaxf(m[0], m[1]));
            // the hardware exp2 / log2 (about 1 ulp each): every term lies in
            // (0, 1] and S in [1, 64], so the result is within a few 1e-7 of
            // the exactly rounded one
            const float S = half_sum(__expf(m[0] - M) + __expf(m[1] - M));
            const float L = M + __logf(S);
            if ((lane & 31) == 0) {
                const int j2 = (int)(t.w0 >> 1) + (wv & 1) * 8 + 4 * ax + 2 * h + (q & 1);
                if ((int)j0 < (int)a.P[0] && (int)j1 < (int)a.P[1] && j2 < (int)a.P[2])
                    a.y[((t.n * a.P[0] + j0) * a.P[1] + j1) * a.P[2] + j2] = L > 0.f ? L : 0.f;
            }
        }
    }
}

}  // namespace

bool conv_pool_lse_mfma_supported(const PoolGeom& pg, const void*, const void*) {
    const Geom& g = pg.g;
    for (int j = 0; j < 3; ++j)
        if (g.k[j] != 3 || g.s[j] != 1 || g.d[j] != 1 || g.p[j] != g.p[0]) return false;
    return g.groups == 1 && g.Cout <= OCB && pg.pool == 2 && mfma333::fits_buffers(g) && mfma333::fits_int32_tiles(g.O[0]) &&
           mfma333::fits_int32_tiles(g.O[1]) && mfma333::fits_int32_tiles(g.O[2]);
}

hipError_t launch_conv_pool_lse_mfma(const float* x, const float* w, const float* bias, float* y,
                                     const PoolGeom& pg, hipStream_t st) {
    const Geom& g = pg.g;
    Args a{};
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.N = g.N;
    a.Cin = g.Cin;
    a.xC = g.Cin;
    a.Cout = g.Cout;
    for (int j = 0; j < 3; ++j) {
        a.S[j] = g.S[j];
        a.O[j] = g.O[j];
        a.P[j] = pg.P[j];
    }
    for (int j = 0; j < 3; ++j) a.pad[j] = g.p[0];
    // only tiles holding at least one complete pooling window are needed
    a.tiles[0] = (int32_t)ceil_div(2 * pg.P[0], Geo<kMT>::TD);
    a.tiles[1] = (int32_t)ceil_div(2 * pg.P[1], TH);
    a.tiles[2] = (int32_t)ceil_div(2 * pg.P[2], TW);
    a.oc_blocks = 1;
    const int64_t blocks = g.N * a.tiles[0] * a.tiles[1] * a.tiles[2];
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(conv_pool_lse_mfma_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace c3d
