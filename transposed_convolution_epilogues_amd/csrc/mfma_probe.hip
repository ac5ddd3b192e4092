// mfma_probe.hip - a throughput probe of the fp32 matrix cores, to check the
// peak that the kernels' roofline fractions are quoted against.
//
// Every wave runs kChains independent accumulation chains of
// v_mfma_f32_32x32x2f32 (4096 FLOP each) back to back, with two waves per SIMD
// (2048 workgroups of 4 waves on 256 CUs).  Each thread writes the sum of its
// accumulators, so the work cannot be dropped.
#include "c3d_internal.h"

namespace c3d {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChains = 4;

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_probe_kernel(
    int64_t iters, float* out) {
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    const float a = 1e-3f * (float)(threadIdx.x & 63), b = 1.f / (float)(1 + (threadIdx.x & 7));
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// The same chains with NV independent non-MFMA VALU instructions (fp32 FMAs
// on registers the MFMAs do not touch) after every 4 MFMAs: how much VALU work
// beside the matrix cores costs them.  The FMA chains are kept by a test that
// never holds (a NaN check), so the output equals the plain probe's.
template <int NV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_valu_probe_kernel(
    int64_t iters, float* out) {
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    float t[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) t[v] = (float)(threadIdx.x + v);
    const float a = 1e-3f * (float)(threadIdx.x & 63), b = 1.f / (float)(1 + (threadIdx.x & 7));
    const float c1 = 0.999f + 1e-6f * (float)(threadIdx.x & 3), c2 = 1e-3f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < NV; ++v) t[v] = __builtin_fmaf(t[v], c1, c2);
    }
    float s = 0.f, u = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
#pragma unroll
    for (int v = 0; v < NV; ++v) u += t[v];
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = u != u ? u : s;
}

}  // namespace

bool mfma_valu_probe_supported(int32_t valu_per_4) {
    return valu_per_4 == 2 || valu_per_4 == 4 || valu_per_4 == 8 || valu_per_4 == 16;
}

hipError_t launch_mfma_valu_probe(int64_t iters, int32_t valu_per_4, float* out, hipStream_t st) {
    const dim3 g(kProbeWorkgroups), blk(kThreads);
    switch (valu_per_4) {
        case 2: hipLaunchKernelGGL(mfma_valu_probe_kernel<2>, g, blk, 0, st, iters, out); break;
        case 4: hipLaunchKernelGGL(mfma_valu_probe_kernel<4>, g, blk, 0, st, iters, out); break;
        case 8: hipLaunchKernelGGL(mfma_valu_probe_kernel<8>, g, blk, 0, st, iters, out); break;
        case 16: hipLaunchKernelGGL(mfma_valu_probe_kernel<16>, g, blk, 0, st, iters, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int64_t mfma_probe_out_len() { return (int64_t)kProbeWorkgroups * kThreads; }

int64_t mfma_probe_flop(int64_t iters) { return (int64_t)kProbeWorkgroups * (kThreads / 64) * iters * kChains * 4096; }

hipError_t launch_mfma_probe(int64_t iters, float* out, hipStream_t st) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(kProbeWorkgroups), dim3(kThreads), 0, st, iters, out);
    return hipGetLastError();
}

}  // namespace c3d
