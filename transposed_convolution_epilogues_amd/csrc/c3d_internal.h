// c3d_internal.h - geometry block and launch declarations shared by the HIP
// translation units of the library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace c3d {

// Resolved geometry of one convolution call (direct or transposed).
// S = input spatial dims, O = output spatial dims (before any pooling).
struct Geom {
    int64_t N, Cin, Cout;
    int64_t S[3];
    int64_t O[3];
    int32_t k[3], s[3], p[3], d[3];
    int32_t groups, cin_g, cout_g;
};

// Geometry plus pooled dims for the fused epilogues.
struct PoolGeom {
    Geom g;
    int32_t pool;      // window = stride
    int64_t P[3];      // pooled dims (floor)
    int64_t C[3];      // cells per dim = ceil(O / pool): pooled windows plus a partial tail cell
};

// ------------------------------------------------------------ generic paths
hipError_t launch_conv3d_direct(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                hipStream_t st);
hipError_t launch_convT_gather(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                               hipStream_t st);
hipError_t launch_conv_pool_lse_relu_direct(const float* x, const float* w, const float* bias, float* y,
                                            const PoolGeom& pg, hipStream_t st);

// convT_bn_avgpool: phase 1 writes pre-normalisation pooled means into y and
// per-block (sum, sum of squares) partials in float64 into ws; phase 2 merges
// the partials per channel and applies the affine map in place (and blends
// the batch statistics into the running ones when asked).
//
// Eval-mode BatchNorm: when gamma is set, phase 1 writes the final output
// gamma_c (avg + bias_c - mean_c) / sqrt(var_c + eps) + beta_c with the
// running statistics (the BN affine commutes with the linear average pool)
// and computes no partials; ws is not used and phase 2 does not run.
struct BnEval {
    const float* gamma;
    const float* beta;
    const float* mean;
    const float* var;
    const float* bias;
    float eps;
};

// scale and shift of the eval-mode map for channel c
__device__ inline void bn_eval_affine(const BnEval& ev, int64_t c, float& sc, float& sh) {
    const double s = (double)ev.gamma[c] / sqrt((double)ev.var[c] + (double)ev.eps);
    sc = (float)s;
    sh = (float)((double)ev.beta[c] + ((ev.bias ? (double)ev.bias[c] : 0.0) - (double)ev.mean[c]) * s);
}

// Running-statistics update of phase 2 (training mode): with m = momentum,
// mean <- (1 - m) mean + m * batch mean, var <- (1 - m) var + m * unbiased batch var.
struct BnRunning {
    float* mean;
    float* var;
    float momentum;
};

size_t convT_bn_pool_partials(const PoolGeom& pg, int fast);

// matrix-core throughput probe (mfma_probe.hip)
constexpr int kProbeWorkgroups = 2048;
int64_t mfma_probe_out_len();
int64_t mfma_probe_flop(int64_t iters);
hipError_t launch_mfma_probe(int64_t iters, float* out, hipStream_t st);
bool mfma_valu_probe_supported(int32_t valu_per_4);
hipError_t launch_mfma_valu_probe(int64_t iters, int32_t valu_per_4, float* out, hipStream_t st);
hipError_t launch_convT_bn_pool_phase1_direct(const float* x, const float* w, float* y, double* ws,
                                              const PoolGeom& pg, const BnEval& ev, hipStream_t st);
hipError_t launch_bn_pool_phase2(float* y, const double* ws, int64_t parts_per_channel, const float* conv_bias,
                                 const float* gamma, const float* beta, float eps, float* mean_out,
                                 float* var_out, const BnRunning& run, const PoolGeom& pg, hipStream_t st);

// ------------------------------------------------------------- fast paths
// Each returns hipErrorNotSupported (without launching) when the geometry is
// outside what the kernel handles; the caller then takes the generic path.
bool conv3x3x3_mfma_supported(const Geom& g, const void* x, const void* w, const void* y);
hipError_t launch_conv3x3x3_mfma(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                 hipStream_t st);
bool conv_pool_lse_mfma_supported(const PoolGeom& pg, const void* x, const void* w);
hipError_t launch_conv_pool_lse_mfma(const float* x, const float* w, const float* bias, float* y,
                                     const PoolGeom& pg, hipStream_t st);
bool convT_s2_sublattice_supported(const Geom& g, const void* x, const void* w, const void* y);
hipError_t launch_convT_s2_sublattice(const float* x, const float* w, const float* bias, float* y,
                                      const Geom& g, hipStream_t st);
bool convT_phase_mfma_supported(const Geom& g, const void* x, const void* w, const void* y);
hipError_t launch_convT_phase_mfma(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                   hipStream_t st);
bool convT_phasegroup_supported(const Geom& g);
hipError_t launch_convT_phasegroup(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                   hipStream_t st);
bool convT_scatter_supported(const Geom& g);
hipError_t launch_convT_scatter(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                hipStream_t st);
bool conv_k1last_supported(const Geom& g, const void* x, const void* w, const void* y);
hipError_t launch_conv_k1last(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                              hipStream_t st);
// The page's module (k3 s2 p1, pool 4, Cin <= 3, Cout <= 32) with the sums
// swapped: pooled sums from summed weights on the matrix cores, batch
// statistics from lag correlations of the input and Gram matrices of its
// boundary.  Training mode (tr set) runs the whole module: it writes the
// normalised y, the batch statistics and the running update, using ws
// (convT_bn_swap_workspace_bytes, 8-byte aligned); eval mode (ev.gamma set)
// writes y with the running statistics and uses no workspace.
struct BnSwapTrain {
    const float* bias;
    const float* gamma;
    const float* beta;
    float eps;
    float* mean_out;
    float* var_out;
    BnRunning run;
};
bool convT_bn_swap_supported(const PoolGeom& pg, const void* x);
size_t convT_bn_swap_workspace_bytes(const PoolGeom& pg);
hipError_t launch_convT_bn_swap(const float* x, const float* w, float* y, void* ws, const PoolGeom& pg,
                                const BnEval& ev, const BnSwapTrain* tr, hipStream_t st);
bool convT_bn_pool_fast_supported(const PoolGeom& pg, const void* x);
bool convT_bn_pool_mfma_supported(const PoolGeom& pg, const void* x);
size_t convT_bn_pool_mfma_partials(const PoolGeom& pg);
hipError_t launch_convT_bn_pool_phase1_mfma(const float* x, const float* w, float* y, double* ws,
                                            const PoolGeom& pg, const BnEval& ev, hipStream_t st);
hipError_t launch_convT_bn_pool_phase1_fast(const float* x, const float* w, float* y, double* ws,
                                            const PoolGeom& pg, const BnEval& ev, hipStream_t st);

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace c3d
