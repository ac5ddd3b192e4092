// convT_phase.hip - ConvTranspose3d of any stride up to 4 per dim, padding,
// dilation, output padding and groups on the MFMA engine, one output phase at
// a time ("Kimi-K2.6 l1_p77", the residue-class decomposition of the gather
// form, carried through for every residue).
//
// Write each output index per dim as o = s*q + r with r = o mod s.  Tap k
// reaches o from input i = (o + p - k*d) / s, an integer exactly when
// r + p - k*d is a multiple of s, and then i = q + delta with
// delta = (r + p - k*d) / s.  So output phase r = (r0, r1, r2) is a stride-1
// correlation of the input with its own tap list, the product of the per-dim
// lists T_j(r_j) = {k : s_j divides r_j + p_j - k*d_j}; every tap belongs to
// exactly one residue per dim, so the phases together do exactly the valid
// work of the gather form.  A phase whose list is empty in some dim receives
// no tap at all and equals the bias.
//
// A workgroup computes one phase of one 4 x 4 x 32 tile of q positions x 64
// output channels of one group (mainloop_taps in conv333_mfma.h), stages the
// result in LDS 32 channels at a time and writes its outputs, which lie at
// stride s in each dim.
// The phases of a tile are consecutive workgroups, so after the XCD remap
// they run at the same time on one XCD and their interleaved writes meet in
// that XCD's L2 before they reach HBM.
//
// Supported: s_j <= 4; in every phase at most 3 taps per dim, whose input
// offsets span at most 3 consecutive positions (the engine's halo is the
// tile + 2 per dim); Cin/groups >= 4 and Cout/groups >= 8.  Other geometries
// take the gather kernel.
#include <limits.h>

#include "conv333_mfma.h"

namespace c3d {
namespace {

using namespace mfma333;

constexpr int kMT = 4;  // tile depth; the result staging (32 channels at a time) reuses the K-loop LDS
constexpr int TD = Geo<kMT>::TD;
constexpr int kStage = TD * TH * TW + 1;  // LDS floats per channel of the result staging (padded)
constexpr int kLdsFloats = Geo<kMT>::LDS_MAIN > 32 * kStage ? Geo<kMT>::LDS_MAIN : 32 * kStage;
constexpr int kMaxS = 4;                  // largest stride per dim
constexpr int kMaxT = 3;                  // most taps per dim and phase

// Tap lists of one dim, per residue r < s.
struct DimPhases {
    int32_t s;
    int32_t n[kMaxS];            // taps of residue r
    int32_t k[kMaxS][kMaxT];     // kernel index of each tap
    int32_t off[kMaxS][kMaxT];   // halo offset of each tap: delta - min delta (0..2)
    int32_t org[kMaxS];          // -min delta: the halo starts at q0 - org
    int64_t Q[kMaxS];            // outputs of residue r: ceil((O - r) / s)
};

struct PhaseArgs {
    Args a;                 // engine arguments for group 0 (a.Cin / a.Cout per group, a.xC = all channels)
    DimPhases dim[3];
    int32_t K[3];           // kernel extents
    int32_t nph;            // s0 * s1 * s2
    int32_t groups;
    int64_t yC;             // channels per sample of y
    int64_t x_gstride;      // floats between groups: x, w, y
    int64_t w_gstride;
    int64_t y_gstride;
};

__device__ __forceinline__ DimTaps dim_taps(const DimPhases& dp, int r) {
    DimTaps t;
    t.n = dp.n[r];
#pragma unroll
    for (int i = 0; i < kMaxT; ++i) {
        t.k[i] = dp.k[r][i];
        t.off[i] = dp.off[r][i];
    }
    return t;
}

// two workgroups per CU: all 256 registers per lane hold the 4-plane tile's accumulators and the prefetch
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void convT_phase_kernel(
    PhaseArgs pa) {
    __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
    __shared__ float sbias[OCB];

    // workgroup -> (n, tile, group, oc block, phase), phase fastest, after the
    // same XCD remap as tile_of
    const Args& a0 = pa.a;
    const int64_t nb = (int64_t)gridDim.x;
    int64_t b = blockIdx.x;
    if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    const int ph = (int)(b % pa.nph);
    b /= pa.nph;
    Tile t;
    t.oc0 = (b % a0.oc_blocks) * OCB;
    b /= a0.oc_blocks;
    const int64_t grp = b % pa.groups;
    b /= pa.groups;
    const int64_t tw = b % a0.tiles[2];
    b /= a0.tiles[2];
    const int64_t th = b % a0.tiles[1];
    b /= a0.tiles[1];
    const int64_t td = b % a0.tiles[0];
    t.n = b / a0.tiles[0];
    t.d0 = td * TD;
    t.h0 = th * TH;
    t.w0 = tw * TW;
    const int r2 = ph % pa.dim[2].s;
    const int r1 = (ph / pa.dim[2].s) % pa.dim[1].s;
    const int r0 = ph / (pa.dim[2].s * pa.dim[1].s);
    const int64_t Q0 = pa.dim[0].Q[r0], Q1 = pa.dim[1].Q[r1], Q2 = pa.dim[2].Q[r2];
    if (t.d0 >= Q0 || t.h0 >= Q1 || t.w0 >= Q2) return;  // the whole tile is outside this phase

    Args a = a0;
    a.x += grp * pa.x_gstride;
    a.w += grp * pa.w_gstride;
    const float* bias = a.bias ? a.bias + grp * a.Cout : nullptr;
    float* yg = a.y + grp * pa.y_gstride;

    if (threadIdx.x < OCB)
        sbias[threadIdx.x] = (bias && t.oc0 + threadIdx.x < a.Cout) ? bias[t.oc0 + threadIdx.x] : 0.f;

    TapSet ts;
    ts.d[0] = dim_taps(pa.dim[0], r0);
    ts.d[1] = dim_taps(pa.dim[1], r1);
    ts.d[2] = dim_taps(pa.dim[2], r2);
    ts.K1 = pa.K[1];
    ts.K2 = pa.K[2];
    ts.Kvol = pa.K[0] * pa.K[1] * pa.K[2];
    const bool has_taps = ts.d[0].n > 0 && ts.d[1].n > 0 && ts.d[2].n > 0;  // workgroup-uniform

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    f32x16 acc[kMT][2];
    if (has_taps) {
        const int32_t pad[3] = {pa.dim[0].org[r0], pa.dim[1].org[r1], pa.dim[2].org[r2]};
        mainloop_taps<kMT>(a, t, ts, pad, lds, acc);
    }
    const int ocs = (int)(a.Cout - t.oc0 < OCB ? a.Cout - t.oc0 : OCB);
    const int s0 = pa.dim[0].s, s1 = pa.dim[1].s, s2 = pa.dim[2].s;
    const int64_t O1 = a.Y[1], O2 = a.Y[2];
    const int x = lane & 31;
    const int64_t q2 = t.w0 + x;
    const bool x_ok = q2 < Q2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();  // every wave is done reading the operand tiles, or the previous half
        if (has_taps) {
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    int xx, y, z;
                    acc_voxel(lane, wv, mt, i, xx, y, z);
                    lds[(lane & 31) * kStage + (z * TH + y) * TW + xx] = acc[mt][half][i];
                }
        }
        __syncthreads();  // staging (and sbias) visible to every wave
        // write the half: row (oc, z, y) holds q2 = w0 + x for x < 32, at output
        // (s0 (d0 + z) + r0, s1 (h0 + y) + r1, s2 q2 + r2); a wave writes two
        // rows per instruction, one per half-wave
        const int oh0 = 32 * half;
        const int ocs_h = ocs - oh0 < 32 ? ocs - oh0 : 32;
        const int rows = (ocs_h > 0 ? ocs_h : 0) * TD * TH;
        for (int row = wv * 2 + (lane >> 5); row < rows; row += 8) {
            const int oc = row / (TD * TH);
            const int zy = row - oc * (TD * TH);
            const int z = zy / TH, y = zy - z * TH;
            const int64_t qd = t.d0 + z, qh = t.h0 + y;
            if (!x_ok || qd >= Q0 || qh >= Q1) continue;
            const float v = (has_taps ? lds[oc * kStage + zy * TW + x] : 0.f) + sbias[oh0 + oc];
            const int64_t od = s0 * qd + r0, oh = s1 * qh + r1, ow = s2 * q2 + r2;
            yg[(((t.n * pa.yC + t.oc0 + oh0 + oc) * a.Y[0] + od) * O1 + oh) * O2 + ow] = v;
        }
    }
}

// Per-dim tap lists of every residue; false when a phase needs more than the
// engine's halo or taps per dim.
bool build_dim_phases(int64_t S, int64_t O, int32_t K, int32_t s, int32_t p, int32_t d, DimPhases& dp) {
    if (s < 1 || s > kMaxS) return false;
    dp = DimPhases{};
    dp.s = s;
    for (int r = 0; r < s; ++r) {
        int n = 0, dmin = INT_MAX, dmax = INT_MIN;
        int ks[16], ds[16];
        for (int k = 0; k < K; ++k) {
            const int num = r + p - k * d;
            if (((num % s) + s) % s != 0) continue;
            if (n == kMaxT) return false;
            ks[n] = k;
            ds[n] = num / s;  // exact
            dmin = ds[n] < dmin ? ds[n] : dmin;
            dmax = ds[n] > dmax ? ds[n] : dmax;
            ++n;
        }
        if (n > 0 && dmax - dmin > 2) return false;
        dp.n[r] = n;
        dp.org[r] = n > 0 ? -dmin : 0;
        for (int i = 0; i < n; ++i) {
            dp.k[r][i] = ks[i];
            dp.off[r][i] = ds[i] - dmin;
        }
        dp.Q[r] = O > r ? (O - r + s - 1) / s : 0;
    }
    (void)S;
    return true;
}

bool build_phase_args(const Geom& g, PhaseArgs& pa) {
    pa = PhaseArgs{};
    for (int j = 0; j < 3; ++j)
        if (!build_dim_phases(g.S[j], g.O[j], g.k[j], g.s[j], g.p[j], g.d[j], pa.dim[j])) return false;
    return true;
}

}  // namespace

bool convT_phase_mfma_supported(const Geom& g, const void*, const void*, const void*) {
    if (g.cin_g < 4 || g.cout_g < 8) return false;
    for (int j = 0; j < 3; ++j)
        if (!mfma333::fits_int32_tiles(g.O[j]) || g.k[j] > 16) return false;
    // the K loop's buffer resources (a chunk of input planes, a group's
    // weights) stay below 2^31 bytes
    if ((int64_t)mfma333::ICC * g.S[0] * g.S[1] * g.S[2] * 4 >= (1ll << 31) ||
        g.cin_g * g.cout_g * g.k[0] * g.k[1] * g.k[2] * 4 >= (1ll << 31))
        return false;
    PhaseArgs pa;
    return build_phase_args(g, pa);
}

hipError_t launch_convT_phase_mfma(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                   hipStream_t st) {
    PhaseArgs pa;
    if (!build_phase_args(g, pa)) return hipErrorNotSupported;
    Args& a = pa.a;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.N = g.N;
    a.Cin = g.cin_g;
    a.Cout = g.cout_g;
    a.xC = g.Cin;
    int64_t qmax[3];
    for (int j = 0; j < 3; ++j) {
        a.S[j] = g.S[j];
        a.Y[j] = g.O[j];
        qmax[j] = ceil_div(g.O[j], g.s[j]);
        a.O[j] = qmax[j];
        pa.K[j] = g.k[j];
    }
    a.tiles[0] = (int32_t)ceil_div(qmax[0], TD);
    a.tiles[1] = (int32_t)ceil_div(qmax[1], TH);
    a.tiles[2] = (int32_t)ceil_div(qmax[2], TW);
    a.oc_blocks = (int32_t)ceil_div(g.cout_g, OCB);
    pa.nph = g.s[0] * g.s[1] * g.s[2];
    pa.groups = g.groups;
    pa.yC = g.Cout;
    pa.x_gstride = (int64_t)g.cin_g * g.S[0] * g.S[1] * g.S[2];
    pa.w_gstride = (int64_t)g.cin_g * g.cout_g * g.k[0] * g.k[1] * g.k[2];
    pa.y_gstride = (int64_t)g.cout_g * g.O[0] * g.O[1] * g.O[2];
    const int64_t blocks =
        g.N * (int64_t)a.tiles[0] * a.tiles[1] * a.tiles[2] * g.groups * a.oc_blocks * pa.nph;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(convT_phase_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, pa);
    return hipGetLastError();
}

}  // namespace c3d
