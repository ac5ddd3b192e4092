// convT_scatter.hip - ConvTranspose3d in its scatter form, accumulated in an
// LDS output tile without atomics ("Kimi-K2.6 l1_p77": the scatter
// formulation o = i*s - p + k*d, and the observation that for one tap offset
// the map from inputs to outputs is injective, so a pass over one tap needs
// no atomics).
//
// A workgroup owns a box of 4 x 8 x 32 outputs and 16 output channels of one
// group, accumulated in LDS (64 KB, plus the tap's weights).  For every tap k it walks the inputs
// whose output o = i*s - p + k*d falls inside the box; distinct inputs reach
// distinct outputs for a fixed k, so each thread forms its input's
// contribution (summed over the group's input channels in registers) and adds
// it to its own outputs, for all 16 channels, without atomics.  A barrier
// separates the taps (two taps can reach the same output).  The box starts
// at the bias and is written out once, row by row.
//
// Any stride, padding, dilation, output padding and groups (Cin/groups up to
// 256).  Each (input, tap, output channel) is one LDS read-modify-write and
// the MACs are plain fp32 VALU work: it is the second algorithm, selected by
// variant 4, to compare with the gather and per-phase kernels.
#include "c3d_internal.h"

namespace c3d {
namespace {

constexpr int kThreads = 256;
constexpr int TD = 4, TH = 8, TW = 32;
constexpr int kBox = TD * TH * TW;  // 1024 outputs
constexpr int kCt = 16;             // output channels per workgroup
constexpr int kMaxCinG = 256;       // input channels per group held in LDS per tap

struct ScatterArgs {
    const float* x;
    const float* w;
    const float* bias;
    float* y;
    Geom g;
    int32_t tiles[3];
    int32_t oc_blocks;  // per group
};

__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

__global__ __launch_bounds__(kThreads) void convT_scatter_kernel(ScatterArgs a) {
    __shared__ float acc[kCt * kBox];
    __shared__ float wk[kMaxCinG * kCt];
    const Geom& g = a.g;
    int64_t b = blockIdx.x;
    const int ocb = (int)(b % a.oc_blocks);
    b /= a.oc_blocks;
    const int64_t grp = b % g.groups;
    b /= g.groups;
    const int64_t tw = b % a.tiles[2];
    b /= a.tiles[2];
    const int64_t th = b % a.tiles[1];
    b /= a.tiles[1];
    const int64_t td = b % a.tiles[0];
    const int64_t n = b / a.tiles[0];
    const int64_t o0[3] = {td * TD, th * TH, tw * TW};
    const int T[3] = {TD, TH, TW};
    const int64_t oc0 = grp * g.cout_g + (int64_t)ocb * kCt;  // absolute channel
    const int ocs = (int)(g.cout_g - (int64_t)ocb * kCt < kCt ? g.cout_g - (int64_t)ocb * kCt : kCt);

    for (int e = threadIdx.x; e < kCt * kBox; e += kThreads) {
        const int oc = e / kBox;
        acc[e] = (a.bias && oc < ocs) ? a.bias[oc0 + oc] : 0.f;
    }
    const int64_t splane = g.S[0] * g.S[1] * g.S[2];
    const int kvol = g.k[0] * g.k[1] * g.k[2];
    const float* xg = a.x + (n * g.Cin + grp * g.cin_g) * splane;
    for (int kk = 0; kk < kvol; ++kk) {
        const int k[3] = {kk / (g.k[1] * g.k[2]), (kk / g.k[2]) % g.k[1], kk % g.k[2]};
        __syncthreads();  // the previous tap's adds are done (and, first, the bias fill)
        // this tap's weights, [ic][oc] for the group's input channels and the block's channels
        for (int e = threadIdx.x; e < g.cin_g * kCt; e += kThreads) {
            const int64_t ic = grp * g.cin_g + e / kCt;
            const int oc = e % kCt;
            wk[e] = oc < ocs ? a.w[(ic * g.cout_g + (int64_t)ocb * kCt + oc) * kvol + kk] : 0.f;
        }
        // inputs of this tap landing in the box: o0 <= i*s - p + k*d <= o0 + T - 1, o < O
        int32_t lo[3], cnt[3];
        for (int j = 0; j < 3; ++j) {
            const int64_t off = (int64_t)g.p[j] - (int64_t)k[j] * g.d[j];
            int64_t l = -floor_div(-(o0[j] + off), g.s[j]);  // ceil
            int64_t h = floor_div(o0[j] + T[j] - 1 + off, g.s[j]);
            const int64_t hmax = floor_div(g.O[j] - 1 + off, g.s[j]);
            if (l < 0) l = 0;
            if (h > g.S[j] - 1) h = g.S[j] - 1;
            if (h > hmax) h = hmax;
            lo[j] = (int32_t)l;
            cnt[j] = h >= l ? (int32_t)(h - l + 1) : 0;
        }
        __syncthreads();  // wk visible
        const int total = cnt[0] * cnt[1] * cnt[2];  // at most 4 * 8 * 32 (one input per output)
        for (int e = threadIdx.x; e < total; e += kThreads) {
            const int i2 = lo[2] + e % cnt[2];
            const int i1 = lo[1] + (e / cnt[2]) % cnt[1];
            const int i0 = lo[0] + e / (cnt[2] * cnt[1]);
            const float* xi = xg + ((int64_t)i0 * g.S[1] + i1) * g.S[2] + i2;
            float t[kCt];
#pragma unroll
            for (int oc = 0; oc < kCt; ++oc) t[oc] = 0.f;
            for (int64_t ic = 0; ic < g.cin_g; ++ic) {
                const float xv = xi[ic * splane];
#pragma unroll
                for (int oc = 0; oc < kCt; ++oc) t[oc] = fmaf(xv, wk[ic * kCt + oc], t[oc]);
            }
            const int q0 = i0 * g.s[0] - g.p[0] + k[0] * g.d[0] - (int)o0[0];
            const int q1 = i1 * g.s[1] - g.p[1] + k[1] * g.d[1] - (int)o0[1];
            const int q2 = i2 * g.s[2] - g.p[2] + k[2] * g.d[2] - (int)o0[2];
            float* dst = acc + (q0 * TH + q1) * TW + q2;
#pragma unroll
            for (int oc = 0; oc < kCt; ++oc) dst[oc * kBox] += t[oc];
        }
    }
    __syncthreads();
    // write the box, row by row (rows of TW = 32 outputs, two per wave instruction)
    const int64_t oplane = g.O[0] * g.O[1] * g.O[2];
    float* yb = a.y + (n * g.Cout + oc0) * oplane;
    for (int r = threadIdx.x >> 5; r < ocs * TD * TH; r += kThreads / 32) {
        const int oc = r / (TD * TH), zy = r % (TD * TH), z = zy / TH, yy = zy % TH;
        const int x = threadIdx.x & 31;
        const int64_t od = o0[0] + z, oh = o0[1] + yy, ow = o0[2] + x;
        if (od < g.O[0] && oh < g.O[1] && ow < g.O[2])
            yb[oc * oplane + (od * g.O[1] + oh) * g.O[2] + ow] = acc[oc * kBox + zy * TW + x];
    }
}

}  // namespace

bool convT_scatter_supported(const Geom& g) {
    for (int j = 0; j < 3; ++j)
        if (g.O[j] >= (1ll << 30) || g.S[j] >= (1ll << 30) || (int64_t)g.k[j] * g.d[j] + g.p[j] >= (1ll << 30))
            return false;
    return g.cin_g <= kMaxCinG;
}

hipError_t launch_convT_scatter(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                hipStream_t st) {
    ScatterArgs a{};
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.g = g;
    a.tiles[0] = (int32_t)ceil_div(g.O[0], TD);
    a.tiles[1] = (int32_t)ceil_div(g.O[1], TH);
    a.tiles[2] = (int32_t)ceil_div(g.O[2], TW);
    a.oc_blocks = (int32_t)ceil_div(g.cout_g, kCt);
    const int64_t blocks = g.N * (int64_t)a.tiles[0] * a.tiles[1] * a.tiles[2] * g.groups * a.oc_blocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(convT_scatter_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace c3d
