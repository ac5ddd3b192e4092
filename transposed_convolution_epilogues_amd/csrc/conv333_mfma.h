// conv333_mfma.h - implicit-GEMM engine for 3x3x3, stride-1, dilation-1
// convolutions on CDNA4 fp32 matrix cores (v_mfma_f32_32x32x2f32), shared by
// the fused conv->maxpool->logsumexp->ReLU kernel, the stride-2 transposed-conv
// sub-lattice kernel and the plain conv3d kernel.
//
// GEMM view ("Kimi-K2.6 l2_p43", the tall-skinny implicit GEMM with rows =
// output voxels, K = Cin x 27 taps, N = Cout):
//   acc[voxel, oc] += sum_{ic, tap} X[ic, voxel + tap - pad] * W[oc, ic, tap]
//
// Work decomposition
//   workgroup  = 256 threads (4 waves), output tile TD x TH x TW = 2 x 4 x 32
//                voxels x 64 output channels
//   wave       = 2 (D) x 2 (H) x 16 (W) voxels x 64 channels = 2 x 2 MFMA tiles
//                of 32 x 32 (M = voxels, N = channels), 64 accumulator VGPRs
//   M tile     = 1 (D) x 2 (H) x 16 (W) voxels: row r holds x = r % 16,
//                y = r / 16, and the wave's two M tiles are the two D planes.
//                A-operand lanes 0-15 then read 16 consecutive voxels (256
//                contiguous bytes of LDS, no bank conflict).  In the MFMA result
//                a lane holds rows {8a + 4*(lane/32) + b}: x = 8(a%2) + 4h + b,
//                y = a/2, in both M tiles, i.e. four complete 2x2x2 windows, so
//                a 2x2x2 max pool is lane-local.
//   K loop     = input-channel chunks of 8; per chunk the input halo
//                (TD+2)(TH+2)(TW+2) x 8 and the weights 27 x 8 x 64 are staged
//                in LDS; per tap a lane fetches 4 K-steps of its A operand
//                (4 consecutive channels of one voxel) and of its B operand
//                (4 consecutive channels of one output channel) with one
//                16-byte LDS read each.
//   K order    = within a chunk, K-step s and lane half h use channel
//                4h + s; A and B agree on it, so the contraction is exact.
// LDS: 26,112 B input + 55,728 B weights = 81,840 B -> two workgroups per CU.
#pragma once

#include <float.h>
#include <math.h>

#include "c3d_internal.h"

namespace c3d {
namespace mfma333 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int TD = 2, TH = 4, TW = 32;           // output tile per workgroup
constexpr int HD = TD + 2, HH = TH + 2, HW = TW + 2;
constexpr int HPOS = HD * HH * HW;               // 816 halo positions
constexpr int ICC = 8;                            // input channels per chunk
constexpr int OCB = 64;                           // output channels per workgroup
constexpr int LDS_X = 2 * HPOS * 4;               // floats, layout [g][pos][4]
constexpr int WTAP = 2 * 2 * 32 * 4 + 4;          // floats per tap, padded: staging writes
                                                  // of consecutive taps fall on distinct banks
constexpr int LDS_W = 27 * WTAP;                  // floats, layout [tap][nt][h][n][s]
constexpr int LDS_FLOATS = LDS_X + LDS_W;

// How the B operand (weights) is read from global memory.
enum WeightMode {
    kConvWeights = 0,   // w[oc][ic][tap]             (Conv3d layout)
    kConvTFlipped = 1,  // w[ic][oc][26 - tap]        (ConvTranspose3d, flipped)
};

struct Args {
    const float* x;
    const float* w;
    const float* bias;
    float* y;
    int64_t N, Cin, Cout;
    int64_t S[3];   // input dims
    int64_t O[3];   // conv output dims (stride 1)
    int32_t pad;    // same padding on all dims
    int32_t tiles[3];  // tiles per dim (D, H, W)
    int32_t oc_blocks;
    int64_t P[3];   // pooled dims (fused pooling epilogue)
    int64_t Y[3];   // destination dims (sub-lattice epilogue)
};

// Tile coordinates of this workgroup.  Consecutive workgroup ids are spread
// round-robin over the 8 XCDs; the id is remapped so that each XCD receives a
// contiguous run of tiles, whose halos overlap and so share that XCD's L2.
struct Tile {
    int64_t n;
    int64_t d0, h0, w0;
    int64_t oc0;
};

__device__ __forceinline__ Tile tile_of(const Args& a) {
    const int64_t nb = (int64_t)gridDim.x;
    int64_t b = blockIdx.x;
    if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    Tile t;
    t.oc0 = (b % a.oc_blocks) * OCB;
    b /= a.oc_blocks;
    const int64_t tw = b % a.tiles[2];
    b /= a.tiles[2];
    const int64_t th = b % a.tiles[1];
    b /= a.tiles[1];
    const int64_t td = b % a.tiles[0];
    t.n = b / a.tiles[0];
    t.d0 = td * TD;
    t.h0 = th * TH;
    t.w0 = tw * TW;
    return t;
}

// Input halo chunk -> LDS [g][pos][4], channel ic0 + 4g + j at float j.
// Loads are unconditional (out-of-range elements read a clamped, valid address
// and are replaced by 0 with a select) and issued in batches, so a thread has
// many loads in flight before its first LDS write.
__device__ __forceinline__ void stage_x(const Args& a, const Tile& t, int64_t ic0, float* lx) {
    constexpr int kItems = 2 * HPOS;
    constexpr int kIters = (kItems + kThreads - 1) / kThreads;  // 7
    const int64_t plane = a.S[0] * a.S[1] * a.S[2];
    const float* xn = a.x + (t.n * a.Cin) * plane;
    f32x4 v[kIters];
#pragma unroll
    for (int q = 0; q < kIters; ++q) {
        const int it = threadIdx.x + q * kThreads;
        const int g = it / HPOS;
        const int pos = it - g * HPOS;
        const int pw = pos % HW;
        const int ph = (pos / HW) % HH;
        const int pd = pos / (HW * HH);
        const int64_t gd = t.d0 - a.pad + pd, gh = t.h0 - a.pad + ph, gw = t.w0 - a.pad + pw;
        const bool inb = it < kItems && gd >= 0 && gd < a.S[0] && gh >= 0 && gh < a.S[1] && gw >= 0 &&
                         gw < a.S[2];
        const int64_t off = inb ? (gd * a.S[1] + gh) * a.S[2] + gw : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t ic = ic0 + 4 * g + j;
            const bool ok = inb && ic < a.Cin;
            const float e = xn[ok ? ic * plane + off : 0];
            v[q][j] = ok ? e : 0.f;
        }
    }
#pragma unroll
    for (int q = 0; q < kIters; ++q) {
        const int it = threadIdx.x + q * kThreads;
        if (it < kItems) *reinterpret_cast<f32x4*>(lx + it * 4) = v[q];
    }
}

// Weight chunk -> LDS [tap][nt][h][n][s] with oc = oc0 + 32nt + n and
// ic = ic0 + 4h + s.  Global reads follow the memory order of w; like
// stage_x, loads are unconditional and batched.
template <int kMode>
__device__ __forceinline__ void stage_w(const Args& a, const Tile& t, int64_t ic0, float* lw) {
    constexpr int kItems = 27 * ICC * OCB;       // 13824 = 54 per thread
    constexpr int kBatch = 9;
    static_assert(kItems % (kThreads * kBatch) == 0, "weight staging batches");
    for (int q0 = 0; q0 < kItems / kThreads; q0 += kBatch) {
        float v[kBatch];
        int dst[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int e = threadIdx.x + (q0 + q) * kThreads;
            int oc, j, tap;
            int64_t src;
            bool ok;
            if (kMode == kConvWeights) {
                oc = e / (ICC * 27);
                const int rem = e - oc * (ICC * 27);
                j = rem / 27;
                tap = rem - j * 27;
                const int64_t goc = t.oc0 + oc, gic = ic0 + j;
                ok = goc < a.Cout && gic < a.Cin;
                src = (goc * a.Cin + gic) * 27 + tap;
            } else {
                j = e / (OCB * 27);
                const int rem = e - j * (OCB * 27);
                oc = rem / 27;
                const int tt = rem - oc * 27;
                tap = 26 - tt;
                const int64_t goc = t.oc0 + oc, gic = ic0 + j;
                ok = goc < a.Cout && gic < a.Cin;
                src = (gic * a.Cout + goc) * 27 + tt;
            }
            const float e2 = a.w[ok ? src : 0];
            v[q] = ok ? e2 : 0.f;
            const int nt = oc >> 5, n = oc & 31, h = j >> 2, s = j & 3;
            dst[q] = tap * WTAP + ((nt * 2 + h) * 32 + n) * 4 + s;
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) lw[dst[q]] = v[q];
    }
}

// Runs the whole K loop; acc[mt][nt] holds the 32x32 result tiles.
template <int kMode>
__device__ __forceinline__ void mainloop(const Args& a, const Tile& t, float* lds, f32x16 (&acc)[2][2]) {
    float* lx = lds;
    float* lw = lds + LDS_X;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int r = lane & 31;
    // this lane's A-operand voxel in each M tile (tile-relative), see header
    const int wx = (wv & 1) * 16, wy = (wv >> 1) * 2;
    int abase[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int x = (r & 15) + wx, y = (r >> 4) + wy, z = mt;
        abase[mt] = (h * HPOS + (z * HH + y) * HW + x) * 4;
    }
    const int bbase = (h * 32 + r) * 4;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

    const int64_t nchunks = ceil_div(a.Cin, ICC);
    for (int64_t c = 0; c < nchunks; ++c) {
        __syncthreads();
        stage_x(a, t, c * ICC, lx);
        stage_w<kMode>(a, t, c * ICC, lw);
        __syncthreads();
#pragma unroll
        for (int kd = 0; kd < 3; ++kd)
#pragma unroll
            for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) {
                    const int tap = (kd * 3 + kh) * 3 + kw;
                    const int xoff = ((kd * HH + kh) * HW + kw) * 4;
                    f32x4 av[2], bv[2];
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) av[mt] = *reinterpret_cast<const f32x4*>(lx + abase[mt] + xoff);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        bv[nt] = *reinterpret_cast<const f32x4*>(lw + bbase + tap * WTAP + nt * 256);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
                                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt][s], bv[nt][s],
                                                                                   acc[mt][nt], 0, 0, 0);
                }
    }
}

// Tile-relative voxel of accumulator register i of M tile mt for this lane
// (the MFMA result layout: row = 8*(i/4) + 4*(lane/32) + i%4).
__device__ __forceinline__ void acc_voxel(int lane, int wv, int mt, int i, int& x, int& y, int& z) {
    const int a = i >> 2, b = i & 3, h = lane >> 5;
    x = 8 * (a & 1) + 4 * h + b + (wv & 1) * 16;
    y = (a >> 1) + (wv >> 1) * 2;
    z = mt;
}

inline bool fits_int32_tiles(int64_t v) { return v > 0 && v < (1ll << 30); }

}  // namespace mfma333
}  // namespace c3d
