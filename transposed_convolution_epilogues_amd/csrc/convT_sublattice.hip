// convT_sublattice.hip - stride-1 3x3x3 conv3d and the stride-2 / dilation-2
// transposed conv, both on the MFMA engine of conv333_mfma.h, with an epilogue
// that stages the result tile in LDS and writes whole output rows.
//
// Transposed conv, kernel 3, stride 2, padding 1, dilation 2 ("Kimi-K2.6
// l1_p77"): an input index i and tap k land at o = 2i - 1 + 2k, which is always
// odd, so every output with an even coordinate receives no tap and equals the
// bias (the page's parity argument), and the odd outputs o = 2q + 1 come from
// i = q + 1 - k.  Writing k' = 2 - k, that is i = q - 1 + k': the odd
// sub-lattice is a stride-1, pad-1 conv3d of x with the flipped,
// channel-transposed weights Wf[oc][ic][k'] = W[ic][oc][2 - k'] over a grid of
// the input's own size (the valid-residue decomposition the page arrives at,
// with one non-empty residue per dim).  Each workgroup computes its
// sub-lattice tile and then writes its whole box of output rows, odd positions
// from the tile and everything else as the bias, so each output element is
// written once with coalesced stores.
#include "conv333_mfma.h"

namespace c3d {
namespace {

using namespace mfma333;

constexpr int kStage = TD * TH * TW + 1;  // LDS floats per channel (padded)
static_assert(OCB * kStage <= LDS_FLOATS, "result staging fits the kernel's LDS");

// kLattice = 1: destination o = q (plain conv).  kLattice = 2: destination
// o = 2q + 1 inside a destination grid of size Y (transposed conv).
template <int kMode, int kLattice>
__global__ __launch_bounds__(kThreads) void conv333_store_kernel(Args a) {
    __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];
    const Tile t = tile_of(a);
    f32x16 acc[2][2];
    mainloop<kMode>(a, t, lds, acc);

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    __syncthreads();  // every wave is done reading the operand tiles
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int x, y, z;
                acc_voxel(lane, wv, mt, i, x, y, z);
                const int oc = nt * 32 + (lane & 31);
                lds[oc * kStage + (z * TH + y) * TW + x] = acc[mt][nt][i];
            }
    __syncthreads();

    // destination box of this workgroup
    int64_t lo[3], hi[3];
    const int64_t q0[3] = {t.d0, t.h0, t.w0};
    const int T[3] = {TD, TH, TW};
    for (int j = 0; j < 3; ++j) {
        if (kLattice == 1) {
            lo[j] = q0[j];
            hi[j] = q0[j] + T[j] < a.Y[j] ? q0[j] + T[j] : a.Y[j];
        } else {
            lo[j] = 2 * q0[j];
            hi[j] = (q0[j] + T[j] >= a.O[j]) ? a.Y[j] : 2 * (q0[j] + T[j]);
        }
    }
    const int bd = (int)(hi[0] - lo[0]), bh = (int)(hi[1] - lo[1]), bw = (int)(hi[2] - lo[2]);
    const int ocs = (int)(a.Cout - t.oc0 < OCB ? a.Cout - t.oc0 : OCB);
    const int64_t plane = a.Y[0] * a.Y[1] * a.Y[2];
    float* yn = a.y + (t.n * a.Cout + t.oc0) * plane;
    for (int oc = 0; oc < ocs; ++oc) {
        const float b = a.bias ? a.bias[t.oc0 + oc] : 0.f;
        const float* src = lds + oc * kStage;
        for (int id = 0; id < bd; ++id) {
            const int64_t od = lo[0] + id;
            for (int ih = wv; ih < bh; ih += kThreads / 64) {
                const int64_t oh = lo[1] + ih;
                float* row = yn + oc * plane + (od * a.Y[1] + oh) * a.Y[2] + lo[2];
                if (kLattice == 1) {
                    const float* s = src + (id * TH + ih) * TW;
                    for (int c = lane; c < bw; c += 64) row[c] = s[c] + b;
                } else {
                    const bool odd_row = (od & 1) && (oh & 1);
                    const float* s = src + (odd_row ? (int)((((od - 1) >> 1) - t.d0) * TH + (((oh - 1) >> 1) - t.h0)) * TW : 0);
                    // lo[2] is even, so column c is odd exactly when ow is
                    for (int c = lane; c < bw; c += 64) row[c] = (odd_row && (c & 1)) ? s[c >> 1] + b : b;
                }
            }
        }
    }
}

Args make_args(const float* x, const float* w, const float* bias, float* y, const Geom& g) {
    Args a{};
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.N = g.N;
    a.Cin = g.Cin;
    a.Cout = g.Cout;
    for (int j = 0; j < 3; ++j) a.S[j] = g.S[j];
    a.oc_blocks = (int32_t)ceil_div(g.Cout, OCB);
    return a;
}

}  // namespace

bool conv3x3x3_mfma_supported(const Geom& g, const void*, const void*, const void*) {
    for (int j = 0; j < 3; ++j)
        if (g.k[j] != 3 || g.s[j] != 1 || g.d[j] != 1 || g.p[j] != g.p[0]) return false;
    // the MFMA tile pays off once there are several input channels
    return g.groups == 1 && g.Cin >= 4 && g.Cout >= 8 && mfma333::fits_int32_tiles(g.O[0]) &&
           mfma333::fits_int32_tiles(g.O[1]) && mfma333::fits_int32_tiles(g.O[2]);
}

hipError_t launch_conv3x3x3_mfma(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                 hipStream_t st) {
    Args a = make_args(x, w, bias, y, g);
    a.pad = g.p[0];
    for (int j = 0; j < 3; ++j) {
        a.O[j] = g.O[j];
        a.Y[j] = g.O[j];
    }
    a.tiles[0] = (int32_t)ceil_div(g.O[0], TD);
    a.tiles[1] = (int32_t)ceil_div(g.O[1], TH);
    a.tiles[2] = (int32_t)ceil_div(g.O[2], TW);
    const int64_t blocks = a.N * (int64_t)a.tiles[0] * a.tiles[1] * a.tiles[2] * a.oc_blocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((conv333_store_kernel<kConvWeights, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

bool convT_s2_sublattice_supported(const Geom& g, const void*, const void*, const void*) {
    for (int j = 0; j < 3; ++j)
        if (g.k[j] != 3 || g.s[j] != 2 || g.d[j] != 2 || g.p[j] != 1 || g.O[j] != 2 * g.S[j] + 1) return false;
    return g.groups == 1 && mfma333::fits_int32_tiles(g.O[0]) && mfma333::fits_int32_tiles(g.O[1]) &&
           mfma333::fits_int32_tiles(g.O[2]);
}

hipError_t launch_convT_s2_sublattice(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                      hipStream_t st) {
    Args a = make_args(x, w, bias, y, g);
    a.pad = 1;
    for (int j = 0; j < 3; ++j) {
        a.O[j] = g.S[j];  // sub-lattice grid = input grid
        a.Y[j] = g.O[j];  // destination = the transposed-conv output
    }
    a.tiles[0] = (int32_t)ceil_div(g.S[0], TD);
    a.tiles[1] = (int32_t)ceil_div(g.S[1], TH);
    a.tiles[2] = (int32_t)ceil_div(g.S[2], TW);
    const int64_t blocks = a.N * (int64_t)a.tiles[0] * a.tiles[1] * a.tiles[2] * a.oc_blocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((conv333_store_kernel<kConvTFlipped, 2>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                       a);
    return hipGetLastError();
}

}  // namespace c3d
