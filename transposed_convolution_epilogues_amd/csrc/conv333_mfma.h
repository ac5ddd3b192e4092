// conv333_mfma.h - implicit-GEMM engine for 3x3x3, stride-1, dilation-1
// convolutions on CDNA4 fp32 matrix cores (v_mfma_f32_32x32x2f32), shared by
// the fused conv->maxpool->logsumexp->ReLU kernel, the stride-2 transposed-conv
// sub-lattice kernel and the plain conv3d kernel.
//
// GEMM view ("Kimi-K2.6 l2_p43", the tall-skinny implicit GEMM with rows =
// output voxels, K = Cin x 27 taps, N = Cout):
//   acc[voxel, oc] += sum_{ic, tap} X[ic, voxel + tap - pad] * W[oc, ic, tap]
//
// Work decomposition (kMT = tile depth, 2 or 4)
//   workgroup  = 256 threads (4 waves), output tile TD x TH x TW = kMT x 4 x 32
//                voxels x 64 output channels
//   wave       = kMT (D) x 2 (H) x 16 (W) voxels x 64 channels = kMT x 2 MFMA
//                tiles of 32 x 32 (M = voxels, N = channels), 32 kMT
//                accumulator registers
//   M tile     = 1 (D) x 2 (H) x 16 (W) voxels: row r holds x = r % 16,
//                y = r / 16, and the wave's M tiles are its D planes.
//                A-operand lanes 0-15 then read 16 consecutive voxels (256
//                contiguous bytes of LDS, no bank conflict).  In the MFMA result
//                a lane holds rows {8a + 4*(lane/32) + b}: x = 8(a%2) + 4h + b,
//                y = a/2, in every M tile, so a pair of M tiles holds four
//                complete 2x2x2 windows per lane and a 2x2x2 max pool is
//                lane-local.  The deeper tile doubles the MFMA work between
//                two barriers and cuts the halo overhead (6/4 instead of 4/2
//                planes per output plane).
//   K loop     = input-channel chunks of 8, each split into three weight
//                units of 9 taps (one kd plane).  The chunk's input halo
//                (TD+2)(TH+2)(TW+2) x 8 sits in LDS; the units' weights
//                9 x 8 x 64 are double-buffered in LDS.  While a unit is being
//                computed the next unit's weights (and, during a chunk's last
//                unit, the next chunk's halo) are already being loaded into
//                registers, issued in slices between the unit's taps, so their
//                latency hides under ~9K cycles of MFMA work; they are written
//                to LDS after the unit.  Per tap a lane fetches 4 K-steps of
//                its A operand (4 consecutive channels of one voxel) and of
//                its B operand (4 consecutive channels of one output channel)
//                with one 16-byte LDS read each.
//   K order    = within a chunk, K-step s and lane half h use channel
//                4h + s; A and B agree on it, so the contraction is exact.
// LDS: halo 26,112 B (kMT = 2) or 39,168 B (kMT = 4) + 2 x 18,576 B weights
// (the result staging of the kMT = 2 store epilogue reuses it and needs
// 65,792 B) -> two workgroups per CU either way.
#pragma once

#include <float.h>
#include <math.h>

#include "c3d_internal.h"

namespace c3d {
namespace mfma333 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int TH = 4, TW = 32;                   // output tile per workgroup (H, W)
constexpr int HH = TH + 2, HW = TW + 2;
constexpr int ICC = 8;                            // input channels per chunk
constexpr int OCB = 64;                           // output channels per workgroup
constexpr int WTAP = 2 * 2 * 32 * 4 + 4;          // floats per tap, padded: staging writes
                                                  // of consecutive taps fall on distinct banks
constexpr int UNIT_TAPS = 9;                      // taps per weight unit (one kd plane)
constexpr int LDS_W = UNIT_TAPS * WTAP;           // floats per weight buffer, [tap][nt][h][n][s]

// Sizes that depend on the tile depth kMT.
template <int kMT>
struct Geo {
    static constexpr int TD = kMT;                        // output tile depth
    static constexpr int HD = TD + 2;
    static constexpr int HPOS = HD * HH * HW;             // halo positions: 816 or 1224
    static constexpr int LDS_X = 2 * HPOS * 4;            // floats, layout [g][pos][4]
    static constexpr int LDS_MAIN = LDS_X + 2 * LDS_W;    // floats of the K loop
    static constexpr int XQ = (HPOS + kThreads - 1) / kThreads;  // halo positions per thread
};

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
    int64_t xC;     // channels per sample of x (Cin, or more when x holds several groups)
    int64_t S[3];   // input dims
    int64_t O[3];   // conv output dims (stride 1)
    int32_t pad[3];  // halo origin = tile origin - pad, per dim
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

// (32-bit: the launchers keep the grid below 2^31 workgroups)
template <int kMT>
__device__ __forceinline__ Tile tile_of(const Args& a) {
    const int32_t nb = (int32_t)gridDim.x;
    int32_t b = (int32_t)blockIdx.x;
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
    t.d0 = td * Geo<kMT>::TD;
    t.h0 = th * TH;
    t.w0 = tw * TW;
    return t;
}

// Input halo of one chunk, as two 4-channel groups: LDS layout [g][pos][4]
// holds channels ic0 + 4g .. ic0 + 4g + 3 of halo position pos.  A thread
// owns positions tid + 256q; the channel offsets are wave-uniform, so a
// thread keeps only its position offsets.  Loads are unconditional buffer
// loads: positions outside the input carry an offset past the resource and
// read 0.
template <int kMT>
struct XRegs {
    f32x4 v[2][Geo<kMT>::XQ];
};

template <int kMT>
struct XOffsets {
    int32_t off[Geo<kMT>::XQ];  // spatial offset in the input plane, -1 outside
    uint32_t vo[Geo<kMT>::XQ];  // the same in bytes for buffer loads; kOutside outside
};

// A buffer load or store whose offset is at least the resource's size touches
// no memory (a load returns 0).  Resources here are below 2^31 bytes, so an
// offset of kOutside (plus any channel offset below 2^31) always falls outside.
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int kMT>
__device__ __forceinline__ XOffsets<kMT> x_offsets(const Args& a, const Tile& t, const int32_t (&pad)[3]) {
    constexpr int HPOS = Geo<kMT>::HPOS;
    XOffsets<kMT> o;
#pragma unroll
    for (int q = 0; q < Geo<kMT>::XQ; ++q) {
        const int pos = threadIdx.x + q * kThreads;
        const int pw = pos % HW;
        const int ph = (pos / HW) % HH;
        const int pd = pos / (HW * HH);
        const int64_t gd = t.d0 - pad[0] + pd, gh = t.h0 - pad[1] + ph, gw = t.w0 - pad[2] + pw;
        const bool inb = pos < HPOS && gd >= 0 && gd < a.S[0] && gh >= 0 && gh < a.S[1] && gw >= 0 &&
                         gw < a.S[2];
        o.off[q] = inb ? (int32_t)((gd * a.S[1] + gh) * a.S[2] + gw) : -1;
        o.vo[q] = inb ? 4u * (uint32_t)o.off[q] : kOutside;
    }
    return o;
}

// The same slice with buffer loads: the chunk's 8 channels form one buffer
// resource, the channel is a uniform offset, and positions outside the input
// read 0 by the range check (no address arithmetic per load, no zero select).
template <int kMT>
__device__ __forceinline__ void load_x_slice_buf(const Args& a, const Tile& t, const XOffsets<kMT>& o, int64_t ic0,
                                                 int g, int j, XRegs<kMT>& r) {
    const int64_t plane = a.S[0] * a.S[1] * a.S[2];
    const int c = 4 * g + j;
    const bool icok = (int)ic0 + c < (int)a.Cin;  // 32-bit: a scalar compare
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(a.x + (t.n * a.xC + ic0) * plane, (uint32_t)(ICC * plane * 4));
    const int soff = icok ? (int)(c * plane * 4) : 0;
#pragma unroll
    for (int q = 0; q < Geo<kMT>::XQ; ++q)
        r.v[g][q][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, o.vo[q], soff, 0));
}

template <int kMT>
__device__ __forceinline__ void load_x_buf(const Args& a, const Tile& t, const XOffsets<kMT>& o, int64_t ic0,
                                           XRegs<kMT>& r) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) load_x_slice_buf(a, t, o, ic0, g, j, r);
}

// LDS write of a halo loaded by buffer loads (positions outside are already 0);
// only the channels past Cin of a partial chunk are zeroed
template <int kMT>
__device__ __forceinline__ void store_x_buf(const Args& a, int64_t ic0, const XRegs<kMT>& r, float* lx) {
    constexpr int HPOS = Geo<kMT>::HPOS;
    const bool full = (int)ic0 + ICC <= (int)a.Cin;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int q = 0; q < Geo<kMT>::XQ; ++q) {
            const int pos = threadIdx.x + q * kThreads;
            f32x4 v = r.v[g][q];
            if (!full) {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = (int)ic0 + 4 * g + j < (int)a.Cin ? v[j] : 0.f;
            }
            if (pos < HPOS) *reinterpret_cast<f32x4*>(lx + (g * HPOS + pos) * 4) = v;
        }
}

// One weight unit: the 9 taps (kd, *, *) of 8 input channels x 64 output
// channels, LDS layout [tap % 9][nt][h][n][s] with oc = oc0 + 32nt + n and
// ic = ic0 + 4h + s.  A thread owns the (oc, ic) pairs tid and tid + 256 and
// reads each pair's 9 taps, which are consecutive in w (conv weights
// w[oc][ic][tap]; transposed weights w[ic][oc][t] with tap = 26 - t, flipped).
constexpr int W_PAIRS_PER_THREAD = ICC * OCB / kThreads;  // 2
static_assert(ICC * OCB % kThreads == 0, "weight unit pairs");

struct WRegs {
    float v[W_PAIRS_PER_THREAD][UNIT_TAPS];
};

// Buffer-load form of the weight unit loads: per thread and pair a byte
// offset fixed for the tile (kOutside for output channels past Cout), the
// input-channel chunk and kd plane as a uniform offset, the 9 taps as
// immediate offsets.
struct WOffsets {
    uint32_t vo[W_PAIRS_PER_THREAD];
};

template <int kMode>
__device__ __forceinline__ WOffsets w_offsets(const Args& a, const Tile& t) {
    WOffsets o;
#pragma unroll
    for (int q = 0; q < W_PAIRS_PER_THREAD; ++q) {
        const int p = threadIdx.x + q * kThreads;
        const int oc = p >> 3, j = p & 7;
        const int64_t goc = t.oc0 + oc;
        // first element of the pair's run for ic0 = 0, kd = 0 (transposed: without the 18 - 9 kd)
        const int64_t first = kMode == kConvWeights ? (goc * a.Cin + j) * 27 : ((int64_t)j * a.Cout + goc) * 27;
        o.vo[q] = goc < a.Cout ? (uint32_t)(first * 4) : kOutside;
    }
    return o;
}

template <int kMode>
__device__ __forceinline__ void load_w_pair_buf(const Args& a, const WOffsets& o, int64_t ic0, int kd, int q,
                                                WRegs& r) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.w, (uint32_t)(a.Cout * a.Cin * 27 * 4));
    const int64_t ue = kMode == kConvWeights ? ic0 * 27 + kd * UNIT_TAPS : ic0 * a.Cout * 27 + (18 - kd * UNIT_TAPS);
    const int j = (threadIdx.x + q * kThreads) & 7;
    // channels past Cin (a partial last chunk) read nothing
    const uint32_t vo = (int)ic0 + j < (int)a.Cin ? o.vo[q] : kOutside;
#pragma unroll
    for (int u = 0; u < UNIT_TAPS; ++u)
        r.v[q][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo + 4u * u, (int)(ue * 4), 0));
}

// LDS write of a weight unit loaded by buffer loads (pairs outside are already
// 0).  Conv: source tap kd*9 + u is unit tap u; transposed: source t = 18 - 9kd
// + u is tap 26 - t = 8 + 9kd - u, i.e. unit tap 8 - u.
template <int kMode>
__device__ __forceinline__ void store_w_buf(const WRegs& r, float* lw) {
#pragma unroll
    for (int q = 0; q < W_PAIRS_PER_THREAD; ++q) {
        const int p = threadIdx.x + q * kThreads;
        const int oc = p >> 3, j = p & 7;
        const int nt = oc >> 5, n = oc & 31, h = j >> 2, s = j & 3;
        float* dst = lw + ((nt * 2 + h) * 32 + n) * 4 + s;
#pragma unroll
        for (int u = 0; u < UNIT_TAPS; ++u) dst[(kMode == kConvWeights ? u : 8 - u) * WTAP] = r.v[q][u];
    }
}

// Side work of a kernel that does not overlap anything with the K loop.
struct NoSideWork {
    static constexpr int kTap = 0;
    __device__ void operator()(int64_t, int64_t) const {}
};

// Runs the whole K loop; acc[mt][nt] holds the 32x32 result tiles.  side(u, n)
// is called once per weight unit u of n, after the MFMAs and the slice of
// prefetch loads of the unit's tap Side::kTap are issued: work placed there
// (stores that do not depend on the result) overlaps the matrix-core work.
// It must not touch the operand LDS.
template <int kMode, int kMT, class Side = NoSideWork>
__device__ __forceinline__ void mainloop(const Args& a, const Tile& t, float* lds, f32x16 (&acc)[kMT][2],
                                         const Side& side = Side()) {
    constexpr int HPOS = Geo<kMT>::HPOS;
    float* lx = lds;
    float* lw0 = lds + Geo<kMT>::LDS_X;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int r = lane & 31;
    // this lane's A-operand voxel in each M tile (tile-relative), see header
    const int wx = (wv & 1) * 16, wy = (wv >> 1) * 2;
    int abase[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        const int x = (r & 15) + wx, y = (r >> 4) + wy, z = mt;
        abase[mt] = (h * HPOS + (z * HH + y) * HW + x) * 4;
    }
    const int bbase = (h * 32 + r) * 4;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

    const int64_t nchunks = ceil_div(a.Cin, ICC);
    const XOffsets<kMT> xo = x_offsets<kMT>(a, t, a.pad);
    const WOffsets wo = w_offsets<kMode>(a, t);
    {
        XRegs<kMT> xr;
        WRegs wr;
        load_x_buf(a, t, xo, 0, xr);
#pragma unroll
        for (int q = 0; q < W_PAIRS_PER_THREAD; ++q) load_w_pair_buf<kMode>(a, wo, 0, 0, q, wr);
        store_x_buf(a, 0, xr, lx);
        store_w_buf<kMode>(wr, lw0);
        __syncthreads();
    }
    int buf = 0;
    for (int64_t c = 0; c < nchunks; ++c) {
#pragma unroll 1
        for (int kd = 0; kd < 3; ++kd) {
            const bool last_unit = c == nchunks - 1 && kd == 2;
            const int64_t nc = kd < 2 ? c : c + 1;  // chunk and kd plane of the next unit
            const int nkd = kd < 2 ? kd + 1 : 0;
            WRegs wr;
            XRegs<kMT> xr;
            const float* lw = lw0 + buf * LDS_W;
#pragma unroll
            for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) {
                    const int t9 = kh * 3 + kw;
                    const int xoff = ((kd * HH + kh) * HW + kw) * 4;
                    f32x4 av[kMT], bv[2];
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt) av[mt] = *reinterpret_cast<const f32x4*>(lx + abase[mt] + xoff);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        bv[nt] = *reinterpret_cast<const f32x4*>(lw + bbase + t9 * WTAP + nt * 256);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
                                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt][s], bv[nt][s],
                                                                                   acc[mt][nt], 0, 0, 0);
                    // The next unit's loads are issued in slices behind the taps'
                    // MFMAs (the weights behind taps 0 and 1, the halo's 8 channels
                    // behind taps 1-8), fenced so the compiler keeps them there: a
                    // burst of all of them before the first tap cost about 1% on the
                    // fused conv-pool kernel and 2% on the transposed conv.
                    __builtin_amdgcn_sched_barrier(0);
                    if (t9 < W_PAIRS_PER_THREAD && !last_unit) load_w_pair_buf<kMode>(a, wo, nc * ICC, nkd, t9, wr);
                    if (t9 >= 1 && kd == 2 && !last_unit)
                        load_x_slice_buf(a, t, xo, nc * ICC, (t9 - 1) >> 2, (t9 - 1) & 3, xr);
                    __builtin_amdgcn_sched_barrier(0);
                    // side work goes behind a tap's MFMAs: its stores issue while
                    // the matrix core runs them (about 2% faster on the 32->64
                    // stride-2 dilation-2 transposed conv of x[16,32,16,32,32] than
                    // issuing it before the unit's MFMAs)
                    if (t9 == Side::kTap) side(c * 3 + kd, nchunks * 3);
                }
            if (last_unit) break;
            if (kd == 2) {
                __syncthreads();  // every wave is done with this chunk's halo
                store_x_buf(a, nc * ICC, xr, lx);
            }
            // the other weight buffer was last read by the previous unit, which
            // every wave finished before the previous barrier
            store_w_buf<kMode>(wr, lw0 + (buf ^ 1) * LDS_W);
            __syncthreads();
            buf ^= 1;
        }
    }
}

// ---------------------------------------------------------------------------
// Tap-table variant of the K loop.  The taps are the product of three per-dim
// lists (tap i of dim j: kernel index k[i], halo offset off[i] in 0..2, at
// most 3 taps per dim), so a weight unit is one entry of the dim-0 list with
// its n1 x n2 <= 9 taps, and the K loop runs (input-channel chunks) x n0
// units.  Weights are read in the transposed layout w[ic][oc][kvol] with
// kvol index (k0 * K1 + k1) * K2 + k2.  Used by the transposed-conv phase
// kernel: each output phase of a strided transposed conv sees such a
// product of per-dim tap lists.
struct DimTaps {
    int32_t n;       // taps in this dim (1..3)
    int32_t k[3];    // kernel index of tap i
    int32_t off[3];  // halo offset of tap i
};

struct TapSet {
    DimTaps d[3];
    int32_t K1, K2, Kvol;  // kernel extents of dims 1 and 2, kernel volume
};

__device__ __forceinline__ int32_t pick3(const int32_t (&v)[3], int i) {
    return i == 0 ? v[0] : (i == 1 ? v[1] : v[2]);
}

// dims-1/2 part of unit slot u: weight index and halo offset (floats)
struct SlotTaps {
    int32_t wk[UNIT_TAPS];
    int32_t xo[UNIT_TAPS];
};

__device__ __forceinline__ SlotTaps slot_taps(const TapSet& ts) {
    SlotTaps st;
    const int n2 = ts.d[2].n;
#pragma unroll
    for (int u = 0; u < UNIT_TAPS; ++u) {
        const int i1 = n2 == 1 ? u : (n2 == 2 ? u >> 1 : u / 3);
        const int i2 = u - i1 * n2;
        st.wk[u] = pick3(ts.d[1].k, i1) * ts.K2 + pick3(ts.d[2].k, i2);
        st.xo[u] = (pick3(ts.d[1].off, i1) * HW + pick3(ts.d[2].off, i2)) * 4;
    }
    return st;
}

// Weights of one unit of the tap-table K loop, by buffer loads: per thread and
// pair a byte offset fixed for the tile (kOutside for output channels past
// Cout), the chunk, the unit's dim-0 tap and each slot's dims-1/2 tap as
// uniform offsets; pairs past Cin and slots past the unit's taps read 0.
struct WTapOffsets {
    uint32_t vo[W_PAIRS_PER_THREAD];
};

__device__ __forceinline__ WTapOffsets w_tap_offsets(const Args& a, const Tile& t, const TapSet& ts) {
    WTapOffsets o;
#pragma unroll
    for (int q = 0; q < W_PAIRS_PER_THREAD; ++q) {
        const int p = threadIdx.x + q * kThreads;
        const int oc = p >> 3, j = p & 7;
        const int64_t goc = t.oc0 + oc;
        o.vo[q] = goc < a.Cout ? (uint32_t)(((int64_t)j * a.Cout + goc) * ts.Kvol * 4) : kOutside;
    }
    return o;
}

__device__ __forceinline__ void load_w_taps_buf(const Args& a, const TapSet& ts, const SlotTaps& st,
                                                const WTapOffsets& o, int64_t ic0, int i0, WRegs& r) {
    const int ntu = ts.d[1].n * ts.d[2].n;
    const int wk0 = pick3(ts.d[0].k, i0) * ts.K1 * ts.K2;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.w, (uint32_t)(a.Cin * a.Cout * ts.Kvol * 4));
    const int base = (int)((ic0 * a.Cout * ts.Kvol + wk0) * 4);
#pragma unroll
    for (int q = 0; q < W_PAIRS_PER_THREAD; ++q) {
        const int j = (threadIdx.x + q * kThreads) & 7;
        const uint32_t vo = (int)ic0 + j < (int)a.Cin ? o.vo[q] : kOutside;
#pragma unroll
        for (int u = 0; u < UNIT_TAPS; ++u)
            r.v[q][u] = u < ntu ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo, base + 4 * st.wk[u], 0))
                                : 0.f;
    }
}

template <int kMT>
__device__ __forceinline__ void mainloop_taps(const Args& a, const Tile& t, const TapSet& ts,
                                              const int32_t (&pad)[3], float* lds, f32x16 (&acc)[kMT][2]) {
    constexpr int HPOS = Geo<kMT>::HPOS;
    float* lx = lds;
    float* lw0 = lds + Geo<kMT>::LDS_X;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int r = lane & 31;
    const int wx = (wv & 1) * 16, wy = (wv >> 1) * 2;
    int abase[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        const int x = (r & 15) + wx, y = (r >> 4) + wy, z = mt;
        abase[mt] = (h * HPOS + (z * HH + y) * HW + x) * 4;
    }
    const int bbase = (h * 32 + r) * 4;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

    const int n0 = ts.d[0].n;
    const int ntu = ts.d[1].n * ts.d[2].n;
    const SlotTaps st = slot_taps(ts);
    const int64_t nchunks = ceil_div(a.Cin, ICC);
    const XOffsets<kMT> xo = x_offsets<kMT>(a, t, pad);
    const WTapOffsets wo = w_tap_offsets(a, t, ts);
    {
        XRegs<kMT> xr;
        WRegs wr;
        load_x_buf(a, t, xo, 0, xr);
        load_w_taps_buf(a, ts, st, wo, 0, 0, wr);
        store_x_buf(a, 0, xr, lx);
        store_w_buf<kConvWeights>(wr, lw0);
        __syncthreads();
    }
    int buf = 0;
    for (int64_t c = 0; c < nchunks; ++c) {
#pragma unroll 1
        for (int i0 = 0; i0 < n0; ++i0) {
            const bool chunk_end = i0 == n0 - 1;
            const bool last_unit = c == nchunks - 1 && chunk_end;
            const int64_t nc = chunk_end ? c + 1 : c;  // chunk and dim-0 tap of the next unit
            const int ni0 = chunk_end ? 0 : i0 + 1;
            WRegs wr;
            XRegs<kMT> xr;
            if (!last_unit) load_w_taps_buf(a, ts, st, wo, nc * ICC, ni0, wr);
            if (chunk_end && !last_unit) load_x_buf(a, t, xo, nc * ICC, xr);
            const float* lw = lw0 + buf * LDS_W;
            const int xo0 = pick3(ts.d[0].off, i0) * HH * HW * 4;
#pragma unroll
            for (int u = 0; u < UNIT_TAPS; ++u) {
                if (u < ntu) {
                    const int xoff = xo0 + st.xo[u];
                    f32x4 av[kMT], bv[2];
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt) av[mt] = *reinterpret_cast<const f32x4*>(lx + abase[mt] + xoff);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        bv[nt] = *reinterpret_cast<const f32x4*>(lw + bbase + u * WTAP + nt * 256);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
                                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt][s], bv[nt][s],
                                                                                   acc[mt][nt], 0, 0, 0);
                }
            }
            if (last_unit) break;
            if (chunk_end) {
                __syncthreads();  // every wave is done with this chunk's halo
                store_x_buf(a, nc * ICC, xr, lx);
            }
            // the other weight buffer was last read by the previous unit, which
            // every wave finished before the previous barrier
            store_w_buf<kConvWeights>(wr, lw0 + (buf ^ 1) * LDS_W);
            __syncthreads();
            buf ^= 1;
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

// The buffer resources of the K loop stay below 2^31 bytes: one chunk of input
// channel planes, and the whole weight tensor.
inline bool fits_buffers(const Geom& g) {
    return (int64_t)ICC * g.S[0] * g.S[1] * g.S[2] * 4 < (1ll << 31) && g.Cout * g.Cin * 27 * 4 < (1ll << 31);
}

}  // namespace mfma333
}  // namespace c3d
