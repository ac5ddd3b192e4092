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
// with one non-empty residue per dim).
//
// Every output element is written once.  The even planes, and the even rows
// of the odd planes, hold only the bias and do not depend on any tile, so they
// are shared out over the whole grid, not by tile: they are cut into units of
// one (sample, channel) volume's plane pair (plane 2k whole, the even rows of
// plane 2k + 1), and during K-loop unit u workgroup b writes chunk
// u * gridDim + b of those units in memory order.  The workgroups resident at
// one time then write adjacent chunks, a compact write front that HBM absorbs
// far faster than every workgroup writing its own scattered box.  After the K
// loop a workgroup writes the odd rows of the odd planes of its box, odd
// positions from the tile and even positions as the bias, staging the tile in
// LDS 32 output channels at a time.
#include "conv333_mfma.h"

namespace c3d {
namespace {

using namespace mfma333;

constexpr int kMT = 4;  // tile depth; the result staging (32 channels at a time) reuses the K-loop LDS
constexpr int TD = Geo<kMT>::TD;
constexpr int kStage = TD * TH * TW + 1;  // LDS floats per channel of the result staging (padded)
constexpr int kLdsFloats = Geo<kMT>::LDS_MAIN > 32 * kStage ? Geo<kMT>::LDS_MAIN : 32 * kStage;
constexpr int kMaxBiasLds = 1024;  // output channels whose bias the even-plane pass keeps in LDS

// n / d for 0 <= n, d < 2^22 from a float reciprocal: the rounded product is
// within 1/2 of n / d, so its truncation is off by at most one, which one
// remainder check corrects.
struct Div {
    int d;
    float inv;
    __device__ Div() : d(1), inv(1.f) {}
    __device__ explicit Div(int d_) : d(d_), inv(1.f / (float)(d_ > 0 ? d_ : 1)) {}
    __device__ int quot(int n) const {
        int q = (int)((float)n * inv);
        const int r = n - q * d;
        if (r < 0)
            --q;
        else if (r >= d)
            ++q;
        return q;
    }
};

// Destination box of a workgroup: channels oc0 + oc (oc < ocs), planes
// lo[0] + id (id < bd), rows lo[1] + ih (ih < bh), columns lo[2] + c (c < bw).
struct Box {
    int lo[3];
    int bd, bh, bw, ocs;
    int64_t plane, Y1, Y2;
    float* yn;       // channel oc0 of this workgroup's sample
    bool full_rows;  // the box spans complete rows, so a plane of it is contiguous
    Div div_bw;
};

// A set of runs inside the box.  A run is a contiguous stretch of y: either
// a whole plane of the box (slab; needs full rows) or one row.  Planes
// id = id0 + id_step * i (i < n1); rows ih = ih0 + ih_step * j (j < n2, row
// runs only).  Each run is cut into 16-byte aligned slots of 4 floats counted
// from the run's actual address; item g of the set is slot g % SL of run
// g / SL, and runs are ordered (oc, i, j).
struct RunSet {
    int id0, id_step, n1;
    int ih0, ih_step, n2;
    bool slab;
    int L, SL, items;  // floats per run, slots per run (enough for any alignment), items
    Div div_sl, div_n1, div_n2;
};

__device__ inline int count_from(int first, int step, int end) {
    return first < end ? (end - first + step - 1) / step : 0;
}

__device__ inline RunSet make_runs(const Box& b, int id0, int id_step, int ih0, int ih_step, bool slab) {
    const int n1 = count_from(id0, id_step, b.bd);
    const int n2 = slab ? 1 : count_from(ih0, ih_step, b.bh);
    const int L = slab ? b.bh * b.bw : b.bw;
    const int SL = (L + 6) >> 2;
    return RunSet{id0, id_step, n1, ih0, ih_step, n2, slab, L, SL, b.ocs * n1 * n2 * SL,
                  Div(SL), Div(n1), Div(n2)};
}

// Writes items [g0, g1) of a run set with the whole workgroup.  A slot wholly
// inside its run is written with one 16-byte store, the partial slots at a
// run's two ends float by float.  value(oc, id, ih, c, in) gives the float at
// box coordinates (oc, id, ih, c); in is false for the floats of a partial
// slot that lie outside the run (their value is discarded).
template <class Value>
__device__ __forceinline__ void store_runs(const Box& b, const RunSet& rs, int g0, int g1, const Value& value) {
    for (int g = g0 + (int)threadIdx.x; g < g1; g += kThreads) {
        int r = rs.div_sl.quot(g);
        const int s = g - r * rs.SL;
        int j = 0;
        if (!rs.slab) {
            const int r2 = rs.div_n2.quot(r);
            j = r - r2 * rs.n2;
            r = r2;
        }
        const int oc = rs.div_n1.quot(r);
        const int id = rs.id0 + rs.id_step * (r - oc * rs.n1);
        const int ihr = rs.slab ? 0 : rs.ih0 + rs.ih_step * j;
        float* run = b.yn + oc * b.plane + ((int64_t)(b.lo[0] + id) * b.Y1 + b.lo[1] + ihr) * b.Y2 + b.lo[2];
        const int e0 = 4 * s - (int)(((uintptr_t)run >> 2) & 3);  // run offset of the slot's first float
        // box row and column of the slot's first float; a float before the run
        // start (e0 < 0) gets a negative column and is never stored
        int ih = ihr, c = e0;
        if (rs.slab && e0 > 0) {
            ih = b.div_bw.quot(e0);
            c = e0 - ih * b.bw;
        }
        float v[4];
        bool in[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int ck = c + k, ihk = ih;
            if (rs.slab && ck >= b.bw) {  // slabs have bw >= 4: at most one row change per slot
                ck -= b.bw;
                ++ihk;
            }
            in[k] = e0 + k >= 0 && e0 + k < rs.L;
            v[k] = value(oc, id, ihk, ck, in[k]);
        }
        if (in[0] && in[3]) {
            const f32x4 o = {v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(run + e0) = o;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (in[k]) run[e0 + k] = v[k];
        }
    }
}

// kLattice = 1: box coordinate (id, ih, c) is tile voxel (id, ih, c).
// kLattice = 2: the box starts at even destination coordinates, so a box
// coordinate is odd exactly when the destination coordinate is; odd 2m + 1
// is tile voxel m, and a voxel with any even coordinate is the bias alone.
template <int kLattice>
struct TileValue {
    const float* lds;
    const float* sbias;
    __device__ float operator()(int oc, int id, int ih, int c, bool in) const {
        const bool from_tile = kLattice == 1 || (id & ih & c & 1) != 0;
        const int idx = kLattice == 1 ? (id * TH + ih) * TW + c : ((id >> 1) * TH + (ih >> 1)) * TW + (c >> 1);
        const float tv = lds[oc * kStage + (in && from_tile ? idx : 0)];
        return (from_tile ? tv : 0.f) + sbias[oc];
    }
};

// Side work of the transposed conv: the bias-only outputs of the whole grid.
// Unit k of volume nc (sample-channel) is plane 2k whole and the even rows of
// plane 2k + 1; each run is cut into 16-byte aligned slots counted from its
// address.  The units are split into n * gridDim chunks of near-equal size;
// K-loop unit u of workgroup b writes chunk u * gridDim + b.
// Cache policy of the bias pass's stores: non-temporal (the nt bit), so the
// 435 MB of bias-only planes of the 32->64 stride-2 dilation-2 transposed
// conv of x[16,32,16,32,32] stream out instead of taking the caches from the
// K loop's operands: 0.291 -> 0.257-0.264 ms there in back-to-back calls,
// 0.289 -> 0.293-0.295 ms after a 512 MB write has left the caches dirty.
// (Non-temporal stores of the interleaved odd rows instead cost 0.26 ->
// 0.49 ms: they only pay for whole contiguous lines.)
constexpr int kStream = 2;

// Limits of the bias pass's fixed-count form: plane pairs per call, 16-byte
// stores per thread for one plane pair (an even plane and its odd plane's
// even rows)
constexpr int kMaxRun = 3, kPairIt = 7;

template <bool kFixed>
struct EvenPlanes {
    float* y;
    const float* bias;  // LDS copy of all Cout biases, or null for none
    int64_t P, vol;     // floats per plane and per (sample, channel) volume
    int units;          // (sample, channel) volumes x plane pairs
    int pairs, Y0, Y2, R, SLr, Cout;
    int q, rem;         // units per chunk of the n * gridDim chunks; the first rem chunks take one more
    // Fixed-count form (see below): this thread's byte offsets, from the
    // even plane's start, of its 16-byte and 4-byte stores in a plane pair
    // (kOutside where it has none)
    uint32_t poff[kPairIt], ptoff;
    // the pass goes behind the first tap of each unit (taps 0-5 measured
    // within 0.5 % of each other; the last tap about 2.5 % slower)
    static constexpr int kTap = 0;
    // the 16-byte slot s of a run of L floats whose start is m floats past a
    // 16-byte boundary
    __device__ __forceinline__ void slot(float* run, int m, int s, int L, float v) const {
        const int e0 = 4 * s - m;
        if (e0 >= 0 && e0 + 3 < L) {
            *reinterpret_cast<f32x4*>(run + e0) = f32x4{v, v, v, v};
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (e0 + k >= 0 && e0 + k < L) run[e0 + k] = v;
        }
    }
    // The unit bookkeeping is 32-bit and incremental (one division pair per
    // call): 64-bit divisions here, a long scalar sequence each, held every
    // wave's matrix-core work at each call.
    __device__ void operator()(int64_t u, int64_t) const {
        // chunks in XCD-aware order: consecutive workgroup ids go round-robin
        // to the 8 XCDs, so remapped, each XCD writes one contiguous run of
        // the unit's chunks (about 0.5 % on the 32->64 stride-2 dilation-2
        // transposed conv of x[16,32,16,32,32])
        const int nb = (int)gridDim.x;
        int bx = (int)blockIdx.x;
        if ((nb & 7) == 0) bx = (bx & 7) * (nb >> 3) + (bx >> 3);
        const int chunk = (int)u * nb + bx;
        const int g0 = chunk * q + (chunk < rem ? chunk : rem);
        const int cnt = q + (chunk < rem ? 1 : 0);
        int volume = g0 / pairs;
        int k = g0 - volume * pairs;
        int c = volume % Cout;
        if (kFixed) {
            // Branch-free: kMaxRun plane pairs (the ones past the run write
            // nothing, their resources being empty), each kPairIt 16-byte and
            // one 4-byte buffer store per thread at offsets fixed for the
            // thread.  The even plane and the odd plane's even rows go out as
            // 16-byte stores from their starts (4-byte aligned, which buffer
            // stores allow), their last Y2 % 4 floats as single floats; the
            // resource ends after the even plane when there is no odd plane.
#pragma unroll
            for (int i = 0; i < kMaxRun; ++i) {
                const float v = bias ? bias[c] : 0.f;
                const f32x4 vv = {v, v, v, v};
                float* base = y + (int64_t)volume * vol + (int64_t)(2 * k) * P;
                const uint32_t bytes = i < cnt ? (uint32_t)P * (2 * k + 1 < Y0 ? 8u : 4u) : 0u;
                const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, bytes);
#pragma unroll
                for (int m = 0; m < kPairIt; ++m) __builtin_amdgcn_raw_buffer_store_b128(vv, rs, poff[m], 0, kStream);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, ptoff, 0, kStream);
                if (++k == pairs) {
                    k = 0;
                    ++volume;
                    if (++c == Cout) c = 0;
                }
            }
            return;
        }
        if (cnt == 0) return;
        const Div div_slr(SLr);
        const int Pi = (int)P;
        for (int i = 0; i < cnt; ++i) {
            const float v = bias ? bias[c] : 0.f;
            float* base = y + (int64_t)volume * vol + (int64_t)(2 * k) * P;
            const int mb = (int)(((uintptr_t)base >> 2) & 3);
            // plane 2k: the 16-byte aligned body by buffer stores at a
            // per-thread constant offset from a uniform base, the up to 3
            // floats before and after it one by one
            {
                const int head = (4 - mb) & 3, nbody = (Pi - head) >> 2, tail = (Pi - head) & 3;
                const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base + head, (uint32_t)(nbody * 16));
                const f32x4 vv = {v, v, v, v};
                for (int g = threadIdx.x; g < nbody; g += kThreads)
                    __builtin_amdgcn_raw_buffer_store_b128(vv, rs, 16u * (unsigned)g, 0, 0);
                if ((int)threadIdx.x < head) base[threadIdx.x] = v;
                if ((int)threadIdx.x < tail) base[head + 4 * nbody + threadIdx.x] = v;
            }
            if (2 * k + 1 < Y0) {
                float* odd = base + P;
                const int items = R * SLr;
                for (int j = threadIdx.x; j < items; j += kThreads) {
                    const int r = div_slr.quot(j);
                    float* run = odd + (int64_t)(2 * r) * Y2;
                    slot(run, (int)(((uintptr_t)run >> 2) & 3), j - r * SLr, Y2, v);
                }
            }
            if (++k == pairs) {
                k = 0;
                ++volume;
                if (++c == Cout) c = 0;
            }
        }
    }
};

// kLattice = 1: destination o = q (plain conv).  kLattice = 2: destination
// o = 2q + 1 inside a destination grid of size Y (transposed conv); every
// destination voxel with an even coordinate holds the bias.
// two workgroups per CU: all 256 registers per lane hold the 4-plane tile's accumulators and the prefetch
template <int kMode, int kLattice, bool kFixed = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv333_store_kernel(
    Args a) {
    __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
    __shared__ float sbias[OCB];
    __shared__ float all_bias[kLattice == 2 ? kMaxBiasLds : 1];
    const Tile t = tile_of<kMT>(a);
    if (threadIdx.x < OCB)
        sbias[threadIdx.x] = (a.bias && t.oc0 + threadIdx.x < a.Cout) ? a.bias[t.oc0 + threadIdx.x] : 0.f;
    if (kLattice == 2 && a.bias)
        for (int c = threadIdx.x; c < a.Cout; c += kThreads) all_bias[c] = a.bias[c];
    // (the mainloop's first barrier publishes sbias and all_bias)

    Box b{};
    {
        const int64_t q0[3] = {t.d0, t.h0, t.w0};
        const int T[3] = {TD, TH, TW};
        int hi[3];
        for (int j = 0; j < 3; ++j) {
            if (kLattice == 1) {
                b.lo[j] = (int)q0[j];
                hi[j] = (int)(q0[j] + T[j] < a.Y[j] ? q0[j] + T[j] : a.Y[j]);
            } else {
                b.lo[j] = (int)(2 * q0[j]);
                hi[j] = (int)((q0[j] + T[j] >= a.O[j]) ? a.Y[j] : 2 * (q0[j] + T[j]));
            }
        }
        b.bd = hi[0] - b.lo[0];
        b.bh = hi[1] - b.lo[1];
        b.bw = hi[2] - b.lo[2];
        b.ocs = (int)(a.Cout - t.oc0 < OCB ? a.Cout - t.oc0 : OCB);
        b.plane = a.Y[0] * a.Y[1] * a.Y[2];
        b.Y1 = a.Y[1];
        b.Y2 = a.Y[2];
        b.yn = a.y + (t.n * a.Cout + t.oc0) * b.plane;
        b.full_rows = b.lo[2] == 0 && hi[2] == a.Y[2] && b.bw >= 4;
        b.div_bw = Div(b.bw);
    }

    f32x16 acc[kMT][2];
    if (kLattice == 2) {
        EvenPlanes<kFixed> ep;
        ep.y = a.y;
        ep.bias = a.bias ? all_bias : nullptr;
        ep.P = a.Y[1] * a.Y[2];
        ep.vol = a.Y[0] * ep.P;
        ep.pairs = (int)((a.Y[0] + 1) / 2);
        ep.units = (int)(a.N * a.Cout * ep.pairs);
        const int nch = 3 * (int)ceil_div(a.Cin, ICC) * (int)gridDim.x;  // K-loop units x workgroups
        ep.q = ep.units / nch;
        ep.rem = ep.units - ep.q * nch;
        ep.Y0 = (int)a.Y[0];
        ep.Y2 = (int)a.Y[2];
        ep.R = (int)((a.Y[1] + 1) / 2);
        ep.SLr = (int)((a.Y[2] + 6) >> 2);
        ep.Cout = (int)a.Cout;
        if (kFixed) {
            // The plane pair's 16-byte items: the even plane's P / 4 from its
            // start, then Y2 / 4 from the start of each of the odd plane's R
            // even rows (2 Y2 apart, starting P floats on); its single floats:
            // the even plane's last P % 4, then the last Y2 % 4 of each such
            // row.  The launcher picks kFixed where kPairIt items per thread
            // and one single float per thread suffice.
            const int Pi = (int)ep.P, Y2 = ep.Y2;
            const int nb = Pi >> 2, pr = Pi & 3, sl = Y2 >> 2, rm = Y2 & 3;
            const Div dsl(sl > 0 ? sl : 1), drm(rm > 0 ? rm : 1);
#pragma unroll
            for (int m = 0; m < kPairIt; ++m) {
                const int i = (int)threadIdx.x + m * kThreads;
                const int e = i - nb, r = dsl.quot(e > 0 ? e : 0), j = e - r * sl;
                ep.poff[m] = i < nb                   ? 16u * (unsigned)i
                             : sl > 0 && r < ep.R ? 4u * (unsigned)(Pi + 2 * r * Y2 + 4 * j)
                                                  : kOutside;
            }
            const int l = (int)threadIdx.x, e = l - pr, r = drm.quot(e > 0 ? e : 0), f = e - r * (rm > 0 ? rm : 1);
            ep.ptoff = l < pr                  ? 4u * (unsigned)(4 * nb + l)
                       : rm > 0 && r < ep.R ? 4u * (unsigned)(Pi + 2 * r * Y2 + 4 * sl + f)
                                            : kOutside;
        }
        mainloop<kMode, kMT>(a, t, lds, acc, ep);
    } else {
        mainloop<kMode, kMT>(a, t, lds, acc);
    }

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    if (t.d0 + TD <= a.O[0] && t.h0 + TH <= a.O[1] && t.w0 + TW <= a.O[2]) {
        // A tile wholly inside the grid writes straight from the accumulators:
        // a lane holds 4 consecutive tile voxels x0 .. x0 + 3 of one channel.
        // Plain conv: destination columns x0 .. x0 + 3, one 16-byte store.
        // Transposed conv: the odd rows of the odd planes, destination columns
        // 2x0 .. 2x0 + 7 alternating bias and value, two 16-byte stores.  The
        // stores are buffer stores into the workgroup's channel block, so
        // channels past Cout fall outside the resource and write nothing.
        const int64_t vol = a.Y[0] * a.Y[1] * a.Y[2];
        const int nvalid = (int)(a.Cout - t.oc0 < OCB ? a.Cout - t.oc0 : OCB);
        const __amdgpu_buffer_rsrc_t ys =
            buffer_rsrc(a.y + (t.n * a.Cout + t.oc0) * vol, (uint32_t)(nvalid * vol * 4));
        const int h = lane >> 5, n = lane & 31;
        const int Y1 = (int)a.Y[1], Y2 = (int)a.Y[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float bv = sbias[32 * nt + n];
            const unsigned cb = (unsigned)(32 * nt + n) * (unsigned)vol * 4u;
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int aa = 0; aa < 4; ++aa) {
                    const int y = (aa >> 1) + 2 * (wv >> 1), x0 = 8 * (aa & 1) + 4 * h + 16 * (wv & 1);
                    if (kLattice == 1) {
                        const int row = ((int)t.d0 + mt) * Y1 + (int)t.h0 + y;
                        const unsigned off = cb + 4u * (unsigned)(row * Y2 + (int)t.w0 + x0);
                        const f32x4 v = {acc[mt][nt][4 * aa] + bv, acc[mt][nt][4 * aa + 1] + bv,
                                         acc[mt][nt][4 * aa + 2] + bv, acc[mt][nt][4 * aa + 3] + bv};
                        __builtin_amdgcn_raw_buffer_store_b128(v, ys, off, 0, 0);
                    } else {
                        const int row = (2 * ((int)t.d0 + mt) + 1) * Y1 + 2 * ((int)t.h0 + y) + 1;
                        const unsigned off = cb + 4u * (unsigned)(row * Y2 + 2 * ((int)t.w0 + x0));
                        const f32x4 lo = {bv, acc[mt][nt][4 * aa] + bv, bv, acc[mt][nt][4 * aa + 1] + bv};
                        const f32x4 hi = {bv, acc[mt][nt][4 * aa + 2] + bv, bv, acc[mt][nt][4 * aa + 3] + bv};
                        __builtin_amdgcn_raw_buffer_store_b128(lo, ys, off, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b128(hi, ys, off + 16u, 0, 0);
                        // the even column after the last tile voxel of a row ends the row
                        if (x0 == TW - 4 && 2 * ((int)t.w0 + TW) < Y2)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bv), ys, off + 32u, 0, 0);
                    }
                }
        }
        return;
    }

    // stage and write the tile 32 output channels (one N tile) at a time
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();  // every wave is done reading the operand tiles, or the previous half
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int x, y, z;
                acc_voxel(lane, wv, mt, i, x, y, z);
                lds[(lane & 31) * kStage + (z * TH + y) * TW + x] = acc[mt][half][i];
            }
        __syncthreads();
        Box bh = b;
        bh.yn = b.yn + 32 * half * b.plane;
        bh.ocs = b.ocs - 32 * half < 32 ? b.ocs - 32 * half : 32;
        if (bh.ocs > 0) {
            // all of the box for the plain conv, the odd rows of its odd planes for the transposed conv
            const RunSet rest =
                kLattice == 1 ? make_runs(bh, 0, 1, 0, 1, bh.full_rows) : make_runs(bh, 1, 2, 1, 2, false);
            store_runs(bh, rest, 0, rest.items, TileValue<kLattice>{lds, sbias + 32 * half});
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
    a.xC = g.Cin;
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
    return g.groups == 1 && g.Cin >= 4 && g.Cout >= 8 && mfma333::fits_buffers(g) &&
           (int64_t)OCB * g.O[0] * g.O[1] * g.O[2] * 4 < (1ll << 31) && mfma333::fits_int32_tiles(g.O[0]) &&
           mfma333::fits_int32_tiles(g.O[1]) && mfma333::fits_int32_tiles(g.O[2]);
}

hipError_t launch_conv3x3x3_mfma(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                 hipStream_t st) {
    Args a = make_args(x, w, bias, y, g);
    for (int j = 0; j < 3; ++j) a.pad[j] = g.p[0];
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
    if (g.groups != 1 || g.Cout > kMaxBiasLds || !mfma333::fits_buffers(g) || !mfma333::fits_int32_tiles(g.O[0]) ||
        !mfma333::fits_int32_tiles(g.O[1]) || !mfma333::fits_int32_tiles(g.O[2]))
        return false;
    // the bias pass indexes a plane in 32 bits, decodes row slots below 2^22
    // with float reciprocals and counts its units in 32 bits; the odd-row
    // stores address a 64-channel block of the output with 32-bit byte offsets
    return g.O[1] * g.O[2] < (1 << 25) && (int64_t)OCB * g.O[0] * g.O[1] * g.O[2] * 4 < (1ll << 31) &&
           g.N * g.Cout * ((g.O[0] + 1) / 2) < (1ll << 30);
}

hipError_t launch_convT_s2_sublattice(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                      hipStream_t st) {
    Args a = make_args(x, w, bias, y, g);
    for (int j = 0; j < 3; ++j) a.pad[j] = 1;
    for (int j = 0; j < 3; ++j) {
        a.O[j] = g.S[j];  // sub-lattice grid = input grid
        a.Y[j] = g.O[j];  // destination = the transposed-conv output
    }
    a.tiles[0] = (int32_t)ceil_div(g.S[0], TD);
    a.tiles[1] = (int32_t)ceil_div(g.S[1], TH);
    a.tiles[2] = (int32_t)ceil_div(g.S[2], TW);
    const int64_t blocks = a.N * (int64_t)a.tiles[0] * a.tiles[1] * a.tiles[2] * a.oc_blocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    // the bias pass's counts, as the kernel derives them: plane pairs per call
    // (units over K-loop units x workgroups), 16-byte items and single floats
    // per plane pair (an even plane and its odd plane's even rows)
    const int64_t P = g.O[1] * g.O[2], pairs = (g.O[0] + 1) / 2, R = (g.O[1] + 1) / 2;
    const int64_t units = g.N * g.Cout * pairs, nch = 3 * ceil_div(g.Cin, ICC) * blocks;
    const int64_t run = units / nch + (units % nch ? 1 : 0);
    const bool fixed = run <= kMaxRun && (P >> 2) + R * (g.O[2] >> 2) <= kPairIt * kThreads &&
                       (P & 3) + R * (g.O[2] & 3) <= kThreads;
    if (fixed)
        hipLaunchKernelGGL((conv333_store_kernel<kConvTFlipped, 2, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           st, a);
    else
        hipLaunchKernelGGL((conv333_store_kernel<kConvTFlipped, 2>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                           a);
    return hipGetLastError();
}

}  // namespace c3d
