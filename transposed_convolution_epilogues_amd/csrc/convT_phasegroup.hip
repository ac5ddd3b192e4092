// convT_phasegroup.hip - ConvTranspose3d with all output phases of a tile
// computed from one staged input halo ("Kimi-K2.6 l1_p77", the residue-class
// decomposition of the gather form: per dim o = s*q + r, and tap k reaches
// phase r from input q + delta with delta = (r + p - k*d) / s whenever that
// division is exact).
//
// The per-phase kernel (convT_phase.hip) stages a halo for every phase of a
// tile, so a phase with one tap per dim pays a whole staging pass for one
// tap's products.  Here the phases share the halo: the input offsets delta of
// every residue of a dim lie in a window of at most 3 positions, so one halo
// of tile + (span - 1) per dim serves them all, and every tap of the kernel
// is applied once per staged chunk.
//
// GEMM orientation: M = 32 output channels, N = 32 consecutive q positions
// along dim 2, K = input channels, on v_mfma_f32_32x32x2f32.  A workgroup
// (8 waves) owns 2 x 4 rows of 32 positions (a wave per row) x 32 output
// channels x up to 8 phases; a wave keeps one 32 x 32 accumulator tile per
// phase.  In the result a lane holds one position and 16 channels, so the
// phases r2 = 0, 1 of a stride-2 dim 2 sit side by side in the lane and go
// out as one 8-byte store, and 32 lanes write 256 contiguous bytes.
//
// K loop: chunks of ICC input channels.  A chunk's halo ([half][pos][ICC/2]:
// lane half h supplies channel h*ICC/2 + s in K-step s) and the weights of
// every kernel tap ([tap][half][oc][ICC/2]) sit in one of two LDS buffers;
// the next chunk is loaded into registers while the current one is
// multiplied and written to the other buffer afterwards: one barrier per
// chunk.
//
// When more than 8 phases exist (strides 3 and 4), a workgroup takes the
// phases of its fixed leading residues (a grid dimension) and all residues of
// the trailing dims.
#include <limits.h>

#include <type_traits>

#include "c3d_internal.h"

namespace c3d {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x3 __attribute__((ext_vector_type(3)));

// A buffer load or store whose offset is at least the resource's size touches
// no memory (a load returns 0).  Resources here are below 2^31 bytes, so an
// offset of kOutside (plus any uniform offset below 2^31) always falls outside.
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kR0 = 2, kR1 = 4;  // rows of the tile in dims 0 and 1: a wave per row
constexpr int kTW = 32;          // q positions per row: the MFMA's N
constexpr int kOCB = 32;         // output channels per workgroup: the MFMA's M
constexpr int kHX0 = kR0 + 2, kHX1 = kR1 + 2, kHX2 = kTW + 2;  // halo layout (largest span 3)
constexpr int kHPos = kHX0 * kHX1 * kHX2;
constexpr int kMaxPh = 8;       // phases per workgroup (one accumulator tile each)
constexpr int kMaxS = 4, kMaxT = 3;
constexpr int kMaxTaps = 64;     // kernel taps: the weights of one chunk sit in LDS
constexpr int kMaxGroups = 16;   // phase groups (fixed leading residues)
constexpr int kHaloPer = (kHPos + kThreads - 1) / kThreads;  // halo positions per thread

struct GArgs {
    const float* x;
    const float* w;
    const float* bias;
    float* y;
    int32_t cin, cout;        // per group
    int32_t kvol;
    int32_t S[3], O[3];
    int32_t s[3];
    int32_t org[3];           // halo origin = q origin - org
    int32_t ext[3];           // halo extent beyond a tile row: span of the input offsets - 1
    int32_t Q[3][kMaxS];      // outputs of residue r: ceil((O - r) / s)
    int64_t xC, yC;           // channels per sample of x and y
    int32_t tiles[3];
    int32_t oc_blocks, groups, pgroups, P;
    int32_t vecs;             // s2 when dim 2 is free, s2 > 1 and s2 divides O2: a lane's residues
                              // along dim 2 are contiguous and go out in one store; else 0
    int32_t nchunks;
    int32_t fold;             // 2: rows of at most 16 positions, a wave takes two of them (a half-wave
                              // each); 1 otherwise (always 1 for the fixed geometries)
    int32_t hx1, hx2;         // halo layout strides of dims 1 and 2 (positions)
    int32_t pg_inner;         // more than one phase group and at most two chunks: a workgroup stages
                              // every input channel once and runs pg_per phase groups
    int32_t pg_split, pg_per; // with pg_inner: workgroups per tile, phase groups per workgroup
    int32_t one_tap;          // with pg_inner: two chunks, at most 4 phases per group and one tap
                              // per phase (kernel = stride in every dim); the tap of phase p of
                              // group g is g P + p
    int32_t one_tap_db;       // with one_tap: the P phases of a group are the dim-2 residues and
                              // leave in one P-float store per lane and channel (vecs == P), every
                              // channel block is full and a block's output spans < 2^31 bytes:
                              // the stores of a group are issued between the next group's products
    float inv_e2, inv_e12, inv_kvol;  // reciprocals for the staging index splits
    int64_t x_gstride, w_gstride, y_gstride;
    // tap table: LDS offsets (floats) of each tap's weights and halo window,
    // the taps of phase p of group g at [gbeg[g][p], gbeg[g][p + 1])
    int32_t tapw[kMaxTaps], tapx[kMaxTaps];
    int32_t gbeg[kMaxGroups][kMaxPh + 1];
    int32_t gres[kMaxGroups][kMaxPh];  // residues of phase p of group g: r0 | r1 << 4 | r2 << 8
};

// The two common strided layers with the tap structure fixed at compile time
// (every dim alike, dilation 1): kernel 3, stride 2, padding 1 (the x2
// upsampling layer, any output padding) and kernel 4, stride 2, padding 1.
// Per dim, residue r takes the taps k with (r + p - k) even, from input
// offset (r + p - k) / 2; the LDS offsets then become immediates.
template <int K, int P>
struct FixedDim {
    static constexpr int n(int r) {
        int c = 0;
        for (int k = 0; k < K; ++k) c += ((r + P - k) % 2 + 2) % 2 == 0;
        return c;
    }
    static constexpr int dmin() {
        int m = 1 << 20;
        for (int r = 0; r < 2; ++r)
            for (int k = 0; k < K; ++k)
                if (((r + P - k) % 2 + 2) % 2 == 0 && (r + P - k) / 2 < m) m = (r + P - k) / 2;
        return m;
    }
    static constexpr int k(int r, int i) {
        for (int k = 0, c = 0; k < K; ++k)
            if (((r + P - k) % 2 + 2) % 2 == 0 && c++ == i) return k;
        return 0;
    }
    static constexpr int off(int r, int i) { return (r + P - k(r, i)) / 2 - dmin(); }
};
// KS: 0 = any geometry (tap table), 1 = k3 s2 p1, 2 = k4 s2 p1
template <int KS>
struct Fixed;
template <>
struct Fixed<1> : FixedDim<3, 1> {};
template <>
struct Fixed<2> : FixedDim<4, 1> {};

template <int ICC, int KV>
struct Lay {
    static constexpr int kHalf = ICC / 2;  // K-steps per tap
    // floats per tap of the weights: = kHalf (mod 64), so that the staging
    // writes of consecutive taps land on distinct banks
    static constexpr int kWTS = kOCB * ICC + kHalf;
    static constexpr int kXF = kHPos * ICC;       // floats of the halo
    static constexpr int kBuf = kXF + KV * kWTS;  // floats per buffer
    static constexpr int kUnits = 2 * kOCB * KV;  // staging units (half, oc, tap) of kHalf channels
    static constexpr int kWPer = (kUnits + kThreads - 1) / kThreads;
};

template <int ICC, int KV, int KS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void convT_phasegroup_kernel(
    GArgs a) {
    using L = Lay<ICC, KV>;
    constexpr int H = L::kHalf;
    using VA = typename std::conditional<H == 4, f32x4, f32x2>::type;
    __shared__ __attribute__((aligned(16))) float lds[2 * L::kBuf];
    __shared__ int2 taps[KV];

    // workgroup -> (sample, group, tile, phase group, channel block), channel
    // block fastest so the blocks of one tile meet in one XCD's L2
    const int64_t nb = (int64_t)gridDim.x;
    int64_t b = blockIdx.x;
    if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    const int ocb = (int)(b % a.oc_blocks);
    b /= a.oc_blocks;
    // the phase group (with pg_inner: the first of the workgroup's pg_per)
    const int pgn = a.pg_inner ? a.pg_split : a.pgroups;
    const int pg0 = (int)(b % pgn) * (a.pg_inner ? a.pg_per : 1);
    b /= pgn;
    const int t2 = (int)(b % a.tiles[2]);
    b /= a.tiles[2];
    const int t1 = (int)(b % a.tiles[1]);
    b /= a.tiles[1];
    const int t0 = (int)(b % a.tiles[0]);
    b /= a.tiles[0];
    const int grp = (int)(b % a.groups);
    const int64_t n = b / a.groups;
    const int oc0 = ocb * kOCB;
    // tile: kR0 x (kR1 fold) rows of kTW / fold positions; lane nn of wave
    // (wr0, wr1) takes row (wr0, wr1 fold + nn / (kTW / fold)), position
    // nn % (kTW / fold)
    const int fold = KS == 0 ? a.fold : 1;
    const int rw = kTW / fold;
    const int hx1 = KS == 0 ? a.hx1 : kHX1, hx2 = KS == 0 ? a.hx2 : kHX2;
    const int q0 = t0 * kR0, q1 = t1 * kR1 * fold, q2 = t2 * rw;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int h = lane >> 5, nn = lane & 31;
    const int wr0 = wv / kR1, wr1 = wv % kR1;
    const int lr0 = wr0, lr1 = wr1 * fold + nn / rw, lp = nn % rw;

    if (KS == 0 && tid < a.kvol) taps[tid] = int2{a.tapw[tid], a.tapx[tid]};

    // ---- staging: halo positions of this thread
    const int64_t plane = (int64_t)a.S[0] * a.S[1] * a.S[2];
    const float* xg = a.x + (n * a.xC + (int64_t)grp * a.cin) * plane;
    int xsp[kHaloPer];  // spatial offset in an input channel plane, -1: zero padding
    int xlp[kHaloPer];  // LDS position, -1: no position
    {
        const int e2 = rw + a.ext[2], e12 = (kR1 * fold + a.ext[1]) * e2;
        const int cnt = (kR0 + a.ext[0]) * e12;
#pragma unroll
        for (int u = 0; u < kHaloPer; ++u) {
            const int hp = tid + u * kThreads;
            const int c0 = (int)(((float)hp + 0.5f) * a.inv_e12), r = hp - c0 * e12;
            const int c1 = (int)(((float)r + 0.5f) * a.inv_e2), c2 = r - c1 * e2;
            const int g0 = q0 - a.org[0] + c0, g1 = q1 - a.org[1] + c1, g2 = q2 - a.org[2] + c2;
            const bool in = hp < cnt && g0 >= 0 && g0 < a.S[0] && g1 >= 0 && g1 < a.S[1] && g2 >= 0 && g2 < a.S[2];
            xsp[u] = in ? (g0 * a.S[1] + g1) * a.S[2] + g2 : -1;
            xlp[u] = hp < cnt ? (c0 * hx1 + c1) * hx2 + c2 : -1;
        }
    }
    // ---- staging: weight units (half hh, channel oc, tap) of this thread,
    // each the kHalf input channels hh*kHalf .. of one (oc, tap); packed:
    // weight-buffer offset (bits 0-13), offset in an input channel's run of
    // the block (14-24), hh (25), channel past cout (26); -1: no unit
    const float* wg = a.w + (int64_t)grp * a.w_gstride;
    const int wic = a.cout * a.kvol;  // floats between input channels in w
    const int wrun = kOCB * a.kvol;   // units per half
    const int wbase0 = oc0 * a.kvol;  // the block's first channel in an input channel's run
    static_assert(KV * L::kWTS < (1 << 14) && kOCB * KV <= (1 << 11), "packed weight unit");
    int wel[L::kWPer];
#pragma unroll
    for (int u = 0; u < L::kWPer; ++u) {
        const int m = tid + u * kThreads;
        const int hh = m >= wrun, rem = m - hh * wrun;
        const int oc = (int)(((float)rem + 0.5f) * a.inv_kvol), tap = rem - oc * a.kvol;
        const int wl = tap * L::kWTS + (hh * kOCB + oc) * H;
        wel[u] = m < 2 * wrun ? wl | rem << 14 | hh << 25 | (oc0 + oc >= a.cout) << 26 : -1;
    }

    // byte offsets for the staging buffer loads: a halo position in its
    // channel plane, a weight unit's first element relative to the group's
    // weights (input channel ic0 + s added as a uniform offset); kOutside for
    // zero padding, no unit and channels past cout: the range check makes
    // those loads return 0 without touching memory
    uint32_t xvo[kHaloPer], wvo[L::kWPer];
#pragma unroll
    for (int u = 0; u < kHaloPer; ++u) xvo[u] = xsp[u] >= 0 ? 4u * (uint32_t)xsp[u] : kOutside;
#pragma unroll
    for (int u = 0; u < L::kWPer; ++u) {
        const int v = wel[u];
        const int hh = (v >> 25) & 1, off = wbase0 + ((v >> 14) & 2047);
        wvo[u] = v >= 0 && !((v >> 26) & 1) ? 4u * (uint32_t)(hh * H * wic + off) : kOutside;
    }
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(wg, (uint32_t)(a.w_gstride * 4));

    using XR = float[kHaloPer][ICC];
    using WR = float[L::kWPer][H];
    float xr[kHaloPer][ICC];
    float wr[L::kWPer][H];
    // a chunk's halo and weights into registers xr_, wr_ (buffer loads: no
    // address arithmetic per load); channels past cin (a partial last chunk)
    // read channel ic0 of the halo, zeroed when stored, and nothing of the weights
    auto load_to = [&](int c, XR& xr_, WR& wr_) {
        const int ic0 = c * ICC;
        const bool full = ic0 + ICC <= a.cin;
        const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(xg + (int64_t)ic0 * plane, (uint32_t)(ICC * plane * 4));
#pragma unroll
        for (int i = 0; i < ICC; ++i) {
            const int soff = ic0 + i < a.cin ? (int)(i * plane * 4) : 0;
#pragma unroll
            for (int u = 0; u < kHaloPer; ++u)
                xr_[u][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xrs, xvo[u], soff, 0));
        }
#pragma unroll
        for (int u = 0; u < L::kWPer; ++u) {
            const int hh = (wel[u] >> 25) & 1;
#pragma unroll
            for (int s = 0; s < H; ++s) {
                const uint32_t vo = full || ic0 + hh * H + s < a.cin ? wvo[u] : kOutside;
                wr_[u][s] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(wrs, vo, (int)((ic0 + s) * wic * 4), 0));
            }
        }
    };
    // registers xr_, wr_ of chunk c into LDS buffer buf
    auto store_from = [&](int c, float* buf, const XR& xr_, const WR& wr_) {
        const int ic0 = c * ICC;
        const bool full = ic0 + ICC <= a.cin;
#pragma unroll
        for (int u = 0; u < kHaloPer; ++u) {
            if (xlp[u] < 0) continue;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                VA v;
#pragma unroll
                for (int s = 0; s < H; ++s) v[s] = xr_[u][hh * H + s];
                if (!full) {
#pragma unroll
                    for (int s = 0; s < H; ++s) v[s] = ic0 + hh * H + s < a.cin ? v[s] : 0.f;
                }
                *reinterpret_cast<VA*>(buf + (hh * kHPos + xlp[u]) * H) = v;
            }
        }
        float* wb = buf + L::kXF;
#pragma unroll
        for (int u = 0; u < L::kWPer; ++u) {
            const int v = wel[u];
            if (v < 0) continue;
            VA x;
#pragma unroll
            for (int s = 0; s < H; ++s) x[s] = wr_[u][s];
            *reinterpret_cast<VA*>(wb + (v & 16383)) = x;
        }
    };
    auto load = [&](int c) { load_to(c, xr, wr); };
    auto store = [&](int c, float* buf) { store_from(c, buf, xr, wr); };

    f32x16 acc[kMaxPh];
#pragma unroll
    for (int p = 0; p < kMaxPh; ++p)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[p][i] = 0.f;

    // this lane's operand bases: weights of channel row nn, halo at its position
    const int wbase = L::kXF + (h * kOCB + nn) * H;
    const int xbase = (h * kHPos + (lr0 * hx1 + lr1) * hx2 + lp) * H;

    // ---- epilogue: a lane holds position q2 + nn and channels
    // oc0 + 8(i/4) + 4h + i%4; the channel offsets are uniform multiples of
    // the channel stride, added to one row pointer per phase
    const int64_t O1 = a.O[1], O2 = a.O[2];
    const int64_t cst = (int64_t)a.O[0] * O1 * O2;  // floats between output channels
    const int p0 = q0 + lr0, p1 = q1 + lr1, pq = q2 + lp;
    auto load_bias = [&](float (&bs)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int oc = oc0 + 8 * (i >> 2) + 4 * h + (i & 3);
            bs[i] = (a.bias && oc < a.cout) ? a.bias[(int64_t)grp * a.cout + oc] : 0.f;
        }
    };
    // the accumulators A of group pg (NA = kMaxPh, or 4 on the one-tap path)
    // the stores are buffer stores into this workgroup's output channels
    // oc0 .. (one resource ending at the last channel below cout): a lane past
    // the output in any dim gets offset kOutside, so every store is one
    // instruction with one address add and no branch
    const unsigned cstb = (unsigned)cst * 4u;  // bytes between output channels
    const int nvalid = a.cout - oc0 < kOCB ? a.cout - oc0 : kOCB;
    const __amdgpu_buffer_rsrc_t yrs =
        buffer_rsrc(a.y + (int64_t)grp * a.y_gstride + (n * a.yC + oc0) * cst, (uint32_t)nvalid * cstb);
    auto epilogue_of = [&](int pg, const float (&bs)[16], auto& A) {
        constexpr int NA = std::extent<std::remove_reference_t<decltype(A)>>::value;
        const int vs = a.vecs;
#pragma unroll
        for (int p = 0; p < NA; ++p) {
            if (p >= a.P) break;
            if (vs && p % vs != 0) continue;
            const int res = a.gres[pg][p];
            const int r0 = res & 15, r1 = (res >> 4) & 15, r2 = res >> 8;
            // the residues of dim 2 are phases p .. p + vs - 1 when vs > 1
            const bool ok = p0 < a.Q[0][r0] && p1 < a.Q[1][r1] && pq < a.Q[2][vs ? 0 : r2];
            const int64_t e = ((int64_t)(a.s[0] * p0 + r0) * O1 + (a.s[1] * p1 + r1)) * O2 +
                              (vs ? (int64_t)vs * pq : (int64_t)a.s[2] * pq + r2);
            const unsigned lo = ok ? (unsigned)e * 4u + (unsigned)(4 * h) * cstb : kOutside;
            const int q1i = (p + 1) & (NA - 1), q2i = (p + 2) & (NA - 1), q3i = (p + 3) & (NA - 1);
            if (vs == 2) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    __builtin_amdgcn_raw_buffer_store_b64(f32x2{A[p][i] + bs[i], A[q1i][i] + bs[i]}, yrs,
                                                          lo + (unsigned)(8 * (i >> 2) + (i & 3)) * cstb, 0, 0);
            } else if (vs == 4) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        f32x4{A[p][i] + bs[i], A[q1i][i] + bs[i], A[q2i][i] + bs[i], A[q3i][i] + bs[i]}, yrs,
                        lo + (unsigned)(8 * (i >> 2) + (i & 3)) * cstb, 0, 0);
            } else if (vs == 3) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    __builtin_amdgcn_raw_buffer_store_b96(f32x3{A[p][i] + bs[i], A[q1i][i] + bs[i], A[q2i][i] + bs[i]},
                                                          yrs, lo + (unsigned)(8 * (i >> 2) + (i & 3)) * cstb, 0, 0);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(A[p][i] + bs[i]), yrs,
                                                          lo + (unsigned)(8 * (i >> 2) + (i & 3)) * cstb, 0, 0);
            }
        }
    };
    auto epilogue = [&](int pg, const float (&bs)[16]) { epilogue_of(pg, bs, acc); };

    // products of one staged chunk (buffer buf) for the phases of group pg
    auto compute = [&](const float* buf, int pg) {
        const float* bw = buf + wbase;
        const float* bx = buf + xbase;
        if constexpr (KS != 0) {
            // every phase and tap unrolled: the operand offsets are immediates,
            // and a halo window shared by several phases is read once
            using F = Fixed<KS>;
            constexpr int kK = KS == 1 ? 3 : 4;
#pragma unroll
            for (int p = 0; p < kMaxPh; ++p) {
                const int r0 = p >> 2, r1 = (p >> 1) & 1, r2 = p & 1;
#pragma unroll
                for (int u0 = 0; u0 < F::n(r0); ++u0)
#pragma unroll
                    for (int u1 = 0; u1 < F::n(r1); ++u1)
#pragma unroll
                        for (int u2 = 0; u2 < F::n(r2); ++u2) {
                            const int wo = ((F::k(r0, u0) * kK + F::k(r1, u1)) * kK + F::k(r2, u2)) * L::kWTS;
                            const int xo = ((F::off(r0, u0) * kHX1 + F::off(r1, u1)) * kHX2 + F::off(r2, u2)) * H;
                            const VA av = *reinterpret_cast<const VA*>(bw + wo);
                            const VA bv = *reinterpret_cast<const VA*>(bx + xo);
#pragma unroll
                            for (int s = 0; s < H; ++s)
                                acc[p] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bv[s], acc[p], 0, 0, 0);
                        }
            }
            // operand reads run ahead of the products: a first batch, then a
            // few reads behind every tap's products
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < KV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, H, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        } else {
#pragma unroll
            for (int p = 0; p < kMaxPh; ++p) {
                const int beg = a.gbeg[pg][p], end = a.gbeg[pg][p + 1];
                // four taps per step: their offsets, then all operand reads, then
                // the products, so the later taps' reads overlap the first tap's
                // products; the remaining taps one at a time
                int t = beg;
                for (; t + 4 <= end; t += 4) {
                    int2 o[4];
                    VA av[4], bv[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = taps[t + k];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        av[k] = *reinterpret_cast<const VA*>(bw + o[k].x);
                        bv[k] = *reinterpret_cast<const VA*>(bx + o[k].y);
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k)
#pragma unroll
                        for (int s = 0; s < H; ++s)
                            acc[p] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[k][s], bv[k][s], acc[p], 0, 0, 0);
                    // keep the eight operand reads ahead of the products (the
                    // scheduler otherwise puts each tap's reads right before its
                    // products and waits for them there)
                    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 4 * H, 0);
                }
                for (; t < end; ++t) {
                    const int2 o = taps[t];
                    const VA av = *reinterpret_cast<const VA*>(bw + o.x);
                    const VA bv = *reinterpret_cast<const VA*>(bx + o.y);
#pragma unroll
                    for (int s = 0; s < H; ++s)
                        acc[p] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bv[s], acc[p], 0, 0, 0);
                }
            }
        }
    };

    if (KS == 0 && a.pg_inner) {
        // every input channel fits the two buffers: stage them once and run
        // every phase group from them (more than one group needs a stride
        // above 2, so the fixed geometries never take this path)
        // both chunks' loads in flight together
        float xr1[kHaloPer][ICC];
        float wr1[L::kWPer][H];
        load(0);
        if (a.nchunks > 1) load_to(1, xr1, wr1);
        store(0, lds);
        if (a.nchunks > 1) store_from(1, lds + L::kBuf, xr1, wr1);
        __syncthreads();
        float bs[16];
        load_bias(bs);
        const int pg_end = pg0 + a.pg_per < a.pgroups ? pg0 + a.pg_per : a.pgroups;
        if (a.one_tap) {
            // one tap per phase (P = NP phases): every operand of the group is
            // read before its products, each phase's first product starts from
            // zero, and the next group's tap offsets are read before the stores
            const f32x16 zero = {};
            auto groups = [&](auto npc) {
                constexpr int NP = decltype(npc)::value;
                int2 o[NP];
#pragma unroll
                for (int p = 0; p < NP; ++p) o[p] = taps[pg0 * NP + p];
                for (int pg = pg0; pg < pg_end; ++pg) {
                    // indexed in whole vectors (every offset is a multiple of H floats),
                    // so that each read is one 16- or 8-byte LDS read
                    const VA* lv = reinterpret_cast<const VA*>(lds);
                    VA av[NP][2], bv[NP][2];
#pragma unroll
                    for (int p = 0; p < NP; ++p)
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            av[p][c] = lv[(unsigned)(c * L::kBuf + wbase + o[p].x) / H];
                            bv[p][c] = lv[(unsigned)(c * L::kBuf + xbase + o[p].y) / H];
                        }
                    f32x16 ac[4];
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        ac[p] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[p][0][0], bv[p][0][0], zero, 0, 0, 0);
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int s = c == 0 ? 1 : 0; s < H; ++s)
                                ac[p] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[p][c][s], bv[p][c][s], ac[p], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x100, 4 * NP, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * H * NP, 0);
                    const int pn = pg + 1 < pg_end ? pg + 1 : pg;
#pragma unroll
                    for (int p = 0; p < NP; ++p) o[p] = taps[pn * NP + p];
                    epilogue_of(pg, bs, ac);
                }
            };
            // two accumulator sets: group g + 1's products are issued between
            // group g's stores, which are range-checked buffer stores (lanes
            // past the output get an offset past the block), so the products
            // and the stores form one basic block
            auto groups_db = [&](auto npc) {
                constexpr int NP = decltype(npc)::value;
                using VS = typename std::conditional<NP == 3, f32x3, f32x4>::type;
                const int64_t cst64 = (int64_t)a.O[0] * a.O[1] * a.O[2];
                float* yblk = a.y + (int64_t)grp * a.y_gstride + (n * a.yC + oc0) * cst64;
                const unsigned cstb = (unsigned)cst64 * 4u;  // bytes between channels
                const __amdgpu_buffer_rsrc_t rs =
                    __builtin_amdgcn_make_buffer_rsrc((void*)yblk, (short)0, (int)(kOCB * cstb), 0x00020000);
                // this lane's byte offset in the block for group pg, 0x80000000 when
                // its row or position lies past the output (every store dropped)
                auto lane_off = [&](int pg) -> unsigned {
                    const int res = a.gres[pg][0];
                    const int r0 = res & 15, r1 = (res >> 4) & 15;
                    const bool ok = p0 < a.Q[0][r0] && p1 < a.Q[1][r1] && pq < a.Q[2][0];
                    const unsigned e = (unsigned)(((a.s[0] * p0 + r0) * a.O[1] + a.s[1] * p1 + r1) * a.O[2] + NP * pq);
                    return ok ? e * 4u + (unsigned)(4 * h) * cstb : 0x80000000u;
                };
                const VA* lv = reinterpret_cast<const VA*>(lds);
                int2 o[NP];
                VA av[NP][2], bv[NP][2];
                auto operands = [&]() {
#pragma unroll
                    for (int p = 0; p < NP; ++p)
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            av[p][c] = lv[(unsigned)(c * L::kBuf + wbase + o[p].x) / H];
                            bv[p][c] = lv[(unsigned)(c * L::kBuf + xbase + o[p].y) / H];
                        }
                };
                auto products = [&](f32x16 (&ac)[NP]) {
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        ac[p] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[p][0][0], bv[p][0][0], zero, 0, 0, 0);
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int s = c == 0 ? 1 : 0; s < H; ++s)
                                ac[p] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[p][c][s], bv[p][c][s], ac[p], 0, 0, 0);
                    }
                };
                auto stores = [&](unsigned lo, const f32x16 (&ac)[NP]) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        VS v;
#pragma unroll
                        for (int p = 0; p < NP; ++p) v[p] = ac[p][i] + bs[i];
                        const unsigned off = lo + (unsigned)(8 * (i >> 2) + (i & 3)) * cstb;
                        if constexpr (NP == 3)
                            __builtin_amdgcn_raw_buffer_store_b96(v, rs, off, 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
                    }
                };
                auto taps_of = [&](int pg) {
#pragma unroll
                    for (int p = 0; p < NP; ++p) o[p] = taps[pg * NP + p];
                };
                // operand reads, then the stores of the previous group between
                // the products of this one
                auto interleave = [&]() {
                    __builtin_amdgcn_sched_group_barrier(0x100, 4 * NP, 0);
                    __builtin_amdgcn_sched_group_barrier(0x040, 2, 0);
#pragma unroll
                    for (int k = 0; k < 14; ++k) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);
                    }
                };
                f32x16 acA[NP], acB[NP];
                taps_of(pg0);
                operands();
                products(acA);
                int g = pg0;
                for (;;) {
                    const unsigned loA = lane_off(g);
                    if (g + 1 >= pg_end) {
                        stores(loA, acA);
                        break;
                    }
                    taps_of(g + 1);
                    operands();
                    products(acB);
                    stores(loA, acA);
                    interleave();
                    ++g;
                    const unsigned loB = lane_off(g);
                    if (g + 1 >= pg_end) {
                        stores(loB, acB);
                        break;
                    }
                    taps_of(g + 1);
                    operands();
                    products(acA);
                    stores(loB, acB);
                    interleave();
                    ++g;
                }
            };
            if (a.one_tap_db) {
                if (a.P == 3)
                    groups_db(std::integral_constant<int, 3>{});
                else
                    groups_db(std::integral_constant<int, 4>{});
            } else if (a.P == 3) {
                groups(std::integral_constant<int, 3>{});
            } else {
                groups(std::integral_constant<int, 4>{});
            }
            return;
        }
        for (int pg = pg0; pg < pg_end; ++pg) {
#pragma unroll
            for (int p = 0; p < kMaxPh; ++p)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[p][i] = 0.f;
            for (int c = 0; c < a.nchunks; ++c) compute(lds + c * L::kBuf, pg);
            epilogue(pg, bs);
        }
        return;
    }

    load(0);
    store(0, lds);
    __syncthreads();
    for (int c = 0; c < a.nchunks; ++c) {
        const bool more = c + 1 < a.nchunks;
        if (more) load(c + 1);
        compute(lds + (c & 1) * L::kBuf, pg0);
        if (more) store(c + 1, lds + ((c + 1) & 1) * L::kBuf);
        // the other buffer was last read in the previous chunk, which every wave
        // finished before the previous barrier; this one lets the next chunk
        // read what was just stored
        __syncthreads();
    }
    float bs[16];
    load_bias(bs);
    epilogue(pg0, bs);
}

// Taps of one dim: per residue r the kernel indices k[r][t] and input offsets
// delta; false when a residue has more than 3 taps or the offsets of all
// residues together span more than 3 positions.
struct DimTaps {
    int n[kMaxS];
    int k[kMaxS][kMaxT];
    int off[kMaxS][kMaxT];  // delta - min delta
    int org, ext;
};

bool dim_taps(int32_t K, int32_t s, int32_t p, int32_t d, DimTaps& t) {
    if (s < 1 || s > kMaxS) return false;
    t = DimTaps{};
    int dd[kMaxS][kMaxT];
    int dmin = INT_MAX, dmax = INT_MIN;
    for (int r = 0; r < s; ++r) {
        int cnt = 0;
        for (int k = 0; k < K; ++k) {
            const int num = r + p - k * d;
            if (((num % s) + s) % s != 0) continue;
            if (cnt == kMaxT) return false;
            t.k[r][cnt] = k;
            dd[r][cnt] = num / s;  // exact
            dmin = dd[r][cnt] < dmin ? dd[r][cnt] : dmin;
            dmax = dd[r][cnt] > dmax ? dd[r][cnt] : dmax;
            ++cnt;
        }
        t.n[r] = cnt;
    }
    if (dmin == INT_MAX) return false;  // K >= 1 always gives a tap
    if (dmax - dmin > 2) return false;
    t.org = -dmin;
    t.ext = dmax - dmin;
    for (int r = 0; r < s; ++r)
        for (int i = 0; i < t.n[r]; ++i) t.off[r][i] = dd[r][i] - dmin;
    return true;
}

int fixed_kind(const Geom& g);

template <int ICC, int KV>
bool build_gargs(const Geom& g, GArgs& a) {
    using L = Lay<ICC, KV>;
    a = GArgs{};
    // rows of at most 16 positions fold two to a wave (tap-table kernels only)
    a.fold = fixed_kind(g) == 0 && ceil_div(g.O[2], g.s[2]) <= kTW / 2 ? 2 : 1;
    a.hx1 = kR1 * a.fold + 2;
    a.hx2 = kTW / a.fold + 2;
    static_assert(kHX0 * (kR1 * 2 + 2) * (kTW / 2 + 2) <= kHPos, "folded halo layout");
    const int kvol = g.k[0] * g.k[1] * g.k[2];
    if (kvol > KV || kvol > kMaxTaps) return false;
    DimTaps dt[3];
    for (int j = 0; j < 3; ++j) {
        if (g.S[j] > INT_MAX || g.O[j] < 1 || g.O[j] > INT_MAX) return false;
        if (!dim_taps(g.k[j], g.s[j], g.p[j], g.d[j], dt[j])) return false;
        a.S[j] = (int32_t)g.S[j];
        a.O[j] = (int32_t)g.O[j];
        a.s[j] = g.s[j];
        a.org[j] = dt[j].org;
        a.ext[j] = dt[j].ext;
        for (int r = 0; r < g.s[j]; ++r) a.Q[j][r] = g.O[j] > r ? (int32_t)((g.O[j] - r + g.s[j] - 1) / g.s[j]) : 0;
    }
    // phase groups: every phase when there are at most 8, else fix the
    // leading residues; phase p of a group enumerates the free residues
    // row-major, dim 2 fastest
    const int s0 = g.s[0], s1 = g.s[1], s2 = g.s[2];
    const int nfixed = s0 * s1 * s2 <= kMaxPh ? 0 : (s1 * s2 <= kMaxPh ? 1 : 2);
    int fr[3];
    a.pgroups = 1;
    a.P = 1;
    for (int j = 0; j < 3; ++j) {
        fr[j] = j >= nfixed ? g.s[j] : 1;
        if (j < nfixed) a.pgroups *= g.s[j];
        else a.P *= g.s[j];
    }
    if (a.P > kMaxPh || a.pgroups > kMaxGroups) return false;
    // tap table: weight offset k0 K1 K2 + k1 K2 + k2 taps, halo offset of the
    // tap's input window, both in floats of the LDS layout
    int nt = 0;
    for (int pg = 0; pg < a.pgroups; ++pg) {
        int rb[3], rest = pg;
        for (int j = 2; j >= 0; --j) {
            if (j < nfixed) {
                rb[j] = rest % g.s[j];
                rest /= g.s[j];
            } else {
                rb[j] = 0;
            }
        }
        for (int p = 0; p < kMaxPh; ++p) {
            a.gbeg[pg][p] = nt;
            if (p >= a.P) continue;
            const int r2 = rb[2] + p % fr[2], r1 = rb[1] + (p / fr[2]) % fr[1], r0 = rb[0] + p / (fr[2] * fr[1]);
            a.gres[pg][p] = r0 | r1 << 4 | r2 << 8;
            for (int u0 = 0; u0 < dt[0].n[r0]; ++u0)
                for (int u1 = 0; u1 < dt[1].n[r1]; ++u1)
                    for (int u2 = 0; u2 < dt[2].n[r2]; ++u2) {
                        if (nt == kvol) return false;  // cannot happen: every tap lies in one phase
                        const int kv = (dt[0].k[r0][u0] * g.k[1] + dt[1].k[r1][u1]) * g.k[2] + dt[2].k[r2][u2];
                        const int xo = (dt[0].off[r0][u0] * a.hx1 + dt[1].off[r1][u1]) * a.hx2 + dt[2].off[r2][u2];
                        a.tapw[nt] = kv * L::kWTS;
                        a.tapx[nt] = xo * L::kHalf;
                        ++nt;
                    }
        }
        a.gbeg[pg][kMaxPh] = nt;
    }
    a.vecs = nfixed < 3 && s2 > 1 && g.O[2] % s2 == 0 ? s2 : 0;
    a.cin = (int32_t)g.cin_g;
    a.cout = (int32_t)g.cout_g;
    a.kvol = kvol;
    a.xC = g.Cin;
    a.yC = g.Cout;
    const int R[3] = {kR0, kR1 * a.fold, kTW / a.fold};
    for (int j = 0; j < 3; ++j) {
        const int64_t tl = ceil_div(ceil_div(g.O[j], g.s[j]), R[j]);
        if (tl > INT_MAX) return false;
        a.tiles[j] = (int32_t)tl;
    }
    const int e2 = kTW / a.fold + a.ext[2], e12 = (kR1 * a.fold + a.ext[1]) * e2;
    a.inv_e2 = 1.0f / (float)e2;
    a.inv_e12 = 1.0f / (float)e12;
    a.inv_kvol = 1.0f / (float)kvol;
    a.oc_blocks = (int32_t)ceil_div(g.cout_g, kOCB);
    a.groups = g.groups;
    a.nchunks = (int32_t)ceil_div(g.cin_g, ICC);
    a.pg_inner = a.pgroups > 1 && a.nchunks <= 2;
    a.pg_split = a.pgroups;  // the most workgroups per tile; the launch may merge phase groups
    a.pg_per = 1;
    a.one_tap = a.pg_inner && a.nchunks == 2 && (a.P == 3 || a.P == 4) && nt == a.pgroups * a.P;
    for (int pg = 0; pg < a.pgroups && a.one_tap; ++pg)
        for (int p = 0; p < a.P; ++p) a.one_tap = a.one_tap && a.gbeg[pg][p] == pg * a.P + p;
    a.x_gstride = (int64_t)g.cin_g * g.S[0] * g.S[1] * g.S[2];
    a.w_gstride = (int64_t)g.cin_g * g.cout_g * kvol;
    a.y_gstride = (int64_t)g.cout_g * g.O[0] * g.O[1] * g.O[2];
    // 32-bit offsets inside the kernel: a chunk's weights and an input plane;
    // the staging buffer resources (a chunk of input planes, a group's
    // weights) stay below 2^31 bytes
    if ((int64_t)ICC * g.cout_g * kvol > INT_MAX || g.S[0] * g.S[1] * g.S[2] > INT_MAX) return false;
    if ((int64_t)ICC * g.S[0] * g.S[1] * g.S[2] * 4 >= ((int64_t)1 << 31) || a.w_gstride * 4 >= ((int64_t)1 << 31))
        return false;
    // and the output resource of a workgroup's channel block
    if ((int64_t)kOCB * g.O[0] * g.O[1] * g.O[2] * 4 >= ((int64_t)1 << 31)) return false;
    return true;
}

int64_t grid_blocks(const Geom& g, const GArgs& a) {
    return g.N * (int64_t)g.groups * a.tiles[0] * a.tiles[1] * a.tiles[2] * (a.pg_inner ? a.pg_split : a.pgroups) *
           a.oc_blocks;
}

int cu_count() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, v = 0;
        cus = hipGetDevice(&dev) == hipSuccess &&
                      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
                  ? v
                  : 256;
    }
    return cus;
}

bool build_any(const Geom& g, GArgs& a, bool& small) {
    const int kvol = g.k[0] * g.k[1] * g.k[2];
    small = kvol <= 27;
    return small ? build_gargs<8, 27>(g, a) : build_gargs<4, 64>(g, a);
}

// 1: kernel 3, stride 2, padding 1 in every dim; 2: kernel 4, stride 2,
// padding 1 in every dim (dilation 1 both); 0: other geometries
int fixed_kind(const Geom& g) {
    for (int k : {3, 4}) {
        bool all = true;
        for (int j = 0; j < 3; ++j) all = all && g.k[j] == k && g.s[j] == 2 && g.p[j] == 1 && g.d[j] == 1;
        if (all) return k == 3 ? 1 : 2;
    }
    return 0;
}

}  // namespace

bool convT_phasegroup_supported(const Geom& g) {
    if (g.cin_g < 4 || g.cout_g < 8) return false;
    GArgs a;
    bool small;
    return build_any(g, a, small) && grid_blocks(g, a) <= 0x7fffffff;
}

hipError_t launch_convT_phasegroup(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                                   hipStream_t st) {
    if (!convT_phasegroup_supported(g)) return hipErrorNotSupported;
    GArgs a;
    bool small;
    build_any(g, a, small);
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    if (a.pg_inner) {
        // enough workgroups for one per CU, each taking a run of phase groups
        const int64_t base = g.N * (int64_t)g.groups * a.tiles[0] * a.tiles[1] * a.tiles[2] * a.oc_blocks;
        const int64_t want = ceil_div(cu_count(), base);
        const int split = (int)(want < a.pgroups ? want : a.pgroups);
        a.pg_per = (int32_t)ceil_div(a.pgroups, split);
        a.pg_split = (int32_t)ceil_div(a.pgroups, a.pg_per);
    }
    // the 8- and 16-byte stores need y aligned to their size
    if ((a.vecs == 2 && ((uintptr_t)y & 7) != 0) || (a.vecs == 4 && ((uintptr_t)y & 15) != 0)) a.vecs = 0;
    a.one_tap_db = a.one_tap && a.vecs == a.P && g.cout_g % kOCB == 0 &&
                   (int64_t)kOCB * g.O[0] * g.O[1] * g.O[2] * 4 < ((int64_t)1 << 31);
    static_assert(sizeof(GArgs) <= 4096, "kernel arguments");
    const unsigned blocks = (unsigned)grid_blocks(g, a);
    const int fk = fixed_kind(g);
    if (fk == 1)
        hipLaunchKernelGGL((convT_phasegroup_kernel<8, 27, 1>), dim3(blocks), dim3(kThreads), 0, st, a);
    else if (fk == 2)
        hipLaunchKernelGGL((convT_phasegroup_kernel<4, 64, 2>), dim3(blocks), dim3(kThreads), 0, st, a);
    else if (small)
        hipLaunchKernelGGL((convT_phasegroup_kernel<8, 27, 0>), dim3(blocks), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((convT_phasegroup_kernel<4, 64, 0>), dim3(blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace c3d
