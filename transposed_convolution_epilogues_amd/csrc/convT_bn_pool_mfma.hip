// convT_bn_pool_mfma.hip - phase 1 of convT_bn_avgpool for the page's
// transposed conv (kernel 3, stride 2, padding 1, dilation 1) with pool 4, on
// the matrix cores ("Kimi-K2.6 l2_p72": the module and its parity tables).
//
// Output phases.  An output o takes tap k from input i = (o + 1 - k) / 2, so
// per dim an even o (residue r = 0) has the single tap k = 1 and an odd o
// (r = 1) the taps k = 0 and 2.  The 8 residue classes (r0, r1, r2) are
// therefore 8 dense convolutions with 1, 2, 4 or 8 taps, i.e. GEMMs
//     out[voxel][oc] = sum over (ic, tap) of x[ic][i(voxel, tap)] * W[ic][oc][tap]
// with K = Cin * taps.  Each runs on v_mfma_f32_16x16x4f32: 16 voxels x 16
// output channels, K in steps of 4 (padded with zero weights).
//
// A 4x4x4 output cell holds 8 voxels of each class: o = 4c + r + 2e, e in
// {0, 1} per dim, all reading inputs 2c + {0, 1, 2} per dim (the page's
// window argument).  A workgroup owns a box of 4 x 8 x 8 cells and stages the
// 9 x 17 x 17 inputs per channel they read in LDS; wave w takes the cell
// plane c0 = box + w.  A 16-voxel M tile is two neighbouring cells x the 8
// voxels of one class, so for every class a lane's four accumulators hold
// voxels of the same cell: the lane sums the cell's pooling window across the
// 8 classes in one register, and adds the window halves of lanes l and l ^ 16
// at the end.  Per voxel the lane also accumulates the square for the batch
// variance (float per tile, float64 across tiles).  Positions past the output
// (the tail of the last cell per dim) are masked out of both; the conv bias is
// left out, as it cancels from batch-statistics BN.
//
// The workgroup writes the pooled pre-normalisation means (or, in eval mode,
// the final outputs) and one float64 (sum, sum of squares) pair per channel,
// which phase 2 merges.
#include <type_traits>

#include "c3d_internal.h"

namespace c3d {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int B0 = 4, B1 = 8, B2 = 8;                             // cells per workgroup box
constexpr int R0 = 2 * B0 + 1, R1 = 2 * B1 + 1, R2 = 2 * B2 + 1;  // staged inputs per dim
constexpr int kRegion = R0 * R1 * R2;                             // staged floats per input channel
constexpr int kTiles = B1 * B2 / 2;                               // M tiles per wave and class (two cells each)
constexpr int kCout = 16;                                         // output channels: one N tile

__host__ __device__ constexpr int class_taps(int cls) {
    return ((cls >> 2) & 1 ? 2 : 1) * ((cls >> 1) & 1 ? 2 : 1) * (cls & 1 ? 2 : 1);
}
template <int CIN>
__host__ __device__ constexpr int class_steps(int cls) {
    return (CIN * class_taps(cls) + 3) / 4;
}
template <int CIN>
__host__ __device__ constexpr int max_steps() {
    int m = 0;
    for (int c = 0; c < 8; ++c) m = class_steps<CIN>(c) > m ? class_steps<CIN>(c) : m;
    return m;
}
template <int CIN>
__host__ __device__ constexpr int first_step(int cls) {
    int s = 0;
    for (int c = 0; c < cls; ++c) s += class_steps<CIN>(c);
    return s;
}
template <int CIN>
__host__ __device__ constexpr int total_steps() {
    int s = 0;
    for (int c = 0; c < 8; ++c) s += class_steps<CIN>(c);
    return s;
}

// lanes l and l ^ 16 exchange a value (ds_swizzle in bit-mask mode: no lane
// arithmetic, unlike a generic shuffle)
__device__ __forceinline__ float swizzle_xor16(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// The staged input box: every input channel, dim-0 row a and dim-1 row b.
// load() issues the global loads into registers, store() writes them to LDS
// with the zero padding.  VEC (S2 % 4 == 0, x 16-byte aligned): a staged row
// of R2 = 17 inputs from j2, a multiple of 16, is five aligned 16-byte
// chunks, of which the last contributes its first element; with S2 % 4 == 0
// a chunk lies wholly inside or wholly outside the row.
template <int CIN, bool VEC>
struct StageBox {
    static constexpr int B = 0;
    static constexpr int NB = R1;
    static constexpr int kW = VEC ? (R2 + 3) / 4 : R2;  // items per staged row
    static constexpr int kItems = CIN * R0 * NB * kW;
    static constexpr int kIter = (kItems + kThreads - 1) / kThreads;
    static_assert(kIter <= 64, "one mask bit per staging load");
    typedef typename std::conditional<VEC, f32x4, float>::type V;
    V v[kIter];
    uint64_t inside = 0;

    __device__ __forceinline__ void load(const float* xn, int S0, int S1, int S2, int j0, int j1, int j2) {
#pragma unroll
        for (int q = 0; q < kIter; ++q) {
            const int e = q * kThreads + (int)threadIdx.x;
            const int ec = e < kItems ? e : kItems - 1;
            const int row = ec / kW, c = ec - row * kW;
            const int ic = row / (R0 * NB), r = row - ic * (R0 * NB);
            const int a = r / NB, b = B + (r - a * NB);
            const int i0 = j0 + a, i1 = j1 + b, i2 = j2 + (VEC ? 4 * c : c);
            inside |= (uint64_t)(i0 < S0 && i1 < S1 && i2 < S2) << q;
            const int k0 = i0 < S0 ? i0 : S0 - 1, k1 = i1 < S1 ? i1 : S1 - 1;
            const int k2 = i2 < S2 ? i2 : S2 - (VEC ? 4 : 1);
            const float* src = xn + (int64_t)ic * S0 * S1 * S2 + (k0 * S1 + k1) * S2 + k2;
            if constexpr (VEC) v[q] = *reinterpret_cast<const f32x4*>(src);
            else v[q] = *src;
        }
    }
    __device__ __forceinline__ void store(float* xs) const {
#pragma unroll
        for (int q = 0; q < kIter; ++q) {
            const int e = q * kThreads + (int)threadIdx.x;
            if (e < kItems) {
                const int row = e / kW, c = e - row * kW;
                const int ic = row / (R0 * NB), r = row - ic * (R0 * NB);
                const int a = r / NB, b = B + (r - a * NB);
                const bool ok = (inside >> q) & 1;
                if constexpr (VEC) {
                    float* dst = xs + ((ic * R0 + a) * R1 + b) * R2 + 4 * c;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (4 * c + u < R2) dst[u] = ok ? v[q][u] : 0.f;
                } else {
                    xs[((ic * R0 + a) * R1 + b) * R2 + c] = ok ? v[q] : 0.f;
                }
            }
        }
    }
};

// VEC: S2 % 4 == 0 and x 16-byte aligned, so the input box is staged with
// 16-byte loads
template <int CIN, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(CIN == 4 ? 3 : 4, 4))) void convT_bn_pool_mfma_kernel(
    const float* __restrict__ x, const float* __restrict__ w, float* __restrict__ y, double* __restrict__ ws,
    PoolGeom pg, int32_t nb1, int32_t nb2, int64_t boxes_per_sample, BnEval ev) {
    __shared__ float xs[CIN * kRegion];
    __shared__ double red[kThreads / 64][kCout][2];
    const Geom& g = pg.g;
    // XCD-aware box order: consecutive workgroup ids go round-robin to the 8
    // XCDs; remapped, each XCD takes a contiguous run of boxes, whose input
    // halos overlap in its L2 (about 1 % on the x[64,3,32,32,32] module)
    int64_t bid = blockIdx.x;
    if ((gridDim.x & 7) == 0) bid = (bid & 7) * (int64_t)(gridDim.x >> 3) + (bid >> 3);
    const int64_t n = bid / boxes_per_sample;
    const int64_t bx = bid % boxes_per_sample;
    const int64_t cb2 = (bx % nb2) * B2;
    const int64_t cb1 = ((bx / nb2) % nb1) * B1;
    const int64_t cb0 = (bx / ((int64_t)nb2 * nb1)) * B0;

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int m = lane & 15;   // A row (voxel) of this lane, and its B / D column (output channel)
    const int kq = lane >> 4;  // K quarter of this lane's A and B elements; D rows 4 kq .. 4 kq + 3
    const int oc = m;
    const bool oc_ok = oc < g.Cout;
    // A row m: cell m / 8 of the tile, window offsets e = (m / 4 % 2, m / 2 % 2, m % 2)
    const int am_cell = m >> 3, ae0 = (m >> 2) & 1, ae1 = (m >> 1) & 1, ae2 = m & 1;

    // per class and K step: this lane's A offset in xs (tile 0) and B weight
    // (loaded before the input box, so that the two sets of loads overlap)
    int aoff[total_steps<CIN>()];
    float bw[total_steps<CIN>()];
    {
        int q = 0;
#pragma unroll
        for (int cls = 0; cls < 8; ++cls) {
            const int r0 = (cls >> 2) & 1, r1 = (cls >> 1) & 1, r2 = cls & 1;
            const int n1 = r1 ? 2 : 1, n2 = r2 ? 2 : 1;
            const int taps = class_taps(cls);
#pragma unroll
            for (int s = 0; s < class_steps<CIN>(cls); ++s, ++q) {
                const int k = 4 * s + kq;
                const bool kv = k < CIN * taps;
                const int kk = kv ? k : 0;
                const int ic = kk / taps, t = kk % taps;
                const int t0 = t / (n1 * n2), t1 = (t / n2) % n1, t2 = t % n2;
                // tap per dim: 1 for r = 0, 0 or 2 for r = 1; input offset (r + 2e + 1 - tap) / 2
                const int k0 = r0 ? 2 * t0 : 1, k1 = r1 ? 2 * t1 : 1, k2 = r2 ? 2 * t2 : 1;
                const int d0 = (r0 + 2 * ae0 + 1 - k0) >> 1, d1 = (r1 + 2 * ae1 + 1 - k1) >> 1,
                          d2 = (r2 + 2 * ae2 + 1 - k2) >> 1;
                aoff[q] = ((ic * R0 + 2 * wv + d0) * R1 + d1) * R2 + 2 * am_cell + d2;
                // unconditional load (channel clamped into w), zero selected after it
                const int ocl = oc_ok ? oc : 0;
                bw[q] = w[((ic * g.Cout + ocl) * 3 + k0) * 9 + k1 * 3 + k2];
                bw[q] = (kv && oc_ok) ? bw[q] : 0.f;
            }
        }
    }
    // Stage inputs 2 cb + [0, R) per dim of every input channel, zero outside
    // x.  The loads are unconditional, from addresses clamped into x, and the
    // zero padding is applied when the registers are written to LDS: a
    // conditional load would be a branch, and the compiler waits for every
    // earlier load before one (their destination registers get reused), which
    // serialises the staging.  All of a thread's loads are issued before its
    // first LDS write, so their latencies overlap.  (Staging the box in two
    // parts, so that the first tile rows start before the rest arrives, needs
    // the second part's registers during those rows: 129 VGPRs for 3 input
    // channels, past the 128 that four waves per SIMD allow.)
    const int S0 = (int)g.S[0], S1 = (int)g.S[1], S2 = (int)g.S[2];
    const float* xn = x + n * CIN * (int64_t)S0 * S1 * S2;
    StageBox<CIN, VEC> box;
    box.load(xn, S0, S1, S2, 2 * (int)cb0, 2 * (int)cb1, 2 * (int)cb2);
    box.store(xs);
    __syncthreads();  // input box staged

    const int64_t c0 = cb0 + wv;                        // this wave's cell plane
    const int dcell = kq >> 1, de0 = kq & 1;            // D rows: cell kq / 2 of the tile, e0 = kq % 2
    const bool eval = ev.gamma != nullptr;               // workgroup-uniform
    float sc = 1.f / 64.f, sh = 0.f;
    if (eval && oc_ok) {
        bn_eval_affine(ev, oc, sc, sh);
        sc *= 1.f / 64.f;
    }
    double st = 0.0, sq = 0.0;
    const bool plane_ok = c0 < pg.C[0];  // wave-uniform
    // 32-bit cell coordinates (the supported shapes keep every output index below 2^31)
    const int C1 = (int)pg.C[1], C2 = (int)pg.C[2], P1 = (int)pg.P[1], P2 = (int)pg.P[2];
    const int lim0 = (int)(g.O[0] - 4 * c0);  // o0 - 4 c0 of this plane's outputs stays below lim0
    const int b1 = (int)cb1, b2 = (int)cb2 + dcell;
    const bool row_ok = oc_ok && c0 < pg.P[0];
    float* yl = y + ((n * g.Cout + oc) * pg.P[0] + c0) * (int64_t)P1 * P2;  // this lane's pooled plane

    // Tile rows [jr0, jr1) of the box, starting at row 0.  The tiles of a
    // row share one A offset per K step, which each row
    // advances in place (aoff holds the current row's offsets), and the
    // row's four tiles read at this offset plus an immediate.  A loop over
    // the rows (not unrolled) keeps the kernel small for the instruction
    // cache.
    auto rows = [&](int jr0, int jr1) __attribute__((always_inline)) {
#pragma unroll 1
        for (int jr = jr0; jr < jr1; ++jr) {
            const int c1 = b1 + jr;
            if (c1 >= C1) break;  // wave-uniform: the rows below (and their offsets) are not needed
            const int lim1 = (int)g.O[1] - 4 * c1;
            float stf = 0.f, sqf = 0.f;  // the row's sums, in float over its four tiles
#pragma unroll
            for (int jc = 0; jc < 4; ++jc) {
                const int c2a = (int)cb2 + 2 * jc;  // first cell of the tile
                if (c2a >= C2) break;               // wave-uniform: the tile lies past the output
                const int c2 = b2 + 2 * jc;         // this lane's D cell
                const float* xt = xs + 4 * jc;
                // the 8 classes are independent accumulation chains
                f32x4 acc[8];
                {
                    int q = 0;
#pragma unroll
                    for (int cls = 0; cls < 8; ++cls) {
                        acc[cls] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < class_steps<CIN>(cls); ++s, ++q)
                            acc[cls] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[aoff[q]], bw[q], acc[cls], 0, 0, 0);
                    }
                }
                // two partial sums each, to halve the dependent chains
                float win[2] = {0.f, 0.f}, s2[2] = {0.f, 0.f};
                const int lim2 = (int)g.O[2] - 4 * c2;
                // every voxel of the tile is inside the output (wave-uniform)
                if (lim0 >= 4 && lim1 >= 4 && (int)g.O[2] - 4 * (c2a + 1) >= 4) {
#pragma unroll
                    for (int cls = 0; cls < 8; ++cls)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            win[i & 1] += acc[cls][i];
                            s2[i & 1] = fmaf(acc[cls][i], acc[cls][i], s2[i & 1]);
                        }
                } else {
#pragma unroll
                    for (int cls = 0; cls < 8; ++cls) {
                        const int r0 = (cls >> 2) & 1, r1 = (cls >> 1) & 1, r2 = cls & 1;
                        const bool in0 = r0 + 2 * de0 < lim0;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bool in = in0 && r1 + 2 * (i >> 1) < lim1 && r2 + 2 * (i & 1) < lim2;
                            const float v = in ? acc[cls][i] : 0.f;
                            win[i & 1] += v;
                            s2[i & 1] = fmaf(v, v, s2[i & 1]);
                        }
                    }
                }
                sqf += s2[0] + s2[1];
                float wsum = win[0] + win[1];
                wsum += swizzle_xor16(wsum);  // the other half (e0) of the cell's window
                if (de0 == 0) {
                    stf += wsum;
                    if (row_ok && c1 < P1 && c2 < P2) yl[c1 * P2 + c2] = fmaf(wsum, sc, sh);
                }
            }
            st += (double)stf;
            sq += (double)sqf;
#pragma unroll
            for (int q = 0; q < total_steps<CIN>(); ++q) aoff[q] += 2 * R2;  // next tile row
        }
    };
    if (plane_ok) rows(0, B1);
    if (eval) return;  // workgroup-uniform; no barrier follows in eval mode

    // per channel: lanes m, m + 16, m + 32, m + 48 hold its partials
    st += __shfl_xor(st, 16, 64);
    st += __shfl_xor(st, 32, 64);
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    if (kq == 0) {
        red[wv][m][0] = st;
        red[wv][m][1] = sq;
    }
    __syncthreads();
    if (threadIdx.x < 2 * g.Cout) {
        const int c = threadIdx.x >> 1, k = threadIdx.x & 1;
        double v = 0.0;
#pragma unroll
        for (int i = 0; i < kThreads / 64; ++i) v += red[i][c][k];
        const int64_t parts = g.N * boxes_per_sample;
        ws[2 * ((int64_t)c * parts + n * boxes_per_sample + bx) + k] = v;
    }
}

void box_counts(const PoolGeom& pg, int64_t& nb0, int64_t& nb1, int64_t& nb2) {
    nb0 = ceil_div(pg.C[0], B0);
    nb1 = ceil_div(pg.C[1], B1);
    nb2 = ceil_div(pg.C[2], B2);
}

}  // namespace

bool convT_bn_pool_mfma_supported(const PoolGeom& pg, const void*) {
    const Geom& g = pg.g;
    for (int j = 0; j < 3; ++j)
        if (g.k[j] != 3 || g.s[j] != 2 || g.p[j] != 1 || g.d[j] != 1 || g.O[j] != 2 * g.S[j] - 1) return false;
    // one input channel's plane is indexed in 32 bits
    return g.groups == 1 && pg.pool == 4 && g.Cin >= 1 && g.Cin <= 4 && g.Cout <= kCout &&
           g.S[0] * g.S[1] * g.S[2] < (1ll << 31);
}

size_t convT_bn_pool_mfma_partials(const PoolGeom& pg) {
    int64_t nb0, nb1, nb2;
    box_counts(pg, nb0, nb1, nb2);
    return (size_t)(pg.g.N * nb0 * nb1 * nb2);
}

hipError_t launch_convT_bn_pool_phase1_mfma(const float* x, const float* w, float* y, double* ws,
                                            const PoolGeom& pg, const BnEval& ev, hipStream_t st) {
    int64_t nb0, nb1, nb2;
    box_counts(pg, nb0, nb1, nb2);
    const int64_t bps = nb0 * nb1 * nb2;
    const int64_t blocks = pg.g.N * bps;
    if (blocks > 0x7fffffff || nb1 > 0x7fffffff || nb2 > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kThreads);
    const int32_t b1 = (int32_t)nb1, b2 = (int32_t)nb2;
    const bool vec = pg.g.S[2] % 4 == 0 && ((uintptr_t)x & 15u) == 0;
    if (vec) {
        switch (pg.g.Cin) {
            case 1: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<1, true>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
            case 2: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<2, true>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
            case 3: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<3, true>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
            default: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<4, true>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
        }
    } else {
        switch (pg.g.Cin) {
            case 1: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<1, false>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
            case 2: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<2, false>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
            case 3: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<3, false>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
            default: hipLaunchKernelGGL((convT_bn_pool_mfma_kernel<4, false>), grid, block, 0, st, x, w, y, ws, pg, b1, b2, bps, ev); break;
        }
    }
    return hipGetLastError();
}

}  // namespace c3d
