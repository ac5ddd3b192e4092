// convT_bn_swap.hip - the ConvTranspose3d(k3, s2, p1) -> BatchNorm3d (batch
// statistics) -> AvgPool3d(4) module with its sums swapped ("Kimi-K2.6
// l2_p72": the proposal to swap the order of the pooled sum and the conv sum).
// No transposed-conv output is formed one by one.
//
// Notation: per dim, output o = 2q + r (r = o mod 2, the residue class).
// Residue 0 takes tap k = 1 from input q; residue 1 takes k = 0 from q + 1
// and k = 2 from q (the page's parity tables).  So on class r,
// t_r(q) = sum over its taps a of w_a x_{c_a}(q + delta_a), delta in {0,1}^3,
// t = conv_transpose3d(x, w) without the bias.
//
// 1. Pooled sums.  The window [4j, 4j + 4) of a dim reads inputs 2j + a,
//    a = 0, 1, 2, through taps {1, 2}, {0, 1, 2}, {0}, so the window sum is a
//    stride-2 correlation of x with the 3x3x3 summed-weight kernel Wp: 81
//    MACs per (window, channel) for 3 input channels, a [windows x 81] x
//    [81 x Cout] product on the matrix cores (swap_pool_kernel).
// 2. Statistics over the extended box E = [-1, S-1]^3 of every class (x read
//    as zero outside the input).  E + delta covers the whole input for
//    delta in {0,1}, so
//      sum_E t_r   = sum_a w_a X_{c_a}                      (X_c = sum of channel c)
//      sum_E t_r^2 = sum_{a,b} w_a w_b L_{c_a c_b}(delta_b - delta_a)
//    with L_{cc'}(D) = sum_u x_c(u) x_c'(u + D) the lag correlation over the
//    natural range.  Lag 0 (pairs c <= c'), the 13 lags of a half-space and
//    the channel sums are 126 values for 3 channels (stats_block, on the
//    vector ALUs).
// 3. E holds more than the real outputs of class r: a coordinate at -1, or
//    at S - 1 in a residue-1 dim, is outside the transposed conv.  Split E by
//    type tau in {L, M, H}^3 (q_i = -1, 0 <= q_i <= S_i - 2, q_i = S_i - 1).
//    On a type, x(q + delta) is zero unless delta_i = 1 where tau_i = L and
//    delta_i = 0 where tau_i = H, so t_r is a product with the type's patch
//    vector v(q) (3 channels x 2^(number of M dims) entries).  The Gram
//    matrix Q_tau = sum v v^T (with a constant entry 1 appended, giving the
//    sums and the count) over the 26 boundary types is one 16x16 matrix-core
//    product per type and block of positions (shell_block, run as extra
//    workgroups of swap_stats_shell_kernel when a sample's faces fit in its
//    LDS, else swap_shell_global_kernel); the
//    outputs outside the conv are those of the types with an L only in
//    residue-1 dims and an L or H in at least one of them, and their sums
//    are w_r^T Q_tau w_r.
// 4. swap_reduce_kernel merges the partials in a fixed order;
//    swap_contract_kernel contracts them with the weights into per-channel (sum, sum of squares), and turns
//    them into the batch statistics and the normalisation, which the pooled
//    kernel applies to its sums before the single store of y.
//
// Eval mode runs the pooled kernel alone with the running statistics.
#include "c3d_internal.h"

namespace c3d {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxCin = 3;
constexpr int kMaxCout = 32;
constexpr int kFwd = 13;   // lags of the half-space d0 > 0, or d0 = 0 and (d1 > 0, or d1 = 0 and d2 > 0)
constexpr int kTypes = 26;  // boundary types of {L, M, H}^3 (all but M M M)

__host__ __device__ constexpr int n_stat(int C) { return C + C * (C + 1) / 2 + kFwd * C * C; }
constexpr int kStatRow = 128;  // floats per statistics partial (126 used for 3 channels)

// forward lag index: (0,0,1) -> 0; (0,1,d2) -> 1 + d2 + 1; (1,d1,d2) -> 4 + 3 (d1 + 1) + d2 + 1
__host__ __device__ constexpr int fwd_index(int d0, int d1, int d2) {
    return d0 == 1 ? 4 + 3 * (d1 + 1) + (d2 + 1) : (d1 == 1 ? 1 + (d2 + 1) : 0);
}

// type t in [0, 26) -> (tau0, tau1, tau2), each 0 = L, 1 = M, 2 = H (M M M skipped)
__host__ __device__ inline void type_of(int t, int tau[3]) {
    const int c = t < 13 ? t : t + 1;
    tau[0] = c / 9;
    tau[1] = (c / 3) % 3;
    tau[2] = c % 3;
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Transposing reduction of NA per-lane values over the wave.  A step on lane
// bit b pairs register i with i + H: the lane whose bit b is clear keeps the
// first, its partner the second, and each adds what the partner sends, so
// after the step register i of lane L holds value i + H * bit_b(L) summed
// over the pair.  Bits 5 and 4 use the lane-swap instructions; bit 3 uses
// the 16-lane mirror and bit 2 the 8-lane mirror (both also flip the lower
// bits, which are still unused at that point); bits 1 and 0 use quad
// permutations.  With NA = 128 lane L ends with values 2L and 2L + 1, with
// NA = 64 with value L, with NA = 16 with value L >> 2 (after two plain
// steps over bits 1 and 0).
template <int H>
__device__ __forceinline__ void tstep_swap32(float* v) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + H]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}
template <int H>
__device__ __forceinline__ void tstep_swap16(float* v) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + H]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}
template <int H, int kCtrl>
__device__ __forceinline__ void tstep_dpp(float* v, bool hi) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const float keep = hi ? v[i + H] : v[i];
        const float send = hi ? v[i] : v[i + H];
        v[i] = keep + dpp<kCtrl>(send);
    }
}

// reduces v[0, NA) over the wave and writes the NA totals to out[0, NA)
template <int NA>
__device__ __forceinline__ void wave_reduce_to(float* v, float* out, int lane) {
    static_assert(NA == 16 || NA == 64 || NA == 128, "reduction width");
    if constexpr (NA == 128) {
        tstep_swap32<64>(v);
        tstep_swap16<32>(v);
        tstep_dpp<16, 0x140>(v, (lane >> 3) & 1);
        tstep_dpp<8, 0x141>(v, (lane >> 2) & 1);
        tstep_dpp<4, 0x4E>(v, (lane >> 1) & 1);
        tstep_dpp<2, 0xB1>(v, lane & 1);
        out[2 * lane] = v[0];
        out[2 * lane + 1] = v[1];
    } else if constexpr (NA == 64) {
        tstep_swap32<32>(v);
        tstep_swap16<16>(v);
        tstep_dpp<8, 0x140>(v, (lane >> 3) & 1);
        tstep_dpp<4, 0x141>(v, (lane >> 2) & 1);
        tstep_dpp<2, 0x4E>(v, (lane >> 1) & 1);
        tstep_dpp<1, 0xB1>(v, lane & 1);
        out[lane] = v[0];
    } else {
        tstep_swap32<8>(v);
        tstep_swap16<4>(v);
        tstep_dpp<2, 0x140>(v, (lane >> 3) & 1);
        tstep_dpp<1, 0x141>(v, (lane >> 2) & 1);
        float s = v[0];
        s += dpp<0x4E>(s);
        s += dpp<0xB1>(s);
        if ((lane & 3) == 0) out[lane >> 2] = s;
    }
}

template <int C>
constexpr int reduce_width() {
    return n_stat(C) > 64 ? 128 : (n_stat(C) > 16 ? 64 : 16);
}

// The statistics workgroup has two waves per (column, row group): the first
// half of the waves takes the channel sums, lag 0 and the forward lags 0..5
// ((0,0,1), (0,1,*), (1,-1,-1), (1,-1,0)), the second half the lags 6..12
// ((1,-1,1), (1,0,*), (1,1,*)).  Each keeps 63 accumulators for 3 channels
// instead of 126, so four waves fit a SIMD instead of two.
constexpr int kStatThreads = 512;
constexpr int kLagSplit = 6;
template <int C>
constexpr int half_a() { return C + C * (C + 1) / 2 + kLagSplit * C * C; }  // statistics of the first half
template <int C>
constexpr int half_width() {
    return (half_a<C>() > n_stat(C) - half_a<C>() ? half_a<C>() : n_stat(C) - half_a<C>()) > 16 ? 64 : 16;
}

// ------------------------------------------------------------ statistics
// A workgroup takes kSlab planes of one sample and one 32 x 32 tile of the
// (p1, p2) plane.  Planes go through a ring of three LDS slots: plane p and
// p + 1 are read while plane p + 2 is fetched.  A slot holds the tile with a
// one-element halo (rows -1 .. 32, columns -1 .. 32, zero outside the input).
// Lane l of wave w owns column l % 32 and rows 4g .. 4g + 3 of the tile,
// g = 2w + l / 32, and walks them with a register window: row r of plane
// p + 1 (lags (1, d1, d2)) is reused for three rows, row r + 1 of plane p
// (lags (0, 1, d2)) becomes the next row's own values.
constexpr int kTile = 32;
constexpr int kSlab = 4;
constexpr int kRS = 40;                // row stride: columns -1 .. 32 at 3 .. 36 (16-byte aligned interior)
constexpr int kRows = kTile + 2;       // rows -1 .. 32
constexpr int kChS = kRows * kRS;      // floats per channel in a slot

struct StatArgs {
    const float* x;
    float* part;        // [blocks][kStatRow]
    int32_t S[3];
    int32_t T1, T2;     // tiles per plane
    int32_t slabs;
    int32_t blocks;
};

// 16-byte units of a plane's tile (channel, row, quarter-row) per thread
template <int CIN>
constexpr int fetch_units() { return (CIN * 256 + kStatThreads - 1) / kStatThreads; }

template <int CIN>
__device__ __forceinline__ void fast_fetch(const float* xn, int p, int S0, float4 (&r)[fetch_units<CIN>()]) {
    const int pc = p < S0 ? p : S0 - 1;  // clamped plane, selected below
#pragma unroll
    for (int u = 0; u < fetch_units<CIN>(); ++u) {
        int f = u * kStatThreads + threadIdx.x;
        f = f < CIN * 256 ? f : 0;  // no unit: a valid address, not stored
        const int c = f >> 8, row = (f >> 3) & 31, q = f & 7;
        const float4 v = *reinterpret_cast<const float4*>(xn + ((int64_t)c * S0 + pc) * (kTile * kTile) + row * kTile + 4 * q);
        r[u] = p < S0 ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int CIN>
__device__ __forceinline__ void fast_put(float* slot, const float4 (&r)[fetch_units<CIN>()]) {
#pragma unroll
    for (int u = 0; u < fetch_units<CIN>(); ++u) {
        const int f = u * kStatThreads + threadIdx.x;
        if (f >= CIN * 256) continue;
        const int c = f >> 8, row = (f >> 3) & 31, q = f & 7;
        *reinterpret_cast<float4*>(slot + c * kChS + (row + 1) * kRS + 4 + 4 * q) = r[u];
    }
}

// any shape: the whole halo box, sixteen independent loads per thread at a
// time, zero outside the input
template <int CIN>
__device__ void box_stage(const float* xn, int p, const StatArgs& a, int r0, int c0, float* slot) {
    const int S0 = a.S[0], S1 = a.S[1], S2 = a.S[2];
    constexpr int kBox = kRows * (kTile + 2);
    for (int e0 = 0; e0 < CIN * kBox; e0 += 16 * kStatThreads) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int e = e0 + u * kStatThreads + threadIdx.x;
            const int c = e / kBox, rem = e % kBox;
            const int row = rem / (kTile + 2), col = rem % (kTile + 2);
            const int p1 = r0 + row, p2 = c0 + col;
            const bool in = e < CIN * kBox && p < S0 && p1 >= 0 && p1 < S1 && p2 >= 0 && p2 < S2;
            const float x = xn[in ? (((int64_t)c * S0 + p) * S1 + p1) * S2 + p2 : 0];
            v[u] = in ? x : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int e = e0 + u * kStatThreads + threadIdx.x;
            if (e < CIN * kBox) {
                const int c = e / kBox, rem = e % kBox;
                slot[c * kChS + (rem / (kTile + 2)) * kRS + 3 + rem % (kTile + 2)] = v[u];
            }
        }
    }
}

// Products of 4 rows of one column: A at plane p, B at plane p + 1, both at
// the lane's first row (tile row r = 4g) and column.  Statistic index:
// channel sums c; lag 0 pairs c <= c' next; forward lag L of pair (c, c') at
// F + (L C + c) C + c'.
// First half (63 for 3 channels): sums, lag 0, lags (0,0,1), (0,1,d2), (1,-1,-1),
// (1,-1,0).  Register window: row r of plane p at columns 0 and 1, row r + 1
// of plane p (which becomes the next row's own values), row r - 1 of plane
// p + 1 at columns -1 and 0.
template <int CIN>
__device__ __forceinline__ void stat_rows_a(const float* A, const float* B, float* acc) {
    constexpr int C = CIN;
    constexpr int F = C + C * (C + 1) / 2;
    float a0[C], a1[C];  // plane p: row r, columns 0 and 1
    float an[3][C];      // plane p: row r + 1, columns -1, 0, 1
    float bm[2][C];      // plane p + 1: row r - 1, columns -1, 0
#pragma unroll
    for (int c = 0; c < C; ++c) {
        a0[c] = A[c * kChS];
        a1[c] = A[c * kChS + 1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
            for (int dc = 0; dc < 3; ++dc) an[dc][c] = A[c * kChS + (i + 1) * kRS + dc - 1];
#pragma unroll
            for (int dc = 0; dc < 2; ++dc) bm[dc][c] = B[c * kChS + (i - 1) * kRS + dc - 1];
        }
        int l0 = C;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            acc[c] += a0[c];
#pragma unroll
            for (int cp = c; cp < C; ++cp) acc[l0 + cp - c] = fmaf(a0[c], a0[cp], acc[l0 + cp - c]);
            l0 += C - c;
#pragma unroll
            for (int cp = 0; cp < C; ++cp) {
                acc[F + (0 * C + c) * C + cp] = fmaf(a0[c], a1[cp], acc[F + (0 * C + c) * C + cp]);
#pragma unroll
                for (int dc = 0; dc < 3; ++dc)
                    acc[F + ((1 + dc) * C + c) * C + cp] = fmaf(a0[c], an[dc][cp], acc[F + ((1 + dc) * C + c) * C + cp]);
#pragma unroll
                for (int dc = 0; dc < 2; ++dc)
                    acc[F + ((4 + dc) * C + c) * C + cp] = fmaf(a0[c], bm[dc][cp], acc[F + ((4 + dc) * C + c) * C + cp]);
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            a0[c] = an[1][c];
            a1[c] = an[2][c];
        }
    }
}

// Second half (63 for 3 channels): lags (1,-1,1), (1,0,d2), (1,1,d2), indexed
// from half_a.  Register window: row r - 1 of plane p + 1 at column 1, rows r
// and r + 1 at columns -1, 0, 1 (row r + 1 becomes the next row's r).
template <int CIN>
__device__ __forceinline__ void stat_rows_b(const float* A, const float* B, float* acc) {
    constexpr int C = CIN;
    constexpr int F = C + C * (C + 1) / 2;
    constexpr int H0 = half_a<C>();
    float a0[C];         // plane p: row r, column 0
    float bp[C];         // plane p + 1: row r - 1, column 1
    float b0[3][C];      // plane p + 1: row r
    float b1[3][C];      // plane p + 1: row r + 1
#pragma unroll
    for (int c = 0; c < C; ++c) {
        bp[c] = B[c * kChS - kRS + 1];
#pragma unroll
        for (int dc = 0; dc < 3; ++dc) b0[dc][c] = B[c * kChS + dc - 1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            a0[c] = A[c * kChS + i * kRS];
#pragma unroll
            for (int dc = 0; dc < 3; ++dc) b1[dc][c] = B[c * kChS + (i + 1) * kRS + dc - 1];
        }
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int cp = 0; cp < C; ++cp) {
                acc[F + (6 * C + c) * C + cp - H0] = fmaf(a0[c], bp[cp], acc[F + (6 * C + c) * C + cp - H0]);
#pragma unroll
                for (int dc = 0; dc < 3; ++dc) {
                    acc[F + ((7 + dc) * C + c) * C + cp - H0] =
                        fmaf(a0[c], b0[dc][cp], acc[F + ((7 + dc) * C + c) * C + cp - H0]);
                    acc[F + ((10 + dc) * C + c) * C + cp - H0] =
                        fmaf(a0[c], b1[dc][cp], acc[F + ((10 + dc) * C + c) * C + cp - H0]);
                }
            }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            bp[c] = b0[2][c];
#pragma unroll
            for (int dc = 0; dc < 3; ++dc) b0[dc][c] = b1[dc][c];
        }
    }
}

template <int CIN, bool FAST>
__device__ __forceinline__ void stats_block(const StatArgs& a, float* lds, int blk) {
    constexpr int NS = n_stat(CIN);
    constexpr int NA = half_width<CIN>();
    constexpr int HA = half_a<CIN>();
    constexpr int kSlot = CIN * kChS;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool second = wv >= kStatThreads / 128;  // wave-uniform: which half of the statistics
    int b = blk;
    if ((a.blocks & 7) == 0) b = (b & 7) * (a.blocks >> 3) + (b >> 3);  // neighbouring slabs on one XCD
    const int t2 = b % a.T2;
    b /= a.T2;
    const int t1 = b % a.T1;
    b /= a.T1;
    const int slab = b % a.slabs;
    const int64_t n = b / a.slabs;
    const int S0 = a.S[0];
    const int P = slab * kSlab, Pend = P + kSlab < S0 ? P + kSlab : S0;
    const float* xn = a.x + n * CIN * (int64_t)S0 * a.S[1] * a.S[2];
    const int r0 = t1 * kTile - 1, c0 = t2 * kTile - 1;

    // Plane P is stored before the loop; plane p + 1 is stored at the top of
    // the iteration of plane p, before its barrier, so the loads fetched one
    // iteration earlier had a whole iteration of products to arrive.
    float4 pre[fetch_units<CIN>()];
    if constexpr (FAST) {
        // halos are zero and never written again; the interiors are fetched
        for (int i = tid; i < 3 * kSlot / 4; i += kStatThreads)
            reinterpret_cast<float4*>(lds)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 pre0[fetch_units<CIN>()];
        fast_fetch<CIN>(xn, P, S0, pre0);
        fast_fetch<CIN>(xn, P + 1, S0, pre);
        __syncthreads();
        fast_put<CIN>(lds, pre0);
    } else {
        box_stage<CIN>(xn, P, a, r0, c0, lds);
    }

    float acc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[i] = 0.f;
    const int g = 2 * (wv % (kStatThreads / 128)) + (lane >> 5);
    const int lane_base = (4 * g + 1) * kRS + 4 + (lane & 31);
    for (int p = P; p < Pend; ++p) {
        const int i = p - P;
        // plane p + 1 (zero beyond the input) into the slot after plane p's
        if constexpr (FAST)
            fast_put<CIN>(lds + ((i + 1) % 3) * kSlot, pre);
        else
            box_stage<CIN>(xn, p + 1, a, r0, c0, lds + ((i + 1) % 3) * kSlot);
        __syncthreads();
        if constexpr (FAST) {
            if (p + 1 < Pend) fast_fetch<CIN>(xn, p + 2, S0, pre);  // read by the next plane
        }
        const float* pa = lds + (i % 3) * kSlot + lane_base;
        const float* pb = lds + ((i + 1) % 3) * kSlot + lane_base;
        if (second)
            stat_rows_b<CIN>(pa, pb, acc);
        else
            stat_rows_a<CIN>(pa, pb, acc);
    }
    __syncthreads();
    // every LDS read is done: the first slot takes the waves' totals
    wave_reduce_to<NA>(acc, lds + wv * NA, lane);
    __syncthreads();
    if (tid < NS) {
        constexpr int kHalfW = kStatThreads / 128;  // waves per half
        const int w0 = tid < HA ? 0 : kHalfW, v = tid < HA ? tid : tid - HA;
        float s = lds[w0 * NA + v];
#pragma unroll
        for (int w = 1; w < kHalfW; ++w) s += lds[(w0 + w) * NA + v];
        a.part[(int64_t)blk * kStatRow + tid] = s;
    }
}

template <int CIN, bool FAST>
__global__ __launch_bounds__(kStatThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void swap_stats_kernel(StatArgs a) {
    __shared__ __attribute__((aligned(16))) float lds[3 * CIN * kChS];
    stats_block<CIN, FAST>(a, lds, (int)blockIdx.x);
}

// ----------------------------------------------------------------- shell
// Gram matrices of the 26 boundary types.  Each matrix-core step takes 4
// positions of one type (lane group kq = lane / 16); lane m = lane % 16
// supplies entry m of the position's patch vector, and the same value serves
// as both operands, so D accumulates the 16 x 16 Gram matrix.  Every type's
// partial goes to its own 256-float row; the reduce kernel adds the rows of
// a type (count rows, stride apart).
//
// LDS form (workgroups of the statistics kernel, below): the boundary planes
// staged in LDS, one (sample, face axis, side) per workgroup.  Global form
// (faces too large for LDS, a kernel of its own): a wave takes a run of rows
// of one type and reads x directly.

struct ShellArgs {
    const float* x;
    float* part;  // LDS form: [N][kTypes][256]; global form: [blocks][256]
    int32_t S[3];
    int32_t first_block[kTypes + 1];  // global form
    int32_t rows_total[kTypes];
    int32_t rows_per_wave[kTypes];
};

__device__ inline bool one_lane(int m) { return m == 15; }  // the constant entry of the patch vector

__host__ __device__ inline int type_index(int t0, int t1, int t2) {
    const int c = 9 * t0 + 3 * t1 + t2;
    return c < 13 ? c : c - 1;
}

// LDS layout of the LDS form: slice (channel) holds the face plane with
// row stride Sb + 1 and slice stride = 8 (mod 64) banks, so the 16 entries x
// 4 rows of a step fall in distinct banks or on the same word; a row of
// zeros and a row of ones follow (the lanes of padding entries, of the
// constant entry and of rows beyond the type read them).
__host__ __device__ inline int shell_rs(int Sb) { return Sb + 1; }
__host__ __device__ inline int shell_cs(int Sa, int Sb) {
    const int sl = Sa * shell_rs(Sb);
    return sl + ((8 - sl) % 64 + 64) % 64;
}

// The LDS form inside the statistics kernel: a 256-thread workgroup takes
// one (sample, face axis i): it stages the input planes x_i = 0 and
// x_i = S_i - 1 and takes the types whose first non-M coordinate is i (18, 6
// and 2 types for i = 0, 1, 2: a partition of the boundary).  One wave per
// type, no reduction across waves: the two face types (M, M) on waves 0 and
// 1, the small types alternating on waves 2 and 3; every wave writes its own
// partial rows.  (Measured against splitting each face's rows over the four
// waves, with one workgroup per side: slower.)
__host__ __device__ inline int shell_lds_floats(int C, int Sa, int Sb) {
    // slices of both sides, 8 words of slack (reads past a row end are
    // discarded), zero and ones rows of Sb + 9 with their bank alignment
    return 2 * C * shell_cs(Sa, Sb) + 8 + 2 * (shell_rs(Sb) + 8) + 128;
}

template <int CIN, int NT>
__device__ void shell_block(const ShellArgs& a, int blk, float* pl) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t n = blk / 3;
    const int fi = blk % 3;
    const int ad = fi == 0 ? 1 : 0, bd = fi == 2 ? 1 : 2;
    const int S[3] = {a.S[0], a.S[1], a.S[2]};
    const int Sa = S[ad], Sb = S[bd], Si = S[fi];
    const int st[3] = {S[1] * S[2], S[2], 1};
    const int plane3 = S[0] * S[1] * S[2];
    const float* xn = a.x + n * CIN * (int64_t)plane3;
    const int face = Sa * Sb, RS = shell_rs(Sb), CS = shell_cs(Sa, Sb);
    int zoff = 2 * CIN * CS + 8;
    zoff += ((24 - zoff) % 64 + 64) % 64;
    int ooff = zoff + RS + 8;
    ooff += ((28 - ooff) % 64 + 64) % 64;
    for (int i = tid; i < RS + 8; i += NT) {
        pl[zoff + i] = 0.f;
        pl[ooff + i] = 1.f;
    }
    // stage slices (side, channel), twelve independent loads per thread at a
    // time; the index splits use float reciprocals (exact below 2^22)
    const int total = 2 * CIN * face;
    const float rface = 1.f / (float)face, rsb = 1.f / (float)Sb;
    for (int e0 = 0; e0 < total; e0 += 12 * NT) {
        float v[12];
        int dst[12];
#pragma unroll
        for (int u = 0; u < 12; ++u) {
            const int e = e0 + u * NT + tid;
            const int ec = e < total ? e : total - 1;
            const int sc = (int)(((float)ec + 0.5f) * rface), idx = ec - sc * face;
            const int ia = (int)(((float)idx + 0.5f) * rsb), ib = idx - ia * Sb;
            const int side = sc >= CIN, c = sc - side * CIN;
            v[u] = xn[c * plane3 + (side ? Si - 1 : 0) * st[fi] + ia * st[ad] + ib * st[bd]];
            dst[u] = e < total ? sc * CS + ia * RS + ib : -1;
        }
#pragma unroll
        for (int u = 0; u < 12; ++u)
            if (dst[u] >= 0) pl[dst[u]] = v[u];
    }
    __syncthreads();
    // a type's positions form an na x nb grid; a step takes 4 rows (lane group
    // kq = row within the group) at one column, so within a row group the LDS
    // reads are immediate offsets
    const int m = lane & 15, kq = lane >> 4;
    int small = 0;
    for (int side = 0; side < 2; ++side)
        for (int ta = (ad < fi ? 1 : 0); ta <= (ad < fi ? 1 : 2); ++ta)
            for (int tb = (bd < fi ? 1 : 0); tb <= (bd < fi ? 1 : 2); ++tb) {
                const bool big = ta == 1 && tb == 1;
                const int owner = big ? side : 2 + (small++) % (NT / 64 - 2);
                if (owner != wv) continue;  // uniform per wave
                const int nM = (ta == 1) + (tb == 1);
                const int na = ta == 1 ? Sa - 1 : 1, nb = tb == 1 ? Sb - 1 : 1;
                const bool real = m < (CIN << nM);
                int base = 0;
                if (real) {
                    const int c = m >> nM, bits = m & ((1 << nM) - 1);
                    // entry bits: the M dims in dim order, the first one the highest bit (ad < bd)
                    const int da = ta == 1 ? (bits >> (nM - 1)) & 1 : 0;
                    const int db = tb == 1 ? bits & 1 : 0;
                    const int ia = ta == 0 ? 0 : (ta == 2 ? Sa - 1 : da);
                    const int ib = tb == 0 ? 0 : (tb == 2 ? Sb - 1 : db);
                    base = (side * CIN + c) * CS + ia * RS + ib;
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int groups = na > 0 && nb > 0 ? (na + 3) >> 2 : 0;
                for (int g = 0; g < groups; ++g) {
                    const int row = 4 * g + kq;
                    const bool rok = row < na;
                    const float* src = pl + (real && rok ? base + row * RS : (one_lane(m) && rok ? ooff : zoff));
                    for (int v0 = 0; v0 < nb; v0 += 8) {
                        float e[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) e[u] = src[v0 + u];
#pragma unroll
                        for (int u = 0; u < 8; ++u)
                            if (v0 + u < nb) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(e[u], e[u], acc, 0, 0, 0);
                    }
                }
                int tau[3];
                tau[fi] = side ? 2 : 0;
                tau[ad] = ta;
                tau[bd] = tb;
                float* dst = a.part + ((int64_t)n * kTypes + type_index(tau[0], tau[1], tau[2])) * 256;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(4 * kq + i) * 16 + m] = acc[i];
            }
}

// The statistics kernel with the LDS-form shell workgroups appended: blocks
// [0, stat blocks) take statistics, the others one (sample, face axis) each
// (measured: behind the statistics the shell work fills the tail; in front
// it delays the statistics workgroups).
template <int CIN, bool FAST>
__global__ __launch_bounds__(kStatThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void swap_stats_shell_kernel(StatArgs a, ShellArgs sh) {
    constexpr int kSlot = CIN * kChS;
    __shared__ __attribute__((aligned(16))) float lds[3 * kSlot];
    if ((int)blockIdx.x >= a.blocks) {
        shell_block<CIN, kStatThreads>(sh, (int)blockIdx.x - a.blocks, lds);
        return;
    }
    stats_block<CIN, FAST>(a, lds, (int)blockIdx.x);
}

template <int CIN>
__global__ __launch_bounds__(kThreads) void swap_shell_global_kernel(ShellArgs a) {
    __shared__ float red[kThreads / 64][256];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int b = blockIdx.x;
    int t = 0;
    while (t + 1 < kTypes && a.first_block[t + 1] <= b) ++t;
    int tau[3];
    type_of(t, tau);
    const int S[3] = {a.S[0], a.S[1], a.S[2]};
    const int64_t stride[3] = {(int64_t)S[1] * S[2], (int64_t)S[2], 1};
    const int64_t plane3 = (int64_t)S[0] * S[1] * S[2];
    int Ms[2] = {0, 0}, nM = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (tau[i] == 1) Ms[nM++] = i;
    const int rps = nM == 2 ? S[Ms[0]] - 1 : 1;      // rows per sample
    const int RL = nM >= 1 ? S[Ms[nM - 1]] - 1 : 1;  // row length
    const int64_t sa = nM == 2 ? stride[Ms[0]] : 0;
    const int64_t sb = nM >= 1 ? stride[Ms[nM - 1]] : 0;
    const int m = lane & 15, kq = lane >> 4;
    const bool real = m < (CIN << nM);
    const bool one = m == 15;
    int64_t off = 0;
    if (real) {
        const int c = m >> nM, bits = m & ((1 << nM) - 1);
        off = c * plane3;
        int j = 0;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            int coord;
            if (tau[i] == 0)
                coord = 0;  // q = -1, delta 1
            else if (tau[i] == 2)
                coord = S[i] - 1;  // q = S - 1, delta 0
            else {
                coord = (bits >> (nM - 1 - j)) & 1;  // delta; q added per position
                ++j;
            }
            off += coord * stride[i];
        }
    }
    const int wi = (b - a.first_block[t]) * (kThreads / 64) + wv;
    const int rpw = a.rows_per_wave[t];
    const int64_t rb = (int64_t)wi * rpw;
    const int64_t re0 = rb + rpw, re = re0 < a.rows_total[t] ? re0 : a.rows_total[t];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t r = rb; r < re; ++r) {
        const int64_t n = r / rps;
        const int u = (int)(r - n * rps);
        const float* xr = a.x + n * CIN * plane3 + off + u * sa;
        for (int v0 = 0; v0 < RL; v0 += 16) {
            float e[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int v = v0 + 4 * q + kq;
                const bool ok = v < RL;
                const float ld = xr[(ok ? v : RL - 1) * sb];
                e[q] = ok ? (real ? ld : (one ? 1.f : 0.f)) : 0.f;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(e[q], e[q], acc, 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][(4 * kq + i) * 16 + m] = acc[i];
    __syncthreads();
    float s = red[0][tid];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) s += red[w][tid];
    a.part[(int64_t)b * 256 + tid] = s;
}

// --------------------------------------------------------------- finalize
struct FinArgs {
    const float* stat_part;
    int32_t stat_blocks;
    const float* shell_part;
    int32_t shell_first[kTypes];  // first partial row of each type, rows shell_stride apart
    int32_t shell_count[kTypes];
    int32_t shell_stride;
    double* tot;  // [NS] statistics, then [kTypes][256] Gram matrices
    int32_t* tab; // [entries][9] index table of the contraction
    const float* w;  // [Cin][Cout][27]
    int32_t Cin, Cout;
    int32_t S[3];
    int64_t N;
    const float* bias;
    const float* gamma;
    const float* beta;
    float eps;
    float* mean_out;
    float* var_out;
    float* run_mean;
    float* run_var;
    float momentum;
    float* scsh;  // [2][Cout] scale, shift
    float* wp;    // [Kp][Np]
    int32_t Kp, Np;
};

constexpr int kFinThreads = 1024;

// summed weights: Wp[k][n], k = ic * 27 + (a * 3 + b) * 3 + c over the
// window's input offsets, n the output channel; zero padding beyond
__device__ void build_wp(const float* w, int Cin, int Cout, int Kp, int Np, float* wp, int tid, int nthreads) {
    for (int e = tid; e < Kp * Np; e += nthreads) {
        const int k = e / Np, oc = e % Np;
        float s = 0.f;
        if (k < Cin * 27 && oc < Cout) {
            const int ic = k / 27, t = k % 27;
            const int ao = t / 9, bo = (t / 3) % 3, co = t % 3;
            const int lo[3] = {1, 0, 0}, hi[3] = {2, 2, 0};  // taps reaching the window from input 2j + offset
            for (int k0 = lo[ao]; k0 <= hi[ao]; ++k0)
                for (int k1 = lo[bo]; k1 <= hi[bo]; ++k1)
                    for (int k2 = lo[co]; k2 <= hi[co]; ++k2)
                        s += w[((int64_t)ic * Cout + oc) * 27 + (k0 * 3 + k1) * 3 + k2];
        }
        wp[e] = s;
    }
}

// dst[i] = src[i] for i < n by nthreads threads, eight loads in flight each
template <typename T>
__device__ void copy_batched(T* dst, const T* src, int n, int tid, int nthreads) {
    for (int i0 = 0; i0 < n; i0 += 8 * nthreads) {
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * nthreads + tid;
            v[u] = src[i < n ? i : 0];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * nthreads + tid;
            if (i < n) dst[i] = v[u];
        }
    }
}

// Contraction entries of the classes r = 0 .. 7.  Class r's taps are the
// entries (c, delta), delta over the residue-1 dims of r (the first such dim
// the highest bit): index i = c * 2^|r| + bits.  M entry (r, i, j) is
// L(c_i, c_j, delta_j - delta_i) minus the Gram entries of the boundary types
// of r compatible with both taps (per dim: residue 0 takes M or H; residue 1
// takes M, or L where both deltas are 1, H where both are 0; at least one
// residue-1 dim not M); S entry (r, i) is X_c minus their sum entries.  Then
// sum t^2 = sum_r w_r^T M_r w_r and sum t = sum_r w_r . S_r.
// class r of M entry e (sq = true) or S entry e, and the first entry of r:
// class r has (C 2^|r|)^2 M entries and C 2^|r| S entries
__device__ inline int class_of(int e, int C, bool sq, int& first) {
    int r = 0, base = 0;
    for (;; ++r) {
        const int nr = C << __popc(r), sz = sq ? nr * nr : nr;
        if (e < base + sz || r == 7) break;
        base += sz;
    }
    first = base;
    return r;
}

// entry e (M entries first, then S entries): out[0] = index of its total,
// out[1 .. 8] = indices of the Gram entries it subtracts (-1: none), all into
// the totals array (statistics, then 26 x 256 Gram entries)
__device__ void entry_index(int e, int C, int* out) {
    const int NS = n_stat(C), Mtot = C * C * 125;
    const bool is_m = e < Mtot;
    int first;
    const int r = class_of(is_m ? e : e - Mtot, C, is_m, first);
    const int nb = __popc(r), nr = C << nb;
    const int loc = (is_m ? e : e - Mtot) - first;
    const int i = is_m ? loc / nr : loc, j = is_m ? loc % nr : 0;
    const int c = i >> nb, cp = j >> nb;
    int di[3], dj[3];
    for (int d = 0, k = nb - 1; d < 3; ++d) {
        const bool rd = (r >> (2 - d)) & 1;
        di[d] = rd ? ((i >> k) & 1) : 0;
        dj[d] = rd ? ((j >> k) & 1) : 0;
        if (rd) --k;
    }
    if (is_m) {
        const int D0 = dj[0] - di[0], D1 = dj[1] - di[1], D2 = dj[2] - di[2];
        if (D0 == 0 && D1 == 0 && D2 == 0) {
            const int lo = c < cp ? c : cp, hi = c < cp ? cp : c;
            int l0 = C;
            for (int pa = 0; pa < lo; ++pa) l0 += C - pa;
            out[0] = l0 + hi - lo;
        } else {
            const int F = C + C * (C + 1) / 2;
            const bool fwd = D0 > 0 || (D0 == 0 && (D1 > 0 || (D1 == 0 && D2 > 0)));
            out[0] = fwd ? F + (fwd_index(D0, D1, D2) * C + c) * C + cp
                         : F + (fwd_index(-D0, -D1, -D2) * C + cp) * C + c;
        }
    } else {
        out[0] = c;
    }
    for (int o8 = 0; o8 < 8; ++o8) {
        int tau[3];
        bool ok = true, outside = false;
        for (int d = 0; d < 3; ++d) {
            const bool rd = (r >> (2 - d)) & 1, od = (o8 >> (2 - d)) & 1;
            if (!od) {
                tau[d] = 1;
            } else if (!rd) {
                tau[d] = 2;
            } else {
                if (is_m && di[d] != dj[d]) ok = false;
                tau[d] = di[d] ? 0 : 2;
                outside = true;
            }
        }
        int idx = -1;
        if (ok && outside) {
            int nM = 0, bi = 0, bj = 0;
            for (int d = 0; d < 3; ++d)
                if (tau[d] == 1) {
                    ++nM;
                    bi = 2 * bi + di[d];
                    bj = 2 * bj + dj[d];
                }
            const int mi = (c << nM) | bi, mj = (cp << nM) | bj;
            idx = NS + type_index(tau[0], tau[1], tau[2]) * 256 + (is_m ? mi * 16 + mj : 15 * 16 + mi);
        }
        out[1 + o8] = idx;
    }
}

// Block v < NS sums statistic v over the statistics workgroups; block NS + t
// sums the Gram matrix of type t over its partial rows (entry tid % 256, four
// groups of rows); block NS + 26 builds the summed weights.  Each block
// issues its loads (sixteen in flight per thread) before it computes its
// slice of the contraction's index table.
__global__ __launch_bounds__(kFinThreads) void swap_reduce_kernel(FinArgs a) {
    __shared__ double red[kFinThreads];
    __shared__ float wl[kMaxCin * kMaxCout * 27];
    const int tid = threadIdx.x;
    const int C = a.Cin, NS = n_stat(C);
    const int v = blockIdx.x;
    const int E = C * C * 125 + C * 27;  // contraction entries: sums over classes of (C 2^|r|)^2 and C 2^|r|
    auto table_slice = [&]() {
        const int chunk = (E + (int)gridDim.x - 1) / (int)gridDim.x, e = v * chunk + tid;
        if (tid < chunk && e < E) {
            int o[9];
            entry_index(e, C, o);
            for (int k = 0; k < 9; ++k) a.tab[e * 9 + k] = o[k];
        }
    };
    if (v < NS) {
        // parts b = tid, tid + 1024, ... of statistic v, in order
        double s = 0.0;
        for (int b0 = 0; b0 < a.stat_blocks; b0 += 16 * kFinThreads) {
            float vals[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int bb = b0 + u * kFinThreads + tid;
                vals[u] = a.stat_part[(int64_t)(bb < a.stat_blocks ? bb : 0) * kStatRow + v];
            }
            if (b0 == 0) table_slice();
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (b0 + u * kFinThreads + tid < a.stat_blocks) s += (double)vals[u];
        }
        red[tid] = s;
        __syncthreads();
        for (int h = kFinThreads / 2; h > 0; h >>= 1) {
            if (tid < h) red[tid] += red[tid + h];
            __syncthreads();
        }
        if (tid == 0) a.tot[v] = red[0];
    } else if (v < NS + kTypes) {
        // rows gq, gq + 4, ... of type t, entry e
        const int t = v - NS, e = tid & 255, gq = tid >> 8;
        const int cnt = a.shell_count[t];
        const float* src = a.shell_part + (int64_t)a.shell_first[t] * 256 + e;
        const int64_t step = (int64_t)a.shell_stride * 256;
        double s = 0.0;
        for (int j0 = gq; j0 < cnt; j0 += 4 * 16) {
            float vals[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int j = j0 + 4 * u;
                vals[u] = src[(j < cnt ? j : 0) * step];
            }
            if (j0 == gq) table_slice();
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (j0 + 4 * u < cnt) s += (double)vals[u];
        }
        if (gq >= cnt) table_slice();
        red[tid] = s;
        __syncthreads();
        if (tid < 256) a.tot[NS + t * 256 + tid] = ((red[tid] + red[tid + 256]) + red[tid + 512]) + red[tid + 768];
    } else {
        copy_batched(wl, a.w, C * a.Cout * 27, tid, kFinThreads);
        table_slice();
        __syncthreads();
        build_wp(wl, a.Cin, a.Cout, a.Kp, a.Np, a.wp, tid, kFinThreads);
    }
}

// One block: the contraction of the totals with the weights (both in LDS),
// then the batch statistics, the normalisation and the running update.
__global__ __launch_bounds__(kFinThreads) void swap_contract_kernel(FinArgs a) {
    constexpr int kMaxM = kMaxCin * kMaxCin * 125;
    constexpr int kMaxS = kMaxCin * 27;
    __shared__ float wl[kMaxCin * kMaxCout * 27];
    __shared__ double mr[kMaxM];
    __shared__ double sr[kMaxS];
    __shared__ int tw[kMaxS], ecls[kMaxS], eidx[kMaxS], mf[kMaxS];
    __shared__ double wd[kMaxCout][kMaxS];  // weight of class entry e for output channel oc
    __shared__ double tl[n_stat(kMaxCin) + kTypes * 256];
    const int tid = threadIdx.x;
    const int C = a.Cin, NS = n_stat(C);
    const int Mtot = C * C * 125, Stot = C * 27, E = Mtot + Stot;
    const int Cout = a.Cout;
    // every global load of the kernel at once: weights, totals and this
    // thread's (at most two) rows of the index table
    constexpr int kWPer = (kMaxCin * kMaxCout * 27 + kFinThreads - 1) / kFinThreads;
    constexpr int kTPer = (n_stat(kMaxCin) + kTypes * 256 + kFinThreads - 1) / kFinThreads;
    static_assert(kMaxM + kMaxS <= 2 * kFinThreads, "two table rows per thread");
    const int nw = C * Cout * 27, nt = NS + kTypes * 256;
    float wv[kWPer];
    double tv[kTPer];
    int t9[2][9];
#pragma unroll
    for (int u = 0; u < kWPer; ++u) {
        const int i = u * kFinThreads + tid;
        wv[u] = a.w[i < nw ? i : 0];
    }
#pragma unroll
    for (int u = 0; u < kTPer; ++u) {
        const int i = u * kFinThreads + tid;
        tv[u] = a.tot[i < nt ? i : 0];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = h * kFinThreads + tid;
#pragma unroll
        for (int k = 0; k < 9; ++k) t9[h][k] = a.tab[(e < E ? e : 0) * 9 + k];
    }
#pragma unroll
    for (int u = 0; u < kWPer; ++u)
        if (u * kFinThreads + tid < nw) wl[u * kFinThreads + tid] = wv[u];
#pragma unroll
    for (int u = 0; u < kTPer; ++u)
        if (u * kFinThreads + tid < nt) tl[u * kFinThreads + tid] = tv[u];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = h * kFinThreads + tid;
        if (e >= E) continue;
        double val = tl[t9[h][0]];
#pragma unroll
        for (int k = 1; k < 9; ++k) {
            const int q = t9[h][k];
            if (q >= 0) val -= tl[q];
        }
        if (e < Mtot) {
            mr[e] = val;
        } else {
            const int es = e - Mtot;
            sr[es] = val;
            int first, mfirst = 0;
            const int r = class_of(es, C, false, first);
            for (int q = 0; q < r; ++q) mfirst += (C << __popc(q)) * (C << __popc(q));
            const int nb = __popc(r), i = es - first;
            int k = 0;
            for (int d = 0, b = nb - 1; d < 3; ++d) {
                int kd = 1;
                if ((r >> (2 - d)) & 1) {
                    kd = ((i >> b) & 1) ? 0 : 2;  // delta 1 <- k 0, delta 0 <- k 2
                    --b;
                }
                k = 3 * k + kd;
            }
            tw[es] = (i >> nb) * Cout * 27 + k;
            ecls[es] = r;
            eidx[es] = i;
            mf[es] = mfirst;
        }
    }
    __syncthreads();
    // item (channel, class entry i): w_i (sum_j w_j M_r[i][j]) and w_i S_r[i];
    // tw[e] is the offset in w of class entry e (its channel and tap) without
    // the output channel, mf[e] the first M entry of its row
    for (int it = tid; it < Cout * Stot; it += kFinThreads) {
        const int oc = it / Stot, e = it % Stot;
        wd[oc][e] = (double)wl[tw[e] + oc * 27];
    }
    __syncthreads();
    // a wave per channel: lane l takes the items l and l + 64 (the inner sum
    // runs over at most 8 C entries, unrolled with its loads together), then
    // a fixed butterfly adds the lanes
    constexpr int kMaxRow = 8 * kMaxCin;
    static_assert(kMaxS <= 128, "two items per lane");
    for (int oc0 = 0; oc0 < Cout; oc0 += kFinThreads / 64) {
        const int oc = oc0 + (tid >> 6), l = tid & 63;
        double s1 = 0.0, s2 = 0.0;
        if (oc < Cout) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = l + 64 * h;
                if (e >= Stot) continue;
                const int r = ecls[e], nr = C << __popc(r), i = eidx[e];
                const int e0 = e - i;  // first entry of the class
                const double* wrow = wd[oc] + e0;
                const double* mrow = mr + mf[e0] + i * nr;
                double acc = 0.0;
#pragma unroll
                for (int j = 0; j < kMaxRow; ++j)
                    if (j < nr) acc += wrow[j] * mrow[j];
                const double wi = wd[oc][e];
                s1 += wi * sr[e];
                s2 += wi * acc;
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            s1 += __shfl_xor(s1, off, 64);
            s2 += __shfl_xor(s2, off, 64);
        }
        if (l != 0 || oc >= Cout) continue;
        const double count = (double)a.N * (double)(2 * a.S[0] - 1) * (double)(2 * a.S[1] - 1) * (double)(2 * a.S[2] - 1);
        const double mean = s1 / count;
        double var = s2 / count - mean * mean;
        if (var < 0.0) var = 0.0;
        const double sc = (double)a.gamma[oc] / sqrt(var + (double)a.eps);
        a.scsh[oc] = (float)sc;
        a.scsh[Cout + oc] = (float)((double)a.beta[oc] - mean * sc);
        const double true_mean = mean + (a.bias ? (double)a.bias[oc] : 0.0);
        if (a.mean_out) a.mean_out[oc] = (float)true_mean;
        if (a.var_out) a.var_out[oc] = (float)var;
        if (a.run_mean) {  // count > 1 is checked on the host
            const double mo = (double)a.momentum;
            a.run_mean[oc] = (float)((1.0 - mo) * (double)a.run_mean[oc] + mo * true_mean);
            a.run_var[oc] = (float)((1.0 - mo) * (double)a.run_var[oc] + mo * var * count / (count - 1.0));
        }
    }
}

// --------------------------------------------------------------- pooled
// A workgroup takes 2 pooled planes x 16 x 16 windows of one sample and
// stages the input box they read (5 x 33 x 33 per channel).  An M tile is 16
// windows along the last dim; wave w takes tile rows j1 = w, w + 4, ... of
// both planes, so every tile's LDS offset is a compile-time immediate added
// to the lane's per-step addresses.  K runs over (channel, a, b, c) of the
// window's 3x3x3 inputs, padded to a multiple of 4 (Wp is zero there).
constexpr int kPJ0 = 2;            // pooled planes per workgroup
constexpr int kPJ = 16;            // windows per tile side
constexpr int kBoxD = 2 * kPJ0 + 1;
constexpr int kBoxE = 2 * kPJ + 1;  // 33
constexpr int kPRS = 36;            // row stride (16-byte aligned)
constexpr int kPPS = kBoxE * kPRS;  // plane stride
constexpr int kPCS = kBoxD * kPPS;  // channel stride

struct PoolArgs {
    const float* x;
    float* y;
    const float* wp;    // [Kp][Np], or null: built here from w
    const float* scsh;  // [2][Cout], or null: eval affine from ev
    const float* w;
    BnEval ev;
    int64_t N;
    int32_t Cout;
    int32_t S[3];
    int32_t P[3];
    int32_t J[3];  // workgroup tiles per dim
    int32_t Kp, Np;
    int32_t blocks;
};

template <int CIN, int NT, bool FAST>
__global__ __launch_bounds__(kThreads) void swap_pool_kernel(PoolArgs a) {
    constexpr int KS = (CIN * 27 + 3) / 4;
    __shared__ __attribute__((aligned(16))) float lds[CIN * kPCS];
    __shared__ float wps[FAST ? 1 : (4 * KS) * (16 * NT)];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int b = blockIdx.x;
    if ((a.blocks & 7) == 0) b = (b & 7) * (a.blocks >> 3) + (b >> 3);
    const int Jt2 = b % a.J[2];
    b /= a.J[2];
    const int Jt1 = b % a.J[1];
    b /= a.J[1];
    const int Jt0 = b % a.J[0];
    const int64_t n = b / a.J[0];
    const int S0 = a.S[0], S1 = a.S[1], S2 = a.S[2];
    const float* xn = a.x + n * CIN * (int64_t)S0 * S1 * S2;
    const int i0 = 2 * kPJ0 * Jt0, i1 = 2 * kPJ * Jt1, i2 = 2 * kPJ * Jt2;  // box origin

    const int m = lane & 15, kq = lane >> 4;
    // B operand (summed weights), scale and shift: loads issued with the box's
    float bw[NT][KS];
    float sc[NT], sh[NT];
    if (FAST || a.wp) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bw[nt][s] = a.wp[(4 * s + kq) * (16 * NT) + nt * 16 + m];
    }
    if constexpr (FAST) {
        // S1 = S2 = 32: rows and columns 0 .. 31 from the input, 32 zero; thread
        // tid takes float4 tid of each of the CIN x 5 (channel, plane) slices
        constexpr int kPer = CIN * kBoxD;
        float4 v[kPer];
        const int q = tid & 7, row = tid >> 3;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int c = u / kBoxD, p = i0 + u % kBoxD;
            const int pc = p < S0 ? p : S0 - 1;
            v[u] = *reinterpret_cast<const float4*>(xn + ((int64_t)c * S0 + pc) * 1024 + row * 32 + 4 * q);
        }
        for (int f = tid; f < CIN * kBoxD * (2 * kBoxE - 1); f += kThreads) {
            const int cp = f / (2 * kBoxE - 1), e = f % (2 * kBoxE - 1);
            if (e < kBoxE)
                lds[cp * kPPS + 32 * kPRS + e] = 0.f;  // row 32
            else
                lds[cp * kPPS + (e - kBoxE) * kPRS + 32] = 0.f;  // column 32 of rows 0 .. 31
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int p = i0 + u % kBoxD;
            *reinterpret_cast<float4*>(lds + u * kPPS + row * kPRS + 4 * q) =
                p < S0 ? v[u] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        constexpr int kBox = CIN * kBoxD * kBoxE * kBoxE;
        for (int e0 = 0; e0 < kBox; e0 += 16 * kThreads) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int e = e0 + u * kThreads + tid;
                const int col = e % kBoxE, row = (e / kBoxE) % kBoxE, cp = e / (kBoxE * kBoxE);
                const int c = cp / kBoxD, pl = cp % kBoxD;
                const int p0 = i0 + pl, p1 = i1 + row, p2 = i2 + col;
                const bool in = e < kBox && p0 < S0 && p1 < S1 && p2 < S2;
                const float x = xn[in ? (((int64_t)c * S0 + p0) * S1 + p1) * S2 + p2 : 0];
                v[u] = in ? x : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int e = e0 + u * kThreads + tid;
                if (e < kBox) {
                    const int col = e % kBoxE, row = (e / kBoxE) % kBoxE, cp = e / (kBoxE * kBoxE);
                    lds[cp * kPPS + row * kPRS + col] = v[u];
                }
            }
        }
        if (!a.wp) {
            build_wp(a.w, CIN, a.Cout, 4 * KS, 16 * NT, wps, tid, kThreads);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bw[nt][s] = wps[(4 * s + kq) * (16 * NT) + nt * 16 + m];
        }
    }
    // per-step LDS addresses of this lane
    int addr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int k = 4 * s + kq;
        int off = 0;
        if (k < CIN * 27) {
            const int ic = k / 27, t = k % 27;
            off = (ic * kBoxD + t / 9) * kPPS + ((t / 3) % 3) * kPRS + t % 3;
        }
        addr[s] = off + 2 * m + 2 * wv * kPRS;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int oc = nt * 16 + m;
        sc[nt] = sh[nt] = 0.f;
        if (oc < a.Cout) {
            if (a.scsh) {
                sc[nt] = a.scsh[oc];
                sh[nt] = a.scsh[a.Cout + oc];
            } else {
                bn_eval_affine(a.ev, oc, sc[nt], sh[nt]);
            }
        }
    }
    __syncthreads();
    const int64_t pp = (int64_t)a.P[0] * a.P[1] * a.P[2];
#pragma unroll
    for (int j0l = 0; j0l < kPJ0; ++j0l) {
#pragma unroll
        for (int tt = 0; tt < kPJ / 4; ++tt) {
            const int j0 = kPJ0 * Jt0 + j0l, j1 = kPJ * Jt1 + wv + 4 * tt;
            if (j0 >= a.P[0] || j1 >= a.P[1]) continue;  // uniform per wave
            const float* base = lds + 2 * j0l * kPPS + 8 * tt * kPRS;
            f32x4 acc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const float av = base[addr[s]];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bw[nt][s], acc[nt], 0, 0, 0);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int oc = nt * 16 + m;
                if (oc >= a.Cout) continue;
                float* yr = a.y + ((n * a.Cout + oc) * pp) + ((int64_t)j0 * a.P[1] + j1) * a.P[2];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j2 = kPJ * Jt2 + 4 * kq + i;
                    if (j2 < a.P[2]) yr[j2] = fmaf(acc[nt][i] * (1.f / 64.f), sc[nt], sh[nt]);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ plan
struct SwapPlan {
    StatArgs st;
    ShellArgs sh;
    FinArgs fin;
    PoolArgs pool;
    int32_t stat_blocks, shell_blocks, fin_blocks, pool_blocks;
    bool fast_stats, fast_pool, shell_lds;
    size_t off_stat, off_shell, off_tot, off_tab, off_scsh, off_wp, bytes;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

SwapPlan plan_swap(const PoolGeom& pg, const void* x, bool eval) {
    const Geom& g = pg.g;
    SwapPlan sp{};
    const int C = (int)g.Cin, Cout = (int)g.Cout;
    const int S[3] = {(int)g.S[0], (int)g.S[1], (int)g.S[2]};
    const int NT = Cout > 16 ? 2 : 1;
    const int Kp = 4 * ((C * 27 + 3) / 4), Np = 16 * NT;
    // pooled kernel
    PoolArgs& pa = sp.pool;
    pa.N = g.N;
    pa.Cout = Cout;
    for (int j = 0; j < 3; ++j) {
        pa.S[j] = S[j];
        pa.P[j] = (int32_t)pg.P[j];
    }
    pa.J[0] = (int32_t)ceil_div(pg.P[0], kPJ0);
    pa.J[1] = (int32_t)ceil_div(pg.P[1], kPJ);
    pa.J[2] = (int32_t)ceil_div(pg.P[2], kPJ);
    pa.Kp = Kp;
    pa.Np = Np;
    sp.pool_blocks = (int32_t)(g.N * pa.J[0] * pa.J[1] * pa.J[2]);
    pa.blocks = sp.pool_blocks;
    sp.fast_pool = S[1] == 32 && S[2] == 32 && ((uintptr_t)x & 15u) == 0;
    size_t off = 0;
    if (eval) {
        sp.bytes = 0;
        return sp;
    }
    // statistics
    StatArgs& st = sp.st;
    for (int j = 0; j < 3; ++j) st.S[j] = S[j];
    st.T1 = (int32_t)ceil_div(S[1], kTile);
    st.T2 = (int32_t)ceil_div(S[2], kTile);
    st.slabs = (int32_t)ceil_div(S[0], kSlab);
    sp.stat_blocks = (int32_t)(g.N * st.slabs * st.T1 * st.T2);
    st.blocks = sp.stat_blocks;
    sp.fast_stats = S[1] == 32 && S[2] == 32 && ((uintptr_t)x & 15u) == 0;
    // shell: the LDS form when every face fits, else runs of rows per wave
    ShellArgs& sh = sp.sh;
    for (int j = 0; j < 3; ++j) sh.S[j] = S[j];
    sp.shell_lds = true;  // the LDS form, merged into the statistics kernel
    for (int i = 0; i < 3; ++i) {
        const int ad = i == 0 ? 1 : 0, bd = i == 2 ? 1 : 2;
        if ((int64_t)S[ad] * (S[bd] + 1) > 3 * C * kChS || shell_lds_floats(C, S[ad], S[bd]) > 3 * C * kChS)
            sp.shell_lds = false;
    }
    FinArgs& fn = sp.fin;
    int nb = 0;
    for (int t = 0; t < kTypes; ++t) {
        int tau[3];
        type_of(t, tau);
        int Ms[2] = {0, 0}, nM = 0;
        for (int i = 0; i < 3; ++i)
            if (tau[i] == 1) Ms[nM++] = i;
        const int64_t rps = nM == 2 ? S[Ms[0]] - 1 : 1;
        const int64_t RL = nM >= 1 ? S[Ms[nM - 1]] - 1 : 1;
        const int64_t rows = RL > 0 ? g.N * rps : 0;
        const int64_t steps_per_row = ceil_div(RL > 0 ? RL : 1, 4);
        int64_t rpw = ceil_div(128, steps_per_row);
        if (rpw < 1) rpw = 1;
        const int64_t waves = ceil_div(rows, rpw);
        sh.first_block[t] = nb;
        sh.rows_total[t] = (int32_t)rows;
        sh.rows_per_wave[t] = (int32_t)rpw;
        const int blocks = (int)ceil_div(waves, kThreads / 64);
        if (sp.shell_lds) {
            fn.shell_first[t] = t;
            fn.shell_count[t] = (int32_t)g.N;
        } else {
            fn.shell_first[t] = nb;
            fn.shell_count[t] = blocks;
        }
        nb += blocks;
    }
    sh.first_block[kTypes] = nb;
    fn.shell_stride = sp.shell_lds ? kTypes : 1;
    sp.shell_blocks = sp.shell_lds ? (int32_t)(3 * g.N) : nb;
    const size_t shell_rows = sp.shell_lds ? (size_t)g.N * kTypes : (size_t)nb;
    // finalize
    fn.stat_blocks = sp.stat_blocks;
    sp.fin_blocks = n_stat(C) + kTypes + 1;
    fn.Cin = C;
    fn.Cout = Cout;
    for (int j = 0; j < 3; ++j) fn.S[j] = S[j];
    fn.N = g.N;
    fn.Kp = Kp;
    fn.Np = Np;
    // workspace
    sp.off_stat = off;
    off = align256(off + (size_t)sp.stat_blocks * kStatRow * sizeof(float));
    sp.off_shell = off;
    off = align256(off + shell_rows * 256 * sizeof(float));
    sp.off_tot = off;
    off = align256(off + (size_t)(n_stat(C) + kTypes * 256) * sizeof(double));
    sp.off_tab = off;
    off = align256(off + (size_t)(C * C * 125 + C * 27) * 9 * sizeof(int32_t));
    sp.off_scsh = off;
    off = align256(off + 2 * (size_t)Cout * sizeof(float));
    sp.off_wp = off;
    off = align256(off + (size_t)Kp * Np * sizeof(float));
    sp.bytes = off;
    return sp;
}

template <int CIN>
void launch_training(const SwapPlan& sp, hipStream_t s) {
    if (sp.shell_lds) {
        const unsigned nb = (unsigned)(sp.stat_blocks + sp.shell_blocks);
        if (sp.fast_stats)
            hipLaunchKernelGGL((swap_stats_shell_kernel<CIN, true>), dim3(nb), dim3(kStatThreads), 0, s, sp.st, sp.sh);
        else
            hipLaunchKernelGGL((swap_stats_shell_kernel<CIN, false>), dim3(nb), dim3(kStatThreads), 0, s, sp.st, sp.sh);
    } else if (sp.fast_stats) {
        hipLaunchKernelGGL((swap_stats_kernel<CIN, true>), dim3((unsigned)sp.stat_blocks), dim3(kStatThreads), 0, s, sp.st);
    } else {
        hipLaunchKernelGGL((swap_stats_kernel<CIN, false>), dim3((unsigned)sp.stat_blocks), dim3(kStatThreads), 0, s, sp.st);
    }
    if (!sp.shell_lds)
        hipLaunchKernelGGL(swap_shell_global_kernel<CIN>, dim3((unsigned)sp.shell_blocks), dim3(kThreads), 0, s, sp.sh);
    hipLaunchKernelGGL(swap_reduce_kernel, dim3((unsigned)sp.fin_blocks), dim3(kFinThreads), 0, s, sp.fin);
    hipLaunchKernelGGL(swap_contract_kernel, dim3(1), dim3(kFinThreads), 0, s, sp.fin);
}

template <int CIN, int NT>
void launch_pool(const SwapPlan& sp, hipStream_t s) {
    if (sp.fast_pool && sp.pool.wp)
        hipLaunchKernelGGL((swap_pool_kernel<CIN, NT, true>), dim3((unsigned)sp.pool_blocks), dim3(kThreads), 0, s, sp.pool);
    else
        hipLaunchKernelGGL((swap_pool_kernel<CIN, NT, false>), dim3((unsigned)sp.pool_blocks), dim3(kThreads), 0, s, sp.pool);
}

template <int CIN>
void launch_pool_nt(const SwapPlan& sp, hipStream_t s) {
    if (sp.pool.Np > 16)
        launch_pool<CIN, 2>(sp, s);
    else
        launch_pool<CIN, 1>(sp, s);
}

}  // namespace

bool convT_bn_swap_supported(const PoolGeom& pg, const void*) {
    const Geom& g = pg.g;
    for (int j = 0; j < 3; ++j)
        if (g.k[j] != 3 || g.s[j] != 2 || g.p[j] != 1 || g.d[j] != 1 || g.O[j] != 2 * g.S[j] - 1 ||
            g.S[j] >= (1 << 20))
            return false;
    return g.groups == 1 && pg.pool == 4 && g.Cin >= 1 && g.Cin <= kMaxCin && g.Cout >= 1 && g.Cout <= kMaxCout &&
           g.N * g.S[0] * g.S[1] * g.S[2] * g.Cin < (1ll << 40) && g.N * g.S[0] * g.S[1] < (1ll << 31);
}

size_t convT_bn_swap_workspace_bytes(const PoolGeom& pg) { return plan_swap(pg, nullptr, false).bytes; }

hipError_t launch_convT_bn_swap(const float* x, const float* w, float* y, void* ws, const PoolGeom& pg,
                                const BnEval& ev, const BnSwapTrain* tr, hipStream_t s) {
    const bool eval = ev.gamma != nullptr;
    SwapPlan sp = plan_swap(pg, x, eval);
    PoolArgs& pa = sp.pool;
    pa.x = x;
    pa.y = y;
    pa.w = w;
    pa.ev = ev;
    const int C = (int)pg.g.Cin;
    if (!eval) {
        if (!tr) return hipErrorInvalidValue;
        char* base = (char*)ws;
        sp.st.x = x;
        sp.st.part = (float*)(base + sp.off_stat);
        sp.sh.x = x;
        sp.sh.part = (float*)(base + sp.off_shell);
        FinArgs& fn = sp.fin;
        fn.stat_part = sp.st.part;
        fn.shell_part = sp.sh.part;
        fn.tot = (double*)(base + sp.off_tot);
        fn.tab = (int32_t*)(base + sp.off_tab);
        fn.w = w;
        fn.bias = tr->bias;
        fn.gamma = tr->gamma;
        fn.beta = tr->beta;
        fn.eps = tr->eps;
        fn.mean_out = tr->mean_out;
        fn.var_out = tr->var_out;
        fn.run_mean = tr->run.mean;
        fn.run_var = tr->run.var;
        fn.momentum = tr->run.momentum;
        fn.scsh = (float*)(base + sp.off_scsh);
        fn.wp = (float*)(base + sp.off_wp);
        pa.scsh = fn.scsh;
        pa.wp = fn.wp;
        switch (C) {
            case 1: launch_training<1>(sp, s); break;
            case 2: launch_training<2>(sp, s); break;
            default: launch_training<3>(sp, s); break;
        }
    } else {
        pa.scsh = nullptr;
        pa.wp = nullptr;
    }
    switch (C) {
        case 1: launch_pool_nt<1>(sp, s); break;
        case 2: launch_pool_nt<2>(sp, s); break;
        default: launch_pool_nt<3>(sp, s); break;
    }
    return hipGetLastError();
}

}  // namespace c3d
