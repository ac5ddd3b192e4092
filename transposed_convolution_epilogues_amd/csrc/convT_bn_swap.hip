// convT_bn_swap.hip - the ConvTranspose3d(k3, s2, p1) -> BatchNorm3d (batch
// statistics) -> AvgPool3d(4) module with its sums swapped ("Kimi-K2.6
// l2_p72": the proposal to swap the order of the pooled sum and the conv sum).
// None of the 64 positions of a window, nor any other transposed-conv output,
// is formed one by one.
//
// Notation: per dim, output o = 2q + r (r = o mod 2, the residue).  Residue 0
// takes tap k = 1 from input q; residue 1 takes k = 0 from q + 1 and k = 2
// from q (the page's parity tables).  t = conv_transpose3d(x, w), bias-free.
//
// 1. Pooled sums.  The window [4j, 4j + 4) of a dim reads inputs 2j + a,
//    a = 0, 1, 2, through taps {1, 2}, {0, 1, 2}, {0} respectively, so the
//    window sum is a stride-2 correlation of x with the 3x3x3 kernel
//    Wp[ic][oc][a][b][c] = sum of w[ic][oc][k0][k1][k2] over those tap sets:
//    27 MACs per input channel instead of 216.
// 2. Sum of t.  Extend every residue-1 range by one zero-padded position at
//    each end (q = -1 and q = S - 1, i.e. the fake outputs o = -1 and
//    o = 2S - 1).  Over the extended ranges every input element meets every
//    tap once, so sum_ext t = sum_ic X[ic] * sum_k w[ic][oc][k], X = sum of
//    channel ic; the real sum is that minus the fake outputs' t.
// 3. Sum of t^2.  On an extended residue class, t = sum over its taps a of
//    w_a x_a(q + delta_a), so sum t^2 = sum_{a,b} w_a w_b G_ab with
//    G_ab = sum_q x_a(q + delta_a) x_b(q + delta_b): a lag correlation of the
//    input at lag delta_b - delta_a in {-1, 0, 1}^3, over its natural range
//    (the zero padding makes the extended ranges exactly the natural ones).
//    The 13 "forward" lags with every ordered channel pair, lag 0 with
//    a <= b, and the channel sums are accumulated along input rows; the fake
//    outputs' t^2 are subtracted as in 2.
// (1) needs 81 MACs per pooled output; (2) and (3) about 126 FMAs per input
// element plus the fake outputs (one plane per face of each residue class).
//
// Three kernels do the three parts (statistics rows, pooled windows, fake
// outputs); a reduction kernel merges the float64 partials in a fixed order
// and a one-block kernel contracts them with the weights into per-channel
// (sum, sum of squares), which phase 2 of convT_bn_avgpool turns into the
// normalisation.  Eval mode runs
// the pooled-window role alone with the BN affine.
#include "c3d_internal.h"

namespace c3d {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxCin = 3;
constexpr int kMaxCout = 32;
constexpr int kFwd = 13;  // lags with first nonzero component positive
constexpr int kMaxSeg = 12;

// statistics layout per workgroup: [X: C][lag 0, a <= b: C(C+1)/2][forward lags: 13 C^2]
__host__ __device__ constexpr int n_stat(int C) { return C + C * (C + 1) / 2 + kFwd * C * C; }
constexpr int kMaxStat = n_stat(kMaxCin);  // 126

struct SwapArgs {
    const float* x;
    const float* w;  // [Cin][Cout][27]
    float* y;        // [N][Cout][P0][P1][P2]
    double* stat;    // stat_blocks x n_stat(Cin)
    double* fake;    // fake_blocks x 2 Cout
    int64_t N;
    int32_t Cin, Cout;
    int32_t S[3];
    int32_t P[3];
    int64_t rows;  // N * S0 * S1 input rows
    int32_t stat_blocks, pool_blocks, fake_blocks;
    int64_t windows;  // N * P0 * P1 * P2
    // fake outputs of one sample, by segment: residue class r, face dim j,
    // mixed-radix sizes of (q0, q1, q2)
    int32_t nseg;
    int32_t seg_r[kMaxSeg];
    int32_t seg_j[kMaxSeg];
    int32_t seg_size[kMaxSeg][3];
    int64_t seg_start[kMaxSeg + 1];
    BnEval ev;  // eval mode: gamma set, only the pooled-window role runs
};

__device__ __forceinline__ float wave_sum_f(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// forward lag index: (0,0,1) -> 0; (0,1,d2) -> 1 + d2 + 1; (1,d1,d2) -> 4 + 3 (d1 + 1) + d2 + 1
__host__ __device__ constexpr int fwd_index(int d0, int d1, int d2) {
    return d0 == 1 ? 4 + 3 * (d1 + 1) + (d2 + 1) : (d1 == 1 ? 1 + (d2 + 1) : 0);
}

// ------------------------------------------------------------ statistics role
// One thread per segment of kSeg columns of an input row (n, p0, p1),
// walking p2 with a sliding window of the own row (columns c, c + 1) and of
// the four forward neighbour rows (p0, p1 + 1), (p0 + 1, p1 - 1),
// (p0 + 1, p1), (p0 + 1, p1 + 1) (columns c - 1 .. c + 1).  Out-of-range
// positions read as zero, which restricts each lag to its natural range.
// The workgroup's partials are reduced through LDS in rounds of kRound
// values: every thread stores its round, then 4 threads per value sum 64
// entries each in float64.
constexpr int kSeg = 8;
constexpr int kRound = 32;

template <int CIN, int V0, int V1>
__device__ __forceinline__ void stat_reduce_round(const SwapArgs& a, int blk, const float (&acc)[n_stat(CIN)],
                                                  float* buf, double* part4) {
    constexpr int NS = n_stat(CIN);
    constexpr int CNT = V1 - V0;
#pragma unroll
    for (int v = V0; v < V1; ++v) buf[(v - V0) * kThreads + threadIdx.x] = acc[v];
    __syncthreads();
    if (threadIdx.x < 4 * CNT) {
        const int v = threadIdx.x >> 2, q = threadIdx.x & 3;
        double sum = 0.0;
        for (int i = 0; i < kThreads / 4; ++i) sum += (double)buf[v * kThreads + q * (kThreads / 4) + i];
        part4[v * 4 + q] = sum;
    }
    __syncthreads();
    if (threadIdx.x < CNT) {
        const int v = threadIdx.x;
        a.stat[(int64_t)blk * NS + V0 + v] =
            ((part4[v * 4] + part4[v * 4 + 1]) + part4[v * 4 + 2]) + part4[v * 4 + 3];
    }
    __syncthreads();
}

template <int CIN>
__device__ void stat_role(const SwapArgs& a, int blk, float* buf, double* part4) {
    constexpr int NS = n_stat(CIN);
    const int S0 = a.S[0], S1 = a.S[1], S2 = a.S[2];
    const int segs = (S2 + kSeg - 1) / kSeg;
    const int64_t item = (int64_t)blk * kThreads + threadIdx.x;
    float acc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) acc[i] = 0.f;
    if (item < a.rows * segs) {
        const int64_t row = item / segs;
        const int c0 = (int)(item % segs) * kSeg;
        const int c1 = c0 + kSeg < S2 ? c0 + kSeg : S2;
        const int p1 = (int)(row % S1);
        const int p0 = (int)((row / S1) % S0);
        const int64_t n = row / ((int64_t)S1 * S0);
        const int64_t plane = (int64_t)S0 * S1 * S2;
        const int nr0[5] = {p0, p0, p0 + 1, p0 + 1, p0 + 1};
        const int nr1[5] = {p1, p1 + 1, p1 - 1, p1, p1 + 1};
        int64_t base[5];
        bool ok[5];
#pragma unroll
        for (int e = 0; e < 5; ++e) {
            ok[e] = nr0[e] < S0 && nr1[e] >= 0 && nr1[e] < S1;
            base[e] = n * CIN * plane + ((int64_t)(ok[e] ? nr0[e] : 0) * S1 + (ok[e] ? nr1[e] : 0)) * S2;
        }
        auto ld = [&](int e, int ic, int col) -> float {
            const bool in = ok[e] && col >= 0 && col < S2;
            const float v = a.x[base[e] + ic * plane + (in ? col : 0)];
            return in ? v : 0.f;
        };
        // window: win[e][m][ic] = row e at column c - 1 + m
        float win[5][3][CIN];
#pragma unroll
        for (int e = 0; e < 5; ++e)
#pragma unroll
            for (int ic = 0; ic < CIN; ++ic) {
                win[e][0][ic] = ld(e, ic, c0 - 1);
                win[e][1][ic] = ld(e, ic, c0);
                win[e][2][ic] = ld(e, ic, c0 + 1);
            }
        for (int c = c0; c < c1; ++c) {
#pragma unroll
            for (int ai = 0; ai < CIN; ++ai) {
                const float xa = win[0][1][ai];
                acc[ai] += xa;  // channel sum
                int l0 = CIN;   // lag 0, pairs ai <= bi
#pragma unroll
                for (int pa = 0; pa < ai; ++pa) l0 += CIN - pa;
#pragma unroll
                for (int bi = ai; bi < CIN; ++bi) acc[l0 + bi - ai] += xa * win[0][1][bi];
                constexpr int F = CIN + CIN * (CIN + 1) / 2;
#pragma unroll
                for (int bi = 0; bi < CIN; ++bi) {
                    acc[F + (fwd_index(0, 0, 1) * CIN + ai) * CIN + bi] += xa * win[0][2][bi];
#pragma unroll
                    for (int d2 = -1; d2 <= 1; ++d2)
                        acc[F + (fwd_index(0, 1, d2) * CIN + ai) * CIN + bi] += xa * win[1][d2 + 1][bi];
#pragma unroll
                    for (int d1 = -1; d1 <= 1; ++d1)
#pragma unroll
                        for (int d2 = -1; d2 <= 1; ++d2)
                            acc[F + (fwd_index(1, d1, d2) * CIN + ai) * CIN + bi] += xa * win[2 + d1 + 1][d2 + 1][bi];
                }
            }
            // slide: column c + 2 enters
#pragma unroll
            for (int e = 0; e < 5; ++e)
#pragma unroll
                for (int ic = 0; ic < CIN; ++ic) {
                    win[e][0][ic] = win[e][1][ic];
                    win[e][1][ic] = win[e][2][ic];
                    win[e][2][ic] = ld(e, ic, c + 2);
                }
        }
    }
    stat_reduce_round<CIN, 0, (NS < kRound ? NS : kRound)>(a, blk, acc, buf, part4);
    if constexpr (NS > kRound) stat_reduce_round<CIN, kRound, (NS < 2 * kRound ? NS : 2 * kRound)>(a, blk, acc, buf, part4);
    if constexpr (NS > 2 * kRound)
        stat_reduce_round<CIN, 2 * kRound, (NS < 3 * kRound ? NS : 3 * kRound)>(a, blk, acc, buf, part4);
    if constexpr (NS > 3 * kRound) stat_reduce_round<CIN, 3 * kRound, NS>(a, blk, acc, buf, part4);
}

// --------------------------------------------------------- pooled-window role
// Wp in LDS: [oc][ic][27] (a, b, c input offsets 0..2 per dim).
constexpr int kWp = 28;  // taps per (oc, ic) row of Wp, padded with a zero for 16-byte reads

__device__ void build_wp(const SwapArgs& a, float* wp) {
    const int n = a.Cout * a.Cin * kWp;
    for (int e = threadIdx.x; e < n; e += kThreads) {
        const int t = e % kWp, ic = (e / kWp) % a.Cin, oc = e / (kWp * a.Cin);
        if (t == 27) {
            wp[e] = 0.f;
            continue;
        }
        const int ao = t / 9, bo = (t / 3) % 3, co = t % 3;
        // taps reaching window position a of a dim from input 2j + a
        const int lo[3] = {1, 0, 0}, hi[3] = {2, 2, 0};
        float s = 0.f;
        for (int k0 = lo[ao]; k0 <= hi[ao]; ++k0)
            for (int k1 = lo[bo]; k1 <= hi[bo]; ++k1)
                for (int k2 = lo[co]; k2 <= hi[co]; ++k2)
                    s += a.w[((int64_t)ic * a.Cout + oc) * 27 + (k0 * 3 + k1) * 3 + k2];
        wp[e] = s;
    }
}

template <int CIN>
__device__ void pool_role(const SwapArgs& a, int blk, const float* wp) {
    const int64_t wi = (int64_t)blk * kThreads + threadIdx.x;
    if (wi >= a.windows) return;
    const int64_t pplane = (int64_t)a.P[0] * a.P[1] * a.P[2];
    const int64_t n = wi / pplane;
    const int64_t j = wi % pplane;
    const int j2 = (int)(j % a.P[2]), j1 = (int)((j / a.P[2]) % a.P[1]), j0 = (int)(j / ((int64_t)a.P[2] * a.P[1]));
    const int64_t plane = (int64_t)a.S[0] * a.S[1] * a.S[2];
    float p[CIN][kWp];
#pragma unroll
    for (int ic = 0; ic < CIN; ++ic) {
#pragma unroll
        for (int t = 0; t < 27; ++t) {
            const int i0 = 2 * j0 + t / 9, i1 = 2 * j1 + (t / 3) % 3, i2 = 2 * j2 + t % 3;  // always inside x
            p[ic][t] = a.x[(n * CIN + ic) * plane + ((int64_t)i0 * a.S[1] + i1) * a.S[2] + i2];
        }
        p[ic][27] = 0.f;
    }
    typedef float f4 __attribute__((ext_vector_type(4)));
    for (int oc = 0; oc < a.Cout; ++oc) {
        float s = 0.f;
#pragma unroll
        for (int ic = 0; ic < CIN; ++ic)
#pragma unroll
            for (int t4 = 0; t4 < kWp / 4; ++t4) {
                const f4 wv = *reinterpret_cast<const f4*>(wp + (oc * CIN + ic) * kWp + 4 * t4);
#pragma unroll
                for (int u = 0; u < 4; ++u) s = fmaf(wv[u], p[ic][4 * t4 + u], s);
            }
        float v = s * (1.f / 64.f);
        if (a.ev.gamma) {
            float sc, sh;
            bn_eval_affine(a.ev, oc, sc, sh);
            v = fmaf(v, sc, sh);
        }
        a.y[(n * a.Cout + oc) * pplane + j] = v;
    }
}

// ------------------------------------------------------------ fake-output role
// The fake outputs of one sample are enumerated face by face: for residue
// class r and face dim j (r_j = 1), q_i runs over the real range [0, S_i - 1)
// for residue-1 dims i < j (so each fake output is counted once), over
// {-1, S_j - 1} for i = j, and over the extended range for i > j.  A
// workgroup takes one (sample, segment) pair, so the class is uniform; the 8
// tap combinations are unrolled and the ones the class lacks read zero.
template <int CIN>
__device__ void fake_role(const SwapArgs& a, int blk, const float* wl, double* red) {
    const int s = blk % a.nseg;
    const int64_t n = blk / a.nseg;
    const int r = a.seg_r[s], jf = a.seg_j[s];
    const int sz1 = a.seg_size[s][1], sz2 = a.seg_size[s][2];
    const int cnt = (int)(a.seg_start[s + 1] - a.seg_start[s]);
    const int rr[3] = {(r >> 2) & 1, (r >> 1) & 1, r & 1};
    const int64_t plane = (int64_t)a.S[0] * a.S[1] * a.S[2];
    const float* xn = a.x + n * CIN * plane;
    // taps: combination t = (t0, t1, t2); a residue-0 dim has only t_d = 0 (k 1, delta 0),
    // a residue-1 dim has t_d = 0 (k 0, delta 1) and t_d = 1 (k 2, delta 0)
    int kk[8], dl[8][3];
    bool has[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int td[3] = {t >> 2, (t >> 1) & 1, t & 1};
        has[t] = (td[0] <= rr[0]) && (td[1] <= rr[1]) && (td[2] <= rr[2]);
        int k[3];
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            k[d] = rr[d] ? (td[d] ? 2 : 0) : 1;
            dl[t][d] = (rr[d] && !td[d]) ? 1 : 0;
        }
        kk[t] = (k[0] * 3 + k[1]) * 3 + k[2];
    }
    float f1[kMaxCout], f2[kMaxCout];
#pragma unroll
    for (int oc = 0; oc < kMaxCout; ++oc) f1[oc] = f2[oc] = 0.f;
    for (int g = threadIdx.x; g < cnt; g += kThreads) {
        const int idx[3] = {g / (sz1 * sz2), (g / sz2) % sz1, g % sz2};
        int q[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) q[i] = i < jf ? idx[i] : (i == jf ? (idx[i] ? a.S[i] - 1 : -1) : idx[i] - rr[i]);
        float xv[8][CIN];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            bool in = has[t];
            int i3[3];
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                i3[d] = q[d] + dl[t][d];
                in = in && i3[d] >= 0 && i3[d] < a.S[d];
            }
            // clamped address, value selected: the load never leaves x
            const int64_t off = in ? ((int64_t)i3[0] * a.S[1] + i3[1]) * a.S[2] + i3[2] : 0;
#pragma unroll
            for (int ic = 0; ic < CIN; ++ic) {
                const float v = xn[ic * plane + off];
                xv[t][ic] = in ? v : 0.f;
            }
        }
#pragma unroll
        for (int oc = 0; oc < kMaxCout; ++oc) {
            if (oc < a.Cout) {
                float tv = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int ic = 0; ic < CIN; ++ic) tv = fmaf(wl[(ic * a.Cout + oc) * 27 + kk[t]], xv[t][ic], tv);
                f1[oc] += tv;
                f2[oc] = fmaf(tv, tv, f2[oc]);
            }
        }
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int oc = 0; oc < kMaxCout; ++oc) {
        if (oc < a.Cout) {  // workgroup-uniform
            const float s1 = wave_sum_f(f1[oc]), s2 = wave_sum_f(f2[oc]);
            if (lane == 0) {
                red[wv * 2 * kMaxCout + 2 * oc] = (double)s1;
                red[wv * 2 * kMaxCout + 2 * oc + 1] = (double)s2;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < 2 * a.Cout) {
        double v = 0.0;
        for (int i = 0; i < kThreads / 64; ++i) v += red[i * 2 * kMaxCout + threadIdx.x];
        a.fake[(int64_t)blk * 2 * a.Cout + threadIdx.x] = v;
    }
}

template <int CIN>
__global__ __launch_bounds__(kThreads) void convT_bn_swap_stat_kernel(SwapArgs a) {
    __shared__ __attribute__((aligned(16))) float buf[kRound * kThreads];
    __shared__ double part4[kRound * 4];
    stat_role<CIN>(a, blockIdx.x, buf, part4);
}

template <int CIN>
__global__ __launch_bounds__(kThreads) void convT_bn_swap_pool_kernel(SwapArgs a) {
    __shared__ __attribute__((aligned(16))) float wp[kMaxCout * kMaxCin * kWp];
    build_wp(a, wp);
    __syncthreads();
    pool_role<CIN>(a, blockIdx.x, wp);
}

template <int CIN>
__global__ __launch_bounds__(kThreads) void convT_bn_swap_fake_kernel(SwapArgs a) {
    __shared__ float wl[kMaxCout * kMaxCin * 27];
    __shared__ double red[(kThreads / 64) * 2 * kMaxCout];
    for (int e = threadIdx.x; e < a.Cin * a.Cout * 27; e += kThreads) wl[e] = a.w[e];  // [ic][oc][27]
    __syncthreads();
    fake_role<CIN>(a, blockIdx.x, wl, red);
}

// Reduction of the partials: block v sums value v over all statistics (v <
// n_stat) or fake-output (after that) workgroups, in a fixed order.
__global__ __launch_bounds__(kThreads) void convT_bn_swap_reduce_kernel(SwapArgs a, double* totals) {
    __shared__ double red[kThreads];
    const int NS = n_stat(a.Cin);
    const int v = blockIdx.x;
    const bool st = v < NS;
    const double* src = st ? a.stat + v : a.fake + (v - NS);
    const int64_t stride = st ? NS : 2 * a.Cout;
    const int count = st ? a.stat_blocks : a.fake_blocks;
    double sum = 0.0;
    for (int b = threadIdx.x; b < count; b += kThreads) sum += src[(int64_t)b * stride];
    red[threadIdx.x] = sum;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) totals[v] = red[0];
}

// One block: per channel
//   sum t   = sum_ic X[ic] sum_k w[ic][oc][k] - fake sum
//   sum t^2 = sum over residue classes and tap pairs w_a w_b G_ab - fake sum of squares
// written as one (sum, sum of squares) part per channel for phase 2.  Item
// (oc, class, tap a) of the tap-pair sum goes to one thread; items and the
// final sums are added in a fixed order.
__global__ __launch_bounds__(1024) void convT_bn_swap_contract_kernel(SwapArgs a, const double* totals,
                                                                      double* out) {
    __shared__ double R[kMaxStat + 2 * kMaxCout];
    __shared__ float wl[kMaxCin * kMaxCout * 27];
    __shared__ double part[kMaxCout][8][8];
    const int C = a.Cin, NS = n_stat(C);
    for (int i = threadIdx.x; i < NS + 2 * a.Cout; i += blockDim.x) R[i] = totals[i];
    for (int i = threadIdx.x; i < C * a.Cout * 27; i += blockDim.x) wl[i] = a.w[i];
    __syncthreads();
    const double* F = R + NS;
    for (int item = threadIdx.x; item < 64 * a.Cout; item += blockDim.x) {
        const int oc = item >> 6, cls = (item >> 3) & 7, ta = item & 7;
        const int r[3] = {(cls >> 2) & 1, (cls >> 1) & 1, cls & 1};
        const int nt = (1 + r[0]) * (1 + r[1]) * (1 + r[2]);
        double s = 0.0;
        if (ta < nt) {
            for (int tb = 0; tb < nt; ++tb) {
                int ka[3], kb[3], D[3];
                int ia = ta, ib = tb;
                for (int d = 2; d >= 0; --d) {
                    const int ua = r[d] ? ia % 2 : 0, ub = r[d] ? ib % 2 : 0;
                    if (r[d]) {
                        ia /= 2;
                        ib /= 2;
                    }
                    // residue 1: index 0 -> (k 0, delta 1), 1 -> (k 2, delta 0); residue 0: (k 1, delta 0)
                    ka[d] = r[d] ? (ua ? 2 : 0) : 1;
                    kb[d] = r[d] ? (ub ? 2 : 0) : 1;
                    D[d] = (r[d] ? (ub ? 0 : 1) : 0) - (r[d] ? (ua ? 0 : 1) : 0);
                }
                const int wka = (ka[0] * 3 + ka[1]) * 3 + ka[2], wkb = (kb[0] * 3 + kb[1]) * 3 + kb[2];
                const bool zero = D[0] == 0 && D[1] == 0 && D[2] == 0;
                const bool fwd = D[0] > 0 || (D[0] == 0 && (D[1] > 0 || (D[1] == 0 && D[2] > 0)));
                for (int ca = 0; ca < C; ++ca)
                    for (int cb = 0; cb < C; ++cb) {
                        double g;
                        if (zero) {
                            const int lo = ca < cb ? ca : cb, hi = ca < cb ? cb : ca;
                            int l0 = C;
                            for (int pa = 0; pa < lo; ++pa) l0 += C - pa;
                            g = R[l0 + hi - lo];
                        } else if (fwd) {
                            g = R[C + C * (C + 1) / 2 + (fwd_index(D[0], D[1], D[2]) * C + ca) * C + cb];
                        } else {
                            g = R[C + C * (C + 1) / 2 + (fwd_index(-D[0], -D[1], -D[2]) * C + cb) * C + ca];
                        }
                        s += (double)wl[(ca * a.Cout + oc) * 27 + wka] * (double)wl[(cb * a.Cout + oc) * 27 + wkb] * g;
                    }
            }
        }
        part[oc][cls][ta] = s;
    }
    __syncthreads();
    if (threadIdx.x < a.Cout) {
        const int oc = threadIdx.x;
        double s1 = 0.0;
        for (int ic = 0; ic < C; ++ic) {
            double ws = 0.0;
            for (int k = 0; k < 27; ++k) ws += (double)wl[(ic * a.Cout + oc) * 27 + k];
            s1 += R[ic] * ws;
        }
        double s2 = 0.0;
        for (int cls = 0; cls < 8; ++cls)
            for (int ta = 0; ta < 8; ++ta) s2 += part[oc][cls][ta];
        out[2 * oc] = s1 - F[2 * oc];
        out[2 * oc + 1] = s2 - F[2 * oc + 1];
    }
}

struct SwapPlan {
    SwapArgs a;
    size_t ws_doubles;  // stat + fake partials + 2 Cout finals
};

SwapPlan plan_swap(const PoolGeom& pg, bool eval) {
    const Geom& g = pg.g;
    SwapPlan sp{};
    SwapArgs& a = sp.a;
    a.N = g.N;
    a.Cin = (int32_t)g.Cin;
    a.Cout = (int32_t)g.Cout;
    for (int j = 0; j < 3; ++j) {
        a.S[j] = (int32_t)g.S[j];
        a.P[j] = (int32_t)pg.P[j];
    }
    a.rows = g.N * g.S[0] * g.S[1];
    a.windows = g.N * pg.P[0] * pg.P[1] * pg.P[2];
    a.pool_blocks = (int32_t)ceil_div(a.windows, kThreads);
    int ns = 0;
    int64_t start = 0;
    for (int r = 0; r < 8; ++r) {
        const int rr[3] = {(r >> 2) & 1, (r >> 1) & 1, r & 1};
        for (int j = 0; j < 3; ++j) {
            if (!rr[j]) continue;
            a.seg_r[ns] = r;
            a.seg_j[ns] = j;
            int64_t cnt = 1;
            for (int i = 0; i < 3; ++i) {
                const int real = a.S[i] - rr[i], ext = a.S[i] + rr[i];
                a.seg_size[ns][i] = i < j ? real : (i == j ? 2 : ext);
                cnt *= a.seg_size[ns][i];
            }
            a.seg_start[ns] = start;
            start += cnt;
            ++ns;
        }
    }
    a.nseg = ns;
    a.seg_start[ns] = start;
    if (eval) {
        a.stat_blocks = a.fake_blocks = 0;
        sp.ws_doubles = 0;
        return sp;
    }
    a.stat_blocks = (int32_t)ceil_div(a.rows * ceil_div(a.S[2], kSeg), kThreads);
    a.fake_blocks = (int32_t)(g.N * ns);  // one (sample, segment) pair each
    // partials, then the reduced totals, then the per-channel (sum, sum of squares)
    sp.ws_doubles = (size_t)a.stat_blocks * n_stat(a.Cin) + (size_t)a.fake_blocks * 2 * a.Cout +
                    (size_t)(n_stat(a.Cin) + 2 * a.Cout) + 2 * (size_t)a.Cout;
    return sp;
}

template <int CIN>
void launch_swap_kernels(const SwapArgs& a, hipStream_t st) {
    if (a.stat_blocks)
        hipLaunchKernelGGL(convT_bn_swap_stat_kernel<CIN>, dim3((unsigned)a.stat_blocks), dim3(kThreads), 0, st, a);
    if (a.pool_blocks)
        hipLaunchKernelGGL(convT_bn_swap_pool_kernel<CIN>, dim3((unsigned)a.pool_blocks), dim3(kThreads), 0, st, a);
    if (a.fake_blocks)
        hipLaunchKernelGGL(convT_bn_swap_fake_kernel<CIN>, dim3((unsigned)a.fake_blocks), dim3(kThreads), 0, st, a);
}

}  // namespace

bool convT_bn_swap_supported(const PoolGeom& pg, const void*) {
    const Geom& g = pg.g;
    for (int j = 0; j < 3; ++j)
        if (g.k[j] != 3 || g.s[j] != 2 || g.p[j] != 1 || g.d[j] != 1 || g.O[j] != 2 * g.S[j] - 1 ||
            g.S[j] >= (1 << 20))
            return false;
    return g.groups == 1 && pg.pool == 4 && g.Cin >= 1 && g.Cin <= kMaxCin && g.Cout >= 1 && g.Cout <= kMaxCout &&
           g.N * g.S[0] * g.S[1] * g.S[2] * g.Cin < (1ll << 40);
}

size_t convT_bn_swap_workspace_bytes(const PoolGeom& pg) { return plan_swap(pg, false).ws_doubles * sizeof(double); }

hipError_t launch_convT_bn_swap(const float* x, const float* w, float* y, double* ws, const PoolGeom& pg,
                                const BnEval& ev, double** stats_out, hipStream_t st) {
    SwapPlan sp = plan_swap(pg, ev.gamma != nullptr);
    SwapArgs& a = sp.a;
    a.x = x;
    a.w = w;
    a.y = y;
    a.ev = ev;
    if (!ev.gamma) {
        a.stat = ws;
        a.fake = ws + (size_t)a.stat_blocks * n_stat(a.Cin);
    }
    switch (a.Cin) {
        case 1: launch_swap_kernels<1>(a, st); break;
        case 2: launch_swap_kernels<2>(a, st); break;
        default: launch_swap_kernels<3>(a, st); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ev.gamma) return e;
    double* totals = a.fake + (size_t)a.fake_blocks * 2 * a.Cout;
    double* fin = totals + n_stat(a.Cin) + 2 * a.Cout;
    hipLaunchKernelGGL(convT_bn_swap_reduce_kernel, dim3((unsigned)(n_stat(a.Cin) + 2 * a.Cout)), dim3(kThreads), 0,
                       st, a, totals);
    hipLaunchKernelGGL(convT_bn_swap_contract_kernel, dim3(1), dim3(1024), 0, st, a, (const double*)totals, fin);
    if (stats_out) *stats_out = fin;
    return hipGetLastError();
}

}  // namespace c3d
