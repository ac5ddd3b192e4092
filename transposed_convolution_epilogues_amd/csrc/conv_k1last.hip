// conv_k1last.hip - Conv3d whose last kernel extent is 1 (the (k,k,1) kernel
// on a depth-last tensor x[N,C,H,W,D], "Kimi-K2.6 l1_p59"), stride 1, no
// padding.
//
// With k2 = 1 the last dim is never mixed, so for fixed (n, c, row i0) the
// (i1, i2) plane is one contiguous run and an output row (n, oc, o0) is the
// contiguous run j = o1*S2 + o2 of O1*S2 floats.  Every tap (ic, k0, k1) reads
// that run shifted by k1*d1*S2 from input row o0 + k0*d0 of channel ic - the
// page's observation that D is the fastest dim, taken to its end: the whole
// (w, d) plane is one 1-D axis and no layout transform is needed.
//
// GEMM per output row: D[oc, j] = sum_k W[oc, k] * B[k, j], K = Cin*k0*k1
// (27 for the (3,3,1) kernel on 3 channels, padded to an even count).  On
// v_mfma_f32_32x32x2f32 the rows are output channels (the weights stay in
// VGPRs for the whole kernel) and the columns are output positions.  A wave
// computes blocks of 128 positions (four N tiles) x 64 channels; the four
// waves of a workgroup take the four consecutive blocks of one output row at a
// time, walk the workgroup's two rows together, and share the input they read
// through LDS.  The work is bound by the 2.6 GB of output stores, so both the
// column-to-position map and the order in which the grid visits the output
// are chosen for the stores (see store_block and the row loop); the MFMA work
// runs underneath the stores.
#include "c3d_internal.h"

namespace c3d {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kMaxSteps = 16;  // K <= 32
constexpr int kChunk = 512;    // output positions per workgroup (4 blocks of 128)
constexpr int kRows = 2;       // output rows per workgroup
constexpr int kMaxE = 12288;   // staged floats per workgroup (48 KB of LDS)

struct K1Args {
    const float* x;
    const float* w;
    const float* bias;
    float* y;
    int64_t N, Cin, Cout;
    int64_t S0, S1S2;   // input rows and row length (S1*S2)
    int64_t O0, J;      // output rows and row length (O1*S2)
    int32_t K, k0n, k1n, d0, d1S2;
    int32_t ocb;        // blocks of 64 output channels
    int32_t R, RL, E;   // staged input rows per workgroup, staged row length, staged floats
    int32_t groups;     // row groups per (n, ocb): ceil(O0 / kRows)
    int32_t chunks;     // position chunks per row: ceil(J / kChunk)
    // staged-box offset of tap k (input channel ic, kernel row k0, kernel column
    // k1): (ic R + k0 d0) RL + k1 d1 S2; entries k >= K repeat entry 0
    int32_t toff[2 * kMaxSteps];
};

// A buffer load whose offset is at least the resource's size touches no
// memory and returns 0; the resources here are below 2^31 bytes.
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Block of 128 output positions.  N tile t's column c is position j0 + 4c + t,
// so after the MFMAs a lane holds 4 consecutive positions of each of its 16
// channels per M tile, and one 16-byte store per channel covers them: lanes
// 0-31 then write 512 contiguous bytes of one channel row and lanes 32-63 of
// another.  Measured on MI355X with stores alone, writing this kernel's 2.6 GB
// output in this shape takes ~0.83-0.93 ms (about 3.1 TB/s, whatever the
// workgroup shape), against 1.19 ms with one 4-byte column per lane; only
// long runs within one channel plane go faster (whole 10 KB rows 0.62 ms).  A
// block of 64 channels cannot provide those runs itself; the row loop below
// makes the workgroups that run at the same time provide them together.
template <bool kBias, bool kVec, bool kFull>
__device__ __forceinline__ void store_block(float* yb, uint32_t ystride, const f32x16 (&acc)[2][4],
                                            const float (&brow)[2][16], int64_t j0, int r, int h, int64_t J,
                                            int64_t Cout, int64_t oc0) {
    const int64_t j = j0 + 4 * r;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int oc = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = kBias ? acc[mt][t][i] + brow[mt][i] : acc[mt][t][i];
            char* dst = reinterpret_cast<char*>(yb) + (size_t)(((uint32_t)oc * ystride + (uint32_t)j) * 4u);
            const bool oc_ok = kFull || oc0 + oc < Cout;
            if (kVec) {
                // J % 4 == 0 and 16-byte aligned rows: a lane's 4 positions are all in or all out
                if (kFull || (oc_ok && j < J)) *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (kFull || (oc_ok && j + t < J)) reinterpret_cast<float*>(dst)[t] = v[t];
            }
        }
}

// A workgroup owns kRows consecutive output rows and a chunk of kChunk
// positions of them.  Everything it reads - R = kRows + (k0-1)d0 rows of
// every input channel, RL = kChunk + (k1-1)d1*S2 positions each - is staged in
// LDS once, before its first output store.  The loop over the chunk's blocks
// then issues no global load: on this GPU loads and stores share one in-order
// counter, so a load waited for after stores would also wait for those stores
// to reach memory, and a wave that must drain its stores every block cannot
// keep the HBM write queue full.  Box elements past the end of an input row or
// below the last input row feed only outputs that are never stored, so their
// loads are merely clamped into the image.
// The box is staged row by row: row pr = (ic, row) of the box starts at a
// uniform element offset of sample n's input, so every load is a buffer load
// at that offset plus the thread's column (one add); four rows' loads are in
// flight before they are written.  Rows past the last input row and columns
// past the end of a row read whatever lies there, and offsets past the end of
// the sample read 0 (the whole offset is in the range-checked operand).
__device__ __forceinline__ void stage(const K1Args& a, const __amdgpu_buffer_rsrc_t& xs, int64_t o0b, int64_t jc0,
                                      float* lds) {
    constexpr int kPB = 4;   // box rows per batch
    constexpr int kCI = 3;   // 256-column steps per row and batch
    const int pairs = (int)a.Cin * a.R;
    for (int c0 = 0; c0 < a.RL; c0 += kCI * kThreads)
        for (int pr0 = 0; pr0 < pairs; pr0 += kPB) {
            float v[kPB][kCI];
#pragma unroll
            for (int pb = 0; pb < kPB; ++pb) {
                const int pr = pr0 + pb < pairs ? pr0 + pb : pairs - 1;
                const int ic = pr / a.R, row = pr - ic * a.R;
                const uint32_t rbase = (uint32_t)((ic * a.S0 + o0b + row) * a.S1S2 + jc0 + c0);
#pragma unroll
                for (int ci = 0; ci < kCI; ++ci)
                    v[pb][ci] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        xs, 4u * (rbase + threadIdx.x + ci * kThreads), 0, 0));
            }
#pragma unroll
            for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
                for (int ci = 0; ci < kCI; ++ci) {
                    const int col = c0 + (int)threadIdx.x + ci * kThreads;
                    if (pr0 + pb < pairs && col < a.RL) lds[(pr0 + pb) * a.RL + col] = v[pb][ci];
                }
        }
}

template <int kSteps, bool kBias, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv_k1last_kernel(
    K1Args a) {
    extern __shared__ float lds[];  // E floats
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, r = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Consecutive workgroup ids go round-robin to the 8 XCDs.  Remapped, each
    // XCD takes runs of kXcdRun consecutive (chunk, row-pair) items and the 8
    // XCDs' runs lie side by side, so the rows an XCD's workgroups write and
    // the input rows they share stay within its L2, while the chip's write
    // front stays one compact region.  On the 3->64 layer of
    // x[16,3,256,256,10]: 0.72 ms without a remap, 0.70 ms with one contiguous
    // run per XCD, 0.69 ms with runs of 10 (5: 0.699, 127: 0.715).  Grids that
    // are not a multiple of 8 runs fall back to one run per XCD.
    constexpr int64_t kXcdRun = 10;
    int64_t b = blockIdx.x;
    const int64_t nb = gridDim.x;
    if (nb % (8 * kXcdRun) == 0) {
        const int64_t k = b >> 3;
        b = (k / kXcdRun) * (8 * kXcdRun) + (b & 7) * kXcdRun + k % kXcdRun;
    } else if ((nb & 7) == 0) {
        b = (b & 7) * (nb >> 3) + (b >> 3);
    }
    const int64_t chunk = b % a.chunks;
    b /= a.chunks;
    const int64_t grp = b % a.groups;
    b /= a.groups;
    const int64_t ocb = b % a.ocb;
    const int64_t n = b / a.ocb;
    const int64_t o0b = kRows * grp;        // first output row of this workgroup
    const int64_t jc0 = chunk * kChunk;     // first position of this workgroup
    const int64_t img = a.Cin * a.S0 * a.S1S2;  // floats per sample
    stage(a, buffer_rsrc(a.x + n * img, (uint32_t)(img * 4)), o0b, jc0, lds);
    __syncthreads();

    // A operand (weights): lane holds W[oc][k] with oc = 64*ocb + 32*mt + r and
    // k = 2s + h (buffer loads at immediate offsets 8s; channels past Cout read
    // 0).  Padding rows k >= K get a zero weight and read a valid staged element.
    float wa[2][kSteps];
    int loff[kSteps];
    const __amdgpu_buffer_rsrc_t ws = buffer_rsrc(a.w, (uint32_t)(a.Cout * a.K * 4));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int oc = 64 * (int)ocb + 32 * mt + r;
        const uint32_t vo = oc < a.Cout ? 4u * (uint32_t)(oc * a.K + h) : kOutside;
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            wa[mt][s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ws, vo + 8u * s, 0, 0));
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const bool kv = 2 * s + h < a.K;
        loff[s] = (h ? a.toff[2 * s + 1] : a.toff[2 * s]) + 128 * wave + 4 * r;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) wa[mt][s] = kv ? wa[mt][s] : 0.f;
    }
    // bias of the 32 output channels whose accumulators this lane holds
    float brow[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t oc = 64 * ocb + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
            brow[mt][i] = (kBias && oc < a.Cout) ? a.bias[oc] : 0.f;
        }
    const bool all_oc = 64 * (ocb + 1) <= a.Cout;
    const uint32_t ystride = (uint32_t)(a.O0 * a.J);  // between output channels
    // The four waves walk the workgroup's rows together: at row step q they
    // take the four consecutive 128-position blocks of row o0b + q, so the
    // workgroup writes 2 KB runs of every channel row at once, and the
    // workgroups of the neighbouring chunks (dispatched together) extend those
    // runs along the row.  With two rows per workgroup the rows being written
    // at any moment span less of each channel plane than with four or eight;
    // on MI355X the 3->64 layer of x[16,3,256,256,10] took 0.72 ms with 2
    // rows, 0.81 ms with 3, 0.82 ms with 4, 0.85 ms with 8 and 0.94 ms with 1
    // (3 staged input rows per output row), against 0.90 ms when each wave
    // owned one of 4 rows.
    const int64_t j0 = jc0 + 128 * wave;
    for (int q = 0; q < kRows; ++q) {
        const int64_t o0 = o0b + q;
        const int qoff = q * a.RL;
        if (o0 >= a.O0) break;  // uniform per workgroup
        if (j0 >= a.J) continue;  // uniform per wave
        float* yb = a.y + ((n * a.Cout + 64 * ocb) * a.O0 + o0) * a.J;
        f32x16 acc[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mt][t][i] = 0.f;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            float bx[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) bx[t] = lds[loff[s] + qoff + t];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[mt][s], bx[t], acc[mt][t], 0, 0, 0);
        }
        if (all_oc && j0 + 128 <= a.J)
            store_block<kBias, kVec, true>(yb, ystride, acc, brow, j0, r, h, a.J, 0, 0);
        else
            store_block<kBias, kVec, false>(yb, ystride, acc, brow, j0, r, h, a.J, a.Cout, 64 * ocb);
    }
}

}  // namespace

bool conv_k1last_supported(const Geom& g, const void*, const void*, const void*) {
    if (g.k[2] != 1 || g.groups != 1) return false;
    for (int j = 0; j < 3; ++j)
        if (g.s[j] != 1 || g.p[j] != 0) return false;
    const int64_t K = g.Cin * g.k[0] * g.k[1];
    const int64_t R = kRows + (int64_t)(g.k[0] - 1) * g.d[0];
    const int64_t RL = kChunk + (int64_t)(g.k[1] - 1) * g.d[1] * g.S[2];
    const int64_t E = g.Cin * R * RL;
    // MFMA pays off with many output channels; K must fit the VGPR-resident
    // weights, the staged box the LDS, and offsets 32 bits
    return K >= 2 && K <= 2 * kMaxSteps && g.Cout >= 16 && E <= kMaxE &&
           g.Cin * g.S[0] * g.S[1] * g.S[2] < (1ll << 28) && g.Cout * K < (1ll << 28) &&
           64 * g.O[0] * g.O[1] * g.S[2] < (1ll << 30);
}

hipError_t launch_conv_k1last(const float* x, const float* w, const float* bias, float* y, const Geom& g,
                              hipStream_t st) {
    K1Args a{};
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.y = y;
    a.N = g.N;
    a.Cin = g.Cin;
    a.Cout = g.Cout;
    a.S0 = g.S[0];
    a.S1S2 = g.S[1] * g.S[2];
    a.O0 = g.O[0];
    a.J = g.O[1] * g.S[2];
    a.K = (int32_t)(g.Cin * g.k[0] * g.k[1]);
    a.k0n = g.k[0];
    a.k1n = g.k[1];
    a.d0 = g.d[0];
    a.d1S2 = (int32_t)(g.d[1] * g.S[2]);
    a.ocb = (int32_t)ceil_div(g.Cout, 64);
    a.R = kRows + (g.k[0] - 1) * g.d[0];
    a.RL = kChunk + (g.k[1] - 1) * a.d1S2;
    a.E = (int32_t)(g.Cin * a.R * a.RL);
    a.groups = (int32_t)ceil_div(g.O[0], kRows);
    a.chunks = (int32_t)ceil_div(a.J, kChunk);
    for (int k = 0; k < 2 * kMaxSteps; ++k) {
        const int kk = k < a.K ? k : 0;
        const int k1 = kk % a.k1n, k0 = (kk / a.k1n) % a.k0n, ic = kk / (a.k1n * a.k0n);
        a.toff[k] = (ic * a.R + k0 * a.d0) * a.RL + k1 * a.d1S2;
    }
    const int64_t blocks = g.N * a.ocb * (int64_t)a.groups * a.chunks;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const int steps = (a.K + 1) / 2;
    const bool vec = (a.J % 4 == 0) && ((uintptr_t)y % 16 == 0);
    const size_t lds_bytes = (size_t)a.E * sizeof(float);
    const dim3 grid((unsigned)blocks), block(kThreads);
#define C3D_K1_LAUNCH(S)                                                                                 \
    do {                                                                                                 \
        if (bias) {                                                                                      \
            if (vec) hipLaunchKernelGGL((conv_k1last_kernel<S, true, true>), grid, block, lds_bytes, st, a);  \
            else hipLaunchKernelGGL((conv_k1last_kernel<S, true, false>), grid, block, lds_bytes, st, a);     \
        } else {                                                                                         \
            if (vec) hipLaunchKernelGGL((conv_k1last_kernel<S, false, true>), grid, block, lds_bytes, st, a); \
            else hipLaunchKernelGGL((conv_k1last_kernel<S, false, false>), grid, block, lds_bytes, st, a);    \
        }                                                                                                \
    } while (0)
    if (steps <= 8) C3D_K1_LAUNCH(8);
    else if (steps <= 14) C3D_K1_LAUNCH(14);
    else C3D_K1_LAUNCH(16);
#undef C3D_K1_LAUNCH
    return hipGetLastError();
}

}  // namespace c3d
