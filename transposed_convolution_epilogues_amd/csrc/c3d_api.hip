// c3d_api.hip - the C ABI declared in include/c3d.h: host-side validation,
// output-shape rules, and dispatch to the fast or the generic kernels.
#include <math.h>

#include <mutex>

#include "../../include/c3d.h"
#include "c3d_internal.h"

using c3d::Geom;
using c3d::PoolGeom;

// Scratch of convT_bn_avgpool_noalloc: the BatchNorm partials that the
// allocating entry points keep in the caller's workspace.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code
// never passes the name `scratch` to a kernel (on the host it is only a
// stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[C3D_NOALLOC_SCRATCH_BYTES];

namespace {

// Kernel-variant override of c3d_set_variant.  It is per calling thread, so a
// setting made for an A/B run on one thread never changes the kernels that
// calls from other threads run.
thread_local int t_variant = 0;

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int64_t conv_len(int64_t L, int32_t k, int32_t s, int32_t p, int32_t d) {
    // floor((L + 2p - d(k-1) - 1)/s) + 1  ("Kimi-K2.6 l2_p43", conv output size)
    const int64_t num = L + 2 * (int64_t)p - (int64_t)d * (k - 1) - 1;
    return num < 0 ? 0 : num / s + 1;
}

int64_t convT_len(int64_t L, int32_t k, int32_t s, int32_t p, int32_t d, int32_t op) {
    // (L-1)s - 2p + d(k-1) + op + 1  ("Kimi-K2.6 l1_p77", with dilation)
    return (L - 1) * s - 2 * (int64_t)p + (int64_t)d * (k - 1) + op + 1;
}

c3d_status check_params(const c3d_conv_params* p, bool transposed) {
    for (int j = 0; j < 3; ++j) {
        if (p->kernel[j] < 1 || p->stride[j] < 1 || p->dilation[j] < 1 || p->pad[j] < 0) return C3D_ERR_PARAM;
        if (p->kernel[j] > 64 || p->stride[j] > 1024 || p->dilation[j] > 1024 || p->pad[j] > 65536)
            return C3D_ERR_PARAM;
        if (transposed) {
            const int32_t lim = p->stride[j] > p->dilation[j] ? p->stride[j] : p->dilation[j];
            if (p->output_pad[j] < 0 || p->output_pad[j] >= lim) return C3D_ERR_PARAM;
        } else if (p->output_pad[j] != 0) {
            return C3D_ERR_PARAM;
        }
    }
    if (p->groups < 1) return C3D_ERR_PARAM;
    return C3D_OK;
}

// Resolves and validates the geometry.  No HIP call is made here.
c3d_status resolve(const int64_t xs[5], int64_t cout, const c3d_conv_params* p, bool transposed, Geom* g) {
    if (!xs || !p || !g) return C3D_ERR_NULL;
    c3d_status st = check_params(p, transposed);
    if (st) return st;
    for (int j = 0; j < 5; ++j)
        if (xs[j] < 1 || xs[j] > ((int64_t)1 << 40)) return C3D_ERR_SHAPE;
    // channel counts (and so the per-group counts kept in 32 bits) stay below 2^30
    if (cout < 1 || cout > ((int64_t)1 << 30) || xs[1] > ((int64_t)1 << 30)) return C3D_ERR_SHAPE;
    if (xs[1] % p->groups != 0 || cout % p->groups != 0) return C3D_ERR_SHAPE;
    g->N = xs[0];
    g->Cin = xs[1];
    g->Cout = cout;
    for (int j = 0; j < 3; ++j) {
        g->S[j] = xs[2 + j];
        g->k[j] = p->kernel[j];
        g->s[j] = p->stride[j];
        g->p[j] = p->pad[j];
        g->d[j] = p->dilation[j];
        g->O[j] = transposed ? convT_len(xs[2 + j], p->kernel[j], p->stride[j], p->pad[j], p->dilation[j],
                                         p->output_pad[j])
                             : conv_len(xs[2 + j], p->kernel[j], p->stride[j], p->pad[j], p->dilation[j]);
        if (g->O[j] < 1) return C3D_ERR_SHAPE;
    }
    g->groups = p->groups;
    g->cin_g = (int32_t)(xs[1] / p->groups);
    g->cout_g = (int32_t)(cout / p->groups);
    // total element counts must fit comfortably in int64
    const double outs = (double)g->N * (double)g->Cout * (double)g->O[0] * (double)g->O[1] * (double)g->O[2];
    const double ins = (double)g->N * (double)g->Cin * (double)g->S[0] * (double)g->S[1] * (double)g->S[2];
    if (outs > 9.0e15 || ins > 9.0e15) return C3D_ERR_SHAPE;
    return C3D_OK;
}

c3d_status resolve_pool(const Geom& g, int32_t pool, PoolGeom* pg) {
    if (pool < 1 || pool > 64) return C3D_ERR_PARAM;
    pg->g = g;
    pg->pool = pool;
    for (int j = 0; j < 3; ++j) {
        if (g.O[j] < pool) return C3D_ERR_SHAPE;
        pg->P[j] = (g.O[j] - pool) / pool + 1;  // floor mode
        pg->C[j] = c3d::ceil_div(g.O[j], pool);
    }
    return C3D_OK;
}

c3d_status hip_status(hipError_t e) { return e == hipSuccess ? C3D_OK : C3D_ERR_HIP; }

// Device address of `scratch` on each GPU, looked up once per device (with
// that device current) on the first no-allocation call there.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

c3d_status scratch_on_device(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return C3D_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return C3D_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return C3D_OK;
}

// Kernel choice (the C3D_ALGO_* codes of c3d.h).  Variant 1 forces the
// generic kernels; variant 2 skips the shape-specialised ones (the
// flattened-row conv for (k,k,1) kernels, the sub-lattice kernel of the
// stride-2 dilation-2 transposed conv) so the general fast paths can be
// compared with them; variants 3 and 4 select the second algorithms of the
// ConvT -> BatchNorm -> AvgPool module (swapped sums) and of the transposed
// conv (LDS scatter); for the module the swapped sums are the default and
// variant 3 selects the output-phase classes.
//
// A convolution below 2^19 MAC (the 4->8 channel, 8^3 layer: 442,368) takes
// the one-thread-per-output kernel: the matrix-core engines' workgroup tiles
// (4 x 4 x 32 voxels x 64 channels) would put it on a handful of CUs (that
// layer: 4 workgroups, 31 us), the direct kernel spreads it over all of them.
constexpr double kSmallConvMac = 524288.0;

int conv3d_algo(const Geom& g) {
    const int v = t_variant;
    if (v == 1) return C3D_ALGO_DIRECT;
    const double mac = (double)g.N * (double)g.Cout * (double)g.O[0] * (double)g.O[1] * (double)g.O[2] *
                       (double)g.cin_g * g.k[0] * g.k[1] * g.k[2];
    if (mac < kSmallConvMac) return C3D_ALGO_DIRECT;
    if (v != 2 && c3d::conv_k1last_supported(g, nullptr, nullptr, nullptr)) return C3D_ALGO_K1LAST;
    if (c3d::conv3x3x3_mfma_supported(g, nullptr, nullptr, nullptr)) return C3D_ALGO_MFMA333;
    return C3D_ALGO_DIRECT;
}

// ConvT -> BatchNorm -> AvgPool module: the swapped sums where they apply
// (variants 0 and 4), else the output-phase classes on the matrix cores
// (also variant 2, which skips the shape-specialised path, and variant 3, the
// module's second algorithm), one thread per 4x4x4 cell otherwise or with
// variant 5, generic (variant 1)
int bn_algo(const PoolGeom& pg) {
    const int v = t_variant;
    if (v == 1) return C3D_ALGO_DIRECT;
    if (v != 2 && v != 3 && v != 5 && c3d::convT_bn_swap_supported(pg, nullptr)) return C3D_ALGO_BN_SWAP;
    if (v != 5 && c3d::convT_bn_pool_mfma_supported(pg, nullptr)) return C3D_ALGO_BN_MFMA;
    if (c3d::convT_bn_pool_fast_supported(pg, nullptr)) return C3D_ALGO_BN_CELLS;
    return C3D_ALGO_DIRECT;
}

int convT_algo(const Geom& g) {
    const int v = t_variant;
    if (v == 1) return C3D_ALGO_DIRECT;
    if (v == 4 && c3d::convT_scatter_supported(g)) return C3D_ALGO_SCATTER;
    if (v != 2 && v != 6 && c3d::convT_s2_sublattice_supported(g, nullptr, nullptr, nullptr))
        return C3D_ALGO_SUBLATTICE;
    if (v != 6 && c3d::convT_phasegroup_supported(g)) return C3D_ALGO_PHASE_GROUP;
    if (c3d::convT_phase_mfma_supported(g, nullptr, nullptr, nullptr)) return C3D_ALGO_PHASE;
    return C3D_ALGO_DIRECT;
}

// float64 partials per channel that phase 1 of a training-mode call leaves
// for phase 2, and the workspace bytes the call needs, for kernel `algo`
size_t bn_parts(const PoolGeom& pg, int algo) {
    return algo == C3D_ALGO_BN_MFMA ? c3d::convT_bn_pool_mfma_partials(pg) : c3d::convT_bn_pool_partials(pg, 0);
}

size_t bn_training_bytes(const PoolGeom& pg, int algo) {
    if (algo == C3D_ALGO_BN_SWAP) return c3d::convT_bn_swap_workspace_bytes(pg);
    return bn_parts(pg, algo) * (size_t)pg.g.Cout * 2 * sizeof(double);
}

void write_shape(const Geom& g, int64_t ys[5]) {
    ys[0] = g.N;
    ys[1] = g.Cout;
    for (int j = 0; j < 3; ++j) ys[2 + j] = g.O[j];
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int c3d_set_variant(int variant) {
    const int old = t_variant;
    t_variant = variant;
    return old;
}

c3d_status c3d_probe_mfma_f32(int64_t iters, float* out, int64_t out_len, int64_t* flop, void* stream) {
    if (!out || !flop) return C3D_ERR_NULL;
    if (!aligned4(out)) return C3D_ERR_ALIGN;
    if (iters < 1 || iters > ((int64_t)1 << 24) || out_len < c3d::mfma_probe_out_len()) return C3D_ERR_PARAM;
    *flop = c3d::mfma_probe_flop(iters);
    return hip_status(c3d::launch_mfma_probe(iters, out, (hipStream_t)stream));
}

c3d_status c3d_probe_mfma_valu_f32(int64_t iters, int32_t valu_per_4, float* out, int64_t out_len, int64_t* flop,
                                   void* stream) {
    if (!out || !flop) return C3D_ERR_NULL;
    if (!aligned4(out)) return C3D_ERR_ALIGN;
    if (iters < 1 || iters > ((int64_t)1 << 24) || out_len < c3d::mfma_probe_out_len() ||
        !c3d::mfma_valu_probe_supported(valu_per_4))
        return C3D_ERR_PARAM;
    *flop = c3d::mfma_probe_flop(iters);
    return hip_status(c3d::launch_mfma_valu_probe(iters, valu_per_4, out, (hipStream_t)stream));
}

const char* c3d_status_str(c3d_status status) {
    switch (status) {
        case C3D_OK: return "ok";
        case C3D_ERR_NULL: return "a required pointer is NULL";
        case C3D_ERR_SHAPE:
            return "invalid shape (non-positive dim, channel/groups mismatch, channels above 2^30 or empty output)";
        case C3D_ERR_PARAM: return "invalid parameter (kernel/stride/dilation/padding/output_padding/pool/eps)";
        case C3D_ERR_WORKSPACE: return "workspace missing or too small";
        case C3D_ERR_UNSUPPORTED: return "unsupported request";
        case C3D_ERR_HIP: return "HIP runtime error at launch";
        case C3D_ERR_ALIGN: return "pointer not 4-byte aligned";
        case C3D_ERR_SCRATCH_LIMIT:
            return "the call needs more than the no-allocation entry point's static scratch holds";
        default: return "unknown status";
    }
}

c3d_status c3d_conv3d_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p, int64_t y_shape[5]) {
    if (!y_shape) return C3D_ERR_NULL;
    Geom g;
    c3d_status st = resolve(x_shape, cout, p, false, &g);
    if (st) return st;
    write_shape(g, y_shape);
    return C3D_OK;
}

c3d_status c3d_conv_transpose3d_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                   int64_t y_shape[5]) {
    if (!y_shape) return C3D_ERR_NULL;
    Geom g;
    c3d_status st = resolve(x_shape, cout, p, true, &g);
    if (st) return st;
    write_shape(g, y_shape);
    return C3D_OK;
}

c3d_status c3d_convT_bn_avgpool_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                   int32_t pool, int64_t y_shape[5]) {
    if (!y_shape) return C3D_ERR_NULL;
    Geom g;
    PoolGeom pg;
    c3d_status st = resolve(x_shape, cout, p, true, &g);
    if (st) return st;
    st = resolve_pool(g, pool, &pg);
    if (st) return st;
    y_shape[0] = g.N;
    y_shape[1] = g.Cout;
    for (int j = 0; j < 3; ++j) y_shape[2 + j] = pg.P[j];
    return C3D_OK;
}

c3d_status c3d_conv_maxpool_lse_relu_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                        int32_t pool, int64_t y_shape[5]) {
    if (!y_shape) return C3D_ERR_NULL;
    Geom g;
    PoolGeom pg;
    c3d_status st = resolve(x_shape, cout, p, false, &g);
    if (st) return st;
    st = resolve_pool(g, pool, &pg);
    if (st) return st;
    y_shape[0] = g.N;
    y_shape[1] = 1;
    for (int j = 0; j < 3; ++j) y_shape[2 + j] = pg.P[j];
    return C3D_OK;
}

c3d_status conv3d_fwd(const float* x, const int64_t x_shape[5], const float* w, int64_t cout, const c3d_conv_params* p,
               const float* bias, float* y, void* stream) {
    if (!x || !w || !y) return C3D_ERR_NULL;
    if (!aligned4(x) || !aligned4(w) || !aligned4(y) || !aligned4(bias)) return C3D_ERR_ALIGN;
    Geom g;
    c3d_status st = resolve(x_shape, cout, p, false, &g);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    switch (conv3d_algo(g)) {
        case C3D_ALGO_K1LAST: return hip_status(c3d::launch_conv_k1last(x, w, bias, y, g, s));
        case C3D_ALGO_MFMA333: return hip_status(c3d::launch_conv3x3x3_mfma(x, w, bias, y, g, s));
        default: return hip_status(c3d::launch_conv3d_direct(x, w, bias, y, g, s));
    }
}

c3d_status conv_transpose3d_fwd(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                         const c3d_conv_params* p, const float* bias, float* y, void* stream) {
    if (!x || !w || !y) return C3D_ERR_NULL;
    if (!aligned4(x) || !aligned4(w) || !aligned4(y) || !aligned4(bias)) return C3D_ERR_ALIGN;
    Geom g;
    c3d_status st = resolve(x_shape, cout, p, true, &g);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    switch (convT_algo(g)) {
        case C3D_ALGO_SUBLATTICE: return hip_status(c3d::launch_convT_s2_sublattice(x, w, bias, y, g, s));
        case C3D_ALGO_PHASE_GROUP: return hip_status(c3d::launch_convT_phasegroup(x, w, bias, y, g, s));
        case C3D_ALGO_PHASE: return hip_status(c3d::launch_convT_phase_mfma(x, w, bias, y, g, s));
        case C3D_ALGO_SCATTER: return hip_status(c3d::launch_convT_scatter(x, w, bias, y, g, s));
        default: return hip_status(c3d::launch_convT_gather(x, w, bias, y, g, s));
    }
}

c3d_status c3d_conv3d_algo(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p, int32_t* algo) {
    if (!algo) return C3D_ERR_NULL;
    Geom g;
    const c3d_status st = resolve(x_shape, cout, p, false, &g);
    if (st) return st;
    *algo = conv3d_algo(g);
    return C3D_OK;
}

c3d_status c3d_convT_bn_avgpool_algo(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p, int32_t pool,
                              int32_t* algo) {
    if (!algo) return C3D_ERR_NULL;
    Geom g;
    PoolGeom pg;
    c3d_status st = resolve(x_shape, cout, p, true, &g);
    if (st) return st;
    st = resolve_pool(g, pool, &pg);
    if (st) return st;
    *algo = bn_algo(pg);
    return C3D_OK;
}

c3d_status c3d_conv_transpose3d_algo(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p, int32_t* algo) {
    if (!algo) return C3D_ERR_NULL;
    Geom g;
    const c3d_status st = resolve(x_shape, cout, p, true, &g);
    if (st) return st;
    *algo = convT_algo(g);
    return C3D_OK;
}

size_t convT_bn_avgpool_workspace_bytes(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                        int32_t pool) {
    Geom g;
    PoolGeom pg;
    if (resolve(x_shape, cout, p, true, &g) || resolve_pool(g, pool, &pg)) return 0;
    // two float64 partials (sum, sum of squares) per phase-1 block and channel,
    // or the swapped-sums path's partials, whichever is largest (the kernel
    // choice can change with c3d_set_variant)
    size_t need = c3d::convT_bn_pool_partials(pg, 0) * (size_t)g.Cout * 2 * sizeof(double);
    if (c3d::convT_bn_pool_mfma_supported(pg, nullptr)) {
        const size_t m = c3d::convT_bn_pool_mfma_partials(pg) * (size_t)g.Cout * 2 * sizeof(double);
        need = m > need ? m : need;
    }
    if (c3d::convT_bn_swap_supported(pg, nullptr)) {
        const size_t sw = c3d::convT_bn_swap_workspace_bytes(pg);
        need = sw > need ? sw : need;
    }
    return need;
}

c3d_status convT_bn_avgpool_ex(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                        const c3d_conv_params* p, const float* conv_bias, const float* gamma, const float* beta,
                        float eps, int32_t pool, int32_t training, float momentum, float* running_mean,
                        float* running_var, float* y, void* ws, size_t ws_bytes, float* batch_mean,
                        float* batch_var, void* stream) {
    if (!x || !w || !y || !gamma || !beta) return C3D_ERR_NULL;
    const bool update = running_mean || running_var;
    if (update && !(running_mean && running_var)) return C3D_ERR_NULL;  // both or neither
    if (!training && !update) return C3D_ERR_NULL;                      // eval mode reads them
    if (!aligned4(x) || !aligned4(w) || !aligned4(y) || !aligned4(conv_bias) || !aligned4(gamma) ||
        !aligned4(beta) || !aligned4(batch_mean) || !aligned4(batch_var) || !aligned4(running_mean) ||
        !aligned4(running_var))
        return C3D_ERR_ALIGN;
    if (!(eps > 0.f) || !isfinite(eps)) return C3D_ERR_PARAM;
    if (training && update && !(momentum >= 0.f && momentum <= 1.f)) return C3D_ERR_PARAM;
    Geom g;
    PoolGeom pg;
    c3d_status st = resolve(x_shape, cout, p, true, &g);
    if (st) return st;
    st = resolve_pool(g, pool, &pg);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const int algo = bn_algo(pg);
    if (!training) {
        // eval mode: one pass, the BN affine with the running statistics applied to the pooled values
        const c3d::BnEval ev{gamma, beta, running_mean, running_var, conv_bias, eps};
        switch (algo) {
            case C3D_ALGO_BN_SWAP: return hip_status(c3d::launch_convT_bn_swap(x, w, y, nullptr, pg, ev, nullptr, s));
            case C3D_ALGO_BN_MFMA: return hip_status(c3d::launch_convT_bn_pool_phase1_mfma(x, w, y, nullptr, pg, ev, s));
            case C3D_ALGO_BN_CELLS: return hip_status(c3d::launch_convT_bn_pool_phase1_fast(x, w, y, nullptr, pg, ev, s));
            default: return hip_status(c3d::launch_convT_bn_pool_phase1_direct(x, w, y, nullptr, pg, ev, s));
        }
    }
    if (update && g.N * g.O[0] * g.O[1] * g.O[2] < 2) return C3D_ERR_SHAPE;  // no unbiased variance
    const size_t parts = bn_parts(pg, algo);
    const size_t need = bn_training_bytes(pg, algo);
    if (!ws || ws_bytes < need) return C3D_ERR_WORKSPACE;
    if (((uintptr_t)ws & 7u) != 0) return C3D_ERR_ALIGN;
    const c3d::BnRunning run{update ? running_mean : nullptr, update ? running_var : nullptr, momentum};
    if (algo == C3D_ALGO_BN_SWAP) {
        // the whole module, statistics first, then the normalised pooled sums
        const c3d::BnEval none{nullptr, nullptr, nullptr, nullptr, nullptr, 0.f};
        const c3d::BnSwapTrain tr{conv_bias, gamma, beta, eps, batch_mean, batch_var, run};
        return hip_status(c3d::launch_convT_bn_swap(x, w, y, ws, pg, none, &tr, s));
    }
    double* part = (double*)ws;
    const int64_t nparts = (int64_t)parts;
    const c3d::BnEval none{nullptr, nullptr, nullptr, nullptr, nullptr, 0.f};
    hipError_t e;
    if (algo == C3D_ALGO_BN_MFMA) {
        e = c3d::launch_convT_bn_pool_phase1_mfma(x, w, y, part, pg, none, s);
    } else if (algo == C3D_ALGO_BN_CELLS) {
        e = c3d::launch_convT_bn_pool_phase1_fast(x, w, y, part, pg, none, s);
    } else {
        e = c3d::launch_convT_bn_pool_phase1_direct(x, w, y, part, pg, none, s);
    }
    if (e != hipSuccess) return C3D_ERR_HIP;
    return hip_status(c3d::launch_bn_pool_phase2(y, part, nparts, conv_bias, gamma, beta, eps, batch_mean,
                                                 batch_var, run, pg, s));
}

c3d_status convT_bn_avgpool(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                     const c3d_conv_params* p, const float* conv_bias, const float* gamma, const float* beta,
                     float eps, int32_t pool, float* y, void* ws, size_t ws_bytes, float* batch_mean,
                     float* batch_var, void* stream) {
    return convT_bn_avgpool_ex(x, x_shape, w, cout, p, conv_bias, gamma, beta, eps, pool, 1, 0.f, nullptr, nullptr,
                               y, ws, ws_bytes, batch_mean, batch_var, stream);
}

c3d_status convT_bn_avgpool_noalloc(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                                    const c3d_conv_params* p, const float* conv_bias, const float* gamma,
                                    const float* beta, float eps, int32_t pool, float* y, float* batch_mean,
                                    float* batch_var, void* stream) {
    // the geometry first, so that a request beyond the static scratch is
    // rejected before any HIP call
    Geom g;
    PoolGeom pg;
    c3d_status st = resolve(x_shape, cout, p, true, &g);
    if (st) return st;
    st = resolve_pool(g, pool, &pg);
    if (st) return st;
    if (bn_training_bytes(pg, bn_algo(pg)) > (size_t)C3D_NOALLOC_SCRATCH_BYTES) return C3D_ERR_SCRATCH_LIMIT;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return C3D_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return C3D_ERR_HIP;
        if (sdev != dev) return C3D_ERR_PARAM;  // the scratch looked up is the current device's
    }
    void* ws = nullptr;
    st = scratch_on_device(dev, &ws);
    if (st) return st;
    // the kernels of the allocating entry point, with the scratch as their
    // workspace; phase 1 writes every partial phase 2 reads, so nothing in
    // the scratch has to start at zero
    return convT_bn_avgpool_ex(x, x_shape, w, cout, p, conv_bias, gamma, beta, eps, pool, 1, 0.f, nullptr, nullptr,
                               y, ws, (size_t)C3D_NOALLOC_SCRATCH_BYTES, batch_mean, batch_var, stream);
}

c3d_status conv_maxpool_lse_relu(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                          const c3d_conv_params* p, const float* bias, int32_t pool, float* y, void* stream) {
    if (!x || !w || !y) return C3D_ERR_NULL;
    if (!aligned4(x) || !aligned4(w) || !aligned4(y) || !aligned4(bias)) return C3D_ERR_ALIGN;
    Geom g;
    PoolGeom pg;
    c3d_status st = resolve(x_shape, cout, p, false, &g);
    if (st) return st;
    st = resolve_pool(g, pool, &pg);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (t_variant != 1 && c3d::conv_pool_lse_mfma_supported(pg, x, w))
        return hip_status(c3d::launch_conv_pool_lse_mfma(x, w, bias, y, pg, s));
    return hip_status(c3d::launch_conv_pool_lse_relu_direct(x, w, bias, y, pg, s));
}

}  // extern "C"
#pragma GCC visibility pop
