/*
 * c3d.h - C ABI of the MI355X (gfx950) library for the forward pass of 3D
 * convolution and 3D transposed convolution, with fused epilogues.
 *
 * Sources ("page" = a POPCORNBENCH agent transcript, cited by its title):
 *   "Kimi-K2.6 l1_p59"  Conv3d with a (k,k,1) kernel on a depth-last tensor
 *   "Kimi-K2.6 l2_p72"  ConvTranspose3d -> BatchNorm3d -> AvgPool3d -> AvgPool3d
 *   "Kimi-K2.6 l2_p43"  Conv3d -> MaxPool3d -> logsumexp(dim=1) -> ReLU
 *   "Kimi-K2.6 l1_p77"  ConvTranspose3d with stride, padding and dilation
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are contiguous float32 in device memory, allocated and owned by
 *   the caller; the library never allocates, frees or synchronises.
 * - Shapes are int64_t[5] = {N, C, S0, S1, S2} with S2 fastest.  The kernel,
 *   stride, padding and dilation triples apply to S0, S1, S2 in that order.
 *   A depth-last tensor x[N,C,H,W,D] therefore needs no flag: it is S0=H,
 *   S1=W, S2=D, and a (k,k,1) kernel convolves H and W only ("Kimi-K2.6
 *   l1_p59", the passage that settles how PyTorch reads that kernel).
 * - Arguments are validated on the host before anything is launched; on any
 *   error nothing is launched and a non-zero c3d_status is returned.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *   null stream).  A launch failure reported by hipGetLastError maps to
 *   C3D_ERR_HIP.  No exceptions cross the ABI.  Index arithmetic is 64-bit.
 * - The operators keep no process-wide mutable state and may be called from
 *   several threads at once.  The one piece of library state is the kernel
 *   override of c3d_set_variant, which is held per calling thread: it changes
 *   only the kernels of later calls made from the thread that set it.
 * - The C calls cannot see buffer sizes: every buffer must hold at least the
 *   elements its shape (or the shape queries) implies.  The Python binding
 *   checks every tensor against these shapes before it calls in.
 * - Pointers must be 4-byte aligned; 16-byte alignment enables the fast paths.
 */
#ifndef C3D_H
#define C3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    C3D_OK = 0,
    C3D_ERR_NULL = 1,        /* a required pointer is NULL                           */
    C3D_ERR_SHAPE = 2,       /* a dim is non-positive, channels/groups mismatch,     */
                             /* Cin or Cout above 2^30, or an output dim would be < 1 */
    C3D_ERR_PARAM = 3,       /* kernel/stride/dilation < 1, padding < 0, bad output  */
                             /* padding, bad pool window, eps not finite and > 0     */
    C3D_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the query returns  */
    C3D_ERR_UNSUPPORTED = 5, /* valid request outside what the library implements   */
    C3D_ERR_HIP = 6,         /* the HIP runtime reported an error at launch          */
    C3D_ERR_ALIGN = 7,       /* a pointer is not 4-byte aligned                      */
    C3D_ERR_SCRATCH_LIMIT = 8 /* convT_bn_avgpool_noalloc: the call needs more than  */
                             /* its static scratch of C3D_NOALLOC_SCRATCH_BYTES      */
} c3d_status;

/* Convolution hyper-parameters, as in PyTorch's Conv3d / ConvTranspose3d
 * constructors ("Kimi-K2.6 l1_p59", the module signature with stride,
 * padding, dilation, groups and bias; "Kimi-K2.6 l1_p77", the transposed
 * module with output_padding). */
typedef struct {
    int32_t kernel[3];     /* >= 1                                               */
    int32_t stride[3];     /* >= 1                                               */
    int32_t pad[3];        /* >= 0                                               */
    int32_t dilation[3];   /* >= 1                                               */
    int32_t output_pad[3]; /* transposed conv only: 0 <= op < max(stride, dil);  */
                           /* must be 0 for the direct-conv calls                */
    int32_t groups;        /* >= 1, divides both channel counts                  */
} c3d_conv_params;

/* Output shape of conv3d_fwd: per dim floor((S + 2p - d(k-1) - 1)/s) + 1
 * ("Kimi-K2.6 l2_p43", the conv output-size formula).  Writes y_shape on
 * success. */
c3d_status c3d_conv3d_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                         int64_t y_shape[5]);

/* Output shape of conv_transpose3d_fwd: per dim (S-1)s - 2p + d(k-1) + op + 1
 * ("Kimi-K2.6 l1_p77", the output-size formula with dilation). */
c3d_status c3d_conv_transpose3d_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                   int64_t y_shape[5]);

/* Output shape of convT_bn_avgpool: the transposed-conv shape with each
 * spatial dim pooled in floor mode, floor((O - pool)/pool) + 1
 * ("Kimi-K2.6 l2_p72", the AvgPool3d sizes 63 -> 31 -> 15). */
c3d_status c3d_convT_bn_avgpool_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                   int32_t pool, int64_t y_shape[5]);

/* Output shape of conv_maxpool_lse_relu: [N, 1, P0, P1, P2] with the conv
 * shape pooled in floor mode ("Kimi-K2.6 l2_p43", MaxPool3d(2) then the
 * keepdim logsumexp). */
c3d_status c3d_conv_maxpool_lse_relu_out_dims(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                        int32_t pool, int64_t y_shape[5]);

/* Direct 3D convolution ("Kimi-K2.6 l1_p59", the output formula summed over
 * the input channels of the group; "Kimi-K2.6 l2_p43", the per-output sum
 * over c_in and the 3x3x3 window):
 *   y[n,oc,o] = bias[oc] + sum_{icg,k} w[oc,icg,k] * x[n, g*Cin_g + icg, o*s - p + k*d]
 * with g = oc / (Cout/groups) and zero outside x.
 *   x     [N, Cin, S0, S1, S2]                (device, read)
 *   w     [Cout, Cin/groups, k0, k1, k2]      (device, read)
 *   bias  [Cout] or NULL                      (device, read)
 *   y     [N, Cout, O0, O1, O2]               (device, written in full)
 */
c3d_status conv3d_fwd(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
               const c3d_conv_params* p, const float* bias, float* y, void* stream);

/* 3D transposed convolution in its gather form ("Kimi-K2.6 l1_p77", the
 * passages that map input i and tap k to output o = i*s - p + k*d and invert
 * it as i = (o + p - k*d)/s when divisible; "Kimi-K2.6 l2_p72", the same test
 * for stride 2, padding 1):
 *   y[n, g*Cout_g + ocg, o] = bias + sum over ic of group g and taps k with
 *       (o + p - k*d) divisible by s and i = (o + p - k*d)/s inside x
 *       of x[n, ic, i] * w[ic, ocg, k]
 *   x     [N, Cin, S0, S1, S2]                (device, read)
 *   w     [Cin, Cout/groups, k0, k1, k2]      (device, read; PyTorch's layout)
 *   bias  [Cout] or NULL                      (device, read)
 *   y     [N, Cout, O0, O1, O2]               (device, written in full,
 *                                              including positions no tap reaches)
 */
c3d_status conv_transpose3d_fwd(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                         const c3d_conv_params* p, const float* bias, float* y, void* stream);

/* Bytes of device workspace convT_bn_avgpool (and convT_bn_avgpool_ex in
 * training mode) needs for these arguments, whichever kernel
 * c3d_set_variant selects (the largest of their needs); 0 for invalid
 * arguments. */
size_t convT_bn_avgpool_workspace_bytes(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p,
                                        int32_t pool);

/* Transposed conv -> BatchNorm3d with batch statistics -> average pool
 * ("Kimi-K2.6 l2_p72": the module, the training-mode statistics with biased
 * variance, and the proof that two AvgPool3d(2) stages equal one
 * AvgPool3d(4, stride 4)).
 *   t = conv_transpose3d(x, w, conv_bias)           (never written to HBM)
 *   mean_c, var_c = batch mean and biased variance of t[:, c] over N and all
 *                   O0*O1*O2 positions (including those pooling drops)
 *   y[n,c,j] = gamma_c * (avg_{u in [0,pool)^3} t[n,c,pool*j+u] - mean_c)
 *              / sqrt(var_c + eps) + beta_c
 * Pooling is floor mode with window = stride = pool (pool = 4 is the module's
 * two AvgPool3d(2)).
 *   gamma, beta [Cout]                        (device, read; required)
 *   y      [N, Cout, O0/pool, O1/pool, O2/pool] (device, written)
 *   ws     >= convT_bn_avgpool_workspace_bytes(...) bytes (device, scratch;
 *          its contents on entry do not matter)
 *   batch_mean, batch_var [Cout] or NULL      (device, written if given: the
 *          statistics of t including conv_bias; var is the biased one)
 */
c3d_status convT_bn_avgpool(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                     const c3d_conv_params* p, const float* conv_bias, const float* gamma, const float* beta,
                     float eps, int32_t pool, float* y, void* ws, size_t ws_bytes, float* batch_mean,
                     float* batch_var, void* stream);

/* convT_bn_avgpool with the module's running statistics and its eval mode
 * ("Kimi-K2.6 l2_p72": the eval-mode variant the page ships, which folds
 * BatchNorm into the transposed conv and normalises with the running
 * statistics, and BatchNorm3d's momentum of 0.1).
 *   training != 0: as convT_bn_avgpool; if running_mean and running_var are
 *     given (both or neither), they are then updated in place:
 *       running_mean <- (1 - momentum) running_mean + momentum * batch mean
 *       running_var  <- (1 - momentum) running_var
 *                       + momentum * batch var * count / (count - 1)
 *     with count = N*O0*O1*O2 elements per channel (the running variance
 *     tracks the unbiased batch variance, as BatchNorm3d does).  Requires
 *     0 <= momentum <= 1 (C3D_ERR_PARAM) and count >= 2 (C3D_ERR_SHAPE).
 *   training == 0 (eval): running_mean and running_var are required and
 *     read; one kernel writes
 *       y[n,c,j] = gamma_c * (avg_{u in [0,pool)^3} t[n,c,pool*j+u] - running_mean_c)
 *                  / sqrt(running_var_c + eps) + beta_c
 *     with t = conv_transpose3d(x, w, conv_bias) (the map is applied after
 *     the pool, which it commutes with).  ws, ws_bytes, batch_mean and
 *     batch_var are ignored (ws may be NULL).
 *   running_mean, running_var [Cout] or NULL (device, read; written in
 *     training mode)
 * Calls that update the same running buffers must not overlap. */
c3d_status convT_bn_avgpool_ex(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                        const c3d_conv_params* p, const float* conv_bias, const float* gamma, const float* beta,
                        float eps, int32_t pool, int32_t training, float momentum, float* running_mean,
                        float* running_var, float* y, void* ws, size_t ws_bytes, float* batch_mean,
                        float* batch_var, void* stream);

/* Size of the static device scratch convT_bn_avgpool_noalloc uses (per GPU,
 * held until the process ends). */
#define C3D_NOALLOC_SCRATCH_BYTES (4u << 20)

/* convT_bn_avgpool without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, result and kernels as
 * convT_bn_avgpool (training mode, batch statistics) minus ws / ws_bytes:
 * the float64 BatchNorm partials go to a static device array of
 * C3D_NOALLOC_SCRATCH_BYTES that the library owns, one per GPU.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * the first call on a device looks up that device's copy of the array.
 *   stream   must belong to the current device (else C3D_ERR_PARAM).
 *   Errors   as convT_bn_avgpool; C3D_ERR_SCRATCH_LIMIT when the arguments
 *            need more than C3D_NOALLOC_SCRATCH_BYTES of partials (the
 *            module on x[64,3,32,32,32] with 16 channels needs 2.07 MB with
 *            the sums swapped, 256 KiB on the output-phase kernel);
 *            nothing is launched then.
 * All calls on one GPU share its scratch, which keeps the last call's
 * partials: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Nothing in the
 * scratch needs to start at zero: every kernel of the call writes each
 * value that a later one reads. */
c3d_status convT_bn_avgpool_noalloc(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                                    const c3d_conv_params* p, const float* conv_bias, const float* gamma,
                                    const float* beta, float eps, int32_t pool, float* y, float* batch_mean,
                                    float* batch_var, void* stream);

/* Conv3d -> MaxPool3d(pool, stride pool) -> logsumexp over channels
 * (keepdim) -> ReLU ("Kimi-K2.6 l2_p43": the module, floor-mode pooling and
 * the max-shifted logsumexp):
 *   t = conv3d(x, w, bias)                    (never written to HBM)
 *   m[n,c,j] = max_{u in [0,pool)^3} t[n,c,pool*j+u]
 *   y[n,0,j] = max(0, M + log(sum_c exp(m[n,c,j] - M))),  M = max_c m[n,c,j]
 *   y      [N, 1, O0/pool, O1/pool, O2/pool]  (device, written)
 */
c3d_status conv_maxpool_lse_relu(const float* x, const int64_t x_shape[5], const float* w, int64_t cout,
                          const c3d_conv_params* p, const float* bias, int32_t pool, float* y, void* stream);

/* Human-readable name of a status code (static storage). */
const char* c3d_status_str(c3d_status status);

/* Kernel-variant override for A/B tests: 0 = automatic (default), 1 = force
 * the generic direct kernels, 2 = skip the shape-specialised kernels (the
 * flattened-row conv for (k,k,1) kernels and the stride-2/dilation-2
 * sub-lattice transposed conv) so that the general MFMA paths run where
 * they apply (for convT_bn_avgpool: the output-phase classes on the matrix
 * cores instead of the swapped sums), 3 = as 0 but with the second algorithm
 * of convT_bn_avgpool where the swapped sums apply, the output-phase classes
 * on the matrix cores (see c3d_convT_bn_avgpool_algo), 4 = as
 * 0 but conv_transpose3d_fwd scatters into an LDS output tile
 * (C3D_ALGO_SCATTER: "Kimi-K2.6 l1_p77", the scatter form, which needs no
 * atomics within one tap offset because the input-to-output map is
 * injective there; LDS-bound, the second algorithm to compare against),
 * 5 = as 0 but convT_bn_avgpool uses its one-thread-per-cell fp32 kernel
 * (C3D_ALGO_BN_CELLS), 6 = as 0 but conv_transpose3d_fwd takes the
 * one-phase-per-workgroup kernel (C3D_ALGO_PHASE) wherever it applies, for
 * A/B against the kernel that shares a staged halo among the phases.
 * Returns the previous value.  The setting belongs to the calling thread
 * (thread-local): other threads keep their own, starting at 0. */
int c3d_set_variant(int variant);

/* Diagnostic: a throughput probe of the fp32 matrix cores, to check the peak
 * that roofline fractions are quoted against (not part of any operator).
 * Launches 2048 workgroups of 256 threads on the stream; every wave runs
 * 4 independent chains of `iters` back-to-back v_mfma_f32_32x32x2f32
 * (4096 FLOP each).  out: device, >= 524288 floats (one sum per thread, so
 * the work is kept; caller-owned scratch).  *flop (host) receives the FLOP
 * count of the launch.  Errors: C3D_ERR_NULL (out or flop null),
 * C3D_ERR_ALIGN, C3D_ERR_PARAM (iters outside [1, 2^24] or out too short);
 * nothing is launched then.  Time it with events on the same stream. */
c3d_status c3d_probe_mfma_f32(int64_t iters, float* out, int64_t out_len, int64_t* flop, void* stream);

/* Diagnostic: the same probe with valu_per_4 (2, 4, 8 or 16) independent
 * fp32 FMAs on other registers after every 4 MFMAs of a wave, to measure what
 * non-MFMA vector work beside the matrix cores costs them (not part of any
 * operator).  Same launch, out, *flop (MFMA FLOP only) and output values as
 * c3d_probe_mfma_f32.  Errors: as c3d_probe_mfma_f32, and C3D_ERR_PARAM for
 * any other valu_per_4; nothing is launched then. */
c3d_status c3d_probe_mfma_valu_f32(int64_t iters, int32_t valu_per_4, float* out, int64_t out_len, int64_t* flop,
                                   void* stream);

/* Kernel a call would use (under the current variant), for tests and
 * tuning; host-only, launches nothing. */
enum {
    C3D_ALGO_DIRECT = 0,     /* generic one-thread-per-output fp32 kernel              */
    C3D_ALGO_K1LAST = 1,     /* conv3d, (k,k,1) kernel: flattened-row MFMA GEMM        */
    C3D_ALGO_MFMA333 = 2,    /* conv3d, 3x3x3 stride 1: MFMA implicit GEMM             */
    C3D_ALGO_SUBLATTICE = 3, /* conv_transpose3d, k3 s2 p1 d2: odd sub-lattice on MFMA */
    C3D_ALGO_PHASE = 4,      /* conv_transpose3d, strided: per-output-phase MFMA GEMM  */
    C3D_ALGO_BN_CELLS = 5,   /* convT_bn_avgpool, k3 s2 p1 pool 4: a thread per 4^3 cell */
    C3D_ALGO_BN_SWAP = 6,    /* convT_bn_avgpool, k3 s2 p1 pool 4: swapped sums        */
    C3D_ALGO_SCATTER = 7,    /* conv_transpose3d: scatter into an LDS output tile      */
    C3D_ALGO_BN_MFMA = 8,    /* convT_bn_avgpool, k3 s2 p1 pool 4: output phases on MFMA */
    C3D_ALGO_PHASE_GROUP = 9 /* conv_transpose3d, strided: every output phase of a tile
                                from one staged halo, on MFMA                          */
};

/* Writes the C3D_ALGO_* code conv3d_fwd would use to *algo; returns the
 * validation status conv3d_fwd would return (nothing is written on error). */
c3d_status c3d_conv3d_algo(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p, int32_t* algo);

/* The same for conv_transpose3d_fwd.  The phase paths ("Kimi-K2.6 l1_p77",
 * the residue classes of o mod s, each a stride-1 correlation with its own
 * taps) apply when every stride is at most 4, every residue class has at
 * most 3 taps per dim, and Cin/groups >= 4, Cout/groups >= 8.
 * C3D_ALGO_PHASE_GROUP (the default) needs the input offsets of all residues
 * of a dim together to span at most 3 positions and at most 64 kernel taps;
 * C3D_ALGO_PHASE needs the span per residue only. */
c3d_status c3d_conv_transpose3d_algo(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p, int32_t* algo);

/* The same for convT_bn_avgpool and convT_bn_avgpool_ex.  The default for
 * the page's module (kernel 3, stride 2, padding 1, dilation 1, no output
 * padding, pool 4, groups 1) with Cin <= 3 and Cout <= 32 is the swapped-sums
 * path C3D_ALGO_BN_SWAP ("Kimi-K2.6 l2_p72", the proposal to swap the pooled
 * sum and the conv sum): pooled sums from 3x3x3 summed weights on the matrix
 * cores, batch statistics from lag correlations of the input and Gram
 * matrices of its boundary; no transposed-conv output is formed.  The second
 * algorithm (variant 3, and the default for the other Cin <= 4, Cout <= 16
 * shapes) is C3D_ALGO_BN_MFMA: the 8 output-phase classes of [p72]'s parity
 * tables, each a GEMM over Cin x taps on the matrix cores, pooled and squared
 * in registers.  Other Cin <= 4 shapes, or variant 5, take the
 * one-thread-per-cell fp32 kernel (C3D_ALGO_BN_CELLS). */
c3d_status c3d_convT_bn_avgpool_algo(const int64_t x_shape[5], int64_t cout, const c3d_conv_params* p, int32_t pool,
                              int32_t* algo);

#ifdef __cplusplus
}
#endif
#endif /* C3D_H */
