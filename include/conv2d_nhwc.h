/*
 * conv2d_nhwc.h -- C ABI of the MI355X (gfx950) implicit-GEMM NHWC conv2d library.
 *
 * Operations (deep-learning convolution, i.e. cross-correlation without a
 * filter flip, as aten.conv2d computes it in the CUTLASS Python Conv2d
 * notebook, "Declaring and running a Conv2d Fprop"):
 *
 *   fprop  y[n,p,q,k]   = sum_{r,s,c'} x[n, p*sh-ph+r*dh, q*sw-pw+s*dw, g*C/G+c'] * w[k,r,s,c']
 *                         (+ bias[k]) (ReLU) -- then one rounding to the output type
 *   dgrad  dx = gradient of fprop with respect to x, applied to dy
 *          (torch.nn.grad.conv2d_input in the notebook's "Declaring and running
 *          Conv2d Dgrad and Wgrad"; the input extent H,W is passed explicitly)
 *   wgrad  dw = gradient of fprop with respect to w, applied to dy
 *          (torch.nn.grad.conv2d_weight in the same section)
 *
 * Tensor layouts, all dense and row-major (channel-last, as the notebook's
 * "General setup" declares them):
 *   x, dx   [N][H][W][C]        w, dw   [K][R][S][C/G]
 *   y, dy   [N][P][Q][K]        bias    [K]
 * with P = floor((H + 2*pad_h - dil_h*(R-1) - 1) / stride_h) + 1 and likewise Q
 * (the tensorcore Conv2D page's "Surface" formula, extended by the dilated
 * filter span).  Group g owns input channels [g*C/G, (g+1)*C/G) and output
 * channels [g*K/G, (g+1)*K/G).
 *
 * Element types:
 *   CONV2D_DTYPE_F16, CONV2D_DTYPE_BF16: x, w, y, dx, dw, dy and bias in that
 *     type; products accumulate in fp32; the result is rounded once, to nearest
 *     even.  wgrad always accumulates in fp32 (the TVM CUTLASS wgrad pull request
 *     forces fp32 accumulation for wgrad).
 *   CONV2D_DTYPE_I8: fprop only.  x, w, y int8; bias int32 in accumulator
 *     units; int32 accumulation; then + bias, ReLU if set, multiplication by
 *     act_scale*w_scale/out_scale in double precision, rounding half to even
 *     and saturation to [-128, 127] (the op-graph order of the quantized cuDNN
 *     conv, apply_impl_helper on the "kReluFused" page).
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller owns every buffer.  The library never allocates or
 *     frees memory and keeps no mutable global state.  Device pointers must be
 *     16-byte aligned.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Work is
 *     enqueued on it and the call returns after enqueue; results are ready when
 *     the stream is synchronised.
 *   - Errors: every check runs before anything is enqueued; on error no output
 *     byte is written.  An unsupported case is an error, never a silent switch
 *     to another algorithm (the quantized cuDNN conv's hard failure when no
 *     engine can run it).
 *   - Determinism: the same inputs, problem and algo give identical bits on
 *     every run; reductions run in a fixed order, with no atomics on values.
 */
#ifndef CONV2D_NHWC_H
#define CONV2D_NHWC_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (int). */
#define CONV2D_OK                       0
#define CONV2D_ERR_INVALID_ARGUMENT     1  /* bad sizes, P or Q < 1, C%G or K%G != 0, null pointer */
#define CONV2D_ERR_UNSUPPORTED          2  /* dtype/op pair, alignment, channel multiple */
#define CONV2D_ERR_WORKSPACE_TOO_SMALL  3
#define CONV2D_ERR_DEVICE               4  /* a HIP launch failed */
#define CONV2D_ERR_SCRATCH_LIMIT        5  /* conv2d_wgrad_noalloc: the pass needs more than its static scratch */

/* Element types. */
#define CONV2D_DTYPE_F16   0
#define CONV2D_DTYPE_BF16  1
#define CONV2D_DTYPE_I8    2

/* Operations (for the size and plan queries). */
#define CONV2D_OP_FPROP  0
#define CONV2D_OP_DGRAD  1
#define CONV2D_OP_WGRAD  2

/*
 * Problem descriptor: the parameter set the burn CubeCL conv dispatch
 * (ConvOptions: stride, padding, dilation, groups) and the tensorcore
 * tc_conv2d_* surface pass.  All fields are plain ints; padding is symmetric
 * and zero-valued per axis.
 */
typedef struct conv2d_problem {
    int n, c, h, w;          /* input  [N][H][W][C] */
    int k, r, s;             /* filter [K][R][S][C/G] */
    int pad_h, pad_w;        /* >= 0 */
    int stride_h, stride_w;  /* >= 1 */
    int dil_h, dil_w;        /* >= 1 */
    int groups;              /* >= 1, divides C and K */
} conv2d_problem_t;

/*
 * Optional algorithm override (pass NULL for the library's choice).  The
 * CUTLASS Python notebook exposes the same two knobs ("Tile Description",
 * "Split-K") and requires every choice to give the same answer.
 *   tile:    0 = library choice, otherwise 1 + index into the kernel's tile
 *            table (see conv2d_plan_info).  Out-of-range -> UNSUPPORTED.
 *   split_k: 0 = library choice, otherwise the number of slices the wgrad
 *            reduction over N*P*Q is cut into (partials are summed in a
 *            fixed order by a second kernel).  Ignored by fprop and dgrad.
 *            For groups > 1 whose channels per group are not whole 16-byte
 *            vectors (C/G or K/G not a multiple of 8; 16 for int8), tile 1
 *            is the one-thread-per-output direct kernel and tile 2 (when it
 *            applies) the LDS-tiled or depthwise one; other grouped problems
 *            run one implicit GEMM per group on the implicit-GEMM tiles, and
 *            offer the same direct kernels as the tiles after those.
 *            An ungrouped 1x1 problem with stride 1 and no padding (16-bit
 *            types, no linear-combination epilogue; the summed channel count,
 *            C for fprop and K for dgrad, 64, 128 or 256 and the other a
 *            multiple of 64) has the pointwise kernel as tile 6, the
 *            library's choice: a GEMM over pixels whose filter slice stays in
 *            registers.  Its wgrad, when K and C are 64, 128 or 256 with K*C
 *            <= 16384, runs by default on the pointwise wgrad kernel (tile 3;
 *            each of split_k workgroups streams one slice of pixels and
 *            writes one fp32 partial of dw).
 *            A stride-1, dilation-1 3x3 fp16 problem (no
 *            linear-combination epilogue) also offers, as the last tile of
 *            fprop when C = 64 and K % 16 == 0, and of dgrad when K = 64,
 *            C % 16 == 0 and pad <= 2, Winograd F(2x2, 3x3), the faster 3x3
 *            stride-1 path the tensorcore "Conv2D" page plans ("What's not
 *            done in v0.1").  dgrad then needs workspace for the transformed
 *            filter (16*C*K elements).  bf16 problems are not offered it
 *            (its rounding of the transformed operands to bf16 would leave
 *            rms_scaled near 4e-3).  It is never the library's choice: it
 *            rounds the transformed filter and input tiles to fp16 before
 *            the products, so its results differ from the direct sum by a
 *            few units of fp16 rounding of the transformed terms (exact on
 *            integer-valued data whose transforms are exact).
 */
typedef struct conv2d_algo {
    int tile;
    int split_k;
} conv2d_algo_t;

/* What the library will launch for a problem (diagnostics and tests). */
typedef struct conv2d_plan_info {
    int kernel;        /* 1 = implicit GEMM (or band kernel), 2 = direct (groups > 1),
                          3 = Winograd F(2x2,3x3), 4 = few-channel kernels (C or K
                          off the 16-byte grid), 5 = pointwise (1x1, stride 1;
                          fprop, dgrad and wgrad) */
    int tile;          /* index of the tile configuration used (0-based) */
    int num_tiles;     /* number of tile configurations available for this op/dtype */
    int split_k;       /* reduction slices (wgrad), 1 otherwise */
    int phases;        /* dgrad stride phases launched, 1 otherwise */
    size_t workspace_bytes;
} conv2d_plan_info_t;

/*
 * Output extent of fprop (and extent of dy for dgrad / wgrad).
 * P and Q receive floor((H + 2*pad - dil*(R-1) - 1)/stride) + 1 per axis.
 * Returns INVALID_ARGUMENT for non-positive sizes, negative padding, a
 * dilated filter longer than the padded input (P or Q < 1), or groups that do
 * not divide C and K.  P and Q may be NULL.
 */
int conv2d_output_size(const conv2d_problem_t *prob, int *P, int *Q);

/*
 * Workspace bytes the caller must pass to the given op (0 is a valid answer).
 * A pure function of its arguments.  wgrad uses the workspace for fp32
 * split-K partials; dgrad needs none except on the Winograd tile (its
 * transformed filter) and on the implicit-GEMM tiles when a stride phase
 * sums over more than 2048 (filter tap, K channel) pairs (a filter copy laid
 * out for those long rows); the channel-padded path (C or K off the 16-byte
 * grid) for its zero-padded copies.
 * The caller-allocated scratch with a size query is the tensorcore Conv2D
 * page's "Scratch sizing" convention, minus the im2col buffer.
 */
int conv2d_workspace_size(int op, const conv2d_problem_t *prob, int dtype,
                          const conv2d_algo_t *algo, size_t *bytes);

/* The plan the library would run for (op, prob, dtype, algo).  No device work. */
int conv2d_plan_info(int op, const conv2d_problem_t *prob, int dtype,
                     const conv2d_algo_t *algo, conv2d_plan_info_t *info);

/*
 * Forward convolution (tensorcore tc_conv2d_forward; burn conv_forward_nhwc:
 * implicit GEMM for groups == 1, direct convolution otherwise).
 *   x     device, [N][H][W][C], dtype
 *   w     device, [K][R][S][C/G], dtype
 *   bias  device, [K] or NULL; dtype for F16/BF16, int32 for I8
 *   relu  0 or 1
 *   act_scale, w_scale, out_scale  I8 only (finite, > 0); ignored otherwise
 *   y     device, [N][P][Q][K], dtype; overwritten
 *   workspace / workspace_bytes  as conv2d_workspace_size(CONV2D_OP_FPROP, ...)
 */
int conv2d_fprop(const conv2d_problem_t *prob, int dtype,
                 const void *x, const void *w, const void *bias, int relu,
                 double act_scale, double w_scale, double out_scale,
                 void *y, void *workspace, size_t workspace_bytes,
                 const conv2d_algo_t *algo, void *stream);

/*
 * Data gradient (tensorcore tc_conv2d_backward_input; burn conv_data_backward).
 * Every element of dx is written, including positions no output reads (0).
 *   dy  device, [N][P][Q][K], dtype (F16 or BF16)
 *   w   device, [K][R][S][C/G], dtype
 *   dx  device, [N][H][W][C], dtype; overwritten
 * No bias and no ReLU.  Strided problems run one implicit GEMM per stride
 * phase (h mod stride_h, w mod stride_w) in a single launch.
 */
int conv2d_dgrad(const conv2d_problem_t *prob, int dtype,
                 const void *dy, const void *w, void *dx,
                 void *workspace, size_t workspace_bytes,
                 const conv2d_algo_t *algo, void *stream);

/*
 * Weight gradient (tensorcore tc_conv2d_backward_weight; burn
 * conv_weight_backward).  The reduction runs over all N*P*Q output pixels, in
 * fp32, cut into split_k contiguous pixel slices whose fp32 partials are
 * summed in a fixed order by a second kernel (the "parallel" split-K of the
 * CUTLASS notebook's "Split-K" section, made deterministic).  The stride-1
 * 3x3 64-channel path cuts the pixels into row bands instead (one partial
 * per band).
 *   x   device, [N][H][W][C], dtype (F16 or BF16)
 *   dy  device, [N][P][Q][K], dtype
 *   dw  device, [K][R][S][C/G], dtype; overwritten
 */
int conv2d_wgrad(const conv2d_problem_t *prob, int dtype,
                 const void *x, const void *dy, void *dw,
                 void *workspace, size_t workspace_bytes,
                 const conv2d_algo_t *algo, void *stream);

/*
 * conv2d_wgrad without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same problem, arguments, plan, kernels and
 * results (bit for bit) as conv2d_wgrad; the split-K partials go to a static
 * device buffer of CONV2D_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  It calls no allocating
 * routine.
 *   Errors: as conv2d_wgrad, plus CONV2D_ERR_SCRATCH_LIMIT when the plan's
 *   workspace (conv2d_workspace_size) exceeds the buffer; nothing is enqueued
 *   then.  CONV2D_ERR_DEVICE if the buffer's address cannot be found on the
 *   stream's device.
 *   Concurrency: every call on one GPU shares that GPU's buffer, which keeps
 *   the last call's contents.  Calls whose work overlaps on one GPU (two
 *   streams, or two host threads) race and give undefined results; calls in
 *   order on one stream are safe.
 */
#define CONV2D_NOALLOC_SCRATCH_BYTES (64u << 20)
int conv2d_wgrad_noalloc(const conv2d_problem_t *prob, int dtype,
                         const void *x, const void *dy, void *dw,
                         const conv2d_algo_t *algo, void *stream);

/*
 * Linear-combination epilogue of the three passes: the CUTLASS Python
 * notebook runs fprop, dgrad and wgrad as D = alpha * conv + beta * C with a
 * source tensor C of the output's shape ("Run the Conv2d" and the backward
 * sections); wgrad accumulates in fp32 whatever the output type (the TVM
 * pull request "[CUTLASS] Add wgrad support" makes that the rule), which the
 * out_f32 option hands back unrounded.  With an epilogue each output element is, in fp32,
 *   v = alpha * r + beta * C[same element] (+ bias[k] for fprop)
 * (the products rounded to fp32, then added left to right), then ReLU if
 * set (fprop), then one rounding to the output type (none with out_f32),
 * where r is the fp32 result of the pass.  alpha and beta are converted to
 * fp32.  C may alias the output (each element is read before it is written).
 * A NULL epilogue, or alpha = 1, beta = 0, out_f32 = 0, is the plain pass.
 * F16/BF16 only (INT8 -> UNSUPPORTED).  Band kernels have no such epilogue,
 * so fprop/dgrad with alpha != 1 or beta != 0 run on the implicit GEMM; wgrad
 * always applies it in its split-K reduction, so it needs a workspace even
 * for one slice (conv2d_workspace_size_ex).
 */
typedef struct conv2d_epilogue {
    double alpha;    /* finite (|alpha| < 1e30) */
    double beta;     /* finite; 0 ignores c */
    const void *c;   /* device, laid out like the output; required (16-byte aligned) when beta != 0 */
    int out_f32;     /* wgrad only: dw and c are fp32 (the sum is not rounded) */
    void *db;        /* wgrad only, may be NULL: also the bias gradient db[K] = sum of dy over N, P, Q
                        (as conv2d_bias_grad; fp32 with out_f32, else dtype; 16-byte aligned; alpha and
                        beta do not apply to it).  The workspace then also holds its partials. */
} conv2d_epilogue_t;

/* conv2d_workspace_size for a pass with an epilogue (NULL = plain). */
int conv2d_workspace_size_ex(int op, const conv2d_problem_t *prob, int dtype,
                             const conv2d_algo_t *algo, const conv2d_epilogue_t *epi,
                             size_t *bytes);

/* conv2d_fprop with an epilogue (F16/BF16; no int8 requantisation). */
int conv2d_fprop_ex(const conv2d_problem_t *prob, int dtype,
                    const void *x, const void *w, const void *bias, int relu,
                    const conv2d_epilogue_t *epi, void *y,
                    void *workspace, size_t workspace_bytes,
                    const conv2d_algo_t *algo, void *stream);

/* conv2d_dgrad with an epilogue. */
int conv2d_dgrad_ex(const conv2d_problem_t *prob, int dtype,
                    const void *dy, const void *w, const conv2d_epilogue_t *epi, void *dx,
                    void *workspace, size_t workspace_bytes,
                    const conv2d_algo_t *algo, void *stream);

/* conv2d_wgrad with an epilogue; with out_f32 dw is float32 [K][R][S][C/G]. */
int conv2d_wgrad_ex(const conv2d_problem_t *prob, int dtype,
                    const void *x, const void *dy, const conv2d_epilogue_t *epi, void *dw,
                    void *workspace, size_t workspace_bytes,
                    const conv2d_algo_t *algo, void *stream);

/*
 * Bias gradient.  The forward pass adds bias[k] to every output pixel of
 * channel k (the tensorcore Conv2D page, forward algorithm, step 3; the burn
 * conv module's `bias` argument, "added to each channel"), so the gradient of
 * the loss with respect to the bias is the adjoint of that broadcast:
 *   db[k] = sum over n < N, p < P, q < Q of dy[n][p][q][k],
 * summed in fp32 in a fixed order (row slices of the N*P*Q pixels, each in
 * ascending pixel order, then the slices in ascending order), then rounded
 * once to dtype, or handed back as fp32 with out_f32 = 1.  Bit-identical run
 * to run.  Only N, K and P, Q (from the problem) matter; groups do not.
 *   dy  device, [N][P][Q][K], dtype F16/BF16 (INT8 -> UNSUPPORTED), 16-byte aligned
 *   db  device, [K], dtype (fp32 with out_f32), 16-byte aligned; overwritten
 *   workspace / workspace_bytes  as conv2d_bias_grad_workspace_size; fp32
 *       partials [slices][K rounded up to 4]
 * Errors: INVALID_ARGUMENT (bad problem, null dy/db/workspace, out_f32 not
 * 0/1), UNSUPPORTED (dtype, alignment, more than 2^31 - 1 elements of dy),
 * WORKSPACE_TOO_SMALL; nothing is enqueued on error.
 */
int conv2d_bias_grad_workspace_size(const conv2d_problem_t *prob, int dtype, size_t *bytes);
int conv2d_bias_grad(const conv2d_problem_t *prob, int dtype, const void *dy, void *db, int out_f32,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *conv2d_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_NHWC_H */
