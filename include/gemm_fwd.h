/*
 * gemm_fwd.h — C ABI of the MI355X (gfx950) forward linear-layer GEMM family.
 *
 * The operations are the forward linear kernels of a transformer training
 * engine, defined on the page "matmul ve matmul_residual — Tiled Matrix
 * Multiply (Forward)" (https://llm.istanbul/learn/tr/03_linear_forward),
 * section "Ne Yapar?":
 *
 *   matmul                        Y = X @ W
 *   matmul_residual               Y = X @ W + R           (R added after the sum)
 *   matmul_residual_swiglu_a      Y = (silu(GATE) * UP) @ W + R
 *   *_w16                         the same with IEEE binary16 weights
 *
 * with silu(x) = x * sigmoid(x) and the sigmoid of the page
 * "ffn_gelu_backward ve ffn_swiglu_backward — FFN Activation Backward"
 * (https://llm.istanbul/learn/tr/09_backward_ffn), section "Türevler / SiLU'".
 * The page branches on the sign of x; the kernels evaluate the same function
 * unbranched, as g * u / (1 + exp(-g)), whose overflow for g < -88.7 gives
 * the correct limit, zero.
 * The SwiGLU combine is applied while the A operand is staged, so the hidden
 * [M x K] matrix is never written ("Önemli Optimizasyonlar" §3 of the first
 * page).
 *
 * Layout.  Every array is dense and row-major with no strides:
 *   X, GATE, UP : [M x K] fp32          W : [K x N] fp32 or binary16
 *   R, Y        : [M x N] fp32
 * W is [in x out] as in the page's "Bind Group ABI" (not PyTorch's
 * [out x in] Linear weight).  Arithmetic: fp32 products and fp32 accumulation
 * on the matrix cores; binary16 weights are widened exactly to fp32 before use.
 *
 * Ownership.  All array pointers are device pointers owned by the caller.  The
 * library never allocates or frees device memory.  A call only enqueues work
 * on `stream` (a hipStream_t; NULL means the null stream) and returns; inputs
 * must stay valid and unmodified, and Y must not be read, until the stream has
 * passed the kernel.  Only Y[i][j] for i < M, j < N is written, and nothing
 * outside the inputs is read.  Results are bitwise reproducible from run to
 * run for the same inputs, shape and configuration.
 *
 * State.  The library holds no mutable state and no device memory of its
 * own: gemm_fwd and gemm_fwd_swiglu take nothing but the arrays, the shape
 * and the stream, and every launch they make reads only the inputs and
 * writes only Y.
 *
 * Workspace (the _ex entry points only).  For small output grids with a long
 * K (e.g. M = 512, K = 3072, N = 768) the fastest configurations split K over
 * two or more workgroups per output tile; their fp32 partial tiles meet in a
 * workspace the caller provides (gemm_opts.workspace, device memory of
 * gemm_opts.workspace_bytes bytes, 256-byte aligned, overlapping no array of
 * the call).  gemm_fwd_workspace_bytes() gives the size a shape needs: a
 * 64 KiB block of per-tile arrival counters (so a split-K configuration
 * takes at most 16384 output tiles; more gives GEMM_ERR_CONFIG) followed by
 * one M x N fp32 slot per split.  The workspace must be zero-filled before
 * its first use; every call that completes leaves the counter block zero
 * again (the slots keep partial tiles, which no later call reads before
 * writing), so one zero-fill serves any number of calls of any shape.  Calls that share a workspace must not overlap in time
 * (enqueue them on one stream, or order them with events); calls on
 * different streams need different workspaces.  Without a workspace, or with
 * one that is too small, the library's own choice takes a configuration that
 * does not split K (the same function within the tolerance, not bit for
 * bit); an explicit split-K configuration then gives GEMM_ERR_WORKSPACE.
 *
 * Errors.  Arguments are validated synchronously before anything is enqueued;
 * on a negative status nothing is launched and Y is untouched.  No exception or
 * abort crosses this interface.  Calls may be made from several host threads.
 *
 * Preconditions (the page's host-side rule that K and N be multiples of 4 for
 * the 16-byte vector loads, "Önemli Optimizasyonlar" §1):
 *   0 <= M < 2^31;  0 <= K < 2^21;  0 <= N < 2^21;  K % 4 == 0;  N % 4 == 0;
 *   fp32 arrays 16-byte aligned; binary16 W 8-byte aligned;
 *   Y overlaps none of the inputs (R included).
 * Degenerate shapes: M == 0 or N == 0 enqueues nothing and returns GEMM_OK;
 * K == 0 gives Y = R (or Y = 0 without a residual).  The pointer of an array
 * with no elements (e.g. X and W when K == 0) may be NULL.
 */
#ifndef GEMM_FWD_H
#define GEMM_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GEMM_OK 0
#define GEMM_ERR_NULL (-1)   /* NULL pointer for a non-empty array (R is required by gemm_fwd_swiglu) */
#define GEMM_ERR_SHAPE (-2)  /* negative or too-large dimension, or K % 4 != 0, or N % 4 != 0 */
#define GEMM_ERR_ALIGN (-3)  /* fp32 array not 16-byte aligned, or binary16 W not 8-byte aligned */
#define GEMM_ERR_DTYPE (-4)  /* unknown flag bits or w_dtype */
#define GEMM_ERR_ALIAS (-5)  /* Y overlaps an input */
#define GEMM_ERR_LAUNCH (-6) /* the HIP runtime reported an error at launch */
#define GEMM_ERR_CONFIG (-7) /* a tile configuration index is out of range, or names a tile that keeps W in
                                registers (suffix _wrN) with binary16 W */
#define GEMM_ERR_WORKSPACE (-8) /* an explicit split-K configuration without a large enough workspace, or a
                                   workspace pointer and size that do not match (NULL with a nonzero size,
                                   or a negative size) */

/* gemm_fwd flags. */
#define GEMM_FLAG_W_F16 0x1u /* W holds IEEE binary16 values; otherwise fp32 */

/* gemm_fwd_swiglu weight types. */
#define GEMM_W_F32 0
#define GEMM_W_F16 1

/*
 * matmul / matmul_residual / matmul_w16 / matmul_residual_w16.
 *   X [M x K] fp32, W [K x N] (fp32, or binary16 with GEMM_FLAG_W_F16),
 *   R [M x N] fp32 or NULL (no residual), Y [M x N] fp32 (output).
 *   Y = X @ W (+ R).
 * Returns GEMM_OK or a negative status.
 */
int gemm_fwd(const float *X, const void *W, const float *R, float *Y,
             int64_t M, int64_t K, int64_t N, uint32_t flags, void *stream);

/*
 * matmul_residual_swiglu_a / matmul_residual_swiglu_a_w16.
 *   GATE, UP [M x K] fp32, W [K x N] (w_dtype GEMM_W_F32 or GEMM_W_F16),
 *   R [M x N] fp32 (required), Y [M x N] fp32 (output).
 *   Y = (silu(GATE) * UP) @ W + R, the combine applied as A is staged.
 * Returns GEMM_OK or a negative status.
 */
int gemm_fwd_swiglu(const float *GATE, const float *UP, const void *W, const float *R, float *Y,
                    int64_t M, int64_t K, int64_t N, int w_dtype, void *stream);

/*
 * Options of the _ex entry points.  Every field has a neutral value: a NULL
 * gemm_opts pointer, or one with config = -1 and everything else 0/NULL,
 * makes an _ex call exactly the plain one.
 *   config          -1: the library's choice; otherwise an index below
 *                   gemm_num_configs() (gemm_bwd_num_configs() for the
 *                   backward products).  Every configuration computes the
 *                   same function; they differ in tile shape and speed, and
 *                   results may differ in the last bits between them.
 *   workspace       device memory for split-K partial tiles, or NULL (see
 *   workspace_bytes "Workspace" above); 256-byte aligned.
 *   start_event     hipEvent_t handles created by the caller, or NULL: the
 *   stop_event      kernel's own start and end are recorded into them, so
 *                   hipEventElapsedTime(start, stop) is the kernel's run time
 *                   without the stream's dispatch latency.  Nothing is
 *                   recorded when the status is negative or when there is
 *                   nothing to launch (an empty output).
 * An out-of-range config gives GEMM_ERR_CONFIG, and so does a forward
 * configuration whose name ends in _wrN (W loaded straight into the compute
 * waves' registers, fp32 only) with binary16 W.
 */
typedef struct gemm_opts {
    int64_t config;
    void *workspace;
    int64_t workspace_bytes;
    void *start_event;
    void *stop_event;
} gemm_opts;

int gemm_fwd_ex(const float *X, const void *W, const float *R, float *Y,
                int64_t M, int64_t K, int64_t N, uint32_t flags, const gemm_opts *opts, void *stream);
int gemm_fwd_swiglu_ex(const float *GATE, const float *UP, const void *W, const float *R, float *Y,
                       int64_t M, int64_t K, int64_t N, int w_dtype, const gemm_opts *opts, void *stream);

/*
 * Timing events for gemm_opts.start_event / stop_event (measurement support,
 * no operation of the pages): HIP events created with
 * hipEventDisableSystemFence.  Recording a default timing event at a
 * kernel's end writes back and invalidates the GPU caches at system scope,
 * which lengthens the timed kernel and holds up the launches after it; these
 * events record the kernel's start and end times without that.  They serve
 * timing only: read them with gemm_timing_elapsed_ms once the stream or the
 * device has been synchronised, never to order work or to make results
 * visible to the host.  The caller owns each event and destroys it with
 * gemm_timing_event_destroy.
 *   gemm_timing_event_create   GEMM_ERR_NULL for a NULL `event`,
 *                              GEMM_ERR_LAUNCH when the runtime refuses.
 *   gemm_timing_elapsed_ms     *ms = stop - start in milliseconds;
 *                              GEMM_ERR_NULL for a NULL argument,
 *                              GEMM_ERR_LAUNCH when either event has not been
 *                              recorded or has not completed.
 *   gemm_timing_event_record   records the event on `stream` (hipStream_t,
 *                              NULL for the null stream) as a marker between
 *                              launches, for entry points that take no
 *                              events; GEMM_ERR_NULL for a NULL `event`,
 *                              GEMM_ERR_LAUNCH when the runtime refuses.
 *   gemm_timing_event_destroy  GEMM_ERR_LAUNCH when the runtime refuses.
 */
int gemm_timing_event_create(void **event);
int gemm_timing_event_record(void *event, void *stream);
int gemm_timing_elapsed_ms(void *start, void *stop, float *ms);
int gemm_timing_event_destroy(void *event);

/*
 * For callers that cannot allocate device memory or hand in a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gemm_fwd_swiglu_ex with the library's choice and a workspace
 * the library holds itself, a file-scope device array of 4 MiB + 64 KiB per
 * GPU, kept until the process ends.  Same arguments, results and errors as
 * gemm_fwd_swiglu; a shape whose split-K would need a larger workspace gives
 * GEMM_ERR_WORKSPACE (the library's choice splits K only for outputs of at
 * most 2^19 elements, which always fit).  Nothing is allocated or freed; the
 * first call on a GPU also enqueues a clear of the array's counter block on
 * `stream`.  Every call on a GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (different streams or host threads) race: order
 * them on one stream, or with events.
 */
int gemm_fwd_swiglu_noalloc(const float *GATE, const float *UP, const void *W, const float *R, float *Y,
                            int64_t M, int64_t K, int64_t N, int w_dtype, void *stream);

/*
 * Bytes of workspace a forward call needs: for `config` (>= 0), or for the
 * library's choice when a workspace is given (config = -1); 0 when that
 * configuration does not split K.  swiglu is 0/1, flags as for gemm_fwd.
 * Returns -1 for bad arguments.
 */
int64_t gemm_fwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int swiglu, uint32_t flags, int config);

/* Backward-product flags. */
#define GEMM_FLAG_ACC 0x2u /* add the product to the output's current contents (the *_acc kernels) */

/*
 * Backward linear family.  The page "matmul ve matmul_residual — Tiled
 * Matrix Multiply (Forward)" names these kernels in section "Ne Yapar?"
 * (matmul_t, matmul_t_acc, matmul_at, matmul_at_acc, matmul_at_swiglu_a,
 * matmul_at_acc_swiglu_a) and defers them to a page that is not available;
 * "ffn_gelu_backward ve ffn_swiglu_backward" (section on the pipeline step)
 * says that they do the GEMM part of the backward FFN.  The operations are
 * read from the names: "t" multiplies by the transposed weight (the input
 * gradient of a linear layer), "at" by the transposed activation (its weight
 * gradient), "_acc" accumulates into the output, "_swiglu_a" recomputes the
 * activation A = silu(GATE) * UP while it is staged, as the forward does.
 * Shapes use the forward's names: M rows (tokens), K inputs, N outputs.
 *
 *   gemm_matmul_t:            dX [M x K]  = dY [M x N] @ W^T,  W the forward's [K x N] weight
 *   gemm_matmul_at:           dW [K x N]  = X^T @ dY,          X [M x K]
 *   gemm_matmul_at_swiglu_a:  dW [K x N]  = (silu(GATE) * UP)^T @ dY,  GATE, UP [M x K]
 *
 * With GEMM_FLAG_ACC the product is added to the output (out = out + product,
 * the output read before it is written); otherwise the output is overwritten.
 * All arrays are fp32, dense and row-major, 16-byte aligned, device pointers
 * owned by the caller; the output overlaps no input.  K % 4 == 0 and
 * N % 4 == 0; M (the contraction of matmul_at) is unrestricted; limits as
 * for gemm_fwd.  An empty output enqueues nothing; an empty contraction
 * writes zeros (or leaves the output unchanged with GEMM_FLAG_ACC).  Flags
 * other than GEMM_FLAG_ACC give GEMM_ERR_DTYPE.  The workspace rules of
 * gemm_fwd_ex apply to the _ex forms below.  Returns GEMM_OK or a negative status, validated before
 * anything is enqueued.
 */
int gemm_matmul_t(const float *dY, const float *W, float *dX, int64_t M, int64_t K, int64_t N, uint32_t flags,
                  void *stream);
int gemm_matmul_at(const float *X, const float *dY, float *dW, int64_t M, int64_t K, int64_t N, uint32_t flags,
                   void *stream);
int gemm_matmul_at_swiglu_a(const float *GATE, const float *UP, const float *dY, float *dW, int64_t M, int64_t K,
                            int64_t N, uint32_t flags, void *stream);

/*
 * Fused SwiGLU backward: dH = dY @ W_down^T (matmul_t of the FFN down-
 * projection, never stored) turned directly into the gradients of the
 * SwiGLU inputs, as "ffn_gelu_backward ve ffn_swiglu_backward — FFN
 * Activation Backward" (sections "Ne Yapar?", "Türevler", "Satır Satır")
 * defines them on dH:
 *   dGATE = nan_guard(dH * UP * silu'(GATE)),  dUP = nan_guard(dH * silu(GATE)),
 *   silu'(x) = s(x) (1 + x (1 - s(x))), s the sign-branched sigmoid, and
 *   nan_guard mapping NaN and infinities to 0.
 * dY [M x N], W [K x N] (the down-projection's forward weight, K = d_ff),
 * GATE, UP, dGATE, dUP [M x K]; fp32, 16-byte aligned.  dGATE and dUP may be
 * the very arrays GATE or UP (each element is read before it is written) but
 * may not overlap anything else or each other.  Otherwise as gemm_matmul_t,
 * without accumulation.  One launch replaces matmul_t plus the element-wise
 * kernel and never writes or reads dH.
 */
int gemm_matmul_t_swiglu_bwd(const float *dY, const float *W, const float *GATE, const float *UP, float *dGATE,
                             float *dUP, int64_t M, int64_t K, int64_t N, void *stream);

/* The backward products with options (gemm_opts above; config indexes the
 * backward table, below gemm_bwd_num_configs()).  The lm_head's input
 * gradient (M = 512, K = 768, N = 16384) splits its long contraction over
 * workgroups when a workspace is given. */
int gemm_matmul_t_ex(const float *dY, const float *W, float *dX, int64_t M, int64_t K, int64_t N, uint32_t flags,
                     const gemm_opts *opts, void *stream);
int gemm_matmul_at_ex(const float *X, const float *dY, float *dW, int64_t M, int64_t K, int64_t N, uint32_t flags,
                      const gemm_opts *opts, void *stream);
int gemm_matmul_at_swiglu_a_ex(const float *GATE, const float *UP, const float *dY, float *dW, int64_t M,
                               int64_t K, int64_t N, uint32_t flags, const gemm_opts *opts, void *stream);
int gemm_matmul_t_swiglu_bwd_ex(const float *dY, const float *W, const float *GATE, const float *UP, float *dGATE,
                                float *dUP, int64_t M, int64_t K, int64_t N, const gemm_opts *opts, void *stream);

/* Bytes of workspace a backward call needs (op 1: matmul_t, 2: matmul_at;
 * M, K, N and swiglu as in the calls above; config as for
 * gemm_fwd_workspace_bytes); -1 for bad arguments. */
int64_t gemm_bwd_workspace_bytes(int op, int64_t M, int64_t K, int64_t N, int swiglu, int config);

/* Number and static names of the backward products' configurations, and the
 * one the library picks for a shape (op 1: matmul_t, 2: matmul_at; M, K, N
 * and swiglu as in the calls above; with_workspace 0/1: whether the call has
 * a large enough workspace; -1 for an unknown op). */
int gemm_bwd_num_configs(void);
const char *gemm_bwd_config_name(int config);
int gemm_bwd_select_config(int op, int64_t M, int64_t K, int64_t N, int swiglu, int with_workspace);

/* Number of tile configurations compiled into the library. */
int gemm_num_configs(void);

/* Static name of a configuration ("BMxBNxBK_..."), or NULL if out of range. */
const char *gemm_config_name(int config);

/* The configuration the library picks for a shape (swiglu, w_f16 and
 * with_workspace are 0/1; with_workspace: whether the call has a large enough
 * workspace). */
int gemm_select_config(int64_t M, int64_t K, int64_t N, int swiglu, int w_f16, int with_workspace);

/* Static text for a status code. */
const char *gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_FWD_H */
