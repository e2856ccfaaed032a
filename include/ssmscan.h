/*
 * ssmscan.h -- C ABI of the MI355X (gfx950) selective state-space scan library.
 *
 * The library computes the input-dependent linear recurrence
 *
 *     h_t = A_t h_{t-1} + b_t,      y_t = C_t . h_t,      t = 0 .. L-1,  h_{-1} = h0,
 *
 * over many independent sequences, forward and backward, for three kinds of
 * transition A_t:
 *
 *   - diagonal real.  SSM_REAL_SELECTIVE forms a_t = exp(delta_t * A) and the
 *     Euler input term b_t = delta_t * x_t * B_t (or the zero-order-hold term
 *     (exp(delta_t A) - 1) / A * x_t * B_t) from a step size delta, as in the
 *     selection-and-discretisation step of the lpnh.cn page "Selective State
 *     Space Models (S3M)", section 1.1.  SSM_REAL_DENSE takes a_t and b_t as
 *     given tensors.
 *   - diagonal complex with shared controls (SPARC page, abstract): two
 *     per-step scalars, retention r_t and phase phi_t, drive every complex mode
 *     m through a_{t,m} = exp(r_t ln(lambda_m) + i phi_t theta_m), with
 *     b_t = u_t and the real readout y_t = Re sum_m c_m h_{t,m}.
 *     SSM_COMPLEX_DENSE takes the complex a_{t,m} as a given tensor (same
 *     recurrence and readout).
 *   - PD (Flash PD-SSM page, section "Neuer Selektionsmechanismus"): per step,
 *     argmax over K scores picks one column-one-hot matrix P from a per-head
 *     dictionary; A_t = P diag(d_t), i.e. h_t[i] = b_t[i] + sum over the
 *     columns j whose one sits in row i of d_t[j] h_{t-1}[j].
 *
 * The scan runs as a chunked (tiled) three-phase computation -- local scans
 * inside chunks, a prefix over chunk summaries, a carry correction -- as the
 * Flash PD-SSM page describes under "Hardwarebewusste Implementierung".  The
 * forward leaves the state entering every chunk of chunk_len steps (the
 * checkpoints); the backward recomputes states tile by tile from them, so the
 * on-chip working set is one chunk and nothing of size O(L * state) is stored
 * (PGF page, abstract: exact analytical derivatives by tiled operator-space
 * evolution instead of a materialised graph).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Memory.   Every pointer is a device pointer the caller owns, except where
 *            noted.  Tensors are dense, row-major, in the shapes stated, with
 *            no padding (the last dimension is contiguous), unless the call's
 *            ssm_layout describes them as strided views.  The library never
 *            allocates device memory; scratch memory is the caller's workspace
 *            `ws` of at least ssm_workspace_bytes() bytes (256-byte aligned),
 *            used only during the call's stream work.  No pointer is kept
 *            after return.
 *  Streams.  All work is enqueued on `stream` (a hipStream_t; NULL is the
 *            legacy default stream).  There is no host synchronisation and no
 *            host<->device copy.  Buffers must stay valid until the stream
 *            work completes.  Calls on different streams must use different
 *            workspaces and outputs.
 *  Outputs.  Outputs are overwritten, never accumulated.  A NULL output (or
 *            gradient) is not computed.  Outputs must not overlap inputs or
 *            each other.
 *  Types.    Accumulation is float32 everywhere.  For SSM_REAL_SELECTIVE the
 *            streamed tensors (delta, x, Bm, C, y, gy and their gradients)
 *            share `dtype` (SSM_F32 or SSM_BF16, bf16 rounded to nearest even
 *            on output); A, h0, h_last, checkpoints and gA are float32.  All
 *            other modes are float32 (complex64 = interleaved float32 re, im).
 *  Errors.   0 (SSM_OK) on success, a negative SSM_ERR_* code otherwise.  The
 *            arguments are validated completely before anything is enqueued;
 *            on error nothing is written.  ssm_last_error_detail() returns a
 *            thread-local description of the last error.  Device faults are
 *            asynchronous and surface at the caller's next synchronisation.
 *  Results.  Mathematically independent of chunk_len; bitwise deterministic
 *            run to run (no floating-point atomics).
 */
#ifndef SSMSCAN_H
#define SSMSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 7: adds SSM_HEAD_SCALAR (head_dim field); 6 added strided views (ssm_layout, the layout fields of ssm_scan_args and
 * pd_scan_args) and the ZOH discretisation (discretization field); 5 added
 * ssm_scan_fwd_noalloc and ssm_roof_probe; 4 added SSM_COMPLEX_DENSE; 3 added
 * ssm_sensitivity_rows and SSM_OP_SENS_ROWS; struct layouts as in 2 */
#define SSM_ABI_VERSION 7

/* status codes */
#define SSM_OK               0
#define SSM_ERR_NULL        -1  /* a required pointer is NULL */
#define SSM_ERR_SHAPE       -2  /* a size is < 1 or inconsistent, K or N out of range */
#define SSM_ERR_DTYPE       -3  /* unknown or unsupported element type for the mode */
#define SSM_ERR_LAYOUT      -4  /* misaligned pointer, or an output overlapping another buffer */
#define SSM_ERR_WORKSPACE   -5  /* workspace NULL or smaller than ssm_workspace_bytes() */
#define SSM_ERR_UNSUPPORTED -6  /* valid request this build does not implement (e.g. chunk_len) */
#define SSM_ERR_DEVICE      -7  /* HIP reported an error while enqueuing */

/* element types of streamed tensors */
#define SSM_F32  0
#define SSM_BF16 1

/* transition kinds of ssm_scan_* */
#define SSM_REAL_SELECTIVE 0
#define SSM_REAL_DENSE     1
#define SSM_COMPLEX_SHARED 2
#define SSM_COMPLEX_DENSE  3  /* complex a_t given; f32 only */
#define SSM_HEAD_SCALAR    4  /* one scalar transition per head of head_dim channels (below) */

/* operation ids for ssm_workspace_bytes */
#define SSM_OP_SCAN_FWD 0
#define SSM_OP_SCAN_BWD 1
#define SSM_OP_IMPULSE  2
#define SSM_OP_PD_FWD   3
#define SSM_OP_PD_BWD   4
#define SSM_OP_COMPLEX_RTRL 5
#define SSM_OP_OUTPUT_SENS  6
#define SSM_OP_SENS_ROWS    7

/* discretisations of SSM_REAL_SELECTIVE (S3M page, section 1.1) */
#define SSM_EULER 0   /* b_t = delta_t x_t B_t (the default)                               */
#define SSM_ZOH   1   /* zero-order hold: b_t[n] = (exp(delta_t A[d,n]) - 1) / A[d,n] x_t B_t[n],
                         delta_t x_t B_t[n] where A[d,n] = 0 (the limit)                     */

/*
 * Strided views.  By default every tensor is dense and row-major in the shape
 * stated for it.  A caller whose tensors are views -- slices of a larger
 * buffer, or inputs expanded (broadcast) along a dimension -- passes an
 * ssm_layout: for every tensor role r whose bit (1 << r) is set in `given`,
 * stride[r] holds the element strides of the role's dimensions, outermost
 * first (entries past the role's rank are ignored); other roles stay dense.
 * Rules (checked before anything is enqueued):
 *   - the innermost stride must be 1 (rank-1 inputs excepted: the per-head
 *     A may have any stride, 0 included), strides are >= 0 -> SSM_ERR_LAYOUT;
 *   - stride 0 (broadcast) is allowed on inputs only; an output's strides
 *     must give distinct elements                        -> SSM_ERR_LAYOUT;
 *   - a role the mode or entry point does not take as a view -> SSM_ERR_UNSUPPORTED.
 * Gradients of a broadcast input are returned per broadcast position (in the
 * expanded shape); the caller sums them over the broadcast dimension.
 *
 * Roles of ssm_scan_args.layout (logical shape; dense strides):
 *   SSM_REAL_SELECTIVE, every entry point:
 *     SSM_V_DELTA, SSM_V_X  (B,D,L)    inputs; any batch / channel stride
 *     SSM_V_A               (D,N)      channel stride 0: one A row for every channel
 *     SSM_V_BM, SSM_V_C     (B,D,L,N)  dense = (L*N, 0, N, 1): B_t, C_t shared by the
 *                                      channels.  A nonzero channel stride (on either)
 *                                      gives every channel its own B_t / C_t
 *                                      (ssm_scan_fwd / _bwd only); gBm and gC are then
 *                                      both (B,D,L,N) dense, per channel, not sums over
 *                                      channels.  Batch stride 0: shared by the batch
 *                                      rows (gBm / gC stay per batch row).
 *   SSM_REAL_SELECTIVE, ssm_scan_fwd / ssm_scan_bwd:
 *     SSM_V_Y, SSM_V_GY, SSM_V_GDELTA, SSM_V_GX (B,D,L) outputs / upstream gradient
 *   SSM_COMPLEX_SHARED, ssm_scan_fwd / ssm_scan_bwd / ssm_complex_rtrl:
 *     SSM_V_R, SSM_V_PHI    (B,H,L)    head stride 0: one control signal for all heads
 *     SSM_V_U               (B,H,L,M)  complex elements (one (re, im) pair = 1)
 *     SSM_V_LAM, SSM_V_THETA, SSM_V_CC (H,M) head stride 0: shared per-mode parameters
 * Roles of pd_scan_args.layout:
 *     SSM_V_LOGITS          (B,H,L,K)
 *     SSM_V_PD_D, SSM_V_PD_B, SSM_V_PD_C (B,H,L,N)
 *     SSM_V_DICT            (H,K,N)    head stride 0: one dictionary for every head
 */
#define SSM_V_DELTA   0
#define SSM_V_X       1
#define SSM_V_A       2
#define SSM_V_BM      3
#define SSM_V_C       4
#define SSM_V_Y       5
#define SSM_V_GY      6
#define SSM_V_GDELTA  7
#define SSM_V_GX      8
#define SSM_V_R       9
#define SSM_V_PHI    10
#define SSM_V_U      11
#define SSM_V_LAM    12
#define SSM_V_THETA  13
#define SSM_V_CC     14
#define SSM_V_LOGITS 15
#define SSM_V_PD_D   16
#define SSM_V_PD_B   17
#define SSM_V_PD_C   18
#define SSM_V_DICT   19
#define SSM_V_COUNT  20
typedef struct {
    uint64_t given;                    /* bit r: stride[r] describes role r */
    int64_t  stride[SSM_V_COUNT][4];   /* element strides, outermost dimension first */
} ssm_layout;

/*
 * Arguments of the diagonal scans.  Sizes: batch = B; channels = D (real) or
 * H heads (complex); length = L; state = N (real, 1..16) or M complex modes
 * per head (complex, 1..64).  chunk_len = checkpoint interval T in steps:
 * 0 picks the default (256 selective, 32 dense and complex); the selective
 * mode accepts 64, 128 or 256, the dense and complex modes 32.
 * n_chunks = ceil(L / T).  batch, channels and length may be 0 (an empty
 * problem): nothing is read, outputs with no elements are not touched (their
 * pointers may be NULL), h_last becomes h0 (or 0), gh0 becomes gh_last (or 0)
 * and the parameter gradients 0 (gBm and gC, sums over channels, are zero when
 * channels is 0 and batch, length are not); the sensitivity calls still need
 * 0 <= t_out < L.  state must be >= 1.
 */
typedef struct {
    int32_t mode;      /* SSM_REAL_SELECTIVE, SSM_REAL_DENSE, SSM_COMPLEX_SHARED or SSM_COMPLEX_DENSE */
    int32_t dtype;     /* SSM_F32 or SSM_BF16 (bf16: SSM_REAL_SELECTIVE and SSM_COMPLEX_SHARED) */
    int64_t batch, channels, length, state, chunk_len;
    /* SSM_REAL_SELECTIVE */
    const void*  delta;  /* (B,D,L) dtype, step sizes                      */
    const void*  x;      /* (B,D,L) dtype, inputs                          */
    const float* A;      /* (D,N)  f32, continuous-time diagonal (A < 0)   */
    const void*  Bm;     /* (B,L,N) dtype, input projection B_t (shared over D) */
    /* SSM_REAL_DENSE */
    const float* a;      /* (B,D,L,N) f32, transition diagonal a_t;
                            SSM_COMPLEX_DENSE: (B,H,L,M) complex64 a_{t,m}  */
    const float* b;      /* (B,D,L,N) f32, input term b_t                   */
    /* both real modes */
    const void*  C;      /* (B,L,N) dtype (f32 for dense), readout C_t (shared over D) */
    /* SSM_COMPLEX_SHARED (SSM_COMPLEX_DENSE reads u, c and a instead of r, phi, lam, theta) */
    const void*  r;      /* (B,H,L) dtype retention control r_t            */
    const void*  phi;    /* (B,H,L) dtype phase control phi_t              */
    const float* lam;    /* (H,M) baseline rate, 0 < lambda <= 1           */
    const float* theta;  /* (H,M) baseline frequency                       */
    const void*  u;      /* (B,H,L,M) input b_t = u_t: (re, im) pairs of dtype (complex64 for f32) */
    const float* c;      /* (H,M) complex64 readout                        */
    /* all modes */
    const float* h0;     /* nullable initial state (B,D,N) f32 / (B,H,M) complex64; NULL = 0 */
    /* SSM_REAL_SELECTIVE: step sizes from the input projection, with the
     * discretisation merged into the scan (S3M page, sections 1.1 and 4.1):
     * when delta_bias is non-NULL or delta_softplus is 1, delta holds the
     * projection output z and the scan uses delta = softplus(z + delta_bias[d])
     * (softplus(v) = log(1 + e^v)), or z + delta_bias[d] without softplus;
     * gdelta is then the gradient w.r.t. z.  Both off: delta is used as given. */
    const float* delta_bias;  /* nullable (D) f32 */
    int32_t delta_softplus;   /* 0 or 1 */
    int32_t discretization;   /* SSM_REAL_SELECTIVE: SSM_EULER (0) or SSM_ZOH (ssm_scan_fwd,
                                 ssm_scan_bwd, ssm_scan_fwd_noalloc); other modes: 0 */
    const ssm_layout* layout; /* nullable: strided views (above); NULL = every tensor dense */
    /* SSM_HEAD_SCALAR: channels per head P (16, 32, 48 or 64; channels = H * P).
     * The selective scan with one scalar transition per head, as in the S3M
     * page's matrix form (section 4.1): head h owns channels d = h*P .. h*P+P-1,
     *   a_t = exp(delta[b,h,t] * A[h]),  h_t[d,n] = a_t h_{t-1}[d,n] + delta[b,h,t] x[b,d,t] Bm[b,t,n],
     *   y[b,d,t] = sum_n C[b,t,n] h_t[d,n].
     * Tensors: delta (B,H,L) dtype, x (B,D,L) dtype, A (H) f32, Bm, C (B,L,N)
     * dtype (shared by the channels), h0 (B,D,N); state N in {16, 32, 48, 64};
     * chunk_len 0 or 64.  Forward and backward run the chunked matrix form on
     * the matrix cores (the backward is its exact adjoint, from the 64-step
     * checkpoints or a recompute of them).  Gradients: gdelta
     * (B,H,L) dtype, gx (B,D,L), gA (H) f32, gBm, gC (B,L,N), gh0.  Views:
     * SSM_V_DELTA is (B,H,L), SSM_V_A (H); Bm and C are shared by the channels.
     * No step-size transform, no ZOH.  Other modes: 0. */
    int64_t head_dim;
} ssm_scan_args;

typedef struct {
    void*  y;        /* nullable (B,D,L) dtype (dense: f32)                                */
    float* h_last;   /* nullable h_{L-1}: (B,D,N) f32 / (B,H,M) complex64                  */
    float* ckpt;     /* nullable (B,D,n_chunks,N) f32 / (B,H,n_chunks,M) complex64:
                        ckpt[.., c, :] = state entering chunk c (h_{cT-1}; c = 0 holds h0) */
} ssm_scan_fwd_out;

typedef struct {
    const void*  gy;       /* (B,D,L) dtype (dense: f32): dLoss/dy                        */
    const float* gh_last;  /* nullable dLoss/dh_{L-1}, same layout as h_last; NULL = 0    */
    const float* ckpt;     /* nullable checkpoints from ssm_scan_fwd with the same args;
                              NULL = recomputed into the workspace                         */
} ssm_scan_bwd_in;

/* Gradients of Loss = sum_t <gy_t, y_t> + <gh_last, h_{L-1}>; every pointer
 * nullable.  Complex gradients use the real-pair convention
 * g = dLoss/dRe + i dLoss/dIm (interleaved).  SSM_COMPLEX_DENSE writes ga,
 * gu, gc and gh0 only (the other pointers are ignored). */
typedef struct {
    void*  gdelta;  /* selective (B,D,L) dtype; SSM_HEAD_SCALAR (B,H,L) */
    void*  gx;      /* selective (B,D,L) dtype                  */
    float* gA;      /* selective (D,N) f32 (sum over b and t); SSM_HEAD_SCALAR (H) */
    void*  gBm;     /* selective (B,L,N) dtype (sum over d); (B,D,L,N) for a per-channel Bm */
    float* ga;      /* dense (B,D,L,N) f32; complex dense (B,H,L,M) complex64 */
    float* gb;      /* dense (B,D,L,N) f32                      */
    void*  gC;      /* real (B,L,N) dtype (sum over d); (B,D,L,N) for a per-channel C */
    void*  gu;      /* complex (B,H,L,M) (re, im) pairs of dtype */
    void*  gr;      /* complex (B,H,L) dtype                    */
    void*  gphi;    /* complex (B,H,L) dtype                    */
    float* glam;    /* complex (H,M) f32 (sum over b and t)     */
    float* gtheta;  /* complex (H,M) f32 (sum over b and t)     */
    float* gc;      /* complex (H,M) complex64                  */
    float* gh0;     /* (B,D,N) f32 / (B,H,M) complex64          */
    float* gdelta_bias;  /* selective (D) f32, sum over b and t (bias taken as 0 if delta_bias is NULL) */
} ssm_scan_grads;

/* Arguments of the PD scan.  N = state (1..16), K = dictionary size (1..64).
 * chunk_len: 0 = default 64; only 64 is accepted.  dtype: element type of the
 * streams (logits, d, b, C, and gy, ste_logits, y, gd, gb, gC, glogits of the
 * calls below), SSM_F32 or SSM_BF16; h0, h_last, gh_last, gh0 and checkpoints
 * are always f32, and the recurrence runs in fp32 either way.  batch, heads and
 * length may be 0 (an empty problem: h_last = h0 or 0, gh0 = gh_last or 0,
 * nothing else is touched). */
typedef struct {
    int64_t batch, heads, length, state, dict_size, chunk_len;
    const void*    logits; /* (B,H,L,K) dtype selection scores; may be NULL if sel is given */
    const int32_t* sel;    /* (B,H,L) selected entries; input alternative to logits (used
                              when logits is NULL); values must lie in [0,K) (values outside
                              are a precondition violation: every pass clamps them to
                              [0,K), and pd_scan_fwd reports the clamped selection)        */
    const int32_t* dict;   /* (H,K,N): dict[h,k,j] = row of the one in column j of entry k,
                              values in [0,N) (outside: clamped to [0,N) by every pass)    */
    const void*  d;        /* (B,H,L,N) dtype diagonal d_t                                  */
    const void*  b;        /* (B,H,L,N) dtype input term b_t                                */
    const void*  C;        /* (B,H,L,N) dtype readout C_t                                   */
    const float* h0;       /* nullable (B,H,N) f32                                          */
    int32_t dtype;         /* SSM_F32 or SSM_BF16                                           */
    const ssm_layout* layout;  /* nullable: strided views (roles above); NULL = dense       */
} pd_scan_args;

typedef struct {
    void*    y;       /* nullable (B,H,L) dtype                                         */
    int32_t* sel;     /* nullable (B,H,L): argmax_k logits (lowest index among ties)    */
    float*   h_last;  /* nullable (B,H,N)                                               */
    float*   ckpt;    /* nullable (B,H,n_chunks,N): state entering each chunk           */
} pd_scan_fwd_out;

typedef struct {
    const void*  gy;       /* (B,H,L) dtype                                             */
    const float* gh_last;  /* nullable (B,H,N)                                          */
    const float* ckpt;     /* nullable checkpoints from pd_scan_fwd; NULL = recomputed  */
    const void*  ste_logits; /* (B,H,L,K) dtype selection scores for glogits; required
                                when glogits is wanted, ignored otherwise                */
    float tau;             /* softmax temperature of glogits (> 0, finite)              */
} pd_scan_bwd_in;

/* Gradients with the selection held fixed (argmax is piecewise constant), and
 * optionally the straight-through surrogate gradient of the selection scores
 * (Flash PD-SSM page, gradient propagation: hard argmax in the forward pass, a
 * tempered softmax in its place in the backward pass).  Reading: the
 * transition is sum_k w_k P_k diag(d_t) with w one-hot at the selected entry;
 *   gw[t,k] = dLoss/dw_{t,k} = sum_j lambda_t[dict[h,k,j]] d_t[j] h_{t-1}[j]
 * (lambda_t = dLoss/dh_t of the hard forward) and
 *   glogits[t,k] = (1/tau) s_k (gw[t,k] - sum_i s_i gw[t,i]),
 *   s = softmax(ste_logits[t,:] / tau). */
typedef struct {
    void*  gd;       /* (B,H,L,N) dtype */
    void*  gb;       /* (B,H,L,N) dtype */
    void*  gC;       /* (B,H,L,N) dtype */
    float* gh0;      /* (B,H,N) f32     */
    void*  glogits;  /* (B,H,L,K) dtype surrogate gradient of the scores; NULL = not wanted
                        (with bf16 streams: K <= 16)                                    */
} pd_scan_grads;

/* Workspace size in bytes for operation `op` (SSM_OP_*) with `args`
 * (ssm_scan_args* for the ssm_* ops, pd_scan_args* for the pd_* ops).
 * Host-only; enqueues nothing.  Errors as for the operation itself. */
int ssm_workspace_bytes(int op, const void* args, size_t* out_bytes);

/* Forward scan: y, h_last and checkpoints (each nullable). */
int ssm_scan_fwd(const ssm_scan_args* args, const ssm_scan_fwd_out* out,
                 void* ws, size_t ws_bytes, void* stream);

/* Allocation-free variant of ssm_scan_fwd, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, outputs,
 * results (bit for bit) and errors as ssm_scan_fwd, with the workspace taken
 * from a static device array of SSM_NOALLOC_SCRATCH_BYTES bytes that every
 * device the library runs on holds until the process ends.  Every diagonal,
 * dense and complex forward fits it (at most about 25 MB: complex mode,
 * M = 64, a few thousand sequences).  The SSM_HEAD_SCALAR forward keeps its
 * chunk states there, 4 * B * D * N * ceil(L / 64) bytes plus
 * 4 * B * H * ceil(L / 64): a need beyond the array is refused with
 * SSM_ERR_WORKSPACE before anything is enqueued.  The call allocates nothing.  Calls that overlap on
 * one device (different streams, or different threads) share the array and
 * race: serialise them.  On first use on a device the call looks up the
 * array's device address (hipGetSymbolAddress). */
#define SSM_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int ssm_scan_fwd_noalloc(const ssm_scan_args* args, const ssm_scan_fwd_out* out, void* stream);

/* Exact backward of ssm_scan_fwd by tiled recompute from the checkpoints and a
 * reverse adjoint scan lambda_t = C_t gy_t + A_{t+1}^T lambda_{t+1}. */
int ssm_scan_bwd(const ssm_scan_args* args, const ssm_scan_bwd_in* in,
                 const ssm_scan_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* Impulse-response sensitivity of a selective real scan (PGF page, abstract:
 * sensitivity analysis on a 128,000-step impulse-response benchmark):
 *   s[b,d,t] = d y[b,d,t_out] / d x[b,d,t]
 *            = delta_t sum_n Bm[b,t,n] C[b,t_out,n] exp(A[d,n] sum_{s=t+1..t_out} delta_s)
 * for t <= t_out and 0 for t > t_out, by reverse costate evolution in tiles
 * (workspace O(n_chunks), no checkpoints).  t_out in [0,L); -1 means L-1.
 * y (nullable, (B,D,L) dtype) additionally receives the forward output.
 * s is (B,D,L) dtype.  SSM_REAL_SELECTIVE only. */
int ssm_impulse_sensitivity(const ssm_scan_args* args, int64_t t_out, void* y, void* s,
                            void* ws, size_t ws_bytes, void* stream);

/* Forward-mode (real-time recurrent) gradients of the complex mode w.r.t. its
 * per-mode parameters (SPARC page, abstract: exact structured real-time
 * recurrent learning for online credit assignment).  Carries the state
 * sensitivities S^lambda_t = dh_t/dlambda and S^theta_t = dh_t/dtheta forward
 * with the state:
 *   S^lambda_t = a_t S^lambda_{t-1} + (r_t / lambda) a_t h_{t-1},
 *   S^theta_t  = a_t S^theta_{t-1}  + i phi_t a_t h_{t-1}   (S_{-1} = 0),
 * and accumulates, for Loss = sum_t gy_t y_t + <gh_last, h_{L-1}>,
 *   glam[h,m]   = sum_{b,t} gy_t Re(c_m S^lambda_t) + <gh_last, S^lambda_{L-1}>,
 *   gtheta[h,m] = the same with S^theta.
 * The results equal ssm_scan_bwd's glam and gtheta up to rounding; no
 * checkpoints or reverse pass.  args: mode SSM_COMPLEX_SHARED (the
 * ssm_scan_fwd argument rules).  gy: (B,H,L) dtype, required.  gh_last:
 * nullable (B,H,M) complex64, real-pair convention.  y: nullable (B,H,L) dtype,
 * receives the forward output.  glam, gtheta: nullable (H,M) f32, overwritten.
 * Segments of the sequence run in parallel (workspace from
 * ssm_workspace_bytes(SSM_OP_COMPLEX_RTRL, ...)).  Errors as for ssm_scan_fwd;
 * SSM_ERR_UNSUPPORTED for another mode. */
int ssm_complex_rtrl(const ssm_scan_args* args, const void* gy, const float* gh_last, void* y,
                     float* glam, float* gtheta, void* ws, size_t ws_bytes, void* stream);

/* Sensitivity of one output of a selective real scan to the inputs and to the
 * step sizes (PGF page, abstract: sensitivities of the SSM dynamics), with the
 * reverse costate mu_t = C[b,t_out,:] prod_{s=t+1..t_out} a_s in closed form:
 *   s_x[b,d,t]     = d y[b,d,t_out] / d x[b,d,t]     = delta_t sum_n Bm[b,t,n] mu_t[n],
 *   s_delta[b,d,t] = d y[b,d,t_out] / d delta[b,d,t]
 *                  = sum_n mu_t[n] (A[d,n] a_t[n] h_{t-1}[n] + x_t Bm[b,t,n]),
 * t <= t_out, 0 after; h_{t-1} are the forward states (from h0).  With N = 16,
 * the Euler term, shared Bm and C and a sequence the call cuts into segments
 * the forward's main pass forms both sensitivities from the states it re-runs
 * (workspace as for ssm_impulse_sensitivity); otherwise a separate pass
 * recomputes the states per tile from checkpoints the call writes into its
 * workspace (O(n_chunks * N) per sequence).  t_out in [0,L); -1 means
 * L-1.  y, s_x nullable, s_delta required; all (B,D,L) dtype.  With delta_bias or
 * delta_softplus set, s_delta is the sensitivity to the projection output z.
 * SSM_REAL_SELECTIVE only; workspace from ssm_workspace_bytes(SSM_OP_OUTPUT_SENS, ...). */
int ssm_output_sensitivity(const ssm_scan_args* args, int64_t t_out, void* y, void* s_x, void* s_delta,
                           void* ws, size_t ws_bytes, void* stream);

/* Rows of the input Jacobian of the selective scan (PGF page, abstract:
 * sensitivities of outputs to inputs by reverse costate evolution, O(chunk)
 * working memory).  For the R consecutive output steps tau_r = t_out0 + r:
 *   s[r,b,d,t] = d y[b,d,tau_r] / d x[b,d,t]
 *              = delta_t sum_n B_t[n] C_{tau_r}[n] prod_{t < u <= tau_r} a_u[n]  (t <= tau_r), 0 after,
 * i.e. per channel the (R x L) block of the Jacobian.  One call costs one
 * exp per (t, n) for all R rows: the product is split at t_out0 into the
 * costate of row t_out0 and a per-row weight.  s[r] equals
 * ssm_impulse_sensitivity's s at t_out = tau_r up to rounding.
 * args: mode SSM_REAL_SELECTIVE, chunk_len 0 or 64 (64-step tiles); the step
 * transform (delta_bias, delta_softplus) applies as in ssm_scan_fwd, and s is
 * then still the sensitivity to x.  rows in [1, 16]; 0 <= t_out0 and
 * t_out0 + rows <= L.  s: (rows,B,D,L) dtype, required, every element written.
 * Workspace from ssm_workspace_bytes(SSM_OP_SENS_ROWS, ...) (sized for 16
 * rows).  Errors: SSM_ERR_SHAPE for rows or t_out0 out of range,
 * SSM_ERR_UNSUPPORTED for another mode or chunk_len, otherwise as for
 * ssm_scan_fwd. */
int ssm_sensitivity_rows(const ssm_scan_args* args, int64_t t_out0, int32_t rows, void* s,
                         void* ws, size_t ws_bytes, void* stream);

/* PD forward: selection (argmax of logits unless sel is given), scan, readout. */
int pd_scan_fwd(const pd_scan_args* args, const pd_scan_fwd_out* out,
                void* ws, size_t ws_bytes, void* stream);

/* PD backward with the selection from args->sel (or recomputed from logits). */
int pd_scan_bwd(const pd_scan_args* args, const pd_scan_bwd_in* in,
                const pd_scan_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* Diagnostics: per-kernel timing with HIP events.  After ssm_profile_begin(n)
 * every kernel the entry points enqueue from this thread is bracketed by two
 * HIP events recorded on the same stream (at most n kernels; later ones are
 * not recorded).  ssm_profile_end waits for the last event, writes up to
 * `capacity` per-kernel durations in milliseconds and static kernel names,
 * sets *n_launches to the number recorded, and stops recording.  The events
 * are created by the library and kept for reuse until the process ends. */
int ssm_profile_begin(int max_launches);
int ssm_profile_end(int* n_launches, float* ms, const char** names, int capacity);

/* Diagnostics: issue rate of one VALU instruction class, measured on the
 * device (the arithmetic ceiling the scan kernels' roofline is taken against).
 * Launches `waves` one-wave workgroups (waves / (4 x compute units) waves per
 * SIMD), every lane running `chains` (4 or 8) independent dependency chains of
 * iters x 8 instructions of class `kind`: 0 v_fma_f32 (VOP3), 1 v_mul_f32,
 * 2 v_exp_f32, 3 v_fmac_f32 with a DPP row_shr source (4 chains only),
 * 4 v_permlane32_swap, 5 v_permlane16_swap, 6 v_add_f32, 7 v_fmac_f32 (VOP2,
 * accumulating into its addend; 8 chains only).  Times the launch
 * with two HIP events on `stream`, waits for it, and writes lane operations
 * per second (64 x waves x instructions per lane / seconds).  `sink` is a
 * device buffer of waves x 64 floats that is never written in practice (it
 * keeps the chains live).  Synchronises with the stream. */
int ssm_roof_probe(int kind, int chains, int waves, int iters, float* sink, double* lane_ops_per_s,
                   void* stream);

const char* ssm_status_string(int status);   /* static string for a status code */
const char* ssm_last_error_detail(void);     /* thread-local detail of the last error */
int ssm_abi_version(void);                   /* SSM_ABI_VERSION of the built library */

#ifdef __cplusplus
}
#endif

#endif /* SSMSCAN_H */
