/*
 * selscan.h - C ABI of libselscan: the selective state-space scan (the S6 core of
 * Mamba) and its two vision variants, as hand-written HIP kernels for MI355X (gfx950).
 *
 * What is computed (per batch b, channel d, state n, step t):
 *     delta_t = softplus(delta[b,t,d] + delta_bias[d])   if SELSCAN_FLAG_DELTA_SOFTPLUS,
 *               delta[b,t,d] (+ delta_bias[d])            otherwise
 *     h_t[n]  = exp(delta_t * A[d,n]) * h_{t-1}[n] + delta_t * B[b,t,n] * x[b,t,d],  h_{-1} = 0
 *     y[b,t,d] = (sum_n C[b,t,n] * h_t[n] + D[d] * x[b,t,d]) * silu(z[b,t,d])
 * Sources: "Mamba Series from Selective State Spaces to Visual State Space Models",
 * section 选择性 SSM 的数学形式 (continuous system, Abar = exp(delta A), selection
 * delta = softplus(W x + b), B and C functions of the input, A a fixed diagonal) and
 * section 关键代码 (the selective_scan call with Ds, delta_bias, delta_softplus; the SiLU
 * gate); "从LSTM到Mamba" §2.1 (the D x skip term).  Bbar is taken as delta * B (the
 * first-order form of the page's zero-order-hold Bbar; equal to it as delta*A -> 0); with
 * SELSCAN_FLAG_ZOH the forward uses the zero-order-hold form itself,
 *     h_t[n] = exp(delta_t A[d,n]) h_{t-1}[n] + (exp(delta_t A[d,n]) - 1) / A[d,n] * B[b,t,n] x[b,t,d]
 * (delta_t B where A[d,n] = 0), section 选择性 SSM 的数学形式 of the first page.
 *
 * Conventions shared by every entry point
 *  - Layout: row-major, channels fastest.  Per-token tensors x, delta, z, y are
 *    [batch][seqlen][dim]; B and C are [batch][seqlen][dstate]; A is [dim][dstate] fp32;
 *    D and delta_bias are [dim] fp32.  Variants stack per-direction arrays on a leading
 *    direction axis.
 *  - io_dtype (SELSCAN_F32 or SELSCAN_BF16) is the element type of x, delta, B, C, z
 *    and y.  A, D and delta_bias are always fp32.  The state and all arithmetic are fp32.
 *  - Pointers are device pointers (HIP device memory) owned by the caller.  The library
 *    allocates and frees nothing; it keeps no global mutable state and is re-entrant.
 *    `workspace` is caller-owned scratch of at least selscan_workspace_bytes(...) bytes
 *    (may be NULL when that is 0).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is only
 *    enqueued: the call returns before the kernels run, and a fault during execution
 *    surfaces on the stream, not in the return value.
 *  - Optional pointers (D, z, delta_bias) may be NULL: no skip term, no gate, no bias.
 *  - Every call validates its arguments on the host before any HIP call and returns a
 *    selscan_status; nothing is enqueued unless it returns SELSCAN_OK:
 *      SELSCAN_E_NULL         a required pointer is NULL (non-empty problem)
 *      SELSCAN_E_SHAPE        a size is negative (any zero size is an OK no-op), or a window
 *                             side that does not divide the map
 *      SELSCAN_E_ALIGN        a pointer is not aligned to its element size (4 B for fp32
 *                             arrays, 2 B for bf16 arrays)
 *      SELSCAN_E_ALIAS        y overlaps an input array
 *      SELSCAN_E_UNSUPPORTED  dstate != 16, unknown io_dtype or unknown flag bits, or an SS2D
 *                             map with H*W >= 2^31 pixels
 *      SELSCAN_E_WORKSPACE    workspace smaller than selscan_workspace_bytes(...)
 *      SELSCAN_E_HIP          the kernel launch was rejected by the HIP runtime
 *    Non-finite inputs are not checked; they propagate.
 */
#ifndef SELSCAN_H
#define SELSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SELSCAN_ABI_VERSION 1

typedef enum { SELSCAN_F32 = 0, SELSCAN_BF16 = 1 } selscan_dtype;

typedef enum {
    SELSCAN_OK = 0,
    SELSCAN_E_NULL = 1,
    SELSCAN_E_SHAPE = 2,
    SELSCAN_E_ALIGN = 3,
    SELSCAN_E_ALIAS = 4,
    SELSCAN_E_UNSUPPORTED = 5,
    SELSCAN_E_WORKSPACE = 6,
    SELSCAN_E_HIP = 7
} selscan_status;

/* flag bits */
#define SELSCAN_FLAG_DELTA_SOFTPLUS 1u /* delta_t = softplus(delta + delta_bias) */
/* scan entry points: zero-order-hold Bbar = (exp(delta A) - 1) / A * B in place of delta * B
 * (the page's exact discretisation; see the header comment).  A backward call takes the flag
 * its forward was run with (the chunk states differ between the two forms). */
#define SELSCAN_FLAG_ZOH 2u
/* convolution entry points only: SiLU on the convolution's output */
#define SELSCAN_FLAG_SILU 4u

/* operation codes (scan orders) for selscan_workspace_bytes and the selscan_scan_* calls */
typedef enum { SELSCAN_OP_FWD = 0, SELSCAN_OP_BIDIR = 1, SELSCAN_OP_SS2D = 2, SELSCAN_OP_LOCAL_SS2D = 3 } selscan_op;

/*
 * selscan_fwd - one selective scan over the sequence axis (Mamba's S6 layer core).
 *   x, delta, z, y : [batch][seqlen][dim]     io_dtype
 *   B, C           : [batch][seqlen][dstate]  io_dtype
 *   A              : [dim][dstate]            fp32 (real, normally negative)
 *   D, delta_bias  : [dim]                    fp32, nullable
 *   z              : nullable (no gate)
 *   flags          : SELSCAN_FLAG_DELTA_SOFTPLUS, SELSCAN_FLAG_ZOH (any combination) or 0
 * Writes y only.
 */
int selscan_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
                const void *z, const float *delta_bias, unsigned flags, void *y, int64_t batch, int64_t seqlen,
                int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * selscan_fwd_state - selscan_fwd with the recurrent state carried in and out, for recurrent
 * (step-by-step or chunk-by-chunk) inference: "Mamba论文", section "Computation计算" (the
 * parallel mode for training, the recurrent mode for inference), and with the states a
 * later selscan_bwd needs.  Calling it on [0, m) and then on [m, L) with h0 = the first
 * call's h_last gives the same y as one call on [0, L).
 *   h0           : [batch][dim][dstate] fp32, the state before step 0; NULL = zero state
 *   h_last       : [batch][dim][dstate] fp32, written with the state after step seqlen-1 (h0,
 *                  or zero, when seqlen == 0); NULL = not written
 *   chunk_states : selscan_chunk_states_bytes(...) bytes, 4-byte aligned: the states the
 *                  backward restarts from (the library's own layout; pass it unchanged to
 *                  selscan_bwd with the same inputs); NULL = not written
 * Every other argument is as for selscan_fwd.  h_last may be the same pointer as h0 (in-place
 * update); any other overlap of h_last, chunk_states or h0 with y, or of h_last or
 * chunk_states with an input or with each other, is SELSCAN_E_ALIAS.  All three must be
 * 4-byte aligned (SELSCAN_E_ALIGN).  With seqlen == 0 and a non-NULL h_last, only h0 and h_last
 * are read or written (the other pointers may be NULL).
 */
int selscan_fwd_state(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                      const float *h0, float *h_last, float *chunk_states, int64_t batch, int64_t seqlen,
                      int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Bytes of the chunk_states buffer of selscan_fwd_state / selscan_bwd (0 if a size is not
 * positive or dstate != 16). */
size_t selscan_chunk_states_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * selscan_bwd - gradients of L = sum(dy * y) for y = selscan_fwd(...), with the states
 * recomputed from the chunk states the forward saved instead of stored: "Mamba论文"
 * (backward recomputes the intermediate states) and "Mamba Series from Selective State
 * Spaces to Visual State Space Models", section 核心洞察.  flags: SELSCAN_FLAG_DELTA_SOFTPLUS
 * and SELSCAN_FLAG_ZOH as in the forward call (with the zero-order hold, d Bbar / d delta =
 * exp(delta A) B and d Bbar / dA = delta^2 phi'(delta A) B, phi(y) = (e^y - 1) / y, from
 * section 选择性 SSM 的数学形式).  Inputs are exactly those of the forward call (with its h0
 * folded into chunk_states) plus
 *   dy           : [batch][seqlen][dim] io_dtype, dL/dy
 * Outputs (caller-owned, written in full):
 *   dx, ddelta   : [batch][seqlen][dim] io_dtype; ddelta is with respect to the delta
 *                  argument (before delta_bias and softplus)
 *   dB, dC       : [batch][seqlen][dstate] io_dtype (summed over channels in fp32)
 *   dA           : [dim][dstate] fp32 (required even when seqlen == 0: written with zeros)
 *   dD           : [dim] fp32, nullable; the derivative for the skip weight (also when D is NULL)
 *   dz           : [batch][seqlen][dim] io_dtype, nullable; written only when z is given
 *   ddelta_bias  : [dim] fp32, nullable; sum of ddelta over batch and time
 *   dh0          : [batch][dim][dstate] fp32, nullable; dL/dh0 of the forward's initial state
 * workspace: at least selscan_bwd_workspace_bytes(...) bytes, 4-byte aligned (per-tile fp32
 * partial sums of dB and dC, per-batch-row partials of dA, dD, ddelta_bias).  No output may
 * overlap an input, another output or the workspace (SELSCAN_E_ALIAS).  dB, dC, dA, dD and
 * ddelta_bias are sums in a fixed order: the results are the same from run to run.
 */
int selscan_bwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
                const void *z, const float *delta_bias, unsigned flags, const float *chunk_states, const void *dy,
                void *dx, void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz, float *ddelta_bias,
                float *dh0, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes selscan_bwd needs as `workspace` (0 if batch or dim is not positive or
 * dstate != 16). */
size_t selscan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype);

/*
 * selscan_bidir_fwd - bidirectional scan (Vim): "从LSTM到Mamba" §3.1, a forward scan plus
 * the same scan over the time-reversed sequence with its own parameters.  The two
 * outputs are summed in token order (the page concatenates; summing is the fusion this
 * library implements) and gated once:
 *   y = (scan(x; P0) + reverse(scan(reverse(x); reverse(P1)))) * silu(z)
 *   delta, B, C : [2][batch][seqlen][...]  direction 0 forward, 1 backward, TOKEN order
 *   A           : [2][dim][dstate];  D, delta_bias : [2][dim] (nullable)
 *   x, z, y     : [batch][seqlen][dim]
 * When the directions run one after another (see selscan_workspace_bytes), the workspace holds
 * direction 0's fp32 output rows until direction 1 adds them; with bf16 io and seqlen <= 256
 * that sum is formed on chip instead and the workspace is left untouched.  It is still
 * required, with the same size.
 */
int selscan_bidir_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                      int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * ss2d_fwd - VMamba SS2D four-direction scan with merge: "Mamba Series from Selective
 * State Spaces to Visual State Space Models", section 关键代码 (cross_scan_fwd and
 * SS2Dv0.forwardv0).  On an H x W map with pixels p = h*W + w (row-major), L = H*W,
 * direction k visits pixel pi_k(l) at scan step l:
 *   k = 0 row-major (pi = l); k = 1 column-major (pi = (l % H)*W + l / H);
 *   k = 2 reversed row-major; k = 3 reversed column-major.
 * Each direction runs the scan with its own parameters; its output at step l is added
 * at pixel pi_k(l); the sum of the four is written once:
 *   y[b,p,d] = (sum_k o_k[b, pi_k^-1(p), d]) * silu(z[b,p,d])   (z nullable: no gate)
 *   x, z, y     : [batch][H*W][dim]           pixel order
 *   delta       : [4][batch][H*W][dim]        pixel order (value used when pixel p is visited)
 *   B, C        : [4][batch][H*W][dstate]     pixel order
 *   A           : [4][dim][dstate];  D, delta_bias : [4][dim] (nullable)
 * H*W must be below 2^31 (SELSCAN_E_UNSUPPORTED otherwise).
 */
int ss2d_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
             const void *z, const float *delta_bias, unsigned flags, void *y, int64_t batch, int64_t H, int64_t W,
             int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * local_ss2d_fwd - the four-direction cross-scan of ss2d_fwd with windowed orders: the map is
 * cut into square windows of side `window` and each window is scanned as a whole before the
 * next ("LocalMamba: Visual State Space Model with Windowed Selective Scan", as the deep-paper
 * listing and the CSDN notes on it describe it: divide the image into windows, scan within the
 * windows).  The pages give no more, so the orders are the SS2D ones with windows:
 *   k = 0: windows in row-major order, the pixels of each window in row-major order;
 *   k = 1: the same on the transposed map (windows and pixels column-major);
 *   k = 2, 3: k = 0, 1 reversed.
 * window >= 1 must divide H and W (SELSCAN_E_SHAPE otherwise); window 1, or one window over a
 * square map, is ss2d_fwd.  Every array, the merge and the workspace are as for ss2d_fwd
 * (selscan_workspace_bytes with SELSCAN_OP_LOCAL_SS2D).
 */
int local_ss2d_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
                   const void *z, const float *delta_bias, unsigned flags, void *y, int64_t batch, int64_t H,
                   int64_t W, int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * selscan_scan_fwd - the forward of any of the scan orders above, selected by `op`
 * (SELSCAN_OP_FWD: selscan_fwd; SELSCAN_OP_BIDIR: selscan_bidir_fwd; SELSCAN_OP_SS2D: ss2d_fwd;
 * SELSCAN_OP_LOCAL_SS2D: local_ss2d_fwd), also keeping the chunk states that selscan_scan_bwd
 * restarts from.  Arrays, layouts and workspace are those of the op's own entry point.
 *   seqlen       : tokens (pixels) per batch row; for the two-dimensional orders it must equal
 *                  H * W (SELSCAN_E_SHAPE otherwise), for the others H and W are ignored
 *   window       : window side, read by SELSCAN_OP_LOCAL_SS2D only
 *   chunk_states : selscan_scan_chunk_states_bytes(op, ...) bytes, 4-byte aligned, one block of
 *                  states per direction (the library's own layout); NULL = not written.  It may
 *                  overlap no input, y or the workspace (SELSCAN_E_ALIAS).
 * An unknown op is SELSCAN_E_UNSUPPORTED.
 */
int selscan_scan_fwd(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                     const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                     float *chunk_states, int64_t batch, int64_t seqlen, int64_t H, int64_t W, int64_t window,
                     int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * selscan_scan_fwd_noalloc - selscan_scan_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without `workspace` / `workspace_bytes`.  The partial-sum rows of a multi-direction
 * order live in a static device array of the library, selscan_scan_fwd_noalloc_max_bytes()
 * (128 MiB) on every GPU the library runs on, held until the process ends.  The call allocates
 * and frees nothing; its first use on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, with the device current; the caller's current device is restored).
 *  - A problem whose workspace, selscan_workspace_bytes(op, ...) with one row set per problem
 *    (batch * seqlen * dim * 4 bytes for BIDIR, SS2D and LOCAL_SS2D), exceeds the array is
 *    refused with SELSCAN_E_WORKSPACE before anything is enqueued.  The single-direction order
 *    uses no scratch.
 *  - The array is shared by every call on a GPU and keeps the last call's contents: calls on one
 *    GPU whose executions overlap (two streams, or two host threads without ordering) race on it
 *    and must be serialized by the caller.  No call reads scratch it did not write first.
 *  - `stream` decides the device: the stream's own device, or the current device for NULL.
 * Results equal selscan_scan_fwd's with a workspace of the same size.  SELSCAN_E_HIP if the
 * array's address cannot be obtained.
 */
int selscan_scan_fwd_noalloc(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                             const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                             float *chunk_states, int64_t batch, int64_t seqlen, int64_t H, int64_t W,
                             int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *stream);

/* Bytes of the static device array selscan_scan_fwd_noalloc works in. */
size_t selscan_scan_fwd_noalloc_max_bytes(void);

/*
 * selscan_scan_fwd_clocked - selscan_scan_fwd that also records, for every workgroup of its scan
 * kernel, the shader-clock counter (s_memtime) and the constant 100 MHz real-time counter
 * (s_memrealtime) at the workgroup's start and end: stamps[4 w + 0..3] = clock start, clock end,
 * real time start, real time end, for workgroup w.  sum(clock end - start) * 1e8 /
 * sum(real end - start) is the shader clock the kernel ran at, in Hz.  The results and the work
 * are those of selscan_scan_fwd; recording adds two counter reads and four 8-byte stores per
 * workgroup.  For measuring the library's own kernels under load (the benchmark reports it).
 *   stamps : device memory of selscan_clock_stamps_bytes(op, batch, dim) bytes, 8-byte aligned,
 *            caller-owned; SELSCAN_E_NULL if NULL, SELSCAN_E_ALIGN if misaligned.  It is not
 *            checked for overlap with the other arrays.
 */
int selscan_scan_fwd_clocked(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                             const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                             float *chunk_states, int64_t batch, int64_t seqlen, int64_t H, int64_t W,
                             int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                             size_t workspace_bytes, unsigned long long *stamps, void *stream);

/* Bytes of selscan_scan_fwd_clocked's stamps buffer: 32 per workgroup of the largest grid the call
 * can launch, batch x ceil(dim / 16) x directions (0 for an unknown op or a size that is not
 * positive). */
size_t selscan_clock_stamps_bytes(int op, int64_t batch, int64_t dim);

/* Bytes of the chunk_states buffer of selscan_scan_fwd / selscan_scan_bwd for `op` (0 if op is
 * unknown, a size is not positive or dstate != 16). */
size_t selscan_scan_chunk_states_bytes(int op, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * selscan_scan_bwd - gradients of L = sum(dy * y) for y = selscan_scan_fwd(op, ...), the states
 * recomputed from that call's chunk_states (as selscan_bwd does for one direction).  The merged
 * output is y = (sum_k o_k) * silu(z) with o_k one single-direction scan on direction k's
 * visiting order, so direction k's gradients are the single-direction ones for dL/do_k =
 * dy * silu(z) at the pixels it visits ("从LSTM到Mamba" §3.1 for the two directions; "Mamba
 * Series from Selective State Spaces to Visual State Space Models", section 关键代码, for the
 * four-direction merge; "Mamba论文" for recomputing the states in the backward).
 * Inputs: those of the forward call, chunk_states, and dy [batch][seqlen][dim] io_dtype.
 * Outputs (caller-owned, written in full), in the forward's layouts:
 *   dx           : [batch][seqlen][dim] io_dtype, summed over the directions
 *   ddelta       : [ndir][batch][seqlen][dim] io_dtype (token / pixel order; before
 *                  delta_bias and softplus)
 *   dB, dC       : [ndir][batch][seqlen][dstate] io_dtype (summed over channels in fp32)
 *   dA           : [ndir][dim][dstate] fp32 (required)
 *   dD, ddelta_bias : [ndir][dim] fp32, nullable
 *   dz           : [batch][seqlen][dim] io_dtype, nullable; written only when z is given
 * (ndir = 1, 2, 4 for FWD, BIDIR, SS2D / LOCAL_SS2D; with ndir = 1 the leading axis is absent
 * and the call equals selscan_bwd without dh0.)  workspace: at least
 * selscan_scan_bwd_workspace_bytes(op, ...) bytes, 4-byte aligned.  No output may overlap an
 * input, another output or the workspace (SELSCAN_E_ALIAS).  All sums are in a fixed order:
 * the results are the same from run to run.
 */
int selscan_scan_bwd(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                     const float *D, const void *z, const float *delta_bias, unsigned flags,
                     const float *chunk_states, const void *dy, void *dx, void *ddelta, float *dA, void *dB,
                     void *dC, float *dD, void *dz, float *ddelta_bias, int64_t batch, int64_t seqlen, int64_t H,
                     int64_t W, int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Scratch bytes selscan_scan_bwd needs as `workspace` for `op` (0 if op is unknown, batch or dim
 * is not positive or dstate != 16).  As for selscan_workspace_bytes, small grids get room for
 * per-direction dx and output rows (one direction per workgroup); a workspace without it (two
 * [batch][seqlen][dim] fp32 row sets rather than two per direction) runs the directions in turn,
 * with the same result bit for bit. */
size_t selscan_scan_bwd_workspace_bytes(int op, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                        int io_dtype);

/*
 * causal_conv1d_fwd - the depthwise causal convolution in front of the Mamba block's scan,
 * Conv1D(k=4) -> SiLU ("Mamba Series from Selective State Spaces to Visual State Space Models",
 * section 方法设计, the Mamba block diagram).  Per batch b, step t, channel d:
 *     v = bias[d] + sum_{i<width} weight[d][i] * xin[b][t-(width-1)+i][d],   out = silu(v) with
 *     SELSCAN_FLAG_SILU, else v;
 * xin is x with the width-1 rows of state_in in front (zero rows when state_in is NULL).
 *   x, out      : [batch][seqlen][dim] io_dtype (out may not overlap x: SELSCAN_E_ALIAS)
 *   weight      : [dim][width] fp32, width 1..4 (else SELSCAN_E_UNSUPPORTED); bias [dim] fp32, nullable
 *   state_in    : [batch][width-1][dim] io_dtype, nullable: the input rows before step 0
 *   state_out   : [batch][width-1][dim] io_dtype, nullable: written with the last width-1 rows of
 *                 (state_in rows ++ x rows), the state_in of a call on the following steps.  It may
 *                 not overlap state_in or any other array (double-buffer for streaming).
 *   flags       : SELSCAN_FLAG_SILU or 0
 * seqlen 0 with a state_out only copies the state.  The pages give only k = 4; causality (no
 * step sees a later one) and one filter per channel are the reading this call implements.
 */
int causal_conv1d_fwd(const void *x, const float *weight, const float *bias, const void *state_in, void *state_out,
                      unsigned flags, void *out, int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                      int io_dtype, void *stream);

/*
 * dwconv2d_fwd - the depthwise 3x3 convolution in front of the VSS block's SS2D, DWConv 3x3 ->
 * SiLU (same page, VSS block diagram; section 关键代码, SS2Dv0.forwardv0: conv2d then act), on
 * channels-last maps.  Per batch b, pixel (h, w), channel d:
 *     v = bias[d] + sum_{i,j<3} weight[d][i][j] * x[b][h+i-1][w+j-1][d]   (x = 0 outside the map),
 *     out = silu(v) with SELSCAN_FLAG_SILU, else v
 * (a cross-correlation keeping the map size, stride 1).
 *   x, out   : [batch][H][W][dim] io_dtype (pixel p = h*W + w, as ss2d_fwd's x); out may not
 *              overlap x (SELSCAN_E_ALIAS)
 *   weight   : [dim][3][3] fp32; bias [dim] fp32, nullable; ksize must be 3 (else
 *              SELSCAN_E_UNSUPPORTED)
 */
int dwconv2d_fwd(const void *x, const float *weight, const float *bias, unsigned flags, void *out, int64_t batch,
                 int64_t H, int64_t W, int64_t dim, int64_t ksize, int io_dtype, void *stream);

/*
 * causal_conv1d_bwd - gradients of L = sum(dout * out) for out = causal_conv1d_fwd(x, weight, bias,
 * state_in, flags) (the chain rule through the convolution of the Mamba block diagram, same page
 * and section): with v the pre-activation and dv = dout * act'(v) (act' = silu' with
 * SELSCAN_FLAG_SILU, else 1),
 *     dxin[b][t-(width-1)+i][d] += weight[d][i] * dv[b][t][d],   dweight[d][i] = sum_{b,t} xin * dv,
 *     dbias[d] = sum_{b,t} dv[b][t][d]
 * where xin is state_in's rows followed by x; the rows before step 0 give dstate_in.
 *   x, dout, dx      : [batch][seqlen][dim] io_dtype
 *   weight           : [dim][width] fp32, width 1..4; bias [dim] fp32, nullable; state_in nullable
 *   dweight          : [dim][width] fp32, required; dbias [dim] fp32, nullable (the sum of dv,
 *                      also when bias is NULL); dstate_in [batch][width-1][dim] io_dtype, nullable
 *   flags            : SELSCAN_FLAG_SILU or 0, as in the forward call
 * workspace: at least causal_conv1d_bwd_workspace_bytes(...) bytes, 4-byte aligned (dv in fp32 and
 * per-thread-group partial sums of dweight and dbias).  No output may overlap an input, another
 * output or the workspace (SELSCAN_E_ALIAS).  dweight and dbias are sums in a fixed order: the
 * results are the same from run to run.  seqlen 0 writes zeros to dweight, dbias, dstate_in.
 */
int causal_conv1d_bwd(const void *x, const float *weight, const float *bias, const void *state_in, const void *dout,
                      unsigned flags, void *dx, float *dweight, float *dbias, void *dstate_in, int64_t batch,
                      int64_t seqlen, int64_t dim, int64_t width, int io_dtype, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Scratch bytes causal_conv1d_bwd needs as `workspace` (0 if batch or dim is not positive or the
 * width is not 1..4). */
size_t causal_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int io_dtype);

/*
 * dwconv2d_bwd - gradients of L = sum(dout * out) for out = dwconv2d_fwd(x, weight, bias, flags)
 * (the VSS block's DWConv 3x3, same page): dv = dout * act'(v) and
 *     dx[b][h+i-1][w+j-1][d] += weight[d][i][j] * dv[b][h][w][d]   (pixels inside the map),
 *     dweight[d][i][j] = sum x[b][h+i-1][w+j-1][d] * dv[b][h][w][d],   dbias[d] = sum dv
 *   x, dout, dx : [batch][H][W][dim] io_dtype;  weight, dweight [dim][3][3] fp32 (dweight
 *                 required); bias [dim] fp32, nullable; dbias [dim] fp32, nullable; ksize 3
 * workspace: at least dwconv2d_bwd_workspace_bytes(...) bytes, 4-byte aligned.  Aliasing,
 * determinism and errors as for causal_conv1d_bwd; an empty map writes zeros to dweight and dbias.
 */
int dwconv2d_bwd(const void *x, const float *weight, const float *bias, const void *dout, unsigned flags, void *dx,
                 float *dweight, float *dbias, int64_t batch, int64_t H, int64_t W, int64_t dim, int64_t ksize,
                 int io_dtype, void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes dwconv2d_bwd needs as `workspace` (0 if any size is not positive). */
size_t dwconv2d_bwd_workspace_bytes(int64_t batch, int64_t H, int64_t W, int64_t dim, int io_dtype);

/* Scratch bytes to pass as `workspace` for this problem (0 = none).  Several directions keep fp32
 * partial outputs [batch][seqlen][dim] there.  When batch x ceil(dim/16) is below 1024 (too few
 * workgroups to fill the GPU when each walks every direction) the returned size holds one such
 * row set per direction, and the call runs one direction per workgroup plus an in-order merge;
 * a workspace of a single row set is still accepted and runs the directions one after another.
 * Both give the same result bit for bit. */
size_t selscan_workspace_bytes(int op, int64_t batch, int64_t seqlen_or_hw, int64_t dim, int64_t dstate,
                               int io_dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *selscan_status_str(int status);

/* SELSCAN_ABI_VERSION of the loaded library. */
int selscan_abi_version(void);

/* Text of the HIP error behind the calling thread's most recent SELSCAN_E_HIP ("no error"
 * if there was none).  Static storage per thread; never NULL. */
const char *selscan_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */
