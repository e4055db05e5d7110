/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan (S6).
 *
 * Four operations, all on device memory, all asynchronous on the caller's
 * HIP stream:
 *
 *   ssm_scan_fwd       prefill: run the selective scan over a whole sequence;
 *   ssm_state_update   decode: advance a persistent state by one token;
 *   ssm_conv_scan_fwd  prefill with the block's short causal depthwise
 *                      convolution (and its silu) fused in front of the scan;
 *   ssm_scan_bwd       training: every gradient of a scalar loss through
 *                      ssm_scan_fwd, given dL/dy (and optionally dL/dh_L).
 *
 * ssm_scan_fwd_ex and ssm_state_update_ex are the first two with a choice of
 * how B is discretized (Delta * B, or exact zero-order hold), and
 * ssm_scan_fwd_complex and ssm_state_update_complex are the prefill scan and
 * the decode step with a complex diagonal A.
 *
 * What is computed (for every batch row b and channel d independently):
 *
 *   Delta_l = softplus(delta[b,d,l] + bias[d])   (or delta + bias, flag off)
 *   Abar    = exp(Delta_l * A[d,n])              zero-order hold of A
 *   h[n]    = Abar * h[n] + Delta_l * B[b,n,l] * u[b,d,l]
 *   y[b,d,l]= (sum_n C[b,n,l] * h[n] + D[d] * u[b,d,l]) * silu(z[b,d,l])
 *
 * The state recurrence h <- A h + B x and read-out y = C h are the equations
 * of the Korean Mamba summary ("Mamba: Linear-Time Sequence Modeling with
 * Selective State Spaces", section on the SSM's mathematical definition).  The
 * scan (previous state times A-bar plus current input times B-bar) is the
 * Chinese Mamba explainer's "hardware-aware design: parallel scan" section;
 * the input dependence of Delta, B and C (A fixed and diagonal, N numbers per
 * channel) is from the same explainer's S4-to-S6 sections and the Hebrew
 * overview's "SSM + selection (S6)" section; zero-order hold is named in the
 * explainer's discretization stage (1a/1b).  The pages lost the formulas; the
 * readings taken for the silent points are: Bbar*u = Delta*B*u, no output lag
 * (y_l uses h_l, which already holds u_l), D skip before the gate, silu gate,
 * softplus applied to delta + bias, zero initial state unless h0 is given.
 *
 * Conventions shared by the entry points
 *  - Every pointer is a DEVICE pointer to contiguous, row-major memory (last
 *    index fastest).  The caller owns every buffer; the library never keeps a
 *    pointer after the call returns.
 *  - io dtype (SSM_F32 or SSM_BF16) applies to u, delta, z, B, C and y.  A, D,
 *    delta_bias, h0, last_state and state are always fp32.  All arithmetic is
 *    fp32; bf16 inputs are widened exactly, y is rounded to nearest-even.
 *  - Optional pointers (D, z, delta_bias, h0, last_state) may be NULL:
 *    D = NULL means D = 0, delta_bias = NULL means 0, z = NULL means no gate,
 *    h0 = NULL means a zero initial state, last_state = NULL means not written.
 *  - Sizes: batch, dim, seqlen >= 1 and 1 <= dstate <= 16.
 *  - stream is a hipStream_t (NULL = the default stream).  The call only
 *    enqueues work; device-side faults surface at the caller's next
 *    synchronisation.  The library prints nothing and never aborts.
 *  - Validation (NULL pointers, sizes, dtype, element alignment, overlap of an
 *    output with an input) happens on the host before any HIP call, so an
 *    invalid call returns an error code without touching the device.
 *  - NaN and Inf propagate; nothing is clamped.
 *  - The prefill and decode entry points (ssm_scan_fwd, ssm_scan_fwd_ex,
 *    ssm_scan_fwd_complex, ssm_conv_scan_fwd, ssm_scan_fwd_save and the
 *    ssm_state_update family) allocate no device memory and need no
 *    workspace: a long sequence scanned in parallel segments keeps each
 *    segment's aggregate and carry-in inside that segment's own range of y
 *    before y is written there (y's prior contents are never read as data).
 *    They can therefore be captured into a HIP graph as plain kernel launches.
 *  - The backward entry points (ssm_scan_bwd, ssm_scan_bwd_ex,
 *    ssm_scan_bwd_complex, ssm_scan_bwd_saved, ssm_conv_bwd) take stream-
 *    ordered scratch from a per-device pool of the library (checkpoints and
 *    partial sums), freed on the same stream within the call.  The pool's
 *    release threshold is 0: freed blocks are reused by later calls on the
 *    stream and returned to the device at the next synchronisation.
 *  - Calls on different streams are independent; the library is re-entrant.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 13

struct ihipStream_t; /* the same incomplete type as HIP's hipStream_t */

typedef enum {
  SSM_F32 = 0,  /* 32-bit IEEE float */
  SSM_BF16 = 1  /* bfloat16 (upper half of an fp32) */
} ssm_dtype_t;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,                 /* a required pointer is NULL            */
  SSM_ERR_SHAPE = 2,                /* a size < 1, or a size product overflows */
  SSM_ERR_DSTATE_UNSUPPORTED = 3,   /* dstate > 16                           */
  SSM_ERR_DTYPE = 4,                /* unknown io dtype                      */
  SSM_ERR_ALIGN = 5,                /* a pointer is not element-aligned      */
  SSM_ERR_ALIAS = 6,                /* an output overlaps an input           */
  SSM_ERR_HIP = 7,                  /* a HIP runtime call failed             */
  SSM_ERR_UNSUPPORTED = 8,          /* valid, but outside what this entry point implements */
  SSM_ERR_WORKSPACE = 9             /* needs more scratch than the fixed device array holds */
} ssm_status_t;

/*
 * ssm_scan_fwd -- prefill selective scan over seqlen tokens.
 *
 *   u          [batch, dim, seqlen]     io     input sequence x
 *   delta      [batch, dim, seqlen]     io     raw step size (before bias / softplus)
 *   A          [dim, dstate]            fp32   diagonal state matrix (one row per channel)
 *   B          [batch, dstate, seqlen]  io     input matrix, per token, shared by all channels
 *   C          [batch, dstate, seqlen]  io     output matrix, per token, shared by all channels
 *   D          [dim]                    fp32   skip weight, may be NULL
 *   z          [batch, dim, seqlen]     io     gate input, may be NULL
 *   delta_bias [dim]                    fp32   added to delta, may be NULL
 *   softplus_flag                              nonzero: Delta = softplus(delta + bias)
 *   h0         [batch, dim, dstate]     fp32   initial state, may be NULL; may be the
 *                                              same pointer as last_state (the state is
 *                                              then carried in place); any other overlap
 *                                              with an output is SSM_ERR_ALIAS
 *   y          [batch, dim, seqlen]     io     output, written
 *   last_state [batch, dim, dstate]     fp32   state after the last token, may be NULL
 *
 * y must not overlap any input.  The expanded (batch, dim, seqlen, dstate)
 * state is never written to memory: each channel's dstate values live in
 * registers for the whole scan.
 */
ssm_status_t ssm_scan_fwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                          const void* u, const void* delta, const float* A, const void* B,
                          const void* C, const float* D, const void* z, const float* delta_bias,
                          int softplus_flag, const float* h0, void* y, float* last_state,
                          struct ihipStream_t* stream);

/*
 * ssm_state_update -- one decode step: the recurrence of ssm_scan_fwd for a
 * single token (seqlen = 1), updating the state in place.  This is the
 * recurrent ("RNN") mode the Chinese explainer describes for autoregressive
 * inference: constant work per token because the state has a fixed size.
 *
 *   state      [batch, dim, dstate]     fp32   read, then overwritten with the new state
 *   u, delta   [batch, dim]             io
 *   A          [dim, dstate]            fp32
 *   B, C       [batch, dstate]          io
 *   D          [dim]                    fp32   may be NULL
 *   z          [batch, dim]             io     may be NULL
 *   delta_bias [dim]                    fp32   may be NULL
 *   y          [batch, dim]             io     written; must not overlap any input or state
 *
 * The result equals ssm_scan_fwd with seqlen = 1, h0 = last_state = state.
 */
ssm_status_t ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t io, float* state,
                              const void* u, const void* delta, const float* A, const void* B,
                              const void* C, const float* D, const void* z,
                              const float* delta_bias, int softplus_flag, void* y,
                              struct ihipStream_t* stream);

/*
 * ssm_conv_scan_fwd -- the Mamba block's causal Conv1d fused in front of the
 * scan.  The Hebrew overview ("תחילת העבודה עם Mamba") says the Mamba block
 * runs a causal Conv1d before the selective SSM; the Chinese explainer's
 * section on why a convolution precedes the SSM says it mixes each token
 * with its neighbours first.  Read here as a depthwise (per-channel) causal
 * filter of width K = conv_width (1..4) with an optional bias and silu:
 *
 *   u[b,d,l] = act(conv_bias[d] + sum_{k<K} conv_weight[d,k] * x[b,d,l-(K-1)+k])
 *
 * where x before token 0 is x_prev (the K-1 inputs that preceded this piece
 * of the sequence) or zero, and act is silu when conv_silu is nonzero.  u is
 * rounded to the io dtype, as if it had been stored, and then the scan of
 * ssm_scan_fwd runs on it.  The result equals the conv written to memory
 * followed by ssm_scan_fwd on it; u never touches memory (every kernel path
 * computes it from x in its own prologue) unless u_out asks for it.
 *
 *   x            [batch, dim, seqlen]         io    conv input
 *   conv_weight  [dim, conv_width]            fp32  conv_weight[d, K-1] multiplies the current token
 *   conv_bias    [dim]                        fp32  may be NULL (0)
 *   x_prev       [batch, dim, conv_width-1]   io    may be NULL (zero history); unused when conv_width == 1
 *   conv_silu    nonzero: u = silu(conv + bias)
 *   u_out        [batch, dim, seqlen]         io    the u the scan consumed, may be NULL
 *   delta .. last_state, stream: as ssm_scan_fwd (y must not overlap any input,
 *                                u_out must not overlap any input or output)
 *
 * Errors as ssm_scan_fwd, plus SSM_ERR_SHAPE for conv_width outside 1..4.
 * Allocates nothing.  A u_out that is not 16-byte aligned sends the call to
 * the per-token kernel (SSM_PATH_GENERIC).
 */
ssm_status_t ssm_conv_scan_fwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int64_t conv_width,
                               ssm_dtype_t io, const void* x, const float* conv_weight, const float* conv_bias,
                               const void* x_prev, int conv_silu, const void* delta, const float* A,
                               const void* B, const void* C, const float* D, const void* z,
                               const float* delta_bias, int softplus_flag, const float* h0, void* y,
                               float* last_state, void* u_out, struct ihipStream_t* stream);

/*
 * ssm_conv_bwd -- gradients of the conv that ssm_conv_scan_fwd fuses in front
 * of the scan, for training: given du = dL/du (ssm_scan_bwd's du for the u the
 * scan consumed), with v the pre-activation conv_bias[d] + sum_k
 * conv_weight[d,k] x[b,d,l-(K-1)+k] (recomputed; the io rounding of u is
 * passed through):
 *
 *   dv[b,d,l]         = du[b,d,l] * silu'(v[b,d,l])   (du itself when conv_silu is 0)
 *   dx[b,d,p]         = sum_k conv_weight[d,k] * dv[b,d,p+(K-1)-k]   (dv past the end is 0)
 *   dx_prev[b,d,j]    = sum_{k<=j} conv_weight[d,k] * dv[b,d,j-k]    (the history slots x_prev)
 *   dconv_weight[d,k] = sum_{b,l} dv[b,d,l] * x[b,d,l-(K-1)+k]       (x before token 0 from x_prev)
 *   dconv_bias[d]     = sum_{b,l} dv[b,d,l]
 *
 *   x, conv_weight, conv_bias, x_prev, conv_silu, conv_width: as ssm_conv_scan_fwd
 *   du            [batch, dim, seqlen]         io    read
 *   dx            [batch, dim, seqlen]         io    written
 *   dconv_weight  [dim, conv_width]            fp32  written
 *   dconv_bias    [dim]                        fp32  written when not NULL
 *   dx_prev       [batch, dim, conv_width-1]   io    written when not NULL (ignored when conv_width == 1)
 *
 * Outputs must not overlap inputs or each other.  Errors: SSM_ERR_DTYPE,
 * SSM_ERR_SHAPE (a size below 1, conv_width outside 1..4, sizes that
 * overflow), SSM_ERR_NULL (x, conv_weight, du, dx, dconv_weight),
 * SSM_ERR_ALIGN (io buffers to their element, fp32 buffers to 4 bytes),
 * SSM_ERR_ALIAS, SSM_ERR_UNSUPPORTED (rows of 2^31 bytes or more: seqlen
 * times the io element size).  Uses stream-ordered scratch from the
 * library's pool for the per-block sums; deterministic (fixed summation
 * order).
 */
ssm_status_t ssm_conv_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t conv_width, ssm_dtype_t io,
                          const void* x, const float* conv_weight, const float* conv_bias, const void* x_prev,
                          int conv_silu, const void* du, void* dx, float* dconv_weight, float* dconv_bias,
                          void* dx_prev, struct ihipStream_t* stream);

/*
 * ssm_scan_bwd -- gradients of the scan for training: given dy = dL/dy and
 * (optionally) dlast = dL/dlast_state, the gradients of L with respect to
 * every input of ssm_scan_fwd.  The pages state the training-efficiency aim of
 * the hardware-aware scan (the Chinese explainer's "硬件感知的设计" and S4/S6
 * comparison sections: parallel training without materialising the expanded
 * state); the gradient formulas are the chain rule through the recurrence:
 *
 *   g_t    = dy_t silu(z_t) (dy_t without z);  lambda_t = g_t C_t + Abar_{t+1} lambda_{t+1} (+ dlast at the end)
 *   du     = g D + Delta sum_n lambda B;        dDelta = sum_n lambda (A Abar h_{t-1} + B u)
 *   ddelta = dDelta sigmoid(delta + bias) with softplus, else dDelta
 *   dA[d,n] = sum_{b,t} lambda Delta Abar h_{t-1};  dB[b,n,t] = sum_d lambda Delta u;  dC[b,n,t] = sum_d g h
 *   dD[d] = sum_{b,t} g u;  ddelta_bias[d] = sum_{b,t} ddelta;  dz = dy (C.h + D u) silu'(z);  dh0 = Abar_0 lambda_0
 *
 * The expanded state is never stored: a forward pass writes the state every
 * 16 tokens (stream-ordered scratch from the library's pool, about a 16th of
 * the expanded state) and the backward recomputes each 16-token tile from it.
 *
 *   inputs u .. h0      as ssm_scan_fwd (io dtype for u, delta, z, B, C)
 *   dy          [batch, dim, seqlen]    io
 *   dlast       [batch, dim, dstate]    fp32   may be NULL (0)
 *   du, ddelta  [batch, dim, seqlen]    io     written
 *   dA          [dim, dstate]           fp32   written
 *   dB, dC      [batch, dstate, seqlen] fp32   written (sums over all channels: kept in fp32)
 *   dD, ddelta_bias [dim]               fp32   written when not NULL (the gradient at D = 0 / bias = 0
 *                                              when D / delta_bias is NULL)
 *   dz          [batch, dim, seqlen]    io     written when z and dz are not NULL
 *   dh0         [batch, dim, dstate]    fp32   written when not NULL (the gradient at h0 = 0 when h0 is NULL)
 *
 * Outputs must not overlap inputs or each other.  Supported: dstate in
 * {4, 8, 16}, seqlen a multiple of 8 and below 2^26 bytes per row (seqlen
 * times the io element size), and every (batch, dim, seqlen) and (batch,
 * dstate, seqlen) buffer 16-byte aligned; anything else returns
 * SSM_ERR_UNSUPPORTED.  Deterministic: partial sums are added in a fixed order.
 */
ssm_status_t ssm_scan_bwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                          const void* u, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int softplus_flag,
                          const float* h0, const void* dy, const float* dlast, void* du, void* ddelta,
                          float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                          struct ihipStream_t* stream);

/* How B is discretized (the _ex entry points).  Abar = exp(Delta * A) in both. */
typedef enum {
  SSM_DISC_DELTA_B = 0, /* Bbar * u = Delta * B * u (what every other entry point computes) */
  SSM_DISC_ZOH = 1      /* exact zero-order hold: Bbar * u = (exp(Delta * A) - 1) / A * B * u,
                           Delta * B * u where A = 0                                          */
} ssm_disc_t;

/*
 * ssm_scan_fwd_ex -- ssm_scan_fwd with a choice of discretization for B.
 * The Chinese explainer's discretization stage (1a/1b) turns the continuous
 * parameters into discrete ones by a fixed rule and names zero-order hold as
 * one such rule (its formulas did not survive).  Holding u constant over a
 * step of length Delta and solving dh/dt = A h + B u exactly gives, per state
 * of a diagonal A, Abar = exp(Delta A) and Bbar = (exp(Delta A) - 1) / A * B
 * (SSM_DISC_ZOH); SSM_DISC_DELTA_B keeps Abar and takes Bbar = Delta * B, the
 * form every other entry point uses.  Arguments, layouts, ownership and
 * errors are those of ssm_scan_fwd, plus SSM_ERR_UNSUPPORTED for a disc value
 * outside ssm_disc_t.  With SSM_DISC_DELTA_B the result is bitwise that of
 * ssm_scan_fwd.  fp32 evaluation: where |Delta A| < 1/16 the zero-order-hold
 * factor is taken from its series (exp(x) - 1 cancels there), elsewhere from
 * exp(Delta A) - 1; both are within about 1e-6 relative of the exact factor.
 */
ssm_status_t ssm_scan_fwd_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                             ssm_disc_t disc, const void* u, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z, const float* delta_bias,
                             int softplus_flag, const float* h0, void* y, float* last_state,
                             struct ihipStream_t* stream);

/*
 * ssm_state_update_ex -- ssm_state_update with a choice of discretization for
 * B (as ssm_scan_fwd_ex).  Equals ssm_scan_fwd_ex with seqlen = 1 and
 * h0 = last_state = state.  Errors as ssm_state_update, plus
 * SSM_ERR_UNSUPPORTED for a disc value outside ssm_disc_t.
 */
ssm_status_t ssm_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t io, ssm_disc_t disc,
                                 float* state, const void* u, const void* delta, const float* A, const void* B,
                                 const void* C, const float* D, const void* z, const float* delta_bias,
                                 int softplus_flag, void* y, struct ihipStream_t* stream);

/*
 * ssm_scan_fwd_complex -- the prefill scan with a complex diagonal A.  The
 * pages give A as real (the Chinese explainer's section on the S4 matrix
 * dimensions: N numbers per channel); models of the S4 family also use a
 * complex diagonal A.  Read here as a real system whose state matrix has
 * complex-conjugate eigenvalue pairs, one state of each pair stored:
 *
 *   h[n]     = exp(Delta A[d,n]) h[n] + Delta B[b,n,l] u[b,d,l]      (complex A, B, h)
 *   y[b,d,l] = (2 Re(sum_n C[b,n,l] h[n]) + D[d] u[b,d,l]) * silu(z[b,d,l])
 *
 * (the 2 Re adds each state's conjugate partner).  Delta, u, z, D and the
 * bias are real and as in ssm_scan_fwd.  dstate counts complex states.
 * Complex arrays hold (re, im) pairs in their last index:
 *
 *   A          [dim, dstate, 2]          fp32
 *   B, C       [batch, dstate, seqlen, 2] io
 *   h0         [batch, dim, dstate, 2]   fp32   may be NULL (zero); may equal last_state
 *   last_state [batch, dim, dstate, 2]   fp32   may be NULL
 *   u, delta, z, y, D, delta_bias: as ssm_scan_fwd.
 *
 * Errors as ssm_scan_fwd (dstate above 8, i.e. above 16 real numbers per
 * channel, is SSM_ERR_DSTATE_UNSUPPORTED).  dstate 4 or 8 with seqlen a
 * multiple of 8 and every (batch, dim, seqlen) and B/C buffer 16-byte aligned
 * runs the single-pass kernel (one complex state per wave); every other shape
 * a kernel that walks each channel a token at a time (correct, not fast).
 */
ssm_status_t ssm_scan_fwd_complex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                  const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                  const float* h0, void* y, float* last_state, struct ihipStream_t* stream);

/*
 * ssm_state_update_complex -- one decode step with a complex diagonal A: the
 * recurrence of ssm_scan_fwd_complex for a single token, the state updated in
 * place.  Equals ssm_scan_fwd_complex with seqlen = 1 and h0 = last_state =
 * state.
 *
 *   state      [batch, dim, dstate, 2]  fp32   read, then overwritten
 *   u, delta   [batch, dim]             io
 *   A          [dim, dstate, 2]         fp32
 *   B, C       [batch, dstate, 2]       io
 *   D, z, delta_bias, y: as ssm_state_update
 *
 * dstate counts complex states, 1..8 (above 8 is SSM_ERR_DSTATE_UNSUPPORTED).
 * Errors as ssm_state_update.  Any dstate and element alignment runs; 2, 4
 * and 8 with 16-byte aligned state and A (8-byte B and C in bf16, 16-byte in
 * fp32) take the vector kernel.
 */
ssm_status_t ssm_state_update_complex(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t io, float* state,
                                      const void* u, const void* delta, const float* A, const void* B, const void* C,
                                      const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                      void* y, struct ihipStream_t* stream);

/*
 * Training without the backward's forward pass.  ssm_scan_bwd recomputes the
 * forward to obtain the states at every 16th token (its checkpoints).  A
 * training step runs the forward anyway: ssm_scan_fwd_save is ssm_scan_fwd
 * that also writes those checkpoints, and ssm_scan_bwd_saved is ssm_scan_bwd
 * that reads them instead of recomputing them.  The checkpoints hold fp32
 * states laid out [ceil(seqlen/16)][batch][dstate][dim] (the state before
 * tokens 0, 16, 32, ...), ssm_scan_ckpt_bytes bytes; the caller owns the
 * buffer and must pass the same u, delta, A, B, C, D, z, delta_bias, flags and
 * h0 to both calls (ssm_scan_bwd_saved does not read h0: the checkpoints
 * carry it).  Results equal ssm_scan_fwd and ssm_scan_bwd bit for bit on
 * shapes where ssm_scan_fwd takes the single-pass kernel.
 *
 * ssm_scan_ckpt_bytes: bytes of the checkpoint buffer; errors as ssm_scan_fwd's
 *   size checks.  bytes may be NULL.
 * ssm_scan_fwd_save: arguments of ssm_scan_fwd plus ckpt (written; may overlap
 *   no input or output).  Supported shapes are those of ssm_scan_bwd (dstate in
 *   {4, 8, 16}, seqlen a multiple of 8, 16-byte aligned rows, y included);
 *   others return SSM_ERR_UNSUPPORTED.  It always runs the single-pass kernel.
 * ssm_scan_bwd_saved: arguments of ssm_scan_bwd with ckpt (read) in place of
 *   h0; errors as ssm_scan_bwd, SSM_ERR_NULL for a NULL ckpt.
 */
ssm_status_t ssm_scan_ckpt_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                 int64_t* bytes);

ssm_status_t ssm_scan_fwd_save(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                               const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int softplus_flag,
                               const float* h0, void* y, float* last_state, float* ckpt,
                               struct ihipStream_t* stream);

ssm_status_t ssm_scan_bwd_saved(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                const void* u, const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                const float* ckpt, const void* dy, const float* dlast, void* du, void* ddelta,
                                float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                                struct ihipStream_t* stream);

/*
 * ssm_scan_bwd_saved_noalloc -- ssm_scan_bwd_saved for callers that cannot
 * allocate device memory: code under HIP graph capture, tight training loops,
 * harnesses that forbid allocation.  Same arguments, same kernels, bitwise
 * the same gradients; it calls no allocating routine.  Its scratch (the
 * per-group dB/dC partial sums and the per-batch-row partials of dA, dD and
 * ddelta_bias: 4 * (2 * ceil(dim/64) * batch * dstate * seqlen
 * + batch * dim * (dstate + 2)) bytes) comes from a fixed 64 MiB device
 * array inside the library, one per device, held from the library's load
 * until the process ends.  A call whose scratch is larger returns
 * SSM_ERR_WORKSPACE before any HIP call (the Mamba-130M layer, batch 8 x
 * dim 1536 x dstate 16 x seqlen 2048, takes 49 MiB; the Mamba-1.4B layer,
 * batch 4 x 4096 x 16 x 4096, 129 MiB, does not fit).
 *
 * Every call on a device shares that device's array: calls that overlap on
 * one device (different streams without ordering between them) race and
 * must not be issued.  The first call on each device resolves the array's
 * address (hipGetSymbolAddress); make it outside graph capture.
 */
ssm_status_t ssm_scan_bwd_saved_noalloc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                        const void* u, const void* delta, const float* A, const void* B,
                                        const void* C, const float* D, const void* z, const float* delta_bias,
                                        int softplus_flag, const float* ckpt, const void* dy, const float* dlast,
                                        void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                        float* ddelta_bias, float* dh0, struct ihipStream_t* stream);

/*
 * ssm_scan_bwd_ex -- ssm_scan_bwd for either discretization of B (see
 * ssm_scan_fwd_ex): the gradients of ssm_scan_fwd_ex with the same disc.
 * Under zero-order hold, with phi = (exp(Delta A) - 1) / A per state,
 *   du += sum_n lambda B phi,  dB += lambda phi u,
 *   dDelta = sum_n lambda (A Abar h_{t-1} + Abar B u)      (d phi / d Delta = Abar)
 *   dA += lambda (Delta Abar h_{t-1} + B u d phi / d A),
 *   d phi / d A = (Delta Abar - phi) / A = Delta^2 (x e^x - e^x + 1) / x^2, x = Delta A
 * (its series where |x| < 1/4, Delta^2 / 2 at A = 0).  Arguments, layouts and
 * errors as ssm_scan_bwd, plus SSM_ERR_UNSUPPORTED for a disc value outside
 * ssm_disc_t.  SSM_DISC_DELTA_B gives ssm_scan_bwd's results bit for bit.
 */
ssm_status_t ssm_scan_bwd_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                             ssm_disc_t disc, const void* u, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z, const float* delta_bias,
                             int softplus_flag, const float* h0, const void* dy, const float* dlast, void* du,
                             void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                             float* dh0, struct ihipStream_t* stream);

/*
 * ssm_scan_bwd_complex -- gradients of ssm_scan_fwd_complex for a real loss
 * with dL/dy = dy and dL/dlast_state = dlast.  The gradient with respect to a
 * complex number w (a pair (Re w, Im w)) is returned as the pair
 * (dL/dRe w, dL/dIm w).  With lambda that gradient for the state, q =
 * Abar_t h_{t-1} and g = dL/d(pre-gate output):
 *   lambda_t = 2 g_t conj(C_t) + conj(Abar_{t+1}) lambda_{t+1}   (+ dlast at the end)
 *   dC += 2 g conj(h_t),  dB += lambda Delta u,  dA += lambda conj(Delta q)
 *   du = g D + Delta sum_n Re(lambda conj(B)),  dDelta = sum_n Re(lambda conj(A q + B u))
 *   dh0 = conj(Abar_0) lambda_0;  dz, dD, ddelta_bias as ssm_scan_bwd.
 * Layouts: complex arrays as ssm_scan_fwd_complex ((re, im) last): dA
 * [dim, dstate, 2], dB, dC [batch, dstate, seqlen, 2], dlast and dh0 [batch,
 * dim, dstate, 2], all fp32; du, ddelta, dz as ssm_scan_bwd.  dstate counts
 * complex states: 4 or 8 (other values up to 8 are SSM_ERR_UNSUPPORTED,
 * above 8 SSM_ERR_DSTATE_UNSUPPORTED); seqlen a multiple of 8 and 16-byte
 * aligned rows, as ssm_scan_bwd.  Unlike ssm_scan_fwd_complex it runs on any
 * batch * dim (the checkpointing forward always takes the single-pass kernel).
 */
ssm_status_t ssm_scan_bwd_complex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                  const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                  const float* h0, const void* dy, const float* dlast, void* du, void* ddelta,
                                  float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                                  float* dh0, struct ihipStream_t* stream);

/* Kernel paths of ssm_scan_fwd (reported by ssm_scan_fwd_plan). */
typedef enum {
  SSM_PATH_SPLIT = 0,     /* one pass; a block owns 64 channels, its waves split the states */
  SSM_PATH_SEGMENTED = 1, /* the sequence is cut into segments scanned in parallel, then
                             combined (segment aggregates -> carries -> rescan)            */
  SSM_PATH_GENERIC = 2,   /* one token at a time with scalar loads: any dstate <= 16, any
                             seqlen, any element-aligned pointers                          */
  SSM_PATH_CHUNKED = 3    /* one pass, lanes along the sequence: a wave owns one channel, its
                             lanes 16-token chunks of a tile, combined by a lane scan of the
                             chunks' affine maps and a running carry (dstate 16, either
                             discretization of B, with or without the fused conv; shapes
                             with too few channels for SSM_PATH_SPLIT)                     */
} ssm_path_t;

/*
 * ssm_scan_fwd_plan -- how ssm_scan_fwd would run a problem of this shape,
 * assuming 16-byte aligned buffers (misaligned rows fall back to
 * SSM_PATH_GENERIC at call time): the kernel path, the number of sequence
 * segments scanned in parallel per channel, the segment length in tokens (the
 * last segment ends at seqlen and holds at least 64 tokens), and the scratch
 * bytes the call takes (always 0: the prefill allocates nothing).  Pure host
 * arithmetic; any output pointer may be NULL.  Returns the same status
 * ssm_scan_fwd would return for these sizes.
 */
ssm_status_t ssm_scan_fwd_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                               ssm_dtype_t io, int* path, int64_t* segments, int64_t* segment_len,
                               int64_t* scratch_bytes);

/*
 * ssm_scan_fwd_plan_ex -- ssm_scan_fwd_plan for the other prefill entry
 * points: disc is the discretization of B (ssm_scan_fwd_ex), conv_width the
 * width of the conv fused in front (ssm_conv_scan_fwd; 0 for none).
 * SSM_ERR_UNSUPPORTED for an unknown disc or a conv_width outside 0..4.
 */
ssm_status_t ssm_scan_fwd_plan_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                  ssm_dtype_t io, ssm_disc_t disc, int64_t conv_width, int* path,
                                  int64_t* segments, int64_t* segment_len, int64_t* scratch_bytes);

/* Static English text for a status code (never NULL). */
const char* ssm_status_string(ssm_status_t status);

/* The HIP error code behind the calling thread's last SSM_ERR_HIP (0 if none). */
int ssm_last_hip_error(void);

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
