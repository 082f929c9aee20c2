/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan.
 *
 * Two operations, both from the Mamba selective SSM ("S6"):
 *
 *  ssm_scan_fwd      the whole-sequence scan.  For every (batch b, channel d)
 *                    with a diagonal A of N states and every token t:
 *                      dt      = softplus(delta[b,d,t] + bias[d])
 *                      h[n]    = exp(dt*A[d,n]) * h[n] + dt*B[b,n,t]*u[b,d,t]
 *                      y[b,d,t]= (sum_n C[b,n,t]*h[n] + D[d]*u[b,d,t])
 *                                * silu(z[b,d,t])
 *                    Sources: "Mamba & State Space Models - Guide Complet",
 *                    section 4 "Implementation du SSM selectif (S6)" (A fixed
 *                    and negative, delta/B/C per token, A_bar = exp(delta*A),
 *                    readout h.C_t + D*x_t); the johe.ru page "Mamba и State
 *                    Space Models", sections "SSM as RNN" (input term
 *                    B*delta, readout after the update) and "Selective SSM"
 *                    (output times silu(gate)); the inferownia.pl page, the
 *                    section on the selective scan (discretisation and
 *                    recurrence fused on chip, the expanded state never
 *                    written to HBM).
 *
 *  ssm_state_update  one token of the same recurrence for every (b, d), on a
 *                    state kept in HBM and updated in place: the recurrent
 *                    (decoding) mode of "SSM as RNN", whose state has a fixed
 *                    size whatever the context length.
 *
 * Conventions shared by all entry points
 *  - Every array pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates or frees memory and keeps no pointer of the
 *    caller's; scratch space for the long-sequence split comes from the
 *    caller (see the workspace below), except in ssm_scan_fwd_noalloc, which
 *    uses a fixed scratch array of the library's own.
 *  - Arrays are dense and row-major with the token axis fastest:
 *      u, delta, z, y : (batch, dim, seqlen)      B, C : (batch, dstate, seqlen)
 *      A              : (dim, dstate) fp32        D, delta_bias : (dim) fp32
 *      h0, h_final    : (batch, dim, dstate) fp32
 *    For the decode step: x, delta, z, y : (batch, dim); B, C : (batch,
 *    dstate); state : (batch, dim, dstate) fp32.  dstate (N) is 1..256 for
 *    the scan, decode and backward entry points (see ssm_scan_fwd).
 *  - One activation dtype (ssm_dtype) covers u, delta, B, C, z and y.  A, D,
 *    the bias and every state are fp32.  Arithmetic is fp32 throughout.
 *  - Base pointers must be 4-byte aligned (2-byte for bf16 activations);
 *    wider alignment enables vector loads but is not required.
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *    and return without synchronising.  Results are valid once the stream
 *    has reached that point.  Calls that overlap in time must not write the
 *    same buffers.
 *  - Errors: every call returns an ssm_status.  All argument checks run
 *    before any HIP call, so an invalid call touches neither the device nor
 *    any buffer.  A failing HIP call returns SSM_ERR_HIP.  The message of the
 *    last non-OK status on the calling thread is ssm_last_error().
 *    Nothing is thrown across this ABI.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_ABI_VERSION 1

typedef enum {
    SSM_DTYPE_F32 = 0,   /* activations in fp32 */
    SSM_DTYPE_BF16 = 1   /* activations in bfloat16; y rounded to nearest-even */
} ssm_dtype;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_INVALID_ARG = 1,  /* NULL required pointer, bad size, aliasing, misalignment */
    SSM_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement (e.g. dstate > 256) */
    SSM_ERR_WORKSPACE = 3,    /* workspace missing or smaller than ssm_scan_workspace_size() */
    SSM_ERR_HIP = 4           /* a HIP runtime call failed (no device, launch failure) */
} ssm_status;

/* flags (bitwise OR) */
#define SSM_FLAG_DELTA_SOFTPLUS 1u  /* dt = softplus(delta + bias); without it dt = delta + bias */
/* Input term by exact zero-order hold instead of Euler: dB*u = (exp(dt*A) -
 * 1)/A * B*u per state ("Mamba & State Space Models - Guide Complet",
 * section 1 "Discretisation": B_bar = (exp(dt A) - I) A^-1 B), dt*B*u where
 * A = 0.  Costs about twice the VALU work of the default Euler term. */
#define SSM_FLAG_ZOH_B 2u
/* ssm_scan_bwd only: the workspace already holds the block checkpoints and
 * the pre-gate output that ssm_scan_fwd_save wrote for the same inputs, so
 * the backward skips its own checkpoint pass (a forward recomputation). */
#define SSM_FLAG_BWD_SAVED 4u

/* Returns SSM_SCAN_ABI_VERSION. */
int ssm_abi_version(void);

/* Tokens per sequence chunk that ssm_scan_fwd will use for this shape.
 * requested_chunk = 0 lets the library choose; a positive value asks for
 * chunks of that many tokens (rounded up to the kernel's block of 1024).
 * *chunk_len_out == seqlen means the sequence is not split.  When it is
 * split, chunks are scanned in parallel from a zero state, their end states
 * are chained in order (the affine maps compose: the associative operator of
 * the Guide Complet's "Parallel Associative Scan"), and each later chunk's
 * outputs are corrected for its true incoming state (see ssm_scan_fwd). */
int ssm_scan_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                  int64_t requested_chunk, int64_t *chunk_len_out);

/* Bytes of caller-provided device workspace ssm_scan_fwd needs for this
 * shape and chunk request (0 when the sequence is not split). */
int ssm_scan_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                            int64_t seqlen, int64_t requested_chunk,
                            size_t *bytes);

/* Selective scan forward.
 *  u, delta, B, C      required, activation dtype
 *  A                   required fp32 (dim, dstate); used as given (negative
 *                      for a decaying state; positive values are accepted)
 *  D                   nullable fp32 (dim): skip term D*u, added before the gate
 *  z                   nullable, activation dtype: gate y * silu(z)
 *  delta_bias          nullable fp32 (dim), added to delta before softplus
 *  flags               SSM_FLAG_DELTA_SOFTPLUS and/or SSM_FLAG_ZOH_B
 *  h0                  nullable fp32 initial state (zero state if NULL)
 *  y                   required output, activation dtype; must not overlap
 *                      any input
 *  h_final             nullable fp32 output: the state after the last token;
 *                      must not overlap h0
 *  batch, dim, seqlen  >= 1;  dstate 1..256 (the S6 module's d_state,
 *                      "Mamba & State Space Models - Guide Complet", section
 *                      4, and the larger states of its section 5; 16, the
 *                      pages' value, runs the tuned instances, with A and the
 *                      carried state in scalar registers; any other count
 *                      holds state n in lane n % 64 of vector register n / 64
 *                      of a wave).  The same range holds for every scan,
 *                      decode and backward entry point below
 *  requested_chunk     0 = automatic; see ssm_scan_plan
 *  workspace           device scratch of >= ssm_scan_workspace_size() bytes,
 *                      256-byte aligned; may be NULL when that size is 0.  Its
 *                      contents on entry do not matter; it is in use until
 *                      the enqueued work completes.
 *  stream              hipStream_t or NULL
 * Long sequences with few channels are split into chunks (ssm_scan_plan).
 * A later chunk starts from a zero state; its outputs are then corrected by
 * silu(z_t) * sum_n C[t,n] * exp(A[n]*S_t) * h_in[n], S_t being the running
 * sum of dt inside the chunk, until every decay factor exp(A[n]*S_t) has
 * fallen below 2^-40 (valid because the factors never grow when A <= 0 and
 * dt >= 0).  When a channel has some A > 0, or softplus is off so dt may be
 * negative, the correction runs over the whole chunk. */
int ssm_scan_fwd(const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *z,
                 const float *delta_bias, unsigned flags, const float *h0,
                 void *y, float *h_final, int64_t batch, int64_t dim,
                 int64_t dstate, int64_t seqlen, int dtype,
                 int64_t requested_chunk, void *workspace,
                 size_t workspace_bytes, void *stream);

/* ssm_scan_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, computation and results, but no workspace argument.
 * A sequence that ssm_scan_plan splits into chunks keeps its chunk states in
 * a fixed scratch array inside the library (16 MiB per GPU, held by each GPU
 * the library runs on until the process ends), so a split whose workspace
 * (ssm_scan_workspace_size) exceeds 16 MiB returns SSM_ERR_WORKSPACE, before
 * any HIP call.  Nothing is allocated, freed or cleared: every chunk state
 * is written before it is read.  All calls on one GPU share that GPU's
 * scratch, so calls whose work may overlap in time on one GPU (on different
 * streams, or from different threads) race and must be serialised by the
 * caller; calls enqueued in order on one stream are safe.  The scratch
 * belongs to the device of `stream` (the current device for NULL); its
 * address is looked up on the first call on that device. */
int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A,
                         const void *B, const void *C, const float *D,
                         const void *z, const float *delta_bias, unsigned flags,
                         const float *h0, void *y, float *h_final,
                         int64_t batch, int64_t dim, int64_t dstate,
                         int64_t seqlen, int dtype, int64_t requested_chunk,
                         void *stream);

/* Selective scan whose input u is produced inside the kernel from the
 * pre-convolution activations x by the Mamba block's depthwise causal
 * convolution and SiLU ("Mamba & State Space Models - Guide Complet",
 * section 4 architecture figure: Conv1D -> SiLU -> SSM; section 7: a
 * depthwise Conv1d with padding d_conv - 1 whose output is trimmed to the
 * first L positions; d_conv = 4 on the inferownia.pl page):
 *   u[b,d,t] = silu(conv_b[d] + sum_{k<d_conv} conv_w[d,k] * x[b,d,t-d_conv+1+k])
 * with x = 0 before t = 0; then exactly ssm_scan_fwd with that u (the D
 * skip uses u).  u never touches HBM.
 *  x        required, activation dtype (batch, dim, seqlen)
 *  conv_w   required fp32 (dim, d_conv); conv_b nullable fp32 (dim)
 *  d_conv   1..4 (SSM_ERR_UNSUPPORTED above 4)
 *  dstate   1..64 here (SSM_ERR_UNSUPPORTED above: with more states the
 *           fused prologue gave intermittent wrong outputs near the start
 *           of the sequence, cause not yet found)
 * All other arguments, conventions, the chunk plan and the workspace are
 * those of ssm_scan_fwd. */
int ssm_conv_scan_fwd(const void *x, const float *conv_w, const float *conv_b,
                      int d_conv, const void *delta, const float *A,
                      const void *B, const void *C, const float *D,
                      const void *z, const float *delta_bias, unsigned flags,
                      const float *h0, void *y, float *h_final, int64_t batch,
                      int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                      int64_t requested_chunk, void *workspace,
                      size_t workspace_bytes, void *stream);

/* One decoding step, in place on `state`.
 *  state      required fp32 (batch, dim, dstate): read, advanced by one token
 *             and written back
 *  x, delta   required, activation dtype (batch, dim)
 *  A          required fp32 (dim, dstate)
 *  B, C       required, activation dtype (batch, dstate)
 *  D, z, delta_bias, flags   as for ssm_scan_fwd
 *  y          required output, activation dtype (batch, dim)
 * batch at most 131070 and batch * dim below 2^32 in this build (else
 * SSM_ERR_UNSUPPORTED).  Applying it to tokens 0..L-1 in order reproduces
 * ssm_scan_fwd's y and, in `state`, its h_final. */
int ssm_state_update(float *state, const void *x, const void *delta,
                     const float *A, const void *B, const void *C,
                     const float *D, const void *z, const float *delta_bias,
                     unsigned flags, void *y, int64_t batch, int64_t dim,
                     int64_t dstate, int dtype, void *stream);

/* One decoding step with the fused conv prologue of ssm_conv_scan_fwd: the
 * token's input first goes through the depthwise causal conv1d and SiLU
 * (the Mamba block's Conv1D -> SiLU before the SSM; "Mamba & State Space
 * Models - Guide Complet", sections 4 and 7), whose window of the previous
 * d_conv - 1 inputs is kept per channel, then the step of ssm_state_update:
 *   u     = silu(conv_b[d] + sum_k conv_w[d, k] * w_k),
 *           w = (conv_state[b, d, 0 .. d_conv-2], x[b, d])   (oldest first)
 *   then ssm_state_update with u in place of x (D skip on u, gate by z);
 *   conv_state[b, d, :] <- (w_1 .. w_{d_conv-1}), the window moved by one.
 * A fresh sequence starts with conv_state zero (inputs before t = 0 count
 * as 0, as in ssm_conv_scan_fwd), so T steps reproduce ssm_conv_scan_fwd
 * over the same T tokens.
 *  conv_state     in/out, activation dtype (batch, dim, d_conv - 1);
 *                 may be NULL only when d_conv = 1
 *  conv_w, conv_b fp32 (dim, d_conv) and (dim); conv_b nullable
 *  d_conv         1..4 (larger: SSM_ERR_UNSUPPORTED)
 *  the rest       as for ssm_state_update; conv_state must not overlap any
 *                 other argument. */
int ssm_conv_state_update(float *state, void *conv_state, const void *x,
                          const float *conv_w, const float *conv_b, int d_conv,
                          const void *delta, const float *A, const void *B,
                          const void *C, const float *D, const void *z,
                          const float *delta_bias, unsigned flags, void *y,
                          int64_t batch, int64_t dim, int64_t dstate, int dtype,
                          void *stream);


/* Bytes of caller-provided device workspace ssm_scan_bwd needs for this
 * shape and activation dtype: the block-start checkpoints
 * (batch*dim*ceil(seqlen/1024)*dstate fp32), the pre-gate output
 * (batch*dim*seqlen, activation dtype), partial sums of dB and dC (2 *
 * batch*slots*dstate*seqlen fp32: a workgroup holds 8 channels, and takes
 * ceil(groups/slots) of the groups = ceil(dim/8) one after another, adding
 * into one row; slots is the smallest count that costs no extra round of 256
 * resident workgroups: 128 of 640 groups for the 2.8B layer's batch of 2),
 * and per-(channel, chunk) partials of dA, dD and the bias.
 * Shapes with few channels and long rows split the sequence (below) and
 * add, each under 1 % of the partial sums: the checkpoint pass's per-block
 * dt sums and per-chunk states, and the sweep's per-chunk adjoints (3 x
 * batch*dim*chunks*dstate fp32). */
int ssm_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                int64_t seqlen, int dtype, size_t *bytes);

/* How ssm_scan_bwd will run this shape (no HIP call), in plan_out[4]:
 *  [0] tokens per chunk of the reverse sweep (seqlen: not split)
 *  [1] tokens per chunk of its checkpoint pass (a forward scan; seqlen: not
 *      split)
 *  [2] dB/dC partial-sum rows per batch entry (the workspace's partial sums)
 *  [3] launches of the sweep kernel: launch k takes channel groups
 *      k*[2] .. (k+1)*[2]-1 (8 channels a group), each adding into its
 *      row, so the rows are sums in a fixed order
 * Errors as ssm_scan_bwd_workspace_size (NULL plan_out: SSM_ERR_INVALID_ARG). */
int ssm_scan_bwd_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                      int64_t *plan_out);

/* Backward pass of ssm_scan_fwd: the gradients of
 * a scalar loss with respect to every input, given its gradient dy with
 * respect to y and dh_final (nullable -> 0) with respect to the final state.
 * The chain rule through the recurrence, taken in reverse token order; the
 * states are recomputed from block-start checkpoints rather than stored
 * (the inferownia.pl page on the selective scan, "Cena selekcji": the
 * backward pass recomputes the intermediate states).  Definitions:
 *   lambda_t = dL/dh_t = dy_t silu(z_t) C_t + exp(dt_{t+1} A) lambda_{t+1},
 *              lambda_{L-1} also gets dh_final
 *   du_t     = sum_n lambda_t,n dt_t B_t,n + dy_t silu(z_t) D
 *   ddelta_t = (sum_n lambda_t,n (B_t,n u_t + A_n exp(dt_t A_n) h_t-1,n))
 *              * sigmoid(delta_t + bias)        (without softplus: * 1)
 *   dA_n     = sum_b,t lambda_t,n exp(dt_t A_n) h_t-1,n dt_t
 *   dB_t,n   = sum_d lambda_t,n dt_t u_t     dC_t,n = sum_d dy_t silu(z_t) h_t,n
 *   dD       = sum_b,t dy_t silu(z_t) u_t    dbias  = sum_b,t ddelta_t
 *   dz_t     = dy_t yc_t silu'(z_t), yc_t = sum_n C_t,n h_t,n + D u_t
 *   dh0      = exp(dt_0 A) lambda_0
 * With SSM_FLAG_ZOH_B the input coefficient dt becomes c_t,n = (exp(dt_t A_n)
 * - 1)/A_n ("Mamba & State Space Models - Guide Complet", section 1), with
 * dc/ddt = exp(dt A) and dc/dA = (dt exp(dt A) - c)/A (dt^2/2 at A = 0):
 *   du_t     = sum_n lambda_t,n c_t,n B_t,n + dy_t silu(z_t) D
 *   ddelta_t = (sum_n lambda_t,n exp(dt_t A_n) (B_t,n u_t + A_n h_t-1,n))
 *              * sigmoid(delta_t + bias)
 *   dA_n     = sum_b,t lambda_t,n (exp(dt_t A_n) h_t-1,n dt_t
 *              + dc/dA_n B_t,n u_t)
 *   dB_t,n   = sum_d lambda_t,n c_t,n u_t
 * Arguments:
 *  u, delta, A, B, C, D, z, delta_bias, flags, h0   as for ssm_scan_fwd
 *                      (flags: SSM_FLAG_DELTA_SOFTPLUS, SSM_FLAG_ZOH_B,
 *                      SSM_FLAG_BWD_SAVED)
 *  dy                  required, activation dtype (batch, dim, seqlen)
 *  dh_final            nullable fp32 (batch, dim, dstate)
 *  du, ddelta          required outputs, activation dtype (batch, dim, seqlen)
 *  dA                  required output fp32 (dim, dstate)
 *  dB, dC              required outputs fp32 (batch, dstate, seqlen)
 *  dD, ddelta_bias     nullable outputs fp32 (dim); when given they receive
 *                      the gradient (with respect to a zero D / bias where
 *                      D / delta_bias is NULL)
 *  dz                  nullable output, activation dtype; only with z
 *  dh0                 nullable output fp32 (batch, dim, dstate)
 *  workspace           device scratch of >= ssm_scan_bwd_workspace_size()
 *                      bytes, 256-byte aligned, in use until the enqueued work
 *                      completes; its contents on entry do not matter, except
 *                      with SSM_FLAG_BWD_SAVED (flags may add it): then its
 *                      checkpoint region must hold what ssm_scan_fwd_save
 *                      wrote for the same u, delta, A, B, C, D, delta_bias,
 *                      h0 and softplus flag (not checked)
 * No output may overlap an input, another output or the workspace.
 * A wave takes one channel.  When the channels alone give the GPU fewer
 * than two rounds of waves and the rows hold at least 16384 tokens, the
 * sequence is cut into up to 16 chunks of whole 1024-token blocks, swept in
 * parallel: each chunk after the first first yields, from a zero input on
 * its right, the dL/dh it passes to its left and its decay product (over
 * its decay horizon: contributions below 2^-40 are dropped when every A < 0
 * under softplus), these are chained from the last chunk, and each chunk
 * is swept from its true incoming dL/dh.  The checkpoint pass is split like
 * ssm_scan_fwd.  The results then differ from the unsplit order of
 * summation by rounding only. */
int ssm_scan_bwd(const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *z,
                 const float *delta_bias, unsigned flags, const float *h0,
                 const void *dy, const float *dh_final, void *du, void *ddelta,
                 float *dA, float *dB, float *dC, float *dD,
                 float *ddelta_bias, void *dz, float *dh0, int64_t batch,
                 int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Forward pass for training: the same computation and outputs (y, h_final)
 * as ssm_scan_fwd, which in addition keeps what the backward recomputes
 * otherwise -- the state entering every 1024-token block and the output
 * before the gate -- in the backward's workspace.  It splits long rows of
 * few channels exactly as ssm_scan_fwd with requested_chunk = 0 does (its
 * chunk buffers are in that workspace), the checkpoints and the pre-gate
 * output fixed up like y.  A following ssm_scan_bwd on the same inputs with
 * SSM_FLAG_BWD_SAVED and that workspace then skips its checkpoint pass.
 * (The inferownia.pl page on Mamba, section "Cena selekcji": the backward
 * recomputes the intermediate states rather than storing them; here one
 * state per block is kept.)
 *  arguments as for ssm_scan_fwd, except:
 *  flags           SSM_FLAG_DELTA_SOFTPLUS and/or SSM_FLAG_ZOH_B (the following
 *                  ssm_scan_bwd must be given the same flags)
 *  bwd_workspace   required, >= ssm_scan_bwd_workspace_size() bytes for the
 *                  same shape and dtype, 256-byte aligned, not overlapping any
 *                  argument; its checkpoint region is overwritten
 * The shape limits of ssm_scan_bwd apply. */
int ssm_scan_fwd_save(const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z,
                      const float *delta_bias, unsigned flags, const float *h0,
                      void *y, float *h_final, int64_t batch, int64_t dim,
                      int64_t dstate, int64_t seqlen, int dtype, void *bwd_workspace,
                      size_t bwd_workspace_bytes, void *stream);

/* Bytes of caller-provided device workspace ssm_conv_scan_bwd needs: that
 * of ssm_scan_bwd_workspace_size for the same shape and dtype, then u and
 * its gradient (batch*dim*seqlen each, activation dtype) and batch*dim*5
 * fp32 per-row sums of the conv's gradients. */
int ssm_conv_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                     int64_t seqlen, int dtype, size_t *bytes);

/* Backward pass of ssm_conv_scan_fwd: the gradients of ssm_scan_bwd, with
 * the gradient of u carried back through the SiLU and the depthwise causal
 * convolution of the Mamba block's prologue ("Mamba & State Space Models -
 * Guide Complet", section 4 architecture figure and section 7):
 *   pre_t    = conv_b + sum_k conv_w[k] x_{t-d_conv+1+k},  u_t = silu(pre_t)
 *   g_t      = du_t silu'(pre_t)       (du_t as ssm_scan_bwd defines it)
 *   dx_s     = sum_k conv_w[k] g_{s+d_conv-1-k}
 *   dconv_w[d,k] = sum_b,t g_t x_{t-d_conv+1+k},  dconv_b[d] = sum_b,t g_t
 * u is formed again from x into the workspace (in the activation dtype: for
 * bf16 runs it is the forward's fp32 u rounded to nearest even) and the
 * scan's backward runs on it.
 *  x, conv_w, conv_b, d_conv     as for ssm_conv_scan_fwd
 *  delta ... dh_final, flags     as for ssm_scan_bwd (SSM_FLAG_BWD_SAVED is
 *                                refused: there is no saving conv forward)
 *  dx                required output, activation dtype (batch, dim, seqlen)
 *  dconv_w           required output fp32 (dim, d_conv)
 *  dconv_b           nullable output fp32 (dim)
 *  ddelta ... dh0    as for ssm_scan_bwd (du is replaced by dx)
 *  workspace         >= ssm_conv_scan_bwd_workspace_size() bytes, 256-byte
 *                    aligned
 * Conventions, limits and errors as for ssm_scan_bwd; every check runs
 * before the first kernel is enqueued. */
int ssm_conv_scan_bwd(const void *x, const float *conv_w, const float *conv_b,
                      int d_conv, const void *delta, const float *A,
                      const void *B, const void *C, const float *D,
                      const void *z, const float *delta_bias, unsigned flags,
                      const float *h0, const void *dy, const float *dh_final,
                      void *dx, float *dconv_w, float *dconv_b, void *ddelta,
                      float *dA, float *dB, float *dC, float *dD,
                      float *ddelta_bias, void *dz, float *dh0, int64_t batch,
                      int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of caller-provided device workspace ssm_ssd_fwd needs: per chunk of
 * 64 tokens and group, the causal G = C^T B (64 x 64 fp32) and C
 * transposed (64 x dstate bf16). */
int ssm_ssd_workspace_size(int64_t batch, int64_t ngroups, int64_t dstate,
                           int64_t seqlen, size_t *bytes);

/* Mamba-2 "SSD" (state space dual) forward ("Mamba & State Space Models -
 * Guide Complet", section 5: d_state 64-256; y = (L o S) u with L the
 * causal mask and S a structured semiseparable matrix), with one scalar
 * decay per head and B, C shared by the heads of a group:
 *   dt[b,h,t]  = softplus(dt_raw[b,h,t] + dt_bias[h])   (flag; else + only)
 *   S[t,s]     = (C[b,g,:,t] . B[b,g,:,s]) exp(A[h] sum_{s<r<=t} dt_r) dt_s
 *   y[b,h,p,t] = (sum_{s<=t} S[t,s] x[b,h,p,s] + C[b,g,:,t] . (exp(A[h]
 *                sum_{r<=t} dt_r) h0[b,h,p,:]) + D[h] x[b,h,p,t]) silu(z)
 *   h_final    = the state after the last token (the same recurrence as
 *                ssm_scan_fwd with A[h] for every state)
 * computed in chunks of 64 tokens: the masked products inside a chunk and
 * the carried head state run on the matrix cores (bf16 operands, fp32
 * accumulation; the carried state is fp32).
 *  x, z, y        bf16 (batch, nheads, headdim, seqlen); z nullable
 *  dt             bf16 (batch, nheads, seqlen)
 *  A, D, dt_bias  fp32 (nheads); D, dt_bias nullable
 *  B, C           bf16 (batch, ngroups, dstate, seqlen); nheads % ngroups == 0
 *  h0, h_final    fp32 (batch, nheads, headdim, dstate), nullable
 *  flags          SSM_FLAG_DELTA_SOFTPLUS (SSM_FLAG_ZOH_B: SSM_ERR_UNSUPPORTED)
 *  dtype          SSM_DTYPE_BF16 (SSM_DTYPE_F32: SSM_ERR_UNSUPPORTED)
 *  headdim 64 and dstate 64, 128 or 256, dstate * seqlen < 2^30 in this
 *  build (else SSM_ERR_UNSUPPORTED); workspace as ssm_ssd_workspace_size(),
 *  256-byte aligned.  Conventions as for ssm_scan_fwd. */
int ssm_ssd_fwd(const void *x, const void *dt, const float *A, const void *B,
                const void *C, const float *D, const void *z,
                const float *dt_bias, unsigned flags, const float *h0, void *y,
                float *h_final, int64_t batch, int64_t nheads, int64_t headdim,
                int64_t ngroups, int64_t dstate, int64_t seqlen, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char *ssm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
