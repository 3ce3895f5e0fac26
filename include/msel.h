/*
 * msel.h -- C ABI of the MI355X (gfx950) selective-scan library, libmsel.so.
 *
 * The library computes the selective state-space scan at the heart of Mamba, per batch row b,
 * channel d and state n:
 *
 *   Delta_t = softplus(delta_t + bias[d])   (or delta_t + bias[d] when the softplus flag is 0)
 *   dA_t    = exp(Delta_t * A[d,n])         zero-order hold for the transition
 *   dB_t x_t = Delta_t * B[b,n,t] * u_t      Euler for the input
 *   h_t     = dA_t * h_{t-1} + dB_t x_t      the selective recurrence (h_{-1} = h0 or 0)
 *   y_t     = sum_n C[b,n,t] * h_t + D[d] * u_t
 *   out_t   = y_t * silu(z_t)                (out_t = y_t when z is NULL)
 *
 * Sources (five web pages collected on "mamba paper"): the selection mechanism that makes
 * Delta, B and C functions of the token (page 1, abstract paragraph); the mix of zero-order
 * hold and Euler discretization (page 5, Mamba-3 post, discretization bullet); the recurrent
 * mode that reads one time step at a time (page 3); the work-efficient parallel scan of the
 * recurrence (page 1); the fused scan that splits long sequences into chunks and continues
 * from the intermediate state of the previous chunk (page 4, Appendix D "Hardware-aware
 * Algorithm For Selective SSMs", Speed paragraph); states recomputed, not stored, in the
 * backward pass (page 1; page 4 Appendix D, Memory paragraph); the cache that keeps the SSM
 * state after the scan (page 1, page 2).  The D skip term inside the gate and the gate itself
 * follow the plainest reading of that description.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device, contiguous, row-major.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no state between
 *    calls (but for the device counters read by msel_ring_timeouts and, in the checked build,
 *    msel_bound_violations), is re-entrant, and never
 *    synchronizes: work is enqueued on `stream` and the call returns.  Errors in the arguments are detected on the host before anything is
 *    enqueued; the return value is then not MSEL_OK and no device memory is touched.
 *  - Inputs are read-only.  Outputs must not be the same pointer as any input (checked),
 *    except where a field says otherwise (a state updated in place).
 *  - Layouts:
 *      u, delta, z, out                  [batch, dim, seqlen]     activation dtype
 *      B, C                              [batch, dstate, seqlen]  activation dtype
 *      A                                 [dim, dstate]            fp32
 *      D, delta_bias                     [dim]                    fp32
 *      h0, final_state                   [batch, dim, dstate]     fp32
 *      chunk_states                      [batch, dim, n_chunks, dstate] fp32,
 *                                        n_chunks = ceil(seqlen / msel_chunk_len()),
 *                                        entry c = state before time step c*chunk_len
 *  - Activation dtype: MSEL_F32 (fp32) or MSEL_BF16 (bfloat16, stored 2 bytes, rounded to
 *    nearest even on output).  The state, every accumulation and A, D, bias are fp32.
 *  - Activation pointers must be 16-byte aligned.
 */
#ifndef MSEL_H
#define MSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t and hipEvent_t, declared the same way the HIP runtime declares them. */
typedef struct ihipStream_t *hipStream_t;
typedef struct ihipEvent_t *hipEvent_t;

#define MSEL_ABI_VERSION 1

typedef enum {
    MSEL_OK = 0,
    MSEL_ERR_NULL = 1,        /* a required pointer is NULL                                */
    MSEL_ERR_SHAPE = 2,       /* a size is < 1, or above the supported range (seqlen up to  */
                              /* MSEL_MAX_SEQLEN, batch*dim up to 2^30)                     */
    MSEL_ERR_DTYPE = 3,       /* dtype is not MSEL_F32 / MSEL_BF16, or a 0/1 flag is not 0/1 */
    MSEL_ERR_ALIGN = 4,       /* an activation pointer is not 16-byte aligned              */
    MSEL_ERR_UNSUPPORTED = 5, /* dstate outside 1..MSEL_MAX_DSTATE, or a convolution width  */
                              /* outside 1..MSEL_MAX_CONV_WIDTH                             */
    MSEL_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than msel_scan_bwd_workspace_bytes */
    MSEL_ERR_ALIAS = 7,       /* an output pointer equals an input pointer                 */
    MSEL_ERR_HIP = 8,         /* the HIP runtime reported an error at launch               */
    MSEL_ERR_VERSION = 9,     /* args->abi_version != MSEL_ABI_VERSION                     */
    MSEL_ERR_TOO_LARGE = 10   /* msel_scan_bwd_noalloc: the problem's workspace would exceed */
                              /* MSEL_NOALLOC_SCRATCH_BYTES                                 */
} msel_status;

typedef enum { MSEL_F32 = 0, MSEL_BF16 = 1 } msel_dtype;

#define MSEL_MAX_DSTATE 16
#define MSEL_MAX_SEQLEN (1 << 28)
#define MSEL_MAX_CONV_WIDTH 4

/* Problem description shared by the three entry points. */
typedef struct {
    int32_t abi_version;    /* must be MSEL_ABI_VERSION                                    */
    int32_t batch;          /* >= 1                                                        */
    int32_t dim;            /* channels, >= 1                                              */
    int32_t dstate;         /* N, 1..MSEL_MAX_DSTATE                                       */
    int32_t seqlen;         /* L, >= 1                                                     */
    int32_t dtype;          /* msel_dtype of u, delta, z, B, C, out (and of the gradients   */
                            /* du, ddelta, dz, dout)                                       */
    int32_t delta_softplus; /* 1: Delta = softplus(delta + bias); 0: Delta = delta + bias   */
    int32_t reserved;       /* must be 0                                                   */
    const void *u;          /* required                                                    */
    const void *delta;      /* required: raw Delta before bias and softplus                */
    const void *B;          /* required                                                    */
    const void *C;          /* required by fwd and bwd; ignored by chunk_carry             */
    const void *z;          /* optional gate input; NULL means out = y                     */
    const float *A;         /* required                                                    */
    const float *D;         /* optional skip weight; NULL means 0                          */
    const float *delta_bias;/* optional; NULL means 0                                      */
    const float *h0;        /* optional initial state; NULL means 0                        */
    void *out;              /* fwd: required output                                        */
    float *final_state;     /* fwd / chunk_carry: optional output, state after step L-1;
                               may equal h0 (the state is then updated in place)          */
    float *chunk_states;    /* fwd: optional output; chunk_carry: required output;          */
                            /* bwds: optional input (rebuilt into the workspace if NULL)   */
} msel_scan_args;

/* Gradients of a scalar loss given dL/dout.  Every output is overwritten, not accumulated. */
typedef struct {
    const void *dout;       /* required, activation dtype                                  */
    void *du;               /* required, activation dtype                                  */
    void *ddelta;           /* required, activation dtype: gradient w.r.t. the raw delta    */
    void *dz;               /* activation dtype; required iff args->z != NULL               */
    float *dA;              /* optional [dim, dstate]                                      */
    float *dB;              /* optional [batch, dstate, seqlen]                             */
    float *dC;              /* optional [batch, dstate, seqlen]                             */
    float *dD;              /* optional [dim] (computed even when args->D is NULL)          */
    float *ddelta_bias;     /* optional [dim]                                              */
    float *dh0;             /* optional [batch, dim, dstate]: gradient w.r.t. h0            */
} msel_scan_grads;

/* Version of this ABI, MSEL_ABI_VERSION of the built library. */
int32_t msel_abi_version(void);

/* Length T of the chunks the scan is split into (a multiple of 64); chunk_states hold one
 * state per chunk. */
int32_t msel_chunk_len(void);

/* ceil(seqlen / msel_chunk_len()), or 0 if seqlen < 1. */
int32_t msel_num_chunks(int32_t seqlen);

/* Human-readable name of a status code (static storage, never NULL). */
const char *msel_status_string(msel_status status);

/* Host-only argument checks used by the entry points below; they touch no device memory and
 * make no HIP call.  `grads` and `workspace` are checked by msel_validate_bwd only. */
msel_status msel_validate_fwd(const msel_scan_args *args);
msel_status msel_validate_chunk_carry(const msel_scan_args *args);
msel_status msel_validate_bwd(const msel_scan_args *args, const msel_scan_grads *grads,
                              const void *workspace, size_t workspace_bytes);

/* Fused forward scan (page 4, Appendix D, Speed: one fused pass, chunked with carried
 * states).  Reads u, delta, B, C, z once, keeps the state on chip, writes out, and optionally
 * final_state and chunk_states.  Deterministic: the same inputs give the same bits.
 * seqlen == 1 is the recurrent (decode) step of page 3, recurrent mode: h0 is the cached state
 * and final_state, which may be the same buffer, receives the next one; it runs a dedicated
 * kernel (one 16-lane row per channel). */
msel_status msel_scan_fwd(const msel_scan_args *args, hipStream_t stream);

/* Chunk-carry pass (page 4, Appendix D, Speed: "as long as we have the intermediate scan
 * states, we can continue the scan with the next chunk").  For every chunk it computes the
 * state transition over the chunk and the chunk's local end state, then links them,
 * H_{c+1} = P_c * H_c + S_c with H_0 = h0, into chunk_states (required) and final_state
 * (optional).  Reads u, delta, B, A, delta_bias, h0 only. */
msel_status msel_scan_chunk_carry(const msel_scan_args *args, hipStream_t stream);

/* Workspace the backward needs, in bytes, for the plan it takes (msel_scan_bwd_fused):
 *  - chunk-parallel: the adjoint carry per chunk and state, two floats per chunk, and the
 *    chunk-start states when args->chunk_states is NULL (in all about
 *    4*batch*dim*n_chunks*(dstate + 2) bytes, twice the state part without chunk_states);
 *  - fused: the adjoint carry per state, and partial sums: of dB and dC per workgroup (about
 *    256 in all, each 2*dstate*512 floats per chunk: 16 MiB per chunk at 16 states), and of
 *    dA, dD and ddelta_bias per batch row and chunk (about 68 MiB in all for 8 x 1536
 *    channels, 16 states and 2048 steps).
 * Returns 0 for invalid args.  The workspace must be 256-byte aligned; its contents on entry
 * do not matter. */
size_t msel_scan_bwd_workspace_bytes(const msel_scan_args *args);

/* Backward with recomputation (page 1; page 4 Appendix D, Memory: intermediate states are
 * recomputed, not stored).  One of two plans, chosen from the sizes (msel_scan_bwd_fused):
 *  - chunk-parallel: launches on `stream` zero-fills of the summed outputs, per-chunk
 *    summaries of the states and of the adjoint, their link across chunks (the chunk carry
 *    run forward and backward), and the chunk-parallel gradient kernel.  Only chunk-boundary
 *    values live in the workspace.  Reductions over channels (dB, dC) and over batch and time
 *    (dA, dD, ddelta_bias) use fp32 atomics, so those outputs may differ in the last bits
 *    between runs; du, ddelta, dz and dh0 are deterministic;
 *  - fused (chunk_states given, a few chunks): one gradient kernel walks each channel's chunks
 *    from the last to the first, carrying the adjoint from chunk to chunk itself (the chunk
 *    carry run backward inside it), and stores partial sums that a reduce kernel adds in a
 *    fixed order.  No summary, link or atomics: every output is deterministic.
 * The two plans compute the same values up to fp32 rounding order. */
msel_status msel_scan_bwd(const msel_scan_args *args, const msel_scan_grads *grads,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  msel_scan_bwd without the workspace
 * argument: the same launches and results, with the workspace taken from a static device
 * array of MSEL_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); on its first call on a device it looks up that device's address of the array.
 * It takes the fused plan only when that plan's workspace fits in the array, else the
 * chunk-parallel one.  Problems whose chunk-parallel workspace exceeds
 * MSEL_NOALLOC_SCRATCH_BYTES are refused with MSEL_ERR_TOO_LARGE before anything is enqueued
 * (with chunk_states given, it is about 4 * batch * dim * n_chunks * (dstate + 2) bytes;
 * rebuilt, twice the state part).
 * Every call on a device shares that device's array: calls that overlap on one device (on
 * different streams, or from different threads) race and give wrong results; calls in one
 * stream's order are safe.  The workspace needs no clearing between calls: the backward
 * writes every value of it before reading it. */
#define MSEL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
msel_status msel_scan_bwd_noalloc(const msel_scan_args *args, const msel_scan_grads *grads,
                                  hipStream_t stream);

/* msel_scan_bwd for profiling: the same launches and results, and in addition the caller's
 * events ev_begin and ev_end (hipEvent_t created by the caller; either may be NULL) are
 * recorded on `stream` immediately before and after the gradient kernel (of either plan),
 * the longest of the backward's launches, so that it can be timed on the stream it runs on.
 * A failed event record returns MSEL_ERR_HIP. */
msel_status msel_scan_bwd_profiled(const msel_scan_args *args, const msel_scan_grads *grads,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t ev_begin, hipEvent_t ev_end);

/* The backward gradient kernels (msel_scan_bwd, msel_scan_trap_bwd, msel_scan_complex_bwd)
 * hand the rows of their dB/dC accumulators from wavefront to wavefront through flags in LDS.
 * Each wait on such a flag is bounded: after a poll limit it gives up, so that a fault in the
 * hand-over ends the kernel instead of hanging the device, and it is counted.
 * msel_ring_timeouts waits for the current device to finish its work, stores in *count the
 * number of waits that gave up on that device since the last call (0 in any correct run; a
 * call with a nonzero count may have wrong dB and dC), and clears the count.  It is the one
 * place where the library keeps state: a counter per device.  MSEL_ERR_NULL if count is NULL,
 * MSEL_ERR_HIP if the runtime fails. */
msel_status msel_ring_timeouts(unsigned long long *count);

/* 1 if msel_scan_bwd takes the fused plan for these args (with a workspace of
 * msel_scan_bwd_workspace_bytes(args)), 0 if the chunk-parallel one or the args are invalid.
 * By default the fused plan is taken when chunk_states is given, n_chunks <= 4 and its grid
 * (a workgroup per batch row and group of channels, about 256 in all) has at least 128
 * workgroups.  The trapezoidal and complex backwards always take their chunk-parallel plan. */
int32_t msel_scan_bwd_fused(const msel_scan_args *args);

/* Changes that choice for calls made after it in this process: mode 0 restores the default,
 * 1 takes the fused plan wherever it applies (chunk_states given), -1 never.  For tests that
 * compare the two plans at any size.  msel_scan_bwd_workspace_bytes follows the setting, so
 * size a workspace after setting it.  Not thread-safe against concurrent backward calls. */
void msel_set_bwd_fused(int32_t mode);

/* Sets the poll limit of those waits for calls made after it in this process: `polls`
 * polls, each after a sleep of about 64 clocks; 0 restores the default of 2^22 polls (about
 * 0.1 s).  For tests of the timeout path, which set a tiny limit so that waits give up while
 * every kernel still ends normally.  Not thread-safe against concurrent backward calls. */
void msel_set_ring_spin_limit(uint32_t polls);

/* ------------------------------------------------------------------------------------------
 * The checked build.  libmsel_checked.so is the same library compiled with MSEL_CHECKED: every
 * index that a kernel forms into a global buffer or an LDS array is compared with the extent
 * of what it indexes.  An index out of range is counted in a device record of its source file
 * and replaced by 0, so the access stays inside the buffer and the kernel ends normally (a
 * failed check never traps, faults or hangs).  Outputs are those of the release build; the
 * kernels are slower.  For tests and debugging (these checks are not from the pages).
 */

/* 1 in the checked build, 0 in the release build. */
int msel_checked_build(void);

/* Waits for the current device to finish its work, then stores the number of out-of-range
 * indexes that the kernels met on that device since the last call in *count and, when the
 * count is nonzero, where the first one was: *file (1 scan_fwd.hip, 2 chunk_carry.hip,
 * 3 scan_bwd.hip, 4 conv1d.hip, 5 scan_cplx.hip, 6 scan_cplx_bwd.hip; the first file with a
 * nonzero count) and *line (its source line); 0 and 0 otherwise.  Clears the records.  The
 * release build always reports 0.  MSEL_ERR_NULL if a pointer is NULL, MSEL_ERR_HIP if the
 * runtime fails. */
msel_status msel_bound_violations(unsigned long long *count, uint32_t *file, uint32_t *line);

/* Checked build: enqueues on `stream` one kernel that forms index 1 of a one-element device
 * array, which its check must count (file 1) and redirect to element 0.  The release build
 * returns MSEL_ERR_UNSUPPORTED and enqueues nothing. */
msel_status msel_bounds_selftest(hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * The exponential-trapezoidal variant of the scan (Mamba-3).
 *
 * The input integral over a step is taken from both ends of the interval and mixed by a
 * data-dependent weight lambda, the earlier end carried over the step by the exact transition
 * (page 5, the Mamba-3 post, first bullet on the new discretization):
 *
 *   h_t = dA_t h_{t-1} + Delta_t * ( lambda_t B_t u_t + (1 - lambda_t) dA_t B_{t-1} u_{t-1} )
 *
 * with everything else as above.  lambda_t = 1 is the zero-order-hold/Euler scan of
 * msel_scan_fwd; lambda_t = 1/2 is the trapezoidal rule.  The step before the first takes u_prev
 * and B_prev (the last step of a sequence being continued, e.g. the previous decode step), or 0.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
    const void *lambda;     /* required [batch, dim, seqlen], activation dtype, in [0, 1],   */
                            /* 16-byte aligned                                             */
    const void *u_prev;     /* optional [batch, dim], activation dtype: u at step -1         */
    const void *B_prev;     /* optional [batch, dstate], activation dtype: B at step -1      */
} msel_trap_args;

/* Host-only checks of msel_scan_trap_fwd's arguments (those of msel_validate_fwd, and the
 * trapezoidal inputs'). */
msel_status msel_validate_trap_fwd(const msel_scan_args *args, const msel_trap_args *trap);

/* Fused forward scan with the exponential-trapezoidal rule: the same single pass, outputs
 * (out, final_state, chunk_states) and conventions as msel_scan_fwd, reading lambda as one
 * more input stream.  seqlen == 1 is the decode step (state in place allowed).  Its backward
 * is msel_scan_trap_bwd, its chunk-carry pass msel_scan_trap_chunk_carry. */
msel_status msel_scan_trap_fwd(const msel_scan_args *args, const msel_trap_args *trap,
                               hipStream_t stream);

/* Host-only checks of msel_scan_trap_chunk_carry's arguments (those of
 * msel_validate_chunk_carry, and the trapezoidal inputs'). */
msel_status msel_validate_trap_chunk_carry(const msel_scan_args *args,
                                           const msel_trap_args *trap);

/* Chunk-carry pass of the exponential-trapezoidal rule (page 4, Appendix D, Speed: the scan
 * continues chunk by chunk from the intermediate state; page 5, the rule): chunk_states
 * (required) and final_state (optional) equal to msel_scan_trap_fwd's for the same inputs,
 * from u, delta, lambda, B, A, delta_bias, h0, u_prev and B_prev alone (C, z, D unread).
 * Per chunk, the transition and the local end state in closed form, where each step's input
 * also reaches back to the previous step's B and u; then the link. */
msel_status msel_scan_trap_chunk_carry(const msel_scan_args *args, const msel_trap_args *trap,
                                       hipStream_t stream);

/* The trapezoidal variant's gradients beyond msel_scan_grads.  Overwritten, not
 * accumulated. */
typedef struct {
    void *dlambda;          /* required [batch, dim, seqlen], activation dtype, 16-byte     */
                            /* aligned: gradient w.r.t. lambda                             */
    float *du_prev;         /* optional [batch, dim]: gradient w.r.t. u_prev                */
    float *dB_prev;         /* optional [batch, dstate]: gradient w.r.t. B_prev             */
} msel_trap_grads;

/* Host-only checks of msel_scan_trap_bwd's arguments (those of msel_validate_bwd, the
 * trapezoidal inputs and gradients, no output equal to an input, the
 * workspace or another output). */
msel_status msel_validate_trap_bwd(const msel_scan_args *args, const msel_trap_args *trap,
                                   const msel_scan_grads *grads,
                                   const msel_trap_grads *trap_grads, const void *workspace,
                                   size_t workspace_bytes);

/* Backward of msel_scan_trap_fwd with recomputation (page 1; page 4 Appendix D, Memory):
 * the same three launches as msel_scan_bwd and the same outputs, plus trap_grads.
 * args->chunk_states holds msel_scan_trap_fwd's chunk states for the same inputs, or is NULL:
 * then msel_scan_trap_chunk_carry's pass rebuilds them into the front of the workspace first.
 * The workspace is msel_scan_bwd_workspace_bytes(args).  du_prev and dB_prev let
 * a caller that split a sequence across calls carry the gradient into the earlier call.
 * Same determinism as msel_scan_bwd (dB_prev is an fp32 atomic sum over channels). */
msel_status msel_scan_trap_bwd(const msel_scan_args *args, const msel_trap_args *trap,
                               const msel_scan_grads *grads, const msel_trap_grads *trap_grads,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * The complex-valued (rotational) variant of the scan (Mamba-3).
 *
 * A complex state recovers state tracking (parity) that the real one cannot do; it is written
 * as a scaling and a rotation in a plane (page 5, the Mamba-3 post, second bullet).  States
 * (2j, 2j+1) of a channel are the real and imaginary parts of one complex state, A[d, 2j] and
 * A[d, 2j+1] the real and imaginary parts of its rate, rows 2j and 2j+1 of B and C its input
 * and readout weights:
 *
 *   h_t = exp(Delta_t (A_re + i A_im)) h_{t-1} + Delta_t u_t (B_{2j} + i B_{2j+1})
 *   y_t = sum_j ( C_{2j} Re h_t + C_{2j+1} Im h_t ) + D u_t,    out_t = y_t silu(z_t)
 *
 * The arguments, layouts and outputs are msel_scan_fwd's (h0, final_state and chunk_states
 * hold (Re, Im) pairs); dstate must be even (else MSEL_ERR_SHAPE).  With every A[d, 2j+1] = 0
 * this is msel_scan_fwd with A[d, 2j+1] = A[d, 2j].  seqlen == 1 is the decode step (state in
 * place allowed).  Its backward is msel_scan_complex_bwd, its chunk-carry pass
 * msel_scan_complex_chunk_carry.
 * ---------------------------------------------------------------------------------------- */
msel_status msel_validate_complex_fwd(const msel_scan_args *args);
msel_status msel_scan_complex_fwd(const msel_scan_args *args, hipStream_t stream);

/* Host-only checks of msel_scan_complex_chunk_carry's arguments (those of
 * msel_validate_chunk_carry, and dstate even). */
msel_status msel_validate_complex_chunk_carry(const msel_scan_args *args);

/* Chunk-carry pass of the complex-valued scan (page 4, Appendix D, Speed; page 5, the complex
 * state as a scaling and a rotation): chunk_states (required) and final_state (optional)
 * equal to msel_scan_complex_fwd's for the same inputs, from u, delta, A, B, delta_bias and h0
 * alone.  Per chunk, the complex transition exp(A * sum of Delta) and the local end state in
 * closed form; then the link, a complex product per state pair. */
msel_status msel_scan_complex_chunk_carry(const msel_scan_args *args, hipStream_t stream);

/* Host-only checks of msel_scan_complex_bwd's arguments: those of msel_validate_bwd and
 * dstate even. */
msel_status msel_validate_complex_bwd(const msel_scan_args *args, const msel_scan_grads *grads,
                                      const void *workspace, size_t workspace_bytes);

/* Backward of msel_scan_complex_fwd with recomputation (page 1; page 4 Appendix D, Memory):
 * zero-fills, per-chunk adjoint summaries, their link across chunks (with conjugated
 * transitions) and a gradient kernel with one wavefront per state pair.  args->chunk_states
 * holds msel_scan_complex_fwd's chunk states for the same inputs, or is NULL: then
 * msel_scan_complex_chunk_carry's pass rebuilds them into the front of the workspace first.
 * The workspace is msel_scan_bwd_workspace_bytes(args).  The outputs are msel_scan_grads' (dA and
 * dh0 interleaved (Re, Im) like A and h0), with msel_scan_bwd's determinism. */
msel_status msel_scan_complex_bwd(const msel_scan_args *args, const msel_scan_grads *grads,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * The short causal convolution and activation that produce the scan's input.
 *
 * The selective SSM block runs an input projection, a short convolution, an activation, the
 * scan and an output projection; the backward recomputes the convolution and activation
 * outputs rather than storing them (page 4, Appendix D, Memory paragraph).  The layer's cache
 * keeps a convolutional state beside the SSM state, and the fast path calls a dedicated causal
 * convolution kernel (page 1, the paragraphs on the cache and on the kernels).  Per batch row
 * b, channel d and step t, with W taps:
 *
 *   xe      = [state_in[b,d,0..W-2], x[b,d,0..L-1]]     the W-1 earlier inputs, oldest first
 *   pre_t   = bias[d] + sum_k weight[d,k] * xe[t+k]      tap W-1 multiplies x_t (causal)
 *   out_t   = silu(pre_t) = pre_t * sigmoid(pre_t)       (out_t = pre_t when activation = 0)
 *   state_out = the last W-1 entries of xe               (the cache after the call)
 *
 * Layouts: x, out, dout, dx [batch, dim, seqlen] in the activation dtype (16-byte aligned);
 * weight [dim, width] fp32; bias [dim] fp32; state_in, state_out [batch, dim, width-1] in the
 * activation dtype (copies of inputs, so exact); dweight, dbias, dstate_in fp32.  The
 * convolution is computed in fp32.  With width 1 the state pointers are ignored.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
    int32_t abi_version;    /* must be MSEL_ABI_VERSION                                    */
    int32_t batch;          /* >= 1                                                        */
    int32_t dim;            /* channels, >= 1                                              */
    int32_t seqlen;         /* L, 1..MSEL_MAX_SEQLEN                                       */
    int32_t width;          /* W, 1..MSEL_MAX_CONV_WIDTH                                   */
    int32_t dtype;          /* msel_dtype of x, out, state_in, state_out, dout, dx          */
    int32_t activation;     /* 1: SiLU; 0: none                                            */
    int32_t reserved;       /* must be 0                                                   */
    const void *x;          /* required                                                    */
    const float *weight;    /* required                                                    */
    const float *bias;      /* optional; NULL means 0                                      */
    const void *state_in;   /* optional; NULL means the inputs before step 0 are 0          */
    void *out;              /* fwd: required output; ignored by the backward               */
    void *state_out;        /* fwd: optional output; may equal state_in (the cache is then
                               updated in place); ignored by the backward                  */
} msel_conv_args;

/* Gradients of a scalar loss given dL/dout.  Every output is overwritten, not accumulated. */
typedef struct {
    const void *dout;       /* required, activation dtype                                  */
    void *dx;               /* required, activation dtype                                  */
    float *dweight;         /* optional [dim, width]                                       */
    float *dbias;           /* optional [dim] (computed even when args->bias is NULL)       */
    float *dstate_in;       /* optional [batch, dim, width-1]: gradient w.r.t. state_in     */
} msel_conv_grads;

/* Host-only argument checks of the two entry points below (no HIP call, no device access). */
msel_status msel_validate_conv_fwd(const msel_conv_args *args);
msel_status msel_validate_conv_bwd(const msel_conv_args *args, const msel_conv_grads *grads);

/* Fused causal depthwise convolution + bias + SiLU (page 4, Appendix D, Memory; page 1, the
 * kernels paragraph): one read of x, one write of out, the state in and out of the cache.
 * Deterministic.  seqlen == 1 with state_out == state_in is the recurrent (decode) step;
 * it runs a dedicated kernel (one thread per channel row). */
msel_status msel_conv1d_fwd(const msel_conv_args *args, hipStream_t stream);

/* Its backward, recomputing pre and the activation from x (page 4, Appendix D, Memory):
 * zero-fills dweight and dbias, then one pass that reads x and dout and writes dx and
 * dstate_in.  dweight and dbias are sums over batch and time made with fp32 atomics, so they
 * may differ in the last bits between runs; dx and dstate_in are deterministic. */
msel_status msel_conv1d_bwd(const msel_conv_args *args, const msel_conv_grads *grads,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSEL_H */
