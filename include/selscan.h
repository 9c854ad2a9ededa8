/*
 * selscan.h -- C ABI of the MI355X (gfx950) selective-scan forward library, libselscan.so.
 *
 * The operation (one call computes all of it, on the GPU, asynchronously on `stream`):
 *
 *   for every batch row b and channel d, with h = 0 before the first token
 *   ("state-space models", aarnphm.xyz, section "One recurrence, one convolution": the
 *   unrolled recurrence starts from a zero state):
 *     for l = 0 .. L-1:
 *       for n = 0 .. N-1:
 *         Abar = exp(delta[b,l,d] * A[d,n])                       zero-order hold, diagonal A
 *         Bbar = (Abar - 1) / A[d,n] * B[b,l,n]   (delta*B if A[d,n] == 0)
 *         h[n] = Abar * h[n] + Bbar * u[b,l,d]
 *       y[b,l,d] = sum_n C[b,l,n] * h[n] + Dskip[d] * u[b,l,d]
 *       if z:  y[b,l,d] *= z[b,l,d] * sigmoid(z[b,l,d])
 *     last_state[b,d,:] = h
 *
 *   Sources: the ZOH equations of "state-space models" (section "From continuous time to
 *   tokens"); the per-element discretisation functions and their A == 0 fallback on the
 *   Algenta page "Sequence and state-space models" (section on state_space_models); the
 *   selective mechanism (per-token delta, B, C with a fixed diagonal A; B and C shared by
 *   all channels of a token) of "state-space models" (section "Mamba") and the TorchLean
 *   page "Selective Mamba" (Parameters bProj/cProj); the readout of the updated state,
 *   the D * u feed-through and the SiLU gate of "Selective Mamba" (step); the final state
 *   a following chunk resumes from of "Selective Mamba" (State.hidden, runArray).
 *
 * Options (selscan_dims.discretization, selscan_dims.delta_softplus; delta_bias of
 * selective_scan_fwd_ex / selective_scan_step):
 *   step size:  delta_eff[b,l,d] = delta[b,l,d] + delta_bias[d]  (delta_bias NULL = 0), and
 *               with delta_softplus != 0, delta_eff = softplus(delta_eff) = log(1 + exp(.))
 *               (TorchLean "Selective Mamba", step: softplus of the projection plus a
 *               per-channel dtBias; Algenta "Sequence and state-space models",
 *               mamba_delta_softplus).  delta_eff replaces delta everywhere above.
 *   SELSCAN_DISC_EULER:  Bbar = delta_eff * B[b,l,n] for every state, Abar unchanged (the
 *               first-order input coefficient of Algenta's mamba_selective_scan_step, also
 *               TorchLean's step); it differs from ZOH by O(delta * A) relative.
 *
 * Time-invariant mode (fixed coefficients, "state-space models", section "One recurrence,
 * one convolution"): delta is one value per channel and B, C are one N-vector per channel,
 * expressed through strides (see selscan_dims).  The same recurrence is evaluated.
 *
 * Arithmetic: inputs are read in their I/O type and widened to fp32; the state, the
 * discretisation and the reduction over states run in fp32; y is rounded to the I/O type
 * (round-to-nearest-even for bf16).  A, Dskip and last_state are always fp32.  Values are
 * not validated: a positive A or a huge delta may overflow to Inf/NaN, which propagates.
 *
 * Ownership: every tensor pointer is caller-owned device memory on the HIP device that is
 * current when the call is made.  The library keeps no pointer after the call returns and
 * writes only y, last_state and (chunked path) its workspace.  y and last_state must not
 * overlap any input.  The call only enqueues work on `stream` (a hipStream_t; NULL = the
 * null stream) and returns; it never synchronises.  Inputs must stay valid and unchanged
 * until the enqueued work has run.
 *
 * Errors: every entry point returns an int status (enum selscan_status).  Argument errors
 * are detected on the host before anything is enqueued, so nothing runs when a call
 * fails.  No exception crosses the ABI.  Calls on different streams are independent; the
 * library holds no global mutable state except a thread-local last HIP error code.
 */
#ifndef SELSCAN_H_
#define SELSCAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SELSCAN_ABI_VERSION 2

/* Element type of u, delta, B, C, z and y. */
enum selscan_dtype {
  SELSCAN_F32 = 0,  /* IEEE binary32 */
  SELSCAN_BF16 = 1  /* bfloat16 (upper 16 bits of binary32) */
};

enum selscan_status {
  SELSCAN_OK = 0,
  SELSCAN_ERR_NULL = -1,        /* a required pointer (u, delta, A, B, C, y, dims) is NULL;
                                   only A and dims are required when batch * seqlen == 0 */
  SELSCAN_ERR_DIMS = -2,        /* batch < 0, seqlen < 0, dim < 1, dstate < 1, or a negative stride */
  SELSCAN_ERR_UNSUPPORTED = -3, /* dstate > 64, unknown dtype, path or discretization, a B/C/delta stride
                                   pattern that is neither per-token (shared over channels)
                                   nor per-channel (time-invariant), overlapping y rows
                                   (y_sl < dim or y_sb < seqlen * y_sl), or a size beyond the
                                   32-bit tile addressing of the kernels */
  SELSCAN_ERR_ALIGN = -4,       /* a pointer is not aligned to its element size */
  SELSCAN_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed; the HIP error
                                   code is available from selective_scan_last_hip_error() */
  SELSCAN_ERR_WORKSPACE = -6,   /* workspace pointer NULL or smaller than
                                   selective_scan_workspace_size() */
  SELSCAN_ERR_ABI = -7,         /* dims->abi_version != SELSCAN_ABI_VERSION */
  SELSCAN_ERR_SCRATCH_LIMIT = -8 /* selective_scan_fwd_noalloc: the chunked path needs more than
                                    SELSCAN_NOALLOC_SCRATCH_BYTES of scratch */
};

/* Which kernel schedule to run.  AUTO picks by shape; the others exist for tests and
 * measurements and give results equal to AUTO within the fp32 rounding of a different
 * association order. */
enum selscan_path {
  SELSCAN_PATH_AUTO = 0,
  SELSCAN_PATH_SINGLE = 1,   /* one pass along the sequence per (batch, channel group) */
  SELSCAN_PATH_CHUNKED = 2,  /* two passes over chunks of the sequence, joined by a scan
                                of per-chunk affine maps */
  SELSCAN_PATH_CONV = 3,     /* fixed (time-invariant) coefficients only: the causal
                                convolution y = K * u with the lag kernel
                                K_k = sum_n C_n Abar_n^k Bbar_n ("state-space models"
                                (aarnphm.xyz), "One recurrence, one convolution"), as
                                16-token block Toeplitz products on the fp32 matrix cores with
                                the state carried between blocks.  Needs dim % 4 == 0 and
                                u / z / y rows aligned to 4 elements; no initial state.  Other
                                cases return SELSCAN_ERR_UNSUPPORTED.  Results agree with the
                                recurrence within fp32 rounding of a different association. */
  /* Bit that may be or-ed into any path (tests only): use the general per-element kernel
   * even where the software-pipelined kernel applies.  Results agree within fp32
   * rounding. */
  SELSCAN_PATH_FLAG_SCALAR_IO = 0x100
};

/* Input coefficient of the discretisation (the state coefficient is exp(delta * A) in both). */
enum selscan_discretization {
  SELSCAN_DISC_ZOH = 0,    /* Bbar = (exp(delta A) - 1) / A * B   (delta * B where A == 0) */
  SELSCAN_DISC_EULER = 1   /* Bbar = delta * B */
};

/*
 * Sizes and strides.  All strides are in ELEMENTS (not bytes), must be >= 0, and the
 * innermost axis of every tensor is unit-stride:
 *   u[b,l,d]     at u     + b*u_sb     + l*u_sl     + d
 *   delta[b,l,d] at delta + b*delta_sb + l*delta_sl + d
 *   z[b,l,d]     at z     + b*z_sb     + l*z_sl     + d        (if z != NULL)
 *   y[b,l,d]     at y     + b*y_sb     + l*y_sl     + d
 *   B[b,l,d,n]   at B     + b*B_sb     + l*B_sl     + d*B_sd + n   (same for C)
 *   A[d,n]       at A + d*dstate + n          (contiguous [dim][dstate])
 *   Dskip[d]     at Dskip + d                 (contiguous [dim])
 *   last_state[b,d,n] at last_state + (b*dim + d)*dstate + n   (contiguous [batch][dim][dstate])
 * Two stride patterns are supported:
 *   selective:       B_sd == 0 and C_sd == 0 (B, C per token, shared over channels);
 *                    delta may be per token or, with delta_sb == delta_sl == 0, per channel.
 *   time-invariant:  B_sb == B_sl == C_sb == C_sl == 0 and delta_sb == delta_sl == 0
 *                    (B, C one vector per channel, delta one value per channel).
 */
typedef struct selscan_dims {
  int32_t abi_version;  /* must be SELSCAN_ABI_VERSION */
  int32_t io_dtype;     /* enum selscan_dtype */
  int64_t batch;        /* B >= 0 */
  int64_t seqlen;       /* L >= 0 */
  int64_t dim;          /* D >= 1 (channels) */
  int64_t dstate;       /* N, 1 .. 64 (states per channel) */
  int64_t u_sb, u_sl;
  int64_t delta_sb, delta_sl;
  int64_t z_sb, z_sl;
  int64_t y_sb, y_sl;
  int64_t B_sb, B_sl, B_sd;
  int64_t C_sb, C_sl, C_sd;
  int32_t path;         /* enum selscan_path, optionally | SELSCAN_PATH_FLAG_SCALAR_IO; 0 = automatic */
  int32_t chunk_len;    /* chunked path: tokens per chunk, a multiple of 16 (0 = automatic) */
  int32_t discretization;  /* enum selscan_discretization (0 = ZOH) */
  int32_t delta_softplus;  /* nonzero: the step size is softplus(delta + delta_bias) */
} selscan_dims;

/* Fill *dims for contiguous tensors: u, delta, z, y as [batch][seqlen][dim]; B, C as
 * [batch][seqlen][dstate].  With time_invariant != 0: delta as [dim] and B, C as
 * [dim][dstate].  path = AUTO, chunk_len = 0, ZOH, no softplus.  Never fails for a
 * non-NULL dims. */
void selscan_dims_init(selscan_dims* dims, int io_dtype, int64_t batch, int64_t seqlen,
                       int64_t dim, int64_t dstate, int time_invariant);

/*
 * selective_scan_fwd -- enqueue the selective-scan forward pass described above.
 *   u, delta, B, C : inputs in dims->io_dtype, required (non-NULL)
 *   A              : [dim][dstate] fp32, required
 *   Dskip          : [dim] fp32, or NULL for no feed-through term
 *   z              : gate input in dims->io_dtype, or NULL for no gate
 *   y              : output in dims->io_dtype, required
 *   last_state     : [batch][dim][dstate] fp32 output, or NULL to skip it
 *   dims           : sizes, strides and path selection, required
 *   stream         : hipStream_t to enqueue on (NULL = null stream)
 * When batch * seqlen == 0 the per-token tensors (u, delta, B, C, z, y) are not read and
 * may be NULL; A is always required.
 * batch == 0 enqueues nothing.  seqlen == 0 writes nothing to y and, if last_state is
 * given, fills it with zeros (an empty sequence leaves the zero initial state; TorchLean
 * "Selective Mamba", runArray).  The chunked path needs device scratch; this entry point
 * takes it with hipMallocAsync/hipFreeAsync on `stream` (stream-ordered).
 * Returns SELSCAN_OK or an error status; on error nothing was enqueued, except that
 * SELSCAN_ERR_HIP may follow a partially enqueued sequence of launches.
 */
int selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                       const void* C, const float* Dskip, const void* z, void* y,
                       float* last_state, const selscan_dims* dims, void* stream);

/* The path a forward call with these dims takes: SELSCAN_PATH_SINGLE, SELSCAN_PATH_CHUNKED or
 * SELSCAN_PATH_CONV (the automatic choice resolved, assuming the operand pointers are aligned
 * to 4 elements), or a negative status for invalid dims.  Host-only, touches no device. */
int selective_scan_plan_path(const selscan_dims* dims);

/* Bytes of device workspace the chunked path needs for these dims (0 when the automatic
 * or forced path is the single pass).  Returns 0 for invalid dims. */
size_t selective_scan_workspace_size(const selscan_dims* dims);

/* selective_scan_fwd with caller-provided workspace (device memory, 256-byte aligned,
 * at least selective_scan_workspace_size(dims) bytes; may be NULL when that size is 0).
 * Never allocates.  The workspace must not be used by other work until the enqueued
 * scan has finished on `stream`. */
int selective_scan_fwd_ws(const void* u, const void* delta, const float* A, const void* B,
                          const void* C, const float* Dskip, const void* z, void* y,
                          float* last_state, const selscan_dims* dims, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * selective_scan_fwd_ex -- the forward pass continuing from a given state.
 *   initial_state  : [batch][dim][dstate] fp32, the state h_{-1} the sequence starts from,
 *                    or NULL for the zero state (then this is selective_scan_fwd /
 *                    selective_scan_fwd_ws).  It may be the same buffer as last_state
 *                    (continue in place): it is read before last_state is written; any
 *                    other overlap with an output is undefined.  Selective coefficients
 *                    only: with time-invariant ones a non-NULL initial_state returns
 *                    SELSCAN_ERR_UNSUPPORTED.
 *   workspace, workspace_bytes : as selective_scan_fwd_ws; a NULL workspace makes the call
 *                    take it stream-ordered on `stream` when the chunked path needs it.
 *   delta_bias     : [dim] fp32 added to delta before the optional softplus, or NULL.
 *   Other arguments as selective_scan_fwd.
 * seqlen == 0 copies initial_state (zeros if NULL) to last_state.
 * A call over tokens [0, k) followed by a call over [k, L) whose initial_state is the
 * first call's last_state gives the result of one call over [0, L), up to the fp32
 * rounding of the carried state (TorchLean "Selective Mamba": step and runArray carry an
 * explicit hidden state from one chunk to the next).
 */
int selective_scan_fwd_ex(const void* u, const void* delta, const float* delta_bias, const float* A,
                          const void* B, const void* C, const float* Dskip, const void* z, void* y,
                          const float* initial_state, float* last_state, const selscan_dims* dims,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * selective_scan_fwd_noalloc -- selective_scan_fwd_ex for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * It allocates nothing: no hipMalloc / hipFree / stream-ordered allocation and no
 * allocating library call.  When the chunked path runs, its scratch (each chunk's end
 * state and step sum, then the carried-in states) is a device array inside the library,
 * SELSCAN_NOALLOC_SCRATCH_BYTES per GPU, created when the library's code is loaded on that
 * GPU and held until the process ends; its device address is looked up on the first call
 * on each GPU (the GPU of `stream`).
 *   Arguments as selective_scan_fwd_ex without the workspace pair; dims as for the
 *   forward (selective_scan_workspace_size(dims) is the scratch a call uses).
 *   Returns SELSCAN_ERR_SCRATCH_LIMIT, before anything is enqueued, when
 *   selective_scan_workspace_size(dims) > SELSCAN_NOALLOC_SCRATCH_BYTES (use
 *   selective_scan_fwd_ws or selective_scan_fwd_ex with a workspace instead); other errors
 *   as selective_scan_fwd_ex.
 * Every call on one GPU shares that GPU's array.  Nothing in it needs to start at zero
 * (each call writes every slot it reads), but two calls whose execution overlaps on one
 * GPU (different streams, or another thread's call) race on it: callers serialise them.
 */
#define SELSCAN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int selective_scan_fwd_noalloc(const void* u, const void* delta, const float* delta_bias,
                               const float* A, const void* B, const void* C, const float* Dskip,
                               const void* z, void* y, const float* initial_state,
                               float* last_state, const selscan_dims* dims, void* stream);

/*
 * selective_scan_step -- one recurrent decode step: the forward pass over a single token
 * per batch row, updating the running state in place (aarnphm "state-space models", section
 * "One recurrence, one convolution": the recurrent form yields one output per step from
 * the state; chipfoundry glossary, "Computational Considerations": a fixed-size state per
 * generated token).
 *   dims   : dims->seqlen must be 1 (else SELSCAN_ERR_DIMS); strides as for the forward
 *            pass (token strides are not used); both coefficient patterns are supported;
 *            dims->path and dims->chunk_len are ignored.
 *   state  : [batch][dim][dstate] fp32, required: read as h_{-1}, overwritten with h_0.
 *   u, delta, A, B, C, Dskip, z, y : as selective_scan_fwd, for the one token.
 *   delta_bias : as selective_scan_fwd_ex.
 * Never allocates.  Same status codes as selective_scan_fwd.
 */
int selective_scan_step(const void* u, const void* delta, const float* delta_bias, const float* A,
                        const void* B, const void* C, const float* Dskip, const void* z, void* y,
                        float* state, const selscan_dims* dims, void* stream);

/*
 * selective_scan_bwd -- the backward pass: gradients of the forward pass of
 * selective_scan_fwd_ex with the same inputs and options, given the gradient dy of y and,
 * optionally, the gradient dlast_state reaching its last_state (the vector-Jacobian product).
 * It follows the reverse-time recurrence over the states of the rustytorch commit log's
 * hand-written VJP of the selective scan ("Hand-written VJP of the selective-scan forward"):
 * with lambda_t = dL/dh_t, lambda_t = dy'_t C_t + Abar_{t+1} lambda_{t+1}, where dy'_t is dy_t
 * through the gate, and each input's gradient is the chain rule through one step.  States are
 * recomputed from checkpoints taken every 16 tokens, so nothing from the forward call is
 * needed.
 *   u, delta, delta_bias, A, B, C, Dskip, z, initial_state : the forward call's inputs
 *                    (dims->discretization and dims->delta_softplus as in that call), with
 *                    selective (per-token) or fixed (per-channel delta, B and C) coefficients.
 *   dy             : gradient of y, in dims->io_dtype with the y strides of dims, required.
 *   dlast_state    : [batch][dim][dstate] fp32 gradient of last_state, or NULL (zero).
 * Outputs (device memory, all written, never accumulated into):
 *   du, ddelta, dz : [batch][seqlen][dim] contiguous, in dims->io_dtype.  ddelta is the
 *                    gradient of the delta argument as given (of the softplus argument's
 *                    raw part when delta_softplus).  dz is written only if z and dz are both
 *                    non-NULL.  du and ddelta are required.
 *   dB, dC         : [batch][seqlen][dstate] contiguous, in dims->io_dtype, required.
 *   Fixed coefficients: ddelta is [dim] and dB, dC are [dim][dstate], contiguous in
 *                    dims->io_dtype: the sums over batch rows and tokens of the per-token
 *                    terms (the same reverse-time recurrence with Abar and the input
 *                    coefficient constant per channel and state).
 *   dA             : [dim][dstate] fp32, required.
 *   dDskip, ddelta_bias : [dim] fp32, or NULL to skip.  ddelta_bias is the sum of ddelta
 *                    over batch and tokens.
 *   dinitial_state : [batch][dim][dstate] fp32 gradient of initial_state, or NULL.
 *   workspace      : device memory of selective_scan_bwd_workspace_size(dims) bytes,
 *                    256-byte aligned, or NULL to take it stream-ordered on `stream`.
 * No output may overlap an input.  Same status codes as selective_scan_fwd.
 */
int selective_scan_bwd(const void* u, const void* delta, const float* delta_bias, const float* A,
                       const void* B, const void* C, const float* Dskip, const void* z,
                       const float* initial_state, const void* dy, const float* dlast_state,
                       void* du, void* ddelta, float* ddelta_bias, float* dA, void* dB, void* dC,
                       float* dDskip, void* dz, float* dinitial_state, const selscan_dims* dims,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace selective_scan_bwd needs for these dims (0 for an empty call
 * or invalid dims): the checkpoints, batch * ceil(seqlen/16) * dim * dstate floats; the
 * per-channel-group partial sums of dB and dC (groups of 64, 32 or 16 channels for dstate up
 * to 16, 32, 64), at most 2 * ceil(dim/16) * batch * seqlen * dstate floats (fixed
 * coefficients: 2 * batch * chunks * dim * dstate); when the sequence is split into chunks,
 * the running sums of delta at the checkpoints, batch * ceil(seqlen/16) * dim floats
 * (selective coefficients), and per-chunk states and adjoints, O(batch * dim * dstate *
 * chunks). */
size_t selective_scan_bwd_workspace_size(const selscan_dims* dims);

/*
 * The scalar-decay ("SSD", Mamba-2) layer: within each head the transition is a scalar,
 * Abar_t = a_t I with a_t = exp(delta_t A_h), and
 *     y_t = sum_{s<=t} (C_t . Bbar_s) (prod_{k=s+1..t} a_k) x_s  (+ Dskip x_t, then * SiLU(z_t)),
 * i.e. Y = (L o C Bbar^T) X per head with the causal decay mask L ("state-space models",
 * aarnphm.xyz, section "Mamba-2 and state-space duality").  Bbar_s = c_s B_s with
 * c_s = (a_s - 1)/A_h (ZOH; delta_s where A_h == 0) or delta_s (SELSCAN_DISC_EULER).  It is
 * the selective scan above with A[d][n] = A_h for every state and channel of head h and one
 * step size per (token, head); it is computed as the page describes Mamba-2's algorithm:
 * matrix products inside 64-token chunks (on the matrix cores), a state carried between them.
 */
typedef struct selscan_ssd_dims {
  int32_t abi_version;     /* SELSCAN_ABI_VERSION */
  int32_t discretization;  /* enum selscan_discretization */
  int64_t batch;           /* >= 0 */
  int64_t seqlen;          /* >= 0 */
  int64_t nheads;          /* H >= 1 */
  int64_t headdim;         /* P: 64 */
  int64_t dstate;          /* N: 64 or 128 */
  int32_t path;            /* 0 automatic; 1 one workgroup per (batch, head) walking the chunks
                              with the state on chip (no workspace); 2 chunk-parallel (chunk
                              states in the workspace, a scan over them, then the outputs);
                              3 on chip over sequence segments: each segment's end state from
                              zero (a state-only walk), composed across segments, then one
                              workgroup per (batch, segment, head) walks its segment from the
                              state carried in (segment states in the workspace) */
  int32_t segments;        /* path 3: number of sequence segments (equal runs of 64-token chunks,
                              at most one per chunk), 0 to choose automatically; 0 otherwise */
} selscan_ssd_dims;

/*
 * selective_scan_ssd_fwd -- enqueue the scalar-decay layer.  Every tensor is contiguous,
 * device memory on the current device; x, delta, B, C, z and y are bfloat16, the rest fp32:
 *   x, z, y        : [batch][seqlen][nheads][headdim]   (z may be NULL: no gate)
 *   delta          : [batch][seqlen][nheads]   step size per (token, head)
 *   A              : [nheads]   (the head's continuous rate, normally negative)
 *   B, C           : [batch][seqlen][dstate]   shared by every head
 *   Dskip          : [nheads * headdim], or NULL
 *   initial_state, last_state : [batch][nheads][headdim][dstate], or NULL (zero / not written)
 *   workspace      : selective_scan_ssd_workspace_size(dims) bytes, 256-byte aligned, or NULL
 *                    to take it stream-ordered on `stream`.
 * x, B, C, z and y must be 16-byte aligned (else SELSCAN_ERR_ALIGN); delta 2-byte aligned.
 * headdim other than 64 or dstate other than 64 / 128 return SELSCAN_ERR_UNSUPPORTED.
 * Other status codes as selective_scan_fwd.
 */
int selective_scan_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, void* y, const float* initial_state,
                           float* last_state, const selscan_ssd_dims* dims, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Workspace bytes of selective_scan_ssd_fwd (0 for an empty call, invalid dims or the
 * on-chip path over the whole sequence): for the chunk-parallel path, per (batch row, head,
 * 64-token chunk) one fp32 [dstate][headdim] chunk state, one decay, and one bf16 carried-in
 * state; for the on-chip path over segments, per (batch row, head, segment) one fp32 state
 * and one decay.  The automatic path takes the chunk-parallel one when batch * nheads *
 * ceil(seqlen / 64) <= 512, else the on-chip one over the segment count a cost model of
 * MI355X times picks (one segment, the whole sequence, where splitting does not pay). */
size_t selective_scan_ssd_workspace_size(const selscan_ssd_dims* dims);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* selective_scan_strerror(int status);

/* The hipError_t of the most recent SELSCAN_ERR_HIP returned on this thread (0 if none). */
int selective_scan_last_hip_error(void);

/* SELSCAN_ABI_VERSION of the loaded library. */
int selective_scan_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H_ */
