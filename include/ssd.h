/*
 * ssd.h -- C ABI of the Mamba-2 SSD (structured state-space duality) forward
 * pass for AMD Instinct MI355X (gfx950).
 *
 * The operator (one selective SSM layer core, per batch b and head h with
 * B/C group g = h / (nheads / ngroups)):
 *
 *     h_t      = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t B_t^T      (P x N state)
 *     y_t      = h_t C_t + D_h * x_t
 *     h_{-1}   = init_state (zeros when NULL);   final_state = h_{L-1}
 *
 * The transition is one scalar per head times the identity (Telegram post
 * "Mamba3", opening paragraph; "Mamba-3 : SSM optimise inference", section
 * "Du training-first a l'inference-first"), discretised with zero-order hold
 * for A and an Euler step for B ("Mamba3", discretisation section). It is
 * evaluated with the blocked two-pass algorithm: the sequence is cut into
 * chunks of Q tokens processed in parallel, and the per-chunk states are then
 * recombined ("Mamba-2 vs Transformers: SSMs, structured state space
 * duality", section "Mamba-2 and the SSD paper: what changed in practice").
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays; the caller
 *    owns them and keeps them alive until the enqueued work has completed.
 *    The library keeps no pointer after a call returns and holds no mutable
 *    global state, so calls from several host threads are safe.
 *  - Calls are asynchronous: kernels are enqueued on `stream` (a hipStream_t;
 *    NULL is the default stream) and nothing is synchronised.
 *  - All arguments are validated before anything is enqueued; on any error
 *    nothing is written. SSD_ERR_HIP reports a failed kernel launch; faults
 *    inside kernels surface at the caller's next synchronisation.
 *  - No C++ exception crosses this boundary.
 *
 * Layouts (row-major, innermost last), with L = seqlen, H = nheads,
 * P = headdim, N = dstate, G = ngroups, Q = chunk size, nc = ceil(L / Q):
 *     x, y            [batch, L, H, P]     io dtype
 *     dt              [batch, L, H]        fp32, used as given (no softplus)
 *     A, D            [H]                  fp32 (A <= 0 expected; D nullable)
 *     B, C            [batch, L, G, N]     io dtype
 *     init_state,
 *     final_state     [batch, H, P, N]     fp32
 *   Chunked intermediates (the workspace; see ssd_workspace_bytes):
 *     dA_cumsum       [batch, H, nc, Q]    fp32, inclusive sum of dt*A within
 *                                          the chunk (positions >= L: dt = 0)
 *     dt_chunked      [batch, H, nc, Q]    fp32, dt regrouped per chunk, 0 past L
 *     states          [batch, H, nc, P, N] state dtype (= io dtype): the local
 *                                          state of each chunk, overwritten in
 *                                          place by the state entering it.
 *
 * dt: every entry point applies the descriptor's dt preprocessing (bias,
 * softplus, clamp) when asked to; with the zero default dt is used as given.
 *
 * Supported: io dtype fp32 or bf16; P in {16, 32, 64, 128};
 * N in {16, 32, 64, 128, 256}; H % G == 0; chunk_size in {0 (default), 64,
 * 128, 256}, except, for bf16, chunk_size 256 with P = 128 and N >= 64,
 * chunk_size 64 with P = 128 and N = 256, and chunk_size 256 with P = 16 and
 * N = 256 (SSD_ERR_UNSUPPORTED: the intra-chunk kernel's register tiles do
 * not fit there; the default, 128 for those headdim/dstate pairs, always
 * does). Base pointers of x, B, C, y, init_state, final_state must be
 * 16-byte aligned, dt/A/D 4-byte aligned, the workspace 256-byte aligned.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SSD_API __attribute__((visibility("default")))
#else
#define SSD_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSD_DTYPE_F32 = 0,
  SSD_DTYPE_BF16 = 1
} ssd_dtype_t;

typedef enum {
  SSD_OK = 0,
  SSD_ERR_NULL_POINTER = 1, /* a required pointer is NULL                     */
  SSD_ERR_BAD_SHAPE = 2,    /* a dimension <= 0, H % G != 0, or too large     */
  SSD_ERR_UNSUPPORTED = 3,  /* P, N, dtype or chunk size outside the set above */
  SSD_ERR_ALIGNMENT = 4,    /* a base pointer is misaligned                    */
  SSD_ERR_WORKSPACE = 5,    /* workspace given but smaller than required       */
  SSD_ERR_ALIAS = 6,        /* an output overlaps an input it must not overlap */
  SSD_ERR_HIP = 7,          /* the HIP runtime reported an error               */
  SSD_ERR_SCRATCH_LIMIT = 8 /* ssd_forward_noalloc: the problem needs more
                               workspace than its fixed scratch array holds     */
} ssd_status_t;

/* Path a whole-forward call took, as recorded in its workspace
 * (ssd_workspace_status). */
typedef enum {
  SSD_PATH_NONE = 0,            /* no forward call recorded in the workspace   */
  SSD_PATH_SPLIT = 1,           /* separate steps, chain over chunks per lane  */
  SSD_PATH_SPLIT_SEGMENTED = 2, /* separate steps, chains cut into segments    */
  SSD_PATH_ONE_PASS = 3         /* the one-pass kernel of ssd_forward_fused    */
} ssd_path_t;

/* Status bits reported by ssd_workspace_status (0 = the call completed as
 * designed). Any bit set means y and final_state of that call are not valid,
 * and, when final_state was the same buffer as init_state, neither is that
 * buffer. */
enum {
  SSD_STATUS_WAIT_CUT_OFF_ONE_PASS = 1u,  /* a one-pass state hand-over wait gave up     */
  SSD_STATUS_WAIT_CUT_OFF_SEGMENTED = 2u, /* a segmented state-passing wait gave up      */
  SSD_STATUS_CHAIN_INCOMPLETE = 4u,       /* a hand-over counter or ticket count is not
                                             at its final value                          */
  SSD_STATUS_NO_RECORD = 8u               /* the workspace holds no forward record for
                                             this descriptor                             */
};

/* Problem description. Plain data; the library reads it during the call only.
 * A zero-initialised tail (dt_bias .. dt_max) means dt is used as given. */
typedef struct {
  int64_t batch;
  int64_t seqlen;     /* L  */
  int64_t nheads;     /* H  */
  int64_t headdim;    /* P  */
  int64_t dstate;     /* N  */
  int64_t ngroups;    /* G  */
  int32_t io_dtype;   /* ssd_dtype_t: dtype of x, B, C, y (and of states)     */
  int32_t chunk_size; /* Q: 0 picks the library default for the shape         */
  /* dt preprocessing of the Mamba-2 layer, applied to every dt the entry
   * points read, in this order (positions past the end of a sequence keep
   * dt = 0):  z = dt + dt_bias[h]      when dt_bias != NULL
   *           z = log(1 + exp(z))      when dt_softplus != 0
   *           z = min(max(z, dt_min), dt_max)   when dt_clamp != 0  */
  const float* dt_bias; /* [H] fp32 device pointer, nullable, 4-byte aligned   */
  int32_t dt_softplus;
  int32_t dt_clamp;     /* requires dt_min <= dt_max                           */
  float dt_min;
  float dt_max;
} ssd_desc_t;

/* Human-readable name of a status code (static string, never NULL). */
SSD_API const char* ssd_status_string(int status);

/* Chunk length Q the library will use for `desc` (resolves chunk_size == 0). */
SSD_API ssd_status_t ssd_effective_chunk_size(const ssd_desc_t* desc, int32_t* chunk_size);

/* Bytes of device workspace ssd_forward needs for `desc`: dA_cumsum,
 * dt_chunked and states, each starting on a 256-byte boundary, in that order.
 * Where the one-pass kernel supports the shape (see ssd_forward_fused), the
 * states region is at least the size of its state hand-over area. For a few
 * long sequences (64 to 1024 chunks, few (batch, head) chains) a scratch
 * area for the segmented state passing follows the states. Pure host
 * computation; no HIP call. */
SSD_API ssd_status_t ssd_workspace_bytes(const ssd_desc_t* desc, size_t* bytes);

/* The whole forward pass: y and (when final_state != NULL) the final state.
 *   x, dt, A, B, C, y        required.
 *   D           nullable: NULL means D = 0 (no skip term).
 *   init_state  nullable: NULL means a zero initial state.
 *   final_state nullable: NULL means it is not written. It may be the same
 *               pointer as init_state (in-place state update); partial
 *               overlap is rejected.
 *   workspace   nullable: NULL makes the library allocate and free it in
 *               stream order (hipMallocAsync / hipFreeAsync); otherwise at
 *               least ssd_workspace_bytes() bytes, 256-byte aligned, not
 *               overlapping any other argument.
 *   y must not overlap any input.
 * Runs the five steps below on `stream`, in order (the path of
 * ssd_forward_split), or, where the one-pass kernel of ssd_forward_fused
 * supports the shape and is the faster choice for it, that path. The
 * environment variable SSD_FORWARD_PATH=split or =fused, read once per
 * process, overrides the choice (fused only where it is supported).
 * SSD_OK means every argument was valid and every kernel was enqueued. Both
 * paths may contain bounded waits between workgroups (see
 * ssd_workspace_status); a wait cut off after the call returned does not
 * change the return value, and ssd_workspace_status reports it. */
SSD_API ssd_status_t ssd_forward(const ssd_desc_t* desc,
                         const void* x, const float* dt, const float* A,
                         const void* B, const void* C, const float* D,
                         const float* init_state,
                         void* y, float* final_state,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* The same forward pass in one pass over x ("Mamba-2 vs Transformers",
 * section "Mamba-2 and the SSD paper: what changed in practice": the chunk
 * states are combined by a scan over the chunks, here a chain of hand-overs
 * between the workgroups of consecutive chunks inside one kernel). Two
 * launches: the dt cumsum, then one kernel that computes every chunk's state,
 * takes the state entering the chunk from the chunk before, passes its own
 * on, and writes y. x is read once and no chunk state goes through the
 * workspace's states array.
 * Arguments, ownership and errors as for ssd_forward, with the same
 * workspace size (ssd_workspace_bytes); the workspace must not be in use by
 * another call that may run at the same time. Supported: bf16 io, chunk
 * length 256, headdim 32 or 64, dstate 32, 64 or 128 (not headdim 32 with
 * dstate 32); anything else returns SSD_ERR_UNSUPPORTED.
 * Results agree with ssd_forward to rounding: the chunk states stay in fp32
 * (ssd_forward rounds them to bf16 between its kernels), and the chunk-state
 * weights are applied to B instead of x before the bf16 rounding.
 * Every wait of one chunk's workgroup for the state of the chunk before is
 * bounded; a wait that is cut off sets a status bit in the workspace instead
 * of hanging, and the call still returns SSD_OK: ssd_workspace_status reads
 * the bit. With the environment variable SSD_DEBUG set, every whole-forward
 * call waits for its kernels and returns SSD_ERR_HIP if a bit is set. */
SSD_API ssd_status_t ssd_forward_fused(const ssd_desc_t* desc,
                               const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* D,
                               const float* init_state,
                               void* y, float* final_state,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* The same forward pass, always on the split path: the five steps below as
 * separate launches on `stream` (fused where a step's kernels allow it: the
 * cumsum with the chunk states), the chunk states going through the
 * workspace between them. This is what ssd_forward runs wherever it does
 * not take the one-pass kernel, so on those shapes the two give identical
 * bits. Arguments, ownership, workspace size and errors as for
 * ssd_forward. */
SSD_API ssd_status_t ssd_forward_split(const ssd_desc_t* desc,
                               const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* D,
                               const float* init_state,
                               void* y, float* final_state,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* Status of the last whole-forward call (ssd_forward, ssd_forward_split or
 * ssd_forward_fused) that ran with `workspace` and this descriptor.
 *
 * Two paths synchronise workgroups of one kernel with bounded waits: the
 * one-pass kernel (each chunk waits for the state of the chunk before) and
 * the segmented state passing of ssd_forward for a few long sequences (each
 * segment waits for the aggregates of the segments before). Every such wait
 * gives up after a fixed number of polls, so a kernel always ends; the wait
 * then sets a bit in a status record the call keeps in its workspace, and the
 * forward call itself has already returned SSD_OK. That record, and for these
 * two paths the hand-over counters and ticket count, are what this call
 * checks. (A cut-off is a defect of the launch, not of the inputs: under the
 * ticket order every wait targets a workgroup that has started and is not
 * blocked, so it is not expected in any run.)
 *
 * Enqueues device-to-host copies of a few words on `stream` and synchronises
 * that stream (so it cannot be captured into a graph). Allocates nothing.
 *   desc       the descriptor the forward call was made with.
 *   workspace  that call's workspace (a caller-provided one: with a NULL
 *              workspace the library's own is freed when the call ends),
 *              at least ssd_workspace_bytes() bytes, 256-byte aligned.
 *   path       nullable; receives the ssd_path_t the call took.
 *   status     receives the SSD_STATUS_* bits, 0 when the call completed as
 *              designed.
 * Returns SSD_ERR_NULL_POINTER, SSD_ERR_ALIGNMENT, SSD_ERR_WORKSPACE for a
 * bad argument, SSD_ERR_HIP when a copy fails. Packed sequences
 * (ssd_forward_varlen) keep their record elsewhere in their workspace: read
 * it with ssd_workspace_status_varlen. */
SSD_API ssd_status_t ssd_workspace_status(const ssd_desc_t* desc, const void* workspace, size_t workspace_bytes,
                                          void* stream, uint32_t* path, uint32_t* status);

/* The whole forward pass of ssd_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): no workspace argument, and nothing is allocated;
 * the workspace comes from a fixed scratch array of 256 MiB that the library
 * holds on every GPU it runs this entry point on, until the process ends.
 * Arguments other than the workspace, the path taken, the results and the
 * errors are those of ssd_forward (same bits); problems whose
 * ssd_workspace_bytes() exceeds 256 MiB return SSD_ERR_SCRATCH_LIMIT before
 * anything is enqueued (the headline layer shape fits up to batch 28 at
 * L = 2048). All calls on one GPU share that GPU's array: calls that may
 * overlap in time on one GPU (several streams or host threads) race and must
 * be ordered by the caller. The first call on each device looks the array's
 * device address up (a HIP runtime query, no allocation). */
SSD_API ssd_status_t ssd_forward_noalloc(const ssd_desc_t* desc,
                                 const void* x, const float* dt, const float* A,
                                 const void* B, const void* C, const float* D,
                                 const float* init_state,
                                 void* y, float* final_state,
                                 void* stream);

/* ---- the steps of the chunked path, each callable on its own ------------ */

/* Step 1, chunk cumulative sum of dt*A ("Mamba-2 vs Transformers", section
 * "Mamba-2 and the SSD paper: what changed in practice": chunks processed in
 * parallel). Writes dA_cumsum and dt_chunked ([batch, H, nc, Q] fp32 each). */
SSD_API ssd_status_t ssd_chunk_cumsum(const ssd_desc_t* desc, const float* dt, const float* A,
                              float* dA_cumsum, float* dt_chunked, void* stream);

/* Step 2, local state of every chunk (same section: the per-chunk SSM
 * states), on matrix cores for bf16:
 *   states[b,h,c] = sum_{j in c} exp(Lam_c - l_j) dt_j x_j B_j^T,
 * with l = dA_cumsum and Lam_c its last entry in chunk c.
 * Writes states [batch, H, nc, P, N] in the io dtype. */
SSD_API ssd_status_t ssd_chunk_state(const ssd_desc_t* desc, const void* x, const void* B,
                             const float* dA_cumsum, const float* dt_chunked,
                             void* states, void* stream);

/* Steps 1 and 2 in one launch: the chunk cumsum of dt*A and the local
 * chunk states. Writes the same dA_cumsum, dt_chunked and states, bit for
 * bit, as ssd_chunk_cumsum followed by ssd_chunk_state; ssd_forward uses it.
 * Same arguments, layouts and alignment as those two calls. */
SSD_API ssd_status_t ssd_cumsum_chunk_state(const ssd_desc_t* desc, const void* x, const void* B,
                                    const float* dt, const float* A,
                                    float* dA_cumsum, float* dt_chunked,
                                    void* states, void* stream);

/* Step 3, inter-chunk state passing (same section: the per-chunk states are
 * recombined). In place over `states`: on return states[b,h,c] holds the
 * state entering chunk c,  H_{-1} = init_state (or 0),
 * Hin_c = H_{c-1},  H_c = exp(Lam_c) H_{c-1} + S_c. Writes final_state
 * (= H_{nc-1}) in fp32 when non-NULL; final_state may equal init_state.
 * This entry point runs the chain chunk by chunk. For a few long sequences,
 * ssd_forward instead cuts each chain into segments of 32 chunks that run in
 * parallel (it has a workspace for their partial states). Its results then
 * differ from this step's only in the fp32 rounding order. */
SSD_API ssd_status_t ssd_state_passing(const ssd_desc_t* desc, void* states, const float* dA_cumsum,
                               const float* init_state, float* final_state, void* stream);

/* Steps 4 and 5 fused, intra-chunk output on matrix cores plus the chunk
 * output from the entering state (the masked dual form inside a chunk,
 * "Mamba-2 vs Transformers", contraction-order table):
 *   y_i = sum_{j<=i in chunk} exp(l_i - l_j) dt_j (C_i . B_j) x_j
 *       + exp(l_i) Hin_c C_i + D_h x_i.
 * `states` must hold the entering states (the output of step 3). */
SSD_API ssd_status_t ssd_chunk_scan(const ssd_desc_t* desc, const void* x, const void* B, const void* C,
                            const float* D, const float* dA_cumsum, const float* dt_chunked,
                            const void* states, void* y, void* stream);

/* ---- packed variable-length sequences -------------------------------------- */

/* Workspace bytes for ssd_forward_varlen (desc->batch = 1, desc->seqlen = T
 * total tokens, num_seqs sequences). Pure host computation. */
SSD_API ssd_status_t ssd_workspace_bytes_varlen(const ssd_desc_t* desc, int64_t num_seqs, size_t* bytes);

/* The forward pass over num_seqs sequences packed back to back: sequence s
 * holds tokens [cu_seqlens[s], cu_seqlens[s+1]) of the [1, T, ...] arrays and
 * runs the recurrence of ssd_forward on its own, from init_states[s] (zeros
 * when init_states is NULL) to final_states[s] (not written when NULL). No
 * state crosses a sequence boundary; no padding is needed.
 *
 * Two ways of cutting the work:
 *  - bf16 io and init_states NULL: fixed chunks of Q tokens over the packed
 *    stream, as for one sequence of T tokens, so a chunk may hold the ends
 *    and starts of several sequences. A start adds -128 to the chunk's dA
 *    cumsum from its token on, so every decay factor across it is
 *    exp(<= -128) = 0 in fp32 (dt*A <= 0): no state or input crosses the
 *    boundary. Each sequence's final state is then its last chunk's local
 *    state up to its last token, plus the decayed fp32 state entering that
 *    chunk. The work is that of ssd_forward on [1, T] (state passing cut
 *    into segments when the chunks are many), plus one partial chunk state
 *    per sequence for the final states. After k starts within one chunk the
 *    cumsum is near -128 k, so the decays of the sequence that follows carry
 *    a relative rounding of up to 2^-17 k (below bf16's 2^-9 for k < 256).
 *  - fp32 io, or init_states given: chunks per sequence (a sequence's first
 *    chunk starts at its first token), each sequence's chain of states
 *    starting from its own initial state; up to ceil(T/Q) + num_seqs
 *    chunks.
 *   cu_seqlens   [num_seqs + 1] int32, DEVICE pointer: 0 = cu[0] <= cu[1]
 *                <= ... <= cu[num_seqs] = T. Offsets are clamped into [0, T]
 *                on the device, so an invalid array gives wrong values but no
 *                access outside the arguments.
 *   x, y [1, T, H, P]; dt [1, T, H]; B, C [1, T, G, N]; A, D [H];
 *   init_states, final_states [num_seqs, H, P, N] fp32 (may be the same
 *   pointer; other overlaps are rejected).
 *   workspace    nullable, at least ssd_workspace_bytes_varlen() bytes.
 * Errors as ssd_forward; SSD_ERR_BAD_SHAPE also when desc->batch != 1,
 * num_seqs < 1 or T >= 2^31. A segmented state passing uses the bounded
 * waits described at ssd_workspace_status and leaves the same record, read
 * with ssd_workspace_status_varlen. */
SSD_API ssd_status_t ssd_forward_varlen(const ssd_desc_t* desc, const int32_t* cu_seqlens, int64_t num_seqs,
                                const void* x, const float* dt, const float* A,
                                const void* B, const void* C, const float* D,
                                const float* init_states, void* y, float* final_states,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Status of the last ssd_forward_varlen call that ran with `workspace`,
 * this descriptor and num_seqs: as ssd_workspace_status (same path values
 * and bits; SSD_PATH_SPLIT for a plain state passing, either cut of the
 * work). Workspace at least ssd_workspace_bytes_varlen() bytes. */
SSD_API ssd_status_t ssd_workspace_status_varlen(const ssd_desc_t* desc, int64_t num_seqs, const void* workspace,
                                                 size_t workspace_bytes, void* stream, uint32_t* path,
                                                 uint32_t* status);

/* ---- the short causal convolution before the SSM --------------------------- */

/* Depthwise causal convolution over time of the packed token vector
 * [x (h, p) | B (g, n) | C (g, n)], width K = conv_width in 1..4, then split
 * into the x, B and C tensors ssd_forward reads (Telegram post "Mamba3" and
 * "Mamba-3 : SSM optimise inference", section "Architecture revisitee": the
 * short causal convolution of Mamba-1/2). Per channel ch of CH = H*P + 2*G*N:
 *   z[t] = bias[ch] + sum_{k<K} weight[ch][k] * in[t - (K-1) + k],
 *   out[t] = silu ? z * sigmoid(z) : z,
 * with in[t < 0] = conv_state_in[b][ch][K-1+t] (zeros when it is NULL).
 *   xbc             [batch, L, CH]        io dtype, 16-byte aligned
 *   weight          [CH, K]               fp32
 *   bias            [CH]                  fp32, nullable, 16-byte aligned
 *   conv_state_in   [batch, CH, K-1]      fp32, nullable
 *   conv_state_out  [batch, CH, K-1]      fp32, nullable: the last K-1 inputs
 *                                         (continues the sequence in a later
 *                                         call); must not overlap conv_state_in
 *   x [batch, L, H, P], B, C [batch, L, G, N]   io dtype outputs
 * Outputs must not overlap inputs or each other. */
SSD_API ssd_status_t ssd_conv1d_split(const ssd_desc_t* desc, int32_t conv_width, const void* xbc,
                              const float* weight, const float* bias, int32_t silu,
                              const float* conv_state_in, float* conv_state_out,
                              void* x, void* B, void* C, void* stream);

/* ---- the recurrent (decode) step ------------------------------------------ */

/* One token of a batch of sequences through the recurrence, the state kept
 * between calls ("Mamba-2 vs Transformers", table "Evaluation criteria ...":
 * recurrent mode, O(1) state per token). desc->seqlen must be 1 (chunk_size
 * is ignored); shapes are those of ssd_forward with L = 1:
 *     x, y     [batch, H, P]      io dtype
 *     dt       [batch, H]         fp32 (the descriptor's dt preprocessing applies)
 *     A, D     [H]                fp32 (D nullable: no skip term)
 *     B, C     [batch, G, N]      io dtype
 *     state    [batch, H, P, N]   fp32, read and overwritten in place:
 *     state <- exp(dt A) state + dt x B^T;  y = state C + D x  (the new state).
 * The same result as ssd_forward on the one token with init_state = state and
 * final_state = state. state and y must not overlap each other or any input.
 * Base pointers 16-byte aligned (dt, A, D: 4). No workspace. */
SSD_API ssd_status_t ssd_decode_step(const ssd_desc_t* desc, const void* x, const float* dt,
                             const float* A, const void* B, const void* C, const float* D,
                             float* state, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
