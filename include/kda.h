/*
 * kda.h — C ABI of libkda: Kimi Delta Attention (KDA) and its Complex-KDA
 * (CKDA) range extension on AMD Instinct MI355X (gfx950).
 *
 * The recurrence (per batch b and head h):
 *   S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 * Update: "Semidirect Fourier Delta Attention" (arXiv 2607.11897), §1 eq. (1)
 * and the affine form §2.2 eq. (9); read-out from the post-update state with no
 * scale factor: same page, §3 eq. (14).  Ranges: KDA has alpha in [0,1] and
 * beta in [0,1] (same page, §3); CKDA allows alpha in [-1,1] and beta in [0,2]
 * ("Complex KDA: Understanding and Enhancing the Expressivity of Kimi Delta
 * Attention", the abstract).  The state S is d_k x d_v (§2.2), decayed along
 * its d_k rows.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates or frees memory, never synchronises (except where a flag
 *    says so) and never keeps a pointer after the call returns.  It creates
 *    no stream; events only for KDA_FLAG_STAGE_EVENTS (on first use).  The
 *    second stream of the overlapped forward is the caller's
 *    (kda_chunk_forward_side).
 *  - Layouts are row-major and contiguous:
 *      q, k, alpha : [B, T, H, Dk]     v, out : [B, T, H, Dv]    beta : [B, T, H]
 *      state       : [B, H, Dk, Dv]
 *    (decode uses the same layouts with T = 1).
 *  - q, k, v and out share `dtype`; alpha, beta and every state are fp32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream),
 *    part of it on the caller's second stream for kda_chunk_forward_side,
 *    joined back to `stream` by the caller's events, and is asynchronous:
 *    argument errors are reported synchronously, before any
 *    HIP call is made; launch failures come back as KDA_ERR_HIP; faults during
 *    execution surface at the caller's next synchronisation.
 *  - The library does not normalise q or k, applies no gate parameterisation
 *    and no output scale.
 *  - Supported shapes: Dk in {16, 32, 64, 128}; Dv a multiple of 16 in
 *    [16, 128]; chunk in {16, 32, 64}; B, H >= 1.  With dtype F32 the chunked
 *    forward with Dk = 128 additionally needs chunk = 64.
 *  - Alignment: q, k and alpha of the chunked forward, its workspace and the
 *    decode state are read with 16-byte vector accesses and must be 16-byte
 *    aligned; every other pointer must be aligned to its element size
 *    (KDA_ERR_MISALIGNED otherwise).
 *  - Thread safety: calls on different streams may run concurrently.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 18

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    KDA_ERR_BAD_SHAPE = 2,           /* a size is out of range or overflows */
    KDA_ERR_UNSUPPORTED = 3,         /* shape / dtype / mode / flag not supported */
    KDA_ERR_MISALIGNED = 4,          /* a pointer breaks the alignment rule below */
    KDA_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes below the queried size */
    KDA_ERR_ALIAS = 6,               /* an output overlaps an input it must not */
    KDA_ERR_HIP = 7,                 /* a HIP runtime call or launch failed */
    KDA_ERR_RANGE = 8,               /* KDA_FLAG_VALIDATE_RANGES found an input out of range */
    KDA_ERR_SCRATCH_LIMIT = 9        /* kda_chunk_forward_noalloc: workspace above its scratch */
} kda_status_t;

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype_t;

/* Admissible input ranges.  The mathematics is identical for both; the mode
 * states the caller's contract (KDA: alpha in [0,1], beta in [0,1]; CKDA:
 * alpha in [-1,1] incl. exact 0 and -1, beta in [0,2]).  Inputs outside the
 * stated range give results of the same formula but carry no accuracy
 * guarantee. */
typedef enum { KDA_MODE_KDA = 0, KDA_MODE_CKDA = 1 } kda_mode_t;

/* flags: check the inputs against the mode's ranges on the device before any
 * work is enqueued: every alpha in [0,1] (KDA) or [-1,1] (CKDA), every beta in
 * [0,1] (KDA) or [0,2] (CKDA), every theta of the phase variant finite; NaN is
 * out of range.  One extra read of alpha, beta (and theta); the call then
 * synchronises `stream` and returns KDA_ERR_RANGE, with nothing enqueued and
 * no output written, if any element is out of range.  Accepted by
 * kda_chunk_forward, its _states, _phase and _varlen forms and every
 * kda_decode_step form; the _prologue forms check nothing (their gates are
 * in range by construction); the backward entry points refuse the flag
 * (KDA_ERR_UNSUPPORTED).  Under graph capture of `stream` the call returns
 * KDA_ERR_UNSUPPORTED (the check must synchronise).  A debugging aid, not
 * for the timed path. */
#define KDA_FLAG_VALIDATE_RANGES 1u

/* flags: attach a pair of HIP events to every kernel launch of this call
 * (hipExtLaunchKernelGGL start/stop events, stamped by the kernel's own start
 * and end) so that kda_last_stage_times() can report per-kernel durations;
 * performs no extra work on the data. */
#define KDA_FLAG_STAGE_EVENTS 2u
/* flags: never cut a sequence into segments.  By default a dense forward whose
 * (b, h, 16-column) chains would leave most of the GPU idle (at most 64 of
 * them) and that has at least 128 chunks runs each (b, h) as several segments
 * side by side: each segment's affine map is computed ("Semidirect Fourier
 * Delta Attention" §2.2 eq. (10): affine maps compose), the segment start
 * states are chained in fp32, and every segment then runs from its own start.
 * The results agree with the unsegmented path up to rounding. */
#define KDA_FLAG_NO_SEGMENTS 4u
/* flags: with kda_chunk_forward_side, run every kernel on `stream` anyway (the
 * side stream and its events are not touched).  Calls without a side stream
 * always run on `stream` alone. */
#define KDA_FLAG_SINGLE_STREAM 8u
/* flags: with kda_chunk_forward_side, take the streamed form where it applies
 * (see kda_chunk_forward_side).  Opt-in because it needs a side stream with
 * a hardware queue of its own (kda_side_stream_create): on a shared queue
 * every call waits out the chain's 10 ms bound before its fallback runs. */
#define KDA_FLAG_STREAMED 16u

/* ABI version of the loaded library (KDA_ABI_VERSION it was built with). */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_string(int status);

/*
 * Bytes of device workspace kda_chunk_forward needs for these sizes
 * (the per-chunk WY factors of "Semidirect Fourier Delta Attention" §2.2).
 * Returns KDA_OK and writes *bytes, or an argument error (same rules as
 * kda_chunk_forward).  Makes no HIP call.
 */
kda_status_t kda_chunk_forward_workspace_size(int B, int T, int H, int Dk, int Dv,
                                              int chunk, kda_dtype_t dtype,
                                              size_t* bytes);

/*
 * Chunked forward over T tokens (prefill / training forward).  Executes the
 * chunkwise form: the state is carried from chunk to chunk and each chunk's
 * interior is solved in parallel through a compact WY representation of the
 * product of its diagonal-plus-rank-one transitions (triangular solve), which
 * reproduces the sequential recurrence up to rounding ("Kimi Delta Attention:
 * a bounded case study", Exercise 2; "Semidirect Fourier Delta Attention",
 * §1 and §2.2).
 *   q, k, v, alpha, beta : inputs, layouts above.  T >= 0 (T = 0 only copies
 *                          the initial state to final_state).  T need not be
 *                          a multiple of chunk.
 *   initial_state        : [B,H,Dk,Dv] fp32, or NULL for a zero state.
 *   out                  : [B,T,H,Dv] in dtype; must not overlap any input.
 *   final_state          : [B,H,Dk,Dv] fp32, or NULL.  May be exactly the
 *                          same pointer as initial_state (resume in place);
 *                          any other overlap with an input is KDA_ERR_ALIAS.
 *   workspace            : device buffer of at least the queried size; its
 *                          contents on entry are ignored and on exit are
 *                          unspecified.  Must not overlap any other argument.
 *   mode, flags          : see above; unknown flag bits -> KDA_ERR_UNSUPPORTED.
 *   stream               : hipStream_t to enqueue on.
 */
kda_status_t kda_chunk_forward(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta,
                               const float* initial_state,
                               void* out, float* final_state,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * kda_chunk_forward that also stores the chunk-start states: the state carried
 * from chunk to chunk in the chunkwise form ("Kimi Delta Attention: a bounded
 * case study", Exercise 2), i.e. for chunk n the state after tokens
 * 0 .. n*chunk - 1 (n = 0: initial_state, or zero), which a backward pass or a
 * resumed segment starts from.
 *   chunk_states : [B,H,NC,Dk,Dv] in dtype (NC = ceil(T / chunk)), rounded
 *                  to nearest even from the fp32 carried state for bf16;
 *                  required when T > 0; must not overlap any other argument.
 * Every other argument, rule and error is that of kda_chunk_forward.  The
 * states cost one extra write of B*H*NC*Dk*Dv elements.
 */
kda_status_t kda_chunk_forward_states(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta,
                                      const float* initial_state,
                                      void* out, float* final_state, void* chunk_states,
                                      int B, int T, int H, int Dk, int Dv, int chunk,
                                      kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Input parameterisation fused into the chunked forward ("Semidirect Fourier
 * Delta Attention" §3, the stable parameterisation, eqs. (15), (17), (18)):
 *   alpha = alpha_min + (alpha_max - alpha_min) * sigmoid(gate)        (15)
 *   beta  = beta_max * sigmoid(beta_logit)                             (17)
 *   k     = k_raw / (||k_raw||_2 + eps), over the Dk channels          (18)
 *   q     = q_raw / (||q_raw||_2 + eps) when normalize_q, else q_raw
 * computed in fp32 per token inside the kernels (a zero vector with eps = 0
 * stays zero; normalised q, k are rounded to dtype once).  The parameters
 * must lie in the mode's ranges: KDA 0 <= alpha_min <= alpha_max <= 1 and
 * 0 <= beta_max <= 1; CKDA -1 <= alpha_min <= alpha_max <= 1 (the gate range
 * of the "Complex KDA" abstract; alpha_min = -1, alpha_max = 1 gives
 * 2 sigmoid - 1) and 0 <= beta_max <= 2; eps >= 0; normalize_q 0 or 1.
 */
typedef struct {
    float alpha_min, alpha_max;
    float beta_max;
    float eps;
    int normalize_q;
} kda_prologue_t;

/* Events a kda_side_t carries: one marks the call's start on `stream`, one
 * marks the end of each part's chunk factors on the side stream. */
#define KDA_SIDE_EVENTS 9

/* A second stream and events owned by the caller, lent to one call of
 * kda_chunk_forward_side.  stream: a hipStream_t (default priority) of the same
 * device as the call's stream (another device's stream is ignored: the call
 * then keeps to its own stream); events: KDA_SIDE_EVENTS distinct hipEvent_t
 * (timing may be disabled).  The library records and waits on them only
 * during the call's enqueue; calls enqueued one after another may share one
 * kda_side_t, calls enqueued concurrently from several host threads may not. */
typedef struct {
    void* stream;
    void* events[KDA_SIDE_EVENTS];
} kda_side_t;

/*
 * kda_chunk_forward with a second stream for the overlap of the chunk-factor
 * kernels (intra-chunk WY, "Semidirect Fourier Delta Attention" §2.2) with the
 * state chain (§2.3), in one of two forms; either way the side stream is
 * joined to `stream` by side->events, so the call still ends on `stream` (a
 * graph captured from `stream` takes in the side stream through the events).
 *
 * Streamed (only with KDA_FLAG_STREAMED): bf16, chunk 64, Dk 128 or 64,
 * B H >= 8, no sequence segments, the final state not written over the
 * initial one, `stream` not the null stream, and at most 128 chain
 * workgroups: the (b, h, 16-column) chains taken 1, 2 or 4 column tiles per
 * workgroup (4 only at Dk = 128), the fewest tiles that leave half the
 * compute units to the factor kernels.  The chunk factors are formed on
 * side->stream while the chain,
 * already running on `stream`, consumes them chunk by chunk (each chunk is
 * published in the workspace with a ready word; the chain reads it from the
 * L2 cache of the XCD that formed it).  A chunk that needs the exact factor
 * kernel, or a wait past its bound (10 ms; typically because side->stream and
 * `stream` share a hardware queue: use kda_side_stream_create), makes the
 * chain give up; the call then forms the flagged chunks and reruns the chain
 * after the factors are complete, so results never depend on the timing.
 * The chain is the wide-slice kernel (operands straight into registers);
 * results are bitwise those of kda_chunk_forward (the same products in the
 * same order, whatever the column tiles per workgroup).
 *
 * In parts: otherwise (and without the flag), when the (b, h, 16-column)
 * chains number at most 128
 * (half the GPU or less), no sequence segments are chosen and there are at
 * least 256 chunks, the chunks of every (b, h) run in 8 consecutive parts: the
 * factors of part p + 1 are formed on side->stream while the chain runs part
 * p on `stream`.  The state crosses part boundaries in fp32, so results are
 * bitwise those of kda_chunk_forward.
 *
 * Other shapes, side == NULL or KDA_FLAG_SINGLE_STREAM run as
 * kda_chunk_forward.  The workspace query is kda_chunk_forward_workspace_size
 * (it reserves the ready words and control block of the streamed form, and the
 * state between parts, for every shape that could take them).  Errors: those
 * of kda_chunk_forward; a NULL side->stream or event is KDA_ERR_NULL_POINTER.
 */
kda_status_t kda_chunk_forward_side(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    const float* initial_state, void* out, float* final_state,
                                    int B, int T, int H, int Dk, int Dv, int chunk,
                                    kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    const kda_side_t* side);

/*
 * A kda_side_t for kda_chunk_forward_side on the current device: a stream
 * with a hardware queue of its own (created with a compute-unit mask that
 * holds every compute unit; HIP spreads ordinary streams over a few shared
 * queues, and two streams on one queue cannot run kernels at the same time,
 * which the streamed form needs) and KDA_SIDE_EVENTS events with timing
 * disabled and a device-scope release (they only order work on the device).  The stream is a blocking one: work on the null stream waits for
 * it, so the streamed form is not taken for calls on the null stream.  The
 * caller owns the result and releases it with kda_side_stream_destroy (which
 * first waits for the stream's work).  Errors: KDA_ERR_NULL_POINTER,
 * KDA_ERR_HIP (nothing is left allocated).
 */
kda_status_t kda_side_stream_create(kda_side_t* side);
kda_status_t kda_side_stream_destroy(kda_side_t* side);

/* Size of the built-in scratch of kda_chunk_forward_noalloc (bytes per device). */
#define KDA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * kda_chunk_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same computation and kernels as kda_chunk_forward, with the workspace
 * taken from an array of KDA_NOALLOC_SCRATCH_BYTES inside the library instead
 * of the caller's (one array per device, set aside when the library is loaded
 * on that device and held until the process ends).  The caller still passes
 * inputs and outputs; every argument, rule and result is that of
 * kda_chunk_forward, with these differences:
 *  - shapes whose kda_chunk_forward_workspace_size() exceeds
 *    KDA_NOALLOC_SCRATCH_BYTES return KDA_ERR_SCRATCH_LIMIT (checked before any
 *    HIP call);
 *  - all work runs on `stream`, and the flags
 *    KDA_FLAG_STAGE_EVENTS and KDA_FLAG_VALIDATE_RANGES are refused
 *    (KDA_ERR_UNSUPPORTED): the call creates no stream or event and makes no
 *    allocating call;
 *  - the array used is that of the device `stream` belongs to (the current
 *    device for the null stream); its address is looked up once per device.
 * Every call on a device shares that device's array: calls whose work
 * overlaps in time on one device (different streams, or several host threads
 * without ordering) race on it and give unspecified results.  Calls ordered
 * on one stream are safe; nothing needs clearing between them.
 */
kda_status_t kda_chunk_forward_noalloc(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* initial_state, void* out, float* final_state,
                                       int B, int T, int H, int Dk, int Dv, int chunk,
                                       kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                       void* stream);

/*
 * kda_chunk_forward from raw inputs through the parameterisation above: gate
 * takes alpha's place ([B,T,H,Dk] fp32 logits), beta_logit beta's ([B,T,H]
 * fp32), q_raw and k_raw those of q and k.  Every other argument, rule and
 * error is that of kda_chunk_forward; prologue == NULL is
 * KDA_ERR_NULL_POINTER and parameters outside the mode's ranges are
 * KDA_ERR_UNSUPPORTED.  Costs no extra pass over memory: the transforms run
 * where the kernels load the inputs.
 */
kda_status_t kda_chunk_forward_prologue(const void* q_raw, const void* k_raw, const void* v,
                                        const float* gate, const float* beta_logit,
                                        const kda_prologue_t* prologue,
                                        const float* initial_state, void* out,
                                        float* final_state,
                                        int B, int T, int H, int Dk, int Dv, int chunk,
                                        kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Phase variant ("Semidirect Fourier Delta Attention", §3 eq. (13) in the real
 * form of eq. (2) with the 2x2 rotation blocks of eq. (12)): channels 2p and
 * 2p+1 form one complex coordinate and the decay is
 *   Lambda_t = diag(alpha_t e^{i theta_t}), i.e. the block alpha_p R(theta_p),
 *   R(t) = [[cos t, -sin t], [sin t, cos t]], on state rows 2p, 2p+1;
 * the delta correction and the read-out are those of kda_chunk_forward
 * (theta = 0 is KDA; beta = 0 the rotating diagonal recurrence, Prop. 2.1).
 *   alpha, theta : [B,T,H,Dk/2] fp32, one decay and one phase (radians) per
 *                  channel pair; alpha follows the mode's gate range.
 * Every other argument, rule and error is that of kda_chunk_forward (the
 * workspace query is the same); theta == NULL with T > 0 is
 * KDA_ERR_NULL_POINTER.
 */
kda_status_t kda_chunk_forward_phase(const void* q, const void* k, const void* v,
                                     const float* alpha, const float* theta, const float* beta,
                                     const float* initial_state, void* out, float* final_state,
                                     int B, int T, int H, int Dk, int Dv, int chunk,
                                     kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed (variable-length) batches: N sequences stored back to back, sequence
 * i on token rows cu_seqlens[i] .. cu_seqlens[i+1] - 1 of q, k, alpha
 * [total_T,H,Dk], v, out [total_T,H,Dv] and beta [total_T,H]; every sequence
 * is chunked from its own start and carries its own state
 * (initial_state / final_state [N,H,Dk,Dv] fp32, either may be NULL).
 *   cu_seqlens : device int32 [N + 1], 0 = cu[0] <= cu[1] <= ... <= cu[N] =
 *                total_T.  It is read on the device only: a table that breaks
 *                this rule is clamped (offsets into [0, total_T], made
 *                nondecreasing), so the kernels stay inside the buffers, but
 *                the results for the affected rows are unspecified and rows
 *                past cu[N] are not written.
 *   prologue   : NULL (alpha, beta, q, k as given) or the parameterisation of
 *                kda_chunk_forward_prologue (alpha, beta then hold logits).
 *   workspace  : at least kda_chunk_forward_varlen_workspace_size() bytes.
 * Empty sequences are allowed (their state passes through).  Every other rule
 * and error is that of kda_chunk_forward; N in [1, 2^24].
 */
kda_status_t kda_chunk_forward_varlen_workspace_size(int N, int total_T, int H, int Dk, int Dv,
                                                     int chunk, kda_dtype_t dtype,
                                                     size_t* bytes);
kda_status_t kda_chunk_forward_varlen(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta,
                                      const kda_prologue_t* prologue,
                                      const int* cu_seqlens, int N,
                                      const float* initial_state, void* out,
                                      float* final_state,
                                      int total_T, int H, int Dk, int Dv, int chunk,
                                      kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * One single-token step for every (b, h), applied to a resident fp32 state in
 * place: S <- (I - beta k k^T) diag(alpha) S + beta k v^T, then out = S^T q
 * (eq. (1) and eq. (14) with T = 1).  One read and one write of the state.
 *   q, k : [B,H,Dk] dtype;  v : [B,H,Dv] dtype;  alpha : [B,H,Dk] fp32;
 *   beta : [B,H] fp32;  state : [B,H,Dk,Dv] fp32 (read and written);
 *   out  : [B,H,Dv] dtype; must not overlap state or any input.
 */
kda_status_t kda_decode_step(const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta,
                             float* state, void* out,
                             int B, int H, int Dk, int Dv,
                             kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                             void* stream);

/*
 * kda_decode_step from raw inputs through the parameterisation of
 * kda_prologue_t ("Semidirect Fourier Delta Attention" §3 eqs. (15), (17),
 * (18)): gate takes alpha's place ([B,H,Dk] fp32 logits), beta_logit beta's
 * ([B,H] fp32), q_raw and k_raw those of q and k, so that
 *   alpha = alpha_min + (alpha_max - alpha_min) sigmoid(gate),
 *   beta = beta_max sigmoid(beta_logit),  k = k_raw / (|k_raw| + eps)
 * (q likewise when normalize_q; a zero vector with eps = 0 stays zero), with
 * the normalised q, k rounded to dtype once, as kda_chunk_forward_prologue
 * does.  Every other argument, rule and error is that of kda_decode_step;
 * prologue == NULL is KDA_ERR_NULL_POINTER and parameters outside the
 * mode's ranges are KDA_ERR_UNSUPPORTED.  Same single read and write of the
 * state: the transforms run where the kernel loads the inputs.
 */
kda_status_t kda_decode_step_prologue(const void* q_raw, const void* k_raw, const void* v,
                                      const float* gate, const float* beta_logit,
                                      const kda_prologue_t* prologue, float* state, void* out,
                                      int B, int H, int Dk, int Dv, kda_dtype_t dtype,
                                      kda_mode_t mode, unsigned flags, void* stream);

/*
 * kda_decode_step for the phase variant (see kda_chunk_forward_phase):
 * alpha, theta : [B,H,Dk/2] fp32, one per channel pair; S <- (I - beta k k^T)
 * Lambda S + beta k v^T with Lambda's 2x2 blocks on row pairs, out = S^T q.
 */
kda_status_t kda_decode_step_phase(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* theta, const float* beta,
                                   float* state, void* out,
                                   int B, int H, int Dk, int Dv,
                                   kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                   void* stream);

/*
 * Backward of kda_chunk_forward (dense batches, gates and beta as given):
 * the gradients of the scalar loss
 *   L = sum_t <o_t, d_out_t> + <S_T, d_final_state>
 * with respect to q, k, v, alpha, beta and initial_state, for the recurrence
 * of "Semidirect Fourier Delta Attention" §1 eq. (1) read out by §3 eq. (14)
 * (reverse-mode differentiation of the chunkwise form of "Kimi Delta
 * Attention: a bounded case study", Exercise 2).  The forward is recomputed
 * inside the call; nothing from a previous forward call is needed.
 *   inputs : q, k, v, alpha, beta, initial_state as for kda_chunk_forward
 *            (initial_state NULL = zero); d_out [B,T,H,Dv] in dtype;
 *            d_final_state [B,H,Dk,Dv] fp32 or NULL (= zero)
 *   outputs: dq, dk [B,T,H,Dk] and dv [B,T,H,Dv] in dtype; d_alpha
 *            [B,T,H,Dk] and d_beta [B,T,H] fp32; d_initial_state [B,H,Dk,Dv]
 *            fp32 or NULL (not wanted)
 * Supported: chunk in {32, 64}; Dk in {32, 64, 128} (fp32: Dk, Dv <= 64, else
 * KDA_ERR_UNSUPPORTED);
 * Dv a multiple of 16 up to 128.  q, k, d_out, alpha and the workspace are
 * 16-byte aligned, the rest element-aligned.  No output may overlap an input,
 * another output or the workspace.  The workspace (caller-owned, contents
 * undefined after the call) is at least
 * kda_chunk_backward_workspace_size bytes.  Status codes as for the forward;
 * the call only enqueues kernels on `stream`.
 */
kda_status_t kda_chunk_backward_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk,
                                               kda_dtype_t dtype, size_t* bytes);
kda_status_t kda_chunk_backward(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                const float* initial_state, const void* d_out,
                                const float* d_final_state, void* dq, void* dk, void* dv,
                                float* d_alpha, float* d_beta, float* d_initial_state,
                                int B, int T, int H, int Dk, int Dv, int chunk,
                                kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward and backward of one training step split into two calls, so the
 * backward does not recompute the forward (the backward call above does).
 * kda_chunk_forward_save is kda_chunk_forward (same inputs, outputs and
 * supported set as kda_chunk_backward; out, final_state as for the forward,
 * final_state may be NULL) that also leaves in `saved` what the gradient pass
 * needs: the per-chunk factors, (I + A)^-1 in fp32, the fp32 chunk-start
 * states and Delta of every chunk (the same chunkwise form, "Kimi Delta
 * Attention: a bounded case study", Exercise 2).  `saved` is caller-owned,
 * at least kda_chunk_backward_workspace_size bytes, 16-byte aligned.
 * kda_chunk_backward_saved then gives the gradients of kda_chunk_backward
 * (bit for bit the same) from that workspace and the same q, k, v, alpha,
 * beta (initial_state is not passed again: the saved states hold it).  The
 * saved workspace is used up by one kda_chunk_backward_saved call (the call
 * rearranges its factors in place); a second gradient pass needs a new
 * kda_chunk_forward_save.  Nothing checks that the inputs or the workspace
 * are those of the save call: other data give undefined gradients (never an
 * out-of-bounds access).  Status codes as for kda_chunk_backward; both calls
 * only enqueue kernels on `stream`.
 */
kda_status_t kda_chunk_forward_save(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    const float* initial_state, void* out, float* final_state,
                                    int B, int T, int H, int Dk, int Dv, int chunk,
                                    kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                    void* saved, size_t saved_bytes, void* stream);
kda_status_t kda_chunk_backward_saved(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, const void* d_out,
                                      const float* d_final_state, void* dq, void* dk, void* dv,
                                      float* d_alpha, float* d_beta, float* d_initial_state,
                                      int B, int T, int H, int Dk, int Dv, int chunk,
                                      kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                      void* saved, size_t saved_bytes, void* stream);

/*
 * Backward of kda_chunk_forward_phase ("Semidirect Fourier Delta Attention",
 * §3 eq. (13): the decay of channel pair p is alpha_p R(theta_p)): the
 * gradients of sum_t <o_t, d_out_t> + <S_T, d_final_state> with respect to q,
 * k, v, alpha, theta, beta and initial_state.  With phi_t the running sum of
 * a pair's phases over the sequence, the variant is the plain recurrence on q
 * and k rotated pair by pair by -phi_t with alpha_p on both channels of the
 * pair, its final state rotated back by phi_T; the call forms those inputs
 * (rounded to dtype), runs the plain backward on them and maps its gradients
 * back: dq_t, dk_t rotated by phi_t, the pair's two channel gradients summed
 * into d_alpha, and d_theta_s the sum over t >= s of the derivative of the
 * loss in phi_t.
 *   alpha, theta, d_alpha, d_theta : [B,T,H,Dk/2] fp32 (the forward's layout);
 *   every other argument, layout, rule and status code as kda_chunk_backward;
 *   workspace: at least kda_chunk_backward_phase_workspace_size bytes.
 * theta == NULL or d_theta == NULL with T > 0 is KDA_ERR_NULL_POINTER.
 */
kda_status_t kda_chunk_backward_phase_workspace_size(int B, int T, int H, int Dk, int Dv,
                                                     int chunk, kda_dtype_t dtype, size_t* bytes);
kda_status_t kda_chunk_backward_phase(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* theta, const float* beta,
                                      const float* initial_state, const void* d_out,
                                      const float* d_final_state, void* dq, void* dk, void* dv,
                                      float* d_alpha, float* d_theta, float* d_beta,
                                      float* d_initial_state, int B, int T, int H, int Dk, int Dv,
                                      int chunk, kda_dtype_t dtype, kda_mode_t mode,
                                      unsigned flags, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Backward of kda_chunk_forward_prologue: the same loss gradients with respect
 * to the raw inputs q_raw, k_raw, v, the gate logits (`gate`, alpha's layout),
 * the beta logits ([B,T,H]) and initial_state, through the stable
 * parameterisation of "Semidirect Fourier Delta Attention" §3 (eqs. (15),
 * (17), (18); `prologue` as for the forward).  The transformed inputs are
 * formed first (as the forward forms them), the backward runs on them, and
 * the chain rule through the parameterisation maps the gradients back:
 *   d gate = d alpha (alpha_max - alpha_min) s (1 - s),  d beta_logit = d beta
 *   beta_max s (1 - s) (s the logistic of the logit), d k_raw = d k / (n + eps)
 *   - k_raw <k_raw, d k> / (n (n + eps)^2) with n = |k_raw| (q_raw likewise
 *   when normalize_q, else d q_raw = d q).
 * Outputs dq_raw, dk_raw, dv in dtype; d_gate, d_beta_logit, d_initial_state
 * fp32 (d_initial_state may be NULL).  Shapes, alignment (gate, dq_raw,
 * dk_raw and d_gate 16-byte aligned too), aliasing and status rules as for
 * kda_chunk_backward; the workspace is at least
 * kda_chunk_backward_prologue_workspace_size bytes.
 */
kda_status_t kda_chunk_backward_prologue_workspace_size(int B, int T, int H, int Dk, int Dv,
                                                        int chunk, kda_dtype_t dtype, size_t* bytes);
kda_status_t kda_chunk_backward_prologue(const void* q_raw, const void* k_raw, const void* v,
                                         const float* gate, const float* beta_logit,
                                         const float* initial_state, const void* d_out,
                                         const float* d_final_state, const kda_prologue_t* prologue,
                                         void* dq_raw, void* dk_raw, void* dv, float* d_gate,
                                         float* d_beta_logit, float* d_initial_state,
                                         int B, int T, int H, int Dk, int Dv, int chunk,
                                         kda_dtype_t dtype, kda_mode_t mode, unsigned flags,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of kda_chunk_forward_varlen (packed batch of N sequences, device
 * cu_seqlens [N + 1], the same sanitising rules as the forward): the gradients
 * of sum_t <o_t, d_out_t> + sum_i <S_T,i, d_final_state_i> with respect to q,
 * k, v, alpha, beta ([total_T, H, .] as for the forward) and the per-sequence
 * initial states ([N, H, Dk, Dv]; NULL = zero).  d_final_state and
 * d_initial_state are [N, H, Dk, Dv] fp32 or NULL; an empty sequence has
 * d_initial_state = d_final_state.  Shape support, alignment, aliasing and
 * status rules as for kda_chunk_backward (cu_seqlens 4-byte aligned); the
 * workspace is at least kda_chunk_backward_varlen_workspace_size bytes.
 */
kda_status_t kda_chunk_backward_varlen_workspace_size(int N, int total_T, int H, int Dk, int Dv,
                                                      int chunk, kda_dtype_t dtype, size_t* bytes);
kda_status_t kda_chunk_backward_varlen(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const int* cu_seqlens, int N, const float* initial_state,
                                       const void* d_out, const float* d_final_state, void* dq,
                                       void* dk, void* dv, float* d_alpha, float* d_beta,
                                       float* d_initial_state, int total_T, int H, int Dk, int Dv,
                                       int chunk, kda_dtype_t dtype, kda_mode_t mode,
                                       unsigned flags, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * The raw-input backward (kda_chunk_backward_prologue) of a packed batch
 * (kda_chunk_backward_varlen): gate, beta_logit, q_raw, k_raw, v, d_out and
 * their gradients are [1, total_T, H, *] with the N sequences' rows given by
 * the device table cu_seqlens [N+1]; initial_state, d_final_state and
 * d_initial_state are per sequence [N,H,Dk,Dv].  Every other argument, rule
 * and error is that of the two; cu_seqlens == NULL is KDA_ERR_NULL_POINTER.
 */
kda_status_t kda_chunk_backward_varlen_prologue_workspace_size(int N, int total_T, int H, int Dk,
                                                               int Dv, int chunk,
                                                               kda_dtype_t dtype, size_t* bytes);
kda_status_t kda_chunk_backward_varlen_prologue(
    const void* q_raw, const void* k_raw, const void* v, const float* gate,
    const float* beta_logit, const int* cu_seqlens, int N, const float* initial_state,
    const void* d_out, const float* d_final_state, const kda_prologue_t* prologue, void* dq_raw,
    void* dk_raw, void* dv, float* d_gate, float* d_beta_logit, float* d_initial_state,
    int total_T, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype, kda_mode_t mode,
    unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunk-local gate summary (log-magnitude, sign and zero form of the
 * per-channel decay products inside each chunk; "Kimi Delta Attention: a
 * bounded case study", Chapter 12 §12.1 per-channel decay, with the CKDA gate
 * range of the "Complex KDA" abstract).  For chunk n, local token r and channel
 * c (NC = ceil(T / chunk)):
 *   L[b,h,n,r,c]    = sum over j <= r in the chunk with alpha_j != 0 of
 *                     log2|alpha_j|   (fp32)
 *   meta[b,h,n,r,c] = (zpos << 1) | parity, where parity = (number of
 *                     negative alpha_j, j <= r in the chunk) mod 2 and
 *                     zpos = 1 + (last j <= r with alpha_j == 0), 0 if none
 *   gend[b,h,n,c]   = product of alpha over the chunk (fp32 running product)
 * so that prod_{j=i+1..r} alpha_j = [zpos_r <= i+1] (-1)^(parity_r - parity_i)
 * 2^(L_r - L_i).  alpha : [B,T,H,Dk] fp32.  L : [B,H,NC,chunk,Dk] fp32,
 * meta : [B,H,NC,chunk,Dk] uint8, gend : [B,H,NC,Dk] fp32; entries of a short
 * last chunk past T are written as L = 0, meta = 0.  Same shape rules as the
 * forward (Dk in {16,32,64,128}, chunk in {16,32,64}).  alpha, L and gend are
 * accessed 16 bytes at a time and must be 16-byte aligned, meta 4-byte
 * aligned (KDA_ERR_MISALIGNED otherwise).
 */
kda_status_t kda_gate_prep(const float* alpha, float* L, unsigned char* meta,
                           float* gend, int B, int T, int H, int Dk, int chunk,
                           void* stream);

/*
 * Per-kernel durations, in milliseconds, of the most recent call on this
 * process that passed KDA_FLAG_STAGE_EVENTS.  Waits for that call's events.
 * Writes up to `max` entries to ms[] and (if names != NULL) static kernel names
 * to names[]; *count receives the number of kernels of that call.
 */
kda_status_t kda_last_stage_times(float* ms, const char** names, int max, int* count);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
