/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library with dynamic
 * per-tile FP8-E4M3 fake quantize-dequantize (QDQ) of the recurrent state.
 *
 * The method (the pages: NVIDIA Model-Optimizer pull requests #2497 "GDN
 * state/W QAT foundation", #2519 "Torch GDN/KDA decode QAT", #2506 "KDA
 * prefill numerical emulation"):
 *   - Gated delta rule, per sequence n and head h, state S (dv x dk, row =
 *     value channel, column = key channel), token t:
 *         S <- S * a_t        (a_t = exp(g_t); or S * diag(exp(g_t)) for a
 *                              per-key-channel gate, #2506 "per-key-channel
 *                              retention")
 *         u  = beta_t (v_t - S k_t);   S <- S + u k_t^T;   o_t = S q_t
 *   - Computed chunk-parallel in 64-token chunks (#2497 "What does this PR
 *     do?": fused path with chunk size 64) with WY/UT-transformed W and U and
 *     an exact triangular solve (the default of #2506 "Add KDA prefill
 *     numerical emulation for QAT", "What does this PR do?").
 *   - State QDQ (#2497 "What does this PR do?"): at every chunk boundary, for
 *     every tile of 64 value rows x all dk key columns of every (sequence,
 *     head), scale s = amax / 448 (zero guard: s = 1 when amax / 448 is not
 *     positive), S <- RNE_E4M3(S / s) * s.  The state stays fp32.
 *   - Prefill -> decode handoff (#2519 "What does this PR do?", step 3): QDQ
 *     at the handoff and after every later recurrent write; each output is
 *     taken from the updated working state before that QDQ.
 *   - Optional W QDQ (#2497 "What does this PR do?": independent dynamic FP8
 *     fake QDQ of the WY-transformed W; Usage: grouping per token and head):
 *     per chunk W = T (K * exp(gamma)) with T = (I + A)^-1 diag(beta) and
 *     gamma the in-chunk cumulative log-gate (per key channel with a
 *     per-channel gate: #2506 "What does this PR do?" and "Usage", the KDA
 *     state/W controls and the KDA W quantizer); every row of W (one token of
 *     one head, all dk keys) gets its own scale amax / 448 (same zero guard)
 *     and W <- RNE_E4M3(W / s) * s before the pseudo-values
 *     U' = T V - W S^T use it.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers on the current HIP device unless
 *     stated otherwise.  The caller owns every buffer; the library allocates
 *     nothing and keeps no state beyond a per-device capability cache.
 *   - `stream` is a hipStream_t passed as void*.  Work is enqueued
 *     asynchronously on it; no entry point synchronizes the host.
 *   - Arguments are checked on the host before anything is launched.  A
 *     failed check returns GDN_ERR_INVALID_ARG or GDN_ERR_UNSUPPORTED and
 *     launches nothing; gdn_last_error() then describes the failure.  The
 *     contents of device index arrays (cu_seqlens, lengths) are
 *     preconditions and are not read on the host.
 *   - Non-finite inputs are outside the contract.
 *   - Calls are reentrant; calls that write the same buffers race.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned buffer, bad flag */
    GDN_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head size, dtype combo) */
    GDN_ERR_DEVICE = 3         /* no gfx950 device current, a HIP call failed, or (from */
                               /* gdn_workspace_status) a device-side wait ran out */
} gdn_status_t;

typedef enum {
    GDN_F32 = 0,
    GDN_BF16 = 1
} gdn_dtype_t;

/* qdq_flags bits */
#define GDN_QDQ_CHUNK 1u   /* QDQ after every 64-token chunk of the chunked prefix and at its end (t = P) */
#define GDN_QDQ_WRITE 2u   /* QDQ at the handoff t = P and after every recurrent write t > P */
#define GDN_QDQ_W 4u       /* W QDQ in every chunk of the chunked prefix (either gate; */
                           /* gdn_decode_step and the recurrent suffix have no W and ignore it) */
#define GDN_QDQ_INT8 8u    /* gdn_decode_step only: each per-write QDQ is INT8 block-32 */
                           /* (see gdn_state_qdq_int8) instead of FP8 per tile */

typedef struct {
    int32_t n_seqs;            /* N >= 1 */
    int32_t n_heads;           /* H >= 1 */
    int32_t dk;                /* key head size: 64 or 128 */
    int32_t dv;                /* value head size: a multiple of 64, at most 256 */
    int64_t total_tokens;      /* rows of the packed q/k/v/o buffers (decode: must equal n_seqs) */
    int32_t io_dtype;          /* gdn_dtype_t of q, k, v */
    int32_t o_dtype;           /* gdn_dtype_t of o */
    int32_t gate_per_channel;  /* 0: g is [T, H]; 1: g is [T, H, dk] (per-key-channel gate) */
    uint32_t qdq_flags;        /* GDN_QDQ_* bits */
    int32_t gate_grid_log2;    /* 0, or k in 1 .. 24: log-retention grid of the recurrent */
                               /* writes (see below) */
} gdn_shape_t;

/*
 * Log-retention grid (#2509 "Add experimental GDN/KDA decode and replay QAT",
 * "What does this PR do?": an optional rounding of the log-retention among
 * the per-token decode policies; its pilot selected a grid of 1/256).  With
 * gate_grid_log2 = k > 0, every recurrent write -- each gdn_decode_step token
 * and each token P < t <= L of gdn_chunk_fwd's recurrent suffix -- uses the
 * log-gate rounded to the nearest multiple of 2^-k, ties to even:
 *   g~ = 2^-k * rint(2^k * g)   (per key channel for a per-channel gate)
 * and decays by exp(g~).  The chunked prefix t <= P is unchanged.  With a
 * power-of-two step every operation of the rounding is exact in fp32, so g~
 * is a pure function of the stored fp32 gate.
 */

/* Optional per-boundary record of the chunked prefix, for parity checks, and
 * a timing hook.  Boundary b of sequence n is b = bound_offsets[n] + i for its
 * i-th chunk end (i = 0 .. ceil(P_n / 64) - 1).  All pointers nullable; the
 * record needs bound_offsets when any of its five arrays is set. */
typedef struct {
    const int32_t* bound_offsets;  /* [N + 1] device; prefix sums of ceil(P_n / 64) */
    float* bound_pre;              /* [n_bounds, H, dv, dk] state after the chunk, before QDQ */
    float* bound_post;             /* [n_bounds, H, dv, dk] state after QDQ (= pre when none) */
    float* scales;                 /* [n_bounds, H, dv / 64] QDQ scales (1 when none) */
    void* kernel_start;            /* hipEvent_t or NULL: recorded on the stream just before */
    void* kernel_end;              /* and just after the sequential state kernel (timing hook; */
                                   /* a separate per-chunk solve kernel runs before kernel_start, */
                                   /* a fused one inside the bracket) */
    int32_t schedule;              /* GDN_SCHEDULE_*: how the per-chunk solve is scheduled */
    float* w_pre;                  /* [n_bounds, H, 64, dk] W of chunk b before its QDQ (GDN_QDQ_W) */
    float* w_post;                 /* [n_bounds, H, 64, dk] W after QDQ; rows past the chunk's */
                                   /* end are 0.  Both written only with GDN_QDQ_W. */
    /* Per-token record of the recurrent suffix (tokens P_n < t <= L_n): token t of
     * sequence n at s = suffix_offsets[n] + (t - 1 - P_n).  Needs suffix_offsets. */
    const int32_t* suffix_offsets; /* [N + 1] device; prefix sums of L_n - P_n */
    float* suffix_pre;             /* [n_suffix, H, dv, dk] state after token t, before its QDQ */
    float* suffix_post;            /* [n_suffix, H, dv, dk] state after its QDQ (= pre when none) */
    int32_t* status;               /* device int32 or NULL: receives the call's status word once */
                                   /* its kernels are done (0 clean; 1 a bounded wait ran out; */
                                   /* 2 index arrays out of contract), on the call's stream */
} gdn_debug_t;

/* gdn_debug_t.schedule.  The per-chunk solve (T and P records of every chunk
 * and head) either runs as its own kernel before the sequential state kernel
 * (SPLIT) or inside the same launch, on compute units the state kernel leaves
 * idle, handing each record over through a ready flag (FUSED).  AUTO (also
 * when debug is NULL) fuses when the state kernel's workgroups fill at most
 * half of the compute units; FUSED fuses whenever at least 8 compute units
 * stay free.  Both give bit-identical results, for either gate. */
#define GDN_SCHEDULE_AUTO 0
#define GDN_SCHEDULE_SPLIT 1
#define GDN_SCHEDULE_FUSED 2
/* Test hook for the failure path of the fused launch: the state workgroups
 * run without their producers, so every wait for a record runs out (200 ms of
 * the device's real-time clock per workgroup) and the launch still ends; the
 * state and the outputs after the first chunk come out NaN.  Not for use. */
#define GDN_SCHEDULE_FUSED_NO_PRODUCERS 3

/*
 * gdn_chunk_fwd -- chunked gated delta rule forward over packed sequences.
 *
 *   q, k  [total_tokens, H, dk]   io_dtype, row-major (16-byte aligned)
 *   v     [total_tokens, H, dv]   io_dtype
 *   beta  [total_tokens, H]       fp32
 *   g     [total_tokens, H] or [total_tokens, H, dk]   fp32 natural-log gate (<= 0 expected)
 *   cu_seqlens  [N + 1] int32: storage segment of sequence n is rows
 *               [cu_seqlens[n], cu_seqlens[n+1]); cu_seqlens[N] <= total_tokens.
 *   seq_lens    [N] int32 valid length L_n <= segment length; NULL: the segment length.
 *               Rows of a segment past L_n are padding: they never touch the state
 *               and their o rows are written as 0.
 *   prefix_lens [N] int32 chunked-prefix length P_n <= L_n; NULL: P_n = L_n.  Tokens
 *               P_n < t <= L_n run as recurrent writes (#2519 prefix/suffix split).
 *   initial_state [N, H, dv, dk] fp32 or NULL (zero).  Used as given (not quantized).
 *   o      [total_tokens, H, dv]  o_dtype (output)
 *   final_state [N, H, dv, dk] fp32 (output), may alias initial_state.
 *   workspace   device scratch of at least gdn_chunk_fwd_workspace_bytes(shape)
 *               bytes, 256-byte aligned, owned by the caller; its contents on entry
 *               are ignored.  On return it holds the call's status word (read it
 *               with gdn_workspace_status); the rest is unspecified.  Two calls that
 *               share a workspace must not overlap in time.
 *   debug  NULL or a per-boundary record (see gdn_debug_t).
 *
 * Device-side failures (the call itself returned GDN_OK; gdn_workspace_status
 * reports them once the stream has run the call):
 *   - index arrays out of contract (cu_seqlens decreasing or beyond
 *     total_tokens, a length above its segment, P_n > L_n, a negative entry):
 *     every kernel of the call returns before touching o or final_state;
 *   - a bounded wait of the single-launch schedule for a producer's record
 *     ran out (200 ms, e.g. when the GPU is shared): that (sequence, head)'s
 *     state and outputs from then on are NaN.
 *
 * fp32 q, k, v with dk = 128 run as the token recurrence with the same QDQ
 * points and records (the chunked form regrouped, identical up to rounding;
 * slower, for reference precision); they take no GDN_QDQ_W
 * (GDN_ERR_UNSUPPORTED).
 *
 * QDQ placement for token t of a sequence (1-based): after token t when
 * (GDN_QDQ_CHUNK and t <= P and (t % 64 == 0 or t == P)) or
 * (GDN_QDQ_WRITE and t >= max(P, 1)); chunks start at each sequence's first
 * valid token.
 */
gdn_status_t gdn_chunk_fwd(const gdn_shape_t* shape,
                           const void* q, const void* k, const void* v,
                           const float* beta, const float* g,
                           const int32_t* cu_seqlens, const int32_t* seq_lens,
                           const int32_t* prefix_lens,
                           const float* initial_state,
                           void* o, float* final_state,
                           void* workspace, size_t workspace_bytes,
                           const gdn_debug_t* debug, void* stream);

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and checks as gdn_chunk_fwd,
 * without the workspace: the call uses a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, and calls no allocating routine.
 *   - A shape whose gdn_chunk_fwd_workspace_bytes exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_UNSUPPORTED before anything is
 *     launched (use gdn_chunk_fwd with a caller workspace).
 *   - Every call on a GPU shares that GPU's array: calls that overlap in time
 *     on one GPU (other streams, other threads) race.  Each call clears what
 *     must start at zero; the array keeps the last call's contents.
 *   - The call's status word lives in the array: pass debug->status to receive
 *     it on the stream (gdn_workspace_status has no pointer to read).
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status_t gdn_chunk_fwd_noalloc(const gdn_shape_t* shape,
                                   const void* q, const void* k, const void* v,
                                   const float* beta, const float* g,
                                   const int32_t* cu_seqlens, const int32_t* seq_lens,
                                   const int32_t* prefix_lens,
                                   const float* initial_state,
                                   void* o, float* final_state,
                                   const gdn_debug_t* debug, void* stream);

/*
 * gdn_workspace_status -- the status word a gdn_chunk_fwd or gdn_chunk_bwd_dh
 * call left in its workspace.  Reads the 4 bytes at the workspace's start on
 * `stream` (the stream of that call) and synchronizes it, so it is not for
 * code under graph capture.  Returns GDN_OK when the call
 * ran cleanly, GDN_ERR_INVALID_ARG when the device found its index arrays out
 * of contract (nothing was computed), GDN_ERR_DEVICE when a bounded wait ran
 * out (outputs hold NaN) or the read failed; gdn_last_error() says which.
 *   workspace   the workspace passed to that call (device pointer)
 */
gdn_status_t gdn_workspace_status(const void* workspace, void* stream);

/*
 * gdn_chunk_fwd_workspace_bytes -- bytes of device workspace gdn_chunk_fwd
 * needs for this shape: the per-chunk solve T = (I + A)^-1 diag(beta) and the
 * decayed, masked P = Q K^T of every (chunk, head) (12 KiB each, for the
 * worst-case chunk count ceil(total_tokens / 64) + n_seqs), with GDN_QDQ_W
 * the quantized W of every (chunk, head) (dk * 128 + 1024 bytes each), plus
 * the status word, the chunk offsets and one ready flag per (chunk, head).  Returns 0 for an
 * invalid shape (gdn_last_error() says why).
 */
size_t gdn_chunk_fwd_workspace_bytes(const gdn_shape_t* shape);

/*
 * gdn_state_qdq -- standalone per-tile state QDQ (#2497: one scalar scale per
 * full-key x 64-value-column tile; #2497 "fp8_scalar_qdq" applies a scale per
 * tile).
 *   in, out  [n_states, dv, dk] fp32 (out may alias in); dv % 64 == 0,
 *            dk % 4 == 0, 4 <= dk <= 256, 16-byte aligned.
 *   scales   [n_states, dv / 64] fp32 output, or NULL.
 */
gdn_status_t gdn_state_qdq(const float* in, float* out, float* scales,
                           int64_t n_states, int32_t dv, int32_t dk, void* stream);

/*
 * gdn_state_qdq_int8 -- standalone INT8 block-32 state QDQ (#2519 "What does
 * this PR do?" and its recipe list: dynamic INT8 state quantization with
 * 32-element blocks).  The page gives no formula; the library's reading:
 * every block of 32 consecutive key columns of a state row is one group,
 * scale s = amax / 127 (s = 1 when that is not positive), code = x / s
 * (IEEE fp32 division) rounded half to even and clamped to [-127, 127],
 * stored value code * s (fp32).
 *   in, out  [n_states, dv, dk] fp32 (out may alias in); dv % 64 == 0,
 *            dk % 32 == 0, 32 <= dk <= 256, 16-byte aligned.
 *   scales   [n_states, dv, dk / 32] fp32 output, or NULL.
 */
gdn_status_t gdn_state_qdq_int8(const float* in, float* out, float* scales,
                                int64_t n_states, int32_t dv, int32_t dk, void* stream);

/*
 * gdn_decode_step -- one recurrent token per sequence against a stored state
 * (#2519 step 3: read the stored state, output from the updated working
 * state, QDQ before storing when GDN_QDQ_WRITE is set).
 *   shape->total_tokens must equal shape->n_seqs; GDN_QDQ_CHUNK is ignored.
 *   q, k  [N, H, dk] io_dtype;  v [N, H, dv] io_dtype
 *   beta  [N, H] fp32;  g [N, H] or [N, H, dk] fp32
 *   active [N] int32 or NULL (all active): sequence n takes the step when
 *          active[n] != 0; for the others nothing is read or written (state, o,
 *          state_pre and scales keep their contents) -- sequences of a batch
 *          that end at different lengths (#2519 "What does this PR do?": prefill
 *          and full lengths per sequence)
 *   state [N, H, dv, dk] fp32, read and written in place
 *   o     [N, H, dv] o_dtype
 *   state_pre  [N, H, dv, dk] fp32 or NULL: the updated state before QDQ (parity record)
 *   scales     [N, H, dv / 64] fp32 or NULL: QDQ scales (1 when no QDQ); with
 *              GDN_QDQ_INT8 and GDN_QDQ_WRITE [N, H, dv, dk / 32], one per block
 */
gdn_status_t gdn_decode_step(const gdn_shape_t* shape,
                             const void* q, const void* k, const void* v,
                             const float* beta, const float* g, const int32_t* active,
                             float* state, void* o,
                             float* state_pre, float* scales, void* stream);

/*
 * gdn_chunk_bwd_dh -- backward state recurrence of the chunked forward with
 * identity straight-through gradients through every QDQ (#2497 "What does
 * this PR do?": identity straight-through gradients for QAT/QAD).  For the
 * loss L = sum_t o_t . d_o_t + <S_L, d_final_state> of each sequence, the
 * gradient of the state entering every 64-token chunk, and of v, by the
 * chunk form of the reverse recurrence (per chunk, from the last):
 *     dU' = P^T dO + diag(e^{gamma_C - gamma}) K dh^T,   Y = T^T dU',
 *     dh  <- e^{gamma_C} dh + dO^T (Q o e^gamma) - Y^T (K o e^gamma),
 * with T, P, gamma as in the forward.  The straight-through QDQ leaves the
 * states out of it, so no forward state is needed.  Whole sequences (no
 * prefix/suffix split); scalar gate; bf16 q, k and d_o.
 * The backward of a W-QDQ forward (GDN_QDQ_W): the forward's U' = T V -
 * Wq h^T takes the row-quantized Wq = Q(W), which the quantizer's identity
 * straight-through rule holds fixed in the gradient of h, so the last term
 * is - dU'^T Wq; the call recomputes Wq with the forward's own code (bit for
 * bit the forward's W records).  Y = T^T dU' stays the gradient of v.
 *   shape       as for gdn_chunk_fwd (io_dtype GDN_BF16, gate_per_channel 0,
 *               gate_grid_log2 0; o_dtype is not used).  qdq_flags are those of
 *               the forward: the state QDQ flags (CHUNK, WRITE) do not change
 *               the gradient under the identity straight-through rule;
 *               GDN_QDQ_W selects the backward of the W-QDQ forward;
 *               GDN_QDQ_INT8 (a decode-step codec) is refused.
 *   q, k        [total_tokens, H, dk] bf16;  beta, g [total_tokens, H] fp32
 *   cu_seqlens, seq_lens   as for gdn_chunk_fwd (seq_lens nullable)
 *   d_o         [total_tokens, H, dv] bf16, the gradient of o (padding rows ignored)
 *   d_final_state  [N, H, dv, dk] fp32 or NULL (zero)
 *   dh          [n_bounds, H, dv, dk] fp32 or NULL: chunk i of sequence n at
 *               b = sum_{m<n} ceil(L_m / 64) + i, the gradient of the state
 *               entering that chunk
 *   d_initial_state [N, H, dv, dk] fp32 or NULL: the gradient of the initial
 *               state (d_final_state for an empty sequence)
 *   d_v         [total_tokens, H, dv] fp32 or NULL: the gradient of v (v enters a
 *               chunk only through U = T V, so it is Y); rows of a segment past
 *               L_n are written as 0, rows after cu_seqlens[N] are not written
 *   workspace   at least gdn_chunk_bwd_workspace_bytes(shape) bytes, 256-byte
 *               aligned, caller-owned, contents ignored on entry; holds the call's
 *               status word on return (gdn_workspace_status; index arrays out of
 *               contract: nothing is written).
 */
gdn_status_t gdn_chunk_bwd_dh(const gdn_shape_t* shape,
                              const void* q, const void* k, const float* beta, const float* g,
                              const int32_t* cu_seqlens, const int32_t* seq_lens,
                              const void* d_o, const float* d_final_state,
                              float* dh, float* d_initial_state, float* d_v,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace bytes gdn_chunk_bwd_dh needs: the status word, the chunk offsets and, per
 * (chunk, head) of the worst-case chunk count, T^T and P^T as full 64 x 64
 * records (16 KiB each), and with GDN_QDQ_W the forward's T, P and W records
 * of gdn_chunk_fwd's workspace.  0 for an invalid shape. */
size_t gdn_chunk_bwd_workspace_bytes(const gdn_shape_t* shape);

/* Static description of a status code. */
const char* gdn_status_string(gdn_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
