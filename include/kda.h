/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention library (libkda.so).
 *
 * The operation.  For one sequence and one head, with a d_k x d_v state S
 * (rows = key channels, columns = value channels), every token t applies
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (read after token t's own write)
 *
 * with alpha_t = exp(log_alpha_t) a per-key-channel retention factor.
 * Source: "Kimi K3" study notes (dimensionstp.github.io/study-concept/kimi_k3),
 * section 3-2 "Module breakdown", item 2) Kimi Delta Attention — the state
 * update and read-out equations; "Kimi K3 架构、训练与系统全景解析"
 * (kimi-k3-analysis), section 4.2.2 — the order: decay each key channel,
 * erase along k, write beta k v^T, then read with q.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, who keeps
 *     them alive until the work enqueued on `stream` has completed.  The
 *     library never allocates device memory.
 *   - Alignment: q, k, v, log_alpha, gate, o, the state tensors and the
 *     workspace of kda_chunk_fwd, the state of kda_decode_step, and the
 *     tensors of kda_decode_replay listed with it, must be 16-byte aligned
 *     (they move as 16-byte vectors); every other pointer needs its
 *     element's alignment.  Violations return KDA_ERR_INVALID_ARG.
 *   - Layouts are dense row-major, token-major: q/k/v/log_alpha/o are
 *     [T_total, H, 128]; beta is [T_total, H]; states are [N, H, 128, 128]
 *     fp32 with S[n][h][i][j], i = key channel (row), j = value channel.
 *   - Only d_k = d_v = 128 is supported (KDA_ERR_UNSUPPORTED otherwise).
 *   - Work is asynchronous on `stream` (0 = the null stream); no host sync.
 *     Argument errors are detected on the host and returned before anything
 *     is enqueued.  A failed launch returns KDA_ERR_HIP.
 *   - Preconditions that the fast path does not check (KDA_DEBUG_CHECKS
 *     below checks them on request): log_alpha in
 *     [-5, 0] (the lower-bounded decay of "Kimi K3 架构…" section 4.2.5,
 *     gate_lower_bound = -5 of section 2.1) for kda_chunk_fwd,
 *     kda_chunk_bwd and kda_decode_replay, or any value <= 0 (-inf included,
 *     NaN not) for kda_decode_step and for kda_chunk_fwd and
 *     kda_decode_replay with unbounded_decay set;
 *     beta in [0, 1]; ||q||, ||k||
 *     about 1 per head when no prologue runs; cu_seqlens non-decreasing from
 *     0 to total_tokens.  Outside them the results are undefined (they may
 *     overflow) but every access stays in bounds.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums have int as their underlying type in C++ as well, so that any
 * int a C caller passes is a valid value for the library to check. */
#ifdef __cplusplus
#define KDA_ENUM_BASE : int
#else
#define KDA_ENUM_BASE
#endif

typedef enum KDA_ENUM_BASE {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* NULL where required, bad sizes, illegal overlap */
  KDA_ERR_UNSUPPORTED = 2, /* d_k or d_v other than 128, unknown dtype       */
  KDA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required        */
  KDA_ERR_HIP = 4,         /* a HIP launch or runtime call failed            */
  KDA_ERR_PRECONDITION = 5, /* an input outside the preconditions (only with KDA_DEBUG_CHECKS) */
  KDA_ERR_SCRATCH = 6       /* kda_chunk_fwd_noalloc: the sizes need more than its scratch array */
} kda_status;

/*
 * Precondition checks.  With the environment variable KDA_DEBUG_CHECKS set to
 * anything but "" or "0" (read at every call), each compute entry point first
 * checks the preconditions listed above on the device, waits for the result
 * (a host synchronisation of `stream`, so not under graph capture) and, when
 * one fails, returns KDA_ERR_PRECONDITION without launching its kernels.
 * kda_last_precondition_flags() then gives the failed checks.  The checks
 * of all calls on a device share one device word, so checked calls must not
 * run concurrently on different streams.
 */
enum {
  KDA_CHECK_LOG_ALPHA = 1,  /* a log_alpha value outside the call's range (above), or NaN */
  KDA_CHECK_BETA = 2,       /* a beta value outside [0, 1] or not finite               */
  KDA_CHECK_Q_NORM = 4,     /* a q row (no prologue on q) whose norm is not 1 +- 0.02   */
  KDA_CHECK_K_NORM = 8,     /* a k row (no prologue on k) whose norm is not 1 +- 0.02   */
  KDA_CHECK_CU_SEQLENS = 16 /* cu_seqlens not non-decreasing from 0 to total_tokens    */
};

typedef enum KDA_ENUM_BASE {
  KDA_DTYPE_F32 = 0,  /* q, k, v, gate and o are float                      */
  KDA_DTYPE_BF16 = 1  /* q, k, v, gate and o are bfloat16 (round-to-nearest-even on output) */
} kda_dtype;

/*
 * Optional fused prologue and epilogue ("Kimi K3 架构…" section 4.2.3:
 * ShortConv with kernel size 4, Swish, L2Norm on q and k; section 4.2.6:
 * head-wise RMSNorm of the recurrent output, then a full-rank sigmoid output
 * gate).  Pass NULL for plain KDA.  Each field may be NULL independently.
 *
 *   conv_q_w / conv_k_w  [H*128, 4] fp32 depthwise causal conv weights.  When
 *       given, the q (resp. k) read from memory is the raw projection and the
 *       recurrence uses  x'_t[c] = L2( SiLU( sum_{m=0..3} w[c][m] x_{t-3+m}[c] ) )
 *       with channel c = h*128 + j, zero history before each sequence start,
 *       and L2(x) = x / sqrt(sum_j x_j^2 + l2_eps) over the 128 channels of a head.
 *   gate  [T_total, H, 128] logits in the I/O dtype.  When given, the stored
 *       output is  y_t = o_t / sqrt(mean_j o_t[j]^2 + rms_eps) * norm_w * sigmoid(gate_t).
 *   norm_w  [128] fp32 RMSNorm weight; NULL means all ones.  Used only with gate.
 *   unbounded_decay  0: log_alpha in [-5, 0] (the K3 bound), where every
 *       16-token tile of the chunked prefill runs as dense matrix-core
 *       products.  Nonzero: kda_chunk_fwd accepts any log_alpha <= 0, the
 *       unbounded negative-softplus decay of Kimi Linear ("Kimi K3 架构…"
 *       section 4.2.5); the diagonal 16-token tiles are then formed position
 *       pair by position pair (e^{g_i - g_j} as a running product of the
 *       alphas between the two tokens, never above 1), which is slower.
 *       kda_decode_replay takes the same flag: its block of cached tokens then
 *       forms every pair's decay product from the log_alpha sums between the
 *       two tokens instead of dividing by the cumulative decay.
 *       kda_decode_step needs no flag (it accepts any log_alpha <= 0);
 *       kda_chunk_bwd does not take it.
 *   segment_tokens  scheduling of long sequences when there are too few
 *       (sequence, head) pairs to occupy the GPU: 0 lets the library decide
 *       (it segments only when the sequential schedule would leave more than
 *       two thirds of the compute units idle); a positive multiple of 64
 *       forces the segmented form with segments of that many tokens (any
 *       other positive value is KDA_ERR_INVALID_ARG); a negative value
 *       disables it.  The segmented form needs about
 *       (T_total / segment_tokens + N) * H * 128 KiB of workspace on top of
 *       the factor store (see kda_chunk_fwd_workspace_bytes).  It
 *       ("Kimi K3 架构…" section 7.1, in-device context parallelism) runs every
 *       segment from a zero state and, with V = 0, from the identity, which
 *       gives the affine pair (M_j, B_j) with S_out = M_j S_in + B_j; a scan
 *       composes the pairs into each segment's incoming state; a last pass
 *       writes the outputs.  Results agree with the sequential form up to
 *       rounding.
 *   factor_budget_mib  cap, in MiB, on the factor store of one window of
 *       kda_chunk_fwd (the bulk of its workspace): 0 means the largest, 16384;
 *       values above 16384 are taken as 16384; negative values are
 *       KDA_ERR_INVALID_ARG.  Inputs whose factor blocks exceed the cap run in
 *       several windows, one after another on the stream, with the same
 *       results up to rounding.  The workspace query and the call must be
 *       given the same value.  kda_decode_replay ignores it.
 */
typedef struct {
  const float* conv_q_w;
  const float* conv_k_w;
  const void* gate;
  const float* norm_w;
  float l2_eps;
  float rms_eps;
  int segment_tokens;
  int unbounded_decay;
  int factor_budget_mib;
} kda_fused_opts;

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes and options
 * (host-side computation; it reads the current device's compute-unit count,
 * which the segmented form depends on).  Returns 0 for invalid sizes.
 * Most of it is the factor store: a 70.5 KiB block per (64-token chunk, head)
 * for bf16 I/O, 68.5 KiB per (32-token chunk, head) for fp32.  It is capped at
 * 16 GiB, or at opts->factor_budget_mib; longer inputs run in several windows.
 * The query depends on no environment variable: the same sizes and options
 * give the same value on the same device.
 */
size_t kda_chunk_fwd_workspace_bytes(int num_seqs, int64_t total_tokens, int num_heads, int d_k,
                                     int d_v, kda_dtype dtype, const kda_fused_opts* opts);

/*
 * Chunkwise-parallel prefill over a packed batch of sequences ("Kimi K3 架构…"
 * section 4.2.4 chunkwise parallel form; section 7.1 FlashKDA and in-device
 * sequence splitting).  Sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *
 *   q, k, v        [T_total, H, 128] dtype (raw projections for q/k when the
 *                  prologue convolution is enabled)
 *   log_alpha      [T_total, H, 128] fp32, natural-log per-key-channel decay
 *   beta           [T_total, H] fp32 write strength
 *   initial_state  [N, H, 128, 128] fp32, read only, or NULL for zeros.  It may
 *                  be exactly the same pointer as final_state (in-place
 *                  continuation); any other overlap is KDA_ERR_INVALID_ARG.
 *   cu_seqlens     device int32 [N+1] or NULL (then N must be 1 and the one
 *                  sequence spans all T_total tokens).  Zero-length sequences
 *                  are allowed; their final state equals the initial state.
 *   opts           NULL or the fused prologue/epilogue options above.
 *   num_heads      H, 1 .. 65535 (one chunk's rows of a [T_total, H, 128]
 *                  tensor are addressed with 32-bit offsets); else
 *                  KDA_ERR_INVALID_ARG.  The same bound holds for
 *                  kda_chunk_fwd_noalloc and kda_chunk_bwd.
 *   o              [T_total, H, 128] dtype output; must not overlap any input.
 *   final_state    [N, H, 128, 128] fp32 output or NULL (not written).
 *   workspace      device scratch of at least kda_chunk_fwd_workspace_bytes()
 *                  bytes for the same sizes and options on the same device
 *                  (may be NULL when that is 0).  Contents on entry are
 *                  ignored; it must not be in use by other work on the GPU.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                         int num_seqs, int64_t total_tokens, int num_heads, int d_k, int d_v,
                         kda_dtype dtype, const kda_fused_opts* opts, void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of the device scratch array behind kda_chunk_fwd_noalloc: one copy on
 * every GPU the library runs on, held until the process ends.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * kda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, semantics and results are those of kda_chunk_fwd without the
 * workspace; the library's own scratch array of KDA_NOALLOC_SCRATCH_BYTES on
 * the current device takes its place.  The factor store is cut into as many
 * windows as it takes to fit that array (opts->factor_budget_mib, when
 * positive, caps each window further), so large inputs run in more, smaller
 * windows than kda_chunk_fwd would use.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's copy of the array.
 *
 * Errors: those of kda_chunk_fwd (never KDA_ERR_WORKSPACE), plus
 * KDA_ERR_SCRATCH, returned before anything is enqueued, when even the
 * smallest windows do not fit: the floor is about (N + 2) * H * 70.5 KiB of
 * factor blocks (bf16; 68.5 KiB for fp32) plus N * H * 64 KiB for the state
 * carried between windows, so for example N = 1 fits up to H of about 500 and
 * H = 96 up to N of about 9.
 *
 * Every call on one GPU uses that GPU's one array and leaves its contents
 * behind.  Nothing in it needs to start at zero (each byte a call reads was
 * written earlier in the same call), but calls that overlap in time on one
 * GPU (on different streams, or from different threads) race on it and give
 * wrong results: serialise them.
 */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                                 int num_seqs, int64_t total_tokens, int num_heads, int d_k, int d_v,
                                 kda_dtype dtype, const kda_fused_opts* opts, void* o, float* final_state,
                                 hipStream_t stream);

/*
 * Bytes of device workspace kda_chunk_bwd needs for these sizes (host-side
 * computation; 0 for invalid sizes).  Every chunk of the input is held at
 * once: per (64-token chunk, head) for bf16 I/O about 70.5 KiB of forward
 * factors, 81 KiB for the reverse carry, and 2 x 32 KiB + 2 x 16 KiB of
 * states, gradients and intermediates held in the I/O dtype (about 247.5 KiB,
 * i.e. 3.9 KiB per token and head); fp32 I/O uses 32-token chunks (about
 * 342 KiB per chunk, 10.7 KiB per token and head).
 */
size_t kda_chunk_bwd_workspace_bytes(int num_seqs, int64_t total_tokens, int num_heads, int d_k, int d_v,
                                     kda_dtype dtype);

/*
 * Backward pass of kda_chunk_fwd without the fused prologue and epilogue
 * (training; "Kimi K3 架构…" section 7.1: the FlashKDA kernel serves training
 * as well as prefill).  For the loss
 *
 *     L = sum_t <d_o_t, o_t> + <d_final_state, S_T>       (per sequence and head)
 *
 * it writes the gradients of L with respect to q, k, v, log_alpha, beta and
 * initial_state.  The forward states are recomputed internally (the call
 * needs only the forward's inputs), so it does not depend on a prior
 * kda_chunk_fwd call.
 *
 *   q, k, v, log_alpha, beta, initial_state, cu_seqlens
 *                  as for kda_chunk_fwd (log_alpha in [-5, 0]: the unbounded
 *                  decay is not supported here)
 *   d_o            [T_total, H, 128] dtype: gradient of L with respect to o
 *   d_final_state  [N, H, 128, 128] fp32 or NULL (zero)
 *   dq, dk, dv     [T_total, H, 128] dtype outputs
 *   dlog_alpha     [T_total, H, 128] fp32 output
 *   dbeta          [T_total, H] fp32 output
 *   d_initial_state [N, H, 128, 128] fp32 output, or NULL (not written); for
 *                  a zero-length sequence it equals d_final_state
 *   workspace      at least kda_chunk_bwd_workspace_bytes() bytes (contents
 *                  on entry ignored)
 * No output may overlap an input, another output or the workspace
 * (KDA_ERR_INVALID_ARG).  Alignment as for kda_chunk_fwd; d_o, the gradients
 * and the state gradients need 16 bytes, dbeta 4.  Asynchronous on `stream`
 * like every other call; the recomputed forward uses the same kernels as
 * kda_chunk_fwd, so its rounding is that of the forward.  Every sum runs in a
 * fixed order (no atomics), so repeated calls give the same bits.
 */
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                         const float* initial_state, const int32_t* cu_seqlens, const void* d_o,
                         const float* d_final_state, int num_seqs, int64_t total_tokens, int num_heads, int d_k,
                         int d_v, kda_dtype dtype, void* dq, void* dk, void* dv, float* dlog_alpha, float* dbeta,
                         float* d_initial_state, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward pass for training: kda_chunk_fwd without the fused options and with
 * the bounded decay (its o and final_state, from the same kernels), which
 * also leaves in bwd_workspace everything kda_chunk_bwd would recompute from
 * the inputs: the factor blocks of every chunk and each chunk's incoming
 * state and U = U' - W S ("Kimi K3 架构…" section 7.1: the FlashKDA kernel
 * serves training as well as prefill).  kda_chunk_bwd_saved then starts from
 * them.  One walk over the chunks writes the outputs and those states
 * together.
 *
 *   q, k, v, log_alpha, beta, initial_state, cu_seqlens, num_seqs,
 *   total_tokens, num_heads, d_k, d_v, dtype
 *                  as for kda_chunk_bwd
 *   o              [T_total, H, 128] dtype output
 *   final_state    [N, H, 128, 128] fp32 output or NULL; may be exactly
 *                  initial_state (in-place continuation)
 *   bwd_workspace  at least kda_chunk_bwd_workspace_bytes() bytes; owned by
 *                  the caller, who keeps it unchanged until the matching
 *                  kda_chunk_bwd_saved call
 * Any other overlap of o, final_state and bwd_workspace with an input or with
 * each other is KDA_ERR_INVALID_ARG; alignment as for kda_chunk_bwd.  With
 * KDA_DEBUG_CHECKS the inputs are checked as for kda_chunk_bwd.
 */
kda_status kda_chunk_fwd_save(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                              int64_t total_tokens, int num_heads, int d_k, int d_v, kda_dtype dtype, void* o,
                              float* final_state, void* bwd_workspace, size_t bwd_workspace_bytes,
                              hipStream_t stream);

/*
 * kda_chunk_bwd from the residuals kda_chunk_fwd_save left in `workspace`:
 * the same gradients, bit for bit, without recomputing the forward's factor
 * blocks and chunk states.  The arguments are those of kda_chunk_bwd, with
 * the same checks; q, k, v, log_alpha, beta, cu_seqlens and the sizes must be
 * the ones the forward ran on, unchanged since.  The call cannot tell: other
 * inputs give meaningless gradients, but the chunk tables are rebuilt from
 * this call's cu_seqlens, so every access stays inside the buffers.
 * initial_state is not read (the saved chunk states hold it), so an in-place
 * forward that has overwritten it is fine.
 */
kda_status kda_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                               const void* d_o, const float* d_final_state, int num_seqs, int64_t total_tokens,
                               int num_heads, int d_k, int d_v, kda_dtype dtype, void* dq, void* dk, void* dv,
                               float* dlog_alpha, float* dbeta, float* d_initial_state, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step for N independent sequences: each (n, h) state advances by
 * one token in place ("Kimi K3 架构…" section 4.2.7: decoding keeps one
 * fixed-size d_k x d_v state per head and advances it in place).
 *
 *   state       [N, H, 128, 128] fp32, read and overwritten in place
 *   q, k, v     [N, H, 128] dtype;  log_alpha [N, H, 128] fp32;  beta [N, H] fp32
 *   o           [N, H, 128] dtype output (o_t read after the token's write);
 *               must not overlap any input.
 */
kda_status kda_decode_step(float* state, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, int num_seqs, int num_heads,
                           int d_k, int d_v, kda_dtype dtype, void* o, hipStream_t stream);

/*
 * Multi-token decode from cached per-token inputs: the replay step of
 * speculative decoding ("Kimi K3 架构…" section 7.4, KDA state replay under
 * speculative decoding: the per-token inputs of the draft tokens are kept
 * instead of one state per draft position; after verification the accepted
 * prefix is replayed from the verified state on chip, with the short
 * convolution, the norms and the output gate in the same kernel, and only the
 * final state is written back).  For each sequence n and head h, runs the
 * recurrence above over tokens 0 .. nt-1 of the sequence's max_tokens cached
 * tokens, starting from state_in, where nt = num_tokens[n] clamped to
 * [0, max_tokens] (all of them when num_tokens is NULL).  The state is read
 * once and written at most once, so its HBM traffic per token falls with nt.
 *
 * Typical use: a verification pass over all draft tokens with state_out NULL
 * (outputs only, nothing committed), then a commit pass with num_tokens =
 * accepted + 1 (the accepted drafts and the bonus token) and state_out ==
 * state_in, o NULL.
 *
 *   state_in      [N, H, 128, 128] fp32, read only, or NULL for zeros.
 *   state_out     [N, H, 128, 128] fp32 state after the nt tokens, or NULL
 *                 (not written).  May be exactly state_in (in place); any
 *                 other overlap with a buffer is KDA_ERR_INVALID_ARG.
 *   q, k, v       [N, max_tokens, H, 128] dtype (raw q / k rows when their
 *                 convolution runs); log_alpha [N, max_tokens, H, 128] fp32;
 *                 beta [N, max_tokens, H] fp32.  Rows of tokens past nt are
 *                 not read.
 *   num_tokens    device int32 [N] or NULL.
 *   max_tokens    1 .. 16 (larger values are KDA_ERR_UNSUPPORTED).
 *   opts          NULL or the fused options of kda_chunk_fwd: conv_q_w /
 *                 conv_k_w, gate ([N, max_tokens, H, 128] dtype logits),
 *                 norm_w, l2_eps, rms_eps, unbounded_decay (any log_alpha <= 0,
 *                 -inf included); segment_tokens and factor_budget_mib are
 *                 ignored.
 *   conv_q_state, conv_k_state
 *                 [N, 3, H, 128] dtype: the raw q (k) rows of the three
 *                 positions before token 0, oldest first (zeros at a
 *                 sequence start).  Required when the matching convolution
 *                 weight is given, ignored otherwise.  They are read in every
 *                 call and, only when state_out is given, overwritten with
 *                 the raw rows of the three positions before token nt (the
 *                 history the next call continues from).
 *   o             [N, max_tokens, H, 128] dtype outputs of tokens 0 .. nt-1
 *                 (rows past nt are not written), or NULL.  Must not overlap
 *                 any other buffer.
 * Every pointer needs 16-byte alignment except beta, num_tokens, the
 * convolution weights and norm_w (4 bytes).  Calls whose buffers overlap
 * must not run concurrently.
 */
kda_status kda_decode_replay(const float* state_in, float* state_out, const void* q, const void* k,
                             const void* v, const float* log_alpha, const float* beta,
                             const int32_t* num_tokens, int num_seqs, int max_tokens, int num_heads,
                             int d_k, int d_v, kda_dtype dtype, const kda_fused_opts* opts,
                             void* conv_q_state, void* conv_k_state, void* o, hipStream_t stream);

/* KDA_CHECK_* bits of the last checked call on the calling thread (0 when it passed). */
uint32_t kda_last_precondition_flags(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_string(kda_status s);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
