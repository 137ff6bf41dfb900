/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * The operator (Kimi K3 technical-report digest, discuss.pytorch.kr, section
 * "Kimi Delta Attention", the per-head update equation):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * per head, with q_t, k_t in R^dk, v_t in R^dv, state S_t in R^{dk x dv},
 * per-key-channel retention alpha_t = exp(log_alpha_t) in (0,1]^dk and scalar
 * write strength beta_t in [0,1].  The state is fp32 and lives in a fixed
 * dk x dv block per head (128 x 128 in the K3 layer).
 *
 * Input contract (not clamped in-kernel):
 *   * -5 <= log_alpha <= 0.  The bounded-decay section of the same page fixes
 *     the lower bound g_min = -5, which keeps the 16-token cumulative decay in
 *     [-80, 0] so the chunked factors e^{+-G} stay inside fp32/bf16 range.
 *     Values below -5 are out of contract (results may be Inf/NaN).
 *   * beta in [0, 1].  k is expected L2-normalised by the caller (the page
 *     normalises q and k before the recurrence); the operator applies no
 *     1/sqrt(dk) scale to q.
 *
 * Layouts (row-major, contiguous, N = total_tokens = sum of sequence lengths):
 *   q, k, log_alpha : [N, H, dk]      v : [N, H, dv]      beta : [N, H]
 *   all five share one dtype: KDA_BF16 (bfloat16) or KDA_F32 (float).
 *   cu_seqlens  : int32 [nseq + 1] in DEVICE memory, cu[0] = 0, non-decreasing,
 *                 cu[nseq] = N (sequence s is tokens [cu[s], cu[s+1]); empty
 *                 sequences are allowed).
 *   init_state  : fp32 [nseq, H, dk, dv] or NULL (zero initial state).
 *   o           : fp32 [N, H, dv].
 *   final_state : fp32 [nseq, H, dk, dv] or NULL (not written).  It may alias
 *                 init_state: each (sequence, head) block is read in full
 *                 before it is written.
 *   Decode: q, k, log_alpha [B, H, dk], v [B, H, dv], beta [B, H], state fp32
 *   [B, H, dk, dv] updated in place (the in-place per-step state update that
 *   the serving section names as the decode bottleneck), o fp32 [B, H, dv].
 *   Decode window: as decode with a window axis T after B (see
 *   kda_decode_window).
 *
 * Supported shapes: dk, dv in {16, 32, 64, 128} (any combination); H >= 1;
 * nseq >= 1; total_tokens >= 0 (< 2^31).  Chunk length is fixed at 16 tokens.
 * Launch limits of the prefill-family calls (a dispatch holds fewer than 2^32
 * work-items, and 16-token row extents are kept in 32 bits): nseq * H < 2^20
 * (sequence-head chains), H * max(dk, dv) < 2^24, and for KDA_F32 inputs
 * floor(N/16) + nseq < 2^26 chunk slots; the backward also needs
 * (floor(N/16) + nseq) * H < 2^24 and the context-parallel call
 * nseq * segments * H * dk * max(dk, dv) < 2^31.  Larger shapes return
 * KDA_ERR_SHAPE before any launch.
 *
 * Ownership and synchronisation: every buffer is allocated by the caller; the
 * library never allocates, frees or synchronises.  Pointers are device
 * pointers unless stated otherwise.  Work is enqueued on `stream` (a
 * hipStream_t; NULL = the default stream) and the call returns at once.
 * A call enqueues kernel launches only (no memset, copy or event), so it can
 * be recorded into a HIP graph by stream capture and replayed.
 * Inputs are read-only; o / final_state must not alias the inputs (except the
 * final_state == init_state case above).  Alignment: fp32 buffers (state,
 * o, init/final state, workspace) 16 bytes; q, k, v, log_alpha four elements
 * (8 bytes for bf16, 16 for fp32); beta one element.  With total_tokens == 0
 * the token-indexed pointers may be NULL.
 *
 * Errors: argument errors are detected on the host before any launch and
 * returned as a status; nothing is launched then.  A failed launch returns
 * KDA_ERR_HIP and kda_last_hip_error() gives the hipError_t (per thread).
 * Faults inside a kernel surface at the caller's next synchronisation.  The
 * library does not print, throw or abort.  Results are bitwise reproducible
 * for a given shape on a given device (no atomics, fixed reduction order).
 * Calls are reentrant; concurrent calls on different streams are safe as long
 * as their output buffers (and workspaces) are distinct.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,         /* a required pointer is NULL */
    KDA_ERR_ALIGN = 2,        /* a pointer violates the alignment rules above */
    KDA_ERR_SHAPE = 3,        /* nseq < 1, H < 1, B < 1, total_tokens out of range, or a launch limit exceeded */
    KDA_ERR_UNSUPPORTED = 4,  /* dk / dv not in {16,32,64,128}, or unknown dtype */
    KDA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the call needs */
    KDA_ERR_HIP = 6,          /* a kernel launch failed; see kda_last_hip_error() */
    KDA_ERR_TOO_LARGE = 7     /* kda_prefill_noalloc: workspace above KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,              /* q, k, v, log_alpha, beta are float */
    KDA_BF16 = 1              /* q, k, v, log_alpha, beta are bfloat16 */
} kda_dtype;

#define KDA_CHUNK 16
#define KDA_GATE_LOWER_BOUND (-5.0f)

/* Bytes of device workspace kda_chunk_local / kda_inter_chunk need (and
 * kda_prefill, where it runs those two phases): per chunk slot and head, the
 * 16x16 matrices T' = (I + A_kk)^-1 diag(beta) and A_qk, each as a 1 KiB
 * matrix-core operand fragment (a hi/lo bfloat16 pair per element for
 * KDA_BF16, fp32 for KDA_F32), for floor(N/16) + nseq chunk slots.  The
 * layout is private to the library.  Returns 0 for invalid arguments. */
size_t kda_chunk_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H,
                                 int32_t dk, int32_t dv, kda_dtype dt);

/* Bytes of device workspace kda_prefill needs for these arguments.  KDA_BF16
 * inputs with dk = dv = 128 (the K3 layer's heads) and at least 256
 * (sequence, head) chains run a single-pass kernel that keeps the chunk-local
 * operands on chip: 0 bytes, and the workspace may be NULL.  KDA_BF16 inputs
 * with dk >= 32, at most 64 chains and at least 16,384 tokens per sequence on
 * average run with intra-device context parallelism in R = clamp(128 / chains,
 * 2, 16) segments (kda_prefill_cp): kda_prefill_cp_workspace_bytes(..., R).
 * Every other shape runs the two phases and needs kda_chunk_workspace_bytes(...).
 * 0 is also returned for invalid arguments; kda_prefill then reports which
 * argument is wrong. */
size_t kda_prefill_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H,
                                   int32_t dk, int32_t dv, kda_dtype dt);

/* Chunkwise prefill over packed variable-length sequences.  Computes o for
 * every token and, if final_state != NULL, the state after each sequence's
 * last token.  (Chunked form: same page, "chunk-parallel form" paragraph and
 * equation O_[t] = (Gamma (.) Q_[t]) S_[t] + A_[t] V~_[t].)
 * KDA_BF16 with dk = dv = 128 and nseq * H >= 256: one kernel per call, in which producer waves
 * form the chunk-local operands (cumulative decay, the inverse of I + A_kk,
 * A_qk) two chunks ahead of the waves that carry the state, so the inputs are
 * read from HBM once and nothing goes through a workspace (the overlap of the
 * token-parallel and the serial phases that the page's systems section
 * describes).  Few long chains (see kda_prefill_workspace_bytes): kda_prefill_cp,
 * which spreads each sequence over more compute units (same page, intra-device
 * context parallelism).  Other shapes: the chunk-local phase (kda_chunk_local)
 * then the inter-chunk phase (kda_inter_chunk), with the workspace between them. */
kda_status kda_prefill(const void *q, const void *k, const void *v,
                       const void *log_alpha, const void *beta,
                       const float *init_state, const int32_t *cu_seqlens,
                       int32_t nseq, int64_t total_tokens, int32_t H,
                       int32_t dk, int32_t dv, kda_dtype dt,
                       float *o, float *final_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Phase 1 of kda_prefill, embarrassingly parallel over (chunk, head): the
 * cumulative log-decay of each 16-token chunk, the strictly lower triangular
 * beta-weighted decayed key block A_kk = diag(beta) tril_-1(K+ K-^T), its
 * unit-lower-triangular inverse T = (I + A_kk)^-1 (stored as T diag(beta)),
 * and the decayed query-key block A_qk = tril(Q+ K-^T).  Writes `workspace`.
 * (Bounded-decay section: the -5 floor keeps e^{+-G} in range so the
 * diagonal tiles are dense matrix products.) */
kda_status kda_chunk_local(const void *q, const void *k, const void *log_alpha,
                           const void *beta, const int32_t *cu_seqlens,
                           int32_t nseq, int64_t total_tokens, int32_t H,
                           int32_t dk, kda_dtype dt,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Phase 2 of kda_prefill: the sequential state propagation over the chunks
 * of each sequence, per (sequence, head, 16-column slice of dv), with the
 * fp32 state held on chip.  Reads the workspace written by kda_chunk_local
 * for the same inputs.  (KDA systems section: the recurrence across chunks
 * is the serial, head-parallel phase.) */
kda_status kda_inter_chunk(const void *q, const void *k, const void *v,
                           const void *log_alpha, const float *init_state,
                           const int32_t *cu_seqlens, int32_t nseq,
                           int64_t total_tokens, int32_t H, int32_t dk,
                           int32_t dv, kda_dtype dt, const void *workspace,
                           size_t workspace_bytes, float *o,
                           float *final_state, void *stream);

/* The two prefill kernels with an explicit workgroup shape, for tuning and for
 * tests that must reach every shape (kda_prefill and kda_inter_chunk choose
 * the shape from the number of (sequence, head) chains).  Same arguments,
 * results and errors as kda_prefill / kda_inter_chunk.
 *   kda_prefill_single_pass: the single-pass kernel (KDA_BF16, dk = dv = 128
 *     only) with `consumers` state waves per workgroup, each holding `slices`
 *     16-column slices of dv: (2, 1), (4, 1) or (4, 2); (0, 0) chooses.
 *   kda_inter_chunk_shaped: the warp-specialised inter-chunk kernel (KDA_BF16,
 *     dk >= 32) with `consumers` 16-column state waves and `producers` operand
 *     waves per workgroup: (2, 4) or (4, 4) for dk = dv = 128, (min(dv/16, 4) or
 *     min(dv/16, 2), min(dk/16, 4)) otherwise; (0, 0) chooses.
 * A shape that is not built returns KDA_ERR_UNSUPPORTED before any launch. */
kda_status kda_prefill_single_pass(const void *q, const void *k, const void *v,
                                   const void *log_alpha, const void *beta,
                                   const float *init_state, const int32_t *cu_seqlens,
                                   int32_t nseq, int64_t total_tokens, int32_t H,
                                   int32_t dk, int32_t dv, kda_dtype dt,
                                   int32_t consumers, int32_t slices,
                                   float *o, float *final_state, void *stream);

kda_status kda_inter_chunk_shaped(const void *q, const void *k, const void *v,
                                  const void *log_alpha, const float *init_state,
                                  const int32_t *cu_seqlens, int32_t nseq,
                                  int64_t total_tokens, int32_t H, int32_t dk,
                                  int32_t dv, kda_dtype dt, const void *workspace,
                                  size_t workspace_bytes, int32_t consumers,
                                  int32_t producers, float *o, float *final_state,
                                  void *stream);

/* kda_prefill with intra-device context parallelism: every sequence is split into
 * `segments` chunk-aligned pieces (segment r covers chunks [nc r / R, nc (r+1) / R)
 * of a sequence of nc chunks) that run as independent chains, and the exact state
 * entering each piece is recovered by a scan over the pieces' affine state maps
 * S_out = M S_in + S~ (Kimi K3 report digest, context parallelism of KDA: the same
 * algebra as across devices, here between the compute units of one GPU).  Three
 * recurrence passes over the pieces (S~ from zero states; M from the identity with
 * v = 0; the outputs from the exact states) and one chunk-local pass.  A piece whose
 * transition is provably negligible -- the bound ||M||_2 <= prod_t max_i alpha_t,i
 * max(1, |1 - beta_t ||k_t||^2|), evaluated on the device from its inputs, below 2^-30 --
 * skips the M pass and enters the scan with M = 0.  Same inputs, outputs and precision
 * as kda_prefill; segments = 1 reduces to it (at up to three times the recurrence work).
 *   segments: 1 .. 64.
 *   workspace: kda_prefill_cp_workspace_bytes(...) bytes, 16-byte aligned (chunk-local
 *   operands of the pieces; per piece and head S~, S_in (dk x dv) and M (dk x dk), fp32,
 *   and a flag). */
size_t kda_prefill_cp_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H,
                                      int32_t dk, int32_t dv, kda_dtype dt,
                                      int32_t segments);

kda_status kda_prefill_cp(const void *q, const void *k, const void *v,
                          const void *log_alpha, const void *beta,
                          const float *init_state, const int32_t *cu_seqlens,
                          int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk,
                          int32_t dv, kda_dtype dt, int32_t segments, float *o,
                          float *final_state, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Backward pass of kda_prefill (for training): the gradients of a loss L with
 * dL/do = d_o and dL/d(final_state) = d_final (NULL = zero) with respect to q,
 * k, v, log_alpha, beta and the initial state, for the same inputs as the
 * forward call.  The recurrence (same page, update equation) is differentiated
 * in chunk form: a forward sweep recomputes the state at every chunk start, a
 * reverse sweep carries the state adjoint A (A <- Diag(e^{G_n}) A + Q+^T dO -
 * K+^T dV per chunk), and a parallel pass forms dq, dk, dbeta and the log-decay
 * gradient per chunk.  The log-decay gradient is the reverse cumulative sum over
 * each sequence of q (.) dq - k (.) (the two parts of dk's sum), started from
 * rowsum(d_final (.) final_state); each chunk sums its own tokens and reads the
 * part from all later tokens off its checkpoints, rowsum(A (.) S) with S the
 * state after the chunk, so no sum runs over a whole sequence.  fp32 throughout.
 *   d_o: fp32 [N, H, dv];  d_final, d_init: fp32 [nseq, H, dk, dv] or NULL;
 *   d_q, d_k, d_log_alpha: fp32 [N, H, dk];  d_v: fp32 [N, H, dv];
 *   d_beta: fp32 [N, H];  all written in full (d_init if not NULL).
 *   workspace: kda_prefill_backward_workspace_bytes(...) bytes, 16-byte aligned
 *   (per chunk slot and head: the state and its adjoint, dk x dv fp32 each,
 *   two 16 x dv blocks and four 16 x 16 chunk matrices). */
size_t kda_prefill_backward_workspace_bytes(int64_t total_tokens, int32_t nseq,
                                            int32_t H, int32_t dk, int32_t dv,
                                            kda_dtype dt);

kda_status kda_prefill_backward(const void *q, const void *k, const void *v,
                                const void *log_alpha, const void *beta,
                                const float *init_state,
                                const int32_t *cu_seqlens, int32_t nseq,
                                int64_t total_tokens, int32_t H, int32_t dk,
                                int32_t dv, kda_dtype dt, const float *d_o,
                                const float *d_final, float *d_q, float *d_k,
                                float *d_v, float *d_log_alpha, float *d_beta,
                                float *d_init, void *workspace,
                                size_t workspace_bytes, void *stream);

/* kda_prefill_backward for one long sequence with bounded memory: the sequence
 * is cut into slabs of slab_tokens tokens (a multiple of 16) and only one slab's
 * workspace is held at a time.  A first pass carries the fp32 state through the
 * slabs with the backward's own forward sweep and keeps the state at each slab
 * boundary; the slabs are then differentiated in reverse, each from its boundary
 * state, with the adjoint of the state it hands on -- the adjoint of the next
 * slab's initial state -- as its d_final (the chain rule across the cut is exact,
 * so the result is the unsliced backward's up to fp32 rounding).  The extra cost
 * is one forward sweep over the sequence.  (FlashKDA serves training; the K3
 * report digest's chunkwise-kernel paragraph.)
 *   Arguments as kda_prefill_backward with nseq = 1 and no cu_seqlens;
 *   slab_tokens >= 16, a multiple of 16;
 *   workspace: kda_prefill_backward_slabbed_workspace_bytes(...) bytes, 16-byte
 *   aligned: one slab's backward workspace plus one state per slab boundary
 *   and two (dk x dv fp32 per head each). */
size_t kda_prefill_backward_slabbed_workspace_bytes(int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                                                    kda_dtype dt, int64_t slab_tokens);
kda_status kda_prefill_backward_slabbed(const void *q, const void *k, const void *v, const void *log_alpha,
                                        const void *beta, const float *init_state, int64_t total_tokens, int32_t H,
                                        int32_t dk, int32_t dv, kda_dtype dt, const float *d_o, const float *d_final,
                                        float *d_q, float *d_k, float *d_v, float *d_log_alpha, float *d_beta,
                                        float *d_init, int64_t slab_tokens, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* One recurrent decode step for B x H heads: the state is read once and
 * written once, in place.  (Per-token update equation; serving section:
 * decode is bound by the in-place state update.) */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta,
                           float *state, float *o, int32_t B, int32_t H,
                           int32_t dk, int32_t dv, kda_dtype dt, void *stream);

/* A window of T consecutive tokens per sequence in one call, for speculative
 * decoding: the T draft tokens of each sequence are verified in one pass and
 * the state is advanced only over the tokens the verifier accepted.  (Serving
 * section of the same page: the decode step is bound by the in-place state
 * update, and a speculative-decoding scheme has to replay the recurrence over
 * the accepted tokens; the plain reading taken here is that the accepted
 * tokens are a prefix of the window.)
 *
 * Per (sequence b, head h) this equals T calls of kda_decode_step on the
 * tokens of the window in order, except that the state is read once and
 * written at most once: o receives the output of every token of the window
 * (computed from the running state, as if every draft were accepted so far),
 * while state receives the state after the first acc = clamp(accept[b], 0, T)
 * tokens.  acc == 0 leaves the state untouched (not even rewritten).
 *
 *   q, k, log_alpha : [B, T, H, dk]   v : [B, T, H, dv]   beta : [B, T, H]
 *                     (one dtype, KDA_BF16 or KDA_F32; alignment as above)
 *   state           : fp32 [B, H, dk, dv], device, updated in place.
 *   o               : fp32 [B, T, H, dv], or NULL (outputs not written).
 *   accept          : int32 [B] in DEVICE memory (4-byte aligned), or NULL
 *                     (all T tokens accepted).  Values outside [0, T] are
 *                     clamped.
 *   B, H >= 1, T >= 1, B * T * H < 2^31.
 *
 * State traffic is that of one decode step per window, so a T-token window
 * costs far less than T single steps while T stays small; long windows
 * (hundreds of tokens) belong to kda_prefill instead.
 *
 * Evaluation: token by token on the vector ALUs (the arithmetic of
 * kda_decode_step), except for bf16 inputs with dk = dv = 128 and 6 <= T <= 16,
 * where the window is one 16-token chunk of the prefill's chunked form on the
 * matrix cores (same report section as kda_prefill; split-bf16 products, fp32
 * accumulation), whose arithmetic per state element does not grow with T.  The
 * two forms agree to the prefill's precision, not bit for bit; in either form
 * the committed state depends only on the accepted prefix.  Errors as for
 * kda_decode_step. */
kda_status kda_decode_window(const void *q, const void *k, const void *v,
                             const void *log_alpha, const void *beta,
                             float *state, float *o, const int32_t *accept,
                             int32_t B, int32_t T, int32_t H, int32_t dk,
                             int32_t dv, kda_dtype dt, void *stream);

/* kda_decode_window with the evaluation form named by the caller (for tests
 * and tuning): form 0 = the automatic choice above, 1 = token by token (every
 * shape), 2 = one chunk on the matrix cores (KDA_BF16, dk = dv = 128,
 * T <= 16; KDA_ERR_UNSUPPORTED otherwise).  Other values: KDA_ERR_SHAPE.
 * Arguments and errors otherwise as for kda_decode_window. */
kda_status kda_decode_window_form(const void *q, const void *k, const void *v,
                                  const void *log_alpha, const void *beta,
                                  float *state, float *o, const int32_t *accept,
                                  int32_t B, int32_t T, int32_t H, int32_t dk,
                                  int32_t dv, kda_dtype dt, int32_t form, void *stream);

/* Speculative decoding as a serving loop runs it (Kimi K3 report digest,
 * serving section: the state cannot be rolled back, so the accepted drafts are
 * replayed from their cached projected inputs and only verified states are
 * written back).  The verifier's accepted count for a window is known only after
 * the window ran, so each call first replays, per sequence, the first
 * clamp(replay[b], 0, Tp) tokens of the PREVIOUS window (inputs pq, pk, pv,
 * pgate, pbeta: [B, Tp, H, .] as in kda_decode_window; no outputs), writes the
 * state back once after them (no write when that count is 0), and then runs the
 * T tokens of this window (the bonus token and the new drafts) from that state,
 * writing o [B, T, H, dv] for all of them and committing none.  One state read
 * and at most one write per call.  Tp = 0: nothing to replay (the p* pointers and
 * replay may be NULL).  gate_A_log, out_gate, norm_w, norm_eps, y as in
 * kda_decode_window_fused (the gate applies to replayed and new tokens, the
 * epilogue to the new tokens' outputs).  replay: device int32 [B], 4-byte
 * aligned.  B * T * H and B * Tp * H < 2^31.  The form is chosen as for
 * kda_decode_window, on T + Tp tokens (one chunk holds the replay and the
 * window when T + Tp <= 16).  Errors as for kda_decode_window. */
kda_status kda_decode_window_replay(const void *pq, const void *pk, const void *pv, const void *pgate,
                                    const void *pbeta, const int32_t *replay, int32_t Tp, const void *q,
                                    const void *k, const void *v, const void *gate, const float *gate_A_log,
                                    const void *beta, float *state, float *o, const void *out_gate,
                                    const float *norm_w, float norm_eps, void *y, int32_t B, int32_t T, int32_t H,
                                    int32_t dk, int32_t dv, kda_dtype dt, void *stream);

/* kda_decode_step and kda_decode_window with the layer's gate and epilogue
 * fused in (the passes below, evaluated where the decode kernels already hold
 * the operands, so a decode step of the layer is one launch):
 *   * gate_A_log != NULL: `gate` holds the decay logits z (same layout as
 *     log_alpha) and the kernel takes log-decay g = -5 Sigmoid(exp(A_log[h]) z)
 *     in fp32 (not rounded to the input dtype; a window evaluated as one chunk
 *     enters it into its decay sums as a hi + lo pair of bf16, 16 significant
 *     bits); gate_A_log is fp32 [H].
 *     NULL: `gate` is log_alpha as in kda_decode_step.
 *   * out_gate != NULL: y = Sigmoid(out_gate) * o / sqrt(mean(o^2) + norm_eps)
 *     * norm_w over the dv channels of each output row, written in the input
 *     dtype; out_gate and y are shaped like o (input dtype, 4-element aligned),
 *     norm_w fp32 [dv] (16-byte aligned), norm_eps >= 0.  In the single step
 *     o may then be NULL (not written).  The window computes the epilogue as a
 *     second launch over o (inside the window kernel it cost more than it
 *     saved), so there o is required and out_gate, y are 16-byte aligned.
 * Everything else as in the unfused calls. */
kda_status kda_decode_step_fused(const void *q, const void *k, const void *v,
                                 const void *gate, const float *gate_A_log,
                                 const void *beta, float *state, float *o,
                                 const void *out_gate, const float *norm_w,
                                 float norm_eps, void *y, int32_t B, int32_t H,
                                 int32_t dk, int32_t dv, kda_dtype dt, void *stream);

kda_status kda_decode_window_fused(const void *q, const void *k, const void *v,
                                   const void *gate, const float *gate_A_log,
                                   const void *beta, float *state, float *o,
                                   const int32_t *accept, const void *out_gate,
                                   const float *norm_w, float norm_eps, void *y,
                                   int32_t B, int32_t T, int32_t H, int32_t dk,
                                   int32_t dv, kda_dtype dt, void *stream);

/* One decode step of the whole layer core in one launch: the ShortConv
 * prologue of the new token (the passes below: Swish of the 4-tap causal
 * convolution, with each channel's 3 previous inputs taken from and shifted
 * into conv_cache; q and k then L2-normalised with l2_eps), the gate (as in
 * kda_decode_step_fused when gate_A_log != NULL), the recurrent step and, if
 * out_gate != NULL, the epilogue.
 *   qkv        : [B, H, 2 dk + dv] pre-convolution activations, per head the
 *                q, k and v channels in that order (input dtype; 4-element
 *                aligned);
 *   conv_w     : fp32 [H, 2 dk + dv, 4] (tap j multiplies x_{t-j}), 16-byte
 *                aligned;
 *   conv_cache : fp32 [B, H, 2 dk + dv, 3] (oldest first), updated in place;
 *   gate, beta, state, o, out_gate, norm_w, norm_eps, y as in
 *   kda_decode_step_fused. */
kda_status kda_decode_layer_step(const void *qkv, const float *conv_w,
                                 float *conv_cache, float l2_eps,
                                 const void *gate, const float *gate_A_log,
                                 const void *beta, float *state, float *o,
                                 const void *out_gate, const float *norm_w,
                                 float norm_eps, void *y, int32_t B, int32_t H,
                                 int32_t dk, int32_t dv, kda_dtype dt, void *stream);

/* ------------------------------------------------------------------------
 * The layer's passes around the recurrence (same page: the bounded-decay
 * section for the gate; the paragraph after the update equation for the
 * prologue -- a short convolution of kernel size 4 and Swish on q, k and v,
 * then L2 normalisation of q and k; the output-gate section for the epilogue
 * -- per-head RMSNorm of the recurrent output times a Sigmoid gate).  Each is
 * one streaming pass (HBM-bound), enqueued on `stream` like the calls above;
 * the projections that feed them (z, u, the pre-convolution q/k/v) and W_o are
 * the caller's.  dk, d, dv in {16, 32, 64, 128}; N in [0, 2^31); H >= 1;
 * N * H < 2^31;
 * eps >= 0 and finite.  [.., d] tensors (input dtype, and o) are read and
 * written eight elements at a time and must be 16-byte aligned; fp32 weight
 * arrays 16 bytes, caches 4 bytes.
 * ------------------------------------------------------------------------ */

/* Decay gate: log_alpha = -5 * Sigmoid(exp(A_log[h]) * z), the bounded
 * log-decay the recurrence takes, written in the input dtype (what a caller
 * would pass to kda_prefill).  z, log_alpha: [N, H, dk] (may be the same
 * buffer); A_log: fp32 [H]. */
kda_status kda_gate(const void *z, const float *A_log, int64_t N, int32_t H,
                    int32_t dk, kda_dtype dt, void *log_alpha, void *stream);

/* ShortConv prologue over packed sequences: per (head, channel)
 *   y_t = Swish(sum_{j=0..3} w[h][c][j] * x_{t-j}),  Swish(a) = a Sigmoid(a),
 * then, if l2norm != 0, y_t / sqrt(sum_c y_{t,c}^2 + eps) over the d channels
 * of the head (for q and k).  Inputs before a sequence's first token come from
 * cache_in (the 3 preceding inputs, oldest first; NULL = zeros), so a sequence
 * can be continued from an earlier call; cache_out (or NULL) receives each
 * sequence's last 3 inputs, oldest first (reaching into cache_in when the
 * sequence is shorter than 3), and may be cache_in itself.
 *   x, y: [N, H, d] (input dtype, distinct buffers); w: fp32 [H, d, 4];
 *   cu_seqlens: int32 [nseq + 1] device (as kda_prefill), or NULL with
 *   nseq == N: every token its own sequence (a decode step, the cache carrying
 *   each sequence's history);
 *   cache_in, cache_out: fp32 [nseq, H, d, 3]. */
kda_status kda_short_conv(const void *x, const float *w, const float *cache_in,
                          float *cache_out, const int32_t *cu_seqlens,
                          int32_t nseq, int64_t N, int32_t H, int32_t d,
                          int32_t l2norm, float eps, kda_dtype dt, void *y,
                          void *stream);

/* Speculative decoding of the whole layer core as a serving loop runs it (the
 * replay scheme of kda_decode_window_replay with the prologue of
 * kda_decode_layer_step; Kimi K3 report digest, serving section: the accepted
 * drafts are replayed from their cached projected inputs through the short
 * convolution, the norms, the gate and the recurrence, and only verified state is
 * written back).  Per sequence b the call first replays the first
 * clamp(replay[b], 0, Tp) tokens of the previous window -- pqkv, pgate, pbeta
 * [B, Tp, H, .] as qkv, gate, beta below -- and commits both the recurrent state
 * and the convolution cache after them (neither is written when that count is
 * 0); then it runs the T tokens of this window from there, writing o (and y) for
 * all of them and committing neither.  Each token is convolved in order from the
 * committed cache through the replayed and the new tokens, so the outputs are
 * those of T more kda_decode_layer_step calls after the replayed ones.
 *   qkv   : [B, T, H, 2 dk + dv] pre-convolution activations (as in
 *           kda_decode_layer_step, with the window axis after B);
 *   gate  : [B, T, H, dk] decay logits with gate_A_log (or log-decay with
 *           gate_A_log == NULL); beta [B, T, H];
 *   conv_w, conv_cache (fp32 [B, H, 2 dk + dv, 3], committed in place), l2_eps
 *           as in kda_decode_layer_step;
 *   state, o [B, T, H, dv] (required), out_gate, norm_w, norm_eps, y as in
 *           kda_decode_window_replay.
 * Tp = 0: nothing to replay (the p* pointers and replay may be NULL).
 * Evaluation: with a workspace (device, 16-byte aligned, workspace_bytes at
 * least kda_decode_layer_window_workspace_bytes(B, T, Tp, H, dk, dv, dt)) and
 * bf16 inputs with dk = dv = 128 and 6 <= T + Tp <= 16, a prologue pass writes
 * the convolved, normalised q, k, v and the log-decay rows, rounded to bf16, to
 * the workspace (committing the cache after the prefix), and the window runs as
 * one chunk on the matrix cores (the form of kda_decode_window); otherwise, and
 * with workspace == NULL, it runs token by token in one kernel, q, k, v and the
 * decay staying fp32.  The committed cache is the same in both (it holds raw
 * inputs).  B * T * H and B * Tp * H < 2^31.  Errors as for
 * kda_decode_layer_step; a workspace that is misaligned gives KDA_ERR_ALIGN, one
 * smaller than required KDA_ERR_SHAPE. */
kda_status kda_decode_layer_window_replay(const void *pqkv, const void *pgate, const void *pbeta,
                                          const int32_t *replay, int32_t Tp, const void *qkv,
                                          const void *gate, const void *beta, const float *conv_w,
                                          float *conv_cache, float l2_eps, const float *gate_A_log,
                                          float *state, float *o, const void *out_gate,
                                          const float *norm_w, float norm_eps, void *y, int32_t B,
                                          int32_t T, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                          void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace kda_decode_layer_window_replay needs for its one-chunk form
 * (1,024 B per (sequence, head, token) of T + Tp: bf16 q, k, v and log-decay of
 * 128 channels); 0 when that form does not apply to the shape (then the call
 * runs token by token and needs none) or the shape is invalid. */
size_t kda_decode_layer_window_workspace_bytes(int32_t B, int32_t T, int32_t Tp, int32_t H, int32_t dk,
                                               int32_t dv, kda_dtype dt);

/* Output epilogue: y = Sigmoid(u) * o / sqrt(mean_c(o_c^2) + eps) * w over
 * the dv channels of each (token, head).  o: fp32 [N, H, dv] (the recurrence's
 * output); u: gate logits [N, H, dv] (input dtype); w: fp32 [dv]; y: [N, H, dv]
 * in the input dtype (the operand of the caller's W_o). */
kda_status kda_out_norm_gate(const float *o, const void *u, const float *w,
                             float eps, int64_t N, int32_t H, int32_t dv,
                             kda_dtype dt, void *y, void *stream);

/* The layer core of a prefill in one call, with the prologue applied where the
 * recurrence's kernels load their inputs (same page: the paragraph after the
 * update equation and the bounded-decay section) instead of as separate passes
 * (bit for bit the results of kda_short_conv, kda_gate, kda_prefill's two-kernel
 * path and kda_out_norm_gate run in sequence on bf16-valued caches):
 * q, k and v are the raw (pre-convolution) projections; each goes through the
 * 4-tap causal ShortConv and Swish, q and k are L2-normalised (l2_eps), and the
 * log-decay is g = -5 Sigmoid(exp(A_log[h]) z) from the decay logits z.  These
 * are rounded to bf16 -- the values kda_short_conv and kda_gate would have
 * written -- and then run through the recurrence as in kda_prefill; with
 * out_gate != NULL the epilogue of kda_out_norm_gate follows (a separate pass
 * over o: the row norm spans the whole of dv, which the recurrence's
 * workgroups split).  bf16 with dk = dv = 128 only (else KDA_ERR_UNSUPPORTED).
 *   q, k, z       : [N, H, 128] raw projections and decay logits (bf16);
 *   v             : [N, H, 128] raw projection;  beta : [N, H];
 *   conv_w        : fp32 [H, 2 dk + dv, 4] (q, k, v channels per head, as in
 *                   kda_decode_layer_step; tap j multiplies x_{t-j}), 16-byte
 *                   aligned;
 *   conv_cache_in : fp32 [nseq, H, 2 dk + dv, 3], the 3 inputs before each
 *                   sequence (oldest first), or NULL (zeros).  The prefill
 *                   reads them rounded to bf16 (the inputs they hold are in
 *                   the input dtype; caches written by these calls are exact);
 *   conv_cache_out: same shape or NULL: each sequence's last 3 raw inputs,
 *                   reaching into conv_cache_in for sequences shorter than 3
 *                   tokens (may equal conv_cache_in; written after everything
 *                   else has read it), ready for kda_decode_layer_step;
 *   A_log         : fp32 [H];
 *   init_state, cu_seqlens, nseq, total_tokens, H, final_state: as kda_prefill;
 *   o             : fp32 [N, H, dv], required;
 *   out_gate, y   : [N, H, dv] bf16, 16-byte aligned, with norm_w fp32 [dv]
 *                   (16-byte aligned) and norm_eps >= 0; out_gate NULL = no
 *                   epilogue (y, norm_w unused);
 *   workspace     : kda_prefill_layer_workspace_bytes(...) bytes, 16-byte
 *                   aligned (the chunk-local operands, then the prologue's q,
 *                   k and log-decay in bf16, which the first of the two
 *                   recurrence kernels computes and the second reads; v's
 *                   prologue is applied where the second kernel loads v).
 * Errors as for kda_prefill; l2_eps and norm_eps must be finite and >= 0. */
size_t kda_prefill_layer_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk, int32_t dv,
                                         kda_dtype dt);
kda_status kda_prefill_layer(const void *q, const void *k, const void *v, const float *conv_w,
                             const float *conv_cache_in, float *conv_cache_out, float l2_eps, const void *z,
                             const float *A_log, const void *beta, const float *init_state,
                             const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk,
                             int32_t dv, kda_dtype dt, void *workspace, size_t ws_bytes, float *o,
                             float *final_state, const void *out_gate, const float *norm_w, float norm_eps,
                             void *y, void *stream);

/* kda_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as kda_prefill, without the workspace: the
 * library keeps it in a static device array of KDA_NOALLOC_SCRATCH_BYTES bytes
 * (128 MiB), one per GPU the library runs on, held until the process ends.
 * Problems whose kda_prefill_workspace_bytes exceed it return
 * KDA_ERR_TOO_LARGE before any launch (2 KiB per chunk slot and head:
 * (floor(N/16) + nseq) * H <= 65,536).  The call allocates nothing; on its
 * first call on a device it looks up the array's device address (a failure
 * there returns KDA_ERR_HIP).  Every call on one GPU shares that GPU's array
 * and the array keeps the last call's contents: calls that overlap on one GPU
 * (different streams or threads without ordering) race, so serialise them. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
kda_status kda_prefill_noalloc(const void *q, const void *k, const void *v,
                               const void *log_alpha, const void *beta,
                               const float *init_state, const int32_t *cu_seqlens,
                               int32_t nseq, int64_t total_tokens, int32_t H,
                               int32_t dk, int32_t dv, kda_dtype dt,
                               float *o, float *final_state, void *stream);

/* Opt-in check of a device-resident cu_seqlens against the layout contract above
 * (cu[0] = 0, non-decreasing, every entry in [0, total_tokens], cu[nseq] =
 * total_tokens), which the prefill-family calls assume without reading it on the
 * host.  One small kernel on `stream` writes to *result (device int32, 4-byte
 * aligned): -1 when the contract holds, else the smallest index i whose entry
 * breaks it (0: cu[0] != 0; i: cu[i] < cu[i-1] or out of range; nseq: the last
 * entry is not total_tokens).  For callers that build the offsets on the device
 * (a malformed one makes the kernels read and write outside the caller's
 * buffers).  Kernel launch only, like every call.  Errors: NULL pointers
 * KDA_ERR_NULL, misalignment KDA_ERR_ALIGN, nseq < 1 or total_tokens out of
 * range KDA_ERR_SHAPE. */
kda_status kda_check_cu_seqlens(const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens, int32_t *result,
                                void *stream);

/* Static string naming a status code. */
const char *kda_status_string(kda_status s);

/* hipError_t (as int) of the most recent KDA_ERR_HIP on the calling thread,
 * 0 if none. */
int32_t kda_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
