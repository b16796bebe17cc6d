/*
 * spec_verify.h -- C ABI of the batched speculative-decoding verify step on MI355X (gfx950).
 *
 * The operation ("Speculative Decoding: The Physics of Stolen Time", section 1
 * stage 3 and section 2; the speculative-decoding design note, "The acceptance
 * math"; "The Inference Wall" part 7, "How speculative decoding works";
 * "Speculative Pre-Positioning", section 2.4, Eq. 11):
 *
 *   For every batch row b with draft tokens x_0..x_{k-1}:
 *   SAMPLE mode -- p_i = softmax(target_logits[b,i,:] / T), q_i = softmax(draft_logits[b,i,:] / T);
 *     position i is accepted iff u[b,i,0] < p_i(x_i) / q_i(x_i) (probability min(1, p/q));
 *     at the first rejected position a the token is drawn from norm(max(0, p_a - q_a));
 *     when all k drafts are accepted (a = k) a bonus token is drawn from p_k.
 *     A draw from weights w uses u = u[b,a,1] and returns the smallest j with
 *     sum_{x<=j} w_x > u * sum_x w_x (inverse CDF in vocabulary order).
 *   GREEDY mode -- g_i = argmax target_logits[b,i,:] (lowest index on ties); a = first i
 *     with x_i != g_i, else k; the emitted token at position a is g_a.
 *   Both modes: gap[b,i] = top-1 minus top-2 of the raw target logits of row i (0 on a
 *     tie at the top, +inf when the row has fewer than two finite entries).
 *
 * Readings of points the method leaves open: temperature divides target and draft
 * logits alike and does not enter the gap or greedy mode; uniform channel 0 drives
 * the acceptance test and channel 1 the inverse-CDF draw (u[b,k,0] is unused);
 * q(x) = 0 accepts iff p(x) > 0; a rejection whose residual mass rounds to zero
 * draws from p_a instead.
 *
 * Memory: every pointer argument of spec_verify is a DEVICE pointer on the current HIP
 * device, owned by the caller. Tensors are dense, row-major, innermost index last:
 *   target_logits [B, k+1, V]  float32 or bfloat16 (dtype)
 *   draft_logits  [B, k,   V]  same dtype; may be NULL in GREEDY mode (never read there)
 *   draft_tokens  [B, k]       int32
 *   uniforms      [B, k+1, 2]  float32 in [0, 1); may be NULL in GREEDY mode
 *   accepted_len  [B]          int32 out: number of accepted drafts 0..k, or -1 (invalid row)
 *   out_tokens    [B, k+1]     int32 out: accepted drafts, then one sampled/argmax token,
 *                              then -1 padding; all -1 for an invalid row
 *   gap           [B, k+1]     float32 out
 *   target_prob, draft_prob [B, k] float32 out, optional (NULL to skip): p_i(x_i), q_i(x_i)
 *                              in SAMPLE mode; NaN in GREEDY mode
 * Inputs are only read. Outputs are fully overwritten and must not alias inputs, each
 * other or the workspace.
 *
 * Invalid rows (asynchronous, per batch row): a NaN or +inf logit in any row the mode
 * reads, a row without a finite entry, or a draft token outside [0, V) gives
 * accepted_len[b] = -1 and out_tokens[b,:] = -1. -inf logits are allowed (masked
 * entries, probability 0).
 *
 * Workspace: caller-owned device memory of at least spec_verify_workspace_size() bytes
 * (256-byte aligned). It carries the per-segment and per-batch-row records
 * that one kernel of the call hands to the next; every record is written before it is
 * read, so the workspace needs no initialisation and may be reused freely. One
 * workspace serves one call at a time: calls that overlap in time (e.g. on two
 * streams) need separate workspaces.
 *
 * Execution: spec_verify only enqueues work on `stream` (a hipStream_t; NULL = the null
 * stream) and returns; completion is observed by synchronising that stream. It performs
 * no allocation and no host synchronisation.
 *
 * Errors: 0 = enqueued. A negative return is synchronous and means nothing was enqueued;
 * spec_verify_last_error() then describes it (thread-local string).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_DTYPE_F32 0
#define SPEC_DTYPE_BF16 1

#define SPEC_MODE_SAMPLE 0
#define SPEC_MODE_GREEDY 1

#define SPEC_MAX_K 64
#define SPEC_MAX_V_SAMPLE 8388608   /* largest vocabulary SAMPLE mode accepts (2^23) */

#define SPEC_OK 0
#define SPEC_ERR_NULL (-1)      /* a required pointer is NULL                                   */
#define SPEC_ERR_SHAPE (-2)     /* B < 1, B > 2^21, k outside [0, SPEC_MAX_K], V < 1,
                                   V > SPEC_MAX_V_SAMPLE in SAMPLE mode, V > 2^29, or a size
                                   overflow                                                     */
#define SPEC_ERR_DTYPE (-3)     /* dtype is not SPEC_DTYPE_F32 / SPEC_DTYPE_BF16                */
#define SPEC_ERR_MODE (-4)      /* mode is not SPEC_MODE_SAMPLE / SPEC_MODE_GREEDY              */
#define SPEC_ERR_TEMP (-5)      /* SAMPLE mode with a temperature that is not finite and > 0    */
#define SPEC_ERR_WORKSPACE (-6) /* workspace NULL or smaller than spec_verify_workspace_size()  */
#define SPEC_ERR_ALIGN (-7)     /* a pointer is not aligned to its element size (4 B or 2 B),
                                   or the workspace is not 256-B aligned                        */
#define SPEC_ERR_HIP (-8)       /* the HIP runtime refused the launch                           */
#define SPEC_ERR_VALUE (-9)     /* spec_gate: tau is NaN, or negative under the certified rule  */

#define SPEC_GATE_MARGIN 0      /* spec_gate fires iff gap > tau                                */
#define SPEC_GATE_CERTIFIED 1   /* spec_gate fires iff gap > 0 and 2 * tau <= gap               */

/*
 * Enqueue the verify step. See the file comment for the meaning and layout of every
 * argument. temperature is ignored in GREEDY mode.
 */
int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const float* uniforms, float temperature, int mode, int32_t B, int32_t k, int32_t V,
                int dtype, int32_t* accepted_len, int32_t* out_tokens, float* gap, float* target_prob,
                float* draft_prob, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace spec_verify and spec_verify_ragged need for these sizes (0 if
 * the sizes are invalid).
 * Host-only; makes no HIP call.
 */
size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, int dtype, int mode);

/*
 * The synchronous argument checks of spec_verify, without enqueueing anything.
 * Host-only; makes no HIP call and dereferences no pointer. Returns 0 or a
 * SPEC_ERR_* code (and sets spec_verify_last_error()).
 */
int spec_verify_check_args(const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, const float* uniforms, float temperature,
                           int mode, int32_t B, int32_t k, int32_t V, int dtype,
                           const int32_t* accepted_len, const int32_t* out_tokens, const float* gap,
                           const void* workspace, size_t workspace_bytes);

/*
 * Ragged drafts: the same step when every batch row carries its own number of drafts
 * ("Speculative Decoding: The Physics of Stolen Time", section 6, adaptive k; the
 * speculative-decoding design note, "The acceptance math", variable-length drafting).
 * draft_len [B] int32 (DEVICE pointer, not NULL, 4-byte aligned) holds kb for every
 * batch row; the tensors keep the shapes of spec_verify with k = the largest draft
 * count the caller allows. Row b is verified exactly as spec_verify verifies a call
 * with k = kb on its first kb positions: target rows 0..kb, draft rows and tokens
 * 0..kb-1 and uniforms 0..kb are read, nothing else of the row; the bonus token comes
 * from target row kb. Outputs keep the [B, k+1] / [B, k] layout: gap of rows past kb
 * and target_prob/draft_prob of positions past kb-1 are NaN, out_tokens past the
 * emitted token are -1. A draft_len value outside [0, k] makes the row invalid
 * (accepted_len -1, out_tokens -1, gap NaN); it is not a synchronous error, since
 * the values live on the device. Only the rows in use are streamed from HBM. The
 * workspace, errors and execution are those of spec_verify
 * (spec_verify_workspace_size covers both entry points).
 */
int spec_verify_ragged(const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const int32_t* draft_len,
                       const float* uniforms, float temperature, int mode, int32_t B, int32_t k,
                       int32_t V, int dtype, int32_t* accepted_len, int32_t* out_tokens,
                       float* gap, float* target_prob, float* draft_prob, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * spec_verify (draft_len NULL) or spec_verify_ragged (draft_len set) with phase timing:
 * events points to four hipEvent_t the caller created (timing enabled), recorded on
 * `stream` before the first kernel (events[0]), after pass 1, the scan of every logit
 * (events[1]), after the decisions and pass 2 (events[2]) and after the draw (events[3];
 * greedy mode records events[2] and events[3] together). hipEventElapsedTime between
 * them gives each phase's duration on the device, e.g. the streaming pass alone. Errors
 * as spec_verify, plus SPEC_ERR_NULL when an event is missing. For profiling tools; the
 * results equal spec_verify's.
 */
int spec_verify_timed(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const int32_t* draft_len, const float* uniforms,
                      float temperature, int mode, int32_t B, int32_t k, int32_t V, int dtype,
                      int32_t* accepted_len, int32_t* out_tokens, float* gap, float* target_prob,
                      float* draft_prob, void* workspace, size_t workspace_bytes, void* stream,
                      void* const* events);

/*
 * Confidence gate over n ready distributions ("Speculative Pre-Positioning", section
 * 2.4, Eqs. 11-12, and the gated fast-path serve of Algorithm 2; the certified rule
 * is the argmax-stability bound of the speculative-decoding design note, "Axis 1
 * reuses the gate we already have").
 *   logits [n, V] float32 or bfloat16 (dtype), DEVICE, read only; any rows, e.g. the
 *     cached ready distributions of n sessions, or the target rows [B*(k+1), V] of a
 *     verify batch.
 *   For every row r: argmax[r] = lowest index of the largest logit; gap[r] = top-1
 *     minus top-2 (as spec_verify's gap: 0 on a tie at the top, +inf with fewer than
 *     two finite entries); fire[r] = 1 iff argmax[r] is admissible and
 *       SPEC_GATE_MARGIN:    gap > tau (tau: the gate threshold, 2.0 in the pages);
 *       SPEC_GATE_CERTIFIED: gap > 0 and 2 * tau <= gap (tau: a bound Q on the
 *                            sup-norm of the logit error, e.g. a calibrated quantile);
 *     the comparison is made in float32 on the stored gap. A row with NaN or +inf
 *     anywhere or with no finite entry gives argmax -1, gap NaN, fire 0.
 *   admit: the admissible set A as a V-bit mask, uint32 [(V+31)/32], bit (j & 31) of
 *     word j >> 5 set iff token j is admissible; DEVICE, 4-byte aligned; NULL admits
 *     every token.
 *   argmax int32 [n], gap float32 [n], fire int32 [n]: DEVICE outputs, fully
 *     overwritten.
 * Workspace: at least spec_gate_workspace_size(n, V, dtype) bytes, same rules as
 * spec_verify's. Execution and errors as spec_verify (n < 1 or V < 1 gives
 * SPEC_ERR_SHAPE; an unknown rule SPEC_ERR_MODE; a bad tau SPEC_ERR_VALUE).
 */
int spec_gate(const void* logits, int32_t n, int32_t V, int dtype, int rule, float tau,
              const uint32_t* admit, int32_t* argmax, float* gap, int32_t* fire, void* workspace,
              size_t workspace_bytes, void* stream);

/* Bytes of workspace spec_gate needs (0 if the sizes are invalid). Host-only. */
size_t spec_gate_workspace_size(int32_t n, int32_t V, int dtype);

/*
 * Commit / rollback after a verify step (KV truncation on rejection: "Speculative
 * Decoding: The Physics of Stolen Time", section 6, "KV-cache management", and the
 * speculative-decoding design note's KV rollback; per-position recurrent-state
 * checkpoints of hybrid models: "The Inference Wall" part 7, "Why it inverts,
 * mechanism 2").
 * The verify forward of batch row b consumed k+1 tokens (the pending token, then the
 * k drafts), appended their KV entries at kv_len[b]..kv_len[b]+k, and wrote
 * checkpoint slot j = the recurrent state after the pending token and drafts 0..j-1.
 * With a = accepted_len[b] in [0, k]:
 *   kv_len[b] += 1 + a                (the entries of rejected drafts are dropped),
 *   state[b, :] = slots[b, a, :]      (the state of the committed prefix).
 * Rows with a outside [0, k] (e.g. -1, an invalid verify row) are left unchanged.
 *   accepted_len [B] int32: DEVICE, read only (spec_verify's output).
 *   kv_len [B] int32: DEVICE, updated in place; NULL skips the KV lengths.
 *   slots [B, k+1, state_bytes] and state [B, state_bytes]: DEVICE raw bytes (any
 *     element type), state_bytes a multiple of 4, pointers 4-byte aligned (16-byte
 *     alignment and a 16-byte multiple use 16-byte copies); state_bytes = 0 skips
 *     the state (slots and state may then be NULL). slots and state must not overlap.
 * Needs no workspace. Enqueues one kernel on `stream` (nothing when kv_len is NULL
 * and state_bytes is 0). Errors: SPEC_ERR_SHAPE (B < 1, B > 2^21, k outside
 * [0, SPEC_MAX_K], sizes too large), SPEC_ERR_NULL, SPEC_ERR_ALIGN, SPEC_ERR_HIP.
 */
int spec_commit(const int32_t* accepted_len, int32_t B, int32_t k, int32_t* kv_len,
                const void* slots, void* state, size_t state_bytes, void* stream);

/*
 * Greedy verification fused with an int8 LM head (the verify forward's batched
 * LM-head projection: the speculative-decoding design note, "Cost / correctness
 * constraints", batched verify forward; "Speculative Decoding: The Physics of Stolen
 * Time", section 1, the target's parallel pass; quantized heads as in the 4-bit and
 * GGUF deployments those pages run). The logits are never stored:
 *   logit[m, v] = fl32( fl32( float32(acc[m, v]) * hidden_scale[m] ) * weight_scale[v] ),
 *   acc[m, v]   = sum_j hidden[m, j] * weight[v, j]   (exact integer; float32() rounds
 *                                                      to nearest even),
 * with hidden row m = b*(k+1) + i the target's final hidden state at position i of
 * batch row b. The outputs are exactly spec_verify's GREEDY outputs on those float32
 * logits (argmax with the lowest index on ties, first mismatch, gap; invalid rows as
 * there: a NaN or +inf logit, a row without a finite entry, a draft token outside
 * [0, V)).
 *   hidden [B*(k+1), d] int8, weight [V, d] int8: DEVICE, 16-byte aligned.
 *   hidden_scale [B*(k+1)], weight_scale [V] float32: DEVICE.
 *   draft_tokens [B, k] int32, accepted_len [B], out_tokens [B, k+1], gap [B, k+1]:
 *     DEVICE, as in spec_verify (GREEDY mode).
 * d must be a multiple of 128 in [128, 65536] (so |acc| < 2^31); 1 <= B <= 2^21,
 * 0 <= k <= SPEC_MAX_K, 1 <= V <= 2^29, B*(k+1) <= 2^26. Workspace: at least
 * spec_lmhead_workspace_size() bytes, 256-byte aligned, no initialisation needed,
 * one call at a time. Enqueues three kernels on `stream`; no allocation, no host
 * synchronisation. Errors: SPEC_ERR_SHAPE, SPEC_ERR_NULL, SPEC_ERR_ALIGN,
 * SPEC_ERR_WORKSPACE, SPEC_ERR_HIP (nothing enqueued).
 */
int spec_verify_lmhead(const int8_t* hidden, const float* hidden_scale, const int8_t* weight,
                       const float* weight_scale, const int32_t* draft_tokens, int32_t B, int32_t k,
                       int32_t V, int32_t d, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace spec_verify_lmhead needs (0 if the sizes are invalid). Host-only. */
size_t spec_lmhead_workspace_size(int32_t B, int32_t k, int32_t V, int32_t d);

/*
 * spec_verify_lmhead that also records events[0] before the LM-head kernel,
 * events[1] after it and events[2] after the decisions, on `stream` (three
 * hipEvent_t created by the caller). Same results.
 */
int spec_verify_lmhead_timed(const int8_t* hidden, const float* hidden_scale, const int8_t* weight,
                             const float* weight_scale, const int32_t* draft_tokens, int32_t B, int32_t k,
                             int32_t V, int32_t d, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                             void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * Sampling-mode verification fused with int8 LM heads (modified rejection
 * sampling: "Speculative Decoding: The Physics of Stolen Time", section 2, the
 * acceptance test and the residual; the speculative-decoding design note, "Cost /
 * correctness constraints"; the heads as in spec_verify_lmhead). Target logits
 *   t[m, v] = fl32( fl32( float32(acc_t[m, v]) * target_hidden_scale[m] ) * target_weight_scale[v] ),
 *   acc_t[m, v] = sum_j target_hidden[m, j] * target_weight[v, j]   (exact integer),
 * for target hidden row m = b*(k+1) + i, and draft logits likewise from draft
 * hidden row m = b*k + i and the draft head. The outputs are exactly spec_verify's
 * SAMPLE outputs on those float32 logits (same near-tie rules, same invalid rows).
 * One pass of each head (an MFMA tile per 256 vocabulary rows and up to 256 hidden
 * rows) folds its logits into per-row sums, top-2 and flags, and stores them into
 * the workspace, where the draw of pass 2 reads the two rows each batch row draws
 * from (target row a, and draft row a when a < k); the draft token's logit comes
 * from an exact int8 dot product of its hidden row and head row.
 *   target_hidden [B*(k+1), d] int8, target_weight [V, d] int8: DEVICE, 16-byte aligned.
 *   target_hidden_scale [B*(k+1)], target_weight_scale [V] float32: DEVICE.
 *   draft_hidden [B*k, d] int8 (16-byte aligned), draft_hidden_scale [B*k] float32:
 *     DEVICE; may be NULL when k = 0.
 *   draft_weight [V, d] int8, draft_weight_scale [V] float32: DEVICE, or both NULL
 *     when the draft shares the target's head.
 *   draft_tokens [B, k] int32, uniforms [B, k+1, 2] float32, accepted_len [B],
 *     out_tokens [B, k+1], gap [B, k+1], target_prob [B, k], draft_prob [B, k]
 *     (the last two may be NULL): DEVICE, as in spec_verify (SAMPLE mode).
 * d must be a multiple of 128 in [128, 65536]; 1 <= B <= 2^21, 0 <= k <= SPEC_MAX_K,
 * 1 <= V <= SPEC_MAX_V_SAMPLE, B*(k+1) <= 2^26; temperature finite and > 0.
 * Workspace: at least spec_lmhead_sample_workspace_size() bytes (about
 * B*(2k+1)*V*4 for the logits, plus per-tile records), 256-byte aligned, no
 * initialisation needed, one call at a time. Enqueues five kernels (four when k = 0) on
 * `stream`; no allocation, no host synchronisation. Errors: SPEC_ERR_SHAPE,
 * SPEC_ERR_TEMP, SPEC_ERR_NULL, SPEC_ERR_ALIGN, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP
 * (nothing enqueued).
 */
int spec_verify_lmhead_sample(const int8_t* target_hidden, const float* target_hidden_scale,
                              const int8_t* target_weight, const float* target_weight_scale,
                              const int8_t* draft_hidden, const float* draft_hidden_scale,
                              const int8_t* draft_weight, const float* draft_weight_scale,
                              const int32_t* draft_tokens, const float* uniforms, float temperature, int32_t B,
                              int32_t k, int32_t V, int32_t d, int32_t* accepted_len, int32_t* out_tokens,
                              float* gap, float* target_prob, float* draft_prob, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of workspace spec_verify_lmhead_sample needs (0 if the sizes are invalid). Host-only. */
size_t spec_lmhead_sample_workspace_size(int32_t B, int32_t k, int32_t V, int32_t d);

/*
 * spec_verify_lmhead_sample that also records, on `stream` (four hipEvent_t
 * created by the caller), events[0] before the first head kernel, events[1] after
 * the head passes, events[2] after the merges of their records, and events[3]
 * after the decisions and the draw. Same results.
 */
int spec_verify_lmhead_sample_timed(const int8_t* target_hidden, const float* target_hidden_scale,
                                    const int8_t* target_weight, const float* target_weight_scale,
                                    const int8_t* draft_hidden, const float* draft_hidden_scale,
                                    const int8_t* draft_weight, const float* draft_weight_scale,
                                    const int32_t* draft_tokens, const float* uniforms, float temperature,
                                    int32_t B, int32_t k, int32_t V, int32_t d, int32_t* accepted_len,
                                    int32_t* out_tokens, float* gap, float* target_prob, float* draft_prob,
                                    void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * The LM heads above in a tile-major layout, written once per head (a head is
 * static) so that the head kernels stream it in long contiguous runs: the
 * multiply-adds and results are those of the row-major calls, bit for bit.
 * ("Speculative Decoding: The Physics of Stolen Time", section 1, stage 2, and
 * the gnosis design note, "Cost / correctness constraints": the verify pass
 * applies the head to every speculated position; this only changes where its
 * bytes sit.)
 *
 * Layout: for each vocabulary tile of 256 rows (zeros past V) and each 64 bytes
 * of d, one contiguous 16 KB block holding those 64 bytes of the tile's 256
 * rows in the order the head kernels stage them (row r at 64 r, its 16-byte
 * chunk p holding chunk p ^ ((r >> 2) & 3) of the row's 64 bytes).
 */

/* Bytes of the tile-major copy of an int8 head [V, d]: ceil(V/256)*256*d
 * (0 if V or d is outside the ranges spec_verify_lmhead accepts). Host-only. */
size_t spec_lmhead_packed_size(int32_t V, int32_t d);

/*
 * Enqueue on `stream` the kernel that writes weight (int8 [V, d], row-major,
 * device) into packed (device, at least spec_lmhead_packed_size(V, d) bytes,
 * both 16-byte aligned). The caller owns both buffers. Errors as above
 * (SPEC_ERR_SHAPE, SPEC_ERR_NULL, SPEC_ERR_ALIGN, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP);
 * nothing is enqueued on an argument error.
 */
int spec_lmhead_pack(const int8_t* weight, int32_t V, int32_t d, int8_t* packed, size_t packed_bytes, void* stream);

/*
 * spec_verify_lmhead / spec_verify_lmhead_timed with the head in the tile-major
 * layout (packed_weight as written by spec_lmhead_pack for this V and d).
 * events: NULL, or the three events of spec_verify_lmhead_timed. Same
 * arguments, workspace, results and errors otherwise.
 */
int spec_verify_lmhead_packed(const int8_t* hidden, const float* hidden_scale, const int8_t* packed_weight,
                              const float* weight_scale, const int32_t* draft_tokens, int32_t B, int32_t k,
                              int32_t V, int32_t d, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                              void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * spec_verify_lmhead_sample / _timed with both heads in the tile-major layout
 * (draft_packed_weight NULL for a shared head, as draft_weight there). events:
 * NULL, or the four events of spec_verify_lmhead_sample_timed. Same arguments,
 * workspace, results and errors otherwise.
 */
int spec_verify_lmhead_sample_packed(const int8_t* target_hidden, const float* target_hidden_scale,
                                     const int8_t* target_packed_weight, const float* target_weight_scale,
                                     const int8_t* draft_hidden, const float* draft_hidden_scale,
                                     const int8_t* draft_packed_weight, const float* draft_weight_scale,
                                     const int32_t* draft_tokens, const float* uniforms, float temperature,
                                     int32_t B, int32_t k, int32_t V, int32_t d, int32_t* accepted_len,
                                     int32_t* out_tokens, float* gap, float* target_prob, float* draft_prob,
                                     void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): spec_verify with the
 * library's own device scratch buffer in place of a caller workspace. Every other
 * argument, the outputs, the errors and the execution are those of spec_verify.
 * The scratch is a static device array of SPEC_NOALLOC_SCRATCH_BYTES on each GPU
 * the library runs on, held until the process ends; its device address is looked
 * up once per device on the first call there (hipGetSymbolAddress), and no call
 * allocates or frees anything. Sizes whose workspace
 * (spec_verify_workspace_size) exceeds the scratch return SPEC_ERR_WORKSPACE and
 * enqueue nothing. Every call on one GPU shares that GPU's scratch, which keeps
 * the last call's contents (each call writes every record before reading it):
 * calls that overlap in time on one GPU (e.g. on two streams) race and must be
 * serialised by the caller.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (16u << 20)

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const float* uniforms, float temperature, int mode, int32_t B, int32_t k, int32_t V,
                        int dtype, int32_t* accepted_len, int32_t* out_tokens, float* gap,
                        float* target_prob, float* draft_prob, void* stream);

/* Thread-local description of the last non-zero return of this library. */
const char* spec_verify_last_error(void);

/* Library version string. */
const char* spec_verify_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
