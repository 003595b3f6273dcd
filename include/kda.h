/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) layer on one
 * AMD MI355X (gfx950).
 *
 * The operation
 * -------------
 * "Kimi K3 technical FAQ" (Runpod guide), question "What is KDA, and why does
 * a serving engineer care?": KDA is the delta-rule linear-attention
 * recurrence with a per-channel forget gate; each layer keeps, per head, a
 * recurrent state of shape dk x dv that is updated per chunk, parallel
 * within a chunk and recurrent across chunks.  The question "What does the
 * architecture actually look like?" on the same page adds that the state is
 * fixed-size (it replaces a growing KV cache).  This library reads the
 * recurrence as
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,     scale = dk^(-1/2) unless given,
 *
 * with alpha_t = exp(g_t) in (0,1]^dk (one forget factor per key channel)
 * and beta_t in [0,1].  The gate crosses this boundary in log space, g <= 0,
 * because chunked evaluation needs sums of log-gates and products of alpha
 * underflow fp32 within a chunk.
 *
 * "Day-0 vLLM support for Kimi K3" (vLLM blog), section "Kimi K3's
 * architecture, and how vLLM serves it": prefix caching over recurrent state
 * reuses state snapshots taken at block boundaries.  kda_prefill therefore
 * writes the fp32 state after every `snapshot_interval` tokens of each
 * sequence; passing snapshot j back as `initial_state` with the remaining
 * tokens reproduces the uninterrupted run bit for bit.
 *
 * Conventions for every call
 * --------------------------
 * - All tensors are caller-owned device memory, row-major and contiguous.
 *   The library allocates no device memory and keeps no pointer after a call
 *   returns (kda_prefill_noalloc uses one fixed device array per GPU that the
 *   library holds, below).
 * - Calls are asynchronous on `stream`, a hipStream_t passed as void * so
 *   that this header compiles as plain C without the HIP headers (NULL = the
 *   default stream).  KDA_OK means "validated and enqueued"; results are visible
 *   after the stream is synchronised.
 * - Every argument check happens before anything is enqueued: a call that
 *   returns an error has launched nothing and written nothing.
 *   kda_last_error_detail() then describes the failure (thread-local).
 * - Device tensors of head vectors and states (q, k, v, g, out, states,
 *   snapshots, workspace) must be 16-byte aligned; beta, cu_seqlens_dev and
 *   state_slots_dev 4-byte aligned (KDA_ERR_ALIGNMENT otherwise).
 * - Supported shapes: dk == dv in {16, 32, 64, 128}; anything else returns
 *   KDA_ERR_UNSUPPORTED.  q/k/v are bf16 or fp32 (in_dtype); g, beta, states
 *   and snapshots are fp32; out is fp32 or bf16 (out_dtype).
 * - No call prints, throws across the ABI or exits.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 1

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad cu_seqlens ...  */
    KDA_ERR_UNSUPPORTED = 2, /* shape or dtype the library does not provide */
    KDA_ERR_ALIGNMENT = 3,   /* a device pointer is under-aligned           */
    KDA_ERR_WORKSPACE = 4,   /* workspace smaller than the size required    */
    KDA_ERR_HIP = 5          /* the HIP runtime reported a launch error     */
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

typedef struct {
    int32_t num_heads; /* H                                                 */
    int32_t dk;        /* key/query head dim (rows of the state)            */
    int32_t dv;        /* value head dim (columns of the state)             */
    kda_dtype in_dtype;  /* dtype of q, k, v                                */
    kda_dtype out_dtype; /* dtype of out                                    */
    float scale;       /* output scale; 0 selects dk^(-1/2)                 */
} kda_config;

/* Library version (KDA_VERSION of the build). */
int32_t kda_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *kda_status_string(kda_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *kda_last_error_detail(void);

/*
 * Number of snapshot rows kda_prefill writes for these sequences ("Day-0 vLLM
 * support for Kimi K3", section "Kimi K3's architecture, and how vLLM serves
 * it": prefix caching reuses recurrent-state snapshots taken at block
 * boundaries; one snapshot per interval tokens of each sequence):
 * sum_b floor(L_b / interval), L_b = cu_seqlens_host[b+1] - cu_seqlens_host[b].
 * Sequence b's snapshots occupy rows starting at sum_{b'<b} floor(L_b'/interval),
 * in order j = 1 .. floor(L_b/interval).  Returns 0 when interval <= 0 and
 * -1 when cu_seqlens_host is NULL or decreasing.
 */
int64_t kda_snapshot_count(const int32_t *cu_seqlens_host, int32_t num_seqs,
                           int32_t interval);

/*
 * Bytes of device workspace kda_prefill needs for this problem.  The chunked
 * form ("Kimi K3 technical FAQ", question "What is KDA, and why does a
 * serving engineer care?": parallel within a chunk, recurrent across chunks)
 * computes every chunk's state-independent operands in parallel first and
 * keeps them here for the recurrent pass: three per-sequence index arrays of
 * 4 * (num_seqs + 1) bytes each, each rounded up to 256 (768 B for up to 63
 * sequences), plus (floor(total_tokens / 64) + num_seqs) * num_heads *
 * 115,280 B of per-chunk operands (about 1.8 KB per token and head).  The
 * operand block is laid out for 128 state rows and 128 value columns whatever
 * dk and dv are (rows and columns past them hold zeros), so at dk = dv = 16 it
 * is 8 times larger than the data it holds.  Returns 0 for unsupported
 * configs too; kda_prefill reports those.
 */
size_t kda_prefill_workspace_size(const kda_config *cfg, int32_t num_seqs,
                                  int64_t total_tokens);

/*
 * Chunked prefill over packed variable-length sequences.
 *
 * Sequence b owns tokens [cu[b], cu[b+1]) of every token-major tensor
 * (T = cu[num_seqs] tokens in all):
 *   q, k : [T, H, dk]  in_dtype       v    : [T, H, dv]  in_dtype
 *   g    : [T, H, dk]  fp32, log of the forget gate, every entry <= 0
 *   beta : [T, H]      fp32, in [0, 1]
 *   initial_state : [num_seqs, H, dk, dv] fp32, or NULL for zero states
 * Entries of q and k must be below 2^15 in magnitude (rows of unit L2 norm,
 * as KDA feeds them, are far inside): the decay-scaled query and key factors
 * of the off-diagonal Gram blocks are fp16 MFMA operands.  No other range
 * limit applies beyond fp32's own: the scan's fp16 operands carry a
 * power-of-two exponent per tile (v and initial states scaled by 2^100 and
 * 2^-100 meet the same parity bar as at unit scale).
 *   out  : [T, H, dv]  out_dtype      (written)
 *   final_state : [num_seqs, H, dk, dv] fp32 (written; may alias
 *                 initial_state exactly, no other aliasing allowed)
 *   snapshots : [kda_snapshot_count(...), H, dk, dv] fp32 (written); may be
 *               NULL when that count is 0
 * cu_seqlens_host and cu_seqlens_dev hold the same num_seqs+1 offsets
 * (host memory and device memory): cu[0] == 0, non-decreasing.  Empty
 * sequences are allowed (their final state is their initial state).
 * snapshot_interval: 0 for none, otherwise a positive multiple of 64 (the
 * chunk length); chunks restart at every sequence start.
 * Errors: KDA_ERR_INVALID_ARG (null required pointer, num_seqs < 0, bad
 * offsets, interval not a multiple of 64, snapshots NULL while some are
 * due), KDA_ERR_UNSUPPORTED, KDA_ERR_ALIGNMENT, KDA_ERR_WORKSPACE, KDA_ERR_HIP.
 */
kda_status kda_prefill(const kda_config *cfg, int32_t num_seqs,
                       const int32_t *cu_seqlens_host,
                       const int32_t *cu_seqlens_dev, const void *q,
                       const void *k, const void *v, const float *g,
                       const float *beta, const float *initial_state,
                       void *out, float *final_state,
                       int32_t snapshot_interval, float *snapshots,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device memory kda_prefill_noalloc holds on each GPU it runs on
 * (from its first call there until the process ends): room for
 * kda_prefill_workspace_size() <= 128 MiB, e.g. one sequence of up to 2,303
 * tokens at 32 heads.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)

/*
 * kda_prefill without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The chunk operands go to a fixed device
 * array of KDA_NOALLOC_SCRATCH_BYTES per GPU that the library owns; the call
 * allocates nothing.  Arguments, results and errors are those of kda_prefill
 * (same kernels, bit-identical results), plus KDA_ERR_WORKSPACE when
 * kda_prefill_workspace_size() for the call exceeds the array (nothing is
 * launched then) and KDA_ERR_HIP if the array's device address cannot be
 * obtained.  Every call on one GPU uses that GPU's array: calls that overlap
 * on one GPU (two streams, two host threads) race and must not be issued.
 */
kda_status kda_prefill_noalloc(const kda_config *cfg, int32_t num_seqs,
                               const int32_t *cu_seqlens_host,
                               const int32_t *cu_seqlens_dev, const void *q,
                               const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state,
                               void *out, float *final_state,
                               int32_t snapshot_interval, float *snapshots,
                               void *stream);

/*
 * Prefill over a pool of resident states, with absolute token positions.
 *
 * "Day-0 vLLM support for Kimi K3" (vLLM blog), section "Kimi K3's
 * architecture, and how vLLM serves it": a hybrid cache manager keeps
 * compact recurrent-state blocks for the KDA layers, and prefix caching over
 * recurrent state separates the prefix-match granularity from the physical
 * state-block size, reusing state snapshots taken at block boundaries; the
 * same page, section "Deployment notes, each from a real incident", says
 * prefix caching covers the recurrent KDA state.  Here that means:
 *   - sequence b's first token in this call sits at absolute position
 *     start_pos[b] >= 0 (the tokens before it are the prefix whose state the
 *     pool holds);
 *   - its state lives in row state_slots_dev[b] (or b) of state_pool
 *     [num_slots, H, dk, dv] fp32: read as the state after start_pos[b]
 *     tokens when start_pos[b] > 0 (zero state when start_pos[b] == 0), and
 *     overwritten with the state after the call's tokens;
 *   - snapshots are taken at the absolute positions P in (start_pos[b],
 *     start_pos[b] + L_b] with P % snapshot_interval == 0, in order of P,
 *     sequence b's block starting at the sum of the earlier sequences'
 *     counts (kda_snapshot_count_at), so a snapshot serves as the pool row for
 *     a later call that starts at P, whatever block boundaries the first call
 *     had;
 *   - chunks are cut at absolute multiples of 64, so resuming from a
 *     snapshot at P reproduces the uninterrupted run bit for bit.
 * Other arguments as in kda_prefill (out is [T, H, dv]; the workspace comes
 * from kda_prefill_pool_workspace_size).  Slots must be distinct and
 * < num_slots (not checked on the device).
 * Errors: KDA_ERR_INVALID_ARG (also a negative start_pos, or start_pos + L
 * beyond 2^31 - 1, or num_slots too small), KDA_ERR_UNSUPPORTED,
 * KDA_ERR_ALIGNMENT, KDA_ERR_WORKSPACE, KDA_ERR_HIP.
 */
kda_status kda_prefill_pool(const kda_config *cfg, int32_t num_seqs,
                            const int32_t *cu_seqlens_host,
                            const int32_t *cu_seqlens_dev,
                            const int32_t *start_pos_host,
                            const int32_t *start_pos_dev, const void *q,
                            const void *k, const void *v, const float *g,
                            const float *beta, float *state_pool,
                            const int32_t *state_slots_dev, int32_t num_slots,
                            void *out, int32_t snapshot_interval,
                            float *snapshots, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Snapshot rows kda_prefill_pool writes: sum_b floor((s_b + L_b) / interval)
 * - floor(s_b / interval), s_b = start_pos_host[b].  0 when interval <= 0;
 * -1 for NULL arrays, decreasing offsets or a negative start.
 */
int64_t kda_snapshot_count_at(const int32_t *cu_seqlens_host,
                              const int32_t *start_pos_host, int32_t num_seqs,
                              int32_t interval);

/*
 * Workspace bytes for kda_prefill_pool: the same index arrays as
 * kda_prefill_workspace_size plus (floor(total_tokens / 64) + 2 * num_seqs) *
 * num_heads * 115,280 B (a start position off the 64-token grid can add one
 * chunk per sequence).
 */
size_t kda_prefill_pool_workspace_size(const kda_config *cfg, int32_t num_seqs,
                                       int64_t total_tokens);

/*
 * One decode step: one new token for each of num_seqs sequences against
 * states resident on the device, updated in place.
 *   q, k : [num_seqs, H, dk] in_dtype    v : [num_seqs, H, dv] in_dtype
 *   g    : [num_seqs, H, dk] fp32 (<= 0) beta : [num_seqs, H] fp32
 *   state : [num_slots, H, dk, dv] fp32, read and written in place
 *   state_slots_dev : [num_seqs] int32 device array mapping sequence n to
 *                     its state row, or NULL for the identity; entries must
 *                     be distinct and < num_slots (not checked on device)
 *   out  : [num_seqs, H, dv] out_dtype (written)
 * "Moonshot releases Kimi K3 report" (runtimewire), section "The
 * architecture is built around inference cost": the state is fixed-size, so
 * each step reads and writes exactly H*dk*dv*4 bytes of state per sequence.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_ALIGNMENT,
 * KDA_ERR_HIP.  num_seqs == 0 is a no-op.
 */
kda_status kda_decode(const kda_config *cfg, int32_t num_seqs, const void *q,
                      const void *k, const void *v, const float *g,
                      const float *beta, float *state,
                      const int32_t *state_slots_dev, void *out, void *stream);

/*
 * Several tokens per sequence against resident states, in one launch.
 *
 * "Kimi K3 technical FAQ" (Runpod guide), questions "What does it take to
 * serve K3 today?" and "What is the speculative-decoding story?": K3 is
 * served with a draft model proposing 7 tokens that the target verifies in
 * one pass, so a decode step carries 1 + 7 tokens per sequence.  "Moonshot
 * releases Kimi K3 report..." (runtimewire), section "A third party tripled
 * single-user decoding speed": on average 4.73 (coding) or 2.61 (creative
 * writing) draft tokens are accepted per step.  The modes:
 *   KDA_MULTI_APPLY  all num_tokens tokens applied in order: out holds every
 *                    position's output and the state advances by num_tokens
 *                    (the same as that many chained kda_decode calls);
 *   KDA_MULTI_VERIFY out holds every position's output as if the tokens were
 *                    applied in order; the state is only read;
 *   KDA_MULTI_COMMIT the first accepted_dev[n] tokens of sequence n (clamped
 *                    to [0, num_tokens]) are applied to its state; no output
 *                    (q and out may be NULL).
 * VERIFY then COMMIT is a roll-back path: a state never moves past the
 * accepted tokens, and no per-position state is kept.  Each launch reads
 * each state once (and writes it once in APPLY and COMMIT), whatever
 * num_tokens is.  APPLY is bit-identical to chained kda_decode calls;
 * VERIFY and COMMIT with num_tokens <= 8 use the chunked form of the
 * recurrence (one short chunk), whose results differ from the token-by-token
 * ones only by rounding order.
 */
typedef enum {
    KDA_MULTI_APPLY = 0,
    KDA_MULTI_VERIFY = 1,
    KDA_MULTI_COMMIT = 2
} kda_multi_mode;

/*
 *   q, k : [num_seqs, num_tokens, H, dk] in_dtype (token j of sequence n at
 *          row n*num_tokens + j)
 *   v    : [num_seqs, num_tokens, H, dv] in_dtype
 *   g    : [num_seqs, num_tokens, H, dk] fp32 (<= 0)
 *   beta : [num_seqs, num_tokens, H] fp32
 *   state : [num_slots, H, dk, dv] fp32, read (and written in place by APPLY
 *           and COMMIT)
 *   state_slots_dev : [num_seqs] int32 or NULL (identity), as in kda_decode
 *   accepted_dev : [num_seqs] int32 device array (COMMIT only; else ignored)
 *   out  : [num_seqs, num_tokens, H, dv] out_dtype (APPLY, VERIFY)
 * Errors: KDA_ERR_INVALID_ARG (null required pointer, num_tokens < 1, bad
 * mode), KDA_ERR_UNSUPPORTED, KDA_ERR_ALIGNMENT, KDA_ERR_HIP.
 * num_seqs == 0 is a no-op.
 */
kda_status kda_decode_multi(const kda_config *cfg, int32_t num_seqs,
                            int32_t num_tokens, kda_multi_mode mode,
                            const void *q, const void *k, const void *v,
                            const float *g, const float *beta, float *state,
                            const int32_t *state_slots_dev,
                            const int32_t *accepted_dev, void *out,
                            void *stream);

/*
 * One speculative decoding step in one launch: the previous step's accepted
 * tokens are committed to each state (written back), then the new draft of
 * num_tokens tokens is verified from the committed state (outputs only).
 * The same result as KDA_MULTI_COMMIT on the previous tokens followed by
 * KDA_MULTI_VERIFY on the new ones, bit for bit, with one read and one write
 * of each state instead of two reads and a write.
 *   prev_k, prev_v : [num_seqs, num_tokens, H, d] in_dtype, prev_g fp32,
 *   prev_beta [num_seqs, num_tokens, H] fp32: the previous step's tokens
 *   accepted_dev   : [num_seqs] int32, tokens of the previous step to commit
 *                    (clamped to [0, num_tokens]); NULL = nothing to commit
 *                    (the first step), and the prev_* arrays are ignored
 *   q, k, v, g, beta, out : the new draft and its outputs, as in
 *                    kda_decode_multi
 *   state, state_slots_dev: as in kda_decode_multi (written)
 * Errors as for kda_decode_multi.  num_seqs == 0 is a no-op.
 */
kda_status kda_decode_spec_step(const kda_config *cfg, int32_t num_seqs,
                                int32_t num_tokens, const void *prev_k,
                                const void *prev_v, const float *prev_g,
                                const float *prev_beta,
                                const int32_t *accepted_dev, const void *q,
                                const void *k, const void *v, const float *g,
                                const float *beta, float *state,
                                const int32_t *state_slots_dev, void *out,
                                void *stream);

/*
 * Front end of q and k: short convolution -> Swish -> L2 normalisation.
 *
 * "Kimi K3 technical FAQ" (Runpod guide), question "What is KDA, and why
 * does a serving engineer care?": queries and keys pass through a short
 * convolution, Swish and L2 normalisation before the recurrence.  The page
 * states neither the width nor the exact forms; this library reads them as,
 * for channel c = h*dk + i of token t,
 *
 *     z_t[c] = sum_{j=0}^{W-1} w[c][j] * x_{t-(W-1)+j}[c]
 *     a_t[c] = z_t[c] * sigmoid(z_t[c])
 *     y_t[h] = a_t[h] / sqrt(|a_t[h]|^2 + eps)      (|.| over the dk channels)
 *
 * a depthwise causal convolution along each sequence's own tokens (no bias;
 * tap W-1 weighs the current token), Swish with unit slope, and a per
 * (token, head) L2 normalisation.  q and k have their own taps and states.
 */
typedef struct {
    int32_t num_heads;   /* H                                               */
    int32_t dk;          /* channels per head: 16, 32, 64 or 128            */
    int32_t conv_width;  /* W, taps per channel: 1 .. 8                     */
    kda_dtype in_dtype;  /* dtype of xq, xk and of the convolution states   */
    kda_dtype out_dtype; /* dtype of q_out, k_out (bf16 feeds kda_prefill
                            and kda_decode directly)                        */
    float eps;           /* > 0 and finite                                  */
} kda_frontend_config;

/*
 * The front end over packed variable-length sequences (T = cu[num_seqs]
 * tokens, sequence b owning tokens [cu[b], cu[b+1])), q and k in one call:
 *   xq, xk   : [T, H, dk] in_dtype         raw (pre-convolution) q and k
 *   wq, wk   : [H*dk, W] fp32              taps, channel-major
 *   q_out, k_out : [T, H, dk] out_dtype    (written)
 * Convolution states, one row of W-1 inputs per slot, oldest first:
 *   conv_state_in_q/k  : [num_slots, W-1, H, dk] in_dtype, read: the inputs
 *                        that preceded each sequence; NULL = zero history
 *   conv_state_out_q/k : same layout (written): each sequence's last W-1
 *                        inputs (state rows fill in where a sequence is
 *                        shorter than W-1); NULL = not written.  May equal
 *                        the matching input pointer (in-place update); no
 *                        other overlap is allowed.
 *   state_slots_dev    : [num_seqs] int32 device array, sequence b's state
 *                        row, or NULL for row b; entries distinct and
 *                        < num_slots (not checked on the device).
 * num_slots is the number of rows of the state arrays (>= num_seqs when
 * state_slots_dev is NULL; unused when both states are NULL or W == 1).
 * A decode step is the call with cu = {0, 1, ..., num_seqs} and the states
 * updated in place.  Slots of sequences not in the call are not touched.
 * cu_seqlens_host and cu_seqlens_dev hold the same offsets: cu[0] == 0,
 * non-decreasing; empty sequences are allowed (their output state is their
 * input state, or zeros without one).
 * Alignment: x, out, taps and states 16 bytes; cu and slots 4 bytes.
 * Errors: KDA_ERR_INVALID_ARG (null required pointer, bad offsets, eps,
 * overlapping buffers, num_slots too small), KDA_ERR_UNSUPPORTED (dk, W or
 * dtype), KDA_ERR_ALIGNMENT, KDA_ERR_HIP.  num_seqs == 0 is a no-op.
 */
kda_status kda_qk_frontend(const kda_frontend_config *cfg, int32_t num_seqs,
                           const int32_t *cu_seqlens_host,
                           const int32_t *cu_seqlens_dev, const void *xq,
                           const void *xk, const float *wq, const float *wk,
                           const void *conv_state_in_q,
                           const void *conv_state_in_k,
                           void *conv_state_out_q, void *conv_state_out_k,
                           const int32_t *state_slots_dev, int32_t num_slots,
                           void *q_out, void *k_out, void *stream);

/*
 * Attention Residuals aggregation (block variant): a layer's input as a
 * softmax-weighted sum of earlier block outputs, plus the residual, then
 * RMSNorm, in one launch.
 *
 * "Kimi K3 technical FAQ" (Runpod guide), question "What does the
 * architecture actually look like?": each layer can attend over the
 * embedding plus the preceding block outputs through a learned pseudo-query;
 * K3 uses blocks of 12 layers (about 8 blocks).  "Day-0 vLLM support for
 * Kimi K3" (vLLM blog), section "Kimi K3's architecture, and how vLLM serves
 * it": the fused kernel computes the logits, the softmax across the previous
 * layers and the aggregation, and folds in the residual add and the output
 * RMSNorm.  The pages give no formula; read per token t, with sources s_m
 * (m < num_sources), pseudo-query w, residual x and RMSNorm weight gamma, as
 *
 *     p = softmax_m(logit_scale * <w, s_m,t>),   h = sum_m p_m s_m,t + x_t,
 *     y = h / sqrt(mean over the hidden channels of h^2 + eps) * gamma.
 */
typedef struct {
    int32_t hidden;      /* d: a multiple of 16, at most 8192 (4096 with
                            more than 9 bf16 or 10 fp32 sources)            */
    int32_t num_sources; /* 1 .. 16                                         */
    kda_dtype in_dtype;  /* sources and residual                            */
    kda_dtype out_dtype; /* h and y                                         */
    float logit_scale;   /* finite                                          */
    float eps;           /* > 0, finite                                     */
} kda_attnres_config;

/*
 *   sources_host : host array of num_sources device pointers, each [T, d]
 *                  in_dtype (separate buffers: the embedding and the block
 *                  outputs)
 *   residual     : [T, d] in_dtype, or NULL (no residual add)
 *   query        : [d] fp32 pseudo-query          gamma : [d] fp32 or NULL (1)
 *   h_out        : [T, d] out_dtype, or NULL (not written)
 *   y_out        : [T, d] out_dtype
 * The outputs may not overlap any input.  Device arrays 16-byte aligned.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED (d, num_sources, dtype),
 * KDA_ERR_ALIGNMENT, KDA_ERR_HIP.  num_tokens == 0 is a no-op.
 */
kda_status kda_attnres(const kda_attnres_config *cfg, int64_t num_tokens,
                       const void *const *sources_host, const void *residual,
                       const float *query, const float *gamma, void *h_out,
                       void *y_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
