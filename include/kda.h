/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) Kimi Delta Attention library.
 *
 * The operation (page "Kimi K3 把 3T 级模型、百万上下文和 Agent 训练接成一套系统",
 * ailearn.mscapital.top/kimi-k3.html, card "KDA 单头递归"), per sequence n and
 * head h, for tokens t in order:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                  (the query reads the updated state)
 *
 * with alpha_t = exp(g_t) per key channel.  S is dk x dv (row = key channel,
 * column = value channel), fixed in size whatever the sequence length (same
 * page, section "百万上下文的关键，不是让所有层都保存百万份 KV").  Nothing else
 * is applied: no query scaling, key normalisation, output gate or short
 * convolution.
 *
 * Input range (results are computed without overflow of any intermediate):
 *   - g in [-5, 0] (card "g ∈ (-5, 0)"); outside it intermediate decay factors
 *     may overflow and the result is unspecified.
 *   - fp32 q/k/v: any finite q, k, v and beta whose state stays in fp32 range.
 *   - bf16 q/k/v (the contractions run on fp16 MFMA operands with exact
 *     power-of-two scales): in addition |q_c|, |k_c| <= 1024 per channel, and
 *     for tokens r, i of one 32-token chunk ||q_r|| ||k_i|| <= 32768 and
 *     |beta_r| ||k_r|| ||k_i|| <= 32768.  Chunks whose decay-scaled key
 *     columns would leave fp16 range (large keys under strong decay) are
 *     detected per chunk and evaluated with 16-token references whose factors
 *     are all <= 1, so no key magnitude within these bounds overflows.
 *   - beta has no range of its own.  Each step is non-expansive when
 *     beta ||k||^2 lies in [0, 2]; outside that interval the recurrence itself
 *     amplifies rounding (and, over long runs, the state can leave fp32 range).
 *
 * Conventions for every call:
 *   - Device pointers are on the current HIP device, dense and row-major as
 *     documented; the caller owns every buffer.  No call allocates device
 *     memory.  The library's global state is a per-device record (atomic
 *     bits) that each kernel's LDS limit has been raised; for
 *     kda_prefill_cp_noalloc only, one static device array per GPU
 *     (KDA_STATIC_SCRATCH_BYTES) with its cached address; and, for
 *     kda_backward only, one stream and three events per GPU (see there).
 *     Calls are thread-safe, except that kda_prefill_cp_noalloc calls
 *     overlapping on one GPU share that array.
 *   - Calls are asynchronous on `stream` (0 = the null stream) and never
 *     synchronise (except the opt-in KDA_VALIDATE=1 check of cu_seqlens,
 *     below).  Argument errors are returned before any HIP call; a launch
 *     failure returns KDA_ERR_LAUNCH; device faults surface at the caller's
 *     next synchronisation of `stream`.
 *   - v1 supports dk = dv = 128 only (other sizes: KDA_ERR_UNSUPPORTED).
 *   - Arithmetic: q/k/v/out in `dtype`; g, beta and states fp32; all
 *     accumulation and the carried state are fp32.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *kda_stream_t; /* identical to hipStream_t */

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad dtype, overflowing sizes */
    KDA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. dk != 128) */
    KDA_ERR_LAUNCH = 3,      /* the HIP launch itself failed */
    KDA_ERR_SCRATCH = 4      /* kda_prefill_cp_noalloc: the problem needs more
                                workspace than KDA_STATIC_SCRATCH_BYTES */
} kda_status;

/* Size of the static device scratch behind kda_prefill_cp_noalloc: 256 MiB,
 * held on every GPU the library runs on from the first load of its code object
 * on that GPU until the process ends. */
#define KDA_STATIC_SCRATCH_BYTES (256u * 1024u * 1024u)

typedef enum {
    KDA_F32 = 0,  /* q, k, v, out are fp32 */
    KDA_BF16 = 1  /* q, k, v, out are bf16 (round-to-nearest-even on output) */
} kda_dtype;

/*
 * kda_prefill -- run the recurrence over packed variable-length sequences.
 *
 *   q, k          [total_tokens, num_heads, dk]   dtype
 *   v             [total_tokens, num_heads, dv]   dtype
 *   g             [total_tokens, num_heads, dk]   fp32, log-decay (alpha = exp(g))
 *   beta          [total_tokens, num_heads]       fp32, write strength
 *   initial_state [num_seqs, num_heads, dk, dv]   fp32, or NULL for zeros
 *   cu_seqlens    [num_seqs + 1]                  int32, DEVICE memory:
 *                 cu[0] = 0, non-decreasing, cu[num_seqs] <= total_tokens.
 *                 Sequence n owns tokens [cu[n], cu[n+1]).  It is not read on
 *                 the host; entries outside [0, total_tokens] are clamped on
 *                 the device (memory-safe, result for that sequence unspecified).
 *                 With KDA_VALIDATE=1 in the environment (read at the first
 *                 call), every entry point that takes cu_seqlens copies it to
 *                 the host first, synchronising `stream` (so not under graph
 *                 capture; kda_prefill_cp_noalloc skips it), and returns
 *                 KDA_ERR_INVALID_ARG when these rules do not hold.
 *   out           [total_tokens, num_heads, dv]   dtype; rows of tokens owned
 *                 by a sequence are written, other rows are left untouched.
 *   final_state   [num_seqs, num_heads, dk, dv]   fp32, or NULL (not written).
 *                 final_state == initial_state is allowed (in-place update of
 *                 the carried state); any other overlap is undefined.
 *
 * An empty sequence writes no output and final_state[n] = initial_state[n]
 * (zeros if NULL).  Continuation: passing one call's final_state as the next
 * call's initial_state over the following tokens equals one call over all of
 * them, which is how a state is restored at a token boundary (page section
 * "目标模型太大，缓存和草稿都必须理解 KDA").
 */
kda_status kda_prefill(const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       const float *initial_state, const int32_t *cu_seqlens,
                       int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                       int32_t dk, int32_t dv, kda_dtype dtype,
                       void *out, float *final_state, kda_stream_t stream);

/*
 * kda_prefill_ex -- kda_prefill with explicit kernel tiling (tests, tuning).
 *   chunk    tokens per chunk: 32 or 64 for bf16, 16 or 32 for fp32; 0 = 32
 *   dv_block value columns per workgroup: 16, 32, 64 or 128 (at least 32 for
 *            64-token bf16 chunks); 0 = automatic
 * Any tiling gives the same result up to fp32 rounding order.  Other values
 * return KDA_ERR_UNSUPPORTED.
 */
kda_status kda_prefill_ex(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                          int32_t dk, int32_t dv, kda_dtype dtype,
                          void *out, float *final_state,
                          int32_t chunk, int32_t dv_block, kda_stream_t stream);

/*
 * kda_prefill_snapshots -- kda_prefill that also keeps copies of the state
 * at regular token boundaries, so that a prefix cache can restore the KDA
 * state of any of those prefixes (page ailearn.mscapital.top/kimi-k3.html,
 * section "目标模型太大，缓存和草稿都必须理解 KDA": the prefix cache restores the
 * recurrent state at a token boundary).
 *   snap_every  tokens between snapshots, a positive multiple of 32 (the
 *               chunk); other multiples return KDA_ERR_UNSUPPORTED
 *   max_snaps   snapshots kept per sequence (> 0)
 *   snapshots   [num_seqs, max_snaps, num_heads, dk, dv] fp32, DEVICE:
 *               snapshots[n][j] = the state after the first (j + 1) *
 *               snap_every tokens of sequence n, for every j < max_snaps with
 *               (j + 1) * snap_every <= its length; other entries are left
 *               untouched.
 * Other arguments and conventions as kda_prefill; snapshot j equals, bit for
 * bit, the final state of kda_prefill over that prefix alone.
 */
kda_status kda_prefill_snapshots(const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 const float *initial_state, const int32_t *cu_seqlens,
                                 int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                 int32_t dk, int32_t dv, kda_dtype dtype,
                                 void *out, float *final_state,
                                 int32_t snap_every, int32_t max_snaps, float *snapshots,
                                 kda_stream_t stream);

/*
 * kda_prefill_cp -- kda_prefill with context parallelism inside the device.
 * Each sequence is split into segments of seg_len tokens that
 * run side by side: every segment but a sequence's last is first run from a
 * zero state to give its end state S^0 and its transition M (S_end = M S_in
 * + S^0, the recurrence being affine in the entering state); the segments'
 * entering states are then chained, S_in(s+1) = M_s S_in(s) + S^0_s; finally
 * every segment is run from its entering state for the outputs.  This is the
 * fixed-size-state-fragment scheme of page ailearn.mscapital.top/kimi-k3.html,
 * card "传固定状态片段" (local cumulative transform and zero-state fragment,
 * then a prefix combination), applied across the compute units of one GPU.
 * Results equal kda_prefill up to rounding order; for bf16 inputs the
 * chaining's products M_s S_in run as three bf16 MFMA terms of the values
 * split into high and low halves (about 2^-16 relative error per product).
 * For fp32 inputs, when there are many (segment, head) pairs and segments of
 * at least 1,024 tokens, the zero-state runs and the chaining use summary
 * units of a quarter (or half) segment instead of whole segments, so that they
 * pack the compute units evenly; the outputs still run whole segments.
 * For bf16 inputs, when there are more (segment, head) pairs than compute
 * units, a zero-state run over a segment longer than 36 chunks of 32 tokens
 * first covers the segment's last 36 chunks only.  When the transition
 * over them comes out exactly zero in fp32 (gates that decay: the state
 * entering those chunks cannot reach their end above the smallest fp32
 * subnormal), that run is the segment's S^0, equal to the full run's up to
 * fp32 rounding, and M is zero; otherwise the whole segment is run.  This holds for
 * any inputs: the test is made on the computed transition, not assumed.
 *
 *   seg_len    > 0: tokens per segment, a multiple of 32, counted from each
 *              sequence's start.
 *              < 0: pieces of -seg_len tokens (a multiple of 32).  The 32-token chunks of
 *              all sequences, numbered in packed order, are cut into pieces
 *              of -seg_len / 32 chunks, and every sequence into its parts in
 *              those pieces: a segment ends where a piece or its sequence
 *              ends.  One workgroup per (piece, head) runs its piece's
 *              segments in turn, so every output walk covers the same number
 *              of chunks however the sequence lengths fall.  Zero-state runs
 *              and chaining then use these segments as their units.
 *              0 = automatic: for bf16 inputs, at most 256 sequences and
 *              total_tokens * num_heads / 256 above 32,768, equal pieces,
 *              max(1, 512 / num_heads) per head (two workgroups per compute
 *              unit), each of ceil(chunks / pieces) chunks; otherwise
 *              segments of total_tokens * num_heads / 256 tokens, clamped to
 *              [256, 32768] and rounded up to a multiple of 32.
 *   workspace  device memory of at least kda_prefill_cp_workspace_size(...)
 *              bytes, 256-byte aligned, owned by the caller, contents
 *              ignored on entry; calls that share one workspace must not
 *              overlap in time.
 * Other arguments, conventions and errors as kda_prefill (final_state ==
 * initial_state is allowed).  KDA_ERR_INVALID_ARG if the workspace is
 * missing, misaligned or too small.
 */
size_t kda_prefill_cp_workspace_size(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                     int32_t dk, int32_t dv, kda_dtype dtype, int32_t seg_len);

kda_status kda_prefill_cp(const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                          int32_t dk, int32_t dv, kda_dtype dtype,
                          void *out, float *final_state, int32_t seg_len,
                          void *workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_prefill_cp_noalloc -- kda_prefill_cp for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the workspace is the library's static device array
 * of KDA_STATIC_SCRATCH_BYTES instead of a caller-owned buffer, and the call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 * The caller still owns every input and output.
 *   - Limit: the workspace kda_prefill_cp_workspace_size(...) reports for the
 *     same arguments must not exceed KDA_STATIC_SCRATCH_BYTES (for example
 *     4,096 tokens x 8 heads in bf16 need 56 MiB); larger problems return
 *     KDA_ERR_SCRATCH before any HIP call.
 *   - The array is per GPU and shared by every call on that GPU: calls that
 *     overlap in time on one GPU (other streams, other threads) race on it and
 *     give undefined results.  Serialise them, or use kda_prefill_cp.
 *   - The array keeps the last call's contents; the call needs none of them
 *     (every part of the workspace it reads is written earlier in the call).
 * Arguments, results and other errors as kda_prefill_cp.
 */
kda_status kda_prefill_cp_noalloc(const void *q, const void *k, const void *v,
                                  const float *g, const float *beta,
                                  const float *initial_state, const int32_t *cu_seqlens,
                                  int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                  int32_t dk, int32_t dv, kda_dtype dtype,
                                  void *out, float *final_state, int32_t seg_len,
                                  kda_stream_t stream);

/*
 * kda_decode_step -- one new token per (sequence, head), state updated in place
 * (the same recurrence step; page card "KDA 单头递归").
 *
 *   q, k          [num_seqs, num_heads, dk]       dtype
 *   v             [num_seqs, num_heads, dv]       dtype
 *   g             [num_seqs, num_heads, dk]       fp32
 *   beta          [num_seqs, num_heads]           fp32
 *   state_inout   [num_seqs, num_heads, dk, dv]   fp32, read then overwritten
 *   out           [num_seqs, num_heads, dv]       dtype
 * Each (sequence, head) state is read once and written once.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *state_inout,
                           int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv,
                           kda_dtype dtype, void *out, kda_stream_t stream);

/*
 * kda_decode_tokens -- a few consecutive tokens per (sequence, head) with the
 * state held on chip: it is read once and written at most once, so k tokens
 * cost about one state round trip instead of k.  This is the speculative
 * decoding path of page ailearn.mscapital.top/kimi-k3.html, section
 * "目标模型太大，缓存和草稿都必须理解 KDA": the projected inputs of the draft
 * tokens are cached, the accepted ones are replayed on chip, and a rejected
 * draft is rolled back by not committing its state.  Typical use:
 *   verify:  state_out = NULL, num_tokens = NULL  -> out for every draft token,
 *            the committed state is untouched;
 *   replay:  num_tokens = accepted counts, state_out = state_in, out = NULL
 *            -> the state advanced over the accepted prefix only.
 *
 *   q, k, g       [total_tokens, num_heads, dk]   dtype / fp32
 *   v             [total_tokens, num_heads, dv]   dtype
 *   beta          [total_tokens, num_heads]       fp32
 *   cu_seqlens    [num_seqs + 1]  int32, DEVICE: sequence n owns tokens
 *                 [cu[n], cu[n+1]) (clamped as for kda_prefill)
 *   num_tokens    [num_seqs]      int32, DEVICE, or NULL: process only the
 *                 first min(max(num_tokens[n], 0), cu[n+1] - cu[n]) tokens
 *   state_in      [num_seqs, num_heads, dk, dv]   fp32
 *   state_out     same shape, or NULL (not written); may equal state_in
 *   out           [total_tokens, num_heads, dv]   dtype, or NULL; rows of the
 *                 processed tokens are written, other rows are left untouched
 * Per token the arithmetic is that of kda_decode_step (bitwise identical to
 * applying kda_decode_step token by token).  Intended for a few tokens per
 * sequence; long runs belong to kda_prefill.
 */
kda_status kda_decode_tokens(const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const int32_t *cu_seqlens, const int32_t *num_tokens,
                             const float *state_in, float *state_out,
                             int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                             int32_t dk, int32_t dv, kda_dtype dtype,
                             void *out, kda_stream_t stream);

/*
 * kda_backward -- gradients for training: given dL/d(out) and dL/d(final
 * state) of a scalar loss L, the gradients with respect to q, k, v, g, beta
 * and the initial state, by the chain rule through the recurrence of card
 * "KDA 单头递归" (page ailearn.mscapital.top/kimi-k3.html), in chunk form (32
 * tokens).  Sequences are cut into segments that run side by side, as in
 * kda_prefill_cp (card "传固定状态片段"): the gradient of the state is linear
 * in itself, so each segment's gradient summary combines, in reverse segment
 * order, into the gradient entering every segment; a segment's gradient
 * transition is the transpose of its forward transition.  The forward states
 * at chunk starts and the state gradients at chunk ends are computed by two
 * strands of launches that run side by side: the second runs on a per-device
 * stream of the library (created on first use, default priority, kept until
 * the process ends), forked from `stream` and joined back into it with events,
 * so the call stays ordered on `stream` (also under stream capture).  A final
 * chunk-parallel pass turns each chunk's states and inputs into its gradients.
 * For bf16 inputs with segments of more than 36 chunks, a segment whose
 * forward transition over its first 36 chunks comes out exactly zero in fp32
 * has its gradient summary formed from those chunks alone (nothing later in
 * the segment reaches its start above the smallest fp32 subnormal); the test
 * is made on the computed transition, so inputs that do not decay take the
 * full walk.  Precision as kda_prefill: bf16 inputs run the contractions on
 * fp16 MFMA operands with exact power-of-two scales, fp32 inputs on fp32 MFMA.
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens, dtype: as kda_prefill
 *   dout          [total_tokens, num_heads, dv]   dtype
 *   dfinal        [num_seqs, num_heads, dk, dv]   fp32, or NULL (zero)
 *   dq, dk, dg    [total_tokens, num_heads, dk]   fp32, written
 *   dv            [total_tokens, num_heads, dv]   fp32, written
 *   dbeta         [total_tokens, num_heads]       fp32, written
 *   dinit         [num_seqs, num_heads, dk, dv]   fp32, or NULL (not written)
 *   workspace     device memory of at least kda_backward_workspace_size(...)
 *                 bytes (for the same sizes and dtype), 256-byte aligned, owned
 *                 by the caller (segment plans, chunk and gradient images, the
 *                 states at every chunk start and state gradients at every
 *                 chunk end, each chunk's intermediate products, segment
 *                 summaries and entering states); calls sharing it must not
 *                 overlap
 * Rows of tokens owned by a sequence are written; others are left untouched.
 * Gradients are fp32 whatever the input dtype.  Deterministic: no result is
 * accumulated across workgroups, and every sum has a fixed order.
 */
size_t kda_backward_workspace_size(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                   int32_t dk, int32_t dv, kda_dtype dtype);

kda_status kda_backward(const void *q, const void *k, const void *v,
                        const float *g, const float *beta,
                        const float *initial_state, const int32_t *cu_seqlens,
                        int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                        int32_t dk, int32_t dv, kda_dtype dtype,
                        const void *dout, const float *dfinal,
                        float *dq, float *dk_out, float *dv_out, float *dg, float *dbeta,
                        float *dinit, void *workspace, size_t workspace_bytes,
                        kda_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *kda_status_string(kda_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
