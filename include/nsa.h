/*
 * nsa.h -- C ABI of libnsa, a Native Sparse Attention (NSA) forward library
 * for one AMD Instinct MI355X (gfx950).
 *
 * The method: attention split into three parallel branches whose outputs are
 * merged by per-head gates -- a compressed branch (coarse, over block
 * summaries of the keys and values), a selected branch (fine-grained, over the
 * key blocks a query ranks highest) and a sliding-window branch (the most
 * recent tokens). NSA how-to (qwbw.cn/news/106443), section 1; its
 * parameters are the [model.nsa] fields of section 3 of the same page:
 * compress_block_size, select_block_size, select_top_k, sliding_window and a
 * learned gate (here: gate values passed in as a tensor).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates device memory, never frees, keeps no state between calls
 *    and never synchronises. Scratch memory is the caller's `workspace`, sized
 *    by the matching *_workspace_bytes call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls enqueue their kernels on it and return; results are ready when the
 *    stream reaches that point.
 *  - Arguments are validated on the host before anything is enqueued. On an
 *    argument error (NSA_ERR_INVALID_ARGUMENT, NSA_ERR_UNSUPPORTED,
 *    NSA_ERR_WORKSPACE_TOO_SMALL) nothing is launched and nothing is
 *    written. Kernel attributes are set before the first launch, so a HIP
 *    failure there also launches nothing; NSA_ERR_HIP from a later launch or
 *    event record means the kernels before it are already enqueued and may
 *    have written their outputs or the workspace. nsa_last_error() holds a
 *    message for any failing call (per calling thread). There is no silent
 *    fallback (no dense path, no clamping).
 *  - Strides are in ELEMENTS; the head dimension is always contiguous.
 *  - Element types: in_dtype applies to q, k, v, caches and gates; out_dtype
 *    to out. Supported: (bf16 in, bf16 out), (bf16 in, f32 out),
 *    (f32 in, f32 out). Block summaries and matrix products use the input
 *    type as operands with fp32 accumulation; softmax, block scores, top-k and
 *    the gate combination run in fp32.
 *  - Supported geometry: head_dim in {64, 128}; n_q_heads a multiple of
 *    n_kv_heads with at most 16 query heads per KV head; 1 <= select_top_k
 *    <= 64; sliding_window >= 1; any seqlen >= 1 (a trailing partial block is
 *    allowed). Block sizes: the forward prefill entry points take any
 *    compress_block_size l <= select_block_size l' with l' a multiple of 32
 *    and select_top_k * l' <= 4096 (see nsa_fwd_prefill_general for the
 *    compressed-to-selection mapping); decode, the backward pass and the
 *    prefill that keeps the selected branch need l == l' == 64.
 *  - Query head h reads KV head h / (n_q_heads / n_kv_heads).
 *  - Calls are reentrant; two calls that share a workspace or an output
 *    buffer must be ordered by the caller.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NSA_OK = 0,
  NSA_ERR_INVALID_ARGUMENT = 1,    /* null pointer, bad size, bad stride, ... */
  NSA_ERR_UNSUPPORTED = 2,         /* valid NSA geometry this library does not run */
  NSA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the required size */
  NSA_ERR_HIP = 4                  /* a HIP launch reported an error */
} nsa_status_t;

typedef enum { NSA_F32 = 0, NSA_BF16 = 1 } nsa_dtype_t;

typedef enum {
  NSA_IDX_COMPUTE = 0, /* select blocks; write them to idx when idx != NULL */
  NSA_IDX_INJECT = 1   /* read the selection from idx; no selection is run */
} nsa_idx_mode_t;

/* The [model.nsa] parameters of the NSA how-to (qwbw.cn/news/106443), section 3. */
typedef struct {
  int32_t compress_block_size; /* l: tokens per compressed block; stride l unless nsa_general_t says otherwise */
  int32_t select_block_size;   /* l': tokens per selectable block, l' >= l */
  int32_t select_top_k;        /* n: blocks each query attends to, its own block included */
  int32_t sliding_window;      /* w: window length in tokens, the query itself included */
  float softmax_scale;         /* <= 0 selects 1/sqrt(head_dim); used by all three branches */
} nsa_params_t;

/*
 * Prefill: every position t of every sequence is a query that attends
 * causally within its own sequence.
 *   q     [B, L, Hq, D]  strides q_stride  = (b, t, head)
 *   k, v  [B, L, G,  D]  strides k_stride, v_stride = (b, t, kv head)
 *   gates [B, L, Hq, 3]  strides g_stride  = (b, t, head); the three values
 *                        (compressed, selected, window) are contiguous and are
 *                        used as given (already through their sigmoid).
 *   out   [B, L, Hq, D]  strides o_stride  = (b, t, head)
 *   idx   [B, L, G, n]   int32, dense row-major (no strides).
 */
typedef struct {
  int32_t batch, seqlen, n_q_heads, n_kv_heads, head_dim;
  nsa_dtype_t in_dtype, out_dtype;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t g_stride[3];
  int64_t o_stride[3];
} nsa_prefill_desc_t;

/*
 * Decode: one new query per sequence b, at position seqlens[b]-1, whose K/V
 * are already in the caches.
 *   q        [B, Hq, D]          strides q_stride  = (b, head)
 *   k_cache, v_cache [B, G, max_seqlen, D]  strides (b, kv head, t)
 *   kc_cache, vc_cache [B, G, max_blocks, D] strides (b, kv head, j): entry j
 *            holds the mean of cache tokens [j*l, j*l+l) (see nsa_compress_kv);
 *            entries j < seqlens[b]/l are read, as given.
 *   seqlens  [B] int32 DEVICE array; each value must lie in [1, max_seqlen].
 *            A sequence with a value outside that range gets out = 0 and idx
 *            = -1 and no cache entry of it is read.
 *   gates    [B, Hq, 3]          strides g_stride = (b, head)
 *   out      [B, Hq, D]          strides o_stride = (b, head)
 *   idx      [B, G, n]           int32, dense row-major.
 */
typedef struct {
  int32_t batch, max_seqlen, max_blocks, n_q_heads, n_kv_heads, head_dim;
  nsa_dtype_t in_dtype, out_dtype;
  int64_t q_stride[2];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t kc_stride[3];
  int64_t vc_stride[3];
  int64_t g_stride[2];
  int64_t o_stride[2];
} nsa_decode_desc_t;

/* Required workspace size in bytes for a prefill / decode call with these
 * arguments (idx presence does not matter: the bound covers both).
 * Returns NSA_OK and writes *bytes, or an error status (see conventions). */
nsa_status_t nsa_prefill_workspace_bytes(const nsa_prefill_desc_t* desc,
                                         const nsa_params_t* params, size_t* bytes);
nsa_status_t nsa_decode_workspace_bytes(const nsa_decode_desc_t* desc,
                                        const nsa_params_t* params, size_t* bytes);

/*
 * NSA forward over whole sequences.
 *
 * Computes, for each (b, t, head h in KV group g):
 *   compressed: softmax attention over the means of the key/value blocks
 *               [j*l, j*l+l) that lie wholly at or before t (none -> 0);
 *   selection:  block scores = compressed-attention probabilities summed over
 *               the query heads of group g; the chosen set is the own block
 *               t/l plus the n-1 best-scoring blocks before it (ties to the
 *               lower index; fewer candidates -> all of them). The set is
 *               shared by the group. The score -> top-k -> gather dataflow
 *               is the selector described in the NSA factory write-up
 *               (chencunli.com, "DeepSeek NSA on the Siemens 840D manual"),
 *               section "What dynamic sparsity actually sparsifies";
 *   selected:   softmax attention over the tokens of the chosen blocks at or
 *               before t;
 *   window:     softmax attention over tokens [max(0, t-w+1), t];
 *   out = g_cmp*compressed + g_slc*selected + g_win*window.
 *
 * idx_mode NSA_IDX_COMPUTE: the selection is computed; if idx != NULL it is
 *   written there, each row ascending and padded with -1.
 * idx_mode NSA_IDX_INJECT: idx (required) supplies the selection. Entries
 *   outside [0, t/l] are skipped and repeated entries count once (the
 *   selection is a set of blocks); a row with no usable entry gives a
 *   selected-branch output of 0.
 * With a float32 output, `out` also holds the window + compressed part of
 * each row while the call runs; with a bf16 output that part is kept in
 * float32 in the workspace, so every output element is rounded to bf16
 * once, from the float32 sum of the three gated branches.
 */
nsa_status_t nsa_fwd_prefill(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                             const void* q, const void* k, const void* v, const void* gates,
                             void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * General geometry of the prefill (the [model.nsa] fields of the NSA how-to,
 * qwbw.cn/news/106443, section 3, list compress_block_size and
 * select_block_size separately; the NSA factory write-up, chencunli.com,
 * section "What dynamic sparsity actually sparsifies", compresses each block
 * into one representation with a learned linear map of the flattened block,
 * and the how-to's gate_type is "learned"):
 *   compress_stride d, 1 <= d <= l: compressed block i covers tokens
 *       [i*d, i*d + l) (d < l: overlapping blocks); the blocks that lie wholly
 *       inside the sequence exist, and block i is visible to query t when
 *       i*d + l - 1 <= t;
 *   wk, bk, wv, bv (all or none; NULL: block means): the learned compressor,
 *       kc_i[o] = sum_{p < l, c < D} wk[o][p][c] * k[i*d + p][c] + bk[o] (and
 *       the same for v). wk, wv: [D][l][D] contiguous, 16-byte aligned; bk,
 *       bv: [D]; all in in_dtype;
 *   gate_w, gate_b (both or none; NULL: the gates argument is used): the gate
 *       layer gate[t][h][c] = sigmoid(q[t][h] . gate_w[h][:, c] +
 *       gate_b[h][c]) for the branches c = (compressed, selected, window),
 *       gate_w [Hq][D][3], gate_b [Hq][3] contiguous in in_dtype; the gates
 *       are computed in float32 into the workspace and the gates argument may
 *       be NULL.
 * Selection blocks hold l' = select_block_size tokens; the own block is
 * t / l'. A selection block's score is the compressed-attention mass on its
 * tokens, each compressed block's probability spread evenly over its l tokens
 * (sum over compressed blocks i of p_i * |tokens of i in the block| / l);
 * with d = l = l' this is the plain block score. All else as nsa_fwd_prefill
 * (idx rows hold selection-block indices). The caller owns the weights; they
 * must stay valid until the call completes on the stream.
 */
typedef struct {
  int32_t compress_stride;
  const void* wk;
  const void* bk;
  const void* wv;
  const void* bv;
  const void* gate_w;
  const void* gate_b;
} nsa_general_t;

/* Workspace bytes of nsa_fwd_prefill_general (general may be NULL: the plain
 * stride and block means, gates given). */
nsa_status_t nsa_prefill_general_workspace_bytes(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                                 const nsa_general_t* general, size_t* bytes);
/* nsa_fwd_prefill with the general geometry above; errors as for
 * nsa_fwd_prefill, plus NSA_ERR_INVALID_ARGUMENT for a stride outside [1, l],
 * an incomplete weight set or a misaligned weight. */
nsa_status_t nsa_fwd_prefill_general(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                     const nsa_general_t* general, const void* q, const void* k, const void* v,
                                     const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * nsa_fwd_prefill that also keeps what the backward pass needs of the
 * selected branch (the branch whose keys are gathered per token): its own
 * output o_slc [B, L, Hq, D] (before the gate, contiguous, out_dtype,
 * 16-byte aligned) and the natural-log log-sum-exp of its scaled logits
 * lse_slc [B, L, Hq] (float32, contiguous; -inf where the token has no
 * usable block, whose output is then 0). Both caller-owned and fully
 * written; out and idx are exactly those of nsa_fwd_prefill. Pass them to
 * nsa_bwd_prefill_saved. Errors as for nsa_fwd_prefill, plus
 * NSA_ERR_INVALID_ARGUMENT for a NULL or misaligned o_slc / lse_slc.
 */
nsa_status_t nsa_fwd_prefill_save(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                                  const void* k, const void* v, const void* gates, void* out, int32_t* idx,
                                  nsa_idx_mode_t idx_mode, void* o_slc, float* lse_slc, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Chunked prefill: the NSA forward of query positions [q_offset, seqlen)
 * only, each against the whole context [0, its position] - the prefill half
 * of serving long prompts in pieces, as with the continuous batching switch
 * of the NSA how-to's config (qwbw.cn/news/106443, section 3). desc->seqlen
 * is the context length: k and v hold all seqlen positions as for
 * nsa_fwd_prefill, while q, gates, out and idx hold only the
 * seqlen - q_offset query rows (their strides in desc; idx shaped
 * [B, seqlen - q_offset, G, n]). Every row equals the same row of an
 * nsa_fwd_prefill over the whole context. 0 <= q_offset <= seqlen, else
 * NSA_ERR_INVALID_ARGUMENT; q_offset == seqlen does nothing. The workspace
 * is sized by nsa_prefill_workspace_bytes for the same desc (the context
 * length decides it). The K/V re-layout covers the whole context on every
 * call.
 */
nsa_status_t nsa_fwd_prefill_chunk(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                   int32_t q_offset, const void* q, const void* k, const void* v,
                                   const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Varlen prefill: sequences of different lengths in one call, each with its
 * own query range - batching prompts of mixed lengths, and chunks of them,
 * as the continuous batching switch of the NSA how-to's config (section 3)
 * asks. desc->seqlen is the row capacity of k and v ([B, seqlen, G, D]);
 * seq_lens[b] (device, required) is sequence b's context length and
 * q_offsets[b] (device; NULL means 0) its first query position. Its queries
 * are positions [q_offsets[b], min(seq_lens[b], q_offsets[b] + query_rows)),
 * held in rows 0, 1, ... of q, gates, out and idx, which have query_rows
 * rows per sequence (their strides in desc; idx [B, query_rows, G, n]).
 * Rows past a sequence's queries are not written, and a sequence with
 * seq_lens[b] outside [0, seqlen] or q_offsets[b] outside [0, seq_lens[b]]
 * gets no rows (nothing is written for it). Every row equals the same row of
 * an nsa_fwd_prefill of that sequence alone. 0 <= query_rows <= seqlen, else
 * NSA_ERR_INVALID_ARGUMENT; the workspace is sized by
 * nsa_prefill_workspace_bytes for the same desc.
 */
nsa_status_t nsa_fwd_prefill_varlen(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                    const int32_t* seq_lens, const int32_t* q_offsets,
                                    int32_t query_rows, const void* q, const void* k, const void* v,
                                    const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * NSA forward for one new token per sequence over a KV cache and a block
 * cache (the decode phase, measured apart from prefill as the NSA how-to
 * advises, section 5). Same arithmetic as one prefill row at t = seqlens[b]-1;
 * idx/idx_mode as for prefill, idx shaped [B, G, n].
 */
nsa_status_t nsa_fwd_decode(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                            const void* q, const void* k_cache, const void* v_cache,
                            const void* kc_cache, const void* vc_cache, const int32_t* seqlens,
                            const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * nsa_fwd_decode with the general geometry of nsa_fwd_prefill_general (the
 * [model.nsa] fields of the NSA how-to, qwbw.cn/news/106443, section 3, list
 * compress_block_size and select_block_size separately, and its gate_type
 * is "learned"): compress_stride d (1 <= d <= l), selection blocks of
 * l' = select_block_size tokens (a multiple of 32, l <= l', top_k * l' <=
 * 4096) scored by the compressed-attention mass on their tokens, and
 * optionally the gate layer gate_w, gate_b (then `gates` may be NULL; the
 * gates are computed in float32 into the workspace). kc_cache / vc_cache hold
 * the representations of the compressed blocks [i*d, i*d + l) that lie wholly
 * inside each sequence, used as given: max_blocks must be at least
 * (max_seqlen - l) / d + 1, and how the representations were made (block
 * means, a learned compressor) does not matter here, so wk, bk, wv, bv are
 * not used. The query at position t = seqlens[b] - 1 sees compressed blocks
 * i with i*d + l - 1 <= t; its own selection block is t / l'; idx holds
 * selection-block indices. Workspace from nsa_decode_general_workspace_bytes
 * (general may be NULL: the plain stride, gates given). Errors as for
 * nsa_fwd_decode, plus NSA_ERR_INVALID_ARGUMENT for a stride outside [1, l]
 * or a gate layer with one of its two arrays missing.
 */
nsa_status_t nsa_decode_general_workspace_bytes(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                                const nsa_general_t* general, size_t* bytes);
nsa_status_t nsa_fwd_decode_general(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                    const nsa_general_t* general, const void* q, const void* k_cache,
                                    const void* v_cache, const void* kc_cache, const void* vc_cache,
                                    const int32_t* seqlens, const void* gates, void* out, int32_t* idx,
                                    nsa_idx_mode_t idx_mode, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * nsa_fwd_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the scratch the decode kernel needs (the selection
 * when idx is NULL, and the compressed logits when they do not fit in LDS) is
 * a 40 MiB device array inside the library, one per GPU, held until the
 * process ends (enough for 64 sequences x 4 KV heads of up to 131072 tokens
 * in bf16). A call whose nsa_decode_workspace_bytes exceeds 40 MiB
 * returns NSA_ERR_WORKSPACE_TOO_SMALL and launches nothing. Nothing in the
 * scratch needs to start at zero and no call allocates. Every call on one GPU
 * shares that GPU's scratch, so two calls that may run at the same time on
 * one GPU (different streams, or one stream and graph replays) race: order
 * them. Otherwise as nsa_fwd_decode, with the same results.
 */
nsa_status_t nsa_fwd_decode_noalloc(const nsa_decode_desc_t* desc, const nsa_params_t* params, const void* q,
                                    const void* k_cache, const void* v_cache, const void* kc_cache,
                                    const void* vc_cache, const int32_t* seqlens, const void* gates, void* out,
                                    int32_t* idx, nsa_idx_mode_t idx_mode, void* stream);

/*
 * Block compression, the step that turns each key/value block into one
 * compressed representation (NSA factory write-up, chencunli.com, "DeepSeek
 * NSA on the Siemens 840D manual", section "What dynamic sparsity actually
 * sparsifies"; block size: compress_block_size of the NSA how-to,
 * qwbw.cn/news/106443, section 3). The pages call that step learnable; here,
 * as in the prefill, it is the plain mean of the block.
 * Used by both phases: kc[b, g, j] = mean of k[b, g, t] over
 * t in [j*block_size, (j+1)*block_size), for j < n_tokens / block_size (only
 * complete blocks), and the same for v -> vc. Summation in fp32, one rounding
 * to dtype. k, v are [B, G, n_tokens, D] with strides (b, kv head, t); kc, vc
 * [B, G, n_tokens/block_size, D] with strides (b, kv head, j). block_size must
 * be 64. Writes nothing when n_tokens < block_size.
 */
nsa_status_t nsa_compress_kv(int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                             int32_t head_dim, nsa_dtype_t dtype, int32_t block_size,
                             const void* k, const int64_t k_stride[3],
                             const void* v, const int64_t v_stride[3],
                             void* kc, const int64_t kc_stride[3],
                             void* vc, const int64_t vc_stride[3], void* stream);

/*
 * Timed variants, for per-kernel measurement. Identical to nsa_fwd_prefill /
 * nsa_fwd_decode, and additionally record caller-created hipEvent_t handles
 * (passed as void*) on the stream: before each of the call's kernels and
 * after the last one. Prefill runs 3 kernels (block compression + re-layout;
 * compressed branch + block selection; selected + window branches + gate
 * combination), so stage_events holds 4 events; decode runs 1 kernel
 * (all three branches, selection and combination), so it holds 2, which the
 * kernel's dispatch itself records at the kernel's start and end (the
 * interval excludes the launch latency). A NULL array or entry is
 * NSA_ERR_INVALID_ARGUMENT.
 */
nsa_status_t nsa_fwd_prefill_timed(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                   const void* q, const void* k, const void* v, const void* gates,
                                   void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* stage_events);
nsa_status_t nsa_fwd_decode_timed(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  const void* kc_cache, const void* vc_cache,
                                  const int32_t* seqlens, const void* gates, void* out,
                                  int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace,
                                  size_t workspace_bytes, void* stream, void* const* stage_events);

/*
 * Backward pass of the prefill: the gradients of sum(out * dout) with respect
 * to q, k, v and gates, for the block selection `idx` held fixed (the top-k
 * choice is piecewise constant, so it carries no gradient). NSA is trained end
 * to end, with the backward pass claimed to gain from the same sparsity as the
 * forward (NSA how-to, qwbw.cn/news/106443, section 1); each branch is
 * softmax attention over its key set, and the compressed branch's keys and
 * values are block means, so their gradients are spread evenly over the 64
 * tokens of each complete block.
 *
 * desc, params, q, k, v, gates: as for nsa_fwd_prefill (same layouts, dtypes,
 *   strides and limits). dout [B, L, Hq, D] is the upstream gradient, in
 *   desc->out_dtype with the strides desc->o_stride (element size aligned).
 * idx [B, L, G, top_k] int32, contiguous, required: the selection the
 *   forward used (its NSA_IDX_COMPUTE output, or the injected one), read with
 *   the injected-selection rule (entries outside [0, t/64] and repeats add
 *   nothing).
 * dq [B, L, Hq, D], dk / dv [B, L, G, D], dgates [B, L, Hq, 3]: contiguous
 *   float32 outputs, written in full (dq 16-byte aligned, the rest 4-byte).
 *   dgates[..., x] = dout . o_x, the gradient of gate x of branch x in the
 *   order (compressed, selected, window).
 * workspace: device memory of at least nsa_bwd_prefill_workspace_bytes()
 *   bytes (16-byte aligned), caller-owned, contents not preserved. The call
 *   is asynchronous on `stream`; inputs must stay valid until it completes.
 * dk and dv are sums accumulated with floating-point atomics, so their last
 * bits may differ from call to call. Errors are reported as for the forward
 * entry points.
 */
nsa_status_t nsa_bwd_prefill_workspace_bytes(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                             size_t* bytes);
nsa_status_t nsa_bwd_prefill(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                             const void* k, const void* v, const void* gates, const void* dout,
                             const int32_t* idx, float* dq, float* dk, float* dv, float* dgates,
                             void* workspace, size_t workspace_bytes, void* stream);
/*
 * nsa_bwd_prefill given the selected branch's output and log-sum-exp kept by
 * nsa_fwd_prefill_save for the same inputs and selection (o_slc: out_dtype,
 * 16-byte aligned; lse_slc: float32): the query side then skips that
 * branch's forward recomputation (its blocks are gathered once instead of
 * twice). Same results up to rounding; same errors, plus
 * NSA_ERR_INVALID_ARGUMENT for a NULL or misaligned o_slc / lse_slc.
 */
nsa_status_t nsa_bwd_prefill_saved(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                                   const void* k, const void* v, const void* gates, const void* dout,
                                   const int32_t* idx, const void* o_slc, const float* lse_slc, float* dq,
                                   float* dk, float* dv, float* dgates, void* workspace, size_t workspace_bytes,
                                   void* stream);
nsa_status_t nsa_bwd_prefill_saved_timed(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                         const void* q, const void* k, const void* v, const void* gates,
                                         const void* dout, const int32_t* idx, const void* o_slc,
                                         const float* lse_slc, float* dq, float* dk, float* dv, float* dgates,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         void* const* stage_events);
/* nsa_bwd_prefill with 4 stage events (prep; query side; key side). */
nsa_status_t nsa_bwd_prefill_timed(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                                   const void* k, const void* v, const void* gates, const void* dout,
                                   const int32_t* idx, float* dq, float* dk, float* dv, float* dgates,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* stage_events);

/*
 * Token-level sparse attention with a ReLU indexer (DeepSeek Sparse
 * Attention, DSA; DSA how-to, bjdmk.com.cn/news/5181035): each query token
 * attends only to the top_k tokens (2048 on that page) that a lightweight
 * multi-head indexer ranks highest, which takes the core attention from
 * O(L^2) to O(L * top_k) (section 1); the indexer is a linear layer, a dot
 * product and ReLU with 8 or 16 heads and one cached indexer key per token
 * (section 3); a top_k at or above the sequence length is dense attention
 * (section 5). Computes, for each (b, t):
 *   scores:    I(t, s) = sum_j w[t][j] * max(qi[t][j] . ki[s], 0) for s <= t;
 *   selection: the top_k tokens s <= t by score, ties to the lower token, all
 *              of them when t + 1 <= top_k; shared by all query heads;
 *   attention: out[t][h] = softmax attention of q[t][h] (scale softmax_scale,
 *              <= 0 -> 1/sqrt(head_dim)) over k, v of the chosen tokens in
 *              KV head h / (n_q_heads / n_kv_heads).
 *   q [B, L, Hq, D], k/v [B, L, G, D], out [B, L, Hq, D] with (b, t, head)
 *   strides; qi [B, L, Hi, Di] with (b, t, indexer head) strides; ki [B, L, Di]
 *   and w [B, L, Hi] with (b, t) strides (last dimension contiguous).
 *   idx [B, L, top_k] int32 dense: NSA_IDX_COMPUTE writes the chosen tokens
 *   ascending, padded with -1 (when idx != NULL); NSA_IDX_INJECT reads them
 *   (a set of tokens: entries outside [0, t] and repeats add nothing; no
 *   usable entry gives out = 0) and runs no indexer.
 * Supported: head_dim and idx_dim in {64, 128}; 1 <= idx_heads <= 16;
 * 1 <= top_k <= 2048; seqlen <= 131072 (the page's 128K maximum context);
 * n_q_heads <= 64 with n_q_heads / n_kv_heads at most 16
 * or a multiple of 16; bf16 in / {bf16, f32} out, f32 in / f32 out; strides
 * multiples of 8 elements. The workspace (nsa_dsa_workspace_bytes) holds the
 * float32 indexer scores of every (query, earlier token) pair,
 * B * L * (L + 1) / 2 floats (8 GiB for one 64k sequence) and 256 bytes
 * after them, and the selection when idx is NULL. Errors as for the other
 * entry points.
 */
typedef struct {
  int32_t batch, seqlen, n_q_heads, n_kv_heads, head_dim, idx_heads, idx_dim;
  nsa_dtype_t in_dtype, out_dtype;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int64_t qi_stride[3];
  int64_t ki_stride[2];
  int64_t w_stride[2];
} nsa_dsa_desc_t;

typedef struct {
  int32_t top_k;
  float softmax_scale; /* <= 0 selects 1/sqrt(head_dim) */
} nsa_dsa_params_t;

nsa_status_t nsa_dsa_workspace_bytes(const nsa_dsa_desc_t* desc, const nsa_dsa_params_t* params, size_t* bytes);
nsa_status_t nsa_dsa_prefill(const nsa_dsa_desc_t* desc, const nsa_dsa_params_t* params, const void* q,
                             const void* k, const void* v, const void* qi, const void* ki, const void* w, void* out,
                             int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace, size_t workspace_bytes,
                             void* stream);
/* nsa_dsa_prefill recording 4 caller-created hipEvents (indexer; top-k;
 * attention); with NSA_IDX_INJECT the first two stages are empty. */
nsa_status_t nsa_dsa_prefill_timed(const nsa_dsa_desc_t* desc, const nsa_dsa_params_t* params, const void* q,
                                   const void* k, const void* v, const void* qi, const void* ki, const void* w,
                                   void* out, int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* stage_events);

/* Static name of a status code. */
const char* nsa_status_string(nsa_status_t status);

/* Message describing the last failing call on this thread ("" if none). */
const char* nsa_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t nsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
