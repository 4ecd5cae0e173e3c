/*
 * attn_sink.h -- C ABI of libattnsink.so: grouped-query attention whose softmax
 * includes a learned per-head sink logit, on AMD Instinct MI355X (gfx950).
 *
 * The operation (source: "GPT-OSS on Day 0", section "Attention sinks"): every query
 * head h carries a sink logit sink[h] that joins the softmax over the scaled Q.K
 * scores of its row and has no value vector. For a query row with visible keys J:
 *     M   = max(max_{j in J} s_j, sink[h]),          s_j = softmax_scale * q . k_j
 *     D   = sum_{j in J} exp(s_j - M) + exp(sink[h] - M)
 *     out = sum_{j in J} exp(s_j - M) v_j / D        (bf16)
 *     lse = M + ln D                                  (fp32, natural log, sink included)
 * The kernels compute this with an online (streaming) softmax whose running maximum
 * is seeded with the head's sink in the first KV chunk only; when the KV range is
 * split, chunk partials are combined by a log-sum-exp merge (same section: heads and
 * the KV length are processed in parallel).
 *
 * Conventions shared by every entry point
 *   - Element types: Q, K, V and `out` are bf16 (passed as void*); sinks, lse and all
 *     partials are fp32; indices and lengths are int32.
 *   - All tensor pointers are DEVICE pointers on the current HIP device; the caller owns
 *     every buffer (workspace included). The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t; NULL = default
 *     stream). Launch shapes depend only on host scalars, so calls may be captured
 *     into a HIP graph.
 *   - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - Masks are computed from indices (no mask tensor). With Lq query tokens and Lk keys
 *     in a sequence, query token t sits at absolute position p = Lk - Lq + t (new tokens
 *     are the last ones). causal != 0: key j visible iff j <= p. window > 0: key j also
 *     needs p - j < window (window keys including the query's own position).
 *   - `sinks` may be NULL: every head then behaves as sink = -inf (plain attention).
 *     Individual entries may be -inf.
 *   - A query row with no visible key returns out = 0 and lse = sink[h] (-inf when the
 *     sink is disabled); no NaN is produced.
 *   - head_dim must be 64.
 *   - bf16 tensors (q, k, v, the caches, out, q_out) and o_partial must start on a 16-byte
 *     boundary (every torch allocation does), else ATTN_SINK_ERR_INVALID_ARG.
 *   - Errors: arguments are validated on the host before anything is enqueued; invalid
 *     arguments return ATTN_SINK_ERR_INVALID_ARG and unsupported shapes
 *     ATTN_SINK_ERR_UNSUPPORTED, with nothing launched. A failed launch returns
 *     ATTN_SINK_ERR_HIP. Device-side faults surface at the caller's next
 *     synchronisation. Nothing aborts the process.
 *   - Paged entry points: a sequence's capacity, max_pages_per_seq * page_size tokens,
 *     must be below 2^31, else ATTN_SINK_ERR_UNSUPPORTED.
 *   - Memory safety against bad device metadata: sequence lengths, cu_seqlens offsets and
 *     page ids read on the device are clamped into the ranges the host scalars declare,
 *     so inconsistent metadata yields wrong numbers for the affected rows, never an
 *     out-of-bounds access.
 */
#ifndef ATTN_SINK_H_
#define ATTN_SINK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_SINK_OK = 0,
  ATTN_SINK_ERR_INVALID_ARG = 1,
  ATTN_SINK_ERR_UNSUPPORTED = 2,
  ATTN_SINK_ERR_WORKSPACE_TOO_SMALL = 3,
  ATTN_SINK_ERR_HIP = 4
} attn_sink_status;

/*
 * Packed variable-length self-attention without a KV cache: causal prefill,
 * sliding-window prefill and bidirectional (embedding) batches ("GPT-OSS on Day 0",
 * section "Attention sinks": the same kernel family serves prefill; "Fast Embeddings on
 * GPUs", ragged-attention section: embedding batches run ragged, without padding).
 *
 *   q            bf16 [total_q, num_q_heads, 64], contiguous.
 *   k, v         bf16 [total_kv, num_kv_heads, 64], contiguous.
 *   sinks        fp32 [num_q_heads] or NULL.
 *   cu_seqlens_q, cu_seqlens_kv
 *                int32 [batch + 1] on the device, non-decreasing, starting at 0:
 *                sequence b owns Q rows [cu_q[b], cu_q[b+1]) and KV rows
 *                [cu_kv[b], cu_kv[b+1]). The same pointer may be passed for both.
 *   total_q, total_kv
 *                rows in q and in k/v (bounds for the clamping of device offsets).
 *   max_seqlen_q, max_seqlen_kv
 *                host upper bounds of the per-sequence lengths (they size the launch
 *                grid; longer sequences are truncated to them).
 *   softmax_scale  multiplies q.k (e.g. 1/sqrt(64)); the sink is NOT scaled.
 *   causal, window  see the conventions above (window <= 0: no window).
 *   out          bf16 [total_q, num_q_heads, 64].
 *   lse          fp32 [total_q, num_q_heads] or NULL.
 * Constraints: batch >= 0, num_q_heads % num_kv_heads == 0, head_dim == 64,
 * softmax_scale finite and > 0; q, k, v, out and the cu_seqlens pointers non-NULL when
 * batch > 0 and total_q > 0. One sequence's Q rows (max_seqlen_q * num_q_heads * 128
 * bytes) and K or V rows (plus one 64-key tile) must each span less than 2^31 bytes,
 * and the launch (one workgroup per block of up to 512 query rows of one KV head, per
 * sequence) must stay under 2^31 workgroups, else ATTN_SINK_ERR_UNSUPPORTED.
 */
attn_sink_status attn_sink_prefill(
    const void* q, const void* k, const void* v, const float* sinks,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    int32_t batch, int32_t total_q, int32_t total_kv,
    int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float softmax_scale, int32_t causal, int32_t window,
    void* out, float* lse, void* stream);

/*
 * Chunked prefill against a paged KV cache: each sequence's queries are its newest tokens,
 * whose K/V (together with the cached context before them) are already in the cache ("Fast
 * Embeddings on GPUs", attention section: the LLM path runs prefill as well as decode on
 * paged KV, next to the ragged path of attn_sink_prefill).
 *
 *   q            bf16 [total_q, num_q_heads, 64]; sequence b owns rows
 *                [cu_seqlens_q[b], cu_seqlens_q[b+1]), its Lq_b newest tokens: query token t
 *                sits at absolute position kv_lens[b] - Lq_b + t.
 *   k_cache, v_cache, page_table, max_pages_per_seq, num_pages, page_size
 *                as for attn_sink_decode_paged (HND pages, page_size a power of two in
 *                [16, 256]).
 *   cu_seqlens_q int32 [batch + 1] on the device, non-decreasing, starting at 0.
 *   kv_lens      int32 [batch] on the device: tokens in the cache per sequence, the chunk
 *                included (clamped to [0, min(max_kv_len, max_pages_per_seq * page_size)]).
 *   total_q, max_seqlen_q, max_kv_len
 *                rows in q and host upper bounds of the chunk and cache lengths.
 *   sinks, softmax_scale, causal, window, out, lse
 *                as for attn_sink_prefill.
 * No workspace: every chunk's rows are finished in one pass. Errors as above; one
 * sequence's Q rows must span less than 2^31 bytes and the launch stay under 2^31
 * workgroups (as for attn_sink_prefill).
 */
attn_sink_status attn_sink_prefill_paged(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    const int32_t* cu_seqlens_q, const int32_t* kv_lens, const float* sinks,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float softmax_scale, int32_t causal, int32_t window,
    void* out, float* lse, void* stream);

/*
 * Paged decode (q_len = 1) and multi-token verify decode (q_len 2..8, causal inside the
 * block) against a paged KV cache, split along the KV length into kv_chunk-token
 * chunks whose partials are merged by log-sum-exp ("GPT-OSS on Day 0", section
 * "Attention sinks": split across blocks along the sequence, sink only in the first
 * chunk; "Fast Embeddings on GPUs": paged decode; "Accelerating Sonar through
 * speculation": verification of several draft tokens per sequence).
 *
 *   q            bf16 [batch * q_len, num_q_heads, 64]; row b*q_len + t is query token t
 *                of sequence b, at absolute position kv_lens[b] - q_len + t.
 *   k_cache, v_cache
 *                bf16 [num_pages, num_kv_heads, page_size, 64] ("HND": one page of one KV
 *                head is a contiguous page_size x 64 block). Token j of sequence b is in
 *                physical page page_table[b * max_pages_per_seq + j / page_size], slot
 *                j % page_size.
 *   page_table   int32 [batch, max_pages_per_seq] on the device.
 *   kv_lens      int32 [batch] on the device; KV length of each sequence INCLUDING its
 *                q_len new tokens (already appended). Clamped to
 *                [0, min(max_kv_len, max_pages_per_seq * page_size)].
 *   sinks        fp32 [num_q_heads] or NULL.
 *   max_kv_len   host upper bound of kv_lens (sizes the grid and the workspace).
 *   kv_chunk     tokens per split-KV chunk: a positive multiple of 64 that is also a
 *                multiple of page_size; <= 0 means one chunk spanning max_kv_len.
 *   workspace    caller-owned device buffer of at least
 *                attn_sink_decode_workspace_size(...) bytes, 256-byte aligned. Layout, with
 *                R = batch * q_len rows, C = chunks per row bound = max(1, ceil(max_kv_len /
 *                kv_chunk)), NP = R * C, each region starting at a 256-byte boundary:
 *                  int32 partial_indptr[R + 1]   (plan: row r owns partials
 *                                                 [indptr[r], indptr[r+1]); exclusive scan)
 *                  int32 chunk_counts[R]          (plan: n_r = max(1, ceil(L_b / kv_chunk)))
 *                  fp32  o_partial[NP][num_q_heads][64]  (chunk outputs, each normalised)
 *                  fp32  lse_partial[NP][num_q_heads]    (chunk log-sum-exp, natural log)
 *                Partial indptr[r] + c holds chunk c of row r; chunk 0 carries the sink.
 *                The plan and the partials are valid after the call completes.
 *   out, lse     bf16 [batch * q_len, num_q_heads, 64]; fp32 [batch * q_len, num_q_heads]
 *                or NULL.
 * Constraints: 1 <= q_len <= 8, q_len * (num_q_heads / num_kv_heads) <= 64,
 * page_size a power of two in [16, 256] and at most kv_chunk, head_dim == 64,
 * num_pages >= 1, max_pages_per_seq >= 1. Enqueues two kernels (split-KV chunks, then
 * the merge).
 */
attn_sink_status attn_sink_decode_paged(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    const int32_t* kv_lens, const float* sinks,
    int32_t batch, int32_t q_len, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float softmax_scale, int32_t causal, int32_t window, int32_t kv_chunk,
    void* workspace, size_t workspace_bytes,
    void* out, float* lse, void* stream);

/* Ramp forms of YaRN's frequency blend (argument yarn_ramp of attn_sink_rope_append). */
typedef enum {
  ATTN_SINK_YARN_RAMP_TURNS = 0, /* g_i linear in the turns r_i (the YaRN paper's ramp function) */
  ATTN_SINK_YARN_RAMP_INDEX = 1  /* g_i linear in the pair index i, i.e. in ln r_i */
} attn_sink_yarn_ramp;

/*
 * The step before attention for new tokens: YaRN rotary position encoding of their Q and K
 * and the append of their K and V into the paged cache ("GPT-OSS on Day 0", section
 * "GPT-OSS on Hopper": the model encodes positions with YaRN, as DeepSeek-V3 does; the
 * method is YaRN's published one). The pair (x[i], x[i + 32]) of a head vector at position p
 * is rotated by the angle p * f_i; f_i = rope_theta^(-i / 32), and with yarn_factor s > 1,
 * r_i = yarn_original_len * f_i / (2 pi) (turns of pair i over the original context) and a
 * ramp g_i that is 1 where r_i >= yarn_beta and 0 where r_i <= yarn_alpha give
 * f_i <- g_i f_i + (1 - g_i) f_i / s; cos and sin are scaled by 0.1 ln s + 1 (by 1 when
 * s <= 1). Inside the band the ramp is
 *   ATTN_SINK_YARN_RAMP_TURNS: g_i = (r_i - yarn_alpha) / (yarn_beta - yarn_alpha), or
 *   ATTN_SINK_YARN_RAMP_INDEX: g_i = ln(r_i / yarn_alpha) / ln(yarn_beta / yarn_alpha), which is
 *     linear in the pair index between the (real) indices where r_i = yarn_beta and
 *     r_i = yarn_alpha (the form of released YaRN implementations that compute correction
 *     dimensions); the page does not say which form its model uses.
 *
 *   q            bf16 [total_q, num_q_heads, 64], the new tokens; sequence b owns rows
 *                [cu_seqlens_q[b], cu_seqlens_q[b+1]), its newest tokens: row t sits at
 *                position kv_lens[b] - Lq_b + t.
 *   k, v         bf16 [total_q, num_kv_heads, 64], the new tokens' K and V.
 *   cu_seqlens_q int32 [batch + 1], kv_lens int32 [batch] on the device; kv_lens counts the
 *                new tokens (clamped to min(max_kv_len, max_pages_per_seq * page_size)).
 *   page_table, max_pages_per_seq, num_pages, page_size
 *                as for attn_sink_decode_paged.
 *   k_cache, v_cache
 *                bf16 [num_pages, num_kv_heads, page_size, 64]: the rotated K and the V of
 *                each new token are written at page page_table[b][p / page_size], slot
 *                p % page_size; nothing else in the caches is touched.
 *   yarn_ramp    an attn_sink_yarn_ramp value (ignored when yarn_factor <= 1).
 *   q_out        bf16 [total_q, num_q_heads, 64], the rotated Q (may be q itself).
 * Errors: rope_theta <= 1, yarn_factor <= 0, or (for yarn_factor > 1) yarn_original_len <= 0,
 * yarn_alpha >= yarn_beta, yarn_alpha <= 0 with the index ramp, or an unknown yarn_ramp:
 * ATTN_SINK_ERR_INVALID_ARG; head_dim != 64, page sizes as for decode, batch > 65535:
 * ATTN_SINK_ERR_UNSUPPORTED. Enqueues one kernel.
 */
attn_sink_status attn_sink_rope_append(
    const void* q, const void* k, const void* v,
    const int32_t* cu_seqlens_q, const int32_t* kv_lens,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    void* k_cache, void* v_cache,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float rope_theta, float yarn_factor, int32_t yarn_original_len, float yarn_alpha, float yarn_beta,
    int32_t yarn_ramp, void* q_out, void* stream);

/*
 * attn_sink_decode_paged without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The plan and the chunk partials go to a scratch array inside the library
 * (attn_sink_decode_noalloc_capacity() bytes, 64 MiB: e.g. 64 sequences of up to 8192 keys at
 * q_len 1 in 512-token chunks need 16.3 MiB, 32 sequences of up to 16384 keys at q_len 5 in
 * 2048-token chunks 20.3 MiB); each GPU the library runs on holds its own copy from the first
 * call on it until the process ends. The call allocates nothing and calls no allocating
 * routine. The same kernels run as for attn_sink_decode_paged, with the same results.
 *
 * Arguments, constraints and error codes as for attn_sink_decode_paged without workspace and
 * workspace_bytes; a call whose workspace (attn_sink_decode_workspace_size of its scalars)
 * exceeds the capacity returns ATTN_SINK_ERR_WORKSPACE_TOO_SMALL with nothing launched. Every
 * call on one GPU uses that GPU's one scratch array: calls that may run at the same time on
 * one GPU (different streams, or different host threads) race on it and must be ordered by
 * the caller. The scratch keeps the last call's plan and partials; nothing in it needs to
 * start at zero. Enqueues two kernels (split-KV chunks, then the merge).
 */
attn_sink_status attn_sink_decode_paged_noalloc(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    const int32_t* kv_lens, const float* sinks,
    int32_t batch, int32_t q_len, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float softmax_scale, int32_t causal, int32_t window, int32_t kv_chunk,
    void* out, float* lse, void* stream);

/* Bytes of scratch attn_sink_decode_paged_noalloc can use on each GPU (a constant). */
size_t attn_sink_decode_noalloc_capacity(void);

/*
 * Verification of a draft tree in one step ("Accelerating Sonar through speculation", EAGLE
 * section: tree-shaped drafts need a custom attention mask, which a full-sequence mask made
 * costly). The mask is a bitmap per draft row: the q_len draft tokens are the last q_len of
 * each sequence's kv_lens[b] tokens, and row b * q_len + t sees every earlier (prefix) token
 * plus the draft tokens i whose bit i is set in tree_mask[b * q_len + t] (set bits >= q_len
 * are ignored). A window > 0 also bounds every key by position (p - j < window).
 *
 *   tree_mask    int32 [batch * q_len] on the device (a chain, bits 0..t for row t, is the
 *                causal verify of attn_sink_decode_paged).
 * Every other argument, constraint and error code as for attn_sink_decode_paged (there is no
 * causal flag: the bitmaps decide inside the draft block); tree_mask NULL is
 * ATTN_SINK_ERR_INVALID_ARG. Enqueues two kernels (split-KV chunks, then the merge).
 */
attn_sink_status attn_sink_decode_paged_tree(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    const int32_t* kv_lens, const int32_t* tree_mask, const float* sinks,
    int32_t batch, int32_t q_len, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float softmax_scale, int32_t window, int32_t kv_chunk,
    void* workspace, size_t workspace_bytes,
    void* out, float* lse, void* stream);

/*
 * The split-KV pass of attn_sink_decode_paged alone: writes the plan and the chunk partials
 * into the workspace (layout above) and does not merge them. Arguments, constraints and
 * error codes as for attn_sink_decode_paged, without out and lse. For callers that merge
 * later, e.g. after exchanging partials of different KV ranges between devices (the merge
 * is then attn_sink_merge_partials over partial_indptr). Enqueues one kernel.
 */
attn_sink_status attn_sink_decode_paged_partials(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    const int32_t* kv_lens, const float* sinks,
    int32_t batch, int32_t q_len, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float softmax_scale, int32_t causal, int32_t window, int32_t kv_chunk,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The split-KV pass over one contiguous range of each sequence's keys, for context
 * parallelism: the keys of a sequence are spread over several devices, each holding one
 * range, and each device emits the chunk partials of its range ("GPT-OSS on Day 0", section
 * "Attention sinks": the attention is split along the sequence, the partials are combined by
 * their log-sum-exp, and the sink counts once).
 *
 *   kv_lens[b]     keys of this range (paged as for attn_sink_decode_paged: page_table row b
 *                  lists this range's pages, its key 0 first).
 *   kv_start[b]    int32 [batch] on the device: absolute position of this range's first key.
 *   kv_total[b]    int32 [batch] on the device: keys of the whole sequence; its last q_len
 *                  positions are the query tokens.
 * Causal and window masks use absolute positions: key j of the range is position
 * kv_start[b] + j, query token t is position kv_total[b] - q_len + t. Only a range with
 * kv_start[b] == 0 counts the head's sink, so exactly one range of each sequence must start
 * at 0 (an empty range elsewhere takes any other start). The partials of all ranges of a sequence, listed
 * per row in any order and merged by attn_sink_merge_partials, give what
 * attn_sink_decode_paged gives for the whole sequence (up to rounding). A range with no keys
 * yields one partial: the sink alone if kv_start[b] == 0, else an empty one (lse -inf).
 * Positions that break 0 <= kv_start[b] <= kv_total[b] - kv_lens[b] give unspecified values
 * but no out-of-range access (they only enter the masks). kv_start or kv_total NULL (with
 * batch > 0) is ATTN_SINK_ERR_INVALID_ARG. Everything else, including the workspace layout,
 * as for attn_sink_decode_paged_partials. Enqueues one kernel.
 */
attn_sink_status attn_sink_decode_paged_range_partials(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    const int32_t* kv_lens, const int32_t* kv_start, const int32_t* kv_total, const float* sinks,
    int32_t batch, int32_t q_len, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float softmax_scale, int32_t causal, int32_t window, int32_t kv_chunk,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The split-KV pass of attn_sink_decode_paged_tree alone (the tree counterpart of
 * attn_sink_decode_paged_partials): plan and chunk partials in the workspace, no merge.
 * Arguments, constraints and error codes as for attn_sink_decode_paged_tree, without out and
 * lse. Enqueues one kernel.
 */
attn_sink_status attn_sink_decode_paged_tree_partials(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    const int32_t* kv_lens, const int32_t* tree_mask, const float* sinks,
    int32_t batch, int32_t q_len, int32_t max_kv_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    float softmax_scale, int32_t window, int32_t kv_chunk,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chooses kv_chunk for a decode call from the sequences' lengths, which the caller knows on
 * the host (the plan metadata a serving runtime builds before attention: "Accelerating
 * Sonar through speculation", inference runtime section). The split-KV kernel deals its
 * work items (sequence, chunk, KV head) to a fixed grid of resident workgroups round-robin,
 * and a call lasts as long as its most loaded workgroup. For every candidate length (the
 * multiples of max(256, page_size) up to one chunk per sequence) this function deals the
 * items the same way. It charges each item its keys plus a fixed cost of 1024 keys, which
 * was fitted on MI355X to whole-call times of the verify-shaped workloads. The merge reads a
 * sequence's partials 16 per memory round trip, so it adds 384 keys per 16 chunks (rounded
 * up) of the sequence with the most chunks; that cost was fitted to whole-call times over
 * batches of 1-64 sequences of 2048-32768 keys. The cost of a candidate is its most loaded workgroup's
 * load plus that merge cost. It returns the candidate of lowest cost; ties go to the longer
 * chunk.
 *   kv_lens      int32 [batch] on the HOST: the lengths the call will see.
 *   workgroups   resident workgroups of the split kernel; <= 0 asks the current device
 *                (a HIP device must then be present).
 *   kv_chunk     out: the chosen length, a positive multiple of 64 and of page_size.
 * q_len, num_q_heads, num_kv_heads and page_size are constrained as for
 * attn_sink_decode_paged. Host arithmetic only, nothing enqueued; size the workspace for
 * the returned chunk. NULL kv_chunk, or NULL kv_lens with batch > 0, is
 * ATTN_SINK_ERR_INVALID_ARG.
 */
attn_sink_status attn_sink_decode_plan_chunk(const int32_t* kv_lens, int32_t batch, int32_t q_len,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t page_size,
                                             int32_t workgroups, int32_t* kv_chunk);

/*
 * Bytes of workspace attn_sink_decode_paged needs for these host scalars (0 if they are
 * invalid). Monotone non-decreasing in batch, q_len, max_kv_len and num_q_heads.
 */
size_t attn_sink_decode_workspace_size(int32_t batch, int32_t q_len, int32_t max_kv_len,
                                       int32_t num_q_heads, int32_t head_dim, int32_t kv_chunk);

/* Where the decode entry points put the plan and the partials inside the workspace. */
typedef struct {
  int64_t rows;        /* batch * q_len query rows */
  int64_t chunks;      /* chunk bound per row: max(1, ceil(max_kv_len / chunk length)) */
  int64_t partials;    /* rows * chunks partial slots */
  int64_t off_indptr;  /* byte offset of int32 partial_indptr[rows + 1] */
  int64_t off_counts;  /* byte offset of int32 chunk_counts[rows] */
  int64_t off_o;       /* byte offset of fp32 o_partial[partials][num_q_heads][64] */
  int64_t off_lse;     /* byte offset of fp32 lse_partial[partials][num_q_heads] */
  int64_t total;       /* workspace bytes (attn_sink_decode_workspace_size) */
} attn_sink_decode_layout;

/*
 * Fills *layout for these host scalars (the layout documented at attn_sink_decode_paged, the
 * same one the decode entry points use), so that callers read the plan and the partials back
 * without re-deriving the offsets. Returns ATTN_SINK_ERR_INVALID_ARG for a NULL layout or
 * scalars for which attn_sink_decode_workspace_size returns 0. Host-only; enqueues nothing.
 */
attn_sink_status attn_sink_decode_workspace_layout(int32_t batch, int32_t q_len, int32_t max_kv_len,
                                                   int32_t num_q_heads, int32_t head_dim, int32_t kv_chunk,
                                                   attn_sink_decode_layout* layout);

/*
 * Log-sum-exp merge of split-KV partials ("GPT-OSS on Day 0", section "Attention
 * sinks": attention split into several blocks along the sequence). For row r and head h,
 * over partials p in [partial_indptr[r], partial_indptr[r+1]):
 *     LSE = ln sum_p exp(lse_partial[p][h]),  out = sum_p exp(lse_partial[p][h] - LSE) o_partial[p][h]
 * Partials with lse = -inf (or NaN) carry weight 0 and their o is not used (it may hold
 * anything, NaN included); a row whose partials are all -inf (or that has none) returns
 * out = 0, lse = -inf.
 *
 *   o_partial    fp32 [num_partials, num_q_heads, 64]; each partial already normalised.
 *   lse_partial  fp32 [num_partials, num_q_heads], natural log.
 *   partial_indptr  int32 [num_rows + 1] on the device, non-decreasing; entries are
 *                clamped to [0, num_partials].
 *   out, lse     bf16 [num_rows, num_q_heads, 64]; fp32 [num_rows, num_q_heads] or NULL.
 */
attn_sink_status attn_sink_merge_partials(
    const float* o_partial, const float* lse_partial, int32_t num_partials,
    const int32_t* partial_indptr, int32_t num_rows,
    int32_t num_q_heads, int32_t head_dim,
    void* out, float* lse, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* attn_sink_status_string(attn_sink_status status);

/* Library version string, e.g. "attn_sink 0.1.0 gfx950". */
const char* attn_sink_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SINK_H_ */
