/*
 * sinkattn -- grouped-query attention with a learned per-head sink logit,
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (Perplexity, "GPT-OSS on day 0", sections "Hopper: attention
 * with sinks (GQA)" and "GPT-OSS kernels / Sink attention"): every query head
 * h owns one scalar sink z_h that joins the softmax as an extra logit with no
 * value vector.  For query row i with valid key set J(i):
 *
 *     s_j = softmax_scale * <q_i, k_j>,   M = max(z_h, max_j s_j)
 *     den = exp(z_h - M) + sum_j exp(s_j - M)
 *     o_i = sum_j exp(s_j - M) v_j / den,   lse_i = M + ln(den)
 *
 * The sink is in logit units: softmax_scale multiplies q.k only.  The online
 * form starts the running max at z_h and the denominator at 1; when the key
 * sequence is split, only the first split starts from the sink.  Layers are
 * either causal over the full context or restricted to a sliding window of
 * the last W keys (NVIDIA gpt-oss announcement, model description: full
 * context and 128-token window layers alternate).  Window semantics: query i
 * sees key j iff j <= i and (W <= 0 or j > i - W); W counts the query itself.
 *
 * GQA mapping: query head h reads KV head h / G with G = Hq / Hkv.
 *
 * Conventions shared by every entry point:
 *  - Every pointer is a DEVICE pointer except where stated; q/k/v/o/workspace
 *    must be 16-byte aligned.  Tensors are dense row-major with the layouts
 *    given below (token-major, then head, then head_dim).
 *  - bf16 is stored as raw 16-bit patterns (uint16); outputs are rounded to
 *    nearest even from fp32 accumulators.
 *  - The caller allocates and owns every buffer, including the workspace.
 *    These entry points never allocate or free device memory and (outside
 *    the debug mode below) never synchronise: work is enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL is the default stream) and the
 *    call returns.
 *  - Host-checkable argument errors return a status before anything is
 *    launched; a launch failure returns SINKATTN_ERR_HIP.  The message of the
 *    last failure on the calling thread is sinkattn_last_error().  No C++
 *    exception crosses this interface.
 *  - Device-side preconditions: cu_seqlens is non-decreasing with
 *    cu_seqlens[0] = 0 and every length <= max_seqlen (prefill:
 *    cu_seqlens[batch] <= total_tokens); decode lengths are >= 1; sinks are
 *    finite or -inf (-inf = that head has no sink); q/k/v hold no NaN/Inf;
 *    merge partials hold no NaN/Inf (lse_parts may be -inf = empty part).
 *    They are not checked by default.  With SINKATTN_DEBUG_CHECKS=1 in the
 *    environment (read on every call) each entry point first checks them on
 *    the device, synchronising `stream`, and returns SINKATTN_ERR_INVALID_ARG
 *    naming the failed conditions without launching the attention kernels.
 *    Debug checks of calls that overlap on one device share one flag word.
 *  - Supported shapes: head_dim == 64 (other values: SINKATTN_ERR_UNSUPPORTED),
 *    num_q_heads % num_kv_heads == 0, softmax_scale finite and > 0.
 */
#ifndef SINKATTN_H_
#define SINKATTN_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SINKATTN_API __attribute__((visibility("default")))
#else
#define SINKATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sinkattn_status {
  SINKATTN_OK = 0,
  SINKATTN_ERR_INVALID_ARG = 1,
  SINKATTN_ERR_UNSUPPORTED = 2,
  SINKATTN_ERR_WORKSPACE = 3,
  SINKATTN_ERR_HIP = 4
} sinkattn_status;

/*
 * Varlen self-attention prefill with sinks (Perplexity, "GPT-OSS on day 0",
 * Sink attention: the prefill template extended with the sink; window layers
 * from the NVIDIA gpt-oss announcement).
 *
 *   q           bf16 [total_tokens, num_q_heads, head_dim]
 *   k, v        bf16 [total_tokens, num_kv_heads, head_dim]
 *   sinks       fp32 [num_q_heads], or NULL for "no sink" on every head
 *   cu_seqlens  int32 [batch + 1], device; sequence b owns tokens
 *               [cu_seqlens[b], cu_seqlens[b+1]); queries and keys of a
 *               sequence coincide (positions local to the sequence)
 *   max_seqlen  host int, >= every sequence length
 *   window      <= 0: full causal; W > 0: i - W < j <= i
 *   o           bf16 [total_tokens, num_q_heads, head_dim] (written)
 *   lse         fp32 [total_tokens, num_q_heads], natural log, sink
 *               included; NULL to skip.  A row with no key and no sink gets
 *               o = 0 and lse = -inf.
 *
 * Additionally required: max_seqlen * num_kv_heads * head_dim * 2 < 2^31
 * (one sequence's K/V rows are addressed with 32-bit byte offsets), and
 * num_kv_heads * ceil(group / 8) * floor((total_tokens + 31 * batch) / 32)
 * below 2^24 (workgroups of one launch, one per 32-query tile of each KV
 * head and group of 8 query heads); otherwise SINKATTN_ERR_UNSUPPORTED.
 */
SINKATTN_API sinkattn_status sinkattn_prefill_varlen(
    const void* q, const void* k, const void* v,
    const float* sinks,
    const int32_t* cu_seqlens, int32_t batch,
    int32_t max_seqlen, int32_t total_tokens,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale,
    void* o, float* lse, void* stream);

/*
 * Append prefill with sinks: chunked prefill against a cache that already
 * holds a sequence's earlier tokens, and multi-token-query decode (the draft
 * tokens a speculative or multi-token-prediction decoder hands to the target
 * model for verification: Perplexity, "GPT-OSS on day 0", in-house inference
 * engine; Baseten, "How to run GPT OSS 120B at 500+ tokens per second on
 * NVIDIA GPUs", next performance optimizations).
 *
 * Sequence b has Lk_b = cu_seqlens_k[b+1] - cu_seqlens_k[b] key/value rows
 * (every token up to and including its newest) and Lq_b = cu_seqlens_q[b+1]
 * - cu_seqlens_q[b] <= Lk_b queries, its newest tokens: query r sits at
 * position p = Lk_b - Lq_b + r and sees key j iff j <= p and (W <= 0 or
 * j > p - W), the causal mask aligned at the bottom right.  Lq_b = Lk_b is
 * sinkattn_prefill_varlen; Lq_b = 1 is the single-token decode.
 *
 *   q             bf16 [total_q, num_q_heads, head_dim]
 *   k, v          bf16 [total_k, num_kv_heads, head_dim]
 *   sinks         fp32 [num_q_heads], or NULL for "no sink" on every head
 *   cu_seqlens_q  int32 [batch + 1], device, offsets of the query rows
 *   cu_seqlens_k  int32 [batch + 1], device, offsets of the key/value rows
 *                 (the same array as cu_seqlens_q only together with equal
 *                 maxima and totals: that is self-attention prefill)
 *   max_seqlen_q, max_seqlen_k   host ints, >= every Lq_b, resp. Lk_b
 *   total_q, total_k             host ints, rows of q/o, resp. k/v
 *   window        <= 0: full causal; W > 0: p - W < j <= p
 *   o             bf16 [total_q, num_q_heads, head_dim] (written)
 *   lse           fp32 [total_q, num_q_heads], natural log, sink included;
 *                 NULL to skip
 *
 * Device-side preconditions besides the shared ones (for both offset
 * arrays): Lq_b <= Lk_b for every b; a sequence that breaks it is skipped
 * (its rows are not written) and SINKATTN_DEBUG_CHECKS=1 reports it.
 * max_seqlen_k == 0 with queries present is SINKATTN_ERR_INVALID_ARG.
 * Shape limits as sinkattn_prefill_varlen, with max_seqlen_k in the 2^31
 * bound and total_q in the workgroup bound.
 */
SINKATTN_API sinkattn_status sinkattn_prefill_append(
    const void* q, const void* k, const void* v,
    const float* sinks,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q, int32_t total_k,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale,
    void* o, float* lse, void* stream);

/*
 * sinkattn_prefill_append with each query tile's keys split across
 * workgroups, for chunks of few queries over long caches (a 256-token chunk
 * has only 8 query tiles per KV head): the keys a 32-query tile sees are cut
 * into num_splits contiguous shares of 64-key tiles (trailing shares may be
 * empty), each share's output is normalised on its own and written to the
 * workspace in fp32 with its lse, the sink counted in the first share only,
 * and the shares are combined with the log-sum-exp merge of
 * sinkattn_merge_lse before returning (Perplexity, "GPT-OSS on day 0", Sink
 * attention: attention parallelised over heads and KV length, the sink
 * initialising only the first chunk).  The merge is exact, so the result
 * equals sinkattn_prefill_append's up to fp32 rounding.
 *
 *   (arguments as sinkattn_prefill_append, plus)
 *   num_splits     1 to 1024; 1 runs sinkattn_prefill_append's path
 *   workspace      device buffer, 256-byte aligned, of at least
 *                  sinkattn_decode_workspace_bytes(total_q, num_q_heads,
 *                  head_dim, num_splits) bytes when num_splits > 1
 *                  (SINKATTN_ERR_WORKSPACE otherwise): fp32 partial outputs
 *                  [num_splits, total_q, num_q_heads, head_dim], then fp32
 *                  partial lse [num_splits, total_q, num_q_heads]; owned by
 *                  the caller, overwritten; may be NULL when num_splits == 1
 *   workspace_bytes  its size
 *
 * num_splits < 1 is SINKATTN_ERR_INVALID_ARG, above 1024
 * SINKATTN_ERR_UNSUPPORTED.  Calls that share one workspace on overlapping
 * streams race.  With num_splits > 1 the merge writes every one of the
 * total_q rows of o (and lse): rows that belong to no sequence (past
 * cu_seqlens_q[batch], or of a sequence that breaks Lq_b <= Lk_b) hold
 * unspecified values afterwards, where sinkattn_prefill_append leaves them
 * untouched.
 */
SINKATTN_API sinkattn_status sinkattn_prefill_append_splitkv(
    const void* q, const void* k, const void* v,
    const float* sinks,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q, int32_t total_k,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Bytes of workspace sinkattn_decode_splitkv needs for num_splits > 1:
 * fp32 partial outputs [num_splits, batch, num_q_heads, head_dim] and fp32
 * partial lse [num_splits, batch, num_q_heads], each 256-byte aligned.
 * Returns 0 when num_splits <= 1 and 0 for invalid (negative) sizes.
 */
SINKATTN_API size_t sinkattn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                       int32_t head_dim, int32_t num_splits);

/*
 * Split-KV decode: one query token per sequence against a packed KV cache
 * (Perplexity, "GPT-OSS on day 0", Sink attention: attention parallelised
 * over heads and KV length; with the KV length split into chunks, the sink
 * initialises only the first chunk).
 *
 *   q              bf16 [batch, num_q_heads, head_dim]; the query of
 *                  sequence b sits at position L_b - 1
 *   k_cache,
 *   v_cache        bf16 [total_kv, num_kv_heads, head_dim], packed by
 *                  cu_seqlens_k (int32 [batch + 1], device); L_b >= 1
 *   max_seqlen_k   host int, >= every L_b
 *   window         <= 0: keys [0, L_b); W > 0: keys [max(0, L_b - W), L_b)
 *   num_splits     S >= 1: the key range of every sequence is cut into S
 *                  contiguous chunks of ceil(n / S) keys (trailing chunks may
 *                  be empty); chunk 0 holds the lowest positions and carries
 *                  the sink.  With S > 1 each chunk's partial is normalised
 *                  on its own, written to the workspace in fp32, and the
 *                  partials are combined with the log-sum-exp merge
 *                  (sinkattn_merge_lse) before returning.  The merge is
 *                  exact, so every S gives the same result up to fp32
 *                  rounding; when the range is at most 256 keys, or the
 *                  chunks would hold at most 32 keys of a range of at most
 *                  1024 (window layers with several splits), the range is
 *                  evaluated whole (as S = 1) and the workspace is not
 *                  touched.
 *   workspace      device buffer of >= sinkattn_decode_workspace_bytes(...)
 *                  bytes when S > 1 (SINKATTN_ERR_WORKSPACE otherwise); may
 *                  be NULL when S == 1
 *   o              bf16 [batch, num_q_heads, head_dim]
 *   lse            fp32 [batch, num_q_heads] or NULL
 *
 * Additionally supported: G = num_q_heads / num_kv_heads <= 32 (larger
 * groups return SINKATTN_ERR_UNSUPPORTED).
 */
SINKATTN_API sinkattn_status sinkattn_decode_splitkv(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_k,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Allocation-free form of sinkattn_decode_splitkv, for callers that cannot
 * allocate device memory around the call (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * computation, kernels and errors, minus the workspace: the split-KV
 * partials go to a static device array of SINKATTN_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that the library holds on each device it runs on until the
 * process ends.  The call itself allocates and frees nothing; its first call
 * on a device looks the array's address up (hipGetSymbolAddress).
 *
 * Limit: sinkattn_decode_workspace_bytes(batch, num_q_heads, head_dim,
 * num_splits) must not exceed SINKATTN_NOALLOC_SCRATCH_BYTES
 * (SINKATTN_ERR_WORKSPACE otherwise, before any launch; e.g. 64 sequences x
 * 64 query heads fit up to 31 splits).  num_splits = 1 uses no scratch.
 * Calls that overlap on one device (two streams, two threads) share the
 * array and race; serialise them.
 */
#define SINKATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
SINKATTN_API sinkattn_status sinkattn_decode_splitkv_noalloc(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_k,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* o, float* lse, void* stream);

/*
 * Split-KV decode against an FP8 KV cache (vLLM, "GPT-OSS performance
 * optimizations on NVIDIA Blackwell", FlashInfer integration: the KV cache
 * is stored in FP8).  The page names neither the 8-bit format nor the
 * scaling; this entry point takes OCP E4M3 codes (1 sign, 4 exponent and 3
 * mantissa bits, bias 7, no infinities; 0x7f and 0xff are NaN) with one fp32
 * scale per tensor:
 *     K[t, g, d] = k_scale * e4m3(k_cache[t, g, d]),
 *     V[t, g, d] = v_scale * e4m3(v_cache[t, g, d]),
 * and otherwise computes exactly what sinkattn_decode_splitkv computes on
 * those K and V (same arguments, splits, sink rule, workspace and errors).
 *
 *   k_cache,
 *   v_cache        uint8 E4M3 codes [total_kv, num_kv_heads, head_dim],
 *                  16-byte aligned; NaN codes are a precondition violation
 *                  (reported under SINKATTN_DEBUG_CHECKS=1)
 *   k_scale,
 *   v_scale        host floats, finite and > 0 (SINKATTN_ERR_INVALID_ARG
 *                  otherwise)
 *
 * Workspace: sinkattn_decode_workspace_bytes(batch, num_q_heads, head_dim,
 * num_splits), as for the bf16 cache.
 */
SINKATTN_API sinkattn_status sinkattn_decode_splitkv_fp8(
    const void* q, const void* k_cache, const void* v_cache,
    float k_scale, float v_scale,
    const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_k,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Split-KV decode against a paged KV cache: keys and values live in
 * fixed-size pages of a shared pool, addressed per sequence through a block
 * table (the serving layout around the decode that the Perplexity page's
 * in-house inference engine and the FlashInfer decode template it extends
 * read from; Baseten, "How to run GPT OSS 120B at 500+ tokens per second on
 * NVIDIA GPUs": KV-cache-aware routing).  Token j of sequence b is slot
 * j % page_size of page block_table[b][j / page_size]; otherwise the result
 * is exactly sinkattn_decode_splitkv's on the gathered cache.
 *
 *   q              bf16 [batch, num_q_heads, head_dim]
 *   k_pages,
 *   v_pages        bf16 [num_pages, page_size, num_kv_heads, head_dim]
 *   block_table    int32 [batch, max_pages], device: page ids in
 *                  [0, num_pages); entries past a sequence's last page are
 *                  not read
 *   seq_lens       int32 [batch], device: L_b >= 1, <= max_seqlen_k
 *   page_size      a power of two in [16, 2^20] (SINKATTN_ERR_UNSUPPORTED
 *                  otherwise); max_pages * page_size >= max_seqlen_k;
 *                  num_pages * page_size < 2^31
 *   window, softmax_scale, num_splits, workspace, o, lse
 *                  as sinkattn_decode_splitkv (workspace sized by
 *                  sinkattn_decode_workspace_bytes(batch, ...))
 *
 * Device-side preconditions: the lengths and the page ids a sequence uses
 * (SINKATTN_DEBUG_CHECKS=1 checks them).  Page ids outside the pool are
 * clamped into it, so a bad table gives wrong values, never an access
 * outside k_pages / v_pages.
 */
SINKATTN_API sinkattn_status sinkattn_decode_paged(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
    int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t max_seqlen_k,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Multi-token-query split-KV decode: each sequence's newest tokens are
 * queries against its cache, the draft tokens a speculative or
 * multi-token-prediction decoder hands to the target model for verification
 * (Perplexity, "GPT-OSS on day 0", in-house inference engine; Baseten, "How
 * to run GPT OSS 120B at 500+ tokens per second on NVIDIA GPUs", next
 * performance optimizations).  The result equals sinkattn_prefill_append on
 * the same arguments (query r of sequence b at position Lk_b - Lq_b + r,
 * bottom-right causal, optional window), computed by the decode kernels: one
 * pass over each split of the keys serves all Lq_b tokens and the query
 * heads of a KV head together, so the cache is read once per KV head.
 *
 *   q             bf16 [total_q, num_q_heads, head_dim], packed by
 *                 cu_seqlens_q (int32 [batch + 1], device)
 *   k_cache,
 *   v_cache       bf16 [total_kv, num_kv_heads, head_dim], packed by
 *                 cu_seqlens_k (int32 [batch + 1], device)
 *   max_seqlen_q  host int >= every Lq_b; max_seqlen_q * (num_q_heads /
 *                 num_kv_heads) <= 64 (else SINKATTN_ERR_UNSUPPORTED): up
 *                 to 8 draft tokens per sequence at 8 query heads per KV head
 *   max_seqlen_k  host int >= every Lk_b (>= 1)
 *   total_q       rows of q / o / lse
 *   num_splits,
 *   workspace     as sinkattn_decode_splitkv, sized by
 *                 sinkattn_decode_workspace_bytes(total_q, num_q_heads,
 *                 head_dim, num_splits); the sink enters split 0 only
 *   o, lse        bf16 [total_q, num_q_heads, head_dim]; fp32
 *                 [total_q, num_q_heads] or NULL
 *
 * Device-side preconditions besides the shared ones: 0 <= Lq_b <= Lk_b and
 * Lk_b >= 1 (SINKATTN_DEBUG_CHECKS=1 reports violations).
 */
SINKATTN_API sinkattn_status sinkattn_decode_splitkv_multi(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Append (chunked) prefill against a paged cache: the queries, offsets,
 * masks and outputs of sinkattn_prefill_append with the keys and values in
 * the pages of sinkattn_decode_paged.  The result equals
 * sinkattn_prefill_append's on the gathered cache (sequence b's Lq_b queries
 * are its newest tokens, bottom-right causal, optional window): a prompt
 * chunk, or draft tokens, attending to a paged KV cache.
 *
 *   q, cu_seqlens_q, max_seqlen_q, total_q, sinks, window, softmax_scale,
 *   o, lse         as sinkattn_prefill_append
 *   k_pages, v_pages, block_table, max_pages, page_size, num_pages
 *                  as sinkattn_decode_paged
 *   seq_lens_k     int32 [batch], device: Lk_b >= Lq_b, <= max_seqlen_k
 *
 * Device-side preconditions: those of both entry points (SINKATTN_DEBUG_CHECKS=1
 * checks the offsets, lengths, table and operands).  Page ids outside the pool
 * are clamped into it.
 */
SINKATTN_API sinkattn_status sinkattn_prefill_append_paged(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, const int32_t* seq_lens_k, const int32_t* cu_seqlens_q, int32_t batch,
    int32_t max_pages, int32_t page_size, int32_t num_pages,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale,
    void* o, float* lse, void* stream);

/*
 * sinkattn_prefill_append_paged with each query tile's keys split across
 * workgroups: short chunks of a prompt appended to a long paged cache (vLLM
 * and FlashInfer page their KV caches; "GPT-OSS on day 0", Perplexity, Sink
 * attention, for the split with the sink in the first chunk).  The split,
 * the workspace (sinkattn_decode_workspace_bytes(total_q, num_q_heads,
 * head_dim, num_splits) bytes, 256-byte aligned, when num_splits > 1), the
 * limits and the unspecified rows outside every sequence are those of
 * sinkattn_prefill_append_splitkv; the other arguments and checks those of
 * sinkattn_prefill_append_paged.
 */
SINKATTN_API sinkattn_status sinkattn_prefill_append_paged_splitkv(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, const int32_t* seq_lens_k, const int32_t* cu_seqlens_q, int32_t batch,
    int32_t max_pages, int32_t page_size, int32_t num_pages,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Split-KV decode against a paged FP8 cache: the pages and block table of
 * sinkattn_decode_paged holding the E4M3 codes and per-tensor scales of
 * sinkattn_decode_splitkv_fp8.  The result equals sinkattn_decode_splitkv_fp8's
 * on the gathered cache.
 *
 *   k_pages,
 *   v_pages        uint8 E4M3 codes [num_pages, page_size, num_kv_heads,
 *                  head_dim], 16-byte aligned
 *   k_scale,
 *   v_scale        as sinkattn_decode_splitkv_fp8
 *   everything else
 *                  as sinkattn_decode_paged (workspace sized by
 *                  sinkattn_decode_workspace_bytes(batch, ...))
 *
 * Device-side preconditions: those of both entry points (SINKATTN_DEBUG_CHECKS=1
 * checks the table, the lengths and every code of the pool).
 */
SINKATTN_API sinkattn_status sinkattn_decode_paged_fp8(
    const void* q, const void* k_pages, const void* v_pages,
    float k_scale, float v_scale,
    const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
    int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t max_seqlen_k,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Multi-token-query decode against an FP8 (E4M3) cache: the draft-token
 * verification of sinkattn_decode_splitkv_multi over the E4M3 cache of
 * sinkattn_decode_splitkv_fp8 (vLLM, "GPT-OSS performance optimizations on
 * NVIDIA Blackwell", FlashInfer integration: FP8 KV cache; Perplexity,
 * "GPT-OSS on day 0", in-house inference engine: speculative and MTP
 * decoders).  K = k_scale * e4m3(k_cache), V = v_scale * e4m3(v_cache); the
 * result equals sinkattn_decode_splitkv_multi on those K and V.
 *
 *   q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, total_q,
 *   num_splits, workspace, o, lse
 *                  as sinkattn_decode_splitkv_multi
 *   k_cache,
 *   v_cache        uint8 E4M3 codes [total_kv, num_kv_heads, head_dim]
 *   k_scale,
 *   v_scale        host floats, finite and > 0
 *
 * Preconditions and errors: those of sinkattn_decode_splitkv_multi and of
 * sinkattn_decode_splitkv_fp8 (NaN codes reported under
 * SINKATTN_DEBUG_CHECKS=1).
 */
SINKATTN_API sinkattn_status sinkattn_decode_splitkv_multi_fp8(
    const void* q, const void* k_cache, const void* v_cache,
    float k_scale, float v_scale,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Multi-token-query decode against a paged cache: the draft-token
 * verification of sinkattn_decode_splitkv_multi, with the keys and values in
 * the pages of sinkattn_decode_paged.  The result equals
 * sinkattn_decode_splitkv_multi's on the gathered cache (sequence b's newest
 * Lq_b tokens are its queries, bottom-right causal, optional window).
 *
 *   q, cu_seqlens_q, max_seqlen_q, total_q, o, lse
 *                  as sinkattn_decode_splitkv_multi
 *   k_pages, v_pages, block_table, seq_lens, max_pages, page_size,
 *   num_pages, max_seqlen_k
 *                  as sinkattn_decode_paged (seq_lens holds Lk_b)
 *   window, softmax_scale, num_splits
 *                  as sinkattn_decode_splitkv
 *   workspace      sized by sinkattn_decode_workspace_bytes(total_q,
 *                  num_q_heads, head_dim, num_splits)
 *
 * Device-side preconditions: those of both entry points, 0 <= Lq_b <= Lk_b
 * among them (SINKATTN_DEBUG_CHECKS=1 reports violations).  Page ids outside
 * the pool are clamped into it.
 */
SINKATTN_API sinkattn_status sinkattn_decode_paged_multi(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t batch,
    int32_t max_pages, int32_t page_size, int32_t num_pages,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * Multi-token-query decode against a paged cache of E4M3 codes: the queries
 * of sinkattn_decode_paged_multi with the pages and per-tensor scales of
 * sinkattn_decode_paged_fp8 (vLLM, FlashInfer integration: FP8 KV cache;
 * Perplexity, in-house inference engine: speculative and MTP decoders).  The
 * result equals sinkattn_decode_splitkv_multi_fp8 on the gathered cache.
 *
 *   k_pages,
 *   v_pages        uint8 E4M3 codes [num_pages, page_size, num_kv_heads,
 *                  head_dim]
 *   k_scale,
 *   v_scale        host floats, finite and > 0
 *   (the other arguments as sinkattn_decode_paged_multi)
 *
 * Preconditions and errors: those of sinkattn_decode_paged_multi and of
 * sinkattn_decode_paged_fp8.
 */
SINKATTN_API sinkattn_status sinkattn_decode_paged_multi_fp8(
    const void* q, const void* k_pages, const void* v_pages,
    float k_scale, float v_scale,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t batch,
    int32_t max_pages, int32_t page_size, int32_t num_pages,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
    const float* sinks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t window, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes,
    void* o, float* lse, void* stream);

/*
 * The rotary step before attention, fused: rotate the query heads into q_out
 * and write the rotated key heads and the value heads of each new token into
 * its cache row (vLLM, "GPT-OSS performance optimizations on NVIDIA
 * Blackwell", minimum latency: RoPE + Q + cache fusion; NVIDIA gpt-oss
 * announcement, model description: RoPE; Perplexity, "GPT-OSS on day 0",
 * Hopper section: YaRN position encoding).  The pages give no formula; the
 * rotation is the RoFormer one with dimension i pairing with i + head_dim/2:
 *     (x_i, x_{i+32}) -> m * (x_i cos a - x_{i+32} sin a, x_{i+32} cos a + x_i sin a),
 *     a = position * f_i,  f_i = rope_theta^(-2i/64),
 * and for yarn_factor s > 1 YaRN's NTK-by-parts rescaling (Peng et al.) in
 * the form its own code and the GPT-OSS / DeepSeek-V3 models use: with
 * L = yarn_original_max_position, the pair index at which a frequency turns
 * beta times over the original context is c(beta) = 32 ln(L / (2 pi beta)) /
 * ln(rope_theta); low = c(yarn_beta_fast), high = c(yarn_beta_slow) (floor
 * and ceil when yarn_truncate != 0, as DeepSeek-V3; unrounded when 0, as
 * GPT-OSS), clamped to [0, 63]; gamma_i = clamp((i - low) / (high - low), 0,
 * 1) and f_i -> (1 - gamma_i) f_i + gamma_i f_i / s; the temperature
 * m = 0.1 ln s + 1 (m = 1 for s <= 1).
 *
 *   qkv           bf16 [num_tokens, num_q_heads + 2 num_kv_heads, head_dim]:
 *                 the q heads, then the k heads, then the v heads of a token
 *   positions     int32 [num_tokens], device: each token's position
 *   slot_mapping  int32 [num_tokens], device: the cache row of the token's k
 *                 and v (for a paged cache, page * page_size + slot), or -1
 *                 to write none; rows must be distinct
 *   q_out         bf16 [num_tokens, num_q_heads, head_dim] (written)
 *   k_cache,
 *   v_cache       bf16 [cache_rows, num_kv_heads, head_dim]; only the rows
 *                 named by slot_mapping are written (k rotated, v copied)
 *
 * Angles are reduced modulo 2 pi in fp64 before sin / cos in fp32, so the
 * phase of large positions is kept.  Errors: rope_theta must be finite and
 * > 1, yarn_factor finite and > 0, and with yarn_factor > 1 the original
 * context >= 1 and finite yarn_beta_fast > yarn_beta_slow > 0
 * (SINKATTN_ERR_INVALID_ARG); head_dim 64 only.  Slots outside
 * [-1, cache_rows) are skipped; slots out of range or repeated are reported
 * under SINKATTN_DEBUG_CHECKS=1.
 */
SINKATTN_API sinkattn_status sinkattn_rope_qkv_append(
    const void* qkv, const int32_t* positions, const int32_t* slot_mapping, int32_t num_tokens,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    double rope_theta, double yarn_factor, int32_t yarn_original_max_position,
    double yarn_beta_fast, double yarn_beta_slow, int32_t yarn_truncate,
    void* q_out, void* k_cache, void* v_cache, int32_t cache_rows, void* stream);

/*
 * Output projection with bias, the step after attention (Perplexity,
 * "GPT-OSS on day 0", section "GPT-OSS on Hopper": the output projection
 * carries a bias):
 *     y[n, e] = sum_k o[n, k] * W[e, k] + bias[e]
 *
 *   o             bf16 [num_rows, in_features]: attention outputs with the
 *                 query heads concatenated (the o of the attention entry
 *                 points viewed as [rows, num_q_heads * head_dim])
 *   w             bf16 [out_features, in_features]: one row per output
 *                 feature
 *   bias          fp32 [out_features], or NULL for none
 *   y             bf16 [num_rows, out_features] (written; fp32 accumulation,
 *                 rounded to nearest even once)
 *
 * in_features must be a multiple of 128 and out_features of 32, and
 * num_rows at most 65535 * 64 (SINKATTN_ERR_UNSUPPORTED otherwise).  Shaped
 * for decode-sized row counts, where the weight is the traffic: the weight is
 * read from memory once per 64 rows, and when the (64-row, 64-feature) tiles
 * alone would leave the chip idle, K is split across workgroups whose fp32
 * partial sums go to the workspace (device, 256-byte aligned, at least
 * sinkattn_oproj_workspace_bytes(num_rows, in_features, out_features) bytes,
 * 0 when no split is made; SINKATTN_ERR_WORKSPACE otherwise) and a second
 * kernel adds them and the bias.  Above 256 rows an LDS-tiled GEMM runs
 * instead (no workspace).  Under SINKATTN_DEBUG_CHECKS=1 NaN / Inf in o or w
 * is reported.
 */
SINKATTN_API size_t sinkattn_oproj_workspace_bytes(int32_t num_rows, int32_t in_features,
                                                  int32_t out_features);
SINKATTN_API sinkattn_status sinkattn_oproj_bias(
    const void* o, const void* w, const float* bias,
    int32_t num_rows, int32_t in_features, int32_t out_features,
    void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Log-sum-exp merge of num_parts partial results, each normalised by its own
 * denominator (the combination step that the split-KV form of the
 * Perplexity page's online softmax implies; the page does not print it):
 *     M = max_s lse_s,  w_s = exp(lse_s - M),
 *     o = sum_s w_s o_s / sum_s w_s,  lse = M + ln(sum_s w_s).
 * A partial with lse = -inf is empty; if all are empty, o = 0, lse = -inf.
 * A sink can be merged as one more partial with lse = z and o = 0.
 *
 *   o_parts    fp32 [num_parts, n, num_heads, head_dim]
 *   lse_parts  fp32 [num_parts, n, num_heads]
 *   o          bf16 [n, num_heads, head_dim]
 *   lse        fp32 [n, num_heads] or NULL
 */
SINKATTN_API sinkattn_status sinkattn_merge_lse(
    const float* o_parts, const float* lse_parts,
    int32_t num_parts, int32_t n, int32_t num_heads, int32_t head_dim,
    void* o, float* lse, void* stream);

/* Message describing the last failed call on this thread ("" if none). */
SINKATTN_API const char* sinkattn_last_error(void);

/* Library version string. */
SINKATTN_API const char* sinkattn_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* SINKATTN_H_ */
