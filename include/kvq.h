/*
 * kvq.h -- paged FP8 / INT8 (and KIVI-style INT4 / INT2) KV cache for MI355X (gfx950).
 *
 * C ABI of libkvq.so.  Every pointer argument except `cache` and `bytes` is a
 * DEVICE pointer owned by the caller; the library never allocates, frees or
 * synchronises.  All work is enqueued on the caller's HIP stream.  Scalars are
 * validated on the host before any HIP call; an invalid request returns a
 * kvq_status other than KVQ_OK and launches nothing.  The contents of device
 * arrays (slot mappings, block tables, context lengths) are the caller's
 * contract and are not read by the host.
 *
 * What the calls compute (pages cited by title and section):
 *  - The KV cache is re-read in full at every decode step and keeps growing by
 *    one K/V row per token ("KV cache FP8로 동시 요청 76배 수용하기",
 *    storycompiler.tistory.com, sections 1-2).
 *  - Quantization happens once, when a token's K/V row is stored, from the
 *    full-precision values; the scales are kept in BF16 next to the codes, and
 *    dequantization is fused into the attention kernel, whose arithmetic stays
 *    in high precision ("KV 캐시 양자화(KV cache quantization): FP8/INT8 K 및 V가
 *    실제로 제공하는 이점과 한계점", molayo1419.me, section "KV 캐시 양자화란
 *    실제로 무엇인가"; "KV Cache 압축", ryotta.opik.net, sections 5.1 and 6.3).
 *  - Formats: FP8 E4M3 (and E5M2, the wider-range, lower-precision FP8) and
 *    INT8 per-token asymmetric with a (scale, zero_point) pair; per-tensor and
 *    per-head static scales (molayo1419.me, formats table notes and the
 *    serving-flag values; ryotta.opik.net section 3.1).  KIVI: K quantized per
 *    channel, V per token, the most recent tokens kept in full precision
 *    (ryotta.opik.net section 3.1, KIVI, an asymmetric 2-bit method;
 *    molayo1419.me formats notes on mixed 4-bit).
 *  - Storage is paged: fixed-size blocks in one pool, mapped per request by a
 *    block table ("FP8 KV Cache부터 INT4 Weight-Only까지", daewooki.github.io,
 *    core concept 2) PagedAttention).
 *  - Accumulation is fp32 (storycompiler.tistory.com, section 4).
 *
 * Numeric definitions (the pages give no formula; these readings are fixed):
 *  FP8 per-(token,head):  s = bf16_ceil(amax / 448), code = e4m3_rne_sat(x / s)
 *  FP8 static:            code = e4m3_rne_sat(x / s_static)
 *  E5M2:                  the same two rules with 57344 and e5m2_rne_sat
 *  INT8 per-(token,head): z = bf16_floor(min), s = bf16_ceil((max - z) / 255),
 *                         code = clamp(rne((x - z) / s), 0, 255), x^ = code*s + z
 *  KIVI INT4 / INT2:      the same asymmetric rule with 15 / 3 steps; K over
 *                         the 32 tokens of a group per channel, V over the
 *                         channels of a token.  s == 0 (constant row) gives
 *                         all-zero codes.
 *  Every "/" is one IEEE float32 division; E4M3 is the OCP encoding (max 448),
 *  E5M2 the OCP encoding (max 57344; saturating, so no infinities are stored).
 *
 * Page records.  A pool holds num_pages x num_kv_heads records; record
 * (page p, head h) starts at byte (p * num_kv_heads + h) * kvq_record_bytes().
 * A record stores, in order:
 *   page_size rows of head_dim code bytes (token-major; INT4 K: head_dim/2
 *   bytes per row, low nibble = even channel; INT4 V: the rows of tokens 2m and
 *   2m + 1 interleaved in 16-bit units, i.e. 32-bit word q of pair row m holds
 *   channels 4q..4q+3 of token 2m in bits 0-15 and of token 2m + 1 in bits
 *   16-31, channel 4q + i in bits 4i..4i+3 of each half;  INT2: half as many
 *   rows, each the INT4 row layout above in which every 4-bit field holds two
 *   2-bit codes, bits 0-1 for the first half of the page's tokens and bits 2-3
 *   for the second: INT2 K row j (64 bytes) holds tokens j and j + 16, INT2 V
 *   pair row m (128 bytes) holds token pairs m and m + 8), then
 *   per-(token,head) modes: page_size bf16 scales, then (INT8) page_size bf16
 *   zero-points;  KIVI K: head_dim bf16 scales then head_dim bf16 zero-points
 *   (one per channel for the page's 32-token group);  KIVI V: page_size bf16
 *   scales then page_size bf16 zero-points;
 *   padded to a multiple of 16 bytes, plus 32 bytes when that size is a
 *   multiple of 1024 (static-scale FP8 records: 2048 -> 2080 at page 16), so
 *   that a page of records is not a power-of-two stride in the pool.
 * Token t of a sequence lives in page block_table[seq][t / page_size], row
 * t % page_size.  slot = page * page_size + row.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_EINVAL = -1,          /* null pointer, negative size, inconsistent descriptor     */
    KVQ_EUNSUPPORTED = -2,    /* well-formed but outside what the kernels implement      */
    KVQ_EWORKSPACE = -3,      /* workspace smaller than kvq_decode_workspace_bytes()     */
    KVQ_EHIP = -4             /* a HIP runtime call or a kernel launch failed            */
} kvq_status;

typedef enum kvq_dtype {
    KVQ_FP8_E4M3 = 1,         /* OCP E4M3, 1 byte per element                            */
    KVQ_INT8_ASYM = 2,        /* u8 code with per-(token,head) scale and zero-point      */
    KVQ_INT4_KIVI = 3,        /* 4-bit codes, K per channel / V per token, fp16 window   */
    KVQ_FP8_E5M2 = 4,         /* OCP E5M2, 1 byte per element; records as KVQ_FP8_E4M3  */
    KVQ_INT2_KIVI = 5         /* 2-bit codes, otherwise as KVQ_INT4_KIVI                  */
} kvq_dtype;

/* Attention options of a cache (kvq_cache.attn_flags). */
typedef enum kvq_attn_flag {
    /* FP8-domain QK (FP8 E4M3 / E5M2 caches): the query row is quantized to
     * E4M3 with the K rows' own rule (s_q = bf16_ceil(amax(q) / 448), codes
     * e4m3_rne_sat(q / s_q)) and QK runs on the FP8 matrix cores:
     *   score_t = softmax_scale * s_q * s_k[t] * (q codes . k codes),
     * i.e. the attention of the dequantized query q^ = s_q * e4m3(q codes)
     * over the cache.  Softmax and PV keep their precision.  Some backends
     * compute attention in FP8 ("FP8 KV Cache부터 INT4 Weight-Only까지",
     * daewooki.github.io, core concept 3).  Not for INT8 or KIVI caches. */
    KVQ_ATTN_FP8_QK = 1,
    /* FP8 score-V product (FP8 E4M3 / E5M2 caches; the same page names QK
     * and the score-V product in the FP8 domain): the weights of each block of
     * 32 tokens from token 0, P_t = 2^(lambda_t - mu) * vs_t (lambda_t the
     * score in log2 units, mu = ceil(max lambda over the block), vs_t the
     * token's V scale), are held as E4M3 codes of P_t / S under the block's
     * smallest power-of-two scale S with max P <= 448 S, and multiply the V
     * codes on the scaled FP8 matrix cores:
     *   out = sum_t 2^(mu - M) S e4m3(P_t / S) vcode_t / sum_t 2^(lambda_t - M).
     * The softmax denominator and lse stay exact (fp32).  Combined with
     * KVQ_ATTN_FP8_QK it gives attention with both products in FP8.  With
     * page size 16, partition_pages counts 32-token blocks.  Not for INT8 or
     * KIVI caches. */
    KVQ_ATTN_FP8_PV = 2
} kvq_attn_flag;

typedef enum kvq_scale_mode {
    KVQ_SCALE_PER_TENSOR = 0,      /* one static bf16 scale for K and one for V (FP8 only) */
    KVQ_SCALE_PER_HEAD = 1,        /* one static bf16 scale per KV head for K and V (FP8)  */
    KVQ_SCALE_PER_TOKEN_HEAD = 2   /* computed at append time per (token, KV head)         */
} kvq_scale_mode;

/* Descriptor of one layer's cache.  Plain data; the library keeps no copy. */
typedef struct kvq_cache {
    int32_t dtype;            /* kvq_dtype                                               */
    int32_t scale_mode;       /* kvq_scale_mode; INT8 and KIVI need PER_TOKEN_HEAD       */
    int32_t num_pages;        /* pages in each pool                                      */
    int32_t page_size;        /* tokens per page: 16 or 32 (KIVI: 32 = the group size)   */
    int32_t num_kv_heads;     /* >= 1                                                    */
    int32_t head_dim;         /* 128                                                     */
    void* k_pages;            /* device: num_pages*num_kv_heads K records                */
    void* v_pages;            /* device: num_pages*num_kv_heads V records                */
    const void* static_scales;/* device bf16; PER_TENSOR: [2] = {K, V};
                                 PER_HEAD: [2][num_kv_heads]; otherwise NULL             */
    /* KIVI (INT4 / INT2) only: fp16 recent-token window, a ring of window_tokens rows
       per (sequence, KV head); token t sits at row t % window_tokens.          */
    void* k_window;           /* device fp16 [max_seqs][num_kv_heads][window_tokens][head_dim] */
    void* v_window;
    int32_t max_seqs;         /* rows of the window arrays                               */
    int32_t window_tokens;    /* residual + page_size (160 for residual 128, group 32)   */
    int32_t residual;         /* tokens always kept in fp16 (128)                        */
    int32_t attn_flags;       /* kvq_attn_flag bits read by the decode / verify entry
                                 points (0: query and probabilities in bf16 / fp32
                                 precision); the append calls ignore it */
} kvq_cache;

/* Bytes of one page record: which = 0 for K, 1 for V.  0 for an invalid combination. */
size_t kvq_record_bytes(int32_t dtype, int32_t scale_mode, int32_t page_size,
                        int32_t head_dim, int32_t which);

/* Quantize-on-append (FP8 E4M3 / E5M2, INT8; a KIVI cache returns
 * KVQ_EUNSUPPORTED, it has kvq_kivi_append).  Each new token's K and V rows
 * are quantized once, at store time, from the full-precision values, and
 * their BF16 scale (and zero-point) is stored beside the codes ("KV 캐시
 * 양자화(KV cache quantization) ...", molayo1419.me, section "KV 캐시 양자화란
 * 실제로 무엇인가", the storage-side steps of its pipeline; "KV Cache 압축",
 * ryotta.opik.net, section 5.1 steps 1-3).  Per-token scales are per (token,
 * KV head) row; per-tensor and per-head scales are the caller's static ones
 * (molayo1419.me, formats-table notes).
 * k, v:          device bf16 [num_tokens][num_kv_heads][head_dim], contiguous.
 * slot_mapping:  device int32 [num_tokens]; slot = page*page_size + row; a
 *                negative slot (or one beyond the pool) skips that token.
 * Writes the token's code row, scale and zero-point into its page record for K
 * and for V.  Two tokens with the same slot race. */
kvq_status kvq_append(const kvq_cache* cache, const void* k, const void* v,
                      const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream);

/* KIVI-style append (cache->dtype KVQ_INT4_KIVI or KVQ_INT2_KIVI): new tokens of each
 * sequence enter the fp16 window; whole 32-token groups leave it, oldest
 * first, once it would hold more than cache->residual tokens, and are written
 * quantized (K per channel over the group, V per token) into the page that
 * block_table[b][group index] names.  A sequence of n tokens thus holds its
 * first n_q = 32 * floor(max(0, n - residual) / 32) tokens as INT4 / INT2 pages and
 * tokens [n_q, n) as fp16 window rows (token t at row t % window_tokens).
 * k, v:           device bf16 [total new tokens][num_kv_heads][head_dim]; the
 *                 rows of sequence b are [token_offsets[b], token_offsets[b+1]).
 * token_offsets:  device int32 [num_seqs + 1], non-decreasing.
 * context_lens:   device int32 [num_seqs]: tokens sequence b holds BEFORE this
 *                 call (the caller adds the new count afterwards).
 * block_table:    device int32 [num_seqs][max_pages_per_seq].
 * max_new_tokens: host bound on token_offsets[b+1] - token_offsets[b] (grid
 *                 size); larger counts are the caller's error.
 * Sequence b uses window slot b (num_seqs <= cache->max_seqs).  fp16 window
 * values are the bf16 inputs rounded to nearest-even; the quantizers read
 * those fp16 values.  Requires page_size 32 and window_tokens >= residual + 32.
 * KIVI (ryotta.opik.net "KV Cache 압축" section 3.1: asymmetric 2-bit, K per
 * channel, V per token, recent tokens in full precision; molayo1419.me
 * formats-table notes on mixed-precision 4-bit). */
kvq_status kvq_kivi_append(const kvq_cache* cache, const void* k, const void* v,
                           const int32_t* token_offsets, const int32_t* context_lens,
                           const int32_t* block_table, int32_t max_pages_per_seq, int32_t num_seqs,
                           int32_t max_new_tokens, hipStream_t stream);

/* Workspace bytes that kvq_decode_attention, kvq_kivi_decode_attention and
 * kvq_decode_split / kvq_decode_reduce need for this shape: a 256-byte
 * header, num_seqs + 1 ints, and partial results of (ranges + num_seqs) slots
 * per KV head, each slot num_q_heads / num_kv_heads rows of 129 floats.  The
 * automatic plan has at most 2048 ranges over all KV heads, whatever the
 * device; partition_pages > 0 (as in kvq_decode_attention) sizes for that
 * forced range length instead.  Depends only on the descriptor's page size
 * and KV heads and the arguments; no HIP call. */
kvq_status kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_context_len,
                                      int32_t partition_pages, size_t* bytes);

/* One decode step of attention for one query token per sequence, reading the
 * quantized paged FP8 / INT8 cache with dequantization fused in (KIVI caches:
 * kvq_kivi_decode_attention; here they return KVQ_EUNSUPPORTED):
 *   out[b][h] = sum_t softmax_t(softmax_scale * q[b][h] . k^[t]) v^[t]
 * over every cached token t < context_lens[b] of KV head h / (num_q_heads /
 * num_kv_heads).  fp32 accumulation, flash-decoding split over the context.
 * Every cached K and V row is read again at each decode step, so the step is
 * bound by the bytes the cache holds ("KV cache FP8로 동시 요청 76배 수용하기",
 * storycompiler.tistory.com, sections 1 and 4; "FP8 KV Cache부터 INT4
 * Weight-Only까지", daewooki.github.io, core concept 1); dequantization
 * happens inside the attention kernel, whose arithmetic stays in high
 * precision with fp32 accumulation (ryotta.opik.net "KV Cache 압축", section
 * 5.1 steps 4-5 and the kernel-fusion note; storycompiler.tistory.com,
 * section 4); pages come from a per-request block table over one pool
 * (daewooki.github.io, core concept 2) PagedAttention).
 * q:             device bf16 [num_seqs][num_q_heads][head_dim]
 * block_table:   device int32 [num_seqs][max_pages_per_seq]
 * context_lens:  device int32 [num_seqs]; values above max_context_len are
 *                clamped to it; 0 gives out = 0 and lse = -inf.
 * max_context_len: host bound on context_lens (<= max_pages_per_seq*page_size).
 * partition_pages: 0 = balance the work over the resident waves of the device;
 *                >0 = pages of work per wave (testing and tuning).
 * workspace:     device scratch of at least kvq_decode_workspace_bytes().
 * out:           device fp32 [num_seqs][num_q_heads][head_dim]
 * lse:           device fp32 [num_seqs][num_q_heads] natural-log sum-exp of the
 *                scaled scores, or NULL.
 * num_q_heads / num_kv_heads must be 1, 2, 4, 8 or 16, and num_seqs at most
 * 16383 (the kernels keep a per-sequence work table in LDS); beyond either,
 * KVQ_EUNSUPPORTED. */
kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int32_t num_seqs,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float softmax_scale,
                                int32_t partition_pages, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * kvq_decode_attention with the workspace in a static device array of the
 * library, 32 MiB per device (allocated when the library's code is loaded on
 * a device, held until the process ends; its address is looked up on the
 * first call on each device).  Arguments, results and errors as
 * kvq_decode_attention; a shape whose workspace
 * (kvq_decode_workspace_bytes) exceeds 32 MiB returns KVQ_EWORKSPACE and
 * launches nothing.  The call allocates and frees nothing.  All calls on one
 * device share that array: calls that overlap in time on one device (other
 * streams, other threads) race and give wrong results; calls in one stream
 * are ordered.  Nothing in the array needs to start at zero: each call
 * writes what it reads. */
kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int32_t num_seqs,
                                        int32_t num_q_heads, const int32_t* block_table,
                                        int32_t max_pages_per_seq, const int32_t* context_lens,
                                        int32_t max_context_len, float softmax_scale,
                                        int32_t partition_pages, float* out, float* lse,
                                        hipStream_t stream);

/* KIVI-style decode step (cache->dtype KVQ_INT4_KIVI or KVQ_INT2_KIVI; other
 * caches return KVQ_EUNSUPPORTED): the same attention as
 * kvq_decode_attention over tokens held as 4-bit or 2-bit pages (K quantized
 * per channel over each 32-token group, V per token) followed by the fp16
 * window of the most recent tokens, sequence b reading window slot b
 * ("KV Cache 압축", ryotta.opik.net, section 3.1, KIVI: K per channel and V
 * per token, a full-precision window of recent tokens; molayo1419.me,
 * formats-table notes on mixed-precision 4-bit).  Arguments, layouts and
 * errors as kvq_decode_attention; the workspace comes from
 * kvq_decode_workspace_bytes. */
kvq_status kvq_kivi_decode_attention(const kvq_cache* cache, const void* q, int32_t num_seqs,
                                     int32_t num_q_heads, const int32_t* block_table,
                                     int32_t max_pages_per_seq, const int32_t* context_lens,
                                     int32_t max_context_len, float softmax_scale,
                                     int32_t partition_pages, void* workspace, size_t workspace_bytes,
                                     float* out, float* lse, hipStream_t stream);

/* The two launches of kvq_decode_attention and kvq_kivi_decode_attention
 * (every cache dtype), exposed separately so that each
 * kernel can be timed and a context-sharded caller can run the merge itself.
 * kvq_decode_split writes every (sequence, head) whose context one wave covers
 * straight to out/lse and the others as partial results into the workspace;
 * kvq_decode_reduce merges the partial results with log-sum-exp weights,
 * the exact identity for softmax attention over a union of disjoint token
 * sets (out = sum_i e^(lse_i - L) out_i / sum_i e^(lse_i - L), L = max_i
 * lse_i).  Call them in this order on one stream with identical arguments. */
kvq_status kvq_decode_split(const kvq_cache* cache, const void* q, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float softmax_scale,
                            int32_t partition_pages, void* workspace, size_t workspace_bytes,
                            float* out, float* lse, hipStream_t stream);
kvq_status kvq_decode_reduce(const kvq_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                             int32_t max_context_len, int32_t partition_pages,
                             void* workspace, size_t workspace_bytes,
                             float* out, float* lse, hipStream_t stream);

/* Speculative-decoding verification over the quantized paged cache: the
 * target model scores the q_len = K + 1 newest positions of each sequence in
 * one pass, reading the FP8 / INT8 cache and dequantizing as it reads
 * ("KV 캐시 양자화(KV cache quantization) ...", molayo1419.me, section on the
 * interaction with speculative decoding).  The K/V rows of those positions
 * must already be in the cache (kvq_append), so context_lens[b] counts them.
 * Position i of sequence b (0 = oldest of the q_len) attends causally:
 *   out[b][i][h] = sum_t softmax_t(softmax_scale * q[b][i][h] . k^[t]) v^[t]
 * over t < context_lens[b] - (q_len - 1 - i); a position that sees no token
 * (context_lens[b] < q_len) gets out = 0 and lse = -inf.  q_len = 1 is
 * kvq_decode_attention.
 * q:     device bf16 [num_seqs][q_len][num_q_heads][head_dim]
 * out:   device fp32 [num_seqs][q_len][num_q_heads][head_dim]
 * lse:   device fp32 [num_seqs][q_len][num_q_heads] or NULL
 * Other arguments as kvq_decode_attention; the workspace size comes from
 * kvq_verify_workspace_bytes.  The q_len x (num_q_heads / num_kv_heads) query
 * rows of a KV head are one 16-row tile: their product must be <= 16
 * (KVQ_EUNSUPPORTED otherwise).  KIVI caches (INT4 / INT2 pages plus the
 * fp16 window) need q_len - 1 <= cache->residual, so that every position a
 * row cannot see is a window token (KVQ_EUNSUPPORTED otherwise).  The KV
 * bytes are read once for all q_len rows. */
kvq_status kvq_verify_workspace_bytes(const kvq_cache* cache, int32_t num_seqs, int32_t q_len,
                                      int32_t num_q_heads, int32_t max_context_len,
                                      int32_t partition_pages, size_t* bytes);
kvq_status kvq_verify_attention(const kvq_cache* cache, const void* q, int32_t num_seqs, int32_t q_len,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float softmax_scale,
                                int32_t partition_pages, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream);
/* The two launches of kvq_verify_attention (split over the context, then the
 * log-sum-exp merge), as kvq_decode_split / kvq_decode_reduce are for
 * kvq_decode_attention: call them in this order on one stream with identical
 * arguments. */
kvq_status kvq_verify_split(const kvq_cache* cache, const void* q, int32_t num_seqs, int32_t q_len,
                            int32_t num_q_heads, const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, float softmax_scale,
                            int32_t partition_pages, void* workspace, size_t workspace_bytes, float* out,
                            float* lse, hipStream_t stream);
kvq_status kvq_verify_reduce(const kvq_cache* cache, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                             int32_t max_context_len, int32_t partition_pages, void* workspace,
                             size_t workspace_bytes, float* out, float* lse, hipStream_t stream);

/* Static text for a status code. */
const char* kvq_status_string(kvq_status status);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
