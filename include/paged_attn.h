/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged single-query decode
 * attention library, V2 split: per-partition online-softmax attention, then
 * a cross-partition log-sum-exp reduce, with grouped-query head mapping.
 *
 * The operation is the one defined on the page "paged_attention_v2_triton.py
 * -- Triton PagedAttention V2 for BI-V100": its phase-1 partition kernel,
 * its phase-2 reduce kernel, and the host launcher that fixes the tensor
 * layouts and the caller-allocated outputs.
 *
 * Conventions for every entry point below
 *  - All tensor pointers are DEVICE pointers on the current HIP device, in
 *    the dense row-major layouts stated per argument. The caller owns every
 *    buffer; the library never allocates, frees, copies to the host or
 *    synchronises. Work is enqueued on `stream` (a hipStream_t; NULL is the
 *    null stream) and the call returns.
 *  - x = 16 / sizeof(kv element): 4 for fp32, 8 for fp16 / bf16.
 *  - S = num_seqs, H = num_heads, KH = num_kv_heads, G = H / KH (query heads
 *    per kv head; query head h reads kv head h / G), D = head_size,
 *    BS = block_size, B = num_blocks, MB = max_blocks_per_seq,
 *    P = max_num_partitions, PS = partition_size.
 *  - Return value: PA_OK, or a negative PA_ERR_* code with a message readable
 *    through paged_attn_last_error() on the calling thread. Argument errors
 *    are detected on the host before anything is enqueued.
 *  - Preconditions the library cannot check without synchronising (the
 *    caller guarantees them): 0 <= seq_lens[s] <= min(P * PS, MB * BS);
 *    block_tables[s][i] in [0, B) for i < ceil(seq_lens[s] / BS); entries past
 *    that are never read and may hold anything (e.g. -1). Cache slots that no
 *    sequence reads (unreferenced blocks, tail slots of a last block) never
 *    influence any result, whatever they hold (NaN included).
 *  - Outputs must not alias inputs (paged_attn_merge_states states its
 *    in-place exception). Calls on one stream are ordered; the functions keep
 *    no state between calls and are safe to call from several threads on
 *    different streams. No call allocates, fills memory or waits, so calls
 *    may be captured into a HIP graph and replayed.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PA_API __attribute__((visibility("default")))
#else
#define PA_API
#endif

/* Element types of query / key_cache / value_cache (and of `out`).
 * PA_FP8_E4M3 is the OCP 8-bit E4M3 format ("e4m3fn": bias 7, no infinities,
 * largest finite 448); it is a cache type only, taken by the *_fp8 entry
 * points below and by the two sizing queries at the end. */
enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 };

/* Status codes. */
enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                              */
  PA_ERR_SHAPE = -2,       /* negative size, H % KH, D % x, PS <= 0 or PS % BS, P < 1,
                              MB < 1, B < 1                                            */
  PA_ERR_UNSUPPORTED = -3, /* D not in {64,128,256}, BS not in {16,32}, G > 4 with
                              fp32 data, PS / BS > 256, unknown dtype, or out_dtype
                              neither PA_F32 nor kv_dtype                              */
  PA_ERR_ALIGN = -4,       /* a pointer lacks its alignment (16 bytes; lse arrays 4)  */
  PA_ERR_HIP = -5          /* the HIP runtime rejected a launch                        */
};

/*
 * Phase 1 (the page's partition kernel). For every sequence s, kv head kh and
 * partition p < P, over the tokens t in [p*PS, min((p+1)*PS, seq_lens[s])):
 *   score(h, t)       = scale * dot(query[s][h], K_t)   for the G heads h of kh
 *   max_logits[s][h][p] = max_t score
 *   exp_sums[s][h][p]   = sum_t exp(score - max)
 *   tmp_output[s][h][p] = sum_t exp(score - max) * V_t / exp_sums  (normalised)
 * where K_t / V_t are gathered from physical block block_tables[s][t / BS],
 * slot t % BS. A partition with no tokens gets max_logits = -inf,
 * exp_sums = 0 and its tmp_output row is left untouched.
 *
 *   tmp_output   [S, H, P, D] fp32, written
 *   exp_sums     [S, H, P]    fp32, written
 *   max_logits   [S, H, P]    fp32, written
 *   query        [S, H, D]            kv_dtype
 *   key_cache    [B, KH, D/x, BS, x]  kv_dtype
 *   value_cache  [B, KH, D, BS]       kv_dtype
 *   block_tables [S, MB] int32
 *   seq_lens     [S]     int32
 *   scale        multiplies q.k (applied after the dot product)
 *   kv_dtype     PA_F32, PA_F16 or PA_BF16
 * num_seqs == 0 is a successful no-op. Any G with 16-bit data; G <= 4 with
 * fp32. (With G > 32, or G > 16 at D = 256, the heads of a kv head are
 * computed in several launches over the same pages, each reading them again.)
 */
PA_API int paged_attn_v2_partition(float* tmp_output, float* exp_sums, float* max_logits,
                                   const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                   int32_t partition_size, float scale, int32_t kv_dtype,
                                   void* stream);

/*
 * Phase 2 (the page's reduce kernel). For every (s, h), over the
 * n = ceil(seq_lens[s] / PS) partitions the sequence uses:
 *   M = max_p max_logits, Z = sum_p exp(max_logits - M) * exp_sums,
 *   out[s][h] = sum_p exp(max_logits - M) * exp_sums / Z * tmp_output[s][h][p]
 * and out[s][h] = 0 when n == 0. Entries of partitions p >= n never affect
 * the result (NaN there is fine): the statistics of a row's first 64
 * partitions are loaded together with its length, before n is known, and
 * those past n are discarded; tmp_output rows past n are never read, except
 * that with max_num_partitions == 1 each row's single row is loaded together
 * with its statistics (one round trip) and discarded when n == 0. With one
 * partition the weight is exactly 1: out[s][h] is tmp_output[s][h][0], cast.
 *
 *   out          [S, H, D] in out_dtype (PA_F32, or the kv dtype: round to
 *                nearest even from the fp32 result), written
 *   tmp_output, exp_sums, max_logits, seq_lens: as written by phase 1
 * num_seqs == 0 is a successful no-op.
 */
PA_API int paged_attn_v2_reduce(void* out, const float* tmp_output, const float* exp_sums,
                                const float* max_logits, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                int32_t max_num_partitions, int32_t partition_size,
                                int32_t out_dtype, void* stream);

/*
 * Phase 1 then phase 2 on one stream (the page's host launcher): the same
 * arguments and the same `out` as the two calls above, up to fp32 rounding.
 * Every partition of PS tokens is still computed on its own (its max logit,
 * exp sum and normalised row, exactly as phase 1 defines them), and the
 * partitions are combined with phase 2's log-sum-exp rule, but the combine
 * runs where the data already is: a workgroup that holds C consecutive
 * partitions of a (sequence, kv head) combines them in on-chip memory. When
 * its C partitions are all of a row's (P <= C), it writes `out` itself and
 * no second kernel runs; otherwise it stores one combined entry per span of
 * C partitions (statistics and row, in the first ceil(P / C) entries of each
 * row of the workspace) and the reduce combines those entries as partitions
 * of C * PS tokens. C is the launch plan's span (paged_attn_partition_span).
 *
 * tmp_output / exp_sums / max_logits are workspace the caller allocates
 * ([S,H,P,D], [S,H,P], [S,H,P] fp32) and may reuse across calls on the same
 * stream; their contents after this call are unspecified (they may be left
 * unwritten). Phase 1's per-partition rows and statistics are produced by
 * paged_attn_v2_partition.
 */
PA_API int paged_attn_decode(void* out, float* tmp_output, float* exp_sums, float* max_logits,
                             const void* query, const void* key_cache, const void* value_cache,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, int32_t num_blocks,
                             int32_t max_blocks_per_seq, int32_t max_num_partitions,
                             int32_t partition_size, float scale, int32_t kv_dtype,
                             int32_t out_dtype, void* stream);

/*
 * 8-bit key/value caches with per-tensor scales. The page's launcher carries
 * a cache dtype and scalar k_scale / v_scale arguments (Triton PagedAttention
 * V2 for BI-V100, host launcher) and the head all-to-all page moves e4m3fn
 * tensors; neither states the arithmetic, so the reading taken is the plain
 * one: a stored key byte stands for decode(byte) * k_scale and a value byte
 * for decode(byte) * v_scale, everything else as in the two phases above.
 *
 *   query        [S, H, D]           q_dtype: PA_F16 or PA_BF16
 *   key_cache    [B, KH, D/16, BS, 16] E4M3 bytes (x = 16 / 1)
 *   value_cache  [B, KH, D, BS]      E4M3 bytes
 *   k_scale, v_scale                 finite fp32 scalars (PA_ERR_SHAPE otherwise)
 *   outputs as above (fp32 tmp_output / exp_sums / max_logits); the reduce is
 *   the ordinary paged_attn_v2_reduce; out_dtype of the decode is PA_F32 or
 *   q_dtype. Stored NaN bytes in slots the sequences reference are not
 *   covered; slots past a sequence's length may hold anything.
 * The same errors as the 16-bit calls; the plain entry points reject
 * kv_dtype == PA_FP8_E4M3 with PA_ERR_UNSUPPORTED.
 */
PA_API int paged_attn_v2_partition_fp8(float* tmp_output, float* exp_sums, float* max_logits,
                                       const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_size, int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                       int32_t partition_size, float scale, float k_scale,
                                       float v_scale, int32_t q_dtype, void* stream);

PA_API int paged_attn_decode_fp8(void* out, float* tmp_output, float* exp_sums,
                                 float* max_logits, const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                 int32_t num_blocks, int32_t max_blocks_per_seq,
                                 int32_t max_num_partitions, int32_t partition_size, float scale,
                                 float k_scale, float v_scale, int32_t q_dtype, int32_t out_dtype,
                                 void* stream);

/*
 * Several query tokens per sequence (speculative decoding, chunked prefill
 * over the paged cache). The Triton PagedAttention V2 page takes its gather
 * from a multi-row (BLOCK_M) prefill kernel; the Flash Attention Metal page's
 * forward kernel masks keys later than the query position. Reading taken:
 * the M query tokens of sequence s are its last M positions (their keys and
 * values are already in the cache, seq_lens counts them), so query token m
 * sits at L - M + m and attends to keys t <= L - M + m (none if that is
 * negative: its output row is 0). Everything else is per (sequence, query
 * token, head) row:
 *
 *   query        [S, M, H, D]        q_dtype: PA_F16 or PA_BF16
 *   key_cache / value_cache          as above, kv_dtype == q_dtype or PA_FP8_E4M3
 *                                    (k_scale / v_scale apply to 8-bit caches;
 *                                    pass 1 for 16-bit ones)
 *   tmp_output   [S, M, H, P, D] fp32, exp_sums / max_logits [S, M, H, P] fp32
 *   out          [S, M, H, D]        out_dtype PA_F32 or q_dtype
 *
 * A row's partitions past its causal prefix get the sentinels (max -inf, sum
 * 0; tmp_output unspecified). Phase 1 computes one MFMA column per (query
 * token, head) of a kv head, up to 32 columns per pass over the pages (16 at
 * D = 256): when (H / KH) * M is larger, consecutive passes take the next
 * columns (token-major), each reading the K/V pages again (results are the
 * same as in one pass).
 * num_queries = 1 computes exactly what the single-query calls compute.
 */
PA_API int paged_attn_v2_partition_mq(float* tmp_output, float* exp_sums, float* max_logits,
                                      const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t num_queries, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_size,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                      int32_t partition_size, float scale, float k_scale,
                                      float v_scale, int32_t q_dtype, int32_t kv_dtype,
                                      void* stream);

PA_API int paged_attn_v2_reduce_mq(void* out, const float* tmp_output, const float* exp_sums,
                                   const float* max_logits, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                   int32_t head_size, int32_t max_num_partitions,
                                   int32_t partition_size, int32_t out_dtype, void* stream);

PA_API int paged_attn_decode_mq(void* out, float* tmp_output, float* exp_sums, float* max_logits,
                                const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_queries,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                int32_t partition_size, float scale, float k_scale,
                                float v_scale, int32_t q_dtype, int32_t kv_dtype,
                                int32_t out_dtype, void* stream);

/*
 * Row log-sum-exp export. The Flash Attention Metal page's forward kernel
 * stores, next to each normalised output row, the log-sum-exp of the row's
 * scores, m + log(l). Here, for each (sequence, query token, head) row,
 *
 *   lse[row] = M + ln Z,   M = max_p m_p,  Z = sum_p exp(m_p - M) l_p
 *
 * over the row's used partitions, i.e. ln sum_t exp(s_t) over the row's
 * keys (natural log, fp32); -inf for a row with no keys. (out, lse) is the
 * state paged_attn_merge_states combines.
 *
 *   lse   float [S, M, H] (M = num_queries; M = 1 for single-query decode),
 *         4-byte aligned, caller-owned; NULL -> PA_ERR_NULL
 *
 * paged_attn_v2_reduce_lse is paged_attn_v2_reduce_mq plus lse (out is the
 * same bits); paged_attn_decode_lse is paged_attn_decode_mq plus lse (any
 * query / cache dtype pair the other decode calls accept, k_scale / v_scale
 * as for paged_attn_decode_mq). Other arguments and errors as there.
 */
PA_API int paged_attn_v2_reduce_lse(void* out, float* lse, const float* tmp_output,
                                    const float* exp_sums, const float* max_logits,
                                    const int32_t* seq_lens, int32_t num_seqs,
                                    int32_t num_queries, int32_t num_heads, int32_t head_size,
                                    int32_t max_num_partitions, int32_t partition_size,
                                    int32_t out_dtype, void* stream);

PA_API int paged_attn_decode_lse(void* out, float* lse, float* tmp_output, float* exp_sums,
                                 float* max_logits, const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t num_queries,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                 int32_t partition_size, float scale, float k_scale,
                                 float v_scale, int32_t q_dtype, int32_t kv_dtype,
                                 int32_t out_dtype, void* stream);

/*
 * The general form of the two phases: any query / cache dtype pair the other
 * calls accept, one or several query tokens per sequence, optional row
 * log-sum-exp, optional ALiBi position bias.
 *
 * ALiBi. The Triton PagedAttention V2 page's launcher takes per-head
 * alibi_slopes and never reads them; the pages give no formula. Reading
 * taken: the published ALiBi definition (Press, Smith and Lewis, "Train
 * Short, Test Long", ICLR 2022): the score of the key at position t for a
 * query at position i gains slope_h * (t - i) after the scaling of the dot
 * product, i = L - 1 for single-query decode and L - M + m for query token m
 * of M (so the bias is 0 at the query's own position and negative before
 * it). max_logits and lse include the bias.
 *
 *   alibi_slopes  float [num_heads] (query heads), 4-byte aligned, device
 *                 memory read by the partition kernels; NULL: no bias (the
 *                 same kernels and bits as the other calls)
 *   lse           as for paged_attn_decode_lse, or NULL to skip it
 *
 * Other arguments, layouts and errors as for paged_attn_v2_partition_mq /
 * paged_attn_decode_mq (query [S, M, H, D]; M = 1 is single-query decode with
 * query [S, H, D]).
 */
PA_API int paged_attn_v2_partition_ex(float* tmp_output, float* exp_sums, float* max_logits,
                                      const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t num_queries, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_size,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                      int32_t partition_size, float scale, float k_scale,
                                      float v_scale, const float* alibi_slopes,
                                      int32_t q_dtype, int32_t kv_dtype, void* stream);

PA_API int paged_attn_decode_ex(void* out, float* lse, float* tmp_output, float* exp_sums,
                                float* max_logits, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_queries,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                int32_t partition_size, float scale, float k_scale,
                                float v_scale, const float* alibi_slopes, int32_t q_dtype,
                                int32_t kv_dtype, int32_t out_dtype, void* stream);

/*
 * paged_attn_decode_ex without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the span entries live in a static
 * 32 MiB array of device memory that each GPU the library is loaded on holds
 * until the process ends. Nothing is allocated or freed by the call. Same
 * arguments as paged_attn_decode_ex minus tmp_output / exp_sums / max_logits,
 * same results bit for bit.
 *  - The workspace the launch plan needs, num_seqs * num_queries * num_heads *
 *    entries * (head_size + 2) * 4 bytes (entries = span entries per row,
 *    paged_attn_decode_plan; with one span per row it is never touched),
 *    must fit the 32 MiB: larger calls return PA_ERR_UNSUPPORTED and enqueue
 *    nothing.
 *  - Every call on one GPU shares that GPU's array: calls that overlap on a
 *    GPU (other streams, other host threads) race and must be serialised by
 *    the caller. Nothing in the array needs to start at zero.
 */
PA_API int paged_attn_decode_noalloc(void* out, float* lse, const void* query,
                                     const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, const int32_t* seq_lens,
                                     int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_size,
                                     int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_num_partitions,
                                     int32_t partition_size, float scale, float k_scale,
                                     float v_scale, const float* alibi_slopes, int32_t q_dtype,
                                     int32_t kv_dtype, int32_t out_dtype, void* stream);

/*
 * Merge two attention states of the same rows computed over disjoint key sets
 * (a shared prefix and a per-request suffix, or two shards of one long
 * sequence) into the state over their union: the Triton PagedAttention V2
 * page's reduce combine for two parts, each part's (max, exp-sum) pair folded
 * into its lse. Per row, with Mx = max(lse_a, lse_b) and w = exp(lse - Mx):
 *
 *   out     = (w_a a + w_b b) / (w_a + w_b)
 *   out_lse = Mx + ln(w_a + w_b)
 *
 * both lse -inf (no keys on either side) -> out = 0, out_lse = -inf; one side
 * -inf -> the other side's row (the -inf side's row is never used, whatever it
 * holds, NaN included). fp32 arithmetic, one rounding to `dtype` at the end.
 *
 *   a, b, out          [num_rows, head_size] of `dtype` (PA_F32, PA_F16 or
 *                      PA_BF16), 16-byte aligned
 *   lse_a, lse_b       float [num_rows], finite or -inf (a NaN or +inf lse
 *                      gives NaN rows), 4-byte aligned
 *   out_lse            float [num_rows], or NULL to skip it
 *
 * out may be the same pointer as a or b, and out_lse as lse_a or lse_b
 * (in-place merge); partially overlapping buffers are not allowed.
 * head_size in {64, 128, 256}. num_rows == 0 is a no-op. Errors: PA_ERR_SHAPE,
 * PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_UNSUPPORTED, PA_ERR_HIP (launch).
 */
PA_API int paged_attn_merge_states(void* out, float* out_lse, const void* a, const float* lse_a,
                                   const void* b, const float* lse_b, int64_t num_rows,
                                   int32_t head_size, int32_t dtype, void* stream);

/* Text of the last nonzero return on this thread ("" if none). Owned by the
 * library; valid until the next call on the same thread. */
PA_API const char* paged_attn_last_error(void);

/* Version of this ABI (incremented on any incompatible change). 2: the decode
 * calls leave their workspace unspecified (partitions combined in the kernel). */
PA_API int paged_attn_abi_version(void);

/* Partition size the library is tuned for at this geometry (a multiple of
 * block_size); results do not depend on the partition size beyond rounding.
 * Returns a PA_ERR_* code for an unsupported geometry. */
PA_API int paged_attn_default_partition_size(int32_t head_size, int32_t block_size, int32_t kv_dtype,
                                             int32_t group);

/* Partition size for a single-query batch: the longest of 4096 (2048 for
 * 8-bit caches), 2048, 1024, 512, 256 and 128 tokens whose partitions give
 * every workgroup the current device holds at once a work unit
 * (num_seqs * num_kv_heads * ceil(max_seq_len / size) units), else 128; never
 * longer than the shortest candidate >= max_seq_len. Large batches get long
 * partitions (fewer per-partition outputs to write and reduce), small ones
 * enough parallel work. The partition kernels take any sequence lengths with
 * any size the launchers accept: this only picks a fast one. Host-side, no
 * device work; reads the current device's properties (fixed fallbacks
 * without a device). Returns the size (> 0), or PA_ERR_SHAPE / PA_ERR_UNSUPPORTED
 * for sizes, dtypes or head/block sizes the launchers reject.
 * max_num_partitions for the call is then ceil(max_seq_len / size). */
PA_API int paged_attn_plan_partition_size(int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_size,
                                          int32_t block_size, int32_t max_seq_len,
                                          int32_t kv_dtype);

/* Launch plan inspection: how many consecutive partitions of one (sequence,
 * kv head) a workgroup of paged_attn_v2_partition / paged_attn_decode handles
 * for these sizes (1, 2, 4 or 8). Results do not depend on it (each partition is
 * computed and stored on its own); it only groups work. Host-side, no device
 * work; returns a PA_ERR_* code for arguments the launchers would reject on
 * shape or support grounds. */
PA_API int paged_attn_partition_span(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_size, int32_t block_size,
                                     int32_t max_num_partitions, int32_t partition_size,
                                     int32_t kv_dtype);

/* Launch plan inspection for the one-call decode (paged_attn_decode*): writes
 * plan_out[0] = partitions per workgroup (the span C), plan_out[1] = ring
 * slots of the rolling merge (0: the span's parked states are combined at the
 * end; 1 or 2: partitions are merged as the span streams, for spans whose
 * parked states would not fit on chip), plan_out[2] = span entries per row
 * (ceil(P / C); 1: no reduce runs), plan_out[3] = column launches. Results do
 * not depend on the plan beyond fp32 rounding. Host-side, no device work;
 * returns PA_OK or the PA_ERR_* code the decode calls would return for these
 * sizes and dtypes (plan_out NULL: PA_ERR_NULL; num_seqs < 1: PA_ERR_SHAPE). */
PA_API int paged_attn_decode_plan(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                  int32_t max_num_partitions, int32_t partition_size,
                                  int32_t q_dtype, int32_t kv_dtype, int32_t* plan_out);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
