/*
 * pa_ceiling.h -- C ABI of libpa_ceiling.so, a measuring instrument that
 * ships beside the decode library: a read-only kernel that streams the K and
 * V pages a paged decode reads, through the same block tables and with the
 * same 16-byte non-temporal loads, and computes nothing with them. Its
 * bandwidth is the page-gather read ceiling the decode kernels are compared
 * with (the decode reads exactly these bytes and does its arithmetic on
 * them). It follows the gather of the page "paged_attention_v2_triton.py --
 * Triton PagedAttention V2 for BI-V100" (phase-1 partition kernel: token t of
 * sequence s lives in physical block block_tables[s][t / BS]).
 *
 * Every pointer is a DEVICE pointer; nothing is allocated, copied or waited
 * for; work is enqueued on `stream` (a hipStream_t, NULL = null stream).
 */
#ifndef PA_CEILING_H
#define PA_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PA_CEILING_API __attribute__((visibility("default")))
#else
#define PA_CEILING_API
#endif

/* Words of `sink` a call needs: 4 per workgroup, one workgroup per (sequence,
 * kv head, run of 32 blocks of the block-table row). */
PA_CEILING_API int64_t pa_gather_ceiling_sink_words(int32_t num_seqs, int32_t num_kv_heads,
                                                    int32_t max_blocks_per_seq);

/*
 * Read every (block, kv head) page of key_cache and value_cache that the
 * sequences use: blocks block_tables[s][i] for i < ceil(seq_lens[s] / BS),
 * kv heads 0 .. KH-1, page_bytes bytes each (D * BS * element size; a
 * multiple of 1024). Each workgroup folds what it read into four words of
 * `sink` (int32 [pa_gather_ceiling_sink_words]); their values mean nothing.
 *
 *   key_cache, value_cache   [B, KH, page_bytes] bytes, 16-byte aligned
 *   block_tables [S, MB] int32, entries of used blocks in [0, B)
 *   seq_lens     [S] int32, 0 <= seq_lens[s] <= MB * BS
 * Returns 0, or -1 (NULL pointer), -2 (bad size), -4 (misaligned), -5 (launch
 * rejected by the HIP runtime).
 */
PA_CEILING_API int pa_gather_ceiling(int32_t* sink, int64_t sink_words, const void* key_cache,
                                     const void* value_cache, const int32_t* block_tables,
                                     const int32_t* seq_lens, int32_t num_seqs,
                                     int32_t num_kv_heads, int32_t page_bytes,
                                     int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_CEILING_H */
