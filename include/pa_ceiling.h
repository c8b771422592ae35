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

/* Words of `sink` a call needs (4 per workgroup of the fixed grid). */
PA_CEILING_API int64_t pa_gather_ceiling_sink_words(void);

/*
 * Read the K and V page of every (block, kv head) item of a flat page list:
 * blocks[j] for j < num_pages (each used block of each sequence once; the
 * caller gathers them from its block tables), kv heads 0 .. KH-1, page_bytes
 * bytes each (D * BS * element size; 1, 2, 4, 8 or 16 KiB). Each workgroup
 * folds what it read into four words of `sink` (int32
 * [pa_gather_ceiling_sink_words()]); their values mean nothing.
 *
 *   key_cache, value_cache   [B, KH, page_bytes] bytes, 16-byte aligned
 *   blocks                   [num_pages] int32 in [0, B) (clamped into it)
 * Returns 0, or -1 (NULL pointer), -2 (bad size), -4 (misaligned), -5 (launch
 * rejected by the HIP runtime). num_pages == 0 is a no-op.
 */
PA_CEILING_API int pa_gather_ceiling(int32_t* sink, int64_t sink_words, const void* key_cache,
                                     const void* value_cache, const int32_t* blocks,
                                     int64_t num_pages, int32_t num_kv_heads,
                                     int32_t page_bytes, int32_t num_blocks, void* stream);

/*
 * The same reads with the decode kernels' work structure, so that the gap
 * between the decode and pa_gather_ceiling can be split into what the work
 * structure costs and what the arithmetic around the stream costs. Workgroup
 * u (of num_units, launched in index order: the caller lists the units
 * largest first, as the decode ranks them) reads the K and V pages
 * pages[unit_off[u] .. unit_off[u+1]), page p = block * KH + kv head (the
 * caller's list: one unit per (sequence, kv head, span of partitions)); its
 * four wavefronts take every fourth page, each with two pages' loads in
 * flight. The launch asks for the LDS share that fits at most
 * workgroups_per_cu workgroups on a CU (the decode's residency). Each
 * workgroup folds what it read into four words of `sink` (int32
 * [4 * num_units]); their values mean nothing.
 *
 *   key_cache, value_cache   [num_cache_pages, page_bytes] bytes, 16-byte aligned
 *   pages                    [unit_off[num_units]] int32 in [0, num_cache_pages)
 *                            (clamped into it)
 *   unit_off                 [num_units + 1] int32, non-decreasing, from 0
 *   page_bytes               1, 2, 4 or 8 KiB
 * Returns 0, or -1 (NULL pointer), -2 (bad size), -4 (misaligned), -5 (device
 * query or launch rejected by the HIP runtime). num_units == 0 is a no-op.
 */
PA_CEILING_API int pa_gather_units(int32_t* sink, int64_t sink_words, const void* key_cache,
                                   const void* value_cache, const int32_t* pages,
                                   const int32_t* unit_off, int32_t num_units,
                                   int64_t num_cache_pages, int32_t page_bytes,
                                   int32_t workgroups_per_cu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_CEILING_H */
