// Host side of the C ABI declared in include/paged_attn.h: argument
// validation, kernel selection and launch. No allocation, no host copies, no
// synchronisation: everything is enqueued on the caller's stream.
//
// The two phases are the page "paged_attention_v2_triton.py -- Triton
// PagedAttention V2 for BI-V100": phase-1 partition kernel and phase-2
// reduce kernel, launched back to back on one stream by its host launcher.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "paged_attn.h"
#include "pa_kernels.h"
#include "pa_tables.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int elem_size(int32_t dt) { return dt == PA_F32 ? 4 : dt == PA_FP8_E4M3 ? 1 : 2; }
bool is_16bit(int32_t dt) { return dt == PA_F16 || dt == PA_BF16; }

using pa::PartitionArgs;
using pa::ReduceArgs;
using pa::MergeArgs;
using pa::partition_fn;
typedef void (*reduce_fn)(ReduceArgs);
typedef void (*merge_fn)(MergeArgs);

int d_index(int D) { return D == 64 ? 0 : D == 128 ? 1 : D == 256 ? 2 : -1; }
int bs_index(int BS) { return BS == 16 ? 0 : BS == 32 ? 1 : -1; }

// ---------------------------------------------------------------- kernel tables
// Partition kernels: the tables of pa_tables.h, defined in the instantiation
// units; [ALiBi off / on] here, and for the MFMA kernels [column tiles 1 / 2].
const pa::partition_fn (*const kMfma[2][2])[3][2] = {{pa::kMfma_al0, pa::kMfmaW_al0},
                                                     {pa::kMfma_al1, pa::kMfmaW_al1}};
const pa::partition_fn (*const kMfma8[2][2])[3][2] = {{pa::kMfma8_al0, pa::kMfma8W_al0},
                                                      {pa::kMfma8_al1, pa::kMfma8W_al1}};
// the rolling-merge instantiations (one-call decode), 16-bit and 8-bit caches
const pa::partition_fn (*const kMfmaR[2][2])[3][2] = {{pa::kMfmaR_al0, pa::kMfmaRW_al0},
                                                      {pa::kMfmaR_al1, pa::kMfmaRW_al1}};
const pa::partition_fn (*const kMfma8R[2][2])[3][2] = {{pa::kMfma8R_al0, pa::kMfma8RW_al0},
                                                       {pa::kMfma8R_al1, pa::kMfma8RW_al1}};
const pa::partition_fn (*const kVec[2])[3][2][3] = {pa::kVec_al0, pa::kVec_al1};
const pa::partition_fn (*const kVec8[2])[3][2][3] = {pa::kVec8_al0, pa::kVec8_al1};

// [out dtype][D]
const reduce_fn kReduce[3][3] = {
    {pa::reduce_kernel<64, pa::DT_F32>, pa::reduce_kernel<128, pa::DT_F32>,
     pa::reduce_kernel<256, pa::DT_F32>},
    {pa::reduce_kernel<64, pa::DT_F16>, pa::reduce_kernel<128, pa::DT_F16>,
     pa::reduce_kernel<256, pa::DT_F16>},
    {pa::reduce_kernel<64, pa::DT_BF16>, pa::reduce_kernel<128, pa::DT_BF16>,
     pa::reduce_kernel<256, pa::DT_BF16>},
};

// P = 1: [out dtype][D]
const reduce_fn kReduceOne[3][3] = {
    {pa::reduce_one_kernel<64, pa::DT_F32>, pa::reduce_one_kernel<128, pa::DT_F32>,
     pa::reduce_one_kernel<256, pa::DT_F32>},
    {pa::reduce_one_kernel<64, pa::DT_F16>, pa::reduce_one_kernel<128, pa::DT_F16>,
     pa::reduce_one_kernel<256, pa::DT_F16>},
    {pa::reduce_one_kernel<64, pa::DT_BF16>, pa::reduce_one_kernel<128, pa::DT_BF16>,
     pa::reduce_one_kernel<256, pa::DT_BF16>},
};

// [dtype]
const merge_fn kMerge[3] = {pa::merge_states_kernel<pa::DT_F32>,
                            pa::merge_states_kernel<pa::DT_F16>,
                            pa::merge_states_kernel<pa::DT_BF16>};

// Per-device limit on dynamic LDS per workgroup (read once per device).
int max_lds_per_block() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      v = 65536;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// LDS of one CU (if unknown, that of two workgroups at the fallback limit).
int max_lds_per_cu() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 2 * 65536;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        v < 1)
      v = 2 * 65536;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

struct Plan {
  partition_fn fn;
  int lds_bytes;
  int grid;
  int span;
  int lpt;   // largest-first unit order
  int roll;  // one-call decode on the MFMA kernel: ring slots of the rolling merge (0: none)
};

// One-call decode: the partition launches combine each span's partitions
// themselves (combine_store in pa_kernels.h) and, when one span covers a
// whole row, write the output directly.
struct Fuse {
  int on = 0;
  void* out = nullptr;
  float* lse = nullptr;
  int odt = PA_F32;
};

#ifndef PA_SPAN
#define PA_SPAN 0  // >0: force this many partitions per workgroup (measurement builds)
#endif

// Consecutive partitions per workgroup (1, 2, 4 or 8). A longer span
// amortises each workgroup's prologue and epilogue and retires empty
// partitions together with used ones. It is taken only while the grid keeps
// kMinRounds workgroups per resident slot (span_min_grid) and a full span
// reads at most kSpanBytes of K+V; units of 1 MiB or more take the
// largest-first order (see kLptMinUnitBytes), which keeps their tail short.
// Measured against two partitions and 512 KiB at most (512-token partitions):
// up to four partitions and 1 MiB with a fixed floor of 2048 workgroups gave
// GQA bf16 189.5 -> 185.0 us, GQA fp8 94.6 -> 87.7, ALiBi GQA 190.9 -> 185.7,
// wide heads 506.8 -> 502.2, MHA -0.5 %, long context and the multi-token
// windows unchanged; the floor of two rounds with eight partitions and 2 MiB
// then GQA bf16 185.8 -> 182.2 and ALiBi GQA 186.8 -> 183.2, the other
// workloads within 0.3 %. The span's block-table slice must fit the 256-thread
// hoist and its parked state the LDS.
constexpr int kMinRounds = 2;
// tmp_output store policy: device-scope stores when rows have at least
// kThroughMinPartitions partitions, or a unit writes at least
// kThroughMinColumns rows per partition (see store_row in pa_kernels.h).
// Measured on the 16-column GQA window (4 heads x 4 query tokens, 8 or 4
// partitions): 230.5 -> 225.5 us at PS=512, 218.3 -> 214.4 at PS=1024; the
// 4-column single-query GQA batch stays on the default policy (equal at
// PS=512, 2.5 % slower at PS=1024 with device-scope stores).
constexpr int kThroughMinPartitions = 16;
constexpr int kThroughMinColumns = 16;
constexpr long long kSpanBytes = 2 << 20;
#ifndef PA_LPT
#define PA_LPT 1  // measurement builds: 0 index order everywhere, 2 largest-first everywhere
#endif
// Largest-first unit order (lpt_pair in pa_kernels.h) while every workgroup's
// ranking stays cheap: at most this many (sequence, span) pairs. Measured on
// the ragged batches (index order -> largest first): 8-bit GQA 102.7 -> 90.8 µs,
// 8-bit MHA 105.7 -> 102.1, 16-bit MHA (vector kernel) 212.0 -> 207.9; but
// 16-bit GQA (MFMA kernel, two workgroups per CU, so the ranking's extra
// round trip is poorly hidden) 186.8 -> 192.1, and uniform lengths lose
// ~1 % (nothing to reorder). So it is taken for 8-bit caches and the vector
// kernel, and for the 16-bit MFMA kernel only where a unit reads at least
// kLptMinUnitBytes of K+V: there a late long unit costs more than every
// workgroup's ranking (GQA bf16 with 2048-token units 184.7 -> 176.7 us, and
// with 4 query tokens 209.0 -> 196.2; uniform long context 1 % slower;
// 1024-token units of the ragged GQA batch 189.6 -> 195.5, so not there).
constexpr int kLptMaxPairs = 4096;
constexpr long long kLptMinUnitBytes = 1 << 20;
// Upper bound on the LDS of a span's parked state (see span_lds_cap): 80 KiB
// is two workgroups per CU, what the 16-bit MFMA kernel's registers allow at
// head size 128. It admits two-partition spans for 16-column units there (66
// KiB; measured against one-partition units: GQA with 4 query tokens 225.3 ->
// 220.6 us, long context with 2 tokens 192.8 -> 185.5 us).
constexpr int kSpanLdsCap = 80 * 1024;

#ifndef PA_ROLL
#define PA_ROLL 1  // measurement builds: 0 never the rolling merge, 2 always (one-call MFMA spans)
#endif
// The 8-bit one-call decode's spans of two or more partitions run the
// rolling-merge kernel: the plain 8-bit kernel's register budget (4 wavefronts
// per SIMD) leaves each workgroup 40 KiB of LDS, two partitions' parked states
// at 8 columns, so its spans stay short.
#ifndef PA_ROLL8
#define PA_ROLL8 1  // measurement builds: 0 keeps 8-bit caches on combine_store spans
#endif
constexpr bool kRoll8 = PA_ROLL8 != 0;

// Ring slots of the rolling merge for a one-call MFMA span of c partitions
// (roll_ct = the launch's column tiles; 0: not an MFMA one-call launch): 0
// where the span's parked states fit lds_cap (combine_store) and the rolling
// merge is not preferred, else 2 or 1 slots as they fit; -1 if nothing fits.
int span_roll(int PS, int BS, int NC, int D, int c, int roll_ct, int lds_cap,
              bool prefer = false) {
  const bool park = pa::lds_layout(PS, BS, NC, D, c).total <= lds_cap;
  if (roll_ct == 0 || c < 2 || (park && !prefer && PA_ROLL < 2)) return park ? 0 : -1;
  if (PA_ROLL == 0) return park ? 0 : -1;
  if (pa::roll_layout(PS, BS, roll_ct, D, c, 2).total <= lds_cap) return 2;
  if (pa::roll_layout(PS, BS, roll_ct, D, c, 1).total <= lds_cap) return 1;
  return park ? 0 : -1;
}

// A one-call batch whose K+V (at the longest length, every sequence) is at
// most kSmallBatchBytes is launch- and latency-bound: there a span covering
// the whole row (no reduce launch) beats any split. The tiny fp32 batch (two
// sequences, 1 MiB at most): 9.0 -> 6.x us per call.
constexpr long long kSmallBatchBytes = 4 << 20;

int pick_span(int S, int KH, int P, int PS, int BS, int NC, int D, int esz, int lds_cap,
              long long min_grid, int roll_ct = 0, bool fuse = false) {
  const bool small = fuse && (long long)S * KH * P * PS * D * esz * 2 <= kSmallBatchBytes;
  int best = 1;
  for (int c = 2; c <= pa::kMaxSpan && c / 2 < P; c *= 2) {  // (c / 2 >= P: P already covered)
    const long long grid = (long long)S * KH * ((P + c - 1) / c);
    const long long bytes = (long long)c * PS * D * esz * 2;
    if (c * (PS / BS) > pa::kWaves * 64 || span_roll(PS, BS, NC, D, c, roll_ct, lds_cap) < 0)
      break;
    if (PA_SPAN > 0) {
      if (c > PA_SPAN) break;
    } else if (!small && (grid < min_grid || bytes > kSpanBytes)) {
      break;
    }
    best = c;
  }
  return best;
}

// Columns per partition launch. A (sequence, kv head) unit has M*G columns
// (query token, query head); the MFMA kernel takes up to 16 per column tile
// and one or two tiles (two for head sizes up to 128, where both tiles'
// accumulators fit the register budget, and where the device's per-workgroup
// LDS holds their parked state), so wider units run as several launches over
// the same pages. The vector kernel (a single query token, at most 4 heads)
// takes all G in one launch.
#ifndef PA_MAX_TILES
#define PA_MAX_TILES 2  // measurement builds: 1 keeps every launch to one column tile
#endif
int launch_columns(int G, int M, int D, int PS, int BS) {
  bool two = PA_MAX_TILES > 1 && D <= 128;
  if (two && BS > 0 && PS > 0 && PS / BS <= pa::kWaves * 64)  // (else rejected later)
    two = pa::lds_layout(PS, BS, 32, D, 1).total <= max_lds_per_block();
  const int width = two ? 32 : 16;
  const long long total = (long long)G * M;
  return total < width ? (int)total : width;
}

// The partition kernel for a launch of NC columns (query dtype qdt, cache
// kvdt, group G, M query tokens, ALiBi flag al); *vec: the vector kernel.
int select_kernel(int qdt, int kvdt, int M, int G, int NC, int D, int BS, int al,
                  partition_fn* fn, bool* vec) {
  const int di = d_index(D), bi = bs_index(BS);
  if (di < 0 || bi < 0) return fail(PA_ERR_UNSUPPORTED, "unsupported head_size / block_size");
  *vec = false;
  if (M > 1 || (is_16bit(qdt) && G >= 4)) {
    // the MFMA path: one column per (query token, head), launch_columns of
    // them per launch in one or two column tiles
    if (!is_16bit(qdt))
      return fail(PA_ERR_UNSUPPORTED, "several query tokens need an f16/bf16 query");
    const int ct = NC > 16 ? 1 : 0;
    if (NC < 1 || NC > 32 || (ct && di > 1))
      return fail(PA_ERR_UNSUPPORTED, "bad column count %d for head size %d", NC, D);
    *fn = kvdt == PA_FP8_E4M3 ? kMfma8[al][ct][qdt - 1][di][bi] : kMfma[al][ct][qdt - 1][di][bi];
  } else if (G <= 4) {
    const int gi = G == 1 ? 0 : G == 2 ? 1 : 2;
    *fn = kvdt == PA_FP8_E4M3 ? kVec8[al][qdt - 1][di][bi][gi] : kVec[al][qdt][di][bi][gi];
    *vec = true;
  } else {
    return fail(PA_ERR_UNSUPPORTED, "group size %d not supported for this dtype", G);
  }
  return PA_OK;
}

// Workgroups of `fn` that one CU holds by its register use (the HIP runtime's
// occupancy calculator, without LDS; cached per kernel). 2 if unknown.
int wgs_per_cu(partition_fn fn) {
  static std::mutex mu;
  static std::vector<std::pair<partition_fn, int>> seen;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : seen)
      if (e.first == fn) return e.second;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)fn, pa::kWaves * 64, 0) !=
          hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    n = 2;
  }
  std::lock_guard<std::mutex> lock(mu);
  seen.emplace_back(fn, n);
  return n;
}

// LDS a span's parked state may take: the CU's LDS shared by the workgroups
// the kernel's registers allow (a longer span must not cost occupancy), at
// most kSpanLdsCap and the per-workgroup limit.
int span_lds_cap(partition_fn fn, int lds_limit, int wgs = 0) {
  const int per_wg = max_lds_per_cu() / (wgs > 0 ? wgs : wgs_per_cu(fn));
  return std::min(std::min(per_wg, kSpanLdsCap), lds_limit);
}

// Compute units of the current device (256 if unknown).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v < 1)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Fewest workgroups a longer span may leave in the grid: two per resident
// slot (the workgroups per CU that the kernel's registers allow, on every
// CU), so that the largest-first order has a second round to balance.
long long span_min_grid(partition_fn fn, int rounds = kMinRounds, int wgs = 0) {
  return (long long)rounds * (wgs > 0 ? wgs : wgs_per_cu(fn)) * cu_count();
}

// The one-call decode's spans need only one workgroup per resident slot:
// a longer span also means fewer span entries to store and reduce. Measured
// on MI355X against two rounds (eight-partition spans instead of four, one
// round of 512 workgroups): long context 172.4 -> 168.9 us, with 2 query
// tokens 181.0 -> 170.5, with 4 query tokens 189 -> 175; spans of 8 over 2 MiB
// (head size 256) were slower, so the byte limit stays.
constexpr int kMinRoundsFused = 1;
// The 8-bit rolling-merge kernel (three workgroups per CU) takes its spans
// down to a grid of kMinWgsPerCuRoll8 workgroups per CU rather than a full
// round: on the long-context batch at 512-token partitions, spans of eight
// (512 workgroups) against four (1024) measured 90.9 -> 88.7 us.
constexpr int kMinWgsPerCuRoll8 = 2;
// ... and runs at most kRoll8WgsPerCu workgroups per CU: its 128 registers
// would allow four, which measured 3 % slower on the GQA fp8 batch (84.4
// against 82.0 us, same box); the launch asks for enough LDS to keep a fourth
// workgroup off the CU.
constexpr int kRoll8WgsPerCu = 3;
// The 16-bit MFMA kernels run at most kMfma16WgsPerCu workgroups per CU (the
// one-tile kernel's 168 registers would allow three; at three the planned
// spans shrink and the long-context batch measured 2 % slower, the two-call
// GQA step 1.8 % slower).
constexpr int kMfma16WgsPerCu = 2;

// LDS a launch asks for so that at most `wgs` of its workgroups share a CU
// (1 KiB multiples, so that allocation rounding cannot lose one).
int occupancy_lds(int wgs) { return (max_lds_per_cu() / wgs) & ~1023; }

// Host checks shared by the partition entry points; fills `plan` for a launch
// of NC columns. The query has dtype qdt; the caches kvdt (== qdt, or
// PA_FP8_E4M3 with a 16-bit query).
int check_partition(float* tmp_output, float* exp_sums, float* max_logits, const void* query,
                    const void* key_cache, const void* value_cache, const int32_t* block_tables,
                    const int32_t* seq_lens, int32_t S, int32_t H, int32_t KH, int32_t D,
                    int32_t BS, int32_t NB, int32_t MB, int32_t P, int32_t PS, int32_t qdt,
                    int32_t kvdt, int32_t M, int32_t NC, const float* alibi, Plan* plan,
                    int force_span = 0, bool fuse = false) {
  if (S < 0 || H < 0 || KH < 0 || D < 0 || BS < 0 || NB < 0 || MB < 0 || P < 0)
    return fail(PA_ERR_SHAPE, "negative size argument");
  if (M < 1) return fail(PA_ERR_SHAPE, "num_queries must be >= 1");
  if (S == 0) {
    plan->fn = nullptr;
    return PA_OK;  // nothing to do; pointers of empty tensors may be NULL
  }
  if (kvdt == PA_FP8_E4M3) {
    if (!is_16bit(qdt))
      return fail(PA_ERR_UNSUPPORTED, "an 8-bit cache needs an f16 or bf16 query (got %d)", qdt);
  } else if (kvdt != PA_F32 && !is_16bit(kvdt)) {
    return fail(PA_ERR_UNSUPPORTED, "unknown kv dtype %d", kvdt);
  } else if (qdt != kvdt) {
    return fail(PA_ERR_UNSUPPORTED, "query dtype %d differs from kv dtype %d", qdt, kvdt);
  }
  if (!tmp_output || !exp_sums || !max_logits || !query || !key_cache || !value_cache ||
      !block_tables || !seq_lens)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  const int x = 16 / elem_size(kvdt);
  if (H < 1 || KH < 1 || H % KH) return fail(PA_ERR_SHAPE, "num_heads %d not a multiple of num_kv_heads %d", H, KH);
  if (D < 1 || D % x) return fail(PA_ERR_SHAPE, "head_size %d not a multiple of x = %d", D, x);
  if (BS < 1 || PS <= 0 || PS % BS)
    return fail(PA_ERR_SHAPE, "partition_size %d must be a positive multiple of block_size %d", PS, BS);
  if (P < 1) return fail(PA_ERR_SHAPE, "max_num_partitions must be >= 1");
  if (MB < 1) return fail(PA_ERR_SHAPE, "max_blocks_per_seq must be >= 1");
  if (NB < 1) return fail(PA_ERR_SHAPE, "num_blocks must be >= 1");
  const int di = d_index(D), bi = bs_index(BS);
  if (di < 0) return fail(PA_ERR_UNSUPPORTED, "head_size %d not in {64, 128, 256}", D);
  if (bi < 0) return fail(PA_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", BS);
  if (PS / BS > pa::kWaves * 64)
    return fail(PA_ERR_UNSUPPORTED, "partition_size / block_size > %d", pa::kWaves * 64);
  const int G = H / KH;
  const int al = alibi ? 1 : 0;
  if (alibi && !aligned4(alibi)) return fail(PA_ERR_ALIGN, "alibi_slopes must be 4-byte aligned");
  partition_fn fn = nullptr;
  bool vec = false;
  const int rc = select_kernel(qdt, kvdt, M, G, NC, D, BS, al, &fn, &vec);
  if (rc != PA_OK) return rc;
  if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned16(tmp_output))
    return fail(PA_ERR_ALIGN, "query, key_cache, value_cache and tmp_output must be 16-byte aligned");
  // A launch's columns span at most this many query tokens; its tmp_output
  // rows are addressed with 32-bit byte offsets.
  const long long toks = std::min<long long>(M, (NC + G - 2) / G + 1);
  if (((toks - 1) * H + G) * P * D * 4 > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "tmp_output rows of one launch's units exceed 2 GiB");
  const int lds_limit = max_lds_per_block();
  const int lds1 = pa::lds_layout(PS, BS, NC, D, 1).total;
  if (lds1 > lds_limit)
    return fail(PA_ERR_UNSUPPORTED, "needs %d bytes of LDS per workgroup, device allows %d", lds1,
                lds_limit);
  // One-call launches of the MFMA kernel may span more partitions than their
  // parked states fit, with the rolling merge. With an 8-bit cache every
  // one-call span of two or more partitions takes it (kRoll8), and spans are
  // sized for that kernel's occupancy.
  const bool kv8 = kvdt == PA_FP8_E4M3;
  const int roll_ct = fuse && !vec && (!kv8 || kRoll8) ? (NC > 16 ? 2 : 1) : 0;
  const partition_fn rfn =
      roll_ct ? (kv8 ? kMfma8R : kMfmaR)[al][roll_ct - 1][qdt - 1][d_index(D)][bs_index(BS)]
              : nullptr;
  const partition_fn sized = kv8 && rfn ? rfn : fn;
  const int cap_wgs = vec ? 0 : !kv8 ? kMfma16WgsPerCu : rfn ? kRoll8WgsPerCu : 0;
  const int wgs = cap_wgs ? std::min(wgs_per_cu(sized), cap_wgs) : wgs_per_cu(sized);
  const int cap = span_lds_cap(sized, lds_limit, wgs);
  long long min_grid = span_min_grid(sized, fuse ? kMinRoundsFused : kMinRounds, wgs);
  if (kv8 && rfn) min_grid = std::min(min_grid, (long long)kMinWgsPerCuRoll8 * cu_count());
  const int span = force_span > 0 ? force_span
                                  : pick_span(S, KH, P, PS, BS, NC, D, elem_size(kvdt), cap,
                                              min_grid, roll_ct, fuse);
  const long long grid = (long long)S * KH * ((P + span - 1) / span);
  if (grid > 0x7fffffffLL) return fail(PA_ERR_UNSUPPORTED, "too many work units");
  // (a longer span was admitted by pick_span, or is a forced shorter one;
  // one partition's parked state fits lds_limit, checked above)
  plan->roll = roll_ct && span > 1 ? span_roll(PS, BS, NC, D, span, roll_ct, cap, kv8) : 0;
  if (plan->roll < 0) return fail(PA_ERR_UNSUPPORTED, "no LDS layout for a span of %d", span);
  if (plan->roll > 0) fn = rfn;
  plan->fn = fn;
  plan->lds_bytes = plan->roll > 0 ? pa::roll_layout(PS, BS, roll_ct, D, span, plan->roll).total
                                   : pa::lds_layout(PS, BS, NC, D, span).total;
  // (the occupancy caps above, on the kernel that runs: the 8-bit kernel
  // without the rolling merge keeps its four workgroups per CU)
  if (cap_wgs && (!kv8 || plan->roll > 0) && wgs_per_cu(fn) > cap_wgs) {
    const int floor_lds = std::min(lds_limit, occupancy_lds(cap_wgs));
    if (plan->lds_bytes < floor_lds) plan->lds_bytes = floor_lds;
  }
  const long long pairs = (long long)S * ((P + span - 1) / span);
  const long long unit_bytes = (long long)span * PS * D * elem_size(kvdt) * 2;
  plan->lpt = PA_LPT && pairs <= kLptMaxPairs &&
              (vec || kvdt == PA_FP8_E4M3 || unit_bytes >= kLptMinUnitBytes || PA_LPT == 2);
  if (plan->lpt) {
    const int ord = pa::lpt_lds_bytes(S, P, PS, BS, span);
    if (ord > lds_limit) plan->lpt = 0;
    else plan->lds_bytes = plan->lds_bytes > ord ? plan->lds_bytes : ord;
  }
  plan->grid = (int)grid;
  plan->span = span;
  return PA_OK;
}

int launch_partition(const Plan& plan, float* tmp_output, float* exp_sums, float* max_logits,
                     const void* query, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, const int32_t* seq_lens, int32_t S, int32_t H,
                     int32_t KH, int32_t NB, int32_t MB, int32_t P, int32_t PS, float scale,
                     float k_scale, float v_scale, int32_t NC, int32_t Mq, int32_t c0,
                     const float* alibi, const Fuse& fz, hipStream_t stream) {
  PartitionArgs a;
  a.tmp_out = tmp_output;
  a.exp_sums = exp_sums;
  a.max_logits = max_logits;
  a.q = query;
  a.kc = key_cache;
  a.vc = value_cache;
  a.bt = block_tables;
  a.sl = seq_lens;
  a.S = S;
  a.H = H;
  a.KH = KH;
  a.MB = MB;
  a.P = P;
  a.PS = PS;
  a.NB = NB;
  a.Mq = Mq;
  a.NC = NC;
  a.c0 = c0;
  a.C = plan.span;
  a.through = P >= kThroughMinPartitions || NC >= kThroughMinColumns;
  a.qk_scale = scale * k_scale * pa::kLog2e;
  a.v_scale = v_scale;
  a.alibi = alibi;
  a.lpt = plan.lpt;
  // (With one-partition spans and several spans per row, the span entries are
  // the partition rows themselves: the plain phase-1 epilogue writes them.)
  a.Pq = fz.on ? (P + plan.span - 1) / plan.span : P;
  a.fuse = fz.on && (plan.span > 1 || a.Pq == 1);
  a.roll = a.fuse ? plan.roll : 0;
  a.lds_bytes = plan.lds_bytes;
  a.out = fz.out;
  a.lse = fz.lse;
  a.odt = fz.odt;
  hipLaunchKernelGGL(plan.fn, dim3(plan.grid), dim3(pa::kWaves * 64), plan.lds_bytes, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "partition launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int check_reduce(void* out, const float* tmp_output, const float* exp_sums,
                 const float* max_logits, const int32_t* seq_lens, int32_t S, int32_t M,
                 int32_t H, int32_t D, int32_t P, int32_t PS, int32_t odt, reduce_fn* fn) {
  if (S < 0 || H < 0 || D < 0 || P < 0) return fail(PA_ERR_SHAPE, "negative size argument");
  if (M < 1) return fail(PA_ERR_SHAPE, "num_queries must be >= 1");
  if (S == 0) {
    *fn = nullptr;
    return PA_OK;
  }
  if (odt != PA_F32 && odt != PA_F16 && odt != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "unknown out dtype %d", odt);
  if (!out || !tmp_output || !exp_sums || !max_logits || !seq_lens)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (H < 1) return fail(PA_ERR_SHAPE, "num_heads must be >= 1");
  if (PS <= 0) return fail(PA_ERR_SHAPE, "partition_size must be positive");
  if (P < 1) return fail(PA_ERR_SHAPE, "max_num_partitions must be >= 1");
  const int di = d_index(D);
  if (di < 0) return fail(PA_ERR_UNSUPPORTED, "head_size %d not in {64, 128, 256}", D);
  if (!aligned16(out) || !aligned16(tmp_output))
    return fail(PA_ERR_ALIGN, "out and tmp_output must be 16-byte aligned");
  if ((long long)S * M * H > 0x7fffffffLL) return fail(PA_ERR_UNSUPPORTED, "too many rows");
  *fn = P == 1 ? kReduceOne[odt][di] : kReduce[odt][di];
  return PA_OK;
}

int launch_reduce(reduce_fn fn, void* out, float* lse, const float* tmp_output,
                  const float* exp_sums, const float* max_logits, const int32_t* seq_lens,
                  int32_t S, int32_t M, int32_t H, int32_t D, int32_t P, int32_t PS,
                  hipStream_t stream) {
  ReduceArgs a;
  a.out = out;
  a.lse = lse;
  a.tmp_out = tmp_output;
  a.exp_sums = exp_sums;
  a.max_logits = max_logits;
  a.sl = seq_lens;
  a.S = S;
  a.H = H;
  a.P = P;
  a.PS = PS;
  a.M = M;
  a.WPI = pa::reduce_waves_per_row(P, D);
  const long long rows = (long long)S * M * H;
  // (reduce_one_kernel for P = 1: 256 / D rows per wavefront)
  const int rows_per_block = P == 1 ? pa::kWaves * (256 / D) : pa::kWaves / a.WPI;
  hipLaunchKernelGGL(fn, dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(pa::kWaves * 64), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "reduce launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

bool finite(float v) { return v == v && v - v == 0.0f; }

// Block-table row length that holds P partitions of PS tokens (at least 1).
int32_t max_blocks_for(int32_t P, int32_t PS, int32_t BS) {
  if (P < 1 || PS < 1 || BS < 1) return 1;
  const long long mb = ((long long)P * PS + BS - 1) / BS;
  return mb > 0x7fffffffLL ? 0x7fffffff : (int32_t)mb;
}

// Plans for the column launches of a phase-1 call: `full` for launches of nc
// columns, `last` for a narrower final one (all validated before any launch).
int plan_partitions(float* tmp_output, float* exp_sums, float* max_logits, const void* query,
                    const void* key_cache, const void* value_cache, const int32_t* block_tables,
                    const int32_t* seq_lens, int32_t S, int32_t H, int32_t KH, int32_t D,
                    int32_t BS, int32_t NB, int32_t MB, int32_t P, int32_t PS, int32_t qdt,
                    int32_t kvdt, int32_t M, const float* alibi, Plan* full, Plan* last,
                    int* nc, bool fuse = false) {
  const int G = KH > 0 && H >= KH && H % KH == 0 ? H / KH : 1;  // (validated by check_partition)
  const long long total = (long long)G * (M > 0 ? M : 1);
  *nc = launch_columns(G, M > 0 ? M : 1, D, PS, BS);
  int rc = check_partition(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                           block_tables, seq_lens, S, H, KH, D, BS, NB, MB, P, PS, qdt, kvdt, M,
                           *nc, alibi, full, 0, fuse);
  if (rc != PA_OK || S == 0) return rc;
  if (total > 0x7fffffffLL) return fail(PA_ERR_UNSUPPORTED, "too many query columns");
  *last = *full;
  if (total % *nc)
    rc = check_partition(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, S, H, KH, D, BS, NB, MB, P, PS, qdt, kvdt, M,
                         (int)(total % *nc), alibi, last, 0, fuse);
  if (rc == PA_OK && fuse && last->span != full->span) {
    // One span for every column launch (their span entries share one layout):
    // the shorter of the two, which fits both launches' LDS.
    const int span = std::min(full->span, last->span);
    Plan* re = full->span > span ? full : last;
    rc = check_partition(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, S, H, KH, D, BS, NB, MB, P, PS, qdt, kvdt, M,
                         re == full ? *nc : (int)(total % *nc), alibi, re, span, fuse);
  }
  return rc;
}

int launch_partitions(const Plan& full, const Plan& last, int nc, float* tmp_output,
                      float* exp_sums, float* max_logits, const void* query,
                      const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, int32_t S,
                      int32_t H, int32_t KH, int32_t NB, int32_t MB, int32_t P, int32_t PS,
                      float scale, float k_scale, float v_scale, int32_t M, const float* alibi,
                      const Fuse& fz, hipStream_t stream) {
  const int total = H / KH * M;  // (bounded by plan_partitions)
  for (int c0 = 0; c0 < total; c0 += nc) {
    const int n = total - c0 < nc ? total - c0 : nc;
    const int rc = launch_partition(n == nc ? full : last, tmp_output, exp_sums, max_logits,
                                    query, key_cache, value_cache, block_tables, seq_lens, S, H,
                                    KH, NB, MB, P, PS, scale, k_scale, v_scale, n, M, c0, alibi,
                                    fz, stream);
    if (rc != PA_OK) return rc;
  }
  return PA_OK;
}

int partition_entry(float* tmp_output, float* exp_sums, float* max_logits, const void* query,
                    const void* key_cache, const void* value_cache, const int32_t* block_tables,
                    const int32_t* seq_lens, int32_t S, int32_t M, int32_t H, int32_t KH,
                    int32_t D, int32_t BS, int32_t NB, int32_t MB, int32_t P, int32_t PS,
                    float scale, float k_scale, float v_scale, int32_t qdt, int32_t kvdt,
                    void* stream, const float* alibi = nullptr) {
  g_err[0] = 0;
  if (!finite(k_scale) || !finite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be finite");
  Plan full, last;
  int nc = 1;
  int rc = plan_partitions(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                           block_tables, seq_lens, S, H, KH, D, BS, NB, MB, P, PS, qdt, kvdt, M,
                           alibi, &full, &last, &nc);
  if (rc != PA_OK || S == 0) return rc;
  return launch_partitions(full, last, nc, tmp_output, exp_sums, max_logits, query, key_cache,
                           value_cache, block_tables, seq_lens, S, H, KH, NB, MB, P, PS, scale,
                           k_scale, v_scale, M, alibi, Fuse(), (hipStream_t)stream);
}

int decode_entry(void* out, float* lse, float* tmp_output, float* exp_sums, float* max_logits,
                 const void* query, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, int32_t S, int32_t M,
                 int32_t H, int32_t KH, int32_t D, int32_t BS, int32_t NB, int32_t MB,
                 int32_t P, int32_t PS, float scale, float k_scale, float v_scale, int32_t qdt,
                 int32_t kvdt, int32_t out_dtype, void* stream, const float* alibi = nullptr) {
  g_err[0] = 0;
  if (!finite(k_scale) || !finite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be finite");
  if (S > 0 && lse && !aligned4(lse)) return fail(PA_ERR_ALIGN, "lse must be 4-byte aligned");
  Plan full, last;
  int nc = 1;
  int rc = plan_partitions(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                           block_tables, seq_lens, S, H, KH, D, BS, NB, MB, P, PS, qdt, kvdt, M,
                           alibi, &full, &last, &nc, /*fuse=*/true);
  if (rc != PA_OK || S == 0) return rc;
  if (out_dtype != PA_F32 && out_dtype != qdt)
    return fail(PA_ERR_UNSUPPORTED, "out dtype must be PA_F32 or the query dtype");
  // The partition launches combine each span's partitions (Fuse); with one
  // span per row they write out (and lse) themselves and no reduce runs,
  // otherwise the reduce combines the Pq span entries of each row, which
  // stand for partitions of span * PS tokens.
  const int span = full.span;
  const int Pq = (P + span - 1) / span;
  reduce_fn fn = nullptr;
  rc = check_reduce(out, tmp_output, exp_sums, max_logits, seq_lens, S, M, H, D, Pq, PS * span,
                    out_dtype, &fn);
  if (rc != PA_OK) return rc;
  if ((long long)PS * span > 0x7fffffffLL) return fail(PA_ERR_UNSUPPORTED, "partition too long");
  Fuse fz;
  fz.on = 1;
  fz.out = out;
  fz.lse = lse;
  fz.odt = out_dtype;
  rc = launch_partitions(full, last, nc, tmp_output, exp_sums, max_logits, query, key_cache,
                         value_cache, block_tables, seq_lens, S, H, KH, NB, MB, P, PS, scale,
                         k_scale, v_scale, M, alibi, fz, (hipStream_t)stream);
  if (rc != PA_OK || Pq == 1) return rc;
  return launch_reduce(fn, out, lse, tmp_output, exp_sums, max_logits, seq_lens, S, M, H, D, Pq,
                       PS * span, (hipStream_t)stream);
}

int reduce_entry(void* out, float* lse, const float* tmp_output, const float* exp_sums,
                 const float* max_logits, const int32_t* seq_lens, int32_t S, int32_t M,
                 int32_t H, int32_t D, int32_t P, int32_t PS, int32_t out_dtype, void* stream) {
  g_err[0] = 0;
  reduce_fn fn = nullptr;
  int rc = check_reduce(out, tmp_output, exp_sums, max_logits, seq_lens, S, M, H, D, P, PS,
                        out_dtype, &fn);
  if (rc != PA_OK || S == 0) return rc;
  return launch_reduce(fn, out, lse, tmp_output, exp_sums, max_logits, seq_lens, S, M, H, D, P,
                       PS, (hipStream_t)stream);
}

// The one-call decode's launch plan for these sizes, checked as a call would
// check it, with a stand-in for every tensor (never dereferenced: nothing is
// launched). Returns PA_OK or the call's error code.
int plan_with_stand_ins(int32_t S, int32_t M, int32_t H, int32_t KH, int32_t D, int32_t BS,
                        int32_t P, int32_t PS, int32_t qdt, int32_t kvdt, Plan* full,
                        Plan* last, int* nc, bool fuse = true) {
  alignas(16) static const char stand_in[16] = {};
  void* p = (void*)stand_in;
  return plan_partitions((float*)p, (float*)p, (float*)p, p, p, p, (const int32_t*)p,
                         (const int32_t*)p, S, H, KH, D, BS, 1, max_blocks_for(P, PS, BS), P, PS,
                         qdt, kvdt, M, nullptr, full, last, nc, fuse);
}

// ---------------------------------------------------------------- scratch
// The allocation-free decode's workspace: one array per GPU the library is
// loaded on, held until the process ends. Its address on the current device
// comes from hipGetSymbolAddress once per device (in host code `scratch` only
// names the symbol; it is never used as an address).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The current device's scratch address, or nullptr (with the error set).
uint8_t* scratch_address() {
  static std::mutex mu;
  static uint8_t* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    fail(PA_ERR_HIP, "no current HIP device for the scratch workspace");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = (uint8_t*)p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int paged_attn_v2_partition(float* tmp_output, float* exp_sums, float* max_logits,
                            const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_size, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_num_partitions,
                            int32_t partition_size, float scale, int32_t kv_dtype,
                            void* stream) {
  if (kv_dtype == PA_FP8_E4M3) {
    g_err[0] = 0;
    return fail(PA_ERR_UNSUPPORTED, "8-bit caches go through paged_attn_v2_partition_fp8");
  }
  return partition_entry(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, num_seqs, 1, num_heads, num_kv_heads, head_size,
                         block_size, num_blocks, max_blocks_per_seq, max_num_partitions,
                         partition_size, scale, 1.0f, 1.0f, kv_dtype, kv_dtype, stream);
}

int paged_attn_v2_partition_fp8(float* tmp_output, float* exp_sums, float* max_logits,
                                const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_num_partitions, int32_t partition_size, float scale,
                                float k_scale, float v_scale, int32_t q_dtype, void* stream) {
  return partition_entry(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, num_seqs, 1, num_heads, num_kv_heads, head_size,
                         block_size, num_blocks, max_blocks_per_seq, max_num_partitions,
                         partition_size, scale, k_scale, v_scale, q_dtype, PA_FP8_E4M3, stream);
}

int paged_attn_v2_reduce(void* out, const float* tmp_output, const float* exp_sums,
                         const float* max_logits, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_heads, int32_t head_size, int32_t max_num_partitions,
                         int32_t partition_size, int32_t out_dtype, void* stream) {
  return reduce_entry(out, nullptr, tmp_output, exp_sums, max_logits, seq_lens, num_seqs, 1,
                      num_heads, head_size, max_num_partitions, partition_size, out_dtype,
                      stream);
}

int paged_attn_decode(void* out, float* tmp_output, float* exp_sums, float* max_logits,
                      const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t max_num_partitions, int32_t partition_size, float scale,
                      int32_t kv_dtype, int32_t out_dtype, void* stream) {
  if (kv_dtype == PA_FP8_E4M3) {
    g_err[0] = 0;
    return fail(PA_ERR_UNSUPPORTED, "8-bit caches go through paged_attn_decode_fp8");
  }
  return decode_entry(out, nullptr, tmp_output, exp_sums, max_logits, query, key_cache,
                      value_cache,
                      block_tables, seq_lens, num_seqs, 1, num_heads, num_kv_heads, head_size,
                      block_size, num_blocks, max_blocks_per_seq, max_num_partitions,
                      partition_size, scale, 1.0f, 1.0f, kv_dtype, kv_dtype, out_dtype, stream);
}

int paged_attn_decode_fp8(void* out, float* tmp_output, float* exp_sums, float* max_logits,
                          const void* query, const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                          int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_num_partitions, int32_t partition_size, float scale,
                          float k_scale, float v_scale, int32_t q_dtype, int32_t out_dtype,
                          void* stream) {
  return decode_entry(out, nullptr, tmp_output, exp_sums, max_logits, query, key_cache,
                      value_cache,
                      block_tables, seq_lens, num_seqs, 1, num_heads, num_kv_heads, head_size,
                      block_size, num_blocks, max_blocks_per_seq, max_num_partitions,
                      partition_size, scale, k_scale, v_scale, q_dtype, PA_FP8_E4M3, out_dtype,
                      stream);
}

int paged_attn_v2_partition_mq(float* tmp_output, float* exp_sums, float* max_logits,
                               const void* query, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_num_partitions, int32_t partition_size, float scale,
                               float k_scale, float v_scale, int32_t q_dtype, int32_t kv_dtype,
                               void* stream) {
  return partition_entry(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, num_seqs, num_queries, num_heads, num_kv_heads,
                         head_size, block_size, num_blocks, max_blocks_per_seq,
                         max_num_partitions, partition_size, scale, k_scale, v_scale, q_dtype,
                         kv_dtype, stream);
}

int paged_attn_v2_reduce_mq(void* out, const float* tmp_output, const float* exp_sums,
                            const float* max_logits, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_queries, int32_t num_heads, int32_t head_size,
                            int32_t max_num_partitions, int32_t partition_size,
                            int32_t out_dtype, void* stream) {
  return reduce_entry(out, nullptr, tmp_output, exp_sums, max_logits, seq_lens, num_seqs,
                      num_queries, num_heads, head_size, max_num_partitions, partition_size,
                      out_dtype, stream);
}

int paged_attn_decode_mq(void* out, float* tmp_output, float* exp_sums, float* max_logits,
                         const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_queries, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t max_num_partitions,
                         int32_t partition_size, float scale, float k_scale, float v_scale,
                         int32_t q_dtype, int32_t kv_dtype, int32_t out_dtype, void* stream) {
  return decode_entry(out, nullptr, tmp_output, exp_sums, max_logits, query, key_cache,
                      value_cache,
                      block_tables, seq_lens, num_seqs, num_queries, num_heads, num_kv_heads,
                      head_size, block_size, num_blocks, max_blocks_per_seq, max_num_partitions,
                      partition_size, scale, k_scale, v_scale, q_dtype, kv_dtype, out_dtype,
                      stream);
}

int paged_attn_v2_reduce_lse(void* out, float* lse, const float* tmp_output,
                             const float* exp_sums, const float* max_logits,
                             const int32_t* seq_lens, int32_t num_seqs, int32_t num_queries,
                             int32_t num_heads, int32_t head_size, int32_t max_num_partitions,
                             int32_t partition_size, int32_t out_dtype, void* stream) {
  if (num_seqs > 0 && (!lse || !aligned4(lse))) {
    g_err[0] = 0;
    return fail(lse ? PA_ERR_ALIGN : PA_ERR_NULL, "lse must be a non-NULL, 4-byte aligned float*");
  }
  return reduce_entry(out, lse, tmp_output, exp_sums, max_logits, seq_lens, num_seqs,
                      num_queries, num_heads, head_size, max_num_partitions, partition_size,
                      out_dtype, stream);
}

int paged_attn_decode_lse(void* out, float* lse, float* tmp_output, float* exp_sums,
                          float* max_logits, const void* query, const void* key_cache,
                          const void* value_cache, const int32_t* block_tables,
                          const int32_t* seq_lens, int32_t num_seqs, int32_t num_queries,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                          int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_num_partitions, int32_t partition_size, float scale,
                          float k_scale, float v_scale, int32_t q_dtype, int32_t kv_dtype,
                          int32_t out_dtype, void* stream) {
  if (num_seqs > 0 && (!lse || !aligned4(lse))) {
    g_err[0] = 0;
    return fail(lse ? PA_ERR_ALIGN : PA_ERR_NULL, "lse must be a non-NULL, 4-byte aligned float*");
  }
  return decode_entry(out, lse, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                      block_tables, seq_lens, num_seqs, num_queries, num_heads, num_kv_heads,
                      head_size, block_size, num_blocks, max_blocks_per_seq, max_num_partitions,
                      partition_size, scale, k_scale, v_scale, q_dtype, kv_dtype, out_dtype,
                      stream);
}

int paged_attn_v2_partition_ex(float* tmp_output, float* exp_sums, float* max_logits,
                               const void* query, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_num_partitions, int32_t partition_size, float scale,
                               float k_scale, float v_scale, const float* alibi_slopes,
                               int32_t q_dtype, int32_t kv_dtype, void* stream) {
  return partition_entry(tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                         block_tables, seq_lens, num_seqs, num_queries, num_heads, num_kv_heads,
                         head_size, block_size, num_blocks, max_blocks_per_seq,
                         max_num_partitions, partition_size, scale, k_scale, v_scale, q_dtype,
                         kv_dtype, stream, alibi_slopes);
}

int paged_attn_decode_ex(void* out, float* lse, float* tmp_output, float* exp_sums,
                         float* max_logits, const void* query, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_queries,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_num_partitions, int32_t partition_size, float scale,
                         float k_scale, float v_scale, const float* alibi_slopes,
                         int32_t q_dtype, int32_t kv_dtype, int32_t out_dtype, void* stream) {
  return decode_entry(out, lse, tmp_output, exp_sums, max_logits, query, key_cache, value_cache,
                      block_tables, seq_lens, num_seqs, num_queries, num_heads, num_kv_heads,
                      head_size, block_size, num_blocks, max_blocks_per_seq, max_num_partitions,
                      partition_size, scale, k_scale, v_scale, q_dtype, kv_dtype, out_dtype,
                      stream, alibi_slopes);
}

int paged_attn_decode_noalloc(void* out, float* lse, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_queries,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                              int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_num_partitions,
                              int32_t partition_size, float scale, float k_scale,
                              float v_scale, const float* alibi_slopes, int32_t q_dtype,
                              int32_t kv_dtype, int32_t out_dtype, void* stream) {
  g_err[0] = 0;
  const int32_t S = num_seqs, M = num_queries, H = num_heads, D = head_size,
                P = max_num_partitions;
  if (S == 0 && M >= 1)  // the documented no-op (decode_entry checks the rest)
    return decode_entry(out, lse, nullptr, nullptr, nullptr, query, key_cache, value_cache,
                        block_tables, seq_lens, S, M, H, num_kv_heads, D, block_size,
                        num_blocks, max_blocks_per_seq, P, partition_size, scale, k_scale,
                        v_scale, q_dtype, kv_dtype, out_dtype, stream, alibi_slopes);
  // The plan fixes how many span entries per row the workspace holds.
  Plan full, last;
  int nc = 1;
  int rc = plan_with_stand_ins(S, M, H, num_kv_heads, D, block_size, P, partition_size, q_dtype,
                               kv_dtype, &full, &last, &nc);
  if (rc != PA_OK) return rc;
  const long long Pq = (P + full.span - 1) / full.span;
  const long long rows = (long long)S * M * H;
  auto up = [](long long b) { return (b + 255) & ~255LL; };
  const long long tmp_bytes = up(rows * Pq * D * 4), stat_bytes = up(rows * Pq * 4);
  if (tmp_bytes + 2 * stat_bytes > (long long)kScratchBytes)
    return fail(PA_ERR_UNSUPPORTED,
                "workspace of %lld bytes exceeds the %zu-byte scratch of the allocation-free "
                "call (use paged_attn_decode_ex with a caller workspace)",
                tmp_bytes + 2 * stat_bytes, kScratchBytes);
  uint8_t* base = scratch_address();
  if (!base) return PA_ERR_HIP;
  return decode_entry(out, lse, (float*)base, (float*)(base + tmp_bytes),
                      (float*)(base + tmp_bytes + stat_bytes), query, key_cache, value_cache,
                      block_tables, seq_lens, S, M, H, num_kv_heads, D, block_size, num_blocks,
                      max_blocks_per_seq, P, partition_size, scale, k_scale, v_scale, q_dtype,
                      kv_dtype, out_dtype, stream, alibi_slopes);
}

int paged_attn_merge_states(void* out, float* out_lse, const void* a, const float* lse_a,
                            const void* b, const float* lse_b, int64_t num_rows,
                            int32_t head_size, int32_t dtype, void* stream) {
  g_err[0] = 0;
  if (num_rows < 0 || head_size < 0) return fail(PA_ERR_SHAPE, "negative size argument");
  if (num_rows == 0) return PA_OK;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "merge dtype %d not in {PA_F32, PA_F16, PA_BF16}", dtype);
  if (!out || !a || !lse_a || !b || !lse_b) return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (d_index(head_size) < 0)
    return fail(PA_ERR_UNSUPPORTED, "head_size %d not in {64, 128, 256}", head_size);
  if (!aligned16(out) || !aligned16(a) || !aligned16(b))
    return fail(PA_ERR_ALIGN, "out, a and b must be 16-byte aligned");
  if (!aligned4(lse_a) || !aligned4(lse_b) || (out_lse && !aligned4(out_lse)))
    return fail(PA_ERR_ALIGN, "lse arrays must be 4-byte aligned");
  const int tpr = head_size * elem_size(dtype) / 16;  // 8..64 lanes per row
  int shift = 0;
  while ((1 << shift) < tpr) ++shift;
  const long long chunks = (long long)num_rows * tpr;
  const long long blocks = (chunks + 255) / 256;
  if (num_rows > (1LL << 40) || blocks > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "too many rows");
  MergeArgs g;
  g.out = out;
  g.out_lse = out_lse;
  g.a = a;
  g.lse_a = lse_a;
  g.b = b;
  g.lse_b = lse_b;
  g.chunks = chunks;
  g.tpr_shift = shift;
  hipLaunchKernelGGL(kMerge[dtype], dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

const char* paged_attn_last_error(void) { return g_err; }

int paged_attn_abi_version(void) { return 2; }

int paged_attn_partition_span(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_size, int32_t block_size, int32_t max_num_partitions,
                              int32_t partition_size, int32_t kv_dtype) {
  g_err[0] = 0;
  const int S = num_seqs, H = num_heads, KH = num_kv_heads, D = head_size, BS = block_size,
            P = max_num_partitions, PS = partition_size, dt = kv_dtype;
  if (S < 0 || H < 1 || KH < 1 || H % KH) return fail(PA_ERR_SHAPE, "bad head counts");
  if (dt != PA_F32 && dt != PA_F16 && dt != PA_BF16 && dt != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "unknown kv dtype %d", dt);
  if (d_index(D) < 0 || bs_index(BS) < 0)
    return fail(PA_ERR_UNSUPPORTED, "unsupported head_size / block_size");
  if (PS <= 0 || PS % BS || PS / BS > pa::kWaves * 64 || P < 1)
    return fail(PA_ERR_SHAPE, "bad partition size / count");
  if (S == 0) return 1;
  // the phase-1 launch plan itself (check_partition, on stand-in pointers)
  const int qdt = dt == PA_FP8_E4M3 ? PA_BF16 : dt;  // (an 8-bit cache's f16 query: same plan)
  Plan full, last;
  int nc = 1;
  const int rc = plan_with_stand_ins(S, 1, H, KH, D, BS, P, PS, qdt, dt, &full, &last, &nc,
                                     /*fuse=*/false);
  if (rc != PA_OK) return rc;
  return full.span;
}

int paged_attn_decode_plan(int32_t num_seqs, int32_t num_queries, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           int32_t max_num_partitions, int32_t partition_size, int32_t q_dtype,
                           int32_t kv_dtype, int32_t* plan_out) {
  g_err[0] = 0;
  if (!plan_out) return fail(PA_ERR_NULL, "plan_out is NULL");
  if (num_seqs < 1) return fail(PA_ERR_SHAPE, "num_seqs must be >= 1");
  Plan full, last;
  int nc = 1;
  const int rc = plan_with_stand_ins(num_seqs, num_queries, num_heads, num_kv_heads, head_size,
                                     block_size, max_num_partitions, partition_size, q_dtype,
                                     kv_dtype, &full, &last, &nc);
  if (rc != PA_OK) return rc;
  const int span = full.span;
  plan_out[0] = span;
  plan_out[1] = full.roll;
  plan_out[2] = (max_num_partitions + span - 1) / span;
  const long long cols = (long long)(num_heads / num_kv_heads) * num_queries;
  plan_out[3] = (int)((cols + nc - 1) / nc);
  return PA_OK;
}

int paged_attn_plan_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t max_seq_len,
                                   int32_t kv_dtype) {
  g_err[0] = 0;
  const int S = num_seqs, H = num_heads, KH = num_kv_heads, D = head_size, BS = block_size,
            L = max_seq_len, dt = kv_dtype;
  if (S < 0 || H < 1 || KH < 1 || H % KH || L < 0) return fail(PA_ERR_SHAPE, "bad sizes");
  if (dt != PA_F32 && dt != PA_F16 && dt != PA_BF16 && dt != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "unknown kv dtype %d", dt);
  if (d_index(D) < 0 || bs_index(BS) < 0)
    return fail(PA_ERR_UNSUPPORTED, "unsupported head_size / block_size");
  // Longer partitions write fewer per-partition outputs and make longer
  // units, which the largest-first order balances (measured on MI355X, step
  // times against 2048-token partitions: 16-bit GQA -1.3 %, long context
  // -1.8 %, GQA with 4 query tokens -2 %, MHA and 256-wide heads equal; with
  // 8-bit caches 4096 was 3.8 % slower on GQA, so they stop at 2048). No
  // longer than the longest sequence needs: one partition either way.
  int top = dt == PA_FP8_E4M3 ? 2048 : 4096;
  while (top > 128 && top / 2 >= L) top /= 2;
  // The kernel a single-query launch of this geometry uses, and the
  // workgroups the device holds at once.
  const int G = H / KH;
  partition_fn fn = nullptr;
  bool vec = false;
  const int qdt = dt == PA_FP8_E4M3 ? PA_BF16 : dt;
  const int rc =
      select_kernel(qdt, dt, 1, G, launch_columns(G, 1, D, top, BS), D, BS, 0, &fn, &vec);
  if (rc != PA_OK) return rc;
  const long long slots = (long long)wgs_per_cu(fn) * cu_count();
  // The longest candidate whose units (S * KH * parts) fill every resident
  // workgroup, else 128; compared as parts >= ceil(slots / (S * KH)), which
  // cannot overflow. A candidate the decode call would reject on this device
  // (the LDS of one partition's parked state, the 32-bit workspace offsets) is
  // skipped.
  const long long sk = (long long)S * KH;
  auto ok = [&](int ps) {
    if (S == 0) return true;
    Plan full, last;
    int nc = 1;
    const int P = L > ps ? (int)((L + (long long)ps - 1) / ps) : 1;
    return plan_with_stand_ins(S, 1, H, KH, D, BS, P, ps, qdt, dt, &full, &last, &nc) == PA_OK;
  };
  int ps = top;
  for (; ps > 128; ps /= 2) {
    if (!ok(ps)) continue;
    const long long parts = L > ps ? (L + ps - 1) / ps : 1;
    if (sk > 0 && parts >= (slots + sk - 1) / sk) break;
  }
  if (!ok(ps)) {
    Plan full, last;
    int nc = 1;
    const int P = L > ps ? (int)((L + (long long)ps - 1) / ps) : 1;
    const int rc2 = plan_with_stand_ins(S, 1, H, KH, D, BS, P, ps, qdt, dt, &full, &last, &nc);
    return rc2 != PA_OK ? rc2 : ps;
  }
  g_err[0] = 0;
  return ps;
}

int paged_attn_default_partition_size(int32_t head_size, int32_t block_size, int32_t kv_dtype,
                                      int32_t group) {
  if (d_index(head_size) < 0 || bs_index(block_size) < 0)
    return fail(PA_ERR_UNSUPPORTED, "unsupported head_size / block_size");
  if (kv_dtype != PA_F32 && kv_dtype != PA_F16 && kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "unknown kv dtype %d", kv_dtype);
  if (group < 1) return fail(PA_ERR_UNSUPPORTED, "group size %d", group);
  // Measured on MI355X, step time (partition + reduce) against 1024-token
  // partitions: 2048 is faster on the long-context (-2.7 %), MHA (-1.3 %),
  // 256-wide-head (-1.2 %) and 4-token GQA (-2 %) batches and 0.7 % slower on
  // the ragged GQA batch (shorter units balance its tail better); half the
  // partition outputs to write and reduce. With 8-bit caches (half the bytes
  // per token) 2048 against 512: GQA -8 %, long context -7 %, MHA equal.
  return 2048;
}

}  // extern "C"
