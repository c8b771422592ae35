// Instantiations of the partition kernels, one family per compilation:
//   PA_FAMILY 0: MFMA, 16-bit caches     1: MFMA, 8-bit caches
//             2: vector, 16/32-bit       3: vector, 8-bit caches
//             4: MFMA, two column tiles, 16-bit caches
//             5: MFMA, two column tiles, 8-bit caches
//             6: MFMA, rolling merge (one-call decode), 16-bit caches
//             7: MFMA, rolling merge, two column tiles, 16-bit caches
//             8: MFMA, rolling merge, 8-bit caches
//             9: MFMA, rolling merge, two column tiles, 8-bit caches
//   PA_AL     0: no position bias        1: ALiBi
// The build compiles this file once per (family, ALiBi) pair in parallel.
#include <hip/hip_runtime.h>

#include "pa_tables.h"

#if !defined(PA_FAMILY) || !defined(PA_AL)
#error "PA_FAMILY and PA_AL must be defined"
#endif

#define PA_CAT2(a, b) a##b
#define PA_CAT(a, b) PA_CAT2(a, b)
#if PA_AL
#define PA_TABLE(name) PA_CAT(name, _al1)
#else
#define PA_TABLE(name) PA_CAT(name, _al0)
#endif

namespace pa {

constexpr bool kAL = PA_AL != 0;

#if PA_FAMILY != 2 && PA_FAMILY != 3
constexpr bool kKV8 = PA_FAMILY == 1 || PA_FAMILY == 5 || PA_FAMILY == 8 || PA_FAMILY == 9;
constexpr int kCT = PA_FAMILY == 4 || PA_FAMILY == 5 || PA_FAMILY == 7 || PA_FAMILY == 9 ? 2 : 1;
constexpr bool kRoll = PA_FAMILY >= 6;
#define PA_MFMA_BS(DT, D)                                        \
  {partition_mfma_kernel<DT, D, 16, kKV8, kAL, kCT, kRoll>,      \
   partition_mfma_kernel<DT, D, 32, kKV8, kAL, kCT, kRoll>}
#if PA_FAMILY != 4 && PA_FAMILY != 5 && PA_FAMILY != 7 && PA_FAMILY != 9  // one column tile
#define PA_MFMA_D(DT) {PA_MFMA_BS(DT, 64), PA_MFMA_BS(DT, 128), PA_MFMA_BS(DT, 256)}
#else
#define PA_MFMA_D(DT) {PA_MFMA_BS(DT, 64), PA_MFMA_BS(DT, 128), {nullptr, nullptr}}
#endif
#if PA_FAMILY == 0
const partition_fn PA_TABLE(kMfma)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#elif PA_FAMILY == 1
const partition_fn PA_TABLE(kMfma8)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#elif PA_FAMILY == 4
const partition_fn PA_TABLE(kMfmaW)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#elif PA_FAMILY == 5
const partition_fn PA_TABLE(kMfma8W)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#elif PA_FAMILY == 6
const partition_fn PA_TABLE(kMfmaR)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#elif PA_FAMILY == 7
const partition_fn PA_TABLE(kMfmaRW)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#elif PA_FAMILY == 8
const partition_fn PA_TABLE(kMfma8R)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#else
const partition_fn PA_TABLE(kMfma8RW)[2][3][2] = {PA_MFMA_D(DT_F16), PA_MFMA_D(DT_BF16)};
#endif
#undef PA_MFMA_D
#undef PA_MFMA_BS

#else
constexpr bool kKV8 = PA_FAMILY == 3;
#define PA_VEC_GM(DT, D, BS)                                                       \
  {partition_vec_kernel<DT, D, BS, 1, kKV8, kAL>, partition_vec_kernel<DT, D, BS, 2, kKV8, kAL>, \
   partition_vec_kernel<DT, D, BS, 4, kKV8, kAL>}
#define PA_VEC_BS(DT, D) {PA_VEC_GM(DT, D, 16), PA_VEC_GM(DT, D, 32)}
#define PA_VEC_D(DT) {PA_VEC_BS(DT, 64), PA_VEC_BS(DT, 128), PA_VEC_BS(DT, 256)}
#if PA_FAMILY == 2
const partition_fn PA_TABLE(kVec)[3][3][2][3] = {PA_VEC_D(DT_F32), PA_VEC_D(DT_F16),
                                                 PA_VEC_D(DT_BF16)};
#else
const partition_fn PA_TABLE(kVec8)[2][3][2][3] = {PA_VEC_D(DT_F16), PA_VEC_D(DT_BF16)};
#endif
#undef PA_VEC_D
#undef PA_VEC_BS
#undef PA_VEC_GM
#endif

}  // namespace pa
