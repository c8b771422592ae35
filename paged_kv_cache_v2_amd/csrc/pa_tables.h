// Partition-kernel tables shared between the host translation unit and the
// instantiation units (pa_inst.hip, compiled once per family and ALiBi mode
// so that the build runs in parallel). Each table maps the runtime geometry
// to one template instantiation.
#pragma once

#include "pa_kernels.h"

namespace pa {

typedef void (*partition_fn)(PartitionArgs);

// Index helpers: D in {64, 128, 256}, BS in {16, 32}, GM in {1, 2, 4}.
// MFMA tables: [query dtype f16 / bf16][D][BS]; kMfma* one column tile,
// kMfmaW* two (D <= 128 only: null for D = 256); kMfmaR* / kMfmaRW* the same
// with the one-call decode's rolling merge. Vector tables: [dtype
// f32 / f16 / bf16][D][BS][GM] for 16/32-bit caches, [query dtype f16 /
// bf16][D][BS][GM] for 8-bit caches. Suffix: ALiBi off (0) / on (1).
extern const partition_fn kMfma_al0[2][3][2], kMfma_al1[2][3][2];
extern const partition_fn kMfma8_al0[2][3][2], kMfma8_al1[2][3][2];
extern const partition_fn kMfmaW_al0[2][3][2], kMfmaW_al1[2][3][2];
extern const partition_fn kMfma8W_al0[2][3][2], kMfma8W_al1[2][3][2];
extern const partition_fn kMfmaR_al0[2][3][2], kMfmaR_al1[2][3][2];    // rolling merge
extern const partition_fn kMfmaRW_al0[2][3][2], kMfmaRW_al1[2][3][2];  // rolling, two tiles
extern const partition_fn kMfma8R_al0[2][3][2], kMfma8R_al1[2][3][2];    // rolling, 8-bit
extern const partition_fn kMfma8RW_al0[2][3][2], kMfma8RW_al1[2][3][2];  // rolling, 8-bit, two
extern const partition_fn kVec_al0[3][3][2][3], kVec_al1[3][3][2][3];
extern const partition_fn kVec8_al0[2][3][2][3], kVec8_al1[2][3][2][3];

}  // namespace pa
