"""MI355X-native paged single-query decode attention (V2 partition + LSE reduce, GQA).

The computation lives in libpaged_attn.so (hand-written gfx950 HIP kernels
behind the C ABI of include/paged_attn.h); this package is its Python binding
plus the seeded synthetic-input generator.
"""
from .binding import (PA_BF16, PA_FP8_E4M3, PA_ERR_ALIGN, PA_ERR_HIP, PA_ERR_NULL, PA_ERR_SHAPE,  # noqa: F401
                      PA_ERR_UNSUPPORTED, PA_F16, PA_F32, PA_OK, abi_version,
                      decode_plan, default_partition_size, ensure_built, last_error, lib, paged_attn_decode,
                      paged_attn_decode_fp8, paged_attn_v2_partition_fp8,
                      paged_attn_decode_mq, paged_attn_v2_partition_mq, paged_attn_v2_reduce_mq,
                      paged_attn_decode_lse, paged_attn_v2_reduce_lse, paged_attn_merge_states,
                      paged_attn_decode_ex, paged_attn_decode_noalloc, paged_attn_v2_partition_ex,
                      paged_attn_v2_partition, paged_attn_v2_reduce, partition_span,
                      plan_partition_size, workspace)
