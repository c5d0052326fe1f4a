"""kv_cached_decode_amd -- KV-cached decode attention for MI355X (gfx950).

The product is libkvd.so (HIP kernels + the C ABI declared in include/kvd.h);
this package adds the thin Python binding over it and the seeded workload
generators used by the tests and the benchmark.
"""
from .binding import (  # noqa: F401
    KVD_KERNEL_AUTO, KVD_KERNEL_MFMA, KVD_KERNEL_VALU, KVD_ROPE_HALF, KVD_ROPE_INTERLEAVED,
    KvdError, PagedKV, decode_attention, decode_attention_plan, decode_attention_workspace_size,
    decode_attention_lse, decode_step, lib, merge_partials, rope_append_kv, workspace,
)
