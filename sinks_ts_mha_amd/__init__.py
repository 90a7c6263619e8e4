"""MI355X (gfx950) grouped-query attention with sinks and sliding windows: prefill over
packed sequences, prefill of new rows against a paged KV cache, and decode against it.

The compute lives in libts_mha.so (hand-written HIP kernels behind the C ABI of
include/ts_mha.h); this package is its thin Python binding plus the seeded
synthetic workload generators.
"""
from ._binding import (TsMhaError, lib, mha_decode_with_kvcache, mha_prefill,
                       mha_prefill_with_kvcache, ts_mha_decode_with_kvcache,
                       ts_mha_decode_with_kvcache_noalloc, ts_mha_decode_workspace_size,
                       ts_mha_prefill, ts_mha_prefill_with_kvcache, ts_mha_strerror,
                       ts_mha_unmasked_pairs)

__all__ = ["TsMhaError", "lib", "mha_decode_with_kvcache", "mha_prefill",
           "mha_prefill_with_kvcache", "ts_mha_decode_with_kvcache",
           "ts_mha_decode_with_kvcache_noalloc", "ts_mha_decode_workspace_size",
           "ts_mha_prefill", "ts_mha_prefill_with_kvcache", "ts_mha_strerror",
           "ts_mha_unmasked_pairs"]
