"""Paged attention over a block-table KV cache for AMD Instinct MI355X (gfx950).

The computation lives in ``libpa.so`` (hand-written HIP kernels behind the C
ABI of ``include/pa.h``); this package is its thin Python binding:

* :func:`decode`            one query per sequence, optional split-KV + merge
* :func:`decode_noalloc`    the same with the library's fixed device workspace
* :func:`decode_partitions` the split-KV partition kernel alone
* :func:`merge_partitions`  log-sum-exp merge of partition results
* :func:`prefill_chunk`     causal chunked prefill over a paged context
* :func:`mixed_step`        decode rows and prefill chunks as one step
* :func:`stream_read`       a plain read of one buffer (HBM read-rate probe)

``paged_kv_cache_22_amd.checks`` holds opt-in host-side checks of the device
arrays the C ABI does not validate (block-table entries, lengths, cu_q_lens,
slot mappings), for tests and debugging.

Importing the package loads ``libpa.so`` and fails if it is not built
(``python paged_kv_cache_22_amd/build.py``).
"""
from ._binding import (LIB_PATH, PA_BF16, PA_F32, PA_FP8_E4M3, PA_PARTITION_BALANCED, PAError, decode,
                       decode_noalloc, STATIC_WORKSPACE_BYTES, decode_multi_query, decode_shared_prefix, decode_stages, PA_STAGE_ATTENTION, PA_STAGE_MERGE,
                       PA_STAGE_ALL,
                       decode_partitions, decode_workspace_size, lib, merge_partitions,
                       mixed_step, prefill_chunk, status_string, stream_read, STREAM_READ_SINK_WORDS,
                       write_kv)

__all__ = ["decode", "decode_noalloc", "STATIC_WORKSPACE_BYTES", "decode_multi_query", "decode_shared_prefix", "decode_stages", "PA_STAGE_ATTENTION", "PA_STAGE_MERGE",
           "PA_STAGE_ALL", "decode_partitions", "merge_partitions", "mixed_step", "prefill_chunk", "stream_read", "STREAM_READ_SINK_WORDS", "write_kv",
           "decode_workspace_size", "status_string", "PAError", "lib", "LIB_PATH",
           "PA_F32", "PA_BF16", "PA_FP8_E4M3", "PA_PARTITION_BALANCED"]
