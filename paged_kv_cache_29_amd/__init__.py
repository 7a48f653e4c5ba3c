"""Paged decode attention over a paged KV cache for AMD MI355X (gfx950).

The work is done by ``libpagedkv.so`` (hand-written HIP kernels behind the C
ABI in ``include/pagedkv.h``); this package marshals torch tensors into that
ABI.  ``workloads`` builds seeded synthetic inputs and ``blocks`` is a host
block allocator (free list, refcounts, copy-on-write).
"""

from ._lib import (  # noqa: F401
    check_block_tables,
    check_groups,
    check_query_start,
    check_slot_mapping,
    copy_blocks,
    kv_cache_write,
    kv_cache_write_int8,
    kv_cache_write_fp8,
    kv_cache_write_fp8_e5m2,
    kv_cache_write_int4,
    cascade_workspace_size,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    paged_attention_decode_cascade,
    paged_attention_multi_query,
    multi_query_workspace_size,
    paged_attention_decode_partitions,
    paged_attention_decode_reduce,
    paged_attention_decode_step,
    paged_attention_decode_step_partitions,
    partition_tokens,
    balanced_shares,
    probe_tile_read,
    streams_cache,
    workspace_size,
    load as load_library,
    LIB_PATH,
)

from .block_manager import BlockManager  # noqa: F401,E402

__version__ = "0.1.0"
