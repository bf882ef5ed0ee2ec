"""Paged KV cache for AMD Instinct MI355X (gfx950): slot-mapped KV write, split-K paged
decode attention, causal paged prefill attention, whole-block copy-on-write, block swapping to pinned host memory for
preemption and a host block allocator with prefix caching, behind the C ABI
of include/pagedkv.h (libpagedkv.so, built in-tree by ``_build.py``).

The names below are the C ABI's; the binding only marshals arguments.
"""

from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, PreparedDecode, PreparedKVWrite, PA_DTYPE_BF16, PA_DTYPE_F32, PA_DTYPE_FP8_E4M3, PA_DTYPE_MXFP4,
    Allocator, NoBlocksError, mxfp4_cache, mx_row_bytes,
    PagedKVError, UnsupportedError, load, pa_alloc_create, pa_alloc_destroy, pa_alloc_dump,
    pa_alloc_stats, pa_batch_append, pa_block_tables, pa_copy_blocks, pa_decode,
    pa_decode_workspace_bytes, pa_decode_partition_tokens, pa_decode_workspace_init, decode_workspace, pa_kv_write, pa_seq_add, pa_seq_append, pa_seq_fork, pa_seq_free,
    pa_alloc_set_host_blocks, pa_swap_out, pa_swap_in, pa_seq_is_swapped, pa_alloc_dump_host, pa_swap_blocks,
    pa_seq_add_prompt, pa_seq_append_tokens, pa_alloc_dump_cached, pa_prefill, pa_upload, pa_probe_read, pa_decode_noalloc, pa_decode_append,
    PreparedDecodeAppend, PA_PROBE_GRID, PA_PROBE_RANGES, PA_PROBE_TILES,
)
