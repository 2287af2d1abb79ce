"""MI355X (gfx950) paged KV-cache decode: HIP kernels behind a C ABI.

``decode``, ``decode_step``, ``decode_noalloc``, ``decode_multi``, ``decode_shared``, ``decode_shared_tree``,
``share_plan`` with ``decode_shared_planned``, ``reshape_and_cache``,
``copy_blocks`` and ``swap_blocks`` call libpa.so (built
with ``python -m paged_kv_cache_433_amd.build``); the library is loaded on
first use and a missing build raises. ``workloads`` makes seeded inputs.
"""

from .ops import (  # noqa: F401
    PagedAttentionError,
    copy_blocks,
    decode,
    decode_multi,
    decode_noalloc,
    decode_multi_workspace_bytes,
    decode_shared,
    decode_shared_planned,
    decode_shared_tree,
    decode_shared_tree_workspace_bytes,
    decode_step,
    decode_shared_workspace_bytes,
    decode_workspace_bytes,
    probe_copy,
    probe_read,
    probe_read_sink_bytes,
    reshape_and_cache,
    share_plan,
    swap_blocks,
)
