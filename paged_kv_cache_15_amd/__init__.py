"""MI355X-native paged KV cache and PagedAttention decode.

libpagedkv.so (HIP for gfx950 + a C++ host allocator) does the work; ``binding``
is its ctypes binding (same names as include/paged_kv.h), ``cache`` the host-driven
decode step, ``replay`` a runner for scripted workloads, ``build`` the hipcc build.
Touching any entry point loads the library and fails loudly if it has not been
built: there is no fallback.
"""
_ENTRY_POINTS = (
    "PagedKVError", "make_desc", "paged_kv_bytes_per_token", "paged_kv_pool_bytes",
    "paged_kv_pool_create", "paged_kv_pool_destroy", "paged_kv_pool_buffers",
    "paged_kv_pool_get_desc", "paged_kv_seq_create", "paged_kv_seq_fork", "paged_kv_seq_append",
    "paged_kv_append_batch", "paged_kv_seq_free", "paged_kv_block_tables", "paged_kv_seq_info",
    "paged_kv_block_refcount", "paged_kv_stats", "paged_kv_copy_blocks", "reshape_and_cache",
    "paged_attention_workspace_bytes", "paged_attention_decode", "paged_attention_partition",
    "paged_attention_reduce",
)


def __getattr__(name):
    if name in _ENTRY_POINTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
