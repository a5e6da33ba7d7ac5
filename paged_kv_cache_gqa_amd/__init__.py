"""Paged-KV grouped-query attention for MI355X (gfx950).

The library is the C ABI in ``include/pa.h`` (``libpa_mi355x.so``, built from
``csrc/`` by ``paged_kv_cache_gqa_amd.build``); ``binding`` exposes it to
Python with the same names (``attention``, ``plan``, ``merge``, ...).  The
binding is imported lazily so that ``paged_kv_cache_gqa_amd.workloads`` (the
seeded input generator) can be used without torch or a GPU.
"""

_BINDING_NAMES = {
    "attention", "plan", "attention_planned", "merge_planned", "plan_read", "gather_kv", "merge", "validate",
    "check_desc", "workspace_size", "alloc_workspace", "make_desc", "status_string", "abi_version", "lib",
    "PagedAttentionError", "PaDesc", "to_device", "append_kv", "workspace_init", "attention_tree",
    "attention_fp8kv", "attention_shared_prefix", "shared_prefix_workspace", "status_str", "workspace_bytes", "attention_noalloc",
    "read_stream",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
