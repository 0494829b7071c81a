"""libsmla for MI355X (gfx950): sparse MLA over a paged latent KV cache.

The compute lives in the HIP library libsmla.so (built by `python -m
sparse_mla_attention_resolve_amd.build`); this package is its thin Python binding.
The binding loads the library on first use and raises if it is not built.
"""
_EXPORTED = ("KvCache", "SmlaError", "smla_resolve_slots", "smla_sparse_decode", "smla_sparse_decode_workspace",
             "smla_sparse_decode_splits", "smla_sparse_decode_topk", "smla_sparse_decode_noalloc", "DecodeCall", "new_workspace", "smla_sparse_decode_workspace_init", "smla_build_group_union", "smla_grouped_prefill", "smla_kv_write",
             "SMLA_F32", "SMLA_BF16", "SMLA_FP8_E4M3", "LIB_PATH", "EXPORTS", "lib", "smla")


def __getattr__(name):
    if name in _EXPORTED:
        import importlib
        _smla = importlib.import_module(__name__ + ".smla")
        return _smla if name == "smla" else getattr(_smla, name)
    raise AttributeError(name)


__all__ = list(_EXPORTED)
