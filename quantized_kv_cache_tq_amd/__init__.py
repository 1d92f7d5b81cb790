"""TurboQuant KV-cache attention for MI355X (gfx950).

The compute path is the HIP library ``libtq.so`` behind the C ABI declared in
``include/tq.h``; ``quantized_kv_cache_tq_amd.binding`` marshals torch tensors
into that ABI.  Importing this package does not load the library; the first
call into the binding does, and raises if the library was not built.
"""

_BINDING_NAMES = (
    "tq_set_rows", "tq_attn_decode", "tq_attn_decode_workspace", "tq_attn_decode_batch",
    "tq_attn_decode_batch_workspace", "tq_attn_prefill",
    "tq_attn_prefill_workspace", "tq_attn_int8_prompt", "tq_attn_int8_prompt_workspace",
    "tq_codebook", "tq_cache_plane_bytes", "tq_version", "TQCache", "TQError", "new_cache",
    "load_library",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
