"""Grouped-query attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libgqa.so`` (hand-written HIP
kernels, declared in ``include/gqa.h``).  ``binding`` is a thin ctypes layer
over it with the same names; PyTorch only supplies device memory and the
stream.  ``workloads`` draws the seeded synthetic inputs.

The binding is imported on first use so that the input generators can be
used on machines without the built library.
"""

_BINDING_NAMES = (
    "gqa_cache_elems_per_token",
    "gqa_decode_workspace_bytes",
    "gqa_kv_append",
    "gqa_decode",
    "gqa_prefill",
    "GqaError",
    "KVCache",
    "library_path",
    "load_library",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)


__all__ = list(_BINDING_NAMES)
