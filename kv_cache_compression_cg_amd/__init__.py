"""CacheGen-style KV-cache codec for AMD MI355X (gfx950).

The codec itself lives in the HIP library libcg.so (kernels + C ABI, see include/cg.h);
`kv_cache_compression_cg_amd.cg` is its thin Python binding.  Importing this package does
not load the library: `configs` and `synth` (seeded synthetic KV caches) are usable on a
machine without a GPU, and the binding is imported on first attribute access.
"""
from importlib import import_module

__all__ = ["configs", "synth", "cg"]


def __getattr__(name):
    if name in __all__:
        return import_module("." + name, __name__)
    raise AttributeError(name)
