"""JoLT / FlashJoLT KV-cache compression for AMD Instinct MI355X (gfx950).

The compute lives in libjolt.so (HIP kernels behind the C ABI of include/jolt.h);
``kv_cache_compression_layer_amd.jolt`` is its ctypes binding.
"""
from . import jolt  # noqa: F401
