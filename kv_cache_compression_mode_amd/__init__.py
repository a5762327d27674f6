"""JoLT KV-cache codec on AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI.

The native library is ``libjolt.so`` (built in-tree by
``kv_cache_compression_mode_amd.build``); ``jolt`` is its ctypes binding.
"""
from . import jolt  # noqa: F401
from .jolt import (allocate, blob_bytes, decode, encode, plan_from_spectra,  # noqa: F401
                   quantize, rotation, rotation_host)

__all__ = ["jolt", "allocate", "blob_bytes", "decode", "encode", "plan_from_spectra", "quantize",
           "rotation", "rotation_host"]
