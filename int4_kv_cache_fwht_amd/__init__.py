"""int4_kv_cache_fwht_amd -- paged INT4 KV cache with block-Hadamard rotation and INT8 sink/recent
protection, with GQA decode attention, as hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/kv4.h``.

This package is argument marshalling only: every step of the append and decode path runs in
``libkv4.so``.  PyTorch provides device memory and streams.  If the library is missing, importing
the binding raises; there is no fallback.
"""
from ._binding import (  # noqa: F401
    KV4Error,
    Config,
    BufferSizes,
    Cache,
    FORMAT_INT4_PROT,
    FORMAT_INT8,
    FORMAT_BF16,
    EVICT_DUAL_WRITE,
    EVICT_REQUANT,
    STATUS,
    lib,
    lib_path,
    kv4_buffer_sizes_query,
    hbm_probe,
)

lib()  # load now: a missing library fails the import, never a silent fallback

__all__ = ["KV4Error", "Config", "BufferSizes", "Cache", "FORMAT_INT4_PROT", "FORMAT_INT8", "FORMAT_BF16",
           "EVICT_DUAL_WRITE", "EVICT_REQUANT", "STATUS", "lib", "lib_path", "kv4_buffer_sizes_query",
           "hbm_probe"]
