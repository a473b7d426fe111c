"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

* ``allocator`` -- host-side reference-counted block manager (block tables,
  slot mappings, fork, copy-on-write pairs).
* ``prefix_cache`` -- automatic prefix caching by chained block hashes
  (``PrefixCachingAllocator``).
* ``radix_cache``  -- radix-tree prefix cache with LRU leaf eviction
  (``RadixCache``) over a ``BlockAllocator``.
* ``_lib``      -- ctypes binding of ``libpagedkv.so``: the device calls
  ``paged_kv_append``, ``copy_blocks``, ``paged_attention_decode``,
  ``paged_attention_extend`` (+ ``paged_kv_gather``), taking torch tensors on
  the GPU and running on torch's current stream.  It raises if the library
  is missing; there is no other implementation to fall back to.
"""

from .allocator import (BlockAllocator, OutOfBlocks, kv_bytes_per_token,  # noqa: F401
                        shared_prefix_groups)
from .prefix_cache import PrefixCachingAllocator, block_hash  # noqa: F401
from .radix_cache import RadixCache  # noqa: F401


def __getattr__(name):
    # the binding imports torch and loads the HIP library; do that on first use
    if name in ("_lib", "ops"):
        import importlib
        return importlib.import_module("._lib", __name__)
    raise AttributeError(name)
