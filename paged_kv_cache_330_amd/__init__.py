"""MI355X-native paged KV-cache decode path.

Three device operations behind a C-ABI library (``libpagedkv.so``, declared in
``include/pagedkv.h``):

* ``pkv_kv_write``: slot-mapping scatter of new tokens' K/V into the block pool;
* ``pkv_block_copy``: whole-block copies for copy-on-write of shared blocks;
* ``pkv_attention_decode``: decode-step attention through per-sequence block
  tables, split over token partitions with a rescaling reduce.

The Python functions of the same names (``paged_kv_cache_330_amd.ops``) only
marshal torch tensors into that ABI; importing this package does not load the
library, the first call does, and it fails loudly when the library is absent.
"""
from .block_manager import BlockManager, PoolExhausted  # noqa: F401

__all__ = ["BlockManager", "PoolExhausted"]
