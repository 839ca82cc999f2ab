"""paged_kv_cache_427_amd: paged KV-cache attention on AMD Instinct MI355X (gfx950).

The product is the C-ABI library libpa.so (include/pa.h), built from the HIP/C++ sources in csrc/
by `python -m paged_kv_cache_427_amd.build`.  This package is its thin Python binding:
  ops        pa_cache_write, pa_copy_blocks, pa_decode, pa_prefill_chunk, ... (torch tensors in,
             argument marshalling only)
  allocator  BlockAllocator over pa_alloc_* (host block tables, refcounts, copy-on-write)
  engine     PagedKVEngine: replays sequence operations and runs one device step
Importing the package does not load the library; the first call does, and raises if it is missing.
"""
from ._lib import (PA_BF16, PA_F32, PA_FP8_E4M3, LIB_PATH, EXPORTED, OutOfBlocks, PaError,  # noqa: F401
                   PoolDesc, lib)
