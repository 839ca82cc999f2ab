"""CPU oracle for paged KV-cache attention.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import this package.
The product (package `paged_kv_cache_427_amd`, library libpa.so) never imports, links or calls it,
and this package imports nothing from the product.  It shares no code with the GPU path; the only
common module is `synth` (seeded input generators, no arithmetic of the method).

Everything here is plain NumPy in float64 (integers for slots, tables and stored codes), written
for readability, not speed.  Pages cited (by title):
  [ch7]   «第 7 章推理框架：vLLM 与 PagedAttention» (blog.lkad.net)
  [exp]   «vLLM 与 PagedAttention：把 GPU 显存当操作系统内存管» (alishangtian.com)
  [day28] «GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术» (daoyuly.cn)

Every function is pinned by a `-m "not gpu"` test against something other than itself (printed
worked values, closed forms, brute force, library routines, invariants); nothing is
"parity unpinned".
"""
from .sizes import kv_bytes_per_token, kv_cache_bytes  # noqa: F401
from .codecs import (  # noqa: F401
    bf16_bits_to_f64, f32_bits_to_f64, e4m3_decode, e4m3_encode, e4m3_quantise, decode_pool,
)
from .allocator import RefAllocator, AllocError, OutOfBlocks, move_seq  # noqa: F401
from .logical import LogicalSeqs  # noqa: F401
from .cache import (  # noqa: F401
    slot_of, pool_shape, ref_cache_write, ref_copy_blocks, ref_move_blocks, gather_seq,
)
from .attention import (  # noqa: F401
    attend, ref_decode, ref_decode_split, partition_stats, merge_partitions, ref_prefill, ref_lse,
)
