"""The physical KV pool: slot addressing, writing new tokens, block copies, gathering a sequence.

Pool layout (a reading; the pages fix only that a block holds the K/V of b consecutive tokens and
is contiguous inside, [day28] §三 3.1-3.2): K and V are two separate arrays of stored codes
(uint32 fp32 bits, uint16 bf16 bits or uint8 e4m3 codes).  Both are split into (block, KV head)
tiles of b x head_dim codes, contiguous; the K tile is token-major and the V tile dim-major:
  K pool: [num_blocks][num_kv_heads][block_size][head_dim]   (which="k")
  V pool: [num_blocks][num_kv_heads][head_dim][block_size]   (which="v")
so element (token offset o, dim d) of a tile sits at o * head_dim + d in K and d * block_size + o
in V.

Slot of logical position p of a sequence with table T: T[p // b] * b + p % b, as in the
block-table figure of [day28] §三 3.1 (table [7, 1, 3]: logical block 0 -> physical 7 holds
tokens 0-15, block 1 -> physical 1 holds tokens 16-31, block 2 -> physical 3 holds 32-47).
"""
from typing import Sequence

import numpy as np

from .codecs import e4m3_quantise, f32_bits_to_f64, bf16_bits_to_f64


def slot_of(table: Sequence[int], p: int, block_size: int) -> int:
    """Slot (physical block * b + offset) of logical position p."""
    return int(table[p // block_size]) * block_size + p % block_size


def pool_shape(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, which: str):
    """Array shape of a K (which="k") or V (which="v") pool."""
    if which == "k":
        return (num_blocks, num_kv_heads, block_size, head_dim)
    if which == "v":
        return (num_blocks, num_kv_heads, head_dim, block_size)
    raise ValueError(which)


def _block_size(pool: np.ndarray, which: str) -> int:
    return pool.shape[2] if which == "k" else pool.shape[3]


def ref_cache_write(pool: np.ndarray, x_bits: np.ndarray, slots: Sequence[int], kv_dtype: str,
                    act_dtype: str, scale: float = 1.0, which: str = "k") -> None:
    """Write token rows into their slots, in place.

    pool   : stored codes, laid out as pool_shape(..., which)
    x_bits : [T, Hkv, D] bit patterns of the new rows in the activation dtype
             (uint32 for fp32, uint16 for bf16)
    slots  : [T] int; a negative slot means "skip this token"
    For an fp8 pool each value is quantised with `scale` (codecs.e4m3_quantise); otherwise the
    bit pattern is stored unchanged (pool dtype == activation dtype).
    """
    b = _block_size(pool, which)
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = s // b, s % b
        if kv_dtype == "fp8":
            if act_dtype == "bf16":
                vals = bf16_bits_to_f64(x_bits[t]).astype(np.float32)
            else:
                vals = f32_bits_to_f64(x_bits[t]).astype(np.float32)
            codes = e4m3_quantise(vals, scale)
        else:
            assert kv_dtype == act_dtype, "a non-fp8 pool stores the activation dtype"
            codes = x_bits[t]
        if which == "k":
            pool[blk, :, off, :] = codes
        else:
            pool[blk, :, :, off] = codes


def ref_copy_blocks(pool: np.ndarray, pairs: Sequence) -> None:
    """Copy-on-write: block dst receives the content of block src, for each (src, dst) pair, in order
    ([day28] §四 4.2, §六 item 4)."""
    for src, dst in pairs:
        pool[int(dst)] = pool[int(src)].copy()


def ref_move_blocks(dst_pool: np.ndarray, src_pool: np.ndarray, pairs: Sequence) -> None:
    """Swap: block d of dst_pool receives block s of src_pool, for each (s, d) pair ([day28] §六
    question 4).  The two pools hold blocks of one format; stored codes move unchanged."""
    for src, dst in pairs:
        dst_pool[int(dst)] = src_pool[int(src)].copy()


def gather_seq(pool_vals: np.ndarray, table: Sequence[int], length: int, which: str = "k") -> np.ndarray:
    """Contiguous [length, Hkv, D] K (which="k") or V (which="v") of a sequence, rebuilt through its
    block table ([day28] §三 3.1: the kernel reaches scattered K/V by indirection through the table)."""
    b = _block_size(pool_vals, which)
    hkv = pool_vals.shape[1]
    d = pool_vals.shape[3] if which == "k" else pool_vals.shape[2]
    out = np.empty((length, hkv, d), dtype=np.float64)
    for p in range(length):
        blk, off = int(table[p // b]), p % b
        out[p] = pool_vals[blk, :, off, :] if which == "k" else pool_vals[blk, :, :, off]
    return out
