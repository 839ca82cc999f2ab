"""Python binding of libpa's host block allocator (pa_alloc_* in include/pa.h)."""
import ctypes
from typing import List, Sequence, Tuple

import numpy as np

from ._lib import OutOfBlocks, PaError, check, lib  # noqa: F401

_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(_I64P)


class BlockAllocator:
    """Block tables, on-demand blocks, refcounted sharing (fork), copy-on-write (append) and an
    optional prefix cache of full blocks keyed by their token prefix."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Sequence[int] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        h = ctypes.c_void_p()
        order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        check(lib().pa_alloc_create(self.num_blocks, self.block_size, None if order is None else _i32p(order),
                                    ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().pa_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_seq(self, sid: int) -> None:
        check(lib().pa_alloc_add_seq(self._h, int(sid)))

    def fork(self, parent: int, child: int) -> None:
        check(lib().pa_alloc_fork(self._h, int(parent), int(child)))

    def free_seq(self, sid: int) -> None:
        check(lib().pa_alloc_free_seq(self._h, int(sid)))

    def append(self, sid: int, n: int) -> Tuple[np.ndarray, np.ndarray]:
        """(slots int64 [n], cow pairs int32 [k, 2])."""
        slots = np.empty(max(int(n), 1), dtype=np.int64)
        cow = np.empty((1, 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        check(lib().pa_alloc_append(self._h, int(sid), int(n), _i64p(slots), _i32p(cow), 1, ctypes.byref(ncow)))
        return slots[:int(n)], cow[:ncow.value]

    def append_batch(self, sids: Sequence[int], ns: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(sids, dtype=np.int64)
        cnt = np.ascontiguousarray(ns, dtype=np.int32)
        total = int(cnt.sum())
        slots = np.empty(max(total, 1), dtype=np.int64)
        cow = np.empty((max(len(ids), 1), 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        check(lib().pa_alloc_append_batch(self._h, _i64p(ids), _i32p(cnt), len(ids), _i64p(slots), _i32p(cow),
                                          len(ids), ctypes.byref(ncow)))
        return slots[:total], cow[:ncow.value]

    def blocks_needed(self, sid: int, n: int) -> int:
        out = ctypes.c_int32(0)
        check(lib().pa_alloc_blocks_needed(self._h, int(sid), int(n), ctypes.byref(out)))
        return out.value

    def length(self, sid: int) -> int:
        out = ctypes.c_int64(0)
        check(lib().pa_alloc_seq_len(self._h, int(sid), ctypes.byref(out)))
        return out.value

    def table(self, sid: int) -> List[int]:
        n = ctypes.c_int32(0)
        cap = self.num_blocks
        buf = np.empty(max(cap, 1), dtype=np.int32)
        check(lib().pa_alloc_block_table(self._h, int(sid), _i32p(buf), cap, ctypes.byref(n)))
        return buf[:n.value].tolist()

    def fill_tables(self, sids: Sequence[int], max_blocks: int, pad: int = 0) -> np.ndarray:
        ids = np.ascontiguousarray(sids, dtype=np.int64)
        out = np.empty((len(ids), max_blocks), dtype=np.int32)
        check(lib().pa_alloc_fill_tables(self._h, _i64p(ids), len(ids), _i32p(out), int(max_blocks), int(pad)))
        return out

    def refcount(self, blk: int) -> int:
        out = ctypes.c_int32(0)
        check(lib().pa_alloc_refcount(self._h, int(blk), ctypes.byref(out)))
        return out.value

    def stats(self) -> Tuple[int, int, int]:
        f, u, r = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
        check(lib().pa_alloc_stats(self._h, ctypes.byref(f), ctypes.byref(u), ctypes.byref(r)))
        return f.value, u.value, r.value

    def num_free(self) -> int:
        return self.stats()[0]

    def free_list(self) -> List[int]:
        n = ctypes.c_int32(0)
        buf = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        check(lib().pa_alloc_free_list(self._h, _i32p(buf), self.num_blocks, ctypes.byref(n)))
        return buf[:n.value].tolist()

    # -- prefix cache ---------------------------------------------------------------------------
    def enable_prefix_cache(self) -> None:
        check(lib().pa_alloc_enable_prefix_cache(self._h))

    def add_seq_prefix(self, sid: int, tokens: Sequence[int]) -> int:
        """New sequence whose table starts with the cached blocks matching `tokens` (at least one
        token left over); returns the number of prompt tokens those blocks already hold."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = ctypes.c_int32(0)
        buf = tok if tok.size else np.zeros(1, np.int32)
        check(lib().pa_alloc_add_seq_prefix(self._h, int(sid), _i32p(buf), int(tok.size), ctypes.byref(n)))
        return n.value

    def cache_seq(self, sid: int, tokens: Sequence[int]) -> None:
        """Register the full blocks of `sid` holding tokens[:len(tokens)] (their K/V written)."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        buf = tok if tok.size else np.zeros(1, np.int32)
        check(lib().pa_alloc_cache_seq(self._h, int(sid), _i32p(buf), int(tok.size)))

    def cache_stats(self) -> Tuple[int, int]:
        """(cache entries, evictable blocks)."""
        c, e = ctypes.c_int32(0), ctypes.c_int32(0)
        check(lib().pa_alloc_cache_stats(self._h, ctypes.byref(c), ctypes.byref(e)))
        return c.value, e.value

    def num_cached(self) -> int:
        return self.cache_stats()[0]

    def available(self) -> int:
        """Blocks an append can take: free plus evictable."""
        return self.num_free() + self.cache_stats()[1]

    def evictable_list(self) -> List[int]:
        n = ctypes.c_int32(0)
        buf = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        check(lib().pa_alloc_evictable_list(self._h, _i32p(buf), self.num_blocks, ctypes.byref(n)))
        return buf[:n.value].tolist()


def move_seq(src: BlockAllocator, dst: BlockAllocator, sid: int) -> np.ndarray:
    """Move a sequence between two pools' allocators (swap-out or swap-in); returns the int32 [n, 2]
    (source block, destination block) pairs to copy with pa_swap_blocks."""
    n = ctypes.c_int32(0)
    cap = max(src.num_blocks, 1)
    buf = np.empty((cap, 2), dtype=np.int32)
    check(lib().pa_alloc_move_seq(src._h, dst._h, int(sid), _i32p(buf), cap, ctypes.byref(n)))
    return buf[:n.value].copy()
