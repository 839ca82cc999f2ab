"""Reference block allocator: block tables, on-demand allocation, shared blocks, copy-on-write.

What the pages fix:
  * KV cache is cut into fixed-size blocks, 16 tokens by default; each sequence owns a block table
    mapping logical block i to a physical block; a new block is taken only when the last one is
    full ([ch7] 7.1 「三个关键机制」; [day28] §三 3.1 and §四 4.2).
  * the pool is a set of uniform blocks and any free block can serve any sequence; blocks return to
    the pool when a sequence finishes ([ch7] 7.1 「消除碎片」; [day28] §四 4.2, §五).
  * sequences with a common prefix point at the same physical blocks under a reference count; a
    sequence that must write into a shared block first gets a new block, the content is copied and
    the old block's count drops by one ([exp] 「PagedAttention：向操作系统借思路」;
    [day28] §四 4.2 and §六 items 3-4).
  * running out of blocks is still possible ([day28] FAQ Q3).

Prefix caching ([ch7] 7.1 「三个关键机制」 and its vLLM parameter list: requests with the same
system-prompt prefix point at the same physical blocks under a reference count, only the differing
suffixes get blocks of their own; [day28] §七: requests sharing a cached system prompt skip its
prefill; [day28] FAQ Q5: that pays when the shared prefix is long and stable).

Readings taken where the pages are silent:
  * free list: a FIFO queue whose initial order is given; freed blocks join its tail in table order.
  * slot of logical position p: table[p // b] * b + p % b.
  * append is all-or-nothing: if the free list cannot cover every block it needs, nothing changes.
  * prefix cache (when enabled): only full blocks are cached.  A block's key is (the entry id of the
    block before it, or 0 for the first, and its b token ids); entry ids are never reused, so a key
    names one exact token prefix.  A new sequence takes the longest run of cached blocks matching
    its prompt, but always leaves at least one prompt token to compute.  A cached block whose count
    falls to zero is not freed but kept, least recently released first, and is reclaimed (its entry
    dropped) only when the free list is empty.  The cached blocks one release leaves unreferenced
    are queued from the table's last block to its first, so a chain loses its deepest blocks first
    and its head stays matchable.
"""
from collections import OrderedDict, deque
from typing import Dict, List, Optional, Sequence, Tuple


class AllocError(Exception):
    """Invalid request (unknown or duplicate sequence id, bad count)."""


class OutOfBlocks(Exception):
    """Not enough free blocks; the allocator state is unchanged."""


class RefAllocator:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.caching = False
        self.entries: Dict[Tuple[int, Tuple[int, ...]], int] = {}   # key -> entry id
        self.entry_block: Dict[int, int] = {}                        # entry id -> block
        self.entry_key: Dict[int, Tuple[int, Tuple[int, ...]]] = {}
        self.block_entry: List[int] = [0] * num_blocks               # 0: the block is not cached
        self.evictable: "OrderedDict[int, None]" = OrderedDict()     # cached, count 0, oldest first
        self.next_entry = 1

    # -- block supply -------------------------------------------------------------------------
    def enable_prefix_cache(self) -> None:
        self.caching = True

    def available(self) -> int:
        """Blocks an append can take: free ones, then cached ones nobody points at."""
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            return self.free.popleft()
        blk, _ = self.evictable.popitem(last=False)      # least recently released cached block
        eid = self.block_entry[blk]
        del self.entries[self.entry_key.pop(eid)]
        del self.entry_block[eid]
        self.block_entry[blk] = 0
        return blk

    def _release(self, table: Sequence[int]) -> None:
        """Drop one reference to each block of a table.  Blocks left unreferenced join the free list
        in table order, or, when cached, the evictable list from the table's last block to its first:
        a lookup walks a chain from its first block, so the deepest blocks should go first."""
        for blk in table:
            self.ref[blk] -= 1
            if self.ref[blk] == 0 and not self.block_entry[blk]:
                self.free.append(blk)
        for blk in reversed(table):
            if self.ref[blk] == 0 and self.block_entry[blk]:
                self.evictable[blk] = None

    # -- prefix cache -------------------------------------------------------------------------
    def add_seq_prefix(self, sid: int, tokens: Sequence[int]) -> int:
        """New sequence whose prompt is `tokens`: its table starts with the longest run of cached
        full blocks matching the prompt (leaving at least one token).  Returns the tokens covered."""
        self.add_seq(sid)
        if not self.caching:
            return 0
        b = self.block_size
        parent = 0
        table = self.tables[sid]
        while (len(table) + 1) * b <= len(tokens) - 1:
            j = len(table)
            eid = self.entries.get((parent, tuple(int(x) for x in tokens[j * b:(j + 1) * b])))
            if eid is None:
                break
            blk = self.entry_block[eid]
            if self.ref[blk] == 0:
                del self.evictable[blk]
            self.ref[blk] += 1
            table.append(blk)
            parent = eid
        self.lens[sid] = len(table) * b
        return self.lens[sid]

    def cache_seq(self, sid: int, tokens: Sequence[int]) -> None:
        """Register the full blocks of `sid` that hold tokens[0 : len(tokens)] (their K/V written)."""
        if sid not in self.tables:
            raise AllocError(f"unknown sequence {sid}")
        if len(tokens) > self.lens[sid]:
            raise AllocError("more tokens than the sequence holds")
        if not self.caching:
            return
        b = self.block_size
        parent = 0
        table = self.tables[sid]
        for j in range(len(tokens) // b):
            key = (parent, tuple(int(x) for x in tokens[j * b:(j + 1) * b]))
            eid = self.entries.get(key)
            blk = table[j]
            if eid is None:
                if self.block_entry[blk]:
                    raise AllocError(f"block {blk} is cached under other tokens")
                eid = self.next_entry
                self.next_entry += 1
                self.entries[key] = eid
                self.entry_key[eid] = key
                self.entry_block[eid] = blk
                self.block_entry[blk] = eid
            parent = eid

    # -- sequence lifecycle -------------------------------------------------------------------
    def add_seq(self, sid: int) -> None:
        if sid in self.tables:
            raise AllocError(f"sequence {sid} exists")
        self.tables[sid] = []
        self.lens[sid] = 0

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent; each shared block's count rises by one."""
        if parent not in self.tables:
            raise AllocError(f"unknown sequence {parent}")
        if child in self.tables:
            raise AllocError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1

    def free_seq(self, sid: int) -> None:
        """Drop the sequence; blocks whose count reaches zero go back to the tail of the free list."""
        if sid not in self.tables:
            raise AllocError(f"unknown sequence {sid}")
        self._release(self.tables[sid])
        del self.tables[sid]
        del self.lens[sid]

    def blocks_needed(self, sid: int, n: int) -> int:
        """Free blocks an append of n tokens would take (new blocks plus one copy-on-write)."""
        b = self.block_size
        length = self.lens[sid]
        table = self.tables[sid]
        need = 0
        if n > 0 and length % b != 0 and self.ref[table[length // b]] > 1:
            need += 1
        new_len = length + n
        need += -(-new_len // b) - len(table)
        return need

    def append(self, sid: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Give slots to n new tokens of `sid`.

        Returns (slots, cow_pairs): one slot per token, and the (source, destination) block pairs
        whose content must be copied before the new tokens are written.
        """
        if sid not in self.tables:
            raise AllocError(f"unknown sequence {sid}")
        if n < 0:
            raise AllocError("negative token count")
        if self.blocks_needed(sid, n) > self.available():
            raise OutOfBlocks(f"sequence {sid}: need {self.blocks_needed(sid, n)} blocks, "
                              f"{self.available()} available")
        b = self.block_size
        table = self.tables[sid]
        slots: List[int] = []
        cow: List[Tuple[int, int]] = []
        for _ in range(n):
            p = self.lens[sid]
            logical = p // b
            if p % b == 0:
                # first token of a new logical block: take the head of the free list
                blk = self._take()
                self.ref[blk] = 1
                table.append(blk)
            elif self.ref[table[logical]] > 1:
                # writing into a block someone else also points at: copy it first
                old = table[logical]
                new = self._take()
                self.ref[old] -= 1
                self.ref[new] = 1
                table[logical] = new
                cow.append((old, new))
            slots.append(table[logical] * b + p % b)
            self.lens[sid] = p + 1
        return slots, cow

    # -- inspection ---------------------------------------------------------------------------
    def table(self, sid: int) -> List[int]:
        return list(self.tables[sid])

    def length(self, sid: int) -> int:
        return self.lens[sid]

    def refcount(self, blk: int) -> int:
        return self.ref[blk]

    def num_free(self) -> int:
        return len(self.free)

    def num_cached(self) -> int:
        return len(self.entries)

    def evictable_list(self) -> List[int]:
        return list(self.evictable)

    def free_list(self) -> List[int]:
        return list(self.free)

    def check_invariants(self) -> None:
        """Invariants the pages state: tail waste below one block ([day28] §四 4.2), every block is
        either free or referenced ([ch7] 7.1 「消除碎片」), counts equal the number of tables holding
        the block ([day28] §六 item 3)."""
        b = self.block_size
        count = [0] * self.num_blocks
        for sid, tab in self.tables.items():
            assert len(tab) == -(-self.lens[sid] // b), "table length != ceil(len / b)"
            assert len(tab) * b - self.lens[sid] <= b - 1, "tail waste exceeds b - 1 slots"
            for blk in tab:
                count[blk] += 1
        assert count == self.ref, "reference counts differ from table membership"
        free = set(self.free)
        assert len(free) == len(self.free), "duplicate block on the free list"
        used = {i for i, c in enumerate(count) if c > 0}
        idle = set(self.evictable)
        assert not (free & used), "a referenced block is on the free list"
        assert not (idle & used) and not (idle & free), "an evictable block is in use or free"
        assert free | used | idle == set(range(self.num_blocks)), "a block is neither free nor referenced"
        # cache: every entry names one block and back; evictable blocks are exactly the cached ones
        # nobody points at
        assert len(self.entries) == len(self.entry_block) == len(self.entry_key)
        for key, eid in self.entries.items():
            assert self.entry_key[eid] == key and self.block_entry[self.entry_block[eid]] == eid
        cached = {blk for blk in range(self.num_blocks) if self.block_entry[blk]}
        assert cached == set(self.entry_block.values())
        assert idle == {blk for blk in cached if self.ref[blk] == 0}


def move_seq(src: RefAllocator, dst: RefAllocator, sid) -> List[Tuple[int, int]]:
    """Move sequence `sid` from the pool `src` manages to the pool `dst` manages: swap-out (device
    to host) or swap-in (host to device) of a preempted request ([day28] §六 question 4: preemption
    swaps a request's KV cache out to CPU memory, which paging makes a matter of copying the blocks
    its table lists; FAQ Q3: memory can still run out under paging).

    Reading: every block of the table gets a fresh block from dst's supply (free list, then idle
    cached blocks), in table order, and the sequence keeps its length; then the sequence is freed in
    src like any finished one, so a block it shared with another sequence stays in src with one
    reference less.  All-or-nothing: OutOfBlocks, with both states unchanged, when dst cannot supply
    every block.  Returns the (src block, dst block) pairs whose content must be copied."""
    if src.block_size != dst.block_size:
        raise AllocError("the two pools have different block sizes")
    if sid not in src.tables:
        raise AllocError(f"unknown sequence {sid}")
    if sid in dst.tables:
        raise AllocError(f"sequence {sid} exists in the destination")
    table = src.tables[sid]
    if len(table) > dst.available():
        raise OutOfBlocks(f"sequence {sid}: need {len(table)} blocks, {dst.available()} available")
    dst.add_seq(sid)
    pairs = []
    for blk in table:
        nb = dst._take()
        dst.ref[nb] = 1
        dst.tables[sid].append(nb)
        pairs.append((blk, nb))
    dst.lens[sid] = src.lens[sid]
    src.free_seq(sid)
    return pairs
