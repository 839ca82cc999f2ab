"""A synthetic continuous-batching loop over the paged pool, with KV-utilisation accounting.

Every step, finished requests leave and free their blocks, and waiting requests join at once when
the pool can hold them ([ch7] 7.1 and [exp] on continuous batching; [day28] §五: freed blocks serve
new requests immediately).  Policy (a reading; the pages describe the idea, not a policy):

  * admission in arrival order, while the blocks free after the prompt stay at or above a
    watermark (1% of the pool, at least one block), so that a newly admitted request does not
    force a preemption at once;
  * a request's prompt K/V is written when it is admitted (the prefill's cache write; the prefill
    attention itself is `pa_prefill_chunk` and not part of this loop); from the next step on it
    decodes one token per step: the decode attends its L tokens and the new token's K/V goes to
    position L;
  * when a decode cannot get a block, the most recently admitted running request is preempted: its
    blocks are freed and it waits again at the head of the queue, to be recomputed from its prompt
    (the pages' other option, swap, is `pa_alloc_move_seq` + `pa_swap_blocks`).

Accounting per step ([ch7] and [day28] §四 compare the KV memory a paged engine uses with what a
max-length reservation sets aside): tokens held by running requests, against the slots of the
blocks in use (paged) and against max_model_len slots per running request (reservation).
"""
from collections import deque
from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np
import torch

from ._lib import PA_BF16
from .allocator import BlockAllocator, OutOfBlocks
from .ops import make_pool_desc, pa_cache_write, pa_decode, pa_decode_workspace_size


@dataclass
class StepStats:
    step: int
    running: int
    decoded: int
    admitted: int
    finished: int
    preempted: int
    tokens_held: int
    blocks_used: int


@dataclass
class DecodeBatch:
    """What one step's decode computed (kept when the loop runs with keep_batches)."""
    rids: List[int]
    lens: np.ndarray
    q_rows: List[int]
    out: torch.Tensor


class ContinuousBatcher:
    def __init__(self, stream, num_blocks: int, device: str = "cuda", device_work: bool = True,
                 keep_batches: bool = False, watermark: float = 0.01):
        self.s = stream
        self.b = stream.block_size
        self.num_blocks = int(num_blocks)
        self.alloc = BlockAllocator(self.num_blocks, self.b)
        self.device = torch.device(device)
        self.device_work = device_work
        self.keep_batches = keep_batches
        self.waiting = deque()
        self.running = []          # [request, tokens generated so far], in admission order
        self.pending = sorted(stream.requests, key=lambda r: (r.arrival, r.rid))
        self.next_pending = 0
        self.stats: List[StepStats] = []
        self.ops: List[tuple] = []     # the allocator operations, in order (for checking)
        self.batches: List[DecodeBatch] = []
        self.preemptions = 0
        self.watermark_blocks = max(1, int(np.ceil(watermark * self.num_blocks)))
        if device_work:
            st = stream
            self.pool = make_pool_desc(self.num_blocks, self.b, st.num_kv_heads, st.head_dim, PA_BF16)
            nan = 0x7FC0
            self.k_pool = torch.full((self.num_blocks, st.num_kv_heads, self.b, st.head_dim), nan,
                                     dtype=torch.int16, device=self.device).view(torch.bfloat16)
            self.v_pool = torch.full((self.num_blocks, st.num_kv_heads, st.head_dim, self.b), nan,
                                     dtype=torch.int16, device=self.device).view(torch.bfloat16)
            self.k_table = st.k_table.to(self.device)
            self.v_table = st.v_table.to(self.device)
            self.q_table = st.q_table.to(self.device)
            # one workspace for the largest possible batch (every request holds at least one block)
            ws = pa_decode_workspace_size(self.num_blocks, st.num_q_heads, st.head_dim, st.max_model_len, 0)
            self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=self.device)
            self.max_blocks = -(-st.max_model_len // self.b) + 1

    # -- host scheduling ------------------------------------------------------------------------
    def _preempt_newest(self) -> None:
        req, _ = self.running.pop()
        self.alloc.free_seq(req.rid)
        self.ops.append(("free", req.rid))
        self.waiting.appendleft(req)
        self.preemptions += 1

    def step(self, t: int) -> StepStats:
        b = self.b
        pre0 = self.preemptions
        finished = 0
        keep = []
        for req, gen in self.running:
            if gen >= req.output_len:
                self.alloc.free_seq(req.rid)
                self.ops.append(("free", req.rid))
                finished += 1
            else:
                keep.append([req, gen])
        self.running = keep
        while self.next_pending < len(self.pending) and self.pending[self.next_pending].arrival <= t:
            self.waiting.append(self.pending[self.next_pending])
            self.next_pending += 1

        writes = []                # (rid, first position, slots)
        # decode: every running request gets one new token; a shortage preempts the newest request
        decode = []
        i = 0
        while i < len(self.running):
            req, gen = self.running[i]
            L = self.alloc.length(req.rid)
            try:
                slots, cow = self.alloc.append(req.rid, 1)
            except OutOfBlocks:
                self._preempt_newest()
                continue           # retry the same index (or stop if it was the one preempted)
            self.ops.append(("append", req.rid, 1))
            decode.append((req.rid, L))
            writes.append((req.rid, L, slots))
            self.running[i][1] += 1
            i += 1
        # admission, in arrival order, above the watermark
        admitted = 0
        while self.waiting:
            req = self.waiting[0]
            need = -(-req.prompt_len // b)
            if self.alloc.available() - need < self.watermark_blocks:
                break
            self.waiting.popleft()
            self.alloc.add_seq(req.rid)
            slots, _ = self.alloc.append(req.rid, req.prompt_len)
            self.ops += [("add", req.rid), ("append", req.rid, req.prompt_len)]
            writes.append((req.rid, 0, slots))
            self.running.append([req, 0])
            admitted += 1

        if self.device_work:
            self._device_step(writes, decode)
        tokens = sum(self.alloc.length(r.rid) for r, _ in self.running)
        st = StepStats(t, len(self.running), len(decode), admitted, finished, self.preemptions - pre0, tokens,
                       self.num_blocks - self.alloc.available())
        self.stats.append(st)
        return st

    # -- device work ----------------------------------------------------------------------------
    def _device_step(self, writes, decode) -> None:
        s, dev = self.s, self.device
        if writes:
            rows = torch.cat([s.kv_rows(rid, p0, len(sl)) for rid, p0, sl in writes]).to(dev)
            slots = torch.as_tensor(np.concatenate([sl for _, _, sl in writes]).astype(np.int64), device=dev)
            pa_cache_write(self.k_table.index_select(0, rows), self.v_table.index_select(0, rows), slots,
                           self.k_pool, self.v_pool, self.pool)
        if decode:
            rids = [rid for rid, _ in decode]
            lens = np.asarray([L for _, L in decode], np.int32)
            qrows = [s.q_row(rid, int(L)) for rid, L in decode]
            q = self.q_table.index_select(0, torch.as_tensor(qrows, device=dev))
            tabs = torch.as_tensor(self.alloc.fill_tables(rids, self.max_blocks), device=dev)
            out = torch.empty_like(q)
            pa_decode(q, self.k_pool, self.v_pool, self.pool, tabs, torch.as_tensor(lens, device=dev), s.scale, out,
                      int(lens.max()), 0, self.workspace)
            if self.keep_batches:
                self.batches.append(DecodeBatch(rids, lens, qrows, out))

    def run(self, steps: int) -> List[StepStats]:
        for t in range(steps):
            self.step(t)
        return self.stats


def utilisation(stats: List[StepStats], block_size: int, max_model_len: int, num_blocks: int) -> dict:
    """Mean KV utilisation over the steps that hold tokens: tokens held / slots of the blocks in use
    (paged), and tokens held / max_model_len slots per running request (reservation); the number of
    requests a reservation-based pool of the same size could hold at once."""
    act = [s for s in stats if s.tokens_held > 0]
    paged = float(np.mean([s.tokens_held / (s.blocks_used * block_size) for s in act])) if act else 0.0
    reserved = float(np.mean([s.tokens_held / (s.running * max_model_len) for s in act])) if act else 0.0
    return {"paged": paged, "reservation": reserved,
            "mean_running": float(np.mean([s.running for s in act])) if act else 0.0,
            "reservation_capacity": (num_blocks * block_size) // max_model_len,
            "steps": len(stats), "active_steps": len(act)}
