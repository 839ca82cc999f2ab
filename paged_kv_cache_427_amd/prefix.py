"""Prefill of a prompt batch through the allocator's prefix cache, on one layer's pools.

A new request first attaches the cached blocks that already hold the start of its prompt
(pa_alloc_add_seq_prefix), then takes slots for the rest; the step writes and prefills only those
remaining tokens, with the attached blocks as prior context.  After its prefill the request's full
prompt blocks are registered (pa_alloc_cache_seq), so later requests with the same start skip them.
«第 7 章推理框架：vLLM 与 PagedAttention», 7.1 (prefix caching); «GPU 学习日报 Day 28：vLLM 与
PagedAttention：GPU Memory 管理的艺术», §七 (a cached system prompt is not prefilled again).
With caching off, the same driver prefills every prompt in full.
"""
from dataclasses import dataclass
from typing import List, Sequence

import numpy as np
import torch

from ._lib import PA_BF16
from .allocator import BlockAllocator
from .ops import make_pool_desc, pa_cache_write, pa_prefill_chunk


@dataclass
class PrefillInputs:
    """Device inputs of one admitted batch (everything a timed step needs)."""
    seq_ids: List[int]
    cached: np.ndarray          # int32 [n]: prompt tokens each request found in the cache
    chunk: np.ndarray           # int32 [n]: prompt tokens each request computes
    slots: torch.Tensor         # int64 [sum(chunk)]
    k: torch.Tensor             # [sum(chunk), Hkv, D]
    v: torch.Tensor
    q: torch.Tensor             # [sum(chunk), Hq, D]
    tables: torch.Tensor        # int32 [n, max_blocks]
    qsl: torch.Tensor           # int32 [n + 1]
    prior: torch.Tensor         # int32 [n]
    max_chunk: int
    out: torch.Tensor           # [sum(chunk), Hq, D]


class PrefixPrefill:
    """Owns the pools and the host allocator for a prompt batch (package `synth.prefix`)."""

    def __init__(self, batch, device="cuda", caching: bool = True, num_blocks: int = None,
                 poison: int = 0x7FC0):
        if batch.kv_dtype != "bf16" or batch.act_dtype != "bf16":
            raise ValueError("this driver runs bf16 pools and activations")
        self.b = batch
        self.device = torch.device(device)
        self.caching = caching
        nb = batch.num_blocks if num_blocks is None else int(num_blocks)
        self.pool = make_pool_desc(nb, batch.block_size, batch.num_kv_heads, batch.head_dim, PA_BF16)
        fill = poison - (1 << 16) if poison >= (1 << 15) else poison
        k_shape = (nb, batch.num_kv_heads, batch.block_size, batch.head_dim)
        v_shape = (nb, batch.num_kv_heads, batch.head_dim, batch.block_size)
        self.k_pool = torch.full(k_shape, fill, dtype=torch.int16, device=self.device).view(torch.bfloat16)
        self.v_pool = torch.full(v_shape, fill, dtype=torch.int16, device=self.device).view(torch.bfloat16)
        order = batch.free_order if num_blocks is None else np.arange(nb, dtype=np.int32)
        self.alloc = BlockAllocator(nb, batch.block_size, order)
        if caching:
            self.alloc.enable_prefix_cache()

    def admit(self, requests: Sequence[int], seq_ids: Sequence[int] = None) -> PrefillInputs:
        """Host side of admitting `requests` (indices into the batch): cache lookup, slots, tables."""
        b = self.b
        ids = list(requests) if seq_ids is None else [int(x) for x in seq_ids]
        cached, chunk, slots, qs, ks, vs = [], [], [], [], [], []
        for r, sid in zip(requests, ids):
            prompt = b.prompt(r)
            if self.caching:
                n = self.alloc.add_seq_prefix(sid, prompt)
            else:
                self.alloc.add_seq(sid)
                n = 0
            sl, cow = self.alloc.append(sid, len(prompt) - n)
            if len(cow):
                raise RuntimeError("a fresh prompt never writes into a shared block")
            q, k, v = b.rows(r, n, len(prompt))
            cached.append(n)
            chunk.append(len(prompt) - n)
            slots.append(sl)
            qs.append(q)
            ks.append(k)
            vs.append(v)
        dev = self.device
        chunk_a = np.asarray(chunk, np.int32)
        mb = max(max(len(self.alloc.table(s)) for s in ids), 1)
        q = torch.cat(qs).to(dev)
        return PrefillInputs(
            seq_ids=ids, cached=np.asarray(cached, np.int32), chunk=chunk_a,
            slots=torch.as_tensor(np.concatenate(slots).astype(np.int64), device=dev),
            k=torch.cat(ks).to(dev), v=torch.cat(vs).to(dev), q=q,
            tables=torch.as_tensor(self.alloc.fill_tables(ids, mb), device=dev),
            qsl=torch.as_tensor(np.concatenate([[0], np.cumsum(chunk_a)]).astype(np.int32), device=dev),
            prior=torch.as_tensor(np.asarray(cached, np.int32), device=dev),
            max_chunk=int(chunk_a.max()) if len(chunk_a) else 0, out=torch.empty_like(q))

    def write(self, pi: PrefillInputs, stream=None) -> None:
        pa_cache_write(pi.k, pi.v, pi.slots, self.k_pool, self.v_pool, self.pool, stream)

    def prefill(self, pi: PrefillInputs, stream=None) -> None:
        pa_prefill_chunk(pi.q, self.k_pool, self.v_pool, self.pool, pi.tables, pi.qsl, pi.prior, self.b.scale,
                         pi.max_chunk, pi.out, stream)

    def register(self, pi: PrefillInputs, requests: Sequence[int]) -> None:
        """Cache the full prompt blocks of admitted requests (call once their K/V are written)."""
        for r, sid in zip(requests, pi.seq_ids):
            self.alloc.cache_seq(sid, self.b.prompt(r))

    def release(self, pi: PrefillInputs) -> None:
        for sid in pi.seq_ids:
            self.alloc.free_seq(sid)
