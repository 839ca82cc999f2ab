"""A paged-KV step driver: replays a workload's sequence operations on the host allocator and runs
the device calls of one step (copy-on-write copies, cache write, chunked prefill, decode).

Host side: pa_alloc_* (C++), which hands out slots and copy pairs.  Device side: the HIP kernels of
libpa, called through the binding with torch-owned memory on one stream.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from ._lib import PA_BF16, PA_F32, PA_FP8_E4M3, _I32P, check, lib
from .allocator import BlockAllocator
from .ops import (make_pool_desc, pa_cache_write, pa_copy_blocks, pa_decode, pa_decode_workspace_size,
                  pa_prefill_chunk, validate_decode, validate_pairs, validate_prefill, validate_slots)

_PA = {"f32": PA_F32, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}
_CODE_TORCH = {"f32": torch.int32, "bf16": torch.int16, "fp8": torch.uint8}
_VIEW = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


def _signed(code: int, bits: int) -> int:
    return code - (1 << bits) if code >= (1 << (bits - 1)) else code


def untouched_by_step(blocks: np.ndarray, cow_pairs: np.ndarray, slots: np.ndarray, block_size: int) -> bool:
    """True when none of `blocks` is a copy destination of the step (cow_pairs rows are (source,
    destination)) or receives one of its tokens (slot // block_size, slots < 0 unused): a decode
    that reads only those blocks then gives the same result before the step's copies and writes."""
    touched = set(np.asarray(cow_pairs).reshape(-1, 2)[:, 1].tolist())
    slots = np.asarray(slots)
    touched |= set((slots[slots >= 0] // block_size).tolist())
    return not (touched & set(np.asarray(blocks).tolist()))


def leading_shared_blocks(tables: np.ndarray, lens: np.ndarray, block_size: int) -> np.ndarray:
    """For each row, how many leading entries of its table (within its length) are physical blocks
    that another row of the same batch also reads: the pa_decode_ex `shared_blocks` hint (host,
    pa_plan_cache_hint)."""
    t = np.ascontiguousarray(tables, dtype=np.int32)
    l = np.ascontiguousarray(lens, dtype=np.int32)
    out = np.zeros(len(l), dtype=np.int32)
    if len(l) == 0:
        return out
    width = int(t.shape[1]) if t.ndim == 2 else 0
    check(lib().pa_plan_cache_hint(t.ctypes.data_as(_I32P), width, l.ctypes.data_as(_I32P), len(l),
                                   int(block_size), out.ctypes.data_as(_I32P)))
    return out


@dataclass
class StepInputs:
    """Device-resident inputs of one step (everything the timed region needs)."""
    cow_pairs: torch.Tensor                 # int32 [n, 2]
    slots: torch.Tensor                     # int64 [step tokens]
    k_new: torch.Tensor                     # [step tokens, Hkv, D]
    v_new: torch.Tensor
    dec_tables: Optional[torch.Tensor] = None
    dec_lens: Optional[torch.Tensor] = None
    dec_q: Optional[torch.Tensor] = None
    dec_out: Optional[torch.Tensor] = None
    dec_max_len: int = 0
    dec_workspace: Optional[torch.Tensor] = None
    dec_partition: int = 0
    dec_shared: Optional[torch.Tensor] = None   # int32 [seqs]: leading blocks other rows also read
    pre_tables: Optional[torch.Tensor] = None
    pre_qsl: Optional[torch.Tensor] = None
    pre_prior: Optional[torch.Tensor] = None
    pre_q: Optional[torch.Tensor] = None
    pre_out: Optional[torch.Tensor] = None
    pre_max_chunk: int = 0
    host_slots: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    host_cow: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), np.int32))


class PagedKVEngine:
    """Owns the two pools of one layer and the host allocator of a workload (package `synth`)."""

    def __init__(self, wl, device: str = "cuda", poison: Optional[int] = None, allocate_pools: bool = True,
                 validate: bool = False):
        self.wl = wl
        # validate: check every step's slots, copy pairs, tables and lengths on the host before they
        # go to the device (pa_validate_*)
        self.validate = validate
        self.device = torch.device(device)
        self.pool = make_pool_desc(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim,
                                   _PA[wl.kv_dtype], wl.k_scale, wl.v_scale)
        if allocate_pools:
            # K tiles are [block_size][head_dim] (token-major), V tiles [head_dim][block_size] (dim-major)
            k_shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
            v_shape = (wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.block_size)
            bits = {"f32": 32, "bf16": 16, "fp8": 8}[wl.kv_dtype]
            fill = 0 if poison is None else (_signed(poison, bits) if wl.kv_dtype != "fp8" else poison)
            code, view = _CODE_TORCH[wl.kv_dtype], _VIEW[wl.kv_dtype]
            self.k_pool = torch.full(k_shape, fill, dtype=code, device=self.device).view(view)
            self.v_pool = torch.full(v_shape, fill, dtype=code, device=self.device).view(view)
        self.alloc = BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
        self.k_tok = wl.k_tok.to(self.device)
        self.v_tok = wl.v_tok.to(self.device)
        self.history_slots = np.zeros(0, np.int64)

    # -- host replay --------------------------------------------------------------------------
    def _replay(self, ops: Sequence[Tuple], on_cow=None, slots_out=None) -> List[Tuple[int, int]]:
        cows: List[Tuple[int, int]] = []
        for op in ops:
            kind = op[0]
            if kind == "add":
                self.alloc.add_seq(op[1])
            elif kind == "fork":
                self.alloc.fork(op[1], op[2])
            elif kind == "free":
                self.alloc.free_seq(op[1])
            elif kind == "append":
                _, sid, n, tok0 = op
                slots, cow = self.alloc.append(sid, n)
                if len(cow) and on_cow is not None:
                    on_cow(cow)
                cows.extend((int(a), int(b)) for a, b in cow)
                if slots_out is not None:
                    slots_out[tok0:tok0 + n] = slots
            else:
                raise ValueError(kind)
        return cows

    def build_history(self) -> None:
        """Replay the history and write every history token into its slot."""
        wl = self.wl
        h0, h1 = wl.history_token_range()
        slots = np.full(max(h1, 1), -1, dtype=np.int64)
        written = [h0]

        def flush_then_copy(cow):
            # tokens appended so far must land before a copy reads their block
            end = int(np.max(np.nonzero(slots >= 0)[0])) + 1 if (slots >= 0).any() else h0
            self._write_rows(written[0], end, slots)
            written[0] = end
            self._copy_history_blocks(torch.as_tensor(np.asarray(cow, np.int32), device=self.device))

        self._replay(wl.history, on_cow=flush_then_copy, slots_out=slots)
        self._write_rows(written[0], h1, slots)
        self.history_slots = slots[h0:h1].copy()

    def _copy_history_blocks(self, pairs: torch.Tensor) -> None:
        pa_copy_blocks(self.k_pool, self.v_pool, self.pool, pairs)

    def _write_rows(self, a: int, b: int, slots: np.ndarray) -> None:
        if b <= a:
            return
        sl = torch.as_tensor(slots[a:b], device=self.device)
        pa_cache_write(self.k_tok[a:b], self.v_tok[a:b], sl, self.k_pool, self.v_pool, self.pool)

    def prepare_step(self, partition_size: Optional[int] = None) -> StepInputs:
        """Replay the step's allocator ops and stage every device input of the step."""
        wl = self.wl
        s0, s1 = wl.step_token_range()
        slots = np.full(max(s1, 1), -1, dtype=np.int64)
        cows = self._replay(wl.step, slots_out=slots)
        step_slots = slots[s0:s1].copy()
        dev = self.device
        cow = np.asarray(cows, np.int32).reshape(-1, 2)
        if self.validate:
            validate_slots(self.pool, step_slots)
            validate_pairs(self.pool, self.pool, cow)
        si = StepInputs(cow_pairs=torch.as_tensor(cow, device=dev),
                        slots=torch.as_tensor(step_slots, device=dev),
                        k_new=self.k_tok[s0:s1], v_new=self.v_tok[s0:s1],
                        host_slots=step_slots, host_cow=cow)
        part = wl.partition_size if partition_size is None else partition_size
        if wl.decode_seqs:
            lens = np.asarray(wl.decode_lens, np.int32)
            max_len = int(lens.max())
            tabs = [len(self.alloc.table(s)) for s in wl.decode_seqs]
            mb = max(max(tabs), -(-max_len // wl.block_size), 1)
            host_tabs = self.alloc.fill_tables(wl.decode_seqs, mb)
            if self.validate:
                validate_decode(self.pool, host_tabs, lens, max_len)
            si.dec_tables = torch.as_tensor(host_tabs, device=dev)
            si.dec_lens = torch.as_tensor(lens, device=dev)
            shared = leading_shared_blocks(host_tabs, np.asarray(lens), wl.block_size)
            si.dec_shared = torch.as_tensor(shared, device=dev) if shared.any() else None
            si.dec_q = wl.q_decode.to(dev)
            si.dec_out = torch.empty_like(si.dec_q)
            si.dec_max_len = max_len
            ws = pa_decode_workspace_size(len(wl.decode_seqs), wl.num_q_heads, wl.head_dim, max_len, part)
            si.dec_workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
            si.dec_partition = part
        if wl.prefill_seqs:
            prior = np.asarray(wl.prefill_prior, np.int32)
            chunk = np.asarray(wl.prefill_chunk, np.int32)
            tabs = [len(self.alloc.table(s)) for s in wl.prefill_seqs]
            mb = max(max(tabs), 1)
            pre_tabs = self.alloc.fill_tables(wl.prefill_seqs, mb)
            qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
            if self.validate:
                validate_prefill(self.pool, pre_tabs, qsl, prior, int(chunk.max()), int(wl.q_prefill.shape[0]))
            si.pre_tables = torch.as_tensor(pre_tabs, device=dev)
            si.pre_qsl = torch.as_tensor(qsl, device=dev)
            si.pre_prior = torch.as_tensor(prior, device=dev)
            si.pre_q = wl.q_prefill.to(dev)
            si.pre_out = torch.empty_like(si.pre_q)
            si.pre_max_chunk = int(chunk.max())
        return si

    # -- device step --------------------------------------------------------------------------
    def copy_step(self, si: StepInputs, stream=None) -> None:
        pa_copy_blocks(self.k_pool, self.v_pool, self.pool, si.cow_pairs, stream)

    def write_step(self, si: StepInputs, stream=None) -> None:
        pa_cache_write(si.k_new, si.v_new, si.slots, self.k_pool, self.v_pool, self.pool, stream)

    def use_cascade(self, si: StepInputs, width: int) -> None:
        """Decode the batch (requests x `width` branches) reading each request's shared blocks once.
        The shared part reads only full blocks that every branch still shares; when none of them is a
        copy destination or receives a token this step (always so: copies and writes go to a
        branch's last, private block), early_decode_step() runs it before the step's copies, so that
        it does not stream beside their write-back."""
        from .cascade import CascadeDecode
        wl = self.wl
        si.cascade = CascadeDecode(si.dec_tables.cpu().numpy(), np.asarray(wl.decode_lens, np.int32), wl.block_size,
                                   width, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, self.device)
        si.cascade_early = untouched_by_step(si.cascade.shared_blocks(), si.host_cow, si.host_slots, wl.block_size)
        si.cascade_shared_done = False

    def early_decode_step(self, si: StepInputs, stream=None) -> None:
        """The part of the decode that this step's copies and writes cannot change (the beam decode's
        shared blocks), issued first; nothing for other decodes."""
        if si.dec_q is None or getattr(si, "cascade", None) is None or not si.cascade_early:
            return
        si.cascade.run_shared(si.dec_q, self.k_pool, self.v_pool, self.pool, self.wl.scale, stream)
        si.cascade_shared_done = True

    def decode_step(self, si: StepInputs, stream=None, out: Optional[torch.Tensor] = None) -> None:
        if si.dec_q is None:
            return
        if getattr(si, "cascade", None) is not None:
            if not si.cascade_shared_done:
                si.cascade.run_shared(si.dec_q, self.k_pool, self.v_pool, self.pool, self.wl.scale, stream)
            si.cascade.run_tails(si.dec_q, self.k_pool, self.v_pool, self.pool, self.wl.scale,
                                 si.dec_out if out is None else out, stream)
            si.cascade_shared_done = False
            return
        pa_decode(si.dec_q, self.k_pool, self.v_pool, self.pool, si.dec_tables, si.dec_lens, self.wl.scale,
                  si.dec_out if out is None else out, si.dec_max_len, si.dec_partition, si.dec_workspace, stream,
                  shared_blocks=si.dec_shared)

    def prefill_step(self, si: StepInputs, stream=None) -> None:
        if si.pre_q is None:
            return
        pa_prefill_chunk(si.pre_q, self.k_pool, self.v_pool, self.pool, si.pre_tables, si.pre_qsl, si.pre_prior,
                         self.wl.scale, si.pre_max_chunk, si.pre_out, stream)

    def run_step(self, si: StepInputs, stream=None) -> None:
        """One step: CoW copies, then the new tokens' cache write, then prefill and decode (a beam
        decode's shared part first, before the copies)."""
        self.early_decode_step(si, stream)
        self.copy_step(si, stream)
        self.write_step(si, stream)
        self.prefill_step(si, stream)
        self.decode_step(si, stream)

    def finish(self) -> None:
        self._replay(self.wl.post)
