"""Runs a synthetic workload (package `synth`) through the oracle.

`run_paged` builds the whole pool (small workloads): it replays the operation script on
RefAllocator, writes every token into its slot, applies the step's copy-on-write copies and
cache-write, and computes decode and prefill outputs by gathering through the block tables.

`dense_decode` / `dense_prefill` compute chosen outputs from the logical (contiguous) token rows
with no pool at all; they serve large workloads, where only sampled outputs are checked.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from synth import poison_code

from .allocator import RefAllocator
from .attention import attend, ref_decode, ref_decode_split, ref_prefill
from .cache import gather_seq, pool_shape, ref_cache_write, ref_copy_blocks
from .codecs import bf16_bits_to_f64, decode_pool, e4m3_decode, e4m3_quantise, f32_bits_to_f64
from .logical import LogicalSeqs

_CODE_DTYPE = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU/GPU tensor as a NumPy array (uint32 / uint16 / uint8)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype in (torch.uint8, torch.int8):
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def act_values(bits: np.ndarray, act_dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(bits) if act_dtype == "bf16" else f32_bits_to_f64(bits)


@dataclass
class OracleResult:
    k_pool: np.ndarray
    v_pool: np.ndarray
    history_slots: np.ndarray            # [history tokens] int64, in token-row order
    step_slots: np.ndarray               # [step tokens] int64, in token-row order
    step_cow: np.ndarray                 # [n, 2] int32
    k_pool_before_step: np.ndarray = None
    v_pool_before_step: np.ndarray = None
    tables: Dict[int, List[int]] = field(default_factory=dict)
    decode_out: Optional[np.ndarray] = None
    decode_out_split: Optional[np.ndarray] = None
    prefill_out: Optional[np.ndarray] = None
    free_list_after: List[int] = field(default_factory=list)


def _replay(alloc: RefAllocator, logical: LogicalSeqs, ops: Sequence[Tuple], slots: Dict[int, int],
            cow: List[Tuple[int, int]]) -> None:
    for op in ops:
        logical.apply(op)
        kind = op[0]
        if kind == "add":
            alloc.add_seq(op[1])
        elif kind == "fork":
            alloc.fork(op[1], op[2])
        elif kind == "free":
            alloc.free_seq(op[1])
        elif kind == "append":
            _, sid, n, tok0 = op
            s, c = alloc.append(sid, n)
            for i, x in enumerate(s):
                slots[tok0 + i] = x
            cow.extend(c)


def run_paged(wl, split: Optional[int] = None) -> OracleResult:
    """Whole-pool oracle of a (small) workload.  `split`: also compute decode partition by partition."""
    b, hkv, d = wl.block_size, wl.num_kv_heads, wl.head_dim
    code_dt = _CODE_DTYPE[wl.kv_dtype]
    poison = poison_code(wl.kv_dtype)   # input recipe: the initial content of every pool slot
    k_pool = np.full(pool_shape(wl.num_blocks, hkv, b, d, "k"), poison, dtype=code_dt)
    v_pool = np.full(pool_shape(wl.num_blocks, hkv, b, d, "v"), poison, dtype=code_dt)
    k_bits = tensor_bits(wl.k_tok)
    v_bits = tensor_bits(wl.v_tok)
    alloc = RefAllocator(wl.num_blocks, b, wl.free_order)
    logical = LogicalSeqs()

    # history: every append writes its tokens after its own copy-on-write copies
    h_slots: Dict[int, int] = {}
    for op in wl.history:
        cow: List[Tuple[int, int]] = []
        _replay(alloc, logical, [op], h_slots, cow)
        ref_copy_blocks(k_pool, cow)
        ref_copy_blocks(v_pool, cow)
        if op[0] == "append":
            rows = list(range(op[3], op[3] + op[2]))
            sl = [h_slots[r] for r in rows]
            ref_cache_write(k_pool, k_bits[rows], sl, wl.kv_dtype, wl.act_dtype, wl.k_scale)
            ref_cache_write(v_pool, v_bits[rows], sl, wl.kv_dtype, wl.act_dtype, wl.v_scale, which="v")
    h0, h1 = wl.history_token_range()
    history_slots = np.array([h_slots[r] for r in range(h0, h1)], dtype=np.int64)

    k_before, v_before = k_pool.copy(), v_pool.copy()
    # step: allocator ops, then the copy-on-write copies, then one cache-write of every step token
    s_slots: Dict[int, int] = {}
    s_cow: List[Tuple[int, int]] = []
    _replay(alloc, logical, wl.step, s_slots, s_cow)
    ref_copy_blocks(k_pool, s_cow)
    ref_copy_blocks(v_pool, s_cow)
    s0, s1 = wl.step_token_range()
    step_slots = np.array([s_slots[r] for r in range(s0, s1)], dtype=np.int64)
    ref_cache_write(k_pool, k_bits[s0:s1], step_slots, wl.kv_dtype, wl.act_dtype, wl.k_scale)
    ref_cache_write(v_pool, v_bits[s0:s1], step_slots, wl.kv_dtype, wl.act_dtype, wl.v_scale, which="v")

    res = OracleResult(k_pool=k_pool, v_pool=v_pool, history_slots=history_slots, step_slots=step_slots,
                       step_cow=np.array(s_cow, dtype=np.int32).reshape(-1, 2),
                       k_pool_before_step=k_before, v_pool_before_step=v_before)
    kv_k = decode_pool(k_pool, wl.kv_dtype, wl.k_scale)
    kv_v = decode_pool(v_pool, wl.kv_dtype, wl.v_scale)
    for sid in list(wl.decode_seqs) + list(wl.prefill_seqs):
        res.tables[sid] = alloc.table(sid)

    if wl.decode_seqs:
        q = act_values(tensor_bits(wl.q_decode), wl.act_dtype)
        kv = [(gather_seq(kv_k, alloc.table(sid), int(L)), gather_seq(kv_v, alloc.table(sid), int(L), "v"))
              for sid, L in zip(wl.decode_seqs, wl.decode_lens)]
        res.decode_out = ref_decode(q, kv, wl.scale)
        if split:
            res.decode_out_split = ref_decode_split(q, kv, wl.scale, split)
    if wl.prefill_seqs:
        q = act_values(tensor_bits(wl.q_prefill), wl.act_dtype)
        qsl = np.concatenate([[0], np.cumsum(wl.prefill_chunk)])
        kv = []
        for sid, p, c in zip(wl.prefill_seqs, wl.prefill_prior, wl.prefill_chunk):
            n = int(p) + int(c)
            kv.append((gather_seq(kv_k, alloc.table(sid), n), gather_seq(kv_v, alloc.table(sid), n, "v")))
        res.prefill_out = ref_prefill(q, qsl, wl.prefill_prior, kv, wl.scale)

    for op in wl.post:
        _replay(alloc, logical, [op], {}, [])
    alloc.check_invariants()
    res.free_list_after = alloc.free_list()
    return res


# ---- dense (pool-free) reference for sampled outputs -------------------------------------------

def _fp8_stored(vals_f32: np.ndarray, scale: float) -> np.ndarray:
    """The value an fp8 pool holds for fp32 inputs: decode(quantise(x)) * scale."""
    return e4m3_decode(e4m3_quantise(vals_f32, scale)) * float(np.float32(scale))


_BF16_FP8_TABLES: Dict[float, np.ndarray] = {}


def bf16_fp8_table(scale: float) -> np.ndarray:
    """_fp8_stored evaluated once for each of the 65536 bf16 bit patterns: a bf16 input's stored fp8
    value depends on its 16 bits alone, so the table gives, by indexing, exactly what the per-element
    evaluation gives (a pin test compares the two)."""
    key = float(np.float32(scale))
    if key not in _BF16_FP8_TABLES:
        every = bf16_bits_to_f64(np.arange(65536, dtype=np.uint32).astype(np.uint16)).astype(np.float32)
        _BF16_FP8_TABLES[key] = _fp8_stored(every, scale)
    return _BF16_FP8_TABLES[key]


def _stored_values(rows_bits: np.ndarray, wl, which: str) -> np.ndarray:
    """Values the pool holds for these token rows: the activation value, or its fp8 round trip."""
    if wl.kv_dtype == "fp8":
        scale = wl.k_scale if which == "k" else wl.v_scale
        if wl.act_dtype == "bf16":
            return bf16_fp8_table(scale)[np.asarray(rows_bits, dtype=np.uint16)]
        return _fp8_stored(act_values(rows_bits, wl.act_dtype).astype(np.float32), scale)
    return act_values(rows_bits, wl.act_dtype)


def logical_view(wl) -> LogicalSeqs:
    lg = LogicalSeqs()
    lg.apply_all(wl.history)
    lg.apply_all(wl.step)
    return lg


def dense_decode(wl, batch_index: int, heads: Sequence[int], logical: LogicalSeqs = None) -> np.ndarray:
    """Decode outputs [len(heads), D] of one batch entry, from contiguous token rows."""
    lg = logical or logical_view(wl)
    sid = wl.decode_seqs[batch_index]
    length = int(wl.decode_lens[batch_index])
    rows = lg.token_rows(sid, length)
    idx = torch.as_tensor(rows, dtype=torch.long, device=wl.k_tok.device)
    k = _stored_values(tensor_bits(wl.k_tok.index_select(0, idx)), wl, "k")
    v = _stored_values(tensor_bits(wl.v_tok.index_select(0, idx)), wl, "v")
    q = act_values(tensor_bits(wl.q_decode[batch_index]), wl.act_dtype)
    group = wl.group
    return np.stack([attend(q[h], k[:, h // group], v[:, h // group], wl.scale) for h in heads])


def dense_prefill(wl, seq_index: int, query_rows: Sequence[int], heads: Sequence[int],
                  logical: LogicalSeqs = None) -> np.ndarray:
    """Prefill outputs [len(query_rows), len(heads), D] of chunk queries (indices within the chunk)."""
    lg = logical or logical_view(wl)
    sid = wl.prefill_seqs[seq_index]
    p0 = int(wl.prefill_prior[seq_index])
    c = int(wl.prefill_chunk[seq_index])
    rows = lg.token_rows(sid, p0 + c)
    idx = torch.as_tensor(rows, dtype=torch.long, device=wl.k_tok.device)
    k = _stored_values(tensor_bits(wl.k_tok.index_select(0, idx)), wl, "k")
    v = _stored_values(tensor_bits(wl.v_tok.index_select(0, idx)), wl, "v")
    start = int(np.sum(wl.prefill_chunk[:seq_index]))
    q = act_values(tensor_bits(wl.q_prefill[start:start + c]), wl.act_dtype)
    group = wl.group
    out = np.zeros((len(query_rows), len(heads), wl.head_dim))
    for a, i in enumerate(query_rows):
        vis = p0 + int(i) + 1
        for bi, h in enumerate(heads):
            out[a, bi] = attend(q[i, h], k[:vis, h // group], v[:vis, h // group], wl.scale)
    return out
