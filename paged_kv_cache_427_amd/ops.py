"""Python binding of libpa's device calls, with the names of the C ABI (include/pa.h).

Argument marshalling only: torch tensors supply device memory and the current stream; every
computation runs in the library's HIP kernels.  There is no fallback: without libpa.so, or without
a GPU, these calls raise.
"""
import ctypes
from typing import Optional

import numpy as np
import torch

from ._lib import PA_BF16, PA_F32, PA_FP8_E4M3, PoolDesc, check, lib, _I32P, _I64P

_TORCH_TO_PA = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3,
                torch.float8_e4m3fn: PA_FP8_E4M3}


def pa_dtype(t: torch.Tensor) -> int:
    try:
        return _TORCH_TO_PA[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def make_pool_desc(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: int,
                   k_scale: float = 1.0, v_scale: float = 1.0) -> PoolDesc:
    return PoolDesc(num_blocks, block_size, num_kv_heads, head_dim, dtype, k_scale, v_scale)


def pool_torch_dtype(dtype: int) -> torch.dtype:
    return {PA_F32: torch.float32, PA_BF16: torch.bfloat16, PA_FP8_E4M3: torch.uint8}[dtype]


def pa_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_pool: torch.Tensor,
                   v_pool: torch.Tensor, pool: PoolDesc, stream=None) -> None:
    """Scatter rows k, v [T, Hkv, D] into their slots (int64 [T]; negative = skip)."""
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    n = int(slot_mapping.shape[0])
    if k.shape != v.shape or (n and k.shape[0] != n):
        raise ValueError("k, v and slot_mapping disagree in length")
    if n == 0:
        return
    check(lib().pa_cache_write(_dev(k, "k"), _dev(v, "v"), pa_dtype(k), n, _dev(slot_mapping, "slot_mapping"),
                               _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), ctypes.byref(pool),
                               _stream(stream)))


def pa_copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, pool: PoolDesc, pairs: torch.Tensor,
                   stream=None) -> None:
    """Copy whole blocks src -> dst for each row of pairs (int32 [n, 2])."""
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    n = int(pairs.shape[0]) if pairs.numel() else 0
    if n == 0:
        return
    check(lib().pa_copy_blocks(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), ctypes.byref(pool),
                               _dev(pairs, "pairs"), n, _stream(stream)))


def pa_copy_blocks_layers(k_pools: torch.Tensor, v_pools: torch.Tensor, pool: PoolDesc, pairs: torch.Tensor,
                          stream=None) -> None:
    """Copy-on-write copies in every layer: k_pools, v_pools are [layers, num_blocks, ...] tensors."""
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    n = int(pairs.shape[0]) if pairs.numel() else 0
    if n == 0:
        return
    if k_pools.shape[0] != v_pools.shape[0] or k_pools.stride(0) != v_pools.stride(0):
        raise ValueError("k_pools and v_pools must have the same layers and layer stride")
    stride = k_pools.stride(0) * k_pools.element_size()
    check(lib().pa_copy_blocks_layers(_dev(k_pools, "k_pools"), _dev(v_pools, "v_pools"), stride,
                                      int(k_pools.shape[0]), ctypes.byref(pool), _dev(pairs, "pairs"), n,
                                      _stream(stream)))


def pa_swap_blocks(dst_k_pool: torch.Tensor, dst_v_pool: torch.Tensor, dst_pool: PoolDesc,
                   src_k_pool: torch.Tensor, src_v_pool: torch.Tensor, src_pool: PoolDesc, pairs: torch.Tensor,
                   stream=None) -> None:
    """Copy whole blocks between two pools (device memory or pinned host memory): block pairs[i, 1]
    of the destination receives block pairs[i, 0] of the source."""
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    n = int(pairs.shape[0]) if pairs.numel() else 0
    if n == 0:
        return
    for t, name in ((dst_k_pool, "dst_k_pool"), (dst_v_pool, "dst_v_pool"), (src_k_pool, "src_k_pool"),
                    (src_v_pool, "src_v_pool"), (pairs, "pairs")):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a device tensor or pinned host memory")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    check(lib().pa_swap_blocks(dst_k_pool.data_ptr(), dst_v_pool.data_ptr(), ctypes.byref(dst_pool),
                               src_k_pool.data_ptr(), src_v_pool.data_ptr(), ctypes.byref(src_pool),
                               pairs.data_ptr(), n, _stream(stream)))


def pa_decode_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int, max_context_len: int,
                             partition_size: int = 0) -> int:
    out = ctypes.c_size_t(0)
    check(lib().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, partition_size,
                                         ctypes.byref(out)))
    return int(out.value)


def _shared(shared_blocks: Optional[torch.Tensor], num_seqs: int):
    if shared_blocks is None:
        return None
    if shared_blocks.dtype != torch.int32 or shared_blocks.numel() < num_seqs:
        raise TypeError("shared_blocks must be int32 with one entry per sequence")
    return _dev(shared_blocks, "shared_blocks")


def pa_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, pool: PoolDesc,
              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, out: torch.Tensor,
              max_context_len: int, partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
              stream=None, shared_blocks: Optional[torch.Tensor] = None) -> None:
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over each sequence's paged context.
    `shared_blocks` (int32 [num_seqs], optional): leading table entries of each sequence that other
    sequences of the call also read (a cache-policy hint of pa_decode_ex; engine.leading_shared_blocks
    computes it).  Without it the call is pa_decode; with it, pa_decode_ex with dense strides."""
    num_seqs, num_q_heads, head_dim = q.shape
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    need = pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if shared_blocks is None:
        check(lib().pa_decode(_dev(q, "q"), pa_dtype(q), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                              ctypes.byref(pool), _dev(block_tables, "block_tables"), int(block_tables.shape[1]),
                              _dev(context_lens, "context_lens"), num_seqs, num_q_heads, float(scale),
                              partition_size, int(max_context_len), ws_ptr, ws_bytes, _dev(out, "out"),
                              pa_dtype(out), _stream(stream)))
        return
    check(lib().pa_decode_ex(_dev(q, "q"), pa_dtype(q), None, _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                             ctypes.byref(pool), _dev(block_tables, "block_tables"), int(block_tables.shape[1]),
                             _dev(context_lens, "context_lens"), num_seqs, num_q_heads, float(scale),
                             partition_size, int(max_context_len), ws_ptr, ws_bytes, _dev(out, "out"),
                             pa_dtype(out), None, None, _shared(shared_blocks, num_seqs), _stream(stream)))


def pa_decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, pool: PoolDesc,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, out: torch.Tensor,
                      max_context_len: int, partition_size: int = 0, stream=None,
                      shared_blocks: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None) -> None:
    """pa_decode that allocates nothing: the library's static per-GPU workspace replaces the caller's
    (calls on one GPU must not overlap).  Dense q and out; optional log-sum-exp output."""
    num_seqs, num_q_heads, _ = q.shape
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    check(lib().pa_decode_noalloc(_dev(q, "q"), pa_dtype(q), None, _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                  ctypes.byref(pool), _dev(block_tables, "block_tables"), int(block_tables.shape[1]),
                                  _dev(context_lens, "context_lens"), num_seqs, num_q_heads, float(scale),
                                  partition_size, int(max_context_len), _dev(out, "out"), pa_dtype(out), None,
                                  None if lse is None else _dev(lse, "lse"), _shared(shared_blocks, num_seqs),
                                  _stream(stream)))


def pa_decode_ex(q_base: torch.Tensor, q_strides, num_seqs: int, num_q_heads: int, k_pool: torch.Tensor,
                 v_pool: torch.Tensor, pool: PoolDesc, tables_ptr: int, max_blocks_per_seq: int,
                 context_lens: torch.Tensor, scale: float, out_base: torch.Tensor, out_strides, max_context_len: int,
                 lse: Optional[torch.Tensor], workspace: torch.Tensor, partition_size: int = 0, stream=None,
                 shared_blocks: Optional[torch.Tensor] = None) -> None:
    """pa_decode over strided q and out rows (element strides for sequence, KV head, head in the
    group; None = dense) with an optional log-sum-exp output.  `tables_ptr` is a device address
    (a table row stride of max_blocks_per_seq entries may skip rows of a larger table)."""
    qs = None if q_strides is None else (ctypes.c_int64 * 3)(*[int(x) for x in q_strides])
    os_ = None if out_strides is None else (ctypes.c_int64 * 3)(*[int(x) for x in out_strides])
    if context_lens.dtype != torch.int32:
        raise TypeError("context_lens must be int32")
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib().pa_decode_ex(_dev(q_base, "q"), pa_dtype(q_base), qs, _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                             ctypes.byref(pool), int(tables_ptr), int(max_blocks_per_seq),
                             _dev(context_lens, "context_lens"), int(num_seqs), int(num_q_heads), float(scale),
                             int(partition_size), int(max_context_len), _dev(workspace, "workspace"), ws_bytes,
                             _dev(out_base, "out"), pa_dtype(out_base), os_,
                             None if lse is None else _dev(lse, "lse"), _shared(shared_blocks, num_seqs),
                             _stream(stream)))


def pa_merge_states(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
                    out: torch.Tensor, lse_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """Combine two results of the same rows over disjoint key sets (float [rows..., head_dim] each,
    their log-sum-exps float [rows...]) into out (float or bf16)."""
    head_dim = int(o_a.shape[-1])
    rows = o_a.numel() // head_dim
    for t, name in ((o_a, "o_a"), (o_b, "o_b"), (lse_a, "lse_a"), (lse_b, "lse_b")):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if o_b.numel() != o_a.numel() or out.numel() != o_a.numel() or lse_a.numel() != rows or lse_b.numel() != rows:
        raise ValueError("shapes disagree")
    check(lib().pa_merge_states(_dev(o_a, "o_a"), _dev(lse_a, "lse_a"), _dev(o_b, "o_b"), _dev(lse_b, "lse_b"),
                                rows, head_dim, _dev(out, "out"), pa_dtype(out),
                                None if lse_out is None else _dev(lse_out, "lse_out"), _stream(stream)))


def pa_decode_tail_merge(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, pool: PoolDesc,
                         tail_tables: torch.Tensor, tail_lens: torch.Tensor, scale: float, max_tail_len: int,
                         o_prev: torch.Tensor, lse_prev: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out[s, h] = the merge of (o_prev, lse_prev)[s, h] with attention over sequence s's tail of at
    most 32 keys (tail_tables int32 [num_seqs, max_blocks], tail_lens int32 [num_seqs]); q bf16
    [num_seqs, num_q_heads, 128], o_prev float [same], lse_prev float [num_seqs, num_q_heads]."""
    num_seqs, num_q_heads, head_dim = q.shape
    if tail_tables.dtype != torch.int32 or tail_lens.dtype != torch.int32:
        raise TypeError("tail_tables and tail_lens must be int32")
    if o_prev.dtype != torch.float32 or lse_prev.dtype != torch.float32:
        raise TypeError("o_prev and lse_prev must be float32")
    if o_prev.numel() != q.numel() or out.numel() != q.numel() or lse_prev.numel() != num_seqs * num_q_heads:
        raise ValueError("shapes disagree")
    check(lib().pa_decode_tail_merge(_dev(q, "q"), pa_dtype(q), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                     ctypes.byref(pool), _dev(tail_tables, "tail_tables"), int(tail_tables.shape[1]),
                                     _dev(tail_lens, "tail_lens"), int(num_seqs), int(num_q_heads), float(scale),
                                     int(max_tail_len), _dev(o_prev, "o_prev"), _dev(lse_prev, "lse_prev"),
                                     _dev(out, "out"), pa_dtype(out), _stream(stream)))


def pa_decode_beam(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, pool: PoolDesc,
                   tables: torch.Tensor, shared_lens: torch.Tensor, max_shared_len: int, tail_tables: torch.Tensor,
                   tail_lens: torch.Tensor, max_tail_len: int, width: int, scale: float, workspace: torch.Tensor,
                   out: torch.Tensor, phases: int = 3, stream=None) -> None:
    """Beam decode of q bf16 [num_seqs, H, 128] (groups of `width` consecutive branches): each group's
    shared blocks (tables int32 [num_seqs, max_blocks], the first member's row; shared_lens int32
    [num_seqs / width]) once for all its branches, then each branch's tail of at most 32 keys
    (tail_tables int32 [num_seqs, tail_max_blocks], tail_lens int32 [num_seqs]) folded in, into out.
    phases: 1 the shared part only, 2 the tails (after a phase-1 call on the same workspace), 3 both."""
    num_seqs, heads, head_dim = q.shape
    for name, t in (("tables", tables), ("shared_lens", shared_lens), ("tail_tables", tail_tables),
                    ("tail_lens", tail_lens)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    check(lib().pa_decode_beam(_dev(q, "q"), pa_dtype(q), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                               ctypes.byref(pool), _dev(tables, "tables"), int(tables.shape[1]),
                               _dev(shared_lens, "shared_lens"), int(max_shared_len), _dev(tail_tables, "tail_tables"),
                               int(tail_tables.shape[1]), _dev(tail_lens, "tail_lens"), int(max_tail_len),
                               int(num_seqs), int(width), float(scale), _dev(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(), _dev(out, "out"), pa_dtype(out),
                               int(phases), _stream(stream)))


def pa_prefill_chunk(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, pool: PoolDesc,
                     block_tables: torch.Tensor, query_start_loc: torch.Tensor,
                     prior_context_lens: torch.Tensor, scale: float, max_chunk_len: int, out: torch.Tensor,
                     stream=None) -> None:
    """Causal attention of each sequence's chunk of queries over its paged context plus the chunk."""
    num_seqs = int(prior_context_lens.shape[0])
    check(lib().pa_prefill_chunk(_dev(q, "q"), pa_dtype(q), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                 ctypes.byref(pool), _dev(block_tables, "block_tables"),
                                 int(block_tables.shape[1]), _dev(query_start_loc, "query_start_loc"),
                                 _dev(prior_context_lens, "prior_context_lens"), num_seqs, int(q.shape[1]),
                                 float(scale), int(max_chunk_len), _dev(out, "out"), pa_dtype(out),
                                 _stream(stream)))


def pa_fp8_decode_table(out: torch.Tensor, stream=None) -> None:
    """out (float32 [256], device) <- the device's decoding of every e4m3 code."""
    check(lib().pa_fp8_decode_table(_dev(out, "out"), _stream(stream)))


def pa_hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Streams buf (a contiguous device tensor, a multiple of 16 bytes) once with 16-byte loads;
    sink is a device tensor of at least 4 bytes (a measurement aid: time it to read the device's
    streaming read bandwidth)."""
    check(lib().pa_hbm_read_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink"),
                                  _stream(stream)))


# ---- host checks of device-resident inputs (pa_validate_*): numpy arrays, before they are sent ----

def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def validate_decode(pool: PoolDesc, tables, lens, max_context_len: int) -> None:
    """Raise PaError unless every table entry a sequence uses lies in the pool and every length is in
    [0, max_context_len] and fits its row."""
    t, l = _i32(tables), _i32(lens)
    check(lib().pa_validate_decode(ctypes.byref(pool), t.ctypes.data_as(_I32P), int(t.shape[1]),
                                   l.ctypes.data_as(_I32P), len(l), int(max_context_len)))


def validate_prefill(pool: PoolDesc, tables, query_start_loc, prior_lens, max_chunk_len: int, total_q: int) -> None:
    """Raise PaError unless the chunks are ordered, bounded by max_chunk_len and total_q, and every table
    entry of each sequence's prior context plus chunk lies in the pool."""
    t, q, p = _i32(tables), _i32(query_start_loc), _i32(prior_lens)
    check(lib().pa_validate_prefill(ctypes.byref(pool), t.ctypes.data_as(_I32P), int(t.shape[1]),
                                    q.ctypes.data_as(_I32P), p.ctypes.data_as(_I32P), len(p), int(max_chunk_len),
                                    int(total_q)))


def validate_slots(pool: PoolDesc, slots) -> None:
    """Raise PaError unless every non-negative slot lies in the pool and no two tokens share one."""
    s = np.ascontiguousarray(slots, dtype=np.int64)
    check(lib().pa_validate_slots(ctypes.byref(pool), s.ctypes.data_as(_I64P), len(s)))


def validate_pairs(src_pool: PoolDesc, dst_pool: PoolDesc, pairs, in_place: bool = True) -> None:
    """Raise PaError unless every (source, destination) pair lies in its pool, destinations are distinct
    and, for copies within one pool, no destination is also a source."""
    pr = _i32(np.asarray(pairs).reshape(-1, 2))
    check(lib().pa_validate_pairs(ctypes.byref(src_pool), ctypes.byref(dst_pool), pr.ctypes.data_as(_I32P), len(pr),
                                  1 if in_place else 0))
