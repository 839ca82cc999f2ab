"""Decode of beam branches that share their prompt's blocks, reading each shared block once.

The branches of a request share every block of their prompt ([day28] §六 question 3), so a plain
decode reads each shared block once per branch.  Here one pa_decode_ex call reads the shared blocks
of each request once, with the W branches' queries of a KV head as its W query heads (the strides
pick them out of the batch's q, and write the outputs back to the branches' rows), a second call
reads each branch's private tail, and pa_merge_states combines the two results by their
log-sum-exps.  Tails of at most 32 tokens (a beam's tokens since the fork) take pa_decode_beam
instead: the shared part leaves its partial results in the workspace, and one tail launch folds
them into each branch's row as it reads the tail.  Needs one query head per KV head (the branches
then fill the group) and W in {2, 4, 8}; the batch is laid out as requests x W consecutive branches.
"""
import numpy as np
import torch

from ._lib import PA_BEAM_SHARED, PA_BEAM_TAILS, PA_F32, check, lib
from ._lib import _I32P
from .ops import pa_decode_beam, pa_decode_ex, pa_decode_workspace_size, pa_merge_states

TAIL_MERGE_MAX = 32     # longest tail pa_decode_beam takes


def plan_shared_blocks(tables: np.ndarray, lens: np.ndarray, block_size: int, width: int) -> np.ndarray:
    """Leading blocks shared by every branch of each request (host, pa_plan_shared_blocks)."""
    t = np.ascontiguousarray(tables, dtype=np.int32)
    l = np.ascontiguousarray(lens, dtype=np.int32)
    out = np.zeros(len(l) // width, dtype=np.int32)
    check(lib().pa_plan_shared_blocks(t.ctypes.data_as(_I32P), t.shape[1], l.ctypes.data_as(_I32P), len(l),
                                      int(block_size), int(width), out.ctypes.data_as(_I32P)))
    return out


def plan_beam_tails(tables: np.ndarray, lens: np.ndarray, block_size: int, width: int, shared: np.ndarray):
    """Each branch's private tail after its group's shared blocks (host, pa_plan_beam_tails): the
    tail table rows (int32 [num_seqs][longest tail in blocks, at least 1]) and lengths."""
    t = np.ascontiguousarray(tables, dtype=np.int32)
    l = np.ascontiguousarray(lens, dtype=np.int32)
    k = np.ascontiguousarray(shared, dtype=np.int32)
    tail_lens = np.zeros(len(l), dtype=np.int32)
    need = np.zeros(1, dtype=np.int32)
    args = (t.ctypes.data_as(_I32P), t.shape[1], l.ctypes.data_as(_I32P), len(l), int(block_size), int(width),
            k.ctypes.data_as(_I32P))
    check(lib().pa_plan_beam_tails(*args, None, 0, tail_lens.ctypes.data_as(_I32P), need.ctypes.data_as(_I32P)))
    nb = max(int(need[0]), 1)
    tt = np.zeros((len(l), nb), dtype=np.int32)
    check(lib().pa_plan_beam_tails(*args, tt.ctypes.data_as(_I32P), nb, tail_lens.ctypes.data_as(_I32P), None))
    return tt, tail_lens


class CascadeDecode:
    """Device inputs of a beam decode over fixed tables and lengths (rebuilt when they change)."""

    def __init__(self, tables: np.ndarray, lens: np.ndarray, block_size: int, width: int, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, device="cuda"):
        if num_q_heads != num_kv_heads:
            raise ValueError("the branches fill the query group: one query head per KV head")
        if width not in (2, 4, 8) or len(lens) % width:
            raise ValueError("width must be 2, 4 or 8 and divide the batch")
        dev = torch.device(device)
        b = block_size
        self.width, self.hq, self.d = width, num_q_heads, head_dim
        self.n = len(lens)
        self.groups = self.n // width
        k = plan_shared_blocks(tables, lens, b, width)
        self.shared_tokens = k.astype(np.int64) * b
        lens = np.asarray(lens, np.int64)
        # shared part: group g reads the table row of its first branch, k_g blocks
        self.tables = torch.as_tensor(np.ascontiguousarray(tables, dtype=np.int32), device=dev)
        self.tables_host = np.ascontiguousarray(tables, dtype=np.int32)
        self.block_size = b
        self.pre_lens = torch.as_tensor((k * b).astype(np.int32), device=dev)
        self.pre_max = int((k * b).max()) if self.groups else 0
        # private tails: each branch's blocks from its group's k on
        tt, tail_len = plan_beam_tails(tables, lens, b, width, k)
        self.tail_tables = torch.as_tensor(tt, device=dev)
        self.tail_lens = torch.as_tensor(tail_len.astype(np.int32), device=dev)
        self.tail_max = int(tail_len.max()) if self.n else 0
        self.o_pre = torch.empty((self.n, num_q_heads, head_dim), dtype=torch.float32, device=dev)
        self.o_tail = torch.empty_like(self.o_pre)
        self.l_pre = torch.empty((self.n, num_q_heads), dtype=torch.float32, device=dev)
        self.l_tail = torch.empty_like(self.l_pre)
        ws = max(pa_decode_workspace_size(self.groups, width * num_q_heads, head_dim, max(self.pre_max, 1), 0),
                 pa_decode_workspace_size(self.n, num_q_heads, head_dim, max(self.tail_max, 1), 0))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.max_blocks = int(tables.shape[1])

    def shared_blocks(self) -> np.ndarray:
        """Physical ids of the blocks the shared part reads (host)."""
        tabs = self.tables_host
        ids = [tabs[g * self.width, :int(k)] for g, k in enumerate(self.shared_tokens // self.block_size)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)

    def run(self, q: torch.Tensor, k_pool, v_pool, pool, scale: float, out: torch.Tensor, stream=None) -> None:
        self.run_shared(q, k_pool, v_pool, pool, scale, stream)
        self.run_tails(q, k_pool, v_pool, pool, scale, out, stream)

    def beam_call(self, pool) -> bool:
        """Whether pa_decode_beam serves this decode (tails of at most 32 tokens, bf16 or fp8 pool, head
        dim 128); else pa_decode_ex over each part and pa_merge_states."""
        return self.tail_max <= TAIL_MERGE_MAX and pool.dtype != PA_F32 and self.d == 128

    def _beam(self, q, k_pool, v_pool, pool, scale, out, phases, stream):
        pa_decode_beam(q, k_pool, v_pool, pool, self.tables, self.pre_lens, max(self.pre_max, 1), self.tail_tables,
                       self.tail_lens, self.tail_max, self.width, scale, self.workspace, out, phases, stream)

    def run_shared(self, q: torch.Tensor, k_pool, v_pool, pool, scale: float, stream=None) -> None:
        """The shared part: each request's shared blocks once, for all its branches (left as partial
        results in the workspace, or written to o_pre, l_pre)."""
        if self.beam_call(pool):
            self._beam(q, k_pool, v_pool, pool, scale, self.o_pre, PA_BEAM_SHARED, stream)
            return
        W, hq, d = self.width, self.hq, self.d
        # rows of group g: sequence stride W*hq*d; KV head stride d; branch (head in the group) stride hq*d
        strides = (W * hq * d, d, hq * d)
        pa_decode_ex(q, strides, self.groups, W * hq, k_pool, v_pool, pool, self.tables.data_ptr(),
                     W * self.max_blocks, self.pre_lens, scale, self.o_pre, strides, max(self.pre_max, 1),
                     self.l_pre, self.workspace, stream=stream)

    def run_tails(self, q: torch.Tensor, k_pool, v_pool, pool, scale: float, out: torch.Tensor, stream=None) -> None:
        """The private tails, merged with the shared part's result into out."""
        hq, d = self.hq, self.d
        if self.beam_call(pool):
            # short tails: their attention and the fold of the shared part's partial results, one launch
            self._beam(q, k_pool, v_pool, pool, scale, out, PA_BEAM_TAILS, stream)
            return
        pa_decode_ex(q, None, self.n, hq, k_pool, v_pool, pool, self.tail_tables.data_ptr(),
                     int(self.tail_tables.shape[1]), self.tail_lens, scale, self.o_tail, None,
                     max(self.tail_max, 1), self.l_tail, self.workspace, stream=stream)
        pa_merge_states(self.o_pre, self.l_pre, self.o_tail, self.l_tail, out, stream=stream)
