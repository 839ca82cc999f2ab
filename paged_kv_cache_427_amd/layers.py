"""A many-layer decode step: one block table and one allocator for every layer, per-layer pools in
one [layers, num_blocks, ...] tensor, and the step's device calls replayed as a HIP graph.

One block id names the same block in every layer ([ch7] 7.1: the KV cache holds each layer's K and
V, and the per-token size counts every layer), so the host work of a step (slots, copy-on-write
pairs, tables) is done once; the device work is one copy launch for all layers
(pa_copy_blocks_layers), then, per layer, the cache write of the step's tokens and the decode.
A real model computes each layer's q, k and v between these calls; here they are inputs.
"""
from typing import Callable, List, Optional

import numpy as np
import torch

from .engine import PagedKVEngine, StepInputs, _CODE_TORCH, _VIEW, _signed
from .ops import pa_cache_write, pa_copy_blocks_layers, pa_decode


class LayeredEngine(PagedKVEngine):
    """`num_layers` layers of the workload `wl`; layer l's K, V and q rows are layer_rows(rows, l)."""

    def __init__(self, wl, num_layers: int, layer_rows: Callable[[torch.Tensor, int], torch.Tensor],
                 device: str = "cuda", poison: Optional[int] = None):
        self.num_layers = int(num_layers)
        self.layer_rows = layer_rows
        super().__init__(wl, device=device, poison=poison, allocate_pools=False)
        bits = {"f32": 32, "bf16": 16, "fp8": 8}[wl.kv_dtype]
        fill = 0 if poison is None else (_signed(poison, bits) if wl.kv_dtype != "fp8" else poison)
        k_shape = (self.num_layers, wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
        v_shape = (self.num_layers, wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.block_size)
        code = _CODE_TORCH[wl.kv_dtype]
        self.k_layers = torch.full(k_shape, fill, dtype=code, device=self.device).view(_VIEW[wl.kv_dtype])
        self.v_layers = torch.full(v_shape, fill, dtype=code, device=self.device).view(_VIEW[wl.kv_dtype])
        self.k_pool, self.v_pool = self.k_layers[0], self.v_layers[0]

    def _write_rows(self, a: int, b: int, slots: np.ndarray) -> None:
        if b <= a:
            return
        sl = torch.as_tensor(slots[a:b], device=self.device)
        for l in range(self.num_layers):
            pa_cache_write(self.layer_rows(self.k_tok[a:b], l), self.layer_rows(self.v_tok[a:b], l), sl,
                           self.k_layers[l], self.v_layers[l], self.pool)

    def _copy_history_blocks(self, pairs: torch.Tensor) -> None:
        pa_copy_blocks_layers(self.k_layers, self.v_layers, self.pool, pairs)

    def prepare_layers(self, si: StepInputs) -> None:
        """Per-layer step rows and queries, and one output buffer per layer."""
        L = self.num_layers
        si.k_layers_new = torch.stack([self.layer_rows(si.k_new, l) for l in range(L)])
        si.v_layers_new = torch.stack([self.layer_rows(si.v_new, l) for l in range(L)])
        if si.dec_q is not None:
            si.q_layers = torch.stack([self.layer_rows(si.dec_q, l) for l in range(L)])
            si.out_layers = torch.empty_like(si.q_layers)

    def run_layers(self, si: StepInputs, stream=None) -> None:
        """One step of every layer: the copies of all layers, then per layer the write and the decode."""
        pa_copy_blocks_layers(self.k_layers, self.v_layers, self.pool, si.cow_pairs, stream)
        for l in range(self.num_layers):
            pa_cache_write(si.k_layers_new[l], si.v_layers_new[l], si.slots, self.k_layers[l], self.v_layers[l],
                           self.pool, stream)
            if si.dec_q is not None:
                pa_decode(si.q_layers[l], self.k_layers[l], self.v_layers[l], self.pool, si.dec_tables, si.dec_lens,
                          self.wl.scale, si.out_layers[l], si.dec_max_len, si.dec_partition, si.dec_workspace,
                          stream)

    def capture(self, si: StepInputs) -> torch.cuda.CUDAGraph:
        """The step of every layer as one HIP graph (all buffers are fixed; nothing allocates)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run_layers(si)            # warm-up outside the graph, on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            self.run_layers(si)
        return g


def layer_outputs(si: StepInputs) -> List[torch.Tensor]:
    return [si.out_layers[l] for l in range(si.out_layers.shape[0])]
