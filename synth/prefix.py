"""A batch of prompts behind one shared system prompt, for the prefix cache.

Shape from the pages: many requests start with the same long system prompt (a 1000-token one in
«GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术», §六 question 2, and the
prefix-caching switch of «第 7 章推理框架：vLLM 与 PagedAttention», 7.1), on the 40-head,
head_dim 128, bf16 model with 16-token blocks of the same chapter's 例 7-1.

Random draws, in fixed order (seed 4270 + 100 + size index):
  numpy PCG64  : system token ids -> user lengths -> user token ids -> physical free order
  torch Philox : system Q, K, V -> then Q, K, V of each user part in request order

A token's K/V rows depend only on its position in the prompt and the tokens before it, so every
request reuses the system prompt's rows, as a real model would produce them.  The last user part
belongs to a warm-up request that fills the cache before the batch arrives.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np
import torch

SEED = 4270 + 100


@dataclass
class PrefixBatch:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str               # pool storage ("bf16")
    act_dtype: str              # q, k, v rows and out ("bf16")
    scale: float                # fp32 softmax scale held in a python float
    num_blocks: int
    free_order: np.ndarray      # int32 [num_blocks]
    system_tokens: np.ndarray   # int32 [S]
    user_tokens: List[np.ndarray]
    q_sys: torch.Tensor         # [S, Hq, D]
    k_sys: torch.Tensor         # [S, Hkv, D]
    v_sys: torch.Tensor
    q_user: List[torch.Tensor]  # per request [u, Hq, D]
    k_user: List[torch.Tensor]
    v_user: List[torch.Tensor]

    @property
    def num_requests(self) -> int:
        """Requests of the batch (the warm-up request, the last user part, is not one of them)."""
        return len(self.user_tokens) - 1

    @property
    def warm(self) -> int:
        return len(self.user_tokens) - 1

    def prompt(self, r: int) -> np.ndarray:
        return np.concatenate([self.system_tokens, self.user_tokens[r]]).astype(np.int32)

    def prompt_len(self, r: int) -> int:
        return len(self.system_tokens) + len(self.user_tokens[r])

    def rows(self, r: int, a: int, b: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """(q, k, v) rows of prompt positions a .. b-1 of request r."""
        s = len(self.system_tokens)
        parts = []
        for src_sys, src_user in ((self.q_sys, self.q_user[r]), (self.k_sys, self.k_user[r]),
                                  (self.v_sys, self.v_user[r])):
            pieces = []
            if a < s:
                pieces.append(src_sys[a:min(b, s)])
            if b > s:
                pieces.append(src_user[max(a - s, 0):b - s])
            parts.append(torch.cat(pieces) if len(pieces) > 1 else pieces[0])
        return parts[0], parts[1], parts[2]


def _fp32(x: float) -> float:
    return float(np.float32(x))


def make_prefix_batch(size: str = "full", device="cpu") -> PrefixBatch:
    """full: 64 requests, a 1000-token system prompt, user parts U{32..512}, 40/40 heads.
    small: 6 requests, a 192-token system prompt (a whole number of blocks), user parts
    {0, 1, 15, 16, 17, 70} (prompts that end exactly on the prompt, on and around a block edge),
    8 query / 2 KV heads."""
    if size == "full":
        idx, hq, hkv, d, b, s_len = 0, 40, 40, 128, 16, 1000
        rng = np.random.default_rng(SEED + idx)
        sys_tok = rng.integers(0, 32000, size=s_len).astype(np.int32)
        ulens = [int(x) for x in rng.integers(32, 513, size=64 + 1)]
    elif size == "small":
        idx, hq, hkv, d, b, s_len = 1, 8, 2, 128, 16, 192
        rng = np.random.default_rng(SEED + idx)
        sys_tok = rng.integers(0, 32000, size=s_len).astype(np.int32)
        ulens = [0, 1, 15, 16, 17, 70, 40]
    else:
        raise ValueError(size)
    user_tok = [rng.integers(0, 32000, size=u).astype(np.int32) for u in ulens]
    need = sum(-(-(s_len + u) // b) for u in ulens)
    num_blocks = int(math.ceil(1.25 * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED + idx)

    def draw(n, h):
        return torch.randn((n, h, d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)

    q_sys, k_sys, v_sys = draw(s_len, hq), draw(s_len, hkv), draw(s_len, hkv)
    q_u, k_u, v_u = [], [], []
    for u in ulens:
        q_u.append(draw(u, hq))
        k_u.append(draw(u, hkv))
        v_u.append(draw(u, hkv))
    return PrefixBatch(name=f"prefix_cache_bf16/{size}", num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                       block_size=b, kv_dtype="bf16", act_dtype="bf16", scale=_fp32(1.0 / math.sqrt(d)),
                       num_blocks=num_blocks, free_order=free_order, system_tokens=sys_tok,
                       user_tokens=user_tok, q_sys=q_sys, k_sys=k_sys, v_sys=v_sys, q_user=q_u, k_user=k_u,
                       v_user=v_u)
