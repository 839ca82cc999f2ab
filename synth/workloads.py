"""Workload generators: five paged-attention configurations, each at a full and a small size.

Shapes follow the pages' examples: a 40-KV-head, head_dim 128, bf16 model with 16-token blocks
(«第 7 章推理框架：vLLM 与 PagedAttention», 7.2 例 7-1), a Llama-7B-shaped fp16/bf16 model
(«GPU 学习日报 Day 28：vLLM 与 PagedAttention：GPU Memory 管理的艺术», §一), shared
system-prompt prefixes and copy-on-write (same page, §四 4.2 and §六), chunked prefill
mixed with decode (same page, FAQ Q4) and fp8_e4m3 KV (例 7-1's chapter, 「vLLM 关键参数速记」).

Random draws, in fixed order per configuration k (seed 4270 + k):
  numpy PCG64  : lengths -> physical free order -> outlier mask
  torch Philox : Q -> K -> V   (on the requested device; CPU and GPU streams differ)

Operation script entries (tuples):
  ("add", sid)                   new empty sequence
  ("append", sid, n, tok0)       append n tokens whose K/V are rows tok0 .. tok0+n-1 of k_tok/v_tok
  ("fork", parent, child)        child shares every block of parent
  ("free", sid)                  sequence finished
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

CONFIG_NAMES = ("tiny_fp32", "llama7b_bf16", "shared_prefix_bf16", "gqa_long_bf16", "mixed_fp8",
                "fork_storm_bf16")
SEED_BASE = 4270

_ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
# Unused pool slots hold a NaN pattern so that a stray read shows up as NaN in an output.
_POISON = {"f32": 0x7FC00000, "bf16": 0x7FC0, "fp8": 0x7F}


def elem_bytes(dtype: str) -> int:
    return _ELEM_BYTES[dtype]


def poison_code(dtype: str) -> int:
    return _POISON[dtype]


@dataclass
class Workload:
    name: str
    size: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str          # "f32" | "bf16" | "fp8"   (pool storage)
    act_dtype: str         # "f32" | "bf16"           (q, new k/v rows, out)
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks], the allocator's initial FIFO order
    scale: float           # fp32 softmax scale (exact fp32 value held in a python float)
    k_scale: float         # fp32 per-tensor scales of an fp8 pool (1.0 otherwise)
    v_scale: float
    history: List[Tuple]   # ops that build the cache before the step
    step: List[Tuple]      # allocator ops of the step
    post: List[Tuple]      # ops after the step
    k_tok: torch.Tensor    # [T, Hkv, D] act dtype: token K rows in script order
    v_tok: torch.Tensor
    decode_seqs: List[int] = field(default_factory=list)
    decode_lens: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    q_decode: Optional[torch.Tensor] = None      # [Bd, Hq, D]
    prefill_seqs: List[int] = field(default_factory=list)
    prefill_prior: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    prefill_chunk: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    q_prefill: Optional[torch.Tensor] = None     # [sum(chunk), Hq, D]
    partition_size: int = 0                      # 0: the library picks
    beam_width: int = 0                          # > 0: the decode batch is requests x this many branches
    notes: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_tokens(self) -> int:
        return int(self.k_tok.shape[0])

    def step_token_range(self) -> Tuple[int, int]:
        """[first, last) rows of k_tok/v_tok appended by the step."""
        toks = [(op[3], op[3] + op[2]) for op in self.step if op[0] == "append"]
        if not toks:
            return (0, 0)
        return (min(t[0] for t in toks), max(t[1] for t in toks))

    def history_token_range(self) -> Tuple[int, int]:
        toks = [(op[3], op[3] + op[2]) for op in self.history if op[0] == "append"]
        if not toks:
            return (0, 0)
        return (min(t[0] for t in toks), max(t[1] for t in toks))


def _torch_dtype(act: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[act]


class _Script:
    """Collects ops and hands out consecutive token rows."""

    def __init__(self):
        self.ops: List[Tuple] = []
        self.next_tok = 0

    def add(self, sid):
        self.ops.append(("add", sid))

    def append(self, sid, n):
        if n > 0:
            self.ops.append(("append", sid, int(n), self.next_tok))
            self.next_tok += int(n)

    def fork(self, parent, child):
        self.ops.append(("fork", parent, child))

    def free(self, sid):
        self.ops.append(("free", sid))

    def take(self):
        ops, self.ops = self.ops, []
        return ops


def _ceil_div(a, b):
    return -(-int(a) // int(b))


def _pool_blocks(needed: int) -> int:
    return int(math.ceil(1.25 * needed))


def _draw_tokens(gen: torch.Generator, device, t: int, hkv: int, d: int, act: str):
    """Q/K/V ~ N(0,1) drawn in fp32, then rounded to the activation dtype."""
    k = torch.randn((t, hkv, d), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((t, hkv, d), generator=gen, device=device, dtype=torch.float32)
    return k, v


def _fp32(x: float) -> float:
    return float(np.float32(x))


def make_workload(name: str, size: str = "full", device="cpu", block_size: Optional[int] = None) -> Workload:
    """Build configuration `name` at `size` ("full" or "small") with token data on `device`."""
    if name not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {name!r}; choose from {CONFIG_NAMES}")
    if size not in ("full", "small"):
        raise ValueError("size must be 'full' or 'small'")
    k_idx = CONFIG_NAMES.index(name)
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + k_idx))
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED_BASE + k_idx)
    builder = {
        "tiny_fp32": _tiny_fp32,
        "llama7b_bf16": _llama7b_bf16,
        "shared_prefix_bf16": _shared_prefix_bf16,
        "gqa_long_bf16": _gqa_long_bf16,
        "mixed_fp8": _mixed_fp8,
        "fork_storm_bf16": _fork_storm_bf16,
    }[name]
    return builder(name, size, rng, gen, device, block_size)


def _q(gen, device, n, hq, d, act):
    return torch.randn((n, hq, d), generator=gen, device=device, dtype=torch.float32).to(_torch_dtype(act))


def _decode_only(name, size, rng, gen, device, *, hq, hkv, d, b, act, kv, lens, num_blocks=None,
                 outlier_frac=0.0, partition_size=0, notes=""):
    """Independent sequences: history appends L tokens, the step appends the next token (position L)
    and decodes over positions 0..L-1."""
    bsz = len(lens)
    needed = sum(_ceil_div(int(L) + 1, b) for L in lens)
    nb = num_blocks if num_blocks is not None else _pool_blocks(needed)
    free_order = rng.permutation(nb).astype(np.int32)
    sc = _Script()
    for i, L in enumerate(lens):
        sc.add(i)
        sc.append(i, int(L))
    history = sc.take()
    for i in range(bsz):
        sc.append(i, 1)
    step = sc.take()
    t = sc.next_tok
    q = _q(gen, device, bsz, hq, d, act)
    k, v = _draw_tokens(gen, device, t, hkv, d, act)
    if outlier_frac > 0.0:
        mask = rng.random((t, hkv)) < outlier_frac
        k = k * torch.from_numpy(np.where(mask, 8.0, 1.0).astype(np.float32)).to(device)[:, :, None]
    k = k.to(_torch_dtype(act))
    v = v.to(_torch_dtype(act))
    return Workload(
        name=name, size=size, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=b,
        kv_dtype=kv, act_dtype=act, num_blocks=nb, free_order=free_order,
        scale=_fp32(1.0 / math.sqrt(d)), k_scale=1.0, v_scale=1.0,
        history=history, step=step, post=[], k_tok=k, v_tok=v,
        decode_seqs=list(range(bsz)), decode_lens=np.asarray(lens, np.int32), q_decode=q,
        partition_size=partition_size, notes=notes)


def _tiny_fp32(name, size, rng, gen, device, block_size):
    b = block_size or 16
    lens = [5, 16, 17, 40]
    return _decode_only(name, size, rng, gen, device, hq=4, hkv=4, d=64, b=b, act="f32", kv="f32",
                        lens=lens, num_blocks=32,
                        notes="4 sequences, lens {5,16,17,40}, 32-block pool in seeded order")


def _llama7b_bf16(name, size, rng, gen, device, block_size):
    b = block_size or 16
    if size == "full":
        lens = rng.integers(128, 2048, size=64, endpoint=True)
    else:
        lens = rng.integers(20, 300, size=6, endpoint=True)
    return _decode_only(name, size, rng, gen, device, hq=32, hkv=32, d=128, b=b, act="bf16", kv="bf16",
                        lens=[int(x) for x in lens])


def _gqa_long_bf16(name, size, rng, gen, device, block_size):
    b = block_size or 16
    if size == "full":
        z = rng.normal(math.log(4096.0), 1.0, size=128)
        lens = np.clip(np.rint(np.exp(z)), 256, 32768).astype(np.int64)
    else:
        z = rng.normal(math.log(700.0), 1.0, size=6)
        lens = np.clip(np.rint(np.exp(z)), 16, 3000).astype(np.int64)
    return _decode_only(name, size, rng, gen, device, hq=32, hkv=8, d=128, b=b, act="bf16", kv="bf16",
                        lens=[int(x) for x in lens], outlier_frac=0.01, partition_size=512,
                        notes="log-normal lengths (sigma 1), 1% of key vectors x8, 512-token partitions")


def _shared_prefix_bf16(name, size, rng, gen, device, block_size):
    b = block_size or 16
    hq = hkv = 40
    d = 128
    if size == "full":
        bsz, prefix, lo, hi = 256, 512, 512, 2560
    else:
        bsz, prefix, lo, hi = 5, 48, 16, 200
    suffix = []
    for _ in range(bsz):
        while True:
            s = int(rng.integers(lo, hi, endpoint=True))
            if (prefix + s) % b != 0:  # the tail block must be partly filled so the step's write CoWs it
                break
        suffix.append(s)
    lens = [prefix + s for s in suffix]
    pb = _ceil_div(prefix, b)
    needed = pb + sum(_ceil_div(L, b) - pb for L in lens) + bsz
    nb = _pool_blocks(needed)
    free_order = rng.permutation(nb).astype(np.int32)
    root = 1_000_000
    sib = 2_000_000
    sc = _Script()
    sc.add(root)
    sc.append(root, prefix)
    for i in range(bsz):
        sc.fork(root, i)
        sc.append(i, suffix[i])
    sc.free(root)
    history = sc.take()
    for i in range(bsz):
        sc.fork(i, sib + i)        # a sibling branch keeps the old tail -> the tail block is shared
    for i in range(bsz):
        sc.append(i, 1)            # writing position L into a shared tail triggers copy-on-write
    step = sc.take()
    for i in range(bsz):
        sc.free(sib + i)
    post = sc.take()
    t = sc.next_tok
    q = _q(gen, device, bsz, hq, d, "bf16")
    k, v = _draw_tokens(gen, device, t, hkv, d, "bf16")
    return Workload(
        name=name, size=size, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=b,
        kv_dtype="bf16", act_dtype="bf16", num_blocks=nb, free_order=free_order,
        scale=_fp32(1.0 / math.sqrt(d)), k_scale=1.0, v_scale=1.0,
        history=history, step=step, post=post, k_tok=k.to(torch.bfloat16), v_tok=v.to(torch.bfloat16),
        decode_seqs=list(range(bsz)), decode_lens=np.asarray(lens, np.int32), q_decode=q,
        notes=f"{prefix}-token prefix shared by all {bsz} sequences; one CoW per sequence in the step")


def _fork_storm_bf16(name, size, rng, gen, device, block_size):
    """Beam search / parallel sampling (the Day 28 page, §六 question 3: candidate branches share
    their prompt's blocks): every request is forked into W branches that share all its blocks, then
    each branch writes its next token.  All but the last writer of a request copy the shared tail
    block, so one step carries (W - 1) copies per request before the decode of all branches."""
    b = block_size or 16
    hq = hkv = 32
    d = 128
    if size == "full":
        n_req, width, lo, hi = 128, 8, 512, 2048
    else:
        n_req, width, lo, hi = 3, 4, 20, 90
    lens = []
    for _ in range(n_req):
        while True:
            L = int(rng.integers(lo, hi, endpoint=True))
            if L % b != 0:      # a partly filled tail block, so the branches' writes copy it
                break
        lens.append(L)
    needed = sum(_ceil_div(L, b) + width - 1 for L in lens)
    nb = _pool_blocks(needed)
    free_order = rng.permutation(nb).astype(np.int32)
    sc = _Script()
    for r, L in enumerate(lens):
        sc.add(r * width)
        sc.append(r * width, L)
        for j in range(1, width):
            sc.fork(r * width, r * width + j)
    history = sc.take()
    seqs = [r * width + j for r in range(n_req) for j in range(width)]
    for sid in seqs:
        sc.append(sid, 1)
    step = sc.take()
    t = sc.next_tok
    bsz = len(seqs)
    q = _q(gen, device, bsz, hq, d, "bf16")
    k, v = _draw_tokens(gen, device, t, hkv, d, "bf16")
    return Workload(
        name=name, size=size, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=b,
        kv_dtype="bf16", act_dtype="bf16", num_blocks=nb, free_order=free_order,
        scale=_fp32(1.0 / math.sqrt(d)), k_scale=1.0, v_scale=1.0,
        history=history, step=step, post=[], k_tok=k.to(torch.bfloat16), v_tok=v.to(torch.bfloat16),
        decode_seqs=seqs, decode_lens=np.asarray([lens[s // width] for s in seqs], np.int32), q_decode=q,
        beam_width=width,
        notes=f"{n_req} requests x {width} branches sharing every prompt block; "
              f"{n_req * (width - 1)} copy-on-write copies in the step")


def _mixed_fp8(name, size, rng, gen, device, block_size):
    b = block_size or 16
    if size == "full":
        n_pre, n_dec = 16, 192
        prior = rng.integers(0, 4096, size=n_pre, endpoint=True)
        chunk = np.full(n_pre, 512, np.int64)
        dlens = rng.integers(256, 8192, size=n_dec, endpoint=True)
    else:
        n_pre, n_dec = 3, 4
        prior = rng.integers(0, 200, size=n_pre, endpoint=True)
        prior[0] = 0
        chunk = rng.integers(33, 100, size=n_pre, endpoint=True)
        dlens = rng.integers(16, 400, size=n_dec, endpoint=True)
    return mixed_workload(name, size, rng, gen, device, hq=32, hkv=8, d=128, b=b, kv="fp8",
                          prior=[int(x) for x in prior], chunk=[int(x) for x in chunk],
                          dlens=[int(x) for x in dlens],
                          notes="chunked prefill co-scheduled with decode over an fp8 e4m3 pool")


def mixed_workload(name, size, rng, gen, device, *, hq, hkv, d, b, kv, prior, chunk, dlens, notes=""):
    """Prefill sequences (prior context, then a chunk of new queries) plus decode sequences.
    kv "fp8": per-tensor scales map the largest |K| (|V|) of all drawn rows to 448."""
    n_pre, n_dec = len(prior), len(dlens)
    needed = sum(_ceil_div(p + c, b) for p, c in zip(prior, chunk)) + sum(_ceil_div(L + 1, b) for L in dlens)
    nb = _pool_blocks(max(needed, 1))
    free_order = rng.permutation(nb).astype(np.int32)
    pre_ids = list(range(n_pre))
    dec_ids = list(range(n_pre, n_pre + n_dec))
    sc = _Script()
    for sid, p in zip(pre_ids, prior):
        sc.add(sid)
        sc.append(sid, p)
    for sid, L in zip(dec_ids, dlens):
        sc.add(sid)
        sc.append(sid, L)
    history = sc.take()
    for sid, c in zip(pre_ids, chunk):
        sc.append(sid, c)
    for sid in dec_ids:
        sc.append(sid, 1)
    step = sc.take()
    t = sc.next_tok
    n_q = sum(chunk)
    q_pre = _q(gen, device, n_q, hq, d, "bf16")
    q_dec = _q(gen, device, n_dec, hq, d, "bf16") if n_dec else None
    k, v = _draw_tokens(gen, device, t, hkv, d, "bf16")
    k = k.to(torch.bfloat16)
    v = v.to(torch.bfloat16)
    if kv == "fp8":
        # Per-tensor fp32 scales: the largest |K| (|V|) of the step maps to e4m3's largest finite value.
        k_scale = _fp32(float(k.abs().max().float().item()) / 448.0)
        v_scale = _fp32(float(v.abs().max().float().item()) / 448.0)
    else:
        k_scale = v_scale = 1.0
    return Workload(
        name=name, size=size, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=b,
        kv_dtype=kv, act_dtype="bf16", num_blocks=nb, free_order=free_order,
        scale=_fp32(1.0 / math.sqrt(d)), k_scale=k_scale, v_scale=v_scale,
        history=history, step=step, post=[], k_tok=k, v_tok=v,
        decode_seqs=dec_ids, decode_lens=np.asarray(dlens, np.int32), q_decode=q_dec,
        prefill_seqs=pre_ids, prefill_prior=np.asarray(prior, np.int32),
        prefill_chunk=np.asarray(chunk, np.int32), q_prefill=q_pre, notes=notes)


def layer_rows(rows: torch.Tensor, layer: int) -> torch.Tensor:
    """Rows of layer `layer` in a many-layer model: the workload's rows rotated by `layer` places along
    head_dim.  Each layer then holds different values from the same draws (a permutation, exact in
    any dtype), and the layer-0 rows are the workload's own."""
    return torch.roll(rows, shifts=int(layer), dims=-1) if layer else rows


def layer_workload(wl: Workload, layer: int) -> Workload:
    """The workload as layer `layer` of a many-layer model sees it: same operations and tables, K, V
    and Q rows from layer_rows()."""
    import dataclasses
    return dataclasses.replace(
        wl, k_tok=layer_rows(wl.k_tok, layer), v_tok=layer_rows(wl.v_tok, layer),
        q_decode=None if wl.q_decode is None else layer_rows(wl.q_decode, layer),
        q_prefill=None if wl.q_prefill is None else layer_rows(wl.q_prefill, layer))
