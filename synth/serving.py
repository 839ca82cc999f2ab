"""A synthetic request stream for continuous batching, and the K/V/q rows its tokens carry.

Continuous batching admits and retires requests every step ([ch7] 7.1 and its example on
scheduling; [day28] §五: with paging, freed blocks serve new requests at once).  Requests arrive
over the steps with prompt and output lengths drawn uniformly; a request's token at position p
carries K/V row (7919 * rid + p) mod R of one table of R seeded rows, and its decode query at that
position the row (104729 * rid + p) mod R of a second table, so either side can rebuild any
request's dense K/V without storing it.

Random draws, in fixed order (seed 4270 + 200): numpy PCG64 arrivals -> prompt lengths -> output
lengths; torch Philox K table -> V table -> q table (N(0,1), rounded to bf16).
"""
from dataclasses import dataclass
from typing import List

import numpy as np
import torch

SEED = 4270 + 200


@dataclass
class Request:
    rid: int
    arrival: int        # step at which the request arrives
    prompt_len: int
    output_len: int     # tokens decoded before the request finishes


@dataclass
class RequestStream:
    requests: List[Request]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    max_model_len: int  # what a reservation-based engine sets aside per request
    k_table: torch.Tensor   # [R, Hkv, D] bf16
    v_table: torch.Tensor
    q_table: torch.Tensor   # [R, Hq, D] bf16
    scale: float

    def kv_rows(self, rid: int, start: int, n: int) -> torch.Tensor:
        """Row indices (int64) of positions start .. start+n-1 of request rid."""
        r = self.k_table.shape[0]
        return torch.as_tensor((7919 * rid + np.arange(start, start + n, dtype=np.int64)) % r)

    def q_row(self, rid: int, pos: int) -> int:
        return int((104729 * rid + pos) % self.q_table.shape[0])


def make_request_stream(size: str = "full", device="cpu") -> RequestStream:
    """full: 2000 requests arriving over 1000 steps, prompts U{64..1024}, outputs U{16..512}, 32/32
    heads (the Llama-7B shape), 2048-token reservation; small: 24 requests over 12 steps, prompts
    U{5..60}, outputs U{1..20}, 8/2 heads, 128-token reservation."""
    rng = np.random.Generator(np.random.PCG64(SEED))
    if size == "full":
        n, steps, plo, phi, olo, ohi, hq, hkv, d, max_len, rows = 2000, 1000, 64, 1024, 16, 512, 32, 32, 128, 2048, 8192
    elif size == "small":
        n, steps, plo, phi, olo, ohi, hq, hkv, d, max_len, rows = 24, 12, 5, 60, 1, 20, 8, 2, 128, 128, 512
    else:
        raise ValueError(size)
    arrivals = np.sort(rng.integers(0, steps, size=n))
    prompts = rng.integers(plo, phi, size=n, endpoint=True)
    outputs = rng.integers(olo, ohi, size=n, endpoint=True)
    reqs = [Request(i, int(a), int(p), int(o)) for i, (a, p, o) in enumerate(zip(arrivals, prompts, outputs))]
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED)

    def draw(h):
        return torch.randn((rows, h, d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)

    k, v, q = draw(hkv), draw(hkv), draw(hq)
    return RequestStream(reqs, hq, hkv, d, 16, max_len, k, v, q, float(np.float32(1.0 / np.sqrt(d))))
