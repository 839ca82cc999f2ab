"""Attention over a sequence's cached K/V, in float64.

The pages state attention in words only: each new token's query is dotted with every cached key
and the values are combined ([ch7] 7.1 「推理为什么和训练不同」; [day28] §一 and §三 3.2).  The
formula used is the textbook softmax(scale * q K^T) V (a reading; scale is an fp32 argument used
exactly).  Grouped heads (a reading; the pages only say "KV heads", [ch7] 7.1): with Hq query heads
and Hkv KV heads, query head h reads KV head h // (Hq / Hkv).

Split-context form (not on the pages; the method it names is a partition of the context followed by
a merge): each partition k of the keys yields m_k = max z, l_k = sum exp(z - m_k),
o_k = sum exp(z - m_k) v / l_k; the merge is M = max m_k, w_k = l_k exp(m_k - M),
out = sum w_k o_k / sum w_k.  It equals the unsplit result up to rounding.

Prefill ([day28] FAQ Q4: prefill K/V also live in pool blocks; chunked prefill): query i of a chunk
whose sequence already held P tokens sits at absolute position P + i and sees keys 0 .. P + i,
itself included (the causal boundary is a reading).
"""
from typing import List, Sequence, Tuple

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q . k_j) weighted sum of v_j, for one query row q [D] over k, v [L, D]."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64)
    z = float(scale) * (k @ q)
    p = np.exp(z - z.max())
    return (p @ v) / p.sum()


def ref_decode(q: np.ndarray, kv: Sequence[Tuple[np.ndarray, np.ndarray]], scale: float) -> np.ndarray:
    """Decode attention.

    q  : [B, Hq, D] float64
    kv : per sequence (K [L, Hkv, D], V [L, Hkv, D]) float64, logical order
    returns [B, Hq, D] float64
    """
    bsz, hq, d = q.shape
    out = np.zeros((bsz, hq, d), dtype=np.float64)
    for s in range(bsz):
        k, v = kv[s]
        hkv = k.shape[1]
        group = hq // hkv
        for h in range(hq):
            g = h // group
            out[s, h] = attend(q[s, h], k[:, g, :], v[:, g, :], scale)
    return out


def partition_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """(m, l, o) of one partition: running max, exp-sum relative to it, and the normalised output."""
    z = float(scale) * (k @ q)
    m = z.max()
    p = np.exp(z - m)
    l = p.sum()
    return m, l, (p @ v) / l


def ref_lse(q: np.ndarray, k: np.ndarray, scale: float) -> float:
    """Natural log of the softmax denominator of one query over keys k [L, D]: ln sum_j exp(scale q.k_j),
    -inf for no keys.  Written as max + ln(sum of exp(z - max)) so that it does not overflow."""
    if len(k) == 0:
        return float("-inf")
    z = float(scale) * (k @ q)
    m = z.max()
    return float(m + np.log(np.exp(z - m).sum()))


def merge_partitions(ms: Sequence[float], ls: Sequence[float], os: Sequence[np.ndarray]) -> np.ndarray:
    """Combine per-partition (m, l, o) into the full softmax-weighted output."""
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    big = ms.max()
    w = ls * np.exp(ms - big)
    return (w[:, None] * np.asarray(os, dtype=np.float64)).sum(axis=0) / w.sum()


def ref_decode_split(q: np.ndarray, kv, scale: float, partition_size: int) -> np.ndarray:
    """Decode attention computed partition by partition ([512k, 512(k+1)) for size 512), then merged."""
    bsz, hq, d = q.shape
    out = np.zeros((bsz, hq, d), dtype=np.float64)
    for s in range(bsz):
        k, v = kv[s]
        length = k.shape[0]
        group = hq // k.shape[1]
        if length == 0:
            continue
        for h in range(hq):
            g = h // group
            stats = [partition_stats(q[s, h], k[a:a + partition_size, g], v[a:a + partition_size, g], scale)
                     for a in range(0, length, partition_size)]
            out[s, h] = merge_partitions([x[0] for x in stats], [x[1] for x in stats], [x[2] for x in stats])
    return out


def ref_prefill(q: np.ndarray, query_start_loc: Sequence[int], prior_lens: Sequence[int],
                kv: Sequence[Tuple[np.ndarray, np.ndarray]], scale: float) -> np.ndarray:
    """Causal chunked prefill.

    q               : [N, Hq, D] float64, the chunks of all sequences back to back
    query_start_loc : [n + 1] offsets of each sequence's chunk in q
    prior_lens      : [n] tokens each sequence held before its chunk
    kv              : per sequence (K, V) [P + C, Hkv, D] float64 (context then chunk)
    """
    n_tok, hq, d = q.shape
    out = np.zeros((n_tok, hq, d), dtype=np.float64)
    for s in range(len(prior_lens)):
        k, v = kv[s]
        group = hq // k.shape[1]
        a, e = int(query_start_loc[s]), int(query_start_loc[s + 1])
        p0 = int(prior_lens[s])
        for i in range(e - a):
            visible = p0 + i + 1
            for h in range(hq):
                g = h // group
                out[a + i, h] = attend(q[a + i, h], k[:visible, g], v[:visible, g], scale)
    return out
