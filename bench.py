"""Benchmark of one paged-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--block-size B]

A step is the whole device path over one batch: copy-on-write block copies, the cache write of the
step's new tokens, chunked prefill (when the workload has one) and paged decode, with every input
already resident in HBM.  The default workload is the shared-prefix decode (256 sequences of a
512-token shared prefix plus a private suffix of 512..2560 tokens, 40 query = 40 KV heads,
head_dim 128, bf16, 16-token blocks, one copy-on-write per sequence).  `--config prefix_cache_bf16`
instead times 64 prompts behind one shared 1000-token system prompt, prefilled through the prefix
cache and, for comparison, in full without it; `--config swap_llama7b_bf16` times the swap of every
sequence of the Llama-7B-shaped decode workload to pinned host memory and back;
`--config llama7b_32layer_bf16` runs that workload's step for all 32 layers of the model, eager and
as one HIP graph; `--config serving_llama7b_bf16` runs a continuous-batching loop over a synthetic
request stream and reports KV utilisation against a max-length reservation.

Prints one JSON line.  `value` is the decode's unique KV bytes per step (each physical block once)
divided by the step time, in GB/s.  `roofline` prices the decode launch (stream and merge kernels),
timed with HIP events on the launch stream, against the 8 TB/s HBM peak.  `cpu_baseline` is the
fp64 CPU oracle (gather through the block tables, then attention) timed on a bounded sample of the
same workload on this host's cores, in decode tokens/s per layer like `decode_tokens_per_s_per_layer`.

The default run adds labelled side legs to the same line: `prefill_roofline`, the chunked prefill of
the mixed fp8 step (16 chunks of 512 queries over prior contexts of 0..4096 tokens, 32/8 heads, fp8
K/V) against the 2.5 PFLOP/s bf16 MFMA peak, at block sizes 16 (the figure) and 8 and 32; and
`decode_roofline_other_workloads`, the decode of the Llama-7B-shaped, GQA long-context and mixed fp8
workloads against 8 TB/s.  The MFMA-bound prefill runs 12% slower in its first ~70 ms of load on
MI355X while the clocks settle, so every workload with a prefill is warmed up with at least 150 ms
of prefill launches after the `--warmup` steps; the HBM-bound decode is the same either way.  After
timing, a device copy of known size gives the achievable HBM rate (`hbm_achievable`), and the decode
roofline is also stated as a fraction of it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import make_workload, poison_code, elem_bytes  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
# the sources of every decode launch (the stream and merge kernels; the beam decode's tail merge)
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_427_amd", "csrc", f)
               for f in ("decode.hip", "cascade.hip", "decode_records.h")]


def decode_source_hash() -> str:
    """First 16 hex digits of the sha256 of the decode sources, concatenated in DECODE_SRCS order."""
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(config: str, block_size):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary of this workload, or
    None when there is none or the decode sources changed since the counters were taken."""
    import re
    if block_size not in (None, 16):
        return None
    path = os.path.join(ROOT, "profiles", f"decode_{config}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"decode_traffic_bytes_per_launch: (\d+)", text)
    m_h = re.search(r"decode_source_sha256_16: ([0-9a-f]+)", text)
    if not (m_t and m_h):
        return None
    return int(m_t.group(1)) if decode_source_hash() == m_h.group(1) else None


def decode_bytes(wl, tables: np.ndarray):
    """(unique KV bytes, logical KV bytes, other bytes) read/written by one decode launch."""
    b, e = wl.block_size, elem_bytes(wl.kv_dtype)
    row = wl.num_kv_heads * wl.head_dim * e * 2              # K + V of one token, all KV heads
    used = {}
    logical = 0
    for s, L in enumerate(wl.decode_lens):
        L = int(L)
        logical += L
        for j in range(-(-L // b)):
            blk = int(tables[s, j])
            used[blk] = max(used.get(blk, 0), min(b, L - j * b))
    unique_tokens = sum(used.values())
    act = 2 if wl.act_dtype == "bf16" else 4
    qo = 2 * len(wl.decode_lens) * wl.num_q_heads * wl.head_dim * act
    tab = sum(-(-int(L) // b) for L in wl.decode_lens) * 4 + len(wl.decode_lens) * 4
    return unique_tokens * row, logical * row, qo + tab


def prefill_flops(wl) -> float:
    """Causal pairs only: 4 * D * Hq * sum over chunk queries of the keys each one sees."""
    tot = 0
    for p, c in zip(wl.prefill_prior, wl.prefill_chunk):
        p, c = int(p), int(c)
        tot += c * p + c * (c + 1) // 2
    return 4.0 * wl.head_dim * wl.num_q_heads * tot


def host_cores() -> int:
    """Cores this process may run on (the affinity mask, not the machine's count)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(wl, budget_s: float):
    """The fp64 oracle on a bounded sample of the workload's decode sequences, on this host's cores.

    Paged form (the value): the oracle's allocator replays the workload's operations to get every
    sequence's block table; the sampled sequences' K/V are written into a pool of stored codes
    (untimed; pool pages no sample touches are never written); the timed part is the oracle's
    gather through the table, the decoding of the gathered codes and the attention.  Dense form
    (reported beside it): the same sequences' attention on their logical rows alone."""
    from oracle import (RefAllocator, decode_pool, gather_seq, pool_shape, ref_cache_write, ref_decode)
    from oracle.run import logical_view, tensor_bits, act_values, _stored_values
    cores = host_cores()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:
        limiter = None
    alloc = RefAllocator(wl.num_blocks, wl.block_size, wl.free_order)
    for op in list(wl.history) + list(wl.step):
        if op[0] == "add":
            alloc.add_seq(op[1])
        elif op[0] == "fork":
            alloc.fork(op[1], op[2])
        elif op[0] == "free":
            alloc.free_seq(op[1])
        elif op[0] == "append":
            alloc.append(op[1], op[2])
    code_dt = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}[wl.kv_dtype]
    b, hkv, d = wl.block_size, wl.num_kv_heads, wl.head_dim
    k_codes = np.zeros(pool_shape(wl.num_blocks, hkv, b, d, "k"), dtype=code_dt)   # lazily backed
    v_codes = np.zeros(pool_shape(wl.num_blocks, hkv, b, d, "v"), dtype=code_dt)
    lg = logical_view(wl)
    order = np.random.default_rng(0).permutation(len(wl.decode_seqs))
    done, tokens, spent, spent_dense = 0, 0, 0.0, 0.0
    for bi in order:
        sid = wl.decode_seqs[bi]
        L = int(wl.decode_lens[bi])
        table = alloc.table(sid)
        rows = lg.token_rows(sid, L)
        idx = torch.as_tensor(rows, dtype=torch.long, device=wl.k_tok.device)
        kb = tensor_bits(wl.k_tok.index_select(0, idx))
        vb = tensor_bits(wl.v_tok.index_select(0, idx))
        slots = [table[p // b] * b + p % b for p in range(L)]
        ref_cache_write(k_codes, kb, slots, wl.kv_dtype, wl.act_dtype, wl.k_scale)              # untimed
        ref_cache_write(v_codes, vb, slots, wl.kv_dtype, wl.act_dtype, wl.v_scale, which="v")
        q = act_values(tensor_bits(wl.q_decode[bi:bi + 1]), wl.act_dtype)
        t = time.perf_counter()
        k = decode_pool(gather_seq(k_codes, table, L).astype(code_dt), wl.kv_dtype, wl.k_scale)
        v = decode_pool(gather_seq(v_codes, table, L, "v").astype(code_dt), wl.kv_dtype, wl.v_scale)
        ref_decode(q, [(k, v)], wl.scale)
        spent += time.perf_counter() - t
        kd, vd = _stored_values(kb, wl, "k"), _stored_values(vb, wl, "v")                    # untimed
        t = time.perf_counter()
        ref_decode(q, [(kd, vd)], wl.scale)
        spent_dense += time.perf_counter() - t
        done += 1
        tokens += L
        if spent + spent_dense >= budget_s:
            break
    if limiter is not None:
        limiter.unregister()
    row = hkv * d * elem_bytes(wl.kv_dtype) * 2
    return {"value": round(done / spent, 3), "unit": "decode tokens/s per layer", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(wl.decode_seqs)} decode sequences ({tokens} cached tokens), all "
                      f"{wl.num_q_heads} query heads, fp64 NumPy: gather through the block table, decode of "
                      f"the stored codes, attention; {spent:.1f} s",
            "logical_kv_GBps": round(tokens * row / spent / 1e9, 4),
            "dense": {"value": round(done / spent_dense, 3), "unit": "decode tokens/s per layer",
                      "note": "the same sequences' attention on their logical rows, no table gather",
                      "seconds": round(spent_dense, 2)}}


def chunk_flops(prior, chunk, head_dim: int, q_heads: int) -> float:
    """Causal pairs of chunked prefill: 4 * D * Hq * sum over chunks of (C * P + C (C + 1) / 2)."""
    tot = sum(int(c) * int(p) + int(c) * (int(c) + 1) // 2 for p, c in zip(prior, chunk))
    return 4.0 * head_dim * q_heads * tot


def prefix_cache_bench(args, dev):
    """A batch behind one 1000-token system prompt, prefilled through the prefix cache (the prompt
    was cached by a warm-up request) and, for comparison, in full without it.  A step is the cache
    write of the tokens each request computes plus the chunked prefill over them."""
    from synth.prefix import make_prefix_batch
    from paged_kv_cache_427_amd.prefix import PrefixPrefill
    b = make_prefix_batch("full", device=dev)
    reqs = list(range(b.num_requests))
    cached = PrefixPrefill(b, device=dev)
    pw = cached.admit([b.warm], [10**6])
    cached.write(pw)
    cached.prefill(pw)
    torch.cuda.synchronize()
    cached.register(pw, [b.warm])
    cached.release(pw)
    pc = cached.admit(reqs)
    full = PrefixPrefill(b, device=dev, caching=False)
    pf = full.admit(reqs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    prompt_tokens = sum(b.prompt_len(r) for r in reqs)

    def timed(drv, pi):
        for _ in range(args.warmup):
            drv.write(pi)
            drv.prefill(pi)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            drv.write(pi)
            ev[i][1].record(stream)
            drv.prefill(pi)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        w = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        p = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        return ms, w, p

    ms_c, w_c, p_c = timed(cached, pc)
    ms_f, w_f, p_f = timed(full, pf)
    fl_c = chunk_flops(pc.cached, pc.chunk, b.head_dim, b.num_q_heads)
    fl_f = chunk_flops(pf.cached, pf.chunk, b.head_dim, b.num_q_heads)
    used_c = b.num_blocks - cached.alloc.available()
    used_f = b.num_blocks - full.alloc.available()
    achieved = fl_c / (p_c * 1e-3) / 1e12
    res = {"metric": "prefix-cached prefill of a shared-system-prompt batch: prompt tokens/s (one layer)",
           "value": round(prompt_tokens / (ms_c * 1e-3), 1), "unit": "prompt tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_c, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) Q/K/V rounded to bf16, seeded token ids)",
           "uncached": {"value": round(prompt_tokens / (ms_f * 1e-3), 1), "ms_per_step": round(ms_f, 4),
                        "prefill_ms": round(p_f, 4), "cache_write_ms": round(w_f, 4),
                        "prefill_tflops": round(fl_f / (p_f * 1e-3) / 1e12, 1)},
           "speedup": round(ms_f / ms_c, 3),
           "tokens_computed": {"cached": int(pc.chunk.sum()), "uncached": int(pf.chunk.sum())},
           "blocks_used": {"cached": int(used_c), "uncached": int(used_f)},
           "kernel_ms": {"cache_write": round(w_c, 4), "prefill": round(p_c, 4)},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "pa_prefill_chunk over the uncached tails",
                        "algorithmic_flops_per_launch": fl_c},
           "config": {"workload": "prefix_cache_bf16", "requests": len(reqs),
                      "system_prompt": int(len(b.system_tokens)), "user_tokens": "U{32..512}",
                      "q_heads": b.num_q_heads, "kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                      "block_size": b.block_size, "pool_blocks": b.num_blocks,
                      "cached_tokens_per_request": int(np.median(pc.cached))}}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = prefix_cpu_baseline(b, pc, args.cpu_seconds)
    return res


def prefix_cpu_baseline(b, pc, budget_s: float):
    """fp64 oracle prefill of the cached batch's tails, request by request, on the host cores."""
    from oracle import ref_prefill
    threads = host_cores()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:
        limiter = None
    done, tokens, spent = 0, 0, 0.0
    for i in range(len(pc.chunk)):
        L = b.prompt_len(i)
        n = int(pc.cached[i])
        q, k, v = (x.double().cpu().numpy() for x in b.rows(i, 0, L))     # inputs staged untimed
        t = time.perf_counter()
        ref_prefill(q[n:], [0, L - n], [n], [(k, v)], b.scale)
        spent += time.perf_counter() - t
        done += 1
        tokens += L
        if spent >= budget_s:
            break
    if limiter is not None:
        limiter.unregister()
    return {"value": round(tokens / spent, 2), "unit": "prompt tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(pc.chunk)} requests' uncached tails, all {b.num_q_heads} query heads, "
                      f"fp64 NumPy, {spent:.1f} s"}


HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def swap_bench(args, dev):
    """Swap-out of every sequence of the Llama-7B-shaped decode workload to a pinned host pool and
    swap-in back (pa_alloc_move_seq on the host, one pa_swap_blocks launch per direction), timed per
    direction with HIP events; a plain DMA copy of the same bytes is timed beside it."""
    from paged_kv_cache_427_amd.engine import PagedKVEngine
    from paged_kv_cache_427_amd.allocator import BlockAllocator, move_seq
    from paged_kv_cache_427_amd.ops import make_pool_desc, pa_swap_blocks
    from paged_kv_cache_427_amd._lib import PA_BF16
    wl = make_workload("llama7b_bf16", "full", device=dev)
    eng = PagedKVEngine(wl, device=dev, poison=poison_code(wl.kv_dtype))
    eng.build_history()
    si = eng.prepare_step()
    eng.run_step(si)
    torch.cuda.synchronize()
    ref_out = si.dec_out.clone()
    sids = list(wl.decode_seqs)
    n_host = sum(len(eng.alloc.table(s)) for s in sids)
    hk = torch.empty((n_host,) + tuple(eng.k_pool.shape[1:]), dtype=eng.k_pool.dtype, pin_memory=True)
    hv = torch.empty((n_host,) + tuple(eng.v_pool.shape[1:]), dtype=eng.v_pool.dtype, pin_memory=True)
    hpool = make_pool_desc(n_host, wl.block_size, wl.num_kv_heads, wl.head_dim, PA_BF16)
    host = BlockAllocator(n_host, wl.block_size)
    blk = 2 * wl.num_kv_heads * wl.block_size * wl.head_dim * elem_bytes(wl.kv_dtype)
    stream = torch.cuda.current_stream()
    t_out, t_in = [], []
    for i in range(args.warmup + args.steps):
        p_out = np.concatenate([move_seq(eng.alloc, host, s) for s in sids])
        pt = torch.as_tensor(p_out, device=dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        pa_swap_blocks(hk, hv, hpool, eng.k_pool, eng.v_pool, eng.pool, pt)
        e[1].record(stream)
        torch.cuda.synchronize()
        p_in = np.concatenate([move_seq(host, eng.alloc, s) for s in sids])
        pt = torch.as_tensor(p_in, device=dev)
        e[2].record(stream)
        pa_swap_blocks(eng.k_pool, eng.v_pool, eng.pool, hk, hv, hpool, pt)
        e[3].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            t_out.append(e[0].elapsed_time(e[1]))
            t_in.append(e[2].elapsed_time(e[3]))
    # the sequences now live in other device blocks; decode must give the same bits as before
    mb = si.dec_tables.shape[1]
    si.dec_tables = torch.as_tensor(eng.alloc.fill_tables(sids, mb), device=dev)
    eng.decode_step(si)
    torch.cuda.synchronize()
    same = bool(torch.equal(si.dec_out.view(torch.int16), ref_out.view(torch.int16)))
    nbytes = len(p_out) * blk
    ms_out, ms_in = float(np.mean(t_out)), float(np.mean(t_in))
    # DMA reference: one contiguous copy of the same bytes each way
    dbuf = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    hbuf = torch.empty(nbytes // 2, dtype=torch.int16, pin_memory=True)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    hbuf.copy_(dbuf, non_blocking=True)
    e[1].record(stream)
    dbuf.copy_(hbuf, non_blocking=True)
    e[2].record(stream)
    torch.cuda.synchronize()
    dma_out, dma_in = e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])
    gbs_out, gbs_in = nbytes / (ms_out * 1e-3) / 1e9, nbytes / (ms_in * 1e-3) / 1e9
    return {"metric": "swap of a whole decode batch between HBM and pinned host memory: GB/s per direction",
            "value": round(min(gbs_out, gbs_in), 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_out + ms_in, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (the Llama-7B-shaped decode workload's K/V)",
            "swap_out": {"GBps": round(gbs_out, 2), "ms": round(ms_out, 4)},
            "swap_in": {"GBps": round(gbs_in, 2), "ms": round(ms_in, 4)},
            "dma_copy_same_bytes": {"out_GBps": round(nbytes / (dma_out * 1e-3) / 1e9, 2),
                                    "in_GBps": round(nbytes / (dma_in * 1e-3) / 1e9, 2)},
            "decode_identical_after_round_trip": same,
            "roofline": {"bound": "pcie", "achieved": round(min(gbs_out, gbs_in), 2), "peak": HOST_LINK_PEAK_GBS,
                         "unit": "GB/s", "frac": round(min(gbs_out, gbs_in) / HOST_LINK_PEAK_GBS, 4),
                         "traffic": None, "kernel": "pa_swap_blocks (copy_blocks_kernel over the host link)",
                         "algorithmic_bytes_per_launch": int(nbytes)},
            "config": {"workload": "swap_llama7b_bf16", "sequences": len(sids), "blocks": int(len(p_out)),
                       "block_bytes": blk, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                       "head_dim": wl.head_dim, "block_size": wl.block_size}}


def layers_bench(args, dev, num_layers: int = 32):
    """The Llama-7B-shaped decode step for all 32 layers of the model: one allocator and table, per-
    layer pools (46 GB), one copy launch, then per layer the cache write and the decode.  Timed eager
    and replayed as one HIP graph."""
    from synth import layer_rows
    from paged_kv_cache_427_amd.layers import LayeredEngine
    wl = make_workload("llama7b_bf16", "full", device=dev)
    eng = LayeredEngine(wl, num_layers, layer_rows, device=dev, poison=poison_code(wl.kv_dtype))
    eng.build_history()
    si = eng.prepare_step()
    eng.prepare_layers(si)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, e0.elapsed_time(e1) / args.steps

    wall_e, gpu_e = timed(lambda: eng.run_layers(si))
    eager = si.out_layers.clone()
    g = eng.capture(si)
    wall_g, gpu_g = timed(g.replay)
    same = bool(torch.equal(si.out_layers.view(torch.int16), eager.view(torch.int16)))
    # one layer's decode alone, for the kernel roofline
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        eng.k_pool, eng.v_pool = eng.k_layers[num_layers // 2], eng.v_layers[num_layers // 2]
        eng.decode_step(si)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms_dec = ev[0].elapsed_time(ev[1]) / args.steps
    tab = si.dec_tables.cpu().numpy()
    uniq, logical, other = decode_bytes(wl, tab)
    ms = max(wall_g, gpu_g)
    achieved = (uniq + other) / (ms_dec * 1e-3) / 1e9
    return {"metric": "paged decode KV-read GB/s (% of MI355X HBM peak); decode tokens/s per layer",
            "value": round(num_layers * uniq / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (the Llama-7B-shaped decode workload; layer l's rows rotated by l along head_dim)",
            "decode_tokens_per_s_all_layers": round(len(wl.decode_lens) / (ms * 1e-3), 1),
            "eager": {"ms_per_step_wall": round(wall_e, 4), "ms_per_step_gpu": round(gpu_e, 4)},
            "graph": {"ms_per_step_wall": round(wall_g, 4), "ms_per_step_gpu": round(gpu_g, 4),
                      "identical_to_eager": same},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "pa_decode of one layer (stream + merge kernels)",
                         "algorithmic_bytes_per_launch": int(uniq + other)},
            "config": {"workload": "llama7b_32layer_bf16", "layers": num_layers, "num_seqs": len(wl.decode_seqs),
                       "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                       "block_size": wl.block_size, "pool_blocks": wl.num_blocks,
                       "pool_GB_all_layers": round(2 * eng.k_layers.numel() * eng.k_layers.element_size() / 1e9, 2)}}


def serving_bench(args, dev):
    """Continuous batching of 2000 synthetic requests (prompts U{64..1024}, outputs U{16..512},
    Llama-7B-shaped attention) through a 6000-block pool for 1200 steps: every step retires, admits,
    writes the new K/V and decodes every running request.  Reports the KV utilisation of the paged
    pool against a 2048-token reservation per request, and the loop's decode throughput."""
    from synth.serving import make_request_stream
    from paged_kv_cache_427_amd.batching import ContinuousBatcher, utilisation
    st = make_request_stream("full", device=dev)
    nb, steps = 6000, 1200
    cb = ContinuousBatcher(st, nb, device=dev)
    cb.run(20)                                  # warm-up (also the loop's first steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(20, steps):
        cb.step(t)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    decoded = sum(s.decoded for s in cb.stats[20:])
    u = utilisation(cb.stats, st.block_size, st.max_model_len, nb)
    return {"metric": "continuous-batching decode tokens/s (one layer) and KV utilisation, paged vs reservation",
            "value": round(decoded / wall, 1), "unit": "decode tokens/s", "n_gpus": 1, "steps": steps - 20,
            "warmup": 20, "ms_per_step": round(wall * 1e3 / (steps - 20), 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic request stream",
            "kv_utilisation": {"paged": round(u["paged"], 4), "reservation_2048": round(u["reservation"], 4)},
            "mean_running_requests": round(u["mean_running"], 1),
            "reservation_capacity_requests": u["reservation_capacity"],
            "finished_requests": int(sum(s.finished for s in cb.stats)), "preemptions": cb.preemptions,
            "config": {"workload": "serving_llama7b_bf16", "requests": len(st.requests), "pool_blocks": nb,
                       "steps": steps, "q_heads": st.num_q_heads, "kv_heads": st.num_kv_heads,
                       "head_dim": st.head_dim, "block_size": st.block_size}}


def copy_probe(args, dev, res) -> None:
    """After timing (outside the timed region): device copies of a known size.  They calibrate the
    hardware byte counters under rocprofv3, and their rate is the achievable HBM bandwidth that the
    decode's roofline is also priced against (beside the 8 TB/s data-sheet peak)."""
    if args.copy_probe_gib <= 0:
        return
    n = int(args.copy_probe_gib * 2**30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    res["copy_probe_bytes"] = {"read": n * 4, "write": n * 4}
    gbs = 2 * n * 4 / (float(np.median(times[1:])) * 1e-3) / 1e9
    res["hbm_achievable"] = {"GBps": round(gbs, 1), "kernel": "device copy (torch copy_), read + write bytes",
                             "bytes_per_copy": 2 * n * 4, "copies_timed": len(times) - 1}
    # read-only probe: the library's streaming read of the same buffer (16-byte loads, nothing written)
    from paged_kv_cache_427_amd.ops import pa_hbm_read_probe
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    rtimes = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pa_hbm_read_probe(src, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rtimes.append(e0.elapsed_time(e1))
    rgbs = n * 4 / (float(np.median(rtimes[1:])) * 1e-3) / 1e9
    res["hbm_read_achievable"] = {"GBps": round(rgbs, 1), "kernel": "pa_hbm_read_probe (streaming 16-byte loads), bytes read",
                                  "bytes_per_read": n * 4, "reads_timed": len(rtimes) - 1}
    for key in ("roofline",):
        r = res.get(key)
        if r and r.get("bound") == "hbm":
            r["achievable_peak"] = round(gbs, 1)
            r["frac_of_achievable"] = round(r["achieved"] / gbs, 4)
            r["read_achievable_peak"] = round(rgbs, 1)
            r["frac_of_read_achievable"] = round(r["achieved"] / rgbs, 4)
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="shared_prefix_bf16")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--contiguous-blocks", action="store_true",
                    help="give the allocator the free list 0..N-1 instead of the workload's shuffled order, so "
                         "each sequence's blocks lie in ascending, mostly adjacent physical order (the cost of "
                         "the paging indirection is the difference to the default run)")
    ap.add_argument("--plain-decode", action="store_true",
                    help="beam workloads: decode every branch on its own instead of reading shared blocks once")
    ap.add_argument("--no-legs", action="store_true",
                    help="default workload only: skip the side legs (mixed fp8 prefill sweep, other decodes)")
    ap.add_argument("--copy-probe-gib", type=float, default=2.0,
                    help="after timing, run one device copy of this many GiB (a known-size kernel that "
                         "calibrates hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not code)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    modes = {"prefix_cache_bf16": prefix_cache_bench, "swap_llama7b_bf16": swap_bench,
             "llama7b_32layer_bf16": layers_bench, "serving_llama7b_bf16": serving_bench}
    if args.config in modes:
        res = modes[args.config](args, dev)
        copy_probe(args, dev, res)
        print(json.dumps(res), flush=True)
        return
    res = step_bench(args, dev, args.config, args.block_size, args.steps, args.warmup, partition=args.partition,
                     contiguous=args.contiguous_blocks, plain_decode=args.plain_decode,
                     with_cpu=not args.no_cpu_baseline, prefill_warmup_ms=PREFILL_WARMUP_MS)
    if args.config == DEFAULT_CONFIG and not args.no_legs:
        legs(args, dev, res)
    copy_probe(args, dev, res)
    print(json.dumps(res), flush=True)


DEFAULT_CONFIG = "shared_prefix_bf16"
# Prefill clocks settle only after ~70 ms of MFMA load; each prefill leg warms up for at least this long.
PREFILL_WARMUP_MS = 150.0


def step_bench(args, dev, config, block_size, steps, warmup, partition=None, contiguous=False,
               plain_decode=False, with_cpu=False, prefill_warmup_ms=0.0):
    """Time `steps` whole steps of one workload (copy-on-write copies, cache write, prefill, decode;
    a beam decode's shared part before the copies) after `warmup` untimed ones, each launch
    bracketed by HIP events on the launch stream."""
    from paged_kv_cache_427_amd.engine import PagedKVEngine
    t_setup = time.time()
    wl = make_workload(config, "full", device=dev, block_size=block_size)
    if contiguous:
        wl.free_order = np.arange(wl.num_blocks, dtype=np.int32)
    eng = PagedKVEngine(wl, device=dev, poison=poison_code(wl.kv_dtype))
    eng.build_history()
    si = eng.prepare_step(partition)
    if wl.beam_width and not plain_decode:
        eng.use_cascade(si, wl.beam_width)      # shared blocks read once for all branches of a request
    torch.cuda.synchronize()
    print(f"[bench] {config} b={wl.block_size}: setup {time.time() - t_setup:.1f}s, blocks {wl.num_blocks}, "
          f"tokens {wl.num_tokens}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    nev = 6
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]

    def step(ev=None):
        # a beam decode's shared part goes first (the step's copies and writes cannot change it); its
        # time counts as decode time
        if ev: ev[0].record(stream)
        eng.early_decode_step(si)
        if ev: ev[1].record(stream)
        eng.copy_step(si)
        if ev: ev[2].record(stream)
        eng.write_step(si)
        if ev: ev[3].record(stream)
        eng.prefill_step(si)
        if ev: ev[4].record(stream)
        eng.decode_step(si)
        if ev: ev[5].record(stream)

    for _ in range(warmup):
        step()
    if prefill_warmup_ms > 0 and wl.prefill_seqs:
        # MFMA clocks settle under sustained load: run prefill launches until they add up to at
        # least prefill_warmup_ms (timed with events, a few launches at a time)
        spent = 0.0
        while spent < prefill_warmup_ms:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                eng.prefill_step(si)
            e1.record(stream)
            torch.cuda.synchronize()
            spent += e0.elapsed_time(e1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    raw = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(nev - 1)]
                    for i in range(steps)])
    # columns: copy, write, prefill, decode (the early part of a beam decode added to the decode)
    parts = np.stack([raw[:, 1], raw[:, 2], raw[:, 3], raw[:, 0] + raw[:, 4]], axis=1)
    ms_copy, ms_write, ms_prefill, ms_decode = parts.mean(axis=0)

    res = {"metric": "paged decode KV-read GB/s (% of MI355X HBM peak); decode tokens/s per layer",
           "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
           "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": {"bf16": "bf16", "f32": "f32", "fp8": "fp8_e4m3 KV, bf16 q"}[wl.kv_dtype],
           "data": "synthetic (seeded N(0,1) K/V/Q, lengths and block order as in the workload)"}
    cfg = {"workload": config, "num_seqs": len(wl.decode_seqs) or len(wl.prefill_seqs),
           "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
           "block_size": wl.block_size, "pool_blocks": wl.num_blocks, "kv_dtype": wl.kv_dtype,
           "partition": si.dec_partition or 0,
           "block_order": "ascending" if contiguous else "shuffled"}
    tab = si.dec_tables.cpu().numpy() if si.dec_tables is not None else None
    if tab is not None:
        uniq, logical, other = decode_bytes(wl, tab)
        res["value"] = round(uniq / (ms_step * 1e-3) / 1e9, 2)
        res["decode_tokens_per_s_per_layer"] = round(len(wl.decode_lens) / (ms_step * 1e-3), 1)
        achieved = (uniq + other) / (ms_decode * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(config, block_size),
                           "traffic_source": "rocprofv3 FETCH_SIZE + WRITE_SIZE of these decode sources, scaled by "
                                             "a device copy of known size, read from the committed profile "
                                             "(null when the source changed since)",
                           "kernel": ("beam decode: pa_decode_beam (shared blocks once, left as partial records; "
                                      "then the private tails with the records folded in)"
                                      if getattr(si, "cascade", None) is not None else
                                      "pa_decode (stream + merge kernels)"),
                           "algorithmic_bytes_per_launch": int(uniq + other)}
        res["decode_logical_kv_GBps"] = round(logical / (ms_decode * 1e-3) / 1e9, 1)
        cfg["mean_context"] = round(float(np.mean(wl.decode_lens)), 1)
    else:
        res["value"] = None
    if wl.prefill_seqs:
        fl = prefill_flops(wl)
        res["prefill_tflops"] = round(fl / (ms_prefill * 1e-3) / 1e12, 1)
        res["prefill_mfma_frac"] = round(fl / (ms_prefill * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
        res["prefill_flops_per_launch"] = fl
    if len(si.host_cow):
        # copy-on-write copies: each pair reads and writes one whole block, K and V, all KV heads
        blk = 2 * wl.num_kv_heads * wl.block_size * wl.head_dim * elem_bytes(wl.kv_dtype)
        moved = 2 * len(si.host_cow) * blk
        res["copy_roofline"] = {"bound": "hbm", "achieved": round(moved / (ms_copy * 1e-3) / 1e9, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(moved / (ms_copy * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "kernel": "pa_copy_blocks", "pairs": int(len(si.host_cow)),
                                "algorithmic_bytes_per_launch": int(moved)}
    res["kernel_ms"] = {"copy_blocks": round(ms_copy, 4), "cache_write": round(ms_write, 4),
                        "prefill": round(ms_prefill, 4), "decode": round(ms_decode, 4)}
    # spread over the timed steps (kernel_ms holds the means)
    res["kernel_ms_spread"] = {name: {"median": round(float(np.median(parts[:, j])), 4),
                                      "min": round(float(np.min(parts[:, j])), 4),
                                      "p90": round(float(np.percentile(parts[:, j], 90)), 4)}
                               for j, name in ((2, "prefill"), (3, "decode"))
                               if (name == "prefill" and wl.prefill_seqs) or (name == "decode" and wl.decode_seqs)}
    res["config"] = cfg
    if with_cpu and wl.decode_seqs:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    # The workload's memory goes back to torch's cache, not to the driver: a pool allocated after
    # another workload's memory was handed back and mapped again decoded 3-4% slower (the
    # Llama-7B-shaped decode after the shared-prefix one, 0.2103 against 0.2024 ms), so each leg
    # allocates from the cache as a server that sets its pool up once would.
    del eng, si, wl
    return res


def legs(args, dev, res) -> None:
    """Side legs of the default run: the decode roofline of the other decode workloads, then the
    chunked prefill of the mixed fp8 step at each block size (MFMA roofline, with its own warm-up).
    The decode legs go first, so that they run in the state the headline decode ran in rather than
    after the prefill legs' sustained MFMA load."""
    steps = max(5, min(args.steps, 20))
    dec = {}
    for cfg in ("llama7b_bf16", "gqa_long_bf16"):
        r = step_bench(args, dev, cfg, None, steps, max(args.warmup, 3))
        dec[cfg] = {"frac": r["roofline"]["frac"], "achieved": r["roofline"]["achieved"],
                    "ms": r["kernel_ms"]["decode"], "algorithmic_bytes_per_launch":
                    r["roofline"]["algorithmic_bytes_per_launch"], "partition": r["config"]["partition"]}
    sweep = {}
    for bs in (16, 8, 32):
        r = step_bench(args, dev, "mixed_fp8", bs, steps, max(args.warmup, 3), prefill_warmup_ms=PREFILL_WARMUP_MS)
        sweep[bs] = r
    main_r = sweep[16]
    achieved = main_r["prefill_tflops"]
    res["prefill_roofline"] = {
        "bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": main_r["prefill_mfma_frac"], "traffic": None,
        "kernel": "pa_prefill_chunk (bf16 MFMA, fp8 K/V widened in LDS)",
        "algorithmic_flops_per_launch": main_r["prefill_flops_per_launch"],
        "flops_counted": "4 x head_dim x q_heads x causal query-key pairs (masked pairs not counted)",
        "ms_per_launch": main_r["kernel_ms"]["prefill"],
        "ms_spread": main_r["kernel_ms_spread"].get("prefill"),
        "warmup": f"{max(args.warmup, 3)} steps, then at least {PREFILL_WARMUP_MS:.0f} ms of prefill launches",
        "config": {"workload": "mixed_fp8", "prefill_seqs": 16, "chunk": 512, "prior": "U{0..4096}",
                   "q_heads": 32, "kv_heads": 8, "head_dim": 128, "kv_dtype": "fp8_e4m3", "block_size": 16},
        "block_size_sweep": {str(bs): {"frac": r["prefill_mfma_frac"], "tflops": r["prefill_tflops"],
                                       "ms": r["kernel_ms"]["prefill"]} for bs, r in sorted(sweep.items())},
    }
    dec["mixed_fp8"] = {str(bs): {"frac": r["roofline"]["frac"], "ms": r["kernel_ms"]["decode"]}
                        for bs, r in sorted(sweep.items())}
    res["decode_roofline_other_workloads"] = dec


if __name__ == "__main__":
    main()
