"""GPU parity of swap-out / swap-in between the device pool and a pinned host pool, through the
C ABI: the host blocks hold the device blocks' codes bit for bit, the device blocks a sequence left
are overwritten, and after the swap-in the sequence decodes to the same bits as before and to the
fp64 oracle; pairs may sit in device or pinned host memory; pageable memory is refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

from oracle.run import run_paged
from synth import make_workload, poison_code

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _say(*a):
    print("[gpu-test]", *a, flush=True)


def _setup():
    from paged_kv_cache_427_amd.engine import PagedKVEngine
    wl = make_workload("llama7b_bf16", "small")
    eng = PagedKVEngine(wl, poison=poison_code(wl.kv_dtype))
    eng.build_history()
    si = eng.prepare_step()
    eng.run_step(si)
    torch.cuda.synchronize()
    return wl, eng, si


def _host_pools(eng, n_host):
    kshape = (n_host,) + tuple(eng.k_pool.shape[1:])
    vshape = (n_host,) + tuple(eng.v_pool.shape[1:])
    k = torch.zeros(kshape, dtype=eng.k_pool.dtype, pin_memory=True)
    v = torch.zeros(vshape, dtype=eng.v_pool.dtype, pin_memory=True)
    return k, v


def _decode(eng, wl, si, sids):
    from paged_kv_cache_427_amd.ops import pa_decode
    idx = [wl.decode_seqs.index(s) for s in sids]
    lens = si.dec_lens[idx].contiguous()
    mb = si.dec_tables.shape[1]
    tabs = torch.as_tensor(eng.alloc.fill_tables(sids, mb), device="cuda")
    q = si.dec_q[idx].contiguous()
    out = torch.empty_like(q)
    pa_decode(q, eng.k_pool, eng.v_pool, eng.pool, tabs, lens, wl.scale, out, int(lens.max().item()))
    torch.cuda.synchronize()
    return out, idx


@pytest.mark.parametrize("pairs_on_host", [False, True])
def test_swap_out_and_in_round_trip(pairs_on_host):
    from paged_kv_cache_427_amd.allocator import BlockAllocator, move_seq
    from paged_kv_cache_427_amd.ops import make_pool_desc, pa_swap_blocks
    from paged_kv_cache_427_amd._lib import PA_BF16
    wl, eng, si = _setup()
    ref = run_paged(wl)
    sids = wl.decode_seqs[:3]
    before, idx = _decode(eng, wl, si, sids)
    n_host = 64
    hk, hv = _host_pools(eng, n_host)
    hpool = make_pool_desc(n_host, wl.block_size, wl.num_kv_heads, wl.head_dim, PA_BF16)
    host = BlockAllocator(n_host, wl.block_size)

    def pairs_tensor(p):
        t = torch.as_tensor(p)
        return t.pin_memory() if pairs_on_host else t.cuda()

    _say("swap out", sids, "pairs on host" if pairs_on_host else "pairs on device")
    freed = []
    for s in sids:
        p = move_seq(eng.alloc, host, s)
        pa_swap_blocks(hk, hv, hpool, eng.k_pool, eng.v_pool, eng.pool, pairs_tensor(p))
        torch.cuda.synchronize()
        src = torch.as_tensor(p[:, 0].astype(np.int64), device="cuda")
        dst = torch.as_tensor(p[:, 1].astype(np.int64))
        assert torch.equal(hk[dst].view(torch.int16), eng.k_pool[src].cpu().view(torch.int16))
        assert torch.equal(hv[dst].view(torch.int16), eng.v_pool[src].cpu().view(torch.int16))
        freed += p[:, 0].tolist()
    # the device blocks the sequences left are reused by others: overwrite them
    f = torch.as_tensor(np.asarray(freed, np.int64), device="cuda")
    eng.k_pool[f] = torch.randn_like(eng.k_pool[f], dtype=torch.float32).to(eng.k_pool.dtype)
    eng.v_pool[f] = float("nan")
    torch.cuda.synchronize()
    _say("swap in", sids)
    live = []                                    # the launches are asynchronous: keep the pairs alive
    for s in sids:
        p = move_seq(host, eng.alloc, s)
        live.append(pairs_tensor(p))
        pa_swap_blocks(eng.k_pool, eng.v_pool, eng.pool, hk, hv, hpool, live[-1])
    torch.cuda.synchronize()
    del live
    after, _ = _decode(eng, wl, si, sids)
    assert torch.equal(after.view(torch.int16), before.view(torch.int16))
    err = float(np.max(np.abs(after.float().cpu().numpy() - ref.decode_out[idx])))
    _say("decode after swap-in: identical bits, oracle err", err)
    assert err <= TOL_BF16
    assert host.num_free() == n_host


def test_swap_refuses_pageable_memory():
    from paged_kv_cache_427_amd.ops import make_pool_desc
    from paged_kv_cache_427_amd._lib import PA_BF16, PA_ERR_INVALID, lib
    wl, eng, si = _setup()
    hk = torch.zeros((4,) + tuple(eng.k_pool.shape[1:]), dtype=eng.k_pool.dtype)    # pageable
    hv = torch.zeros((4,) + tuple(eng.v_pool.shape[1:]), dtype=eng.v_pool.dtype)
    hpool = make_pool_desc(4, wl.block_size, wl.num_kv_heads, wl.head_dim, PA_BF16)
    pairs = torch.tensor([[int(eng.alloc.table(wl.decode_seqs[0])[0]), 0]], dtype=torch.int32, device="cuda")
    st = lib().pa_swap_blocks(hk.data_ptr(), hv.data_ptr(), ctypes.byref(hpool), eng.k_pool.data_ptr(),
                              eng.v_pool.data_ptr(), ctypes.byref(eng.pool), pairs.data_ptr(), 1, None)
    assert st == PA_ERR_INVALID
    assert b"pinned" in lib().pa_last_error()
    # different block formats
    other = make_pool_desc(4, 32, wl.num_kv_heads, wl.head_dim, PA_BF16)
    st = lib().pa_swap_blocks(eng.k_pool.data_ptr(), eng.v_pool.data_ptr(), ctypes.byref(eng.pool),
                              eng.k_pool.data_ptr(), eng.v_pool.data_ptr(), ctypes.byref(other), pairs.data_ptr(), 1,
                              None)
    assert st == PA_ERR_INVALID
    torch.cuda.synchronize()
