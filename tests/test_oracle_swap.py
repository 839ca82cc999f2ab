"""Pins of the oracle's swap (a preempted sequence moved between the device pool and a host pool):
the content a sequence reads through its table survives a swap-out and a swap-in, with its blocks
reused by others in between; block counts; shared blocks; all-or-nothing on a short supply; and,
under random operation sequences, the content of every sequence follows it across both pools."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import RefAllocator, AllocError, OutOfBlocks, gather_seq, move_seq, ref_move_blocks


def _pool(num_blocks, b, hkv=2, d=4):
    return np.full((num_blocks, hkv, b, d), np.nan)


def _write(pool, slots, rows):
    b = pool.shape[2]
    for s, r in zip(slots, rows):
        pool[s // b, :, s % b, :] = r


def test_swap_out_and_in_keeps_the_sequence_content():
    """[day28] §六 question 4: the preempted request's blocks go to host memory and come back; what
    the sequence reads through its (new) table is what it held before, although its device blocks
    were handed to another request meanwhile."""
    b = 4
    dev, host = RefAllocator(8, b), RefAllocator(6, b)
    dpool, hpool = _pool(8, b), _pool(6, b)
    rng = np.random.default_rng(0)
    rows = rng.normal(size=(13, 2, 4))
    dev.add_seq(1)
    slots, _ = dev.append(1, 13)                 # 4 blocks, the last one partly filled
    _write(dpool, slots, rows)
    assert np.array_equal(gather_seq(dpool, dev.table(1), 13), rows)
    tab = dev.table(1)
    pairs = move_seq(dev, host, 1)
    assert [p[0] for p in pairs] == tab and len(pairs) == 4
    ref_move_blocks(hpool, dpool, pairs)
    assert dev.num_free() == 8 and host.num_free() == 2 and host.length(1) == 13
    assert np.array_equal(gather_seq(hpool, host.table(1), 13), rows)
    # another request takes every device block and overwrites it
    dev.add_seq(2)
    s2, _ = dev.append(2, 32)
    _write(dpool, s2, rng.normal(size=(32, 2, 4)))
    dev.free_seq(2)
    back = move_seq(host, dev, 1)
    ref_move_blocks(dpool, hpool, back)
    assert host.num_free() == 6 and dev.length(1) == 13
    assert np.array_equal(gather_seq(dpool, dev.table(1), 13), rows)
    dev.check_invariants()
    host.check_invariants()


def test_swap_pairs_follow_the_table_and_shared_blocks_stay():
    b = 4
    dev, host = RefAllocator(10, b, list(range(9, -1, -1))), RefAllocator(10, b)
    dev.add_seq(1)
    dev.append(1, 10)                            # blocks 9, 8, 7
    dev.fork(1, 2)                               # 2 shares all three
    dev.append(2, 1)                             # copy-on-write of the tail: 2 -> [9, 8, 6]
    pairs = move_seq(dev, host, 2)
    assert pairs == [(9, 0), (8, 1), (6, 2)]
    assert dev.refcount(9) == 1 and dev.refcount(8) == 1 and dev.refcount(6) == 0
    assert dev.free_list()[-1] == 6              # only the private block returns to the free list
    assert dev.table(1) == [9, 8, 7]
    dev.check_invariants()
    host.check_invariants()


def test_swap_is_all_or_nothing():
    b = 4
    dev, host = RefAllocator(8, b), RefAllocator(2, b)
    dev.add_seq(1)
    dev.append(1, 9)                             # 3 blocks > 2 host blocks
    state = (dev.free_list(), dev.table(1), host.free_list())
    with pytest.raises(OutOfBlocks):
        move_seq(dev, host, 1)
    assert (dev.free_list(), dev.table(1), host.free_list()) == state and 1 not in host.tables
    with pytest.raises(AllocError):
        move_seq(dev, host, 5)
    with pytest.raises(AllocError):
        move_seq(dev, RefAllocator(8, 8), 1)     # block sizes differ


def test_swap_in_reclaims_idle_cached_blocks():
    b = 4
    dev, host = RefAllocator(4, b), RefAllocator(4, b)
    dev.enable_prefix_cache()
    dev.add_seq_prefix(1, list(range(9)))
    dev.append(1, 9)
    dev.cache_seq(1, list(range(9)))
    pairs = move_seq(dev, host, 1)               # cached blocks stay cached, idle
    assert dev.num_cached() == 2 and dev.num_free() == 2
    dev.add_seq(2)
    dev.append(2, 4)                             # one free block left
    back = move_seq(host, dev, 1)                # needs 3: 1 free + 2 reclaimed from the cache
    assert len(back) == 3 and dev.num_cached() == 0
    dev.check_invariants()


_op = st.one_of(
    st.tuples(st.just("add"), st.integers(0, 4)),
    st.tuples(st.just("append"), st.integers(0, 4), st.integers(0, 20)),
    st.tuples(st.just("fork"), st.integers(0, 4), st.integers(0, 4)),
    st.tuples(st.just("free"), st.integers(0, 4)),
    st.tuples(st.just("out"), st.integers(0, 4)),
    st.tuples(st.just("in"), st.integers(0, 4)),
)


@settings(max_examples=300, deadline=None)
@given(st.lists(_op, max_size=50), st.sampled_from([2, 4, 8]), st.integers(2, 20), st.integers(1, 20))
def test_content_follows_sequences_across_pools(ops, b, n_dev, n_host):
    """Pools hold token ids; after every operation each sequence reads, through its table in the
    pool it lives in, exactly the tokens appended to it (forks copy the parent's), and both
    allocators keep their invariants."""
    dev, host = RefAllocator(n_dev, b), RefAllocator(n_host, b)
    pools = {"dev": np.full((n_dev, 1, b, 1), -1.0), "host": np.full((n_host, 1, b, 1), -1.0)}
    alloc = {"dev": dev, "host": host}
    where, content = {}, {}
    nxt = [0]
    for op in ops:
        try:
            if op[0] in ("add", "fork") and op[-1] in where:
                continue                         # ids are unique across both pools
            if op[0] == "add":
                dev.add_seq(op[1])
                where[op[1]], content[op[1]] = "dev", []
            elif op[0] == "append" and op[1] in where:
                a, pool = alloc[where[op[1]]], pools[where[op[1]]]
                slots, cow = a.append(op[1], op[2])
                for s_, d_ in cow:
                    pool[d_] = pool[s_].copy()
                toks = list(range(nxt[0], nxt[0] + op[2]))
                nxt[0] += op[2]
                for s_, t in zip(slots, toks):
                    pool[s_ // b, 0, s_ % b, 0] = t
                content[op[1]] += toks
            elif op[0] == "fork" and op[1] in where and where[op[1]] == "dev":
                dev.fork(op[1], op[2])
                where[op[2]], content[op[2]] = "dev", list(content[op[1]])
            elif op[0] == "free" and op[1] in where:
                alloc[where[op[1]]].free_seq(op[1])
                del where[op[1]], content[op[1]]
            elif op[0] in ("out", "in") and op[1] in where:
                src, dst = ("dev", "host") if op[0] == "out" else ("host", "dev")
                if where[op[1]] != src:
                    continue
                pairs = move_seq(alloc[src], alloc[dst], op[1])
                ref_move_blocks(pools[dst], pools[src], pairs)
                where[op[1]] = dst
        except (AllocError, OutOfBlocks):
            pass
        for sid, loc in where.items():
            a = alloc[loc]
            got = gather_seq(pools[loc], a.table(sid), a.length(sid))[:, 0, 0]
            assert got.tolist() == [float(t) for t in content[sid]]
        dev.check_invariants()
        host.check_invariants()
