"""Pins of the reference allocator: the pages' copy-on-write scenario, stated invariants, OOM."""
import json
import os

import pytest
from hypothesis import given, settings, strategies as st

from oracle import RefAllocator, OutOfBlocks, AllocError


def _cow(golden_dir):
    with open(os.path.join(golden_dir, "cow_scenario.json")) as f:
        return json.load(f)


def test_cow_scenario(golden_dir):
    """Requests A and B share their first two blocks (count 2); B writing into the shared block gets a
    new block holding a copy, and the old block's count drops by one."""
    g = _cow(golden_dir)
    b = g["block_size"]
    a = RefAllocator(8, b)
    a.add_seq("A")
    a.append("A", g["request_a_tokens"])
    a.fork("A", "B")
    ta, tb = a.table("A"), a.table("B")
    n_shared = g["expect_after_fork"]["shared_entries"]
    assert ta[:n_shared] == tb[:n_shared]
    assert all(a.refcount(x) == g["expect_after_fork"]["refcount"] for x in ta[:n_shared])
    old = tb[1]
    slots, cow = a.append("B", 1)
    e = g["expect_after_b_writes"]
    assert len(cow) == e["copies"] and cow[0][0] == old
    new = cow[0][1]
    assert a.table("B")[1] == new and new != old
    assert a.table("A")[1] == old
    assert a.refcount(old) == e["old_block_refcount"]
    assert a.refcount(new) == e["new_block_refcount"]
    assert a.refcount(a.table("A")[0]) == e["block_0_refcount"]
    assert slots == [new * b + g["request_a_tokens"] % b]
    a.check_invariants()


def test_on_demand_allocation():
    """A block is taken only when the previous one is full ([ch7] 7.1: write 16, then take the next)."""
    a = RefAllocator(4, 16)
    a.add_seq(0)
    for n in range(1, 49):
        a.append(0, 1)
        assert len(a.table(0)) == -(-n // 16)
    assert a.num_free() == 1


def test_free_returns_blocks_any_block_serves_anyone():
    a = RefAllocator(3, 4, [2, 0, 1])
    a.add_seq(0)
    a.append(0, 12)
    assert a.table(0) == [2, 0, 1] and a.num_free() == 0
    with pytest.raises(OutOfBlocks):
        a.add_seq(1) or a.append(1, 1)
    a.free_seq(0)
    assert a.free_list() == [2, 0, 1]
    a.append(1, 5)
    assert a.table(1) == [2, 0]


def test_oom_is_all_or_nothing():
    a = RefAllocator(4, 4)
    a.add_seq(0)
    a.append(0, 6)
    a.fork(0, 1)
    before = (a.table(0), a.table(1), a.free_list(), list(a.ref), a.length(1))
    with pytest.raises(OutOfBlocks):
        a.append(1, 11)           # needs 1 CoW + 3 new blocks = 4 > 2 free
    assert (a.table(0), a.table(1), a.free_list(), list(a.ref), a.length(1)) == before
    a.append(1, 6)                # 1 CoW + 1 new block: fits
    a.check_invariants()


def test_shared_prefix_of_1000_tokens_is_stored_once():
    """[day28] §六 question 2: two requests sharing a 1000-token prefix hold its 63 blocks once."""
    a = RefAllocator(200, 16)
    a.add_seq("p")
    a.append("p", 1000)
    a.fork("p", "q")
    used = a.num_blocks - a.num_free()
    assert used == 63
    assert all(a.refcount(x) == 2 for x in a.table("p"))


def test_errors():
    a = RefAllocator(4, 4)
    a.add_seq(0)
    with pytest.raises(AllocError):
        a.add_seq(0)
    with pytest.raises(AllocError):
        a.append(9, 1)
    with pytest.raises(AllocError):
        a.fork(9, 1)
    with pytest.raises(AllocError):
        a.free_seq(9)
    with pytest.raises(AllocError):
        RefAllocator(4, 4, [0, 0, 1, 2])


_op = st.one_of(
    st.tuples(st.just("add"), st.integers(0, 5)),
    st.tuples(st.just("fork"), st.integers(0, 5), st.integers(0, 5)),
    st.tuples(st.just("append"), st.integers(0, 5), st.integers(0, 40)),
    st.tuples(st.just("free"), st.integers(0, 5)),
)


@settings(max_examples=300, deadline=None)
@given(st.lists(_op, max_size=60), st.sampled_from([8, 16, 32]), st.integers(4, 30))
def test_invariants_under_random_ops(ops, b, nblocks):
    """Tail waste below one block, counts equal table membership, free and used partition the pool,
    and the block receiving an append's last token is private to the appending sequence."""
    a = RefAllocator(nblocks, b)
    for op in ops:
        try:
            if op[0] == "add":
                a.add_seq(op[1])
            elif op[0] == "fork":
                a.fork(op[1], op[2])
            elif op[0] == "append":
                slots, cow = a.append(op[1], op[2])
                if op[2] > 0:
                    # the block receiving the last write is private: new or just copied
                    last = a.table(op[1])[(a.length(op[1]) - 1) // b]
                    assert a.refcount(last) == 1
                    assert slots[-1] // b == last
                for src, dst in cow:
                    assert a.refcount(dst) == 1 and a.refcount(src) >= 1
            else:
                a.free_seq(op[1])
        except (AllocError, OutOfBlocks):
            pass
        a.check_invariants()
