"""Pins of the oracle allocator's prefix cache: the pages' shared-prefix example with caching on,
skip-prefill coverage, the one-token rule, reuse of released cached blocks, eviction order, and the
pool invariants under random operation sequences."""
import pytest
from hypothesis import given, settings, strategies as st

from oracle import RefAllocator, OutOfBlocks, AllocError


def _prompt(n, seed):
    return [(seed * 7919 + 31 * i) % 50021 for i in range(n)]


def _serve(a, sid, prompt, extra=0):
    """A request: attach cached blocks, give slots to the rest of the prompt (and `extra` decoded
    tokens), then register its full blocks.  Returns the cached token count."""
    cached = a.add_seq_prefix(sid, prompt)
    a.append(sid, len(prompt) - cached + extra)
    a.cache_seq(sid, prompt)
    return cached


def test_two_requests_sharing_a_1000_token_prompt():
    """[day28] §六 question 2 with prefix caching: the second request with the same 1000-token
    system prompt reuses its 62 full blocks (992 tokens) and computes only the rest (§七: cached
    prompts skip prefill); the partial 63rd block is not shared."""
    b = 16
    a = RefAllocator(300, b)
    a.enable_prefix_cache()
    sys_prompt = _prompt(1000, 1)
    assert _serve(a, "A", sys_prompt + _prompt(40, 2)) == 0
    cached = _serve(a, "B", sys_prompt + _prompt(30, 3))
    assert cached == 992
    ta, tb = a.table("A"), a.table("B")
    assert ta[:62] == tb[:62] and ta[62] != tb[62]
    assert all(a.refcount(x) == 2 for x in ta[:62])
    # A holds ceil(1040/16) = 65 blocks, B adds ceil((1030 - 992) / 16) = 3 of its own
    assert a.num_blocks - a.num_free() == 65 + 3
    a.check_invariants()


def test_at_least_one_prompt_token_is_left_to_compute():
    b = 8
    a = RefAllocator(40, b)
    a.enable_prefix_cache()
    p = _prompt(32, 4)                       # exactly 4 full blocks
    _serve(a, 0, p)
    assert a.add_seq_prefix(1, p) == 24      # 3 blocks: the last block's 8 tokens are recomputed
    assert a.add_seq_prefix(2, p[:25]) == 24
    assert a.add_seq_prefix(3, p[:24]) == 16
    assert a.add_seq_prefix(4, p[:1]) == 0
    a.check_invariants()


def test_released_blocks_are_kept_and_reused():
    """Freeing the only holder keeps the cached blocks (not on the free list); the next request with
    the prompt gets the same physical blocks back."""
    b = 16
    a = RefAllocator(20, b)
    a.enable_prefix_cache()
    p = _prompt(100, 5)
    _serve(a, "A", p)
    kept = a.table("A")[:6]                  # 6 full blocks; the 7th is partial
    a.free_seq("A")
    assert sorted(a.evictable_list()) == sorted(kept)
    assert not set(kept) & set(a.free_list())
    assert _serve(a, "B", p) == 96
    assert a.table("B")[:6] == kept and all(a.refcount(x) == 1 for x in kept)
    a.check_invariants()


def test_eviction_takes_the_least_recently_released_first():
    b = 4
    a = RefAllocator(6, b)
    a.enable_prefix_cache()
    p1, p2 = _prompt(9, 6), _prompt(9, 7)   # 2 full blocks each, plus one partial
    _serve(a, 1, p1)
    _serve(a, 2, p2)
    first, second = a.table(1)[:2], a.table(2)[:2]
    a.free_seq(1)
    a.free_seq(2)
    # each release queues its cached blocks deepest first
    assert a.evictable_list() == first[::-1] + second[::-1] and a.num_free() == 2
    a.add_seq(3)
    a.append(3, 12)                          # 3 blocks: the 2 free ones, then the oldest cached one
    assert a.table(3)[2] == first[1]
    assert a.add_seq_prefix(4, p1) == 4      # p1 keeps its first block, so its head still matches
    assert a.add_seq_prefix(5, p2) == 8      # p2's blocks are intact
    a.check_invariants()


def test_eviction_order_keeps_the_longest_matchable_head():
    """Under pressure a chain shrinks from its end: after k evictions the first (n - k) blocks of an
    n-block prompt still match."""
    b = 4
    a = RefAllocator(10, b)
    a.enable_prefix_cache()
    p = _prompt(33, 9)                       # 8 full blocks + 1 partial
    _serve(a, 1, p)
    a.free_seq(1)                            # 8 cached idle, 2 free (the partial block and one unused)
    for k in range(1, 7):
        a.add_seq(100 + k)
        a.append(100 + k, 4 if k > 1 else 12) # takes the 2 free blocks, then one cached block a time
        assert a.num_cached() == 8 - k
        assert a.add_seq_prefix(200 + k, p) == 4 * (8 - k)
        a.free_seq(200 + k)
    a.check_invariants()


def test_out_of_blocks_counts_the_cached_idle_blocks():
    a = RefAllocator(4, 4)
    a.enable_prefix_cache()
    _serve(a, 1, _prompt(9, 8))              # 3 blocks, 2 of them cached
    a.free_seq(1)
    a.add_seq(2)
    a.append(2, 16)                          # 4 blocks: 2 free (incl. the partial one) + 2 evicted
    with pytest.raises(OutOfBlocks):
        a.append(2, 1)
    assert a.num_cached() == 0
    a.check_invariants()


def test_cache_seq_rejects_tokens_it_does_not_hold():
    a = RefAllocator(8, 4)
    a.enable_prefix_cache()
    a.add_seq(0)
    a.append(0, 8)
    with pytest.raises(AllocError):
        a.cache_seq(0, _prompt(9, 1))
    a.cache_seq(0, _prompt(8, 1))
    with pytest.raises(AllocError):          # the same blocks under different tokens
        a.cache_seq(0, _prompt(8, 2))


def test_caching_off_changes_nothing():
    a, r = RefAllocator(30, 8), RefAllocator(30, 8)
    a.add_seq_prefix(0, _prompt(50, 1))
    a.append(0, 50)
    a.cache_seq(0, _prompt(50, 1))
    r.add_seq(0)
    r.append(0, 50)
    assert a.table(0) == r.table(0) and a.free_list() == r.free_list()
    a.free_seq(0)
    assert a.evictable_list() == [] and a.num_free() == 30


_PROMPTS = [_prompt(40, s) for s in range(3)] + [_prompt(20, 0) + _prompt(20, 9)]

_op = st.one_of(
    st.tuples(st.just("serve"), st.integers(0, 5), st.integers(0, 3), st.integers(1, 40), st.integers(0, 9)),
    st.tuples(st.just("fork"), st.integers(0, 5), st.integers(0, 5)),
    st.tuples(st.just("append"), st.integers(0, 5), st.integers(0, 20)),
    st.tuples(st.just("free"), st.integers(0, 5)),
)


@settings(max_examples=300, deadline=None)
@given(st.lists(_op, max_size=50), st.sampled_from([4, 8]), st.integers(6, 30))
def test_invariants_with_caching_under_random_ops(ops, b, nblocks):
    """Counts equal table membership; free, evictable and used blocks partition the pool; every cache
    entry names one block and back; a sequence's attached blocks hold its prompt's tokens."""
    a = RefAllocator(nblocks, b)
    a.enable_prefix_cache()
    content = {}                             # block -> the token ids it was cached with
    for op in ops:
        try:
            if op[0] == "serve":
                _, sid, pi, n, extra = op
                prompt = _PROMPTS[pi][:n]
                cached = a.add_seq_prefix(sid, prompt)
                assert cached % b == 0 and cached <= len(prompt) - 1
                for j in range(cached // b):
                    blk = a.table(sid)[j]
                    assert content[blk] == tuple(prompt[j * b:(j + 1) * b])
                try:
                    a.append(sid, len(prompt) - cached + extra)
                except OutOfBlocks:
                    a.free_seq(sid)
                    raise
                a.cache_seq(sid, prompt)
                for j in range(len(prompt) // b):
                    content[a.table(sid)[j]] = tuple(prompt[j * b:(j + 1) * b])
            elif op[0] == "fork":
                a.fork(op[1], op[2])
            elif op[0] == "append":
                a.append(op[1], op[2])
            else:
                a.free_seq(op[1])
        except (AllocError, OutOfBlocks):
            pass
        # a block taken back from the cache loses its recorded content
        for blk in list(content):
            if a.block_entry[blk] == 0:
                del content[blk]
        a.check_invariants()
