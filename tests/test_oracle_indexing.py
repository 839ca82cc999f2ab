"""Pins of slot addressing and the pool write/gather against the pages' tables and brute force."""
import json
import os

import numpy as np
import pytest

from oracle import RefAllocator, LogicalSeqs, slot_of, ref_cache_write, gather_seq, f32_bits_to_f64


def _tables(golden_dir):
    with open(os.path.join(golden_dir, "block_tables.json")) as f:
        return json.load(f)


def check_table_7_1_3(g):
    fx = g["table_7_1_3"]
    b, table = fx["block_size"], fx["table"]
    for r in fx["ranges"]:
        for p in range(r["first_token"], r["last_token"] + 1):
            s = slot_of(table, p, b)
            assert s // b == r["physical_block"]
            assert s % b == p - r["first_token"]
    for p, s in fx["slots"].items():
        assert slot_of(table, int(p), b) == s


def test_block_table_figure(golden_dir):
    check_table_7_1_3(_tables(golden_dir))


def _grow(schedule, num_blocks, b=16):
    """Each entry of `schedule` names a sequence that fills one more block."""
    a = RefAllocator(num_blocks, b)
    for sid in sorted(set(schedule)):
        a.add_seq(sid)
    for sid in schedule:
        a.append(sid, b)
    return a


def test_figure_7_2_pointer_maps(golden_dir):
    """Three sequences growing in turn from a pool handed out in order reproduce the scattered
    pointer maps of figure 7-2 (1-based block names)."""
    maps = _tables(golden_dir)["figure_7_2_pointer_maps"]["maps"]
    a = _grow(["seq1", "seq2", "seq1", "seq3", "seq2", "seq3", "seq1", "seq3"], 8)
    for sid, want in maps.items():
        assert [x + 1 for x in a.table(sid)] == want
    a.check_invariants()


def test_figure_7_1_tables(golden_dir):
    maps = _tables(golden_dir)["figure_7_1_tables"]["maps"]
    a = _grow(["seq1", "seq2", "seq3", "seq3", "seq1", "seq2", "seq3", "seq3", "seq1"], 9)
    for sid, want in maps.items():
        assert [x + 1 for x in a.table(sid)] == want


def _random_pool_fill(seed, b, num_blocks=24, hkv=2, d=4):
    """Tiny pools filled through RefAllocator; returns everything needed for brute-force checks."""
    rng = np.random.default_rng(seed)
    a = RefAllocator(num_blocks, b, rng.permutation(num_blocks))
    lg = LogicalSeqs()
    rows = []
    pool = np.zeros((num_blocks, hkv, b, d), dtype=np.uint32)
    tok = 0
    for sid in range(4):
        a.add_seq(sid)
        lg.apply(("add", sid))
    for _ in range(12):
        sid = int(rng.integers(0, 4))
        n = int(rng.integers(1, b + 3))
        if a.blocks_needed(sid, n) > a.num_free():
            continue
        slots, cow = a.append(sid, n)
        assert not cow
        x = rng.standard_normal((n, hkv, d)).astype(np.float32).view(np.uint32)
        ref_cache_write(pool, x, slots, "f32", "f32")
        lg.apply(("append", sid, n, tok))
        rows.append(x)
        tok += n
    return a, lg, pool, np.concatenate(rows)


@pytest.mark.parametrize("b", [8, 16, 32])
def test_brute_force_every_slot_holds_its_token(b):
    """For every sequence and position, the slot's bytes are exactly that token's row."""
    a, lg, pool, rows = _random_pool_fill(b, b)
    for sid in range(4):
        table = a.table(sid)
        for p, r in enumerate(lg.token_rows(sid)):
            s = slot_of(table, p, b)
            assert np.array_equal(pool[s // b, :, s % b, :], rows[r])
        # gather through the table == the contiguous rows
        g = gather_seq(f32_bits_to_f64(pool), table, a.length(sid))
        want = f32_bits_to_f64(rows[lg.token_rows(sid)]) if a.length(sid) else np.zeros((0, 2, 4))
        assert np.array_equal(g, want)


def test_negative_slot_is_skipped():
    pool = np.zeros((2, 1, 4, 2), dtype=np.uint32)
    x = np.ones((2, 1, 2), dtype=np.uint32)
    ref_cache_write(pool, x, [-1, 5], "f32", "f32")
    assert pool.sum() == 2 and pool[1, 0, 1].tolist() == [1, 1]
