"""Pins of slot addressing and the pool write/gather against the pages' tables and brute force."""
import json
import os

import numpy as np
import pytest

from oracle import RefAllocator, LogicalSeqs, slot_of, pool_shape, ref_cache_write, gather_seq, f32_bits_to_f64


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


def _random_pool_fill(seed, b, num_blocks=24, hkv=2, d=4, which="k"):
    """Tiny pools filled through RefAllocator; returns everything needed for brute-force checks."""
    rng = np.random.default_rng(seed)
    a = RefAllocator(num_blocks, b, rng.permutation(num_blocks))
    lg = LogicalSeqs()
    rows = []
    pool = np.zeros(pool_shape(num_blocks, hkv, b, d, which), dtype=np.uint32)
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
        ref_cache_write(pool, x, slots, "f32", "f32", which=which)
        lg.apply(("append", sid, n, tok))
        rows.append(x)
        tok += n
    return a, lg, pool, np.concatenate(rows)


def _flat_offset(which, blk, g, off, d, hkv, b, dim):
    """Element offset in the flat pool array, written out from the documented layout: tiles of
    b x D codes per (block, KV head), token-major for K (off * D + d), dim-major for V (d * b + off)."""
    tile = (blk * hkv + g) * b * dim
    return tile + (off * dim + d if which == "k" else d * b + off)


@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("b", [8, 16, 32])
def test_brute_force_every_slot_holds_its_token(b, which):
    """For every sequence and position, the slot's elements are exactly that token's row, found at
    the flat offsets of the documented tile layout."""
    hkv, dim = 2, 4
    a, lg, pool, rows = _random_pool_fill(b, b, hkv=hkv, d=dim, which=which)
    flat = pool.reshape(-1)
    for sid in range(4):
        table = a.table(sid)
        for p, r in enumerate(lg.token_rows(sid)):
            s = slot_of(table, p, b)
            for g in range(hkv):
                for d in range(dim):
                    assert flat[_flat_offset(which, s // b, g, s % b, d, hkv, b, dim)] == rows[r][g, d]
        # gather through the table == the contiguous rows
        g = gather_seq(f32_bits_to_f64(pool), table, a.length(sid), which)
        want = f32_bits_to_f64(rows[lg.token_rows(sid)]) if a.length(sid) else np.zeros((0, 2, 4))
        assert np.array_equal(g, want)


def test_negative_slot_is_skipped():
    pool = np.zeros((2, 1, 4, 2), dtype=np.uint32)
    x = np.ones((2, 1, 2), dtype=np.uint32)
    ref_cache_write(pool, x, [-1, 5], "f32", "f32")
    assert pool.sum() == 2 and pool[1, 0, 1].tolist() == [1, 1]
    vpool = np.zeros(pool_shape(2, 1, 4, 2, "v"), dtype=np.uint32)
    ref_cache_write(vpool, x, [-1, 5], "f32", "f32", which="v")
    assert vpool.sum() == 2 and vpool[1, 0, :, 1].tolist() == [1, 1]


@pytest.mark.parametrize("which", ["k", "v"])
def test_tile_of_a_block_is_contiguous(which):
    """[day28] §三 3.2: a block's K/V is contiguous.  Every element written for tokens of block blk,
    head g lies inside the tile's b x D range of the flat array, and the tile is filled exactly."""
    b, hkv, dim, nb = 8, 3, 4, 5
    pool = np.zeros(pool_shape(nb, hkv, b, dim, which), dtype=np.uint32)
    x = (np.arange(b * hkv * dim, dtype=np.uint32) + 1).reshape(b, hkv, dim)
    ref_cache_write(pool, x, [2 * b + o for o in range(b)], "f32", "f32", which=which)
    flat = pool.reshape(-1)
    for g in range(hkv):
        lo = (2 * hkv + g) * b * dim
        assert set(flat[lo:lo + b * dim].tolist()) == set(x[:, g, :].reshape(-1).tolist())
    assert np.count_nonzero(flat) == b * hkv * dim
