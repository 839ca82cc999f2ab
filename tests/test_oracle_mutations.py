"""Planted mistakes in the oracle (on the CPU) must each make a pin fail.

Each case swaps one oracle function for a plausibly wrong variant and runs the pin that should catch
it; the pin is expected to raise.  This shows the pins constrain the oracle, not only restate it.
"""
import math

import numpy as np
import pytest

import oracle.attention as att
import oracle.cache as cache
import oracle.codecs as codecs
import test_oracle_attention as TA
import test_oracle_allocator as TAL
import test_oracle_codecs as TC
import test_oracle_indexing as TI
from oracle import RefAllocator


def _expect_pin_failure(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_dropped_scale_is_caught(monkeypatch):
    orig = att.attend
    monkeypatch.setattr(att, "attend", lambda q, k, v, scale: orig(q, k, v, 1.0))
    _expect_pin_failure(TA.test_decode_matches_torch_sdpa, 4, 4)


def test_wrong_group_mapping_is_caught(monkeypatch):
    def bad_decode(q, kv, scale):
        out = np.zeros(q.shape)
        for s in range(q.shape[0]):
            k, v = kv[s]
            for h in range(q.shape[1]):
                g = h % k.shape[1]                   # interleaved instead of contiguous groups
                out[s, h] = att.attend(q[s, h], k[:, g], v[:, g], scale)
        return out
    monkeypatch.setattr(TA, "ref_decode", bad_decode)
    _expect_pin_failure(TA.test_decode_matches_torch_sdpa, 8, 2)


def test_causal_off_by_one_is_caught(monkeypatch):
    def bad_prefill(q, qsl, prior, kv, scale):
        out = np.zeros(q.shape)
        for s in range(len(prior)):
            k, v = kv[s]
            group = q.shape[1] // k.shape[1]
            for i in range(qsl[s + 1] - qsl[s]):
                vis = prior[s] + i                   # forgets the query's own key
                for h in range(q.shape[1]):
                    out[qsl[s] + i, h] = att.attend(q[qsl[s] + i, h], k[:vis, h // group], v[:vis, h // group], scale)
        return out
    monkeypatch.setattr(TA, "ref_prefill", bad_prefill)
    _expect_pin_failure(TA.test_prefill_matches_torch_sdpa_causal_and_masked)


def test_merge_without_rescale_is_caught(monkeypatch):
    def bad_merge(ms, ls, os):
        w = np.asarray(ls)
        return (w[:, None] * np.asarray(os)).sum(0) / w.sum()
    monkeypatch.setattr(TA, "merge_partitions", bad_merge)
    _expect_pin_failure(TA.test_merge_handles_partitions_far_apart)


def test_swapped_slot_fields_are_caught(monkeypatch):
    monkeypatch.setattr(TI, "slot_of", lambda table, p, b: int(table[p % b]) * b + p // b)
    from test_oracle_indexing import _tables
    import os
    golden = os.path.join(os.path.dirname(__file__), "golden")
    _expect_pin_failure(TI.check_table_7_1_3, _tables(golden))


def test_missing_copy_on_write_is_caught(monkeypatch):
    class NoCow(RefAllocator):
        def append(self, sid, n):
            slots = []
            b = self.block_size
            for _ in range(n):
                p = self.lens[sid]
                if p % b == 0:
                    blk = self.free.popleft()
                    self.ref[blk] = 1
                    self.tables[sid].append(blk)
                slots.append(self.tables[sid][p // b] * b + p % b)
                self.lens[sid] = p + 1
            return slots, []
    monkeypatch.setattr(TAL, "RefAllocator", NoCow)
    import os
    _expect_pin_failure(TAL.test_cow_scenario, os.path.join(os.path.dirname(__file__), "golden"))


def test_ties_away_from_zero_are_caught(monkeypatch):
    orig = codecs.e4m3_encode

    def away(y):
        y = np.asarray(y, np.float32)
        code = orig(y)
        # round half away from zero: bump ties that went down to an even code
        lo = codecs.e4m3_decode(code & 0x7F)
        hi = codecs.e4m3_decode(np.minimum((code & 0x7F) + 1, 0x7E).astype(np.uint8))
        tie = np.abs(np.abs(y.astype(np.float64)) - (lo + hi) / 2) == 0
        return np.where(tie, code + 1, code).astype(np.uint8)
    monkeypatch.setattr(TC, "e4m3_encode", away)
    _expect_pin_failure(TC.test_e4m3_ties_go_to_even_code)


def test_bf16_truncation_instead_of_exact_decode_is_caught(monkeypatch):
    monkeypatch.setattr(TC, "bf16_bits_to_f64",
                        lambda bits: codecs.bf16_bits_to_f64(np.asarray(bits, np.uint16) & np.uint16(0xFFF0)))
    _expect_pin_failure(TC.test_bf16_and_f32_bits_match_torch)
