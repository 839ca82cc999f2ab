"""Pins of the attention oracle: closed forms, torch's float64 scaled_dot_product_attention as an
independent library routine, pure-Python brute force, paged == dense, split == unsplit."""
import math

import numpy as np
import pytest
import torch

from oracle import attend, ref_decode, ref_decode_split, ref_prefill, partition_stats, merge_partitions
from oracle.run import run_paged, dense_decode, dense_prefill, logical_view
from synth import make_workload


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---- closed forms ---------------------------------------------------------------------------

def test_single_key_returns_its_value():
    rng = np.random.default_rng(0)
    v = _rand(rng, 1, 16)
    assert np.array_equal(attend(_rand(rng, 16), _rand(rng, 1, 16), v, 0.3), v[0])


def test_zero_query_averages_values():
    rng = np.random.default_rng(1)
    v = _rand(rng, 37, 8)
    np.testing.assert_allclose(attend(np.zeros(8), _rand(rng, 37, 8), v, 0.5), v.mean(0), rtol=0, atol=1e-14)


def test_identical_keys_average_values():
    rng = np.random.default_rng(2)
    k = np.tile(_rand(rng, 1, 8), (23, 1))
    v = _rand(rng, 23, 8)
    np.testing.assert_allclose(attend(_rand(rng, 8), k, v, 0.7), v.mean(0), rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(3)
    q = _rand(rng, 8)
    k = _rand(rng, 30, 8) * 0.01
    k[17] = q * 100.0          # logit ~ 100 |q|^2 * scale, far above the rest
    v = _rand(rng, 30, 8)
    np.testing.assert_allclose(attend(q, k, v, 1.0), v[17], rtol=0, atol=1e-12)


def test_empty_context_gives_zeros():
    assert np.array_equal(attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0), np.zeros(4))


# ---- library routine: torch float64 SDPA on the same numbers -----------------------------------

def _sdpa(q, k, v, scale, mask=None, causal=False):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask,
        is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (32, 8)])
def test_decode_matches_torch_sdpa(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    lens = [1, 7, 33, 64]
    d = 16
    q = _rand(rng, len(lens), hq, d)
    kv = [(_rand(rng, L, hkv, d), _rand(rng, L, hkv, d)) for L in lens]
    scale = float(np.float32(1 / math.sqrt(d)))
    got = ref_decode(q, kv, scale)
    for s, (k, v) in enumerate(kv):
        # torch: [heads, L, D]; repeat each KV head over its group of query heads
        kk = np.repeat(k.transpose(1, 0, 2), hq // hkv, axis=0)
        vv = np.repeat(v.transpose(1, 0, 2), hq // hkv, axis=0)
        ref = _sdpa(q[s][:, None, :], kk, vv, scale)[:, 0, :]
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-13)


def test_prefill_matches_torch_sdpa_causal_and_masked():
    rng = np.random.default_rng(7)
    hq, hkv, d = 4, 2, 8
    prior = [0, 5, 19]
    chunk = [6, 4, 9]
    qsl = np.concatenate([[0], np.cumsum(chunk)])
    q = _rand(rng, int(qsl[-1]), hq, d)
    kv = [(_rand(rng, p + c, hkv, d), _rand(rng, p + c, hkv, d)) for p, c in zip(prior, chunk)]
    got = ref_prefill(q, qsl, prior, kv, 0.25)
    for s, (p, c) in enumerate(zip(prior, chunk)):
        k, v = kv[s]
        kk = np.repeat(k.transpose(1, 0, 2), hq // hkv, axis=0)
        vv = np.repeat(v.transpose(1, 0, 2), hq // hkv, axis=0)
        qq = q[qsl[s]:qsl[s + 1]].transpose(1, 0, 2)
        if p == 0:
            ref = _sdpa(qq, kk, vv, 0.25, causal=True)
        else:
            mask = torch.from_numpy(np.arange(p + c)[None, :] <= (p + np.arange(c))[:, None])
            ref = _sdpa(qq, kk, vv, 0.25, mask=mask)
        np.testing.assert_allclose(got[qsl[s]:qsl[s + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-13)


# ---- brute force ------------------------------------------------------------------------------

def _pure_python_attend(q, k, v, scale):
    z = [scale * sum(qi * ki for qi, ki in zip(q, krow)) for krow in k]
    m = max(z)
    p = [math.exp(x - m) for x in z]
    tot = sum(p)
    return [sum(pj * v[j][i] for j, pj in enumerate(p)) / tot for i in range(len(v[0]))]


def test_tiny_workload_against_pure_python_loops():
    wl = make_workload("tiny_fp32")
    res = run_paged(wl)
    lg = logical_view(wl)
    kt = wl.k_tok.double().numpy()
    vt = wl.v_tok.double().numpy()
    q = wl.q_decode.double().numpy()
    for bi, (sid, L) in enumerate(zip(wl.decode_seqs, wl.decode_lens)):
        rows = lg.token_rows(sid, int(L))
        for h in range(wl.num_q_heads):
            want = _pure_python_attend(q[bi, h].tolist(), kt[rows, h].tolist(), vt[rows, h].tolist(), wl.scale)
            np.testing.assert_allclose(res.decode_out[bi, h], want, rtol=0, atol=1e-12)


# ---- paged == dense, permutation invariance, shared prefix -------------------------------------

@pytest.mark.parametrize("name", ["tiny_fp32", "llama7b_bf16", "shared_prefix_bf16", "mixed_fp8",
                                  "fork_storm_bf16"])
def test_paged_equals_dense(name):
    wl = make_workload(name, "small")
    res = run_paged(wl)
    lg = logical_view(wl)
    heads = list(range(wl.num_q_heads))
    for bi in range(len(wl.decode_seqs)):
        assert np.array_equal(res.decode_out[bi], dense_decode(wl, bi, heads, lg))
    for si in range(len(wl.prefill_seqs)):
        c = int(wl.prefill_chunk[si])
        start = int(np.sum(wl.prefill_chunk[:si]))
        rows = [0, c // 2, c - 1]
        got = res.prefill_out[start:start + c][rows]
        assert np.array_equal(got, dense_prefill(wl, si, rows, heads, lg))


def test_fork_storm_copies_all_but_the_last_writer():
    """Beam branches share all their prompt's blocks (the Day 28 page, §六 question 3); each branch's
    write into the shared tail copies it first, except the last writer, which finds the block
    private again and keeps it (§六 item 4)."""
    wl = make_workload("fork_storm_bf16", "small")
    res = run_paged(wl)
    n_req, width = 3, 4
    assert len(wl.decode_seqs) == n_req * width
    assert len(res.step_cow) == n_req * (width - 1)
    for r in range(n_req):
        tabs = [res.tables[r * width + j] for j in range(width)]
        assert all(t[:-1] == tabs[0][:-1] for t in tabs)
        assert len({t[-1] for t in tabs}) == width
        pairs = res.step_cow[r * (width - 1):(r + 1) * (width - 1)]
        assert {int(a) for a, _ in pairs} == {tabs[-1][-1]}
        assert [int(b) for _, b in pairs] == [t[-1] for t in tabs[:-1]]


def test_result_independent_of_physical_block_order():
    wl = make_workload("llama7b_bf16", "small")
    a = run_paged(wl)
    wl.free_order = wl.free_order[::-1].copy()
    b = run_paged(wl)
    assert not all(np.array_equal(a.tables[s], b.tables[s]) for s in wl.decode_seqs)
    assert np.array_equal(a.decode_out, b.decode_out)


def test_shared_prefix_sequences_with_same_query_agree():
    """Sequences reading the same physical prefix blocks with the same query and content agree exactly."""
    wl = make_workload("shared_prefix_bf16", "small")
    res = run_paged(wl)
    for s in wl.decode_seqs:
        assert res.tables[s][:3] == res.tables[wl.decode_seqs[0]][:3]   # 48-token prefix = 3 blocks
    q = wl.q_decode.double().numpy()
    lg = logical_view(wl)
    rows = lg.token_rows(0, int(wl.decode_lens[0]))
    k = wl.k_tok.double().numpy()[rows]
    v = wl.v_tok.double().numpy()[rows]
    out = ref_decode(np.stack([q[0], q[0]]), [(k, v), (k.copy(), v.copy())], wl.scale)
    assert np.array_equal(out[0], out[1])
    assert np.array_equal(out[0], res.decode_out[0])


# ---- split == unsplit ---------------------------------------------------------------------------

def test_split_equals_unsplit_with_outliers():
    wl = make_workload("gqa_long_bf16", "small")
    res = run_paged(wl, split=512)
    assert max(wl.decode_lens) > 1024      # several partitions
    np.testing.assert_allclose(res.decode_out_split, res.decode_out, rtol=0, atol=1e-12)


def test_merge_handles_partitions_far_apart():
    rng = np.random.default_rng(9)
    d = 8
    q = _rand(rng, d)
    k = _rand(rng, 90, d)
    k[50] = q * 40.0            # a partition whose max is > 80 above the others
    v = _rand(rng, 90, d)
    parts = [partition_stats(q, k[a:a + 30], v[a:a + 30], 0.9) for a in (0, 30, 60)]
    ms = [p[0] for p in parts]
    assert max(ms) - min(ms) > 80
    got = merge_partitions(ms, [p[1] for p in parts], [p[2] for p in parts])
    np.testing.assert_allclose(got, attend(q, k, v, 0.9), rtol=0, atol=1e-12)


# ---- log-sum-exp (cascade merges) ----------------------------------------------------------------

def test_lse_closed_forms():
    """One key: the logit itself; L equal keys: logit + ln L; no keys: -inf; a shift of every logit
    by c shifts the log-sum-exp by c."""
    from oracle import ref_lse
    rng = np.random.default_rng(11)
    q, k = rng.normal(size=8), rng.normal(size=(1, 8))
    assert ref_lse(q, k, 0.5) == pytest.approx(0.5 * float(k[0] @ q), abs=1e-14)
    kk = np.repeat(k, 37, axis=0)
    assert ref_lse(q, kk, 0.5) == pytest.approx(0.5 * float(k[0] @ q) + np.log(37), abs=1e-12)
    assert ref_lse(q, np.zeros((0, 8)), 0.5) == float("-inf")
    big = rng.normal(size=(50, 8)) * 30.0       # logits far beyond exp's range
    z = big @ q
    assert np.isfinite(ref_lse(q, big, 1.0))
    assert ref_lse(q, big, 1.0) == pytest.approx(z.max() + np.log(np.exp(z - z.max()).sum()), rel=1e-14)


def test_merge_of_two_key_sets_by_lse_is_the_whole_softmax():
    """Attention over keys [0, S) and [S, L) combined by their log-sum-exps equals attention over all
    L keys; the combined log-sum-exp is that of all keys."""
    from oracle import ref_lse
    rng = np.random.default_rng(12)
    q, k, v = rng.normal(size=16), rng.normal(size=(90, 16)), rng.normal(size=(90, 16))
    for S in (0, 1, 45, 89, 90):
        la, lb = ref_lse(q, k[:S], 0.3), ref_lse(q, k[S:], 0.3)
        oa = attend(q, k[:S], v[:S], 0.3) if S else np.zeros(16)
        ob = attend(q, k[S:], v[S:], 0.3) if S < 90 else np.zeros(16)
        m = max(la, lb)
        wa, wb = np.exp(la - m), np.exp(lb - m)
        np.testing.assert_allclose((oa * wa + ob * wb) / (wa + wb), attend(q, k, v, 0.3), atol=1e-13)
        assert m + np.log(wa + wb) == pytest.approx(ref_lse(q, k, 0.3), abs=1e-12)
