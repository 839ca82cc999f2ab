"""Pins of the KV size formula against the values the pages print (tests/golden/kv_bytes.json)."""
import json
import os

import pytest

from oracle import kv_bytes_per_token, kv_cache_bytes


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "kv_bytes.json")) as f:
        return json.load(f)


def check_per_token(golden):
    for c in golden["cases"]:
        got = kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["dtype_bytes"])
        assert got == c["bytes_per_token"], (c["what"], got)


def check_multiples(golden):
    for c in golden["multiples"]:
        got = kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["tokens"], c["dtype_bytes"])
        assert got == c["bytes"], (c["what"], got)
        if "printed_mib" in c:
            assert got == c["printed_mib"] * 2**20
        if "printed_mb_approx" in c:
            assert abs(got / 2**20 - c["printed_mb_approx"]) / c["printed_mb_approx"] < 0.05


def test_per_token_worked_values(golden_dir):
    check_per_token(_golden(golden_dir))


def test_multiples(golden_dir):
    check_multiples(_golden(golden_dir))


def test_fp8_halves_bf16():
    # «第 7 章推理框架：vLLM 与 PagedAttention» 7.1 (KV cache 显存估算, 显存优化): an fp8 KV cache
    # takes half the bytes of a bf16 one
    assert 2 * kv_bytes_per_token(32, 8, 128, 1) == kv_bytes_per_token(32, 8, 128, 2)


@pytest.mark.parametrize("layers,heads,dim,e,expected", [(1, 40, 128, 2, 20480), (1, 32, 128, 2, 16384),
                                                          (1, 8, 128, 2, 4096), (1, 8, 128, 1, 2048),
                                                          (1, 4, 64, 4, 2048)])
def test_per_layer_bytes_of_the_workloads(layers, heads, dim, e, expected):
    assert kv_bytes_per_token(layers, heads, dim, e) == expected
