"""Pins of the oracle's KV byte formula against the sizes the pages print."""
import json
import os

import pytest

from oracle import kv_cache_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_bytes_pages.json")
with open(GOLDEN, encoding="utf-8") as f:
    FIX = json.load(f)


@pytest.mark.parametrize("case", FIX["cases"], ids=lambda c: c["printed"])
def test_formula_matches_page_numbers(case):
    got = kv_cache_bytes(*case["args"])
    want = case["page_bytes"]
    assert abs(got - want) <= case["rel_tol"] * want, (case["cite"], got, want)


@pytest.mark.parametrize("case", FIX["ratios"], ids=lambda c: c["printed"])
def test_kv_vs_weights_ratio(case):
    r = kv_cache_bytes(*case["args"]) / case["weights_bytes"]
    lo, hi = case["ratio_range"]
    assert lo <= r <= hi, (case["cite"], r)


def test_gqa_shrinks_kv_by_group_factor():
    # page '生成一个字…', section '显存账本': 64 query heads sharing 8 KV heads
    # cut the cache to 1/8 of the MHA size.
    mha = kv_cache_bytes(80, 64, 128, 4096, 1, 2)
    gqa = kv_cache_bytes(80, 8, 128, 4096, 1, 2)
    assert mha == 8 * gqa


def test_fp8_halves_fp16():
    # page '生成一个字…', section '再往后：压 KV 的三条路线': FP16 -> FP8 halves memory.
    assert kv_cache_bytes(32, 32, 128, 4096, 1, 1) * 2 == kv_cache_bytes(32, 32, 128, 4096, 1, 2)


def test_single_factor_of_two_is_kv_pair():
    # one layer, one head, one dim, one token, one byte: one K byte + one V byte
    assert kv_cache_bytes(1, 1, 1, 1, 1, 1) == 2
    assert kv_cache_bytes(0, 8, 128, 10, 1, 2) == 0


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        kv_cache_bytes(-1, 1, 1, 1, 1, 1)
    with pytest.raises(ValueError):
        kv_cache_bytes(1.5, 1, 1, 1, 1, 1)
