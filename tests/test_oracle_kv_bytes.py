"""Pins the oracle's byte accounting to the sizes the pages print."""
import json
import os

import pytest

from oracle import kv_bytes

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes_pages.json")))


@pytest.mark.parametrize("case", GOLDEN["per_token"], ids=lambda c: c["model"])
def test_per_token_matches_pages(case):
    got = kv_bytes.kv_bytes_per_token(case["n_layers"], case["n_kv_heads"], case["head_dim"],
                                      case["bytes_per_elem"])
    assert got == case["bytes"], case["cite"]


@pytest.mark.parametrize("case", GOLDEN["per_context"], ids=lambda c: f'{c["model"]}-{c["seq_len"]}x{c["batch"]}')
def test_per_context_matches_pages(case):
    got = kv_bytes.kv_cache_bytes(case["n_layers"], case["n_kv_heads"], case["head_dim"],
                                  case["seq_len"], case["batch"], case["bytes_per_elem"])
    assert got == case["bytes"], case["cite"]


@pytest.mark.parametrize("case", GOLDEN["ratios"], ids=lambda c: f'{c["n_q_heads"]}/{c["n_kv_heads"]}')
def test_mha_gqa_ratio_matches_pages(case):
    assert kv_bytes.mha_to_gqa_ratio(case["n_q_heads"], case["n_kv_heads"]) == case["ratio"]


def test_one_llama2_layer_of_the_32gb_example_is_one_gib():
    # 16 sequences x 4096 tokens, 32 KV heads x 128, bf16: one of 32 layers of 32 GiB.
    lens = [4096] * 16
    assert kv_bytes.attended_kv_bytes(lens, 32, 128, 2) == 2 ** 30


def test_formula_is_linear_in_every_factor():
    base = kv_bytes.kv_cache_bytes(3, 5, 7, 11, 13, 2)
    assert kv_bytes.kv_cache_bytes(6, 5, 7, 11, 13, 2) == 2 * base
    assert kv_bytes.kv_cache_bytes(3, 10, 7, 11, 13, 2) == 2 * base
    assert kv_bytes.kv_cache_bytes(3, 5, 14, 11, 13, 2) == 2 * base
    assert kv_bytes.kv_cache_bytes(3, 5, 7, 22, 13, 2) == 2 * base
    assert kv_bytes.kv_cache_bytes(3, 5, 7, 11, 26, 2) == 2 * base
    assert kv_bytes.kv_cache_bytes(3, 5, 7, 11, 13, 4) == 2 * base
