"""Pins of the oracle's sizing formula against the numbers the pages print
(tests/golden/sizing.json holds each number with its page and section)."""
import json
import os

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sizing.json")))


def test_qwen2_5_1_5b_bytes_per_token():
    g = GOLD["qwen2_5_1_5b"]
    # The page prints the product, not L: L = 28 is the only layer count that
    # reproduces it with H_kv = 2, d = 128, b = 2.
    sols = [L for L in range(1, 200)
            if oracle.kv_bytes_per_token(L, g["num_kv_heads"], g["head_dim"], g["elem_bytes"])
            == g["bytes_per_token"]]
    assert sols == [28]
    bpt = oracle.kv_bytes_per_token(28, g["num_kv_heads"], g["head_dim"], g["elem_bytes"])
    assert round(g["lmcache_tokens"] * bpt / 2**30, 4) == g["lmcache_gib_printed"]
    assert round(g["lmcache_tokens"] * bpt / 2**30, 5) == g["lmcache_gib_exact_printed"]
    assert round(g["gpu_tokens"] * bpt / 2**30, 3) == g["gpu_gib_printed"]


def test_qwen2_5_7b_and_mha():
    g = GOLD["qwen2_5_7b"]
    gqa = oracle.kv_bytes_per_token(g["num_layers"], g["num_kv_heads"], g["head_dim"],
                                    g["elem_bytes"])
    mha = oracle.kv_bytes_per_token(g["num_layers"], g["mha_num_kv_heads"], g["head_dim"],
                                    g["elem_bytes"])
    assert gqa == g["kib_per_token"] * 1024
    assert mha == g["mha_kib_per_token"] * 1024
    assert mha // gqa == g["mha_ratio"] and mha % gqa == 0


def test_gqa40_fp16_sizes():
    g = GOLD["gqa40_fp16"]
    bpt = oracle.kv_bytes_per_token(g["num_layers"], g["num_kv_heads"], g["head_dim"],
                                    g["elem_bytes"])
    assert bpt == g["kib_per_token"] * 1024
    for ctx, printed in g["gib_per_sequence_printed"].items():
        assert f"{bpt * int(ctx) / 1024**3:.2f}" == printed
    assert bpt * g["context"] * g["sequences"] == g["total_gib"] * 2**30


def test_fp8_halves_the_cache():
    # ttlab section 2: an fp8 KV cache has b = 1, halving the 16-bit size.
    assert 2 * oracle.kv_bytes_per_token(40, 8, 128, 1) == oracle.kv_bytes_per_token(40, 8, 128, 2)


def test_capacity_and_blocks():
    g = GOLD["granite_capacity"]
    assert g["kv_cache_tokens"] / g["max_model_len"] == g["max_concurrency_printed"]
    b = GOLD["blocks_from_tokens"]
    assert -(-b["tokens"] // b["block_size"]) == b["blocks"]
    assert b["blocks"] - 1 == b["usable_blocks"]  # block 0 is the reserved null block
