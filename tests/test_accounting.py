"""bench.py's byte and flop accounting, pinned to figures the pages print
(tests/golden/page_figures.json) and to closed forms."""
import json
import os

import bench

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_bytes_per_token_matches_printed_qwen3_8b_figure():
    # one decode token of context, K and V, 8 KV heads x 128 dims, bf16, over 36 layers
    per_layer = bench.algorithmic_bytes([1], [0], 32, 8, 128, 64, 2) - 4 - 12   # drop the page id and metadata
    assert per_layer // 2 == GOLD["one_token_one_layer_values"]["value"]       # 2 x 8 x 128 bf16 values
    assert per_layer * 36 == GOLD["qwen3_8b_bf16_bytes_per_token_36_layers"]["value"]
    assert int(1e9 // (per_layer * 36)) == GOLD["qwen3_8b_bf16_tokens_per_GB"]["value"]


def test_layer_cache_and_floor():
    kv = bench.algorithmic_bytes([4096] * 64, [0] * 64, 32, 8, 128, 64, 2) - 64 * 64 * 4 - (2 * 64 + 1) * 4
    assert kv == 1073741824
    assert round(kv / 1e9, 2) == GOLD["layer_cache_64x4096_GB"]["value"]
    assert round(36 * kv / 1e9, 1) == GOLD["all_layers_cache_GB"]["value"]
    assert round(36 * kv / 3.35e12 * 1e3, 1) == GOLD["h100_floor_ms"]["value"]


def test_decode_step_bytes_closed_form():
    b = bench.algorithmic_bytes([4096] * 64, [1] * 64, 32, 8, 128, 64, 2)
    assert b == 1073741824 + 64 * 32 * 128 * 2 * 2 + 64 * 64 * 4 + 129 * 4


def test_prefill_flops_closed_form():
    L, B, Hq, D = 8192, 4, 32, 128
    f = bench.algorithmic_flops([L] * B, [L] * B, Hq, D)
    assert f == 4 * D * Hq * B * L * (L + 1) // 2 == 2199291691008
    assert bench.algorithmic_flops([L] * B, [L] * B, 16, 256) == f
    # a chunk of n tokens over a prefix: token t sees L - n + t + 1 keys
    assert bench.algorithmic_flops([10], [3], 1, 1) == 4 * (8 + 9 + 10)
    assert bench.algorithmic_flops([10], [3], 1, 1, causal=False) == 4 * 30
    # an invalid step with more tokens than positions: early tokens see nothing
    assert bench.algorithmic_flops([2], [4], 1, 1) == 4 * (0 + 0 + 1 + 2)


def test_window_bytes_and_flops_closed_forms():
    # decode with a 1024-position window reads the last 1024 keys: 16 pages of 64
    b = bench.algorithmic_bytes([4096] * 64, [1] * 64, 32, 8, 128, 64, 2, window=1024)
    assert b == 64 * 1024 * 8 * 128 * 2 * 2 + 64 * 32 * 128 * 2 * 2 + 64 * 16 * 4 + 129 * 4
    # a window starting mid-page still counts the page holding its first key
    # (keys 50..99 span pages 0 and 1; keys 70..99 lie in page 1 only)
    assert bench.algorithmic_bytes([100], [1], 1, 1, 8, 64, 2, window=50) == 50 * 8 * 2 * 2 + 8 * 2 * 2 + 2 * 4 + 12
    assert bench.algorithmic_bytes([100], [1], 1, 1, 8, 64, 2, window=30) == 30 * 8 * 2 * 2 + 8 * 2 * 2 + 4 + 12
    # a window wider than the context changes nothing
    assert bench.algorithmic_bytes([300], [5], 4, 2, 64, 16, 2, window=1000) == \
        bench.algorithmic_bytes([300], [5], 4, 2, 64, 16, 2)
    # causal prefill n = L = 8192 with window 4096: rows 0..4095 see t + 1 keys, the rest 4096
    L, W = 8192, 4096
    pairs = W * (W + 1) // 2 + (L - W) * W
    assert bench.algorithmic_flops([L] * 4, [L] * 4, 32, 128, window=W) == 4 * 128 * 32 * 4 * pairs
    assert bench.algorithmic_flops([10], [3], 1, 1, window=2) == 4 * 6
    # not causal: row at pos sees [pos - 1, 10), i.e. 4, 3 and 2 keys
    assert bench.algorithmic_flops([10], [3], 1, 1, causal=False, window=2) == 4 * (4 + 3 + 2)


def test_quantized_cache_bytes_match_printed_int8_figure():
    # one token of context, 8 KV heads x 128 dims, 1-byte codes plus a float32 scale per head vector
    per_layer = bench.algorithmic_bytes([1], [0], 32, 8, 128, 64, 2, kv_code_bytes=1, scale_bytes=4) - 4 - 12
    assert per_layer * 36 == GOLD["qwen3_8b_int8_bytes_per_token_36_layers"]["value"]
    assert int(1e9 // (per_layer * 36)) == GOLD["qwen3_8b_int8_tokens_per_GB"]["value"]
    # the 64 x 4096 decode over an int8 cache moves 132/256 of the bf16 K/V bytes
    b8 = bench.algorithmic_bytes([4096] * 64, [1] * 64, 32, 8, 128, 64, 2, kv_code_bytes=1, scale_bytes=4)
    assert b8 == 64 * 4096 * 8 * 2 * 132 + 64 * 32 * 128 * 2 * 2 + 64 * 64 * 4 + 129 * 4
