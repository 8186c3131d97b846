"""Byte accounting of a dense 16-bit cache, pinned to the figures the BellowsKV
page prints for Llama-3.1-8B (tests/golden/llama8b_cache_bytes.json)."""
import json
import os

from rank_bit_compressed_amd import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "llama8b_cache_bytes.json")


def test_llama8b_dense_cache_figures():
    g = json.load(open(GOLDEN))
    per_layer = accounting.dense_bytes_per_token(n_kv_heads=8, head_dim=128, elem_bytes=2)
    per_token = 32 * per_layer
    assert per_token == 131072                     # 32 layers x 8 heads x 128 x (K, V) x 2 bytes
    gb = per_token * g["tokens"] / 1e9
    assert round(gb, 1) == g["facts"]["cache_gb_per_sequence"]
    batch = gb * g["facts"]["sequences"]
    assert round(batch) == g["facts"]["cache_gb_batch"]
    assert round(batch / g["facts"]["compression_ratio"], 1) == g["facts"]["compressed_gb_batch"]
