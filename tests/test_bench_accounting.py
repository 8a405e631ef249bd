"""The byte and FLOP accounting the benchmark reports (CPU only).

* KV-cache size: the cabseo page ("Memory requirements") gives the cache of
  one sequence as sequence length x 2 (K and V) x layers x hidden size x bytes
  per value, worked for Llama 2 in fp16 at 4096 tokens as about 2 GB; the
  fixture ``golden/kv_cache_llama2.json`` holds that example.
* The decode traffic the benchmark counts per layer is that formula for one
  layer (the K/V rows of every sequence read once) plus q read and o, lse
  written.
* Prefill FLOPs follow the stated convention 4 B Hq Nq Nk d, halved for
  causal: 5.498e11 on the Llama-3-8B layer.
"""
import json
import os

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def test_kv_cache_formula_matches_the_pages_example():
    g = json.load(open(os.path.join(HERE, "golden", "kv_cache_llama2.json")))
    got = bench.kv_cache_bytes(g["sequence_length"], g["num_layers"], g["hidden_size"], g["bytes_per_value"])
    assert got == g["expected_bytes"] == 2 * 1024 ** 3


def test_decode_bytes_is_one_layer_of_the_cache_plus_q_o_lse():
    # a Llama-2-like multi-head layer: 32 heads of width 128 = hidden 4096
    lens = [4096, 17, 30000]
    Hq = Hkv = 32
    d = 128
    cache = sum(bench.kv_cache_bytes(L, 1, Hkv * d, 2) for L in lens)
    B = len(lens)
    assert bench.decode_bytes(lens, Hq, Hkv, d) == cache + 2 * 2 * B * Hq * d + 4 * B * Hq
    # grouped kv-heads: only the Hkv heads' rows are read, for all Hq q-heads
    assert bench.decode_bytes([100], 32, 8, 128) == 100 * 8 * 128 * 2 * 2 + 2 * 2 * 32 * 128 + 4 * 32


def test_prefill_accounting():
    assert bench.prefill_flops(1, 32, 8192, 8192, 128, True) == 4 * 32 * 8192 ** 2 * 128 / 2 == 549755813888.0
    assert bench.prefill_flops(2, 8, 4096, 4096, 64, False) == 4 * 2 * 8 * 4096 ** 2 * 64
    # Q, K, V read once; O and LSE written once
    assert bench.prefill_bytes(1, 32, 8, 8192, 8192, 128) == 2 * (2 * 32 * 8192 * 128 + 2 * 8 * 8192 * 128) + 4 * 32 * 8192
