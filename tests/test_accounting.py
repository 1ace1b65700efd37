"""The byte and FLOP accounting the benchmark's rooflines use, pinned to the figures
the pages print ("Long context", llm-serving.xyz lecture 03, section "The
Architectural Answer: Read Less of the Past": paragraph "Stage 1, the lightning
indexer" and Derivation 4), stored in tests/golden/accounting.json with its
citation.  The benchmark's constants and formulas must reproduce each figure."""
import json
import os

import numpy as np

import bench
from synth import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accounting.json")))


def test_indexer_key_bytes():
    # 128 B FP8 key + 4 B scale = 132 B per token
    assert GOLD["indexer_key_fp8_bytes"] + GOLD["indexer_key_scale_bytes"] == GOLD["indexer_key_bytes"] == 132
    assert bench.FP8_KEY_BYTES == GOLD["indexer_key_fp8_bytes"]
    assert bench.KEY_SCALE_BYTES == GOLD["indexer_key_scale_bytes"]
    assert bench.KEY_BYTES == GOLD["indexer_key_bytes"]
    assert bench.decode_bytes(1, 1) == 132


def test_indexer_flop_per_key():
    # 64 heads x 128 dims x 2 = 16,384 FLOP per key
    assert GOLD["indexer_heads"] * GOLD["indexer_dim"] * 2 == GOLD["indexer_flop_per_key"] == 16384
    assert bench.FLOP_PER_KEY_PER_HEAD * GOLD["indexer_heads"] == GOLD["indexer_flop_per_key"]
    assert bench.decode_flop(1, 1, 64) == 16384


def test_sparse_attention_flop_per_selected_key():
    # absorbed MLA with 128 query heads: 128 x (576 + 512) x 2 = 278,528, "279 KFLOP"
    f = GOLD["mla_query_heads"] * (GOLD["mla_latent_elems"] + GOLD["mla_value_elems"]) * 2
    assert f == 278528
    assert abs(f - GOLD["mla_flop_per_selected_key_approx"]) / GOLD["mla_flop_per_selected_key_approx"] < 0.002
    assert bench.ATTN_FLOP_PER_ROW_PER_HEAD * GOLD["mla_query_heads"] == f
    assert bench.attn_flop(1, 128, 1) == f
    assert bench.LATENT_DIM == GOLD["mla_latent_elems"] and bench.VALUE_DIM == GOLD["mla_value_elems"]


def test_indexer_read_per_layer_at_128k():
    # 131,072 keys x 132 B = 17,301,504 B, "17.3 MB per layer"
    b = bench.decode_bytes(1, 131072)
    assert b == 17301504
    assert abs(b - GOLD["indexer_read_per_layer_at_128k_bytes_approx"]) / 17.3e6 < 0.001


def test_indexer_main_read_crossover():
    # per layer and step the sparse main attention reads k x 576 B and the indexer
    # L x 132 B; the indexer read passes the main read at L = 576 k / 132 ~ 8.9K
    # tokens for k = 2048
    k = 2048
    L = 576 * k / bench.KEY_BYTES
    assert abs(L - GOLD["crossover_tokens_approx"]) / GOLD["crossover_tokens_approx"] < 0.01
    assert bench.decode_bytes(1, int(L) + 1) > k * 576 > bench.decode_bytes(1, int(L))


def test_workload_rooflines():
    # batched decode: 16 x 131072 keys x 132 B = 276,824,064 B; 34.6 us at 8 TB/s,
    # 49.4 us at 70% of it
    sp = workloads.spec("batched_decode")
    b = bench.decode_bytes(sp["B"], sp["S"])
    assert b == 276824064
    t100 = b / (bench.HBM_PEAK_GBS * 1e9)
    assert abs(t100 - 34.6e-6) < 0.05e-6 and abs(t100 / 0.7 - 49.4e-6) < 0.1e-6
    # prefill chunk: the causally visible pairs x 64 heads x 256 FLOP = 8.762 TFLOP
    sp = workloads.spec("prefill_chunk")
    nv = workloads.causal_nv(sp["S"], sp["T"])
    assert int(nv.astype(np.int64).sum()) == 534775808
    assert bench.prefill_flop(nv, sp["H"]) == 534775808 * 16384
    # select-and-attend attention: 64 x 512 rows x 1,152 B gathered; 9.13 GFLOP
    sp = workloads.spec("select_attend")
    assert bench.attn_bytes(sp["B"], sp["Hq"], sp["topk"]) - sp["B"] * sp["Hq"] * (576 + 512) * 2 == \
        64 * 512 * 1152
    assert abs(bench.attn_flop(sp["B"], sp["Hq"], sp["topk"]) - 9.126e9) < 0.001e9
    # compact search: 36 B per key in stage 1 (151 MB), 2,048 x 256 B per row in stage 2
    sp = workloads.spec("compact_search")
    assert bench.compact_bytes(sp["B"], sp["S"], sp["m"]) == 32 * 131072 * 36 + 32 * 2048 * 256
