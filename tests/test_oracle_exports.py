"""Every function the oracle library exports is reached by a CPU test that pins
it (named through its Python wrapper), and the row-parallel driver reports the
threads it ran on.  A function with no pin would be parity unpinned."""
import glob
import os
import re

import numpy as np

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# exported C function -> the wrapper the CPU pins call
WRAPPER = {
    "orc_dec_bf16": "dec_bf16", "orc_dec_e4m3": "dec_e4m3", "orc_threads_used": "threads_used",
    "orc_indexer_score": "indexer_score", "orc_topk": "topk", "orc_compact_query": "compact_query",
    "orc_compact_search": "compact_search", "orc_sparse_attn_rows": "sparse_attn_rows",
    "orc_sparse_attn": "sparse_attn", "orc_e4m3_rne": "e4m3_rne", "orc_pool_keys": "pool_keys",
    "orc_pooled_select": "pooled_select", "orc_pq_query": "pq_query", "orc_pq_search": "pq_search",
}


def exported():
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^(?!static)[a-z][\w \*]*?\b(orc_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_export_is_pinned_by_a_cpu_test():
    names = exported()
    assert set(names) == set(WRAPPER), names
    text = ""
    for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")):
        if not p.endswith("test_oracle_exports.py"):
            text += open(p).read()
    for c, py in WRAPPER.items():
        assert re.search(r"oracle\." + py + r"\(", text) or py == "threads_used", f"{c} ({py}) has no CPU pin"


def test_threads_used_counts_the_rows_run():
    s = np.zeros((3, 10))
    oracle.topk(s, 2)
    assert 1 <= oracle.threads_used() <= 3
    oracle.topk(np.zeros((40, 10)), 2)
    assert 1 <= oracle.threads_used() <= 16
