"""The seeded synthetic workloads: shapes, value distributions and input recipes.

Each workload is named for what it is.  Inputs are pure functions of
(seed, tensor id, flat index) through the generators in gen.c; every one is drawn
in fp64 and rounded to its storage format (fp32, bf16, fp8 E4M3FN + fp32 row
scale, int8 + fp32 row scale).  Smaller variants for parity tests pass overrides
(same recipe, other sizes).
"""
import math

import numpy as np

from . import compact_keys, fp8_rows, normal_bf16, normal_bf16_rows, normal_f32, pq_codebook, pq_encode, uniform_f32

SEED_BASE = 0x5EED0000

# tensor ids within one workload's seed
TID_Q, TID_W, TID_K, TID_P, TID_LATENT, TID_QATT = 1, 2, 3, 4, 5, 6

WORKLOADS = {
    # one query, 4096 fp32 keys, 8 heads, top-64
    "tiny_decode": dict(B=1, T=1, S=4096, H=8, d=128, topk=64, key="f32", q="f32",
                        q_scale=1 / math.sqrt(128), w="uniform", causal=False, seed=SEED_BASE + 1),
    # 16 sequences x 131072 fp8 keys (stride-4 compression of 512K tokens), 64 heads, top-512
    "batched_decode": dict(B=16, T=1, S=131072, H=64, d=128, topk=512, key="fp8", q="bf16",
                           q_scale=1 / math.sqrt(128), w="uniform", causal=False, seed=SEED_BASE + 2),
    # one 4096-query prefill chunk over 131072 bf16 keys, causal, 64 heads, top-512
    "prefill_chunk": dict(B=1, T=4096, S=131072, H=64, d=128, topk=512, key="bf16", q="bf16",
                          q_scale=1.0, w="uniform", causal=True, seed=SEED_BASE + 3),
    # 32 sequences x 131072 keys: int8 32-d compact keys -> 2048 shortlist -> exact top-512
    "compact_search": dict(B=32, T=1, S=131072, H=64, d=128, dc=32, m=2048, topk=512, key="bf16", q="bf16",
                           q_scale=1 / math.sqrt(128), w="uniform", causal=False, seed=SEED_BASE + 4),
    # 64 sequences x 262144 entries: fp8 indexer top-512, then 128-head attention over
    # the selected 576-d bf16 latent rows (values = first 512 dims), tau = 1/sqrt(192)
    "select_attend": dict(B=64, T=1, S=262144, H=64, d=128, topk=512, key="fp8", q="bf16", q_scale=1.0,
                          w="normal", causal=False, Hq=128, dqk=576, dv=512, tau=1 / math.sqrt(192),
                          seed=SEED_BASE + 5),
    # 32 sequences x 131072 keys: product-quantised codes (32 pieces of 4 dims, one
    # byte each into a 256-entry k-means codebook per piece) -> 2048 shortlist ->
    # exact top-512 over the bf16 keys
    "pq_search": dict(B=32, T=1, S=131072, H=64, d=128, m=2048, topk=512, key="bf16", q="bf16",
                      q_scale=1 / math.sqrt(128), w="uniform", causal=False, pq_train_stride=64, pq_iters=8,
                      seed=SEED_BASE + 7),
    # a 4096-query prefill chunk through 8 layers whose history (131072 bf16 indexer
    # keys and 131072 compressed KV rows of 576 bytes per layer) lives in host
    # memory and is streamed through two GPU buffers; causal, 64 heads, top-512
    "layer_stream": dict(B=1, T=4096, S=131072, H=64, d=128, topk=512, L=8, kv_row=576, key="bf16", q="bf16",
                         q_scale=1.0, w="uniform", causal=True, seed=SEED_BASE + 8),
    # 16 sequences x 524288 bf16 token keys pooled four at a time on write (131072
    # fp8 pooled keys each), a 32-head indexer over the pooled keys, top-512 blocks
    # expanded to 2048 tokens
    "pooled_decode": dict(B=16, T=1, L=524288, pool=4, S=131072, H=32, d=128, topk=512, key="bf16", q="bf16",
                          q_scale=1 / math.sqrt(128), w="uniform", causal=False, seed=SEED_BASE + 6),
}


def spec(name, **over):
    s = dict(WORKLOADS[name])
    s.update(over)
    s["name"] = name
    return s


def causal_nv(S, T):
    """Visible keys per query of a prefill chunk: the chunk is the last T tokens of a
    4S-token context compressed at stride 4; token p = 4S - T + t sees compressed
    keys s <= floor(p / 4)."""
    t = np.arange(T, dtype=np.int64)
    p = 4 * S - T + t
    return (p // 4 + 1).astype(np.int32)


def indexer_inputs(sp):
    """Host arrays for an indexer workload: q [B, T, H, d], w [B, T, H], k [B, S, d]
    (+ k_scale [B, S] for fp8 keys), nv [B*T] or None."""
    B, T, S, H, d, seed = sp["B"], sp["T"], sp["S"], sp["H"], sp["d"], sp["seed"]
    out = {}
    if sp["q"] == "f32":
        out["q"] = normal_f32(seed, TID_Q, (B, T, H, d), sp["q_scale"])
    else:
        out["q"] = normal_bf16(seed, TID_Q, (B, T, H, d), sp["q_scale"])
    if sp["w"] == "uniform":
        out["w"] = uniform_f32(seed, TID_W, (B, T, H), 0.0, 1.0)
    else:
        out["w"] = normal_f32(seed, TID_W, (B, T, H), 1.0)
    if sp["key"] == "f32":
        out["k"] = normal_f32(seed, TID_K, (B, S, d), 1.0)
        out["k_scale"] = None
    elif sp["key"] == "bf16":
        out["k"] = normal_bf16(seed, TID_K, (B, S, d), 1.0)
        out["k_scale"] = None
    else:
        codes, scales = fp8_rows(seed, TID_K, B * S, d, 1.0)
        out["k"] = codes.reshape(B, S, d)
        out["k_scale"] = scales.reshape(B, S)
    out["nv"] = np.tile(causal_nv(S, T), B) if sp.get("causal") else None
    return out


def projection(sp):
    """The fixed Gaussian projection P [dc, d], entries N(0, 1/dc), fp32."""
    return normal_f32(sp["seed"], TID_P, (sp["dc"], sp["d"]), 1.0 / math.sqrt(sp["dc"]))


def compact_inputs(sp):
    """q [B, H, d] bf16, w [B, H], full keys [B, S, d] bf16, P [dc, d], compact keys
    c [B, S, dc] int8 with scales cs [B, S]."""
    B, S, H, d, seed = sp["B"], sp["S"], sp["H"], sp["d"], sp["seed"]
    q = normal_bf16(seed, TID_Q, (B, H, d), sp["q_scale"])
    w = uniform_f32(seed, TID_W, (B, H), 0.0, 1.0)
    k_full = normal_bf16(seed, TID_K, (B, S, d), 1.0)
    P = projection(sp)
    c, cs = compact_keys(k_full, P)
    return {"q": q, "w": w, "k_full": k_full, "P": P, "c": c, "cs": cs}


def attn_query(sp):
    """Attention queries [B, Hq, dqk] bf16, N(0, 1)."""
    return normal_bf16(sp["seed"], TID_QATT, (sp["B"], sp["Hq"], sp["dqk"]), 1.0)


def latent_seq(sp, b, out=None):
    """Latent rows of sequence b: [S, dqk] bf16, N(0, 1)."""
    S, dqk = sp["S"], sp["dqk"]
    return normal_bf16(sp["seed"], TID_LATENT, (S, dqk), 1.0, off=b * S * dqk, out=out)


def latent_rows(sp, idx):
    """Rows kv[b, idx[b, i]] for idx [B, k] (entries < 0 give zero rows): [B, k, dqk]."""
    B, k = idx.shape
    S, dqk = sp["S"], sp["dqk"]
    flat = (np.arange(B, dtype=np.int64)[:, None] * S + np.maximum(idx, 0)).reshape(-1)
    rows = normal_bf16_rows(sp["seed"], TID_LATENT, flat, dqk, 1.0).reshape(B, k, dqk)
    rows[idx < 0] = 0
    return rows


def pooled_inputs(sp):
    """q [B, T, H, d] bf16, w [B, T, H], token keys [B, L, d] bf16 N(0, 1) (the
    pooled cache is written from these)."""
    B, T, L, H, d, seed = sp["B"], sp["T"], sp["L"], sp["H"], sp["d"], sp["seed"]
    q = normal_bf16(seed, TID_Q, (B, T, H, d), sp["q_scale"])
    w = uniform_f32(seed, TID_W, (B, T, H), 0.0, 1.0)
    k = normal_bf16(seed, TID_K, (B, L, d), 1.0)
    return {"q": q, "w": w, "k_tokens": k}


def pq_inputs(sp):
    """q [B, H, d] bf16, w [B, H], full keys [B, S, d] bf16 N(0, 1), the codebook cb
    [d/4, 256, 4] int8 + sigma trained on every pq_train_stride-th key of the
    workload, and the keys' codes [B, S, d/4]."""
    B, S, H, d, seed = sp["B"], sp["S"], sp["H"], sp["d"], sp["seed"]
    q = normal_bf16(seed, TID_Q, (B, H, d), sp["q_scale"])
    w = uniform_f32(seed, TID_W, (B, H), 0.0, 1.0)
    k_full = normal_bf16(seed, TID_K, (B, S, d), 1.0)
    sample = np.ascontiguousarray(k_full.reshape(-1, d)[::sp.get("pq_train_stride", 64)])
    cb, sigma = pq_codebook(sample, seed, sp.get("pq_iters", 8))
    codes = pq_encode(k_full, cb, sigma)
    return {"q": q, "w": w, "k_full": k_full, "cb": cb, "sigma": sigma, "codes": codes}


def layer_stream_inputs(sp, out_keys=None, out_kv=None):
    """Per-layer chunk queries q [L, T, H, d] bf16 and weights w [L, T, H], the
    layers' indexer keys [L, S, d] bf16 N(0, 1) and compressed KV rows [L, S, kv_row]
    (opaque bytes on this path: seeded uniform bytes), and nv [T] (causal).
    out_keys / out_kv: preallocated (e.g. pinned) arrays to fill."""
    L, T, S, H, d, seed = sp["L"], sp["T"], sp["S"], sp["H"], sp["d"], sp["seed"]
    q = normal_bf16(seed, TID_Q, (L, T, H, d), sp["q_scale"])
    w = uniform_f32(seed, TID_W, (L, T, H), 0.0, 1.0)
    keys = normal_bf16(seed, TID_K, (L, S, d), 1.0, out=out_keys)
    kv = out_kv if out_kv is not None else np.empty((L, S, sp["kv_row"]), np.uint8)
    rng = np.random.default_rng(seed)
    for l in range(L):
        kv[l] = rng.integers(0, 256, (S, sp["kv_row"]), dtype=np.uint8)
    return {"q": q, "w": w, "keys": keys, "kv": kv, "nv": causal_nv(S, T)}

