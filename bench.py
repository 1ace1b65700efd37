"""Benchmark of the lightning-indexer hot path on one MI355X.

Main line (the JSON `value`): batched decode selection, 16 sequences x 131072 fp8
keys (128 B + a 4 B scale each), 64 bf16 query heads, top-512 per sequence.  One
step = li_indexer_score + li_topk_select over one batch (the decode hot path:
scoring, then selection).  value = keys scored and selected per second
(B * S / step time).  Inputs are resident in HBM before timing starts; the
step rotates over input replicas totalling > 1 GiB so the 256 MB MALL cannot serve
the key stream from cache.

roofline: the scoring kernel, timed with HIP events on the stream it runs on,
against 132 algorithmic bytes per key and the 8 TB/s HBM peak.
cpu_baseline: the fp64 oracle on a bounded sample of the same workload.
secondary: the other workloads (prefill chunk, compact search, select-and-attend),
each timed the same way, reported beside the main line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--main-only]
       python bench.py --workload prefill_chunk|compact_search|select_attend [--steps K]
         (one secondary workload alone, e.g. under a profiler; prints its own JSON line)
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
KEY_BYTES = 132                # 128 fp8 + 4 B scale per indexer key
FLOP_PER_KEY_PER_HEAD = 2 * 128
METRIC = "decode indexer keys scored/s (% HBM peak); prefill indexer TFLOP/s (% MFMA)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(torch, a, kind=None):
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if kind == "fp8":
        return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(a).cuda()


def timed(torch, fn, steps, warmup, inner_events=None):
    """Run fn(i) warmup times, then time `steps` calls; returns (total ms, per-call
    event ms list of the inner region if fn records into inner_events)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    if inner_events is not None:
        inner_events.clear()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def source_sha(rels):
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# HBM traffic of the decode scoring kernel from rocprofv3 PMC runs of this
# benchmark's launch configuration (FETCH_SIZE and WRITE_SIZE, KiB per dispatch,
# each scaled by what the same counter reads for a plain 1 GiB copy: FETCH x2.0,
# WRITE x1.0).  Valid only for the kernel source it was taken on.
SCORE_TRAFFIC = {"sources": ["lightning_indexer_top_amd/csrc/score.hip", "lightning_indexer_top_amd/csrc/common.h"],
                 "sha256_16": "689a15c7e3667b7b", "fetch_kib": 136262.3 * 2.0, "write_kib": 8192.0 * 1.0}


def bench_decode(torch, li, workloads, steps, warmup):
    sp = workloads.spec("batched_decode")
    B, S, H, k = sp["B"], sp["S"], sp["H"], sp["topk"]
    log(f"[decode] generating inputs B={B} S={S} H={H}")
    x = workloads.indexer_inputs(sp)
    q, w = to_dev(torch, x["q"], "bf16"), to_dev(torch, x["w"])
    bytes_one = x["k"].nbytes + x["k_scale"].nbytes
    n_rep = max(2, int(math.ceil(1.1e9 / bytes_one)))
    keys = [to_dev(torch, x["k"], "fp8") for _ in range(n_rep)]
    scales = [to_dev(torch, x["k_scale"]) for _ in range(n_rep)]
    scores = torch.empty((B, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    val = torch.empty((B, k), dtype=torch.float32, device="cuda")
    L = li.lib()
    ws_n = L.li_topk_workspace_bytes(B, S, k)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # C-ABI calls with pre-built arguments: a few microseconds of host time per
    # step, so the GPU queue never drains and the events bracket kernels only
    score_args = [(_p(q), li.LI_BF16, _p(w), _p(keys[r]), li.LI_FP8_E4M3, _p(scales[r]), None, B, 1, S, H, 128,
                   _p(scores), stream) for r in range(n_rep)]
    topk_args = (_p(scores), None, B, S, k, _p(idx), _p(val), _p(ws), ctypes.c_size_t(ws_n), stream)
    ev = []

    def step(i):
        r = i % n_rep
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st = L.li_indexer_score(*score_args[r])
        e1.record()
        st |= L.li_topk_select(*topk_args)
        if st:
            raise RuntimeError(L.li_last_error().decode())
        ev.append((e0, e1))

    total_ms = timed(torch, step, steps, warmup, ev)
    score_in_step_ms = float(np.mean([a.elapsed_time(b) for a, b in ev[-steps:]]))
    ms = total_ms / steps
    # the scoring kernel's average launch duration: HIP events on its stream around
    # a burst of back-to-back launches (events around a single launch also count
    # its dispatch), same arguments and replica rotation as the steps
    burst = max(steps, 20)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(burst):
        if L.li_indexer_score(*score_args[i % n_rep]):
            raise RuntimeError(L.li_last_error().decode())
    e1.record()
    torch.cuda.synchronize()
    score_ms = e0.elapsed_time(e1) / burst
    n_keys = B * S
    achieved = n_keys * KEY_BYTES / (score_ms * 1e-3) / 1e9
    traffic = None
    if SCORE_TRAFFIC["sha256_16"] == source_sha(SCORE_TRAFFIC["sources"]) and SCORE_TRAFFIC["fetch_kib"]:
        traffic = round((SCORE_TRAFFIC["fetch_kib"] + SCORE_TRAFFIC["write_kib"]) * 1024)
    log(f"[decode] step {ms * 1e3:.1f} us, score kernel {score_ms * 1e3:.1f} us ({score_in_step_ms * 1e3:.1f} us "
        f"between the step's events) -> {achieved:.0f} GB/s")
    # the same step through the fused entry point (li_indexer_topk: the scoring
    # kernel lists candidates above a sampled threshold, one exact pass selects)
    fws_n = L.li_indexer_topk_workspace_bytes(B, 1, S, H, k)
    fws = torch.zeros(fws_n, dtype=torch.uint8, device="cuda")
    fused_args = [(_p(q), li.LI_BF16, _p(w), _p(keys[r]), li.LI_FP8_E4M3, _p(scales[r]), None, B, 1, S, H, 128, k,
                   _p(idx), _p(val), _p(fws), ctypes.c_size_t(fws_n), stream) for r in range(n_rep)]

    def fstep(i):
        if L.li_indexer_topk(*fused_args[i % n_rep]):
            raise RuntimeError(L.li_last_error().decode())

    fused_ms = timed(torch, fstep, steps, warmup) / steps
    log(f"[decode] fused step {fused_ms * 1e3:.1f} us")
    return {
        "ms": ms, "score_ms": score_ms, "score_in_step_ms": score_in_step_ms, "keys": n_keys, "replicas": n_rep,
        "fused_ms": fused_ms,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "score_stream_kernel (fp8 keys, 64 heads)",
                     "algorithmic_bytes_per_launch": n_keys * KEY_BYTES,
                     "kernel_us": round(score_ms * 1e3, 2), "kernel_us_in_step": round(score_in_step_ms * 1e3, 2)},
        "x": x, "sp": sp,
    }


def copy_bandwidth_gbs(torch, nbytes=1 << 30, reps=5):
    """Measured HBM ceiling beside the datasheet peak: a plain 1 GiB device copy
    (bytes read plus bytes written over its time), best of a few repetitions."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None or t < best else best
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / best / 1e9


def cpu_baseline_decode(x, sp):
    """Oracle (fp64, C, one thread per row) on the whole decode workload: score
    every key of every sequence, then the top-k of each row."""
    import oracle
    B = sp["B"]
    t0 = time.perf_counter()
    sc = oracle.indexer_score(x["q"], oracle.BF16, x["w"], x["k"], oracle.FP8_E4M3, x["k_scale"])
    oracle.topk(sc, sp["topk"])
    dt = time.perf_counter() - t0
    return {"value": round(B * sp["S"] / dt, 1), "unit": "keys/s", "cores": oracle.threads_used(), "kind": "oracle",
            "sample": f"the whole workload: {B} sequences x {sp['S']} keys (score + top-{sp['topk']}), {dt:.1f} s"}


def bench_prefill(torch, li, workloads, steps, warmup):
    sp = workloads.spec("prefill_chunk")
    B, T, S, H, k = sp["B"], sp["T"], sp["S"], sp["H"], sp["topk"]
    log(f"[prefill] generating inputs T={T} S={S} H={H}")
    x = workloads.indexer_inputs(sp)
    q, w, kk, nv = to_dev(torch, x["q"], "bf16"), to_dev(torch, x["w"]), to_dev(torch, x["k"], "bf16"), \
        to_dev(torch, x["nv"])
    ws = torch.empty(li.indexer_topk_workspace_bytes(B, T, S, H, k), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B * T, k), dtype=torch.int32, device="cuda")
    ev = []

    def step(i):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        li.indexer_topk(q, w, kk, k, None, nv, with_values=False, workspace=ws, out=(idx, None))
        e1.record()
        ev.append((e0, e1))

    timed(torch, step, steps, warmup, ev)
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev[-steps:]]))
    flop = float(x["nv"].astype(np.int64).sum()) * H * FLOP_PER_KEY_PER_HEAD
    tf = flop / (ms * 1e-3) / 1e12
    # the same contraction without selection: li_indexer_score writes all 2 GiB of scores
    scores = torch.empty((B * T, S), dtype=torch.float32, device="cuda")
    ev2 = []

    def step2(i):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        li.indexer_score(q, w, kk, None, nv, out=scores)
        e1.record()
        ev2.append((e0, e1))

    timed(torch, step2, max(3, steps // 2), 1, ev2)
    ms2 = float(np.mean([a.elapsed_time(b) for a, b in ev2[-max(3, steps // 2):]]))
    tf2 = flop / (ms2 * 1e-3) / 1e12
    del scores
    log(f"[prefill] fused {ms:.2f} ms -> {tf:.1f} TFLOP/s; scores only {ms2:.2f} ms -> {tf2:.1f} TFLOP/s")
    return {"workload": "prefill_chunk T=4096 S=131072 H=64 bf16 causal top-512", "ms": round(ms, 4),
            "value": round(tf, 2), "unit": "TFLOP/s", "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "flop": flop, "unfused_score_ms": round(ms2, 4), "unfused_score_tflops": round(tf2, 2),
            "unfused_frac_bf16_peak": round(tf2 / BF16_PEAK_TFLOPS, 4)}


def bench_compact(torch, li, workloads, steps, warmup):
    sp = workloads.spec("compact_search")
    B, S, H, m, k = sp["B"], sp["S"], sp["H"], sp["m"], sp["topk"]
    log(f"[compact] generating inputs B={B} S={S}")
    x = workloads.compact_inputs(sp)
    d = dict(q=to_dev(torch, x["q"], "bf16"), w=to_dev(torch, x["w"]), P=to_dev(torch, x["P"]),
             c=to_dev(torch, x["c"]), cs=to_dev(torch, x["cs"]), kf=to_dev(torch, x["k_full"], "bf16"))
    ws = torch.empty(li.compact_workspace_bytes(B, S, H, m, k), dtype=torch.uint8, device="cuda")
    sl = torch.empty((B, m), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    val = torch.empty((B, k), dtype=torch.float64, device="cuda")
    ev = []

    def step(i):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        li.compact_search_rerank(d["q"], d["w"], d["P"], d["c"], d["cs"], d["kf"], m, k, workspace=ws,
                                 out=(sl, idx, val))
        e1.record()
        ev.append((e0, e1))

    timed(torch, step, steps, warmup, ev)
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev[-steps:]]))
    # recall@k of the two-stage result against exact scoring of the full keys (GPU),
    # and the exact scan's own time on the same data (every bf16 key read: 1.07 GB)
    q4 = d["q"].reshape(B, 1, H, 128)
    w3 = d["w"].reshape(B, 1, H)
    ex_idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ex_ws = torch.zeros(li.lib().li_indexer_topk_workspace_bytes(B, 1, S, H, k), dtype=torch.uint8, device="cuda")
    ev2 = []

    def exact(i):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        li.indexer_topk(q4, w3, d["kf"], k, with_values=False, workspace=ex_ws, out=(ex_idx, None))
        e1.record()
        ev2.append((e0, e1))

    timed(torch, exact, steps, warmup, ev2)
    exact_ms = float(np.mean([a.elapsed_time(b) for a, b in ev2[-steps:]]))
    torch.cuda.synchronize()
    a, b = idx.cpu().numpy(), ex_idx.cpu().numpy()
    recall = float(np.mean([len(np.intersect1d(a[i], b[i])) / k for i in range(B)]))
    stage1_bytes = B * S * 36
    stage2_bytes = B * m * 256
    gbs = (stage1_bytes + stage2_bytes) / (ms * 1e-3) / 1e9
    log(f"[compact] {ms * 1e3:.1f} us, {gbs:.0f} GB/s algorithmic, recall@{k} {recall:.4f}; "
        f"exact scan {exact_ms * 1e3:.1f} us")
    return {"workload": "compact_search B=32 S=131072 int8 32-d shortlist 2048 -> top-512", "ms": round(ms, 4),
            "value": round(B * S / (ms * 1e-3), 1), "unit": "keys/s", "gbs_algorithmic": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "recall_at_512_vs_exact": round(recall, 4),
            "exact_scan_ms": round(exact_ms, 4),
            "exact_scan_gbs": round(B * S * 256 / (exact_ms * 1e-3) / 1e9, 1)}


def bench_select_attend(torch, li, workloads, steps, warmup):
    sp = workloads.spec("select_attend")
    B, S, H, k, Hq = sp["B"], sp["S"], sp["H"], sp["topk"], sp["Hq"]
    log(f"[select_attend] generating indexer inputs B={B} S={S}")
    x = workloads.indexer_inputs(sp)
    q, w, kk, ks = to_dev(torch, x["q"], "bf16"), to_dev(torch, x["w"]), to_dev(torch, x["k"], "fp8"), \
        to_dev(torch, x["k_scale"])
    del x
    log("[select_attend] generating the 576-d latent (18 GiB) sequence by sequence")
    lat = torch.empty((B, S, sp["dqk"]), dtype=torch.bfloat16, device="cuda")
    buf = np.empty((S, sp["dqk"]), np.uint16)
    for b in range(B):
        workloads.latent_seq(sp, b, out=buf)
        lat[b].copy_(torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16))
        if (b + 1) % 16 == 0:
            log(f"[select_attend] {b + 1} of {B} sequences written")
    qa = to_dev(torch, workloads.attn_query(sp), "bf16")
    scores = torch.empty((B, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, sp["dv"]), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    sel_ws = torch.empty(max(1, li.topk_workspace_bytes(B, S, k)), dtype=torch.uint8, device="cuda")
    sel_idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ev = []

    def step(i):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        li.indexer_score(q, w, kk, ks, None, out=scores)
        e[1].record()
        li.topk_select(scores, k, with_values=False, workspace=sel_ws, out=(sel_idx, None))
        e[2].record()
        li.sparse_attn_gather(qa, lat, idx, sp["tau"], out=(out, lse))
        e[3].record()
        ev.append(e)

    # the selection feeds the attention: compute it once so idx is a real top-k
    r_idx, _ = li.topk_select(li.indexer_score(q, w, kk, ks), k, with_values=False)
    idx.copy_(r_idx)
    timed(torch, step, steps, warmup, ev)
    t = np.array([[a.elapsed_time(b) for a, b in zip(e[:-1], e[1:])] for e in ev[-steps:]]).mean(0)
    score_ms, sel_ms, attn_ms = [float(v) for v in t]
    gather_bytes = B * k * sp["dqk"] * 2 + B * Hq * sp["dqk"] * 2 + B * Hq * sp["dv"] * 2
    attn_flop = B * Hq * k * (sp["dqk"] + sp["dv"]) * 2
    res = {
        "workload": "select_attend B=64 S=262144 fp8 indexer top-512 + 128-head attention over 576-d rows",
        "ms": round(score_ms + sel_ms + attn_ms, 4),
        "indexer_keys_per_s": round(B * S / (score_ms * 1e-3), 1),
        "indexer_frac_hbm": round(B * S * KEY_BYTES / (score_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "select_ms": round(sel_ms, 4),
        "attn_ms": round(attn_ms, 4),
        "attn_gbs": round(gather_bytes / (attn_ms * 1e-3) / 1e9, 1),
        "attn_tflops": round(attn_flop / (attn_ms * 1e-3) / 1e12, 2),
    }
    log(f"[select_attend] score {score_ms * 1e3:.1f} us, select {sel_ms * 1e3:.1f} us, attn {attn_ms * 1e3:.1f} us")
    del lat
    return res


SECONDARY = {"prefill_chunk": bench_prefill, "compact_search": bench_compact, "select_attend": bench_select_attend}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--main-only", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run four plain 1 GiB device copies (calibrates the HBM byte counters)")
    ap.add_argument("--workload", choices=sorted(SECONDARY), default=None,
                    help="only time this secondary workload and print its result")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the hot path is not sharded across "
              "GPUs in this library", file=sys.stderr)
        sys.exit(2)

    import torch
    import lightning_indexer_top_amd as li
    from synth import workloads

    if not os.path.exists(li.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    li.lib()
    torch.cuda.init()
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 1 << 30, "copies": 4}))
        return
    if args.workload:
        res = SECONDARY[args.workload](torch, li, workloads, args.steps, args.warmup)
        print(json.dumps(dict(res, steps=args.steps, warmup=args.warmup)), flush=True)
        return
    dec = bench_decode(torch, li, workloads, args.steps, args.warmup)
    ms = dec["ms"]
    copy_gbs = copy_bandwidth_gbs(torch)
    dec["roofline"]["measured_copy_gbs"] = round(copy_gbs, 1)
    dec["roofline"]["frac_of_measured_copy"] = round(dec["roofline"]["achieved"] / copy_gbs, 4)
    log(f"[decode] plain 1 GiB device copy: {copy_gbs:.0f} GB/s (read + write)")
    result = {
        "metric": METRIC,
        "value": round(dec["keys"] / (ms * 1e-3), 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "batched_decode", "sequences": 16, "keys_per_sequence": 131072, "heads": 64,
                   "dim": 128, "key_format": "fp8 e4m3 + fp32 scale", "topk": 512,
                   "step": "indexer_score + topk_select", "input_replicas": dec["replicas"]},
        "roofline": dec["roofline"],
        # the scoring kernel alone (keys scored per second over its own duration)
        "score_keys_per_s": round(dec["keys"] / (dec["score_ms"] * 1e-3), 1),
        "score_frac_hbm": dec["roofline"]["frac"],
        # the same step through li_indexer_topk (scoring kernel with a selection epilogue)
        "fused_step_ms": round(dec["fused_ms"], 5),
        "fused_step_keys_per_s": round(dec["keys"] / (dec["fused_ms"] * 1e-3), 1),
    }
    if not args.no_cpu:
        log("[cpu] timing the oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline_decode(dec["x"], dec["sp"])
    del dec
    if not args.main_only:
        sec = {}
        for name, fn in SECONDARY.items():
            try:
                sec[name] = fn(torch, li, workloads, max(3, args.steps // 2), 2)
            except Exception as e:  # report, keep the main line
                sec[name] = {"error": repr(e)}
            torch.cuda.empty_cache()
        result["secondary"] = sec
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
