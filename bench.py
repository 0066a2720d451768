#!/usr/bin/env python
"""Benchmark of the grouped-query attention hot path on one MI355X.

One step is one pass over every stage of the path on the two headline
workloads, with all inputs resident in HBM:

  1. gqa_rope_table     rotary tables, D = 128, theta = 500000, 8192 positions
  2. gqa_rope_write_kv  rope + paged KV write of 64 new tokens (Llama-3.1-8B
                        shapes, page table into a 9000-page pool)
  3. gqa_decode_paged   paged decode, 64 rows, context lengths U[512, 8192]
  4. gqa_rope_write_kv  rope + KV write of 16384 packed tokens (cache row =
                        segment)
  5. gqa_prefill_packed packed prefill, 16384 tokens, segments U[64, 4096]:
                        its plan (gqa_prefill_packed_plan, from positions and
                        segments only) on a second stream during stages 1-4,
                        then gqa_prefill_packed_planned

Each stage is bracketed by HIP events on the stream it is launched on. The
JSON line reports the paged-decode KV bandwidth as `value` (GB/s), the
packed-prefill throughput (TFLOP/s), both against the MI355X peaks, the
oracle timed on the host cores on a bounded sample, and the per-stage times.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged GQA decode KV GB/s + packed prefill TFLOP/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
SEED_DECODE, SEED_PREFILL, SEED_CHUNKED, SEED_QKV = 3, 4, 6, 7


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the absolute numbers of the three other workload configurations")
    ap.add_argument("--cpu-sample-rows", type=int, default=64)
    ap.add_argument("--cpu-sample-queries", type=int, default=8192)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch's copy kernel), for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


def other_configs(gqa, W, torch, np, stream, reps):
    """Absolute numbers for the three other workload configurations (tiny
    Llama example, GPT-2 f32 decode_rows, gpt-oss SinkAttention): each step
    of the path timed with HIP events on the library's stream, inputs
    resident in HBM. Context beside the benchmark line, not part of it."""
    dev, bf16, f32 = "cuda", torch.bfloat16, torch.float32
    CONTIG = gqa.GQA_CACHE_CONTIGUOUS

    def ev_time(fn, n_rep):
        """Mean microseconds per call over n_rep back-to-back calls (after
        warm-up calls), bracketed by one pair of events."""
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_rep):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n_rep

    def graph_time(fn, result, inputs, n_rep=20):
        """Mean microseconds per replay of fn captured in a HIP graph (no host
        launch cost), or None if a replay's result differs from the eager one
        (three replays, checked bit for bit, with host synchronization between).
        fn rotates q and k in place, so `inputs` are restored before the eager
        reference and before each checked replay."""
        saved = [x.clone() for x in inputs]

        def restore():
            for x, x0 in zip(inputs, saved):
                x.copy_(x0)

        restore()
        fn()
        torch.cuda.synchronize()
        ref = result.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        for _ in range(3):
            restore()
            result.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(result.view(torch.int16), ref.view(torch.int16)):
                return None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs = torch.cuda.current_stream()
        e0.record(gs)
        for _ in range(n_rep):
            graph.replay()
        e1.record(gs)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n_rep

    out = {}
    # ---- tiny Llama example: prefill S=128 then 16 decode steps, MaxSeq 512 ----
    wl = W.TINY_LLAMA
    H, KVH, D, S, NS, MS = wl.heads, wl.kv_heads, wl.head_dim, wl.extra["prefill"], \
        wl.extra["decode_steps"], wl.extra["max_seq"]
    n = S + NS
    q = W.device_normal((n, H, D), 1, "q", bf16)
    k = W.device_normal((n, KVH, D), 1, "k", bf16)
    v = W.device_normal((n, KVH, D), 1, "v", bf16)
    pos = torch.arange(n, dtype=torch.int32, device=dev)
    seg = torch.zeros(S, dtype=torch.int32, device=dev)
    rows = torch.zeros(n, dtype=torch.int32, device=dev)
    tab = torch.empty((2, MS, D // 2), dtype=bf16, device=dev)
    ck = torch.zeros((1, KVH, MS, D), dtype=bf16, device=dev)
    cv = torch.zeros_like(ck)
    o_p = torch.empty((S, H, D), dtype=bf16, device=dev)
    o_d = torch.empty((1, H, D), dtype=bf16, device=dev)
    nbp = gqa.gqa_prefill_packed_workspace(S, H, KVH, D)
    wsp = torch.empty(max(nbp, 256), dtype=torch.uint8, device=dev)
    nbd = gqa.gqa_decode_rows_workspace(1, H, KVH, D, MS)
    wsd = torch.empty(max(nbd, 256), dtype=torch.uint8, device=dev)
    gqa.gqa_rope_table(D, MS, wl.theta, gqa.GQA_BF16, tab)

    def tiny_prefill():
        gqa.gqa_rope_write_kv(S, H, KVH, D, gqa.GQA_BF16, q[:S], k[:S], v[:S], pos[:S], tab, MS,
                              CONTIG, ck, cv, 1, MS, rows[:S], None, None, 0, 0)
        gqa.gqa_prefill_packed(S, H, KVH, D, gqa.GQA_BF16, 0.0, 0, None, q[:S], k[:S], v[:S],
                               pos[:S], seg, o_p, wsp, nbp)

    def tiny_decode():
        for i in range(S, n):
            gqa.gqa_rope_write_kv(1, H, KVH, D, gqa.GQA_BF16, q[i:i + 1], k[i:i + 1], v[i:i + 1],
                                  pos[i:i + 1], tab, MS, CONTIG, ck, cv, 1, MS, rows[i:i + 1],
                                  None, None, 0, 0)
            gqa.gqa_decode_rows(1, H, KVH, D, gqa.GQA_BF16, 0.0, 0, None, q[i:i + 1], ck, cv, MS,
                                pos[i:i + 1], o_d, wsd, nbd)

    t_p = ev_time(tiny_prefill, reps)
    t_d = ev_time(tiny_decode, reps)
    t_dg = graph_time(tiny_decode, o_d, [q, k])
    dec_bytes = sum((p_ + 1) * KVH * D * 2 * 2 for p_ in range(S, n))
    out["tiny_llama"] = {
        "workload": wl.name, "prefill_us": t_p, "prefill_flops": 4 * D * H * S * (S + 1) // 2,
        "prefill_tflops": 4 * D * H * S * (S + 1) // 2 / t_p / 1e6,
        "decode_us_per_step": t_d / NS, "decode_kv_bytes_per_step": dec_bytes // NS,
        "decode_gbs": dec_bytes / t_d / 1e3,
        "decode_us_per_step_graph": None if t_dg is None else t_dg / NS,
        "decode_gbs_graph": None if t_dg is None else dec_bytes / t_dg / 1e3,
        "note": "prefill = rope + KV write + attention; a decode step = rope + KV write + "
                "decode_rows of one token, launched from Python (host-bound) and, in "
                "decode_us_per_step_graph, replayed from a HIP graph of the 16 steps"}
    del q, k, v, ck, cv

    # ---- GPT-2 MHA decode_rows, f32, Batch 32, cache [32, 12, 1024, 64] ----
    wl = W.GPT2_DECODE_ROWS
    H, KVH, D, B, MS = wl.heads, wl.kv_heads, wl.head_dim, wl.extra["batch"], wl.extra["max_seq"]
    g = W.streams(2)
    dpos = W.uniform_positions(B, 0, MS - 1, g["extra"])
    d_pos = torch.from_numpy(dpos).to(dev)
    # The K + V working set (~100 MB attended, 201 MB allocated) fits the
    # 256 MB Infinity Cache: six cache copies rotate so each call reads HBM.
    copies = [(W.device_normal((B, KVH, MS, D), 2, "pool_k", f32) + c,
               W.device_normal((B, KVH, MS, D), 2, "pool_v", f32) + c) for c in range(6)]
    q2 = W.device_normal((B, H, D), 2, "q", f32)
    o2 = torch.empty((B, H, D), dtype=f32, device=dev)
    nb2 = gqa.gqa_decode_rows_workspace(B, H, KVH, D, MS)
    ws2 = torch.empty(max(nb2, 256), dtype=torch.uint8, device=dev)
    it = [0]

    def gpt2_decode():
        ck_, cv_ = copies[it[0] % len(copies)]
        it[0] += 1
        gqa.gqa_decode_rows(B, H, KVH, D, gqa.GQA_F32, 0.0, 0, None, q2, ck_, cv_, MS, d_pos, o2,
                            ws2, nb2)

    t2 = ev_time(gpt2_decode, 10 * len(copies))
    b2 = int(np.sum(dpos.astype(np.int64) + 1)) * KVH * D * 4 * 2 + 2 * B * H * D * 4
    out["gpt2_decode_rows_f32"] = {
        "workload": wl.name, "avg_us": t2, "algorithmic_bytes": b2, "gbs": b2 / t2 / 1e3,
        "frac_of_hbm_peak": b2 / t2 / 1e3 / HBM_PEAK_GBS,
        "note": "six cache copies rotate between calls (the working set would otherwise be "
                "served by the Infinity Cache)"}
    del copies

    # ---- gpt-oss-20b SinkAttention: prefill 4096 + 256 decode steps, W 128 / full ----
    wl = W.GPT_OSS_SINK
    H, KVH, D, S, NS, MS = wl.heads, wl.kv_heads, wl.head_dim, wl.extra["prefill"], \
        wl.extra["decode_steps"], wl.extra["max_seq"]
    n = S + NS
    tab5 = torch.empty((2, MS, D // 2), dtype=bf16, device=dev)
    gqa.gqa_rope_table(D, MS, wl.theta, gqa.GQA_BF16, tab5)
    pos5 = torch.arange(n, dtype=torch.int32, device=dev)
    seg5 = torch.zeros(S, dtype=torch.int32, device=dev)
    rows5 = torch.zeros(n, dtype=torch.int32, device=dev)
    nbp5 = gqa.gqa_prefill_packed_workspace(S, H, KVH, D)
    wsp5 = torch.empty(max(nbp5, 256), dtype=torch.uint8, device=dev)
    nbd5 = gqa.gqa_decode_rows_workspace(1, H, KVH, D, MS)
    wsd5 = torch.empty(max(nbd5, 256), dtype=torch.uint8, device=dev)
    for layer, win in enumerate(wl.extra["windows"]):
        q = W.device_normal((n, H, D), 5, "q", bf16)
        k = W.device_normal((n, KVH, D), 5, "k", bf16)
        v = W.device_normal((n, KVH, D), 5, "v", bf16)
        sinks = W.device_normal((H,), 5 + layer, "sinks", bf16)
        ck = torch.zeros((1, KVH, MS, D), dtype=bf16, device=dev)
        cv = torch.zeros_like(ck)
        o_p = torch.empty((S, H, D), dtype=bf16, device=dev)
        o_d = torch.empty((1, H, D), dtype=bf16, device=dev)

        def oss_prefill():
            gqa.gqa_rope_write_kv(S, H, KVH, D, gqa.GQA_BF16, q[:S], k[:S], v[:S], pos5[:S], tab5,
                                  MS, CONTIG, ck, cv, 1, MS, rows5[:S], None, None, 0, 0)
            gqa.gqa_prefill_packed(S, H, KVH, D, gqa.GQA_BF16, 0.0, win, sinks, q[:S], k[:S], v[:S],
                                   pos5[:S], seg5, o_p, wsp5, nbp5)

        def oss_attn_only():
            gqa.gqa_prefill_packed(S, H, KVH, D, gqa.GQA_BF16, 0.0, win, sinks, q[:S], k[:S], v[:S],
                                   pos5[:S], seg5, o_p, wsp5, nbp5)

        def oss_decode():
            for i in range(S, n):
                gqa.gqa_rope_write_kv(1, H, KVH, D, gqa.GQA_BF16, q[i:i + 1], k[i:i + 1],
                                      v[i:i + 1], pos5[i:i + 1], tab5, MS, CONTIG, ck, cv, 1, MS,
                                      rows5[i:i + 1], None, None, 0, 0)
                gqa.gqa_decode_rows(1, H, KVH, D, gqa.GQA_BF16, 0.0, win, sinks, q[i:i + 1], ck, cv,
                                    MS, pos5[i:i + 1], o_d, wsd5, nbd5)

        t_p = ev_time(oss_prefill, reps)
        t_a = ev_time(oss_attn_only, reps)
        t_d = ev_time(oss_decode, 2)
        t_dg = graph_time(oss_decode, o_d, [q, k], 5)
        if win > 0:
            pairs = sum(min(i + 1, win) for i in range(S))
            kv = sum(min(p_ + 1, win) for p_ in range(S, n))
        else:
            pairs = S * (S + 1) // 2
            kv = sum(p_ + 1 for p_ in range(S, n))
        fl = 4 * D * H * pairs
        kvb = kv * KVH * D * 2 * 2
        out[f"gpt_oss_layer{layer}_window{win}"] = {
            "workload": f"{wl.name}: layer {layer}, window {win or 'none'}", "prefill_us": t_p,
            "attention_us": t_a, "prefill_flops": fl, "attention_tflops": fl / t_a / 1e6,
            "attention_frac_of_mfma_peak": fl / t_a / 1e6 / MFMA_BF16_PEAK_TFLOPS,
            "decode_loop_us": t_d, "decode_us_per_step": t_d / NS,
            "decode_us_per_step_graph": None if t_dg is None else t_dg / NS,
            "decode_kv_bytes_per_step": kvb // NS, "decode_gbs": kvb / t_d / 1e3,
            "decode_gbs_graph": None if t_dg is None else kvb / t_dg / 1e3,
            "note": "prefill = rope + KV write + attention (attention alone beside it); a decode "
                    "step = rope + KV write + decode_rows of one token, launched from Python "
                    "(host-bound) and, in decode_us_per_step_graph, replayed from a HIP graph "
                    "of the 256 steps"}
        del q, k, v, ck, cv
    return out


def oracle_other_configs(o, np, W, only=None):
    """The oracle on the other workload configurations, timed on this host:
    the tiny Llama example (prefill of 128 tokens, then its 16 decode steps),
    GPT-2 f32 decode_rows (all 32 rows) and the gpt-oss layer pair (the
    windowed layer's prefill whole, the full layer's on a sample of queries,
    and a sample of each layer's decode steps). Inputs are seeded draws of the
    same shapes, index layouts and positions as the GPU runs; each entry
    gives the oracle's seconds and its rate on the algorithmic work it did."""
    res = {}
    if only is None or "tiny_llama" in only:
        wl = W.TINY_LLAMA
        H, KVH, D, S, NS, MS = wl.heads, wl.kv_heads, wl.head_dim, wl.extra["prefill"], \
            wl.extra["decode_steps"], wl.extra["max_seq"]
        g = W.streams(1)
        n = S + NS
        q = W.normal(g["q"], (n, H, D)).astype(np.float64)
        k = W.normal(g["k"], (n, KVH, D)).astype(np.float64)
        v = W.normal(g["v"], (n, KVH, D)).astype(np.float64)
        pos = np.arange(n, dtype=np.int32)
        t0 = time.perf_counter()
        c, sn = o.rope_tables(MS, D, wl.theta, "bf16")
        qr = o.rope(q, pos, c, sn, "bf16")
        kr = o.rope(k, pos, c, sn, "bf16")
        o.packed(qr[:S], kr[:S], v[:S], pos[:S], np.zeros(S, np.int32))
        t_p = time.perf_counter() - t0
        cache = np.full((1, KVH, MS, D), np.nan)
        ck, cv, _ = o.write_contiguous(kr, v, pos, cache, cache.copy())
        t0 = time.perf_counter()
        for i in range(S, n):
            o.decode_rows(qr[i:i + 1], ck, cv, pos[i:i + 1])
        t_d = time.perf_counter() - t0
        fl = 4 * D * H * S * (S + 1) // 2
        db = sum((p_ + 1) * KVH * D * 2 * 2 for p_ in range(S, n))
        res["tiny_llama"] = {"seconds": t_p + t_d, "prefill_seconds": t_p, "prefill_flops": fl,
                             "prefill_gflops": fl / t_p / 1e9, "decode_seconds_16_steps": t_d,
                             "decode_gbs": db / t_d / 1e9,
                             "sample": "whole: tables + rope + prefill S=128, 16 decode steps"}
    if only is None or "gpt2_decode_rows_f32" in only:
        wl = W.GPT2_DECODE_ROWS
        H, KVH, D, B, MS = wl.heads, wl.kv_heads, wl.head_dim, wl.extra["batch"], wl.extra["max_seq"]
        g = W.streams(2)
        dpos = W.uniform_positions(B, 0, MS - 1, g["extra"])
        ck = W.normal(g["pool_k"], (B, KVH, MS, D)).astype(np.float64)
        cv = W.normal(g["pool_v"], (B, KVH, MS, D)).astype(np.float64)
        q = W.normal(g["q"], (B, H, D)).astype(np.float64)
        t0 = time.perf_counter()
        o.decode_rows(q, ck, cv, dpos)
        t2 = time.perf_counter() - t0
        b2 = int(np.sum(dpos.astype(np.int64) + 1)) * KVH * D * 4 * 2 + 2 * B * H * D * 4
        res["gpt2_decode_rows_f32"] = {"seconds": t2, "algorithmic_bytes": b2, "gbs": b2 / t2 / 1e9,
                                       "sample": "whole: all 32 rows"}
    if only is None or "gpt_oss" in only:
        wl = W.GPT_OSS_SINK
        H, KVH, D, S, NS, MS = wl.heads, wl.kv_heads, wl.head_dim, wl.extra["prefill"], \
            wl.extra["decode_steps"], wl.extra["max_seq"]
        n = S + NS
        g = W.streams(5)
        q = W.normal(g["q"], (n, H, D)).astype(np.float64)
        k = W.normal(g["k"], (n, KVH, D)).astype(np.float64)
        v = W.normal(g["v"], (n, KVH, D)).astype(np.float64)
        sinks = W.normal(g["sinks"], (H,)).astype(np.float64)
        pos = np.arange(n, dtype=np.int32)
        seg = np.zeros(S, np.int32)
        cache = np.full((1, KVH, MS, D), np.nan)
        ck, cv, _ = o.write_contiguous(k, v, pos, cache, cache.copy())
        layers = {}
        secs = 0.0
        for win in wl.extra["windows"]:
            sel = None if win > 0 else np.arange(0, S, 8, dtype=np.int32)
            qs = np.arange(S) if sel is None else sel
            t0 = time.perf_counter()
            o.packed(q[:S], k[:S], v[:S], pos[:S], seg, window=win, sinks=sinks, sel=sel)
            t_p = time.perf_counter() - t0
            pairs = int(sum(min(int(i) + 1, win) if win > 0 else int(i) + 1 for i in qs))
            steps = np.arange(S, n, 8)
            t0 = time.perf_counter()
            for i in steps:
                o.decode_rows(q[i:i + 1], ck, cv, pos[i:i + 1], window=win, sinks=sinks)
            t_d = time.perf_counter() - t0
            kv = sum(min(int(p_) + 1, win) if win > 0 else int(p_) + 1 for p_ in steps)
            layers[f"window{win}"] = {
                "prefill_seconds": t_p, "prefill_gflops": 4 * D * H * pairs / t_p / 1e9,
                "prefill_sample": "all 4096 queries" if sel is None else f"{len(sel)} of {S} queries",
                "decode_seconds": t_d, "decode_gbs": kv * KVH * D * 2 * 2 / t_d / 1e9,
                "decode_sample": f"{len(steps)} of {NS} steps"}
            secs += t_p + t_d
        res["gpt_oss"] = {"seconds": secs, "layers": layers}
    return res


def gpu_clocks():
    """Current gfx (per XCD) and memory clocks in MHz from amd-smi (None if
    amd-smi is not there)."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                           text=True, timeout=20)
        if r.returncode != 0:
            return None
        data = json.loads(r.stdout)
        clk = data["gpu_data"][0]["clock"] if isinstance(data, dict) else data[0]["clock"]

        def mhz(entry):
            c = entry.get("clk") if isinstance(entry, dict) else None
            return c.get("value") if isinstance(c, dict) else None
        return {"gfx_mhz": [mhz(v) for k, v in sorted(clk.items()) if k.startswith("gfx")],
                "mem_mhz": [mhz(v) for k, v in sorted(clk.items()) if k.startswith("mem")],
                "gfx_max_mhz": next((v["max_clk"]["value"] for k, v in clk.items()
                                     if k.startswith("gfx") and isinstance(v.get("max_clk"), dict)),
                                    None)}
    except Exception:
        return None


def clocks_under_load(fn, seconds=1.5):
    """GPU clocks sampled while fn runs back to back for about `seconds`."""
    import threading
    box = {}
    t = threading.Thread(target=lambda: (time.sleep(seconds / 2), box.update(c=gpu_clocks())))
    t.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or t.is_alive():
        fn()
    t.join()
    return box.get("c")


def host_info(torch, clocks_before, clocks_prefill):
    """Versions, the host CPU and the GPU clocks around the run."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "rocm": rocm, "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "gpu": torch.cuda.get_device_name(0),
            "seeds": {"decode": SEED_DECODE, "prefill": SEED_PREFILL, "chunked": SEED_CHUNKED,
                      "qkv": SEED_QKV},
            "gpu_clocks_idle_before": clocks_before,
            "gpu_clocks_during_prefill": clocks_prefill}


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": 5}), flush=True)
    return 0


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "decoder_attention_rope_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Sources each measured kernel is built from: a committed traffic figure is
# used only while they hash as they did when the counters were taken.
DECODE_SOURCES = ["decode.hip", "decode_mfma.hip", "decode_mfma.h", "common.h"]
PREFILL_SOURCES = ["prefill.hip", "attn_tiles.h", "common.h"]
STEP_SOURCES = ["prefill.hip", "decode_mfma.h", "attn_tiles.h", "common.h"]
QKV_SOURCES = ["qkv.hip", "rope_common.h", "attn_tiles.h", "common.h"]


def traffic_for(kernel, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent or ent.get("source_sha") != source_sha(*sources):
        return None
    return ent.get("bytes_per_launch")


def main():
    args = parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path is measured on one MI355X, see DESIGN.md for how it would "
              "shard)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import decoder_attention_rope_amd as gqa
    import workloads as W

    dev = "cuda"
    bf16 = torch.bfloat16
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    clocks_before = gpu_clocks()

    # ---------------- decode workload (Llama-3.1-8B paged) ----------------
    wd = W.LLAMA8B_PAGED
    ed = wd.extra
    H, KVH, D = wd.heads, wd.kv_heads, wd.head_dim
    gi = W.streams(SEED_DECODE)
    lengths, dpos, table = W.paged_layout(ed["rows"], ed["len_lo"], ed["len_hi"],
                                          ed["num_pages"], ed["page_size"], gi["index"])
    rows, pages, num_pages = ed["rows"], table.shape[1], ed["num_pages"]
    pool_k = W.device_normal((num_pages, KVH, 64, D), SEED_DECODE, "pool_k", bf16)
    pool_v = W.device_normal((num_pages, KVH, 64, D), SEED_DECODE, "pool_v", bf16)
    dq = W.device_normal((rows, H, D), SEED_DECODE, "q", bf16)
    dk = W.device_normal((rows, KVH, D), SEED_DECODE, "k", bf16)
    dv = W.device_normal((rows, KVH, D), SEED_DECODE, "v", bf16)
    d_pos = torch.from_numpy(dpos).to(dev)
    d_table = torch.from_numpy(table).to(dev)
    d_rows = torch.arange(rows, dtype=torch.int32, device=dev)
    d_out = torch.empty((rows, H, D), dtype=bf16, device=dev)
    dws_n = gqa.gqa_decode_paged_workspace(rows, pages, H, KVH, D)
    d_ws = torch.empty(dws_n, dtype=torch.uint8, device=dev)
    theta = wd.theta
    max_pos = 8192
    rope_tab = torch.empty((2, max_pos, D // 2), dtype=bf16, device=dev)

    # ---------------- prefill workload (Llama-3.1-8B packed) ----------------
    wp = W.LLAMA8B_PACKED
    P = wp.extra["p"]
    gp = W.streams(SEED_PREFILL)
    seg_len, ppos, pseg = W.segment_layout(P, wp.extra["seg_lo"], wp.extra["seg_hi"], gp["index"])
    nseg = len(seg_len)
    pq = W.device_normal((P, H, D), SEED_PREFILL, "q", bf16)
    pk = W.device_normal((P, KVH, D), SEED_PREFILL, "k", bf16)
    pv = W.device_normal((P, KVH, D), SEED_PREFILL, "v", bf16)
    p_pos = torch.from_numpy(ppos).to(dev)
    p_seg = torch.from_numpy(pseg).to(dev)
    cache_len = int(max(seg_len))
    p_cache_k = torch.empty((nseg, KVH, cache_len, D), dtype=bf16, device=dev)
    p_cache_v = torch.empty((nseg, KVH, cache_len, D), dtype=bf16, device=dev)
    p_out = torch.empty((P, H, D), dtype=bf16, device=dev)
    pws_n = gqa.gqa_prefill_packed_workspace(P, H, KVH, D)
    p_ws = torch.empty(max(pws_n, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # Host snapshots for the CPU baseline, taken before any library call so
    # the oracle never sees data the library wrote.
    snap = None
    if not args.no_cpu_baseline:
        srows = np.arange(min(args.cpu_sample_rows, rows))
        used = sorted({int(p) for r in srows for p in table[r] if p >= 0})
        remap = {p: i for i, p in enumerate(used)}
        st = np.array([[remap.get(int(p), -1) if p >= 0 else -1 for p in table[r]]
                       for r in srows], dtype=np.int32)
        idx = torch.tensor(used, dtype=torch.long, device=dev)
        sel = W.sample_indices(P, args.cpu_sample_queries, gp["extra"])
        snap = dict(
            rows=srows, table=st,
            pk=pool_k[idx].to(torch.float64).cpu().numpy(),
            pv=pool_v[idx].to(torch.float64).cpu().numpy(),
            q=dq[torch.from_numpy(srows).to(dev)].to(torch.float64).cpu().numpy(),
            pq=pq.to(torch.float64).cpu().numpy(), pk_=pk.to(torch.float64).cpu().numpy(),
            pv_=pv.to(torch.float64).cpu().numpy(), sel=sel)

    # ---------------- one step ----------------
    names = ["rope_table", "rope_write_decode", "decode_paged", "rope_write_prefill",
             "prefill_packed"]

    # The packed prefill's plan depends only on the prefill tokens' positions
    # and segments: each step builds it on a second stream (default priority)
    # while the decode runs, after the previous step's prefill has read it,
    # and the prefill waits for it.
    side = torch.cuda.Stream()
    plan_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    plan_ms = []

    def step(ev, timing=False):
        ev[0].record(stream)
        side.wait_event(ev[0])
        with torch.cuda.stream(side):
            if timing:
                ev[6].record(side)
            gqa.gqa_prefill_packed_plan(P, H, KVH, D, 0, p_pos, p_seg, p_ws, pws_n)
            ev[7].record(side)
        gqa.gqa_rope_table(D, max_pos, theta, gqa.GQA_BF16, rope_tab)
        ev[1].record(stream)
        gqa.gqa_rope_write_kv(rows, H, KVH, D, gqa.GQA_BF16, dq, dk, dv, d_pos, rope_tab, max_pos,
                              gqa.GQA_CACHE_PAGED_TABLE, pool_k, pool_v, num_pages, 64, d_rows,
                              None, d_table, rows, pages)
        ev[2].record(stream)
        gqa.gqa_decode_paged(rows, pages, H, KVH, D, gqa.GQA_BF16, 0.0, 0, None, dq, pool_k,
                             pool_v, num_pages, d_pos, d_table, d_out, d_ws, dws_n)
        ev[3].record(stream)
        gqa.gqa_rope_write_kv(P, H, KVH, D, gqa.GQA_BF16, pq, pk, pv, p_pos, rope_tab, max_pos,
                              gqa.GQA_CACHE_CONTIGUOUS, p_cache_k, p_cache_v, nseg, cache_len,
                              p_seg, None, None, 0, 0)
        ev[4].record(stream)
        stream.wait_event(ev[7])
        gqa.gqa_prefill_packed_planned(P, H, KVH, D, gqa.GQA_BF16, 0.0, 0, None, pq, pk, pv, p_pos,
                                       p_seg, p_out, p_ws, pws_n)
        ev[5].record(stream)

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(8)]

    for _ in range(args.warmup):
        step(new_events())
    torch.cuda.synchronize()
    evs = [new_events() for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in evs:
        step(ev, timing=True)
    torch.cuda.synchronize()
    plan_us = float(np.mean([ev[6].elapsed_time(ev[7]) for ev in evs])) * 1e3
    wall = time.perf_counter() - t0
    per_op_ms = {n: float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in evs]))
                 for i, n in enumerate(names)}
    per_op_pct = {n: [float(np.percentile([ev[i].elapsed_time(ev[i + 1]) * 1e3 for ev in evs], p_))
                      for p_ in (10, 50, 90)] for i, n in enumerate(names)}
    step_ms = float(np.mean([ev[0].elapsed_time(ev[5]) for ev in evs]))

    # Measured ceilings beside the published peaks: one streaming read of the
    # decode's key pool (1.18 GB) by the library's diagnostic read kernel, and
    # a large bf16 GEMM through torch.matmul (hipBLASLt); medians, measured
    # right after the timed steps.
    xor_word = torch.zeros(gqa.GQA_DIAG_READ_BLOCKS, dtype=torch.int32, device=dev)
    pool_bytes = pool_k.numel() * pool_k.element_size()

    def timed_median(fn, n=30):
        for _ in range(5):
            fn()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(n)]
        for e0, e1 in pairs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in pairs])) * 1e-3

    rd_s = timed_median(lambda: gqa.gqa_diag_stream_read(pool_k, pool_bytes, xor_word))
    mm_n = 8192
    ma = W.device_normal((mm_n, mm_n), SEED_QKV, "q", bf16)
    mb = W.device_normal((mm_n, mm_n), SEED_QKV, "k", bf16)
    mmb_s = timed_median(lambda: ma @ mb, 10)
    ceilings = {"stream_read_gbs": pool_bytes / rd_s / 1e9, "stream_read_bytes": pool_bytes,
                "stream_read_us": rd_s * 1e6,
                "bf16_matmul_tflops": 2 * mm_n ** 3 / mmb_s / 1e12, "bf16_matmul_shape": [mm_n] * 3,
                "bf16_matmul_us": mmb_s * 1e6,
                "note": "streaming read: gqa_diag_stream_read (nontemporal 16-byte loads, grid-stride) "
                        "over the paged decode's key pool; matmul: torch.matmul of two seeded N(0,1) "
                        "bf16 matrices"}
    del ma, mb, xor_word

    def prefill_entry():
        gqa.gqa_prefill_packed(P, H, KVH, D, gqa.GQA_BF16, 0.0, 0, None, pq, pk, pv, p_pos, p_seg,
                               p_out, p_ws, pws_n)

    # The one-call entry (plan and attention on one stream), for comparison.
    entry_s = timed_median(prefill_entry, 20)

    def prefill_only():
        prefill_entry()
        torch.cuda.synchronize()
    clocks_prefill = clocks_under_load(prefill_only)

    # ---------------- next row: chunked prefill over a paged prefix ----------------
    # Timed on its own after the step (it is not part of the step): 16 rows of
    # the Llama-3.1-8B paged pool, each with a prefix of U[1024, 7168] keys and
    # a 512-token chunk whose K/V are written first.
    wc = W.LLAMA8B_CHUNKED
    ec = wc.extra
    gc = W.streams(SEED_CHUNKED)
    c_pre, c_rows, c_pos, c_table = W.chunked_layout(ec["rows"], ec["pre_lo"], ec["pre_hi"],
                                                     ec["chunk"], ec["num_pages"], 64,
                                                     gc["index"], ec["max_len"])
    cn = len(c_pos)
    c_pool_k = W.device_normal((ec["num_pages"], KVH, 64, D), SEED_CHUNKED, "pool_k", bf16)
    c_pool_v = W.device_normal((ec["num_pages"], KVH, 64, D), SEED_CHUNKED, "pool_v", bf16)
    c_q = W.device_normal((cn, H, D), SEED_CHUNKED, "q", bf16)
    c_k = W.device_normal((cn, KVH, D), SEED_CHUNKED, "k", bf16)
    c_v = W.device_normal((cn, KVH, D), SEED_CHUNKED, "v", bf16)
    c_drows = torch.from_numpy(c_rows).to(dev)
    c_dpos = torch.from_numpy(c_pos).to(dev)
    c_dtab = torch.from_numpy(c_table).to(dev)
    c_out = torch.empty((cn, H, D), dtype=bf16, device=dev)
    cws_n = gqa.gqa_prefill_cached_workspace(cn, H, KVH, D)
    c_ws = torch.empty(max(cws_n, 256), dtype=torch.uint8, device=dev)
    gqa.gqa_rope_write_kv(cn, H, KVH, D, gqa.GQA_BF16, c_q, c_k, c_v, c_dpos, rope_tab, max_pos,
                          gqa.GQA_CACHE_PAGED_TABLE, c_pool_k, c_pool_v, ec["num_pages"], 64,
                          c_drows, None, c_dtab, c_table.shape[0], c_table.shape[1])

    def chunked():
        gqa.gqa_prefill_cached(cn, H, KVH, D, gqa.GQA_BF16, 0.0, 0, None, c_q, c_drows, c_dpos,
                               gqa.GQA_CACHE_PAGED_TABLE, c_pool_k, c_pool_v, ec["num_pages"], 64,
                               c_dtab, c_table.shape[0], c_table.shape[1], c_out, c_ws, cws_n)

    for _ in range(args.warmup):
        chunked()
    c_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    for e0, e1 in c_ev:
        e0.record(stream)
        chunked()
        e1.record(stream)
    torch.cuda.synchronize()
    c_s = float(np.mean([e0.elapsed_time(e1) for e0, e1 in c_ev])) * 1e-3
    c_flops = 4 * D * H * int(np.sum(c_pos.astype(np.int64) + 1))
    c_tflops = c_flops / c_s / 1e12
    chunk_roof = {"bound": "mfma", "achieved": c_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": c_tflops / MFMA_BF16_PEAK_TFLOPS,
                  "traffic": traffic_for("prefill_cached_paged", PREFILL_SOURCES),
                  "algorithmic_flops": c_flops, "avg_us": c_s * 1e6,
                  "workload": f"{ec['rows']} rows, prefixes U[{ec['pre_lo']}, {ec['pre_hi']}] "
                              f"({int(c_pre.sum())} keys), chunk {ec['chunk']}, paged"}

    # ---------------- next row: step_paged on the same pool ----------------
    # The 16 chunks plus one decode token per row (at the chunk's last
    # position, attending the whole row) in one call.
    s_rows = ec["rows"]
    s_pos = (c_pre + ec["chunk"] - 1).astype(np.int32)
    s_q = W.device_normal((cn + s_rows, H, D), SEED_CHUNKED, "extra", bf16)
    s_out = torch.empty((cn + s_rows, H, D), dtype=bf16, device=dev)
    s_dpos = torch.from_numpy(s_pos).to(dev)
    sws_n = gqa.gqa_step_paged_workspace(cn, s_rows, c_table.shape[1], H, KVH, D)
    s_ws = torch.empty(max(sws_n, 256), dtype=torch.uint8, device=dev)

    def stepped():
        gqa.gqa_step_paged(cn, s_rows, c_table.shape[1], H, KVH, D, gqa.GQA_BF16, 0.0, 0, None, s_q,
                           c_drows, c_dpos, c_pool_k, c_pool_v, ec["num_pages"], c_dtab, s_dpos,
                           s_out, s_ws, sws_n)

    for _ in range(args.warmup):
        stepped()
    s_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    for e0, e1 in s_ev:
        e0.record(stream)
        stepped()
        e1.record(stream)
    torch.cuda.synchronize()
    s_s = float(np.mean([e0.elapsed_time(e1) for e0, e1 in s_ev])) * 1e-3
    s_flops = c_flops + 4 * D * H * int(np.sum(s_pos.astype(np.int64) + 1))
    s_tflops = s_flops / s_s / 1e12
    step_roof = {"bound": "mfma", "achieved": s_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": s_tflops / MFMA_BF16_PEAK_TFLOPS,
                 "traffic": traffic_for("step_paged", STEP_SOURCES),
                 "algorithmic_flops": s_flops, "avg_us": s_s * 1e6,
                 "workload": f"step_paged: the {cn} chunk tokens above + {s_rows} decode tokens"}

    # ---------------- next row: fused q / k / v projections + rope + KV write ----------------
    # Llama-3.1-8B projections of the 16,384 prefill tokens (hidden 4096 ->
    # 32 + 8 + 8 heads of 128), rotated and written into the contiguous cache,
    # timed beside the step; a plain bf16 GEMM of the same shape through
    # torch.matmul (hipBLASLt) is timed as a yardstick.
    hid = 4096
    gx = W.device_normal((P, hid), SEED_QKV, "q", bf16)
    gwq = W.device_normal((H * D, hid), SEED_QKV, "k", bf16) * (hid ** -0.5)
    gwk = W.device_normal((KVH * D, hid), SEED_QKV, "v", bf16) * (hid ** -0.5)
    gwv = W.device_normal((KVH * D, hid), SEED_QKV, "extra", bf16) * (hid ** -0.5)
    g_q = torch.empty((P, H, D), dtype=bf16, device=dev)

    def fused_qkv():
        gqa.gqa_qkv_rope_write(P, hid, H, KVH, D, gqa.GQA_BF16, gx, gwq, gwk, gwv, None, None, None,
                               p_pos, rope_tab, max_pos, g_q, None, None,
                               gqa.GQA_CACHE_CONTIGUOUS, p_cache_k, p_cache_v, nseg, cache_len,
                               p_seg, None, None, 0, 0)

    gwcat = torch.cat([gwq, gwk, gwv], 0).contiguous()

    def timed(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for e0, e1 in pairs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in pairs])) * 1e-3

    q_s = timed(fused_qkv)
    mm_s = timed(lambda: gx @ gwcat.t())
    q_flops = 2 * P * hid * (H + 2 * KVH) * D
    qkv_roof = {"bound": "mfma", "achieved": q_flops / q_s / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": q_flops / q_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "traffic": traffic_for("qkv_rope_write", QKV_SOURCES),
                "algorithmic_flops": q_flops, "avg_us": q_s * 1e6,
                "hipblaslt_gemm_only_us": mm_s * 1e6,
                "workload": f"{P} tokens x hidden {hid} -> (32 + 8 + 8) x 128, rope, contiguous cache"}
    del gx, gwq, gwk, gwv, gwcat, g_q


    # Training pair on the packed prefill batch: the forward with log-sum-exp,
    # then the backward (dq, dk, dv) against a seeded dout. Algorithmic work
    # of the backward: five products the size of one of the forward's two
    # (S and P recomputed, dP, dV, dK, dQ -> 2.5x the forward's flops).
    b_dout = W.device_normal((P, H, D), SEED_PREFILL, "extra", bf16)
    b_lse = torch.empty((P, H), dtype=torch.float32, device=dev)
    b_out = torch.empty((P, H, D), dtype=bf16, device=dev)
    b_dq = torch.empty((P, H, D), dtype=bf16, device=dev)
    b_dk = torch.empty((P, KVH, D), dtype=bf16, device=dev)
    b_dv = torch.empty((P, KVH, D), dtype=bf16, device=dev)
    b_nb = gqa.gqa_prefill_packed_backward_workspace(P, H, KVH, D)
    b_ws = torch.empty(max(b_nb, 256), dtype=torch.uint8, device=dev)

    def fwd_lse():
        gqa.gqa_prefill_packed_lse(P, H, KVH, D, gqa.GQA_BF16, 0.0, 0, pq, pk, pv, p_pos, p_seg, b_out,
                                   b_lse, p_ws, pws_n)

    def bwd():
        gqa.gqa_prefill_packed_backward(P, H, KVH, D, gqa.GQA_BF16, 0.0, 0, pq, pk, pv, b_out, b_dout,
                                        b_lse, p_pos, p_seg, b_dq, b_dk, b_dv, b_ws, b_nb)

    fwd_lse()
    fl_s = timed(fwd_lse)
    bw_s = timed(bwd)
    pairs_b = int(np.sum(seg_len * (seg_len + 1) // 2))
    bw_flops = int(2.5 * 4 * D * H * pairs_b)
    bwd_roof = {"bound": "mfma", "achieved": bw_flops / bw_s / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": bw_flops / bw_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "traffic": None, "algorithmic_flops": bw_flops, "avg_us": bw_s * 1e6,
                "forward_with_lse_us": fl_s * 1e6,
                "workload": f"packed prefill batch above ({P} tokens), dq + dk + dv"}
    del b_dout, b_lse, b_out, b_dq, b_dk, b_dv, b_ws

    # ---------------- the other workload configurations (context) ----------------
    others = None if args.no_other_configs else other_configs(gqa, W, torch, np, stream, 20)

    # ---------------- algorithmic work ----------------
    kv_bytes = int(np.sum(lengths)) * KVH * D * 2 * 2          # K + V of attended keys
    qo_bytes = 2 * rows * H * D * 2                              # q in, out
    decode_bytes = kv_bytes + qo_bytes
    pairs = int(np.sum(seg_len * (seg_len + 1) // 2))
    prefill_flops = 4 * D * H * pairs                            # QK^T + PV, unmasked pairs
    dec_s = per_op_ms["decode_paged"] * 1e-3
    pre_s = per_op_ms["prefill_packed"] * 1e-3
    decode_gbs = decode_bytes / dec_s / 1e9
    prefill_tflops = prefill_flops / pre_s / 1e12

    dec_roof = {"bound": "hbm", "achieved": decode_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": decode_gbs / HBM_PEAK_GBS,
                "traffic": traffic_for("decode_paged", DECODE_SOURCES),
                "algorithmic_bytes": decode_bytes, "avg_us": dec_s * 1e6}
    pre_roof = {"bound": "mfma", "achieved": prefill_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": prefill_tflops / MFMA_BF16_PEAK_TFLOPS,
                "traffic": traffic_for("prefill_packed", PREFILL_SOURCES),
                "algorithmic_flops": prefill_flops, "avg_us": pre_s * 1e6,
                "plan_us_on_second_stream": plan_us, "entry_call_us": entry_s * 1e6,
                "entry_call_frac": prefill_flops / entry_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "note": "avg_us: gqa_prefill_packed_planned in the step (its plan built on a second "
                        "stream during the decode, plan_us_on_second_stream); entry_call_us: the "
                        "one-call gqa_prefill_packed (plan + attention) timed alone"}
    dominant = "prefill_packed" if pre_s >= dec_s else "decode_paged"
    roof = dict(pre_roof if dominant == "prefill_packed" else dec_roof)
    roof["kernel"] = dominant

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    cpu = None
    if snap is not None:
        import oracle
        o = oracle.default()
        threads = o.num_threads()
        # Llama-3.1-8B paged decode: all sampled rows, repeated to ~2 s.
        reps, cpu_dec_s = 0, 0.0
        while reps == 0 or cpu_dec_s < 2.0:
            t = time.perf_counter()
            o.decode_paged(snap["q"], snap["pk"], snap["pv"], dpos[snap["rows"]], snap["table"])
            cpu_dec_s += time.perf_counter() - t
            reps += 1
        s_keys = int(np.sum(lengths[snap["rows"]]))
        s_bytes = s_keys * KVH * D * 2 * 2 + 2 * len(snap["rows"]) * H * D * 2
        # Llama-3.1-8B packed prefill: a sample of the queries.
        t = time.perf_counter()
        o.packed(snap["pq"], snap["pk_"], snap["pv_"], ppos, pseg, sel=snap["sel"])
        cpu_pre_s = time.perf_counter() - t
        s_pairs = int(np.sum(ppos[snap["sel"]].astype(np.int64) + 1))
        s_flops = 4 * D * H * s_pairs
        per_config = {
            "llama8b_paged_decode": {
                "seconds": cpu_dec_s / reps, "algorithmic_bytes": s_bytes,
                "gbs": s_bytes * reps / cpu_dec_s / 1e9,
                "sample": f"{len(snap['rows'])} of {rows} rows ({s_keys} keys), {reps} passes"},
            "llama8b_packed_prefill": {
                "seconds": cpu_pre_s, "algorithmic_flops": s_flops,
                "gflops": s_flops / cpu_pre_s / 1e9,
                "sample": f"{len(snap['sel'])} of {P} queries ({s_pairs} attended pairs per head)"},
        }
        per_config.update(oracle_other_configs(o, np, W))
        # Single-threaded: the tiny Llama example, GPT-2 decode_rows and one
        # pass of the paged decode.
        o.set_num_threads(1)
        single = {}
        t = time.perf_counter()
        o.decode_paged(snap["q"], snap["pk"], snap["pv"], dpos[snap["rows"]], snap["table"])
        t1 = time.perf_counter() - t
        single["llama8b_paged_decode"] = {"seconds": t1, "gbs": s_bytes / t1 / 1e9}
        single.update(oracle_other_configs(o, np, W, only=("tiny_llama", "gpt2_decode_rows_f32")))
        o.set_num_threads(threads)
        total = cpu_dec_s + cpu_pre_s + sum(v.get("seconds", 0.0) for v in per_config.values()
                                            if isinstance(v, dict) and "layers" not in v) + \
            sum(v["seconds"] for v in single.values())
        cpu = {"value": s_bytes * reps / cpu_dec_s / 1e9, "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": (f"decode_paged on {len(snap['rows'])} of {rows} rows "
                          f"({s_keys} keys) x {reps} passes, "
                          f"{cpu_dec_s:.2f} s; "
                          f"packed prefill on {len(snap['sel'])} of {P} queries "
                          f"({s_pairs} attended pairs/head, {cpu_pre_s:.2f} s); the other "
                          "configurations in per_config, single-threaded times in single_thread"),
               "prefill_tflops": s_flops / cpu_pre_s / 1e12,
               "per_config": per_config, "single_thread": single,
               "seconds": total}

    result = {
        "metric": METRIC,
        "value": decode_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q/k/v and page pool, seeded page table and segment layout",
        "config": {
            "workload": "llama-3.1-8b paged decode (64 rows, L~U[512,8192], 9000-page pool, "
                        "PageSize 64) + packed prefill (P=16384, segments U[64,4096]); "
                        "Heads 32, KvHeads 8, D 128, theta 5e5",
            "decode_rows": rows, "decode_keys": int(np.sum(lengths)),
            "prefill_tokens": P, "prefill_segments": nseg, "prefill_pairs_per_head": pairs,
        },
        "prefill_tflops": prefill_tflops,
        "decode_frac_of_hbm_peak": decode_gbs / HBM_PEAK_GBS,
        "prefill_frac_of_mfma_peak": prefill_tflops / MFMA_BF16_PEAK_TFLOPS,
        "measured_ceilings": ceilings,
        "decode_frac_of_stream_read": decode_gbs / ceilings["stream_read_gbs"],
        "prefill_frac_of_bf16_matmul": prefill_tflops / ceilings["bf16_matmul_tflops"],
        "roofline": roof,
        "rooflines": {"decode_paged": dec_roof, "prefill_packed": pre_roof},
        "next_rows": {"prefill_cached_paged": chunk_roof, "step_paged": step_roof,
                      "prefill_packed_backward": bwd_roof,
                      "qkv_rope_write": qkv_roof},
        "per_op_us": {k: v * 1e3 for k, v in per_op_ms.items()},
        "per_op_us_p10_p50_p90": per_op_pct,
        "other_configs": others,
        "wall_s_timed": wall,
        "cpu_baseline": cpu,
        "host": host_info(torch, clocks_before, clocks_prefill),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
