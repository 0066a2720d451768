"""GPU parity: packed prefill attention (the `own` mask, window, sinks) against
the fp64 oracle, from tiny ragged cases to the full Llama-3.1-8B packed
workload (sampled queries) and the gpt-oss 4096-token prefill.
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import oracle
import workloads as W
from tests.gpu_common import (CODE, DEV, TORCH_DT, assert_close, bits, dev, f64, host_values, i32,
                              workspace)

pytestmark = pytest.mark.gpu


def run_prefill(q, k, v, pos, seg, heads, kvh, d, window=0, sinks=None, dtype="bf16"):
    p = q.shape[0]
    out = torch.full((p, heads, d), float("nan"), dtype=TORCH_DT[dtype], device=DEV)
    ws, nb = workspace(gqa.gqa_prefill_packed_workspace(p, heads, kvh, d))
    gqa.gqa_prefill_packed(p, heads, kvh, d, CODE[dtype], 0.0, window, sinks, q, k, v, i32(pos),
                           i32(seg), out, ws, nb)
    torch.cuda.synchronize()
    return out


def make_inputs(seed, p, heads, kvh, d, dtype="bf16", scale_q=1.0):
    g = W.streams(seed)
    q_t, q64 = host_values(W.normal(g["q"], (p, heads, d)) * scale_q, dtype)
    k_t, k64 = host_values(W.normal(g["k"], (p, kvh, d)), dtype)
    v_t, v64 = host_values(W.normal(g["v"], (p, kvh, d)), dtype)
    sinks_t, sinks64 = host_values(W.normal(g["sinks"], (heads,)), dtype)
    return (dev(q_t), dev(k_t), dev(v_t)), (q64, k64, v64), (dev(sinks_t), sinks64), g


@pytest.mark.parametrize("heads,kvh,d", [(8, 8, 64), (32, 8, 128), (64, 8, 64), (4, 2, 128),
                                         (6, 6, 128), (16, 2, 64)])
@pytest.mark.parametrize("window,use_sinks", [(0, False), (0, True), (37, True), (1, False)])
def test_prefill_packed_ragged(heads, kvh, d, window, use_sinks):
    print(f"[case] prefill H={heads} KvH={kvh} D={d} W={window} sinks={use_sinks}", flush=True)
    g0 = W.streams(1000 + heads + d)
    lengths, pos, seg = W.segment_layout(333, 1, 150, g0["index"])
    dv, hv, (sk, sk64), _ = make_inputs(1000 + heads + d, len(pos), heads, kvh, d)
    out = run_prefill(*dv, pos, seg, heads, kvh, d, window, sk if use_sinks else None)
    ref = oracle.default().packed(*hv, pos, seg, window=window, sinks=sk64 if use_sinks else None)
    assert_close(f64(out), ref, "bf16", f"prefill ragged P={len(pos)}")


@pytest.mark.parametrize("heads,kvh,d,window,use_sinks", [(32, 8, 128, 0, False), (8, 8, 64, 37, True),
                                                          (16, 2, 64, 0, True)])
def test_prefill_plan_once_run_twice(heads, kvh, d, window, use_sinks):
    """One plan (built on a second stream, handed over by an event) serves two
    layers' q, k, v; each planned output equals gqa_prefill_packed bit for bit,
    and the first also the oracle."""
    print(f"[case] prefill plan reuse H={heads} KvH={kvh} D={d} W={window} sinks={use_sinks}", flush=True)
    g0 = W.streams(2100 + heads + d)
    lengths, pos, seg = W.segment_layout(700, 1, 300, g0["index"])
    p = len(pos)
    layers = [make_inputs(2100 + heads + d + 17 * i, p, heads, kvh, d) for i in range(2)]
    ws, nb = workspace(gqa.gqa_prefill_packed_workspace(p, heads, kvh, d))
    pos_d, seg_d = i32(pos), i32(seg)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        gqa.gqa_prefill_packed_plan(p, heads, kvh, d, window, pos_d, seg_d, ws, nb)
        built = torch.cuda.Event()
        built.record(side)
    torch.cuda.current_stream().wait_event(built)
    for i, (dv_, hv, (sk, sk64), _) in enumerate(layers):
        sinks = sk if use_sinks else None
        out = torch.full((p, heads, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        gqa.gqa_prefill_packed_planned(p, heads, kvh, d, gqa.GQA_BF16, 0.0, window, sinks, *dv_, pos_d,
                                       seg_d, out, ws, nb)
        torch.cuda.synchronize()
        fused = run_prefill(*dv_, pos, seg, heads, kvh, d, window, sinks)
        assert np.array_equal(bits(out), bits(fused)), f"layer {i}: planned != fused"
        if i == 0:
            ref = oracle.default().packed(*hv, pos, seg, window=window, sinks=sk64 if use_sinks else None)
            assert_close(f64(out), ref, "bf16", f"planned prefill P={p}")


def test_prefill_tiny_llama_example():
    wl = W.TINY_LLAMA
    s = wl.extra["prefill"]
    print(f"[case] {wl.name}: prefill", flush=True)
    pos = np.arange(s, dtype=np.int32)
    seg = np.zeros(s, dtype=np.int32)
    dv, hv, _, _ = make_inputs(1, s, wl.heads, wl.kv_heads, wl.head_dim)
    out = run_prefill(*dv, pos, seg, wl.heads, wl.kv_heads, wl.head_dim)
    ref = oracle.default().packed(*hv, pos, seg)
    assert_close(f64(out), ref, "bf16", "tiny llama prefill S=128")


def test_prefill_arbitrary_order_and_ids():
    """The literal `own` predicate: interleaved, non-contiguous segment ids,
    duplicate positions, shuffled token order."""
    heads, kvh, d = 32, 8, 128
    g = W.streams(4242)
    lengths, pos, seg = W.segment_layout(500, 1, 200, g["index"])
    seg = (seg * 7919 - 13).astype(np.int32)  # arbitrary ids
    perm = g["index"].permutation(len(pos))
    pos, seg = pos[perm], seg[perm]
    pos[::17] = pos[::17] // 2  # duplicates inside segments
    dv, hv, (sk, sk64), _ = make_inputs(4242, len(pos), heads, kvh, d)
    o = oracle.default()
    for window, sinks in ((0, None), (20, sk)):
        out = run_prefill(*dv, pos, seg, heads, kvh, d, window, sinks)
        ref = o.packed(*hv, pos, seg, window=window, sinks=None if sinks is None else sk64)
        assert_close(f64(out), ref, "bf16", f"prefill shuffled/duplicates W={window}")


def extreme_position_layout(g):
    """Packed segments whose positions span the int32 range: one at the top
    (up to 2^31 - 1), one negative, one mixing the extremes with duplicates
    and a plain one; differences of two positions reach 2^32 - 1."""
    imax, imin = np.iinfo(np.int32).max, np.iinfo(np.int32).min
    top = np.arange(imax - 149, imax + 1, dtype=np.int64)
    neg = np.arange(-200, -80, dtype=np.int64)
    mix = g["index"].choice(np.array([imin, imin + 1, imin + 5, -3, -1, 0, 2, imax - 4, imax - 1, imax],
                                     dtype=np.int64), 90)
    plain = np.arange(0, 64, dtype=np.int64)
    pos = np.concatenate([top, neg, mix, plain]).astype(np.int32)
    seg = np.concatenate([np.full(len(a), i) for i, a in enumerate((top, neg, mix, plain))]).astype(np.int32)
    return pos, seg


def test_prefill_extreme_positions():
    """The literal `own` mask and window for positions anywhere in int32."""
    heads, kvh, d = 32, 8, 128
    g = W.streams(4343)
    pos, seg = extreme_position_layout(g)
    print(f"[case] prefill extreme positions P={len(pos)}", flush=True)
    dv, hv, (sk, sk64), _ = make_inputs(4343, len(pos), heads, kvh, d)
    o = oracle.default()
    for window, sinks in ((0, None), (37, sk), (np.iinfo(np.int32).max, None)):
        out = run_prefill(*dv, pos, seg, heads, kvh, d, window, sinks)
        ref = o.packed(*hv, pos, seg, window=window, sinks=None if sinks is None else sk64)
        assert_close(f64(out), ref, "bf16", f"prefill extreme positions W={window}")


def test_prefill_descending_ids_offset_positions():
    """Key tiles that straddle segment boundaries with segment ids in
    descending order (a tile's smallest id sits in its later tokens) and
    positions that start at a per-segment offset: the tile walk may skip a
    key tile only when no pair in it is allowed."""
    heads, kvh, d = 32, 8, 128
    g = W.streams(4343)
    lengths, pos, seg = W.segment_layout(700, 20, 150, g["index"])
    n = len(lengths)
    seg = (n - 1 - seg).astype(np.int32)
    offs = g["index"].integers(0, 300, n).astype(np.int32)
    pos = (pos + offs[n - 1 - seg]).astype(np.int32)
    dv, hv, (sk, sk64), _ = make_inputs(4343, len(pos), heads, kvh, d)
    o = oracle.default()
    for window, sinks in ((0, None), (48, sk)):
        print(f"[case] prefill descending ids W={window}", flush=True)
        out = run_prefill(*dv, pos, seg, heads, kvh, d, window, sinks)
        ref = o.packed(*hv, pos, seg, window=window, sinks=None if sinks is None else sk64)
        assert_close(f64(out), ref, "bf16", f"prefill descending ids W={window}")


def test_prefill_llama8b_packed_full_sampled():
    wl = W.LLAMA8B_PACKED
    p = wl.extra["p"]
    print(f"[case] {wl.name} (full size, sampled queries)", flush=True)
    g = W.streams(4)
    lengths, pos, seg = W.segment_layout(p, wl.extra["seg_lo"], wl.extra["seg_hi"], g["index"])
    dv, hv, _, g2 = make_inputs(4, p, wl.heads, wl.kv_heads, wl.head_dim)
    out = run_prefill(*dv, pos, seg, wl.heads, wl.kv_heads, wl.head_dim)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    ends = np.cumsum(lengths) - 1
    # Every query of each 32-token query tile that a segment boundary cuts
    # (their key tiles mix two segments), every 16th query, the segment ends
    # and a random sample.
    straddle = [np.arange(32 * (b // 32), min(p, 32 * (b // 32) + 32)) for b in starts[1:] if b % 32]
    sel = np.unique(np.concatenate([starts, ends, W.sample_indices(p, 200, g2["extra"]),
                                    np.arange(0, p, 16), [p - 1]] + straddle)).astype(np.int32)
    ref = oracle.default().packed(*hv, pos, seg, sel=sel)
    assert_close(f64(out)[sel], ref, "bf16", f"llama8b packed prefill, {len(sel)} sampled queries")


def test_prefill_long_batch_sampled():
    """40,960 packed tokens (1,280 query tiles, 640 key tiles): the prepared
    walk's paths for more query tiles than one workgroup has threads and for
    more than 8 groups of 64 key tiles."""
    heads, kvh, d, p = 8, 2, 64, 40960
    print(f"[case] prefill long batch P={p}", flush=True)
    g = W.streams(4096)
    lengths, pos, seg = W.segment_layout(p, 64, 4096, g["index"])
    dv, hv, (sk, sk64), g2 = make_inputs(4096, p, heads, kvh, d)
    o = oracle.default()
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    ends = np.cumsum(lengths) - 1
    sel = np.unique(np.concatenate([starts, ends, W.sample_indices(p, 160, g2["extra"]),
                                    np.arange(0, p, 211), [p - 1]])).astype(np.int32)
    for window, sinks in ((0, None), (700, sk)):
        out = run_prefill(*dv, pos, seg, heads, kvh, d, window, sinks)
        ref = o.packed(*hv, pos, seg, window=window, sinks=None if sinks is None else sk64, sel=sel)
        assert_close(f64(out)[sel], ref, "bf16", f"long packed batch W={window}, {len(sel)} sampled queries")


@pytest.mark.parametrize("window", [128, 0])
def test_prefill_gpt_oss_sampled(window):
    wl = W.GPT_OSS_SINK
    s = wl.extra["prefill"]
    print(f"[case] {wl.name}: prefill W={window}", flush=True)
    pos = np.arange(s, dtype=np.int32)
    seg = np.zeros(s, dtype=np.int32)
    dv, hv, (sk, sk64), g = make_inputs(5, s, wl.heads, wl.kv_heads, wl.head_dim)
    out = run_prefill(*dv, pos, seg, wl.heads, wl.kv_heads, wl.head_dim, window, sk)
    sel = np.unique(np.concatenate([[0, 1, 127, 128, 129, s - 1],
                                    W.sample_indices(s, 120, g["extra"])])).astype(np.int32)
    ref = oracle.default().packed(*hv, pos, seg, window=window, sinks=sk64, sel=sel)
    assert_close(f64(out)[sel], ref, "bf16", f"gpt-oss prefill W={window}, sampled")


def test_prefill_mask_probe():
    """q = 0 gives uniform weights over each query's attended set; v one-hot
    per key (dimension = key index within its segment) makes membership
    exact at segment edges, tile edges and window edges."""
    heads, kvh, d = 4, 1, 128
    lengths = [1, 63, 64, 65, 2, 100]
    p = sum(lengths)
    seg = np.repeat(np.arange(len(lengths)), lengths).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    pos = (np.arange(p) - np.repeat(starts, lengths)).astype(np.int32)
    q = torch.zeros((p, heads, d), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((p, kvh, d), dtype=torch.bfloat16)
    v = torch.zeros((p, kvh, d), dtype=torch.bfloat16)
    for j in range(p):
        v[j, 0, pos[j] % d] = 1.0
    for window in (0, 3, 64):
        out = f64(run_prefill(q, dev(k), dev(v), pos, seg, heads, kvh, d, window))
        for i in range(p):
            keys = [j for j in range(p) if seg[j] == seg[i] and pos[j] <= pos[i]
                    and (window == 0 or pos[i] - pos[j] < window)]
            expect = np.zeros(d)
            for j in keys:
                expect[pos[j] % d] += 1.0 / len(keys)
            for h in range(heads):
                assert np.array_equal(out[i, h] > 0, expect > 0), f"query {i} W={window}"
                assert np.max(np.abs(out[i, h] - expect)) < 2e-2


def test_prefill_empty_and_deterministic():
    heads, kvh, d = 32, 8, 128
    ws, nb = workspace(256)
    gqa.gqa_prefill_packed(0, heads, kvh, d, gqa.GQA_BF16, 0.0, 0, None, 1, 1, 1, 1, 1, 1, ws, nb)
    g = W.streams(8)
    lengths, pos, seg = W.segment_layout(1500, 64, 1000, g["index"])
    dv, hv, _, _ = make_inputs(8, len(pos), heads, kvh, d)
    a = run_prefill(*dv, pos, seg, heads, kvh, d)
    b = run_prefill(*dv, pos, seg, heads, kvh, d)
    assert np.array_equal(bits(a), bits(b))
