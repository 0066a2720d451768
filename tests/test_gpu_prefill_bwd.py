"""GPU parity: the packed attention's training pair -- gqa_prefill_packed_lse
(forward + log-sum-exp) and gqa_prefill_packed_backward (dq, dk, dv) --
against the fp64 oracle, over ragged segment layouts, grouped-query shapes,
windows, partial tiles and a Llama-3.1-8B-shaped packed batch (sampled).

Tolerance of the gradients: the bf16 bar of the forward (2e-2 absolute at
unit magnitude) scaled by the magnitude of the value, |got - ref| <=
2e-2 (1 + |ref|): dk and dv sum over every query and the G query heads of a
group, and the result itself is rounded once to bf16 (2^-9 |ref|); the
probabilities and dS enter the matrix cores as bf16 (2^-9 relative each).
The log-sum-exp is an f32 output: <= 1e-4 absolute.
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import oracle
import workloads as W
from tests.gpu_common import DEV, dev, f64, host_values, i32, workspace

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-2
LSE_TOL = 1e-4


def run_pair(seed, p, heads, kvh, d, lo, hi, window, layout=None):
    g = W.streams(seed)
    if layout is None:
        lengths, pos, seg = W.segment_layout(p, lo, hi, g["index"])
    else:
        pos, seg = layout
        p = len(pos)
    q_t, q64 = host_values(W.normal(g["q"], (p, heads, d)), "bf16")
    k_t, k64 = host_values(W.normal(g["k"], (p, kvh, d)), "bf16")
    v_t, v64 = host_values(W.normal(g["v"], (p, kvh, d)), "bf16")
    g_t, g64 = host_values(W.normal(g["extra"], (p, heads, d)), "bf16")
    q, k, v, gd = dev(q_t), dev(k_t), dev(v_t), dev(g_t)
    dpos, dseg = i32(pos), i32(seg)
    bf = torch.bfloat16
    out = torch.full((p, heads, d), float("nan"), dtype=bf, device=DEV)
    lse = torch.full((p, heads), float("nan"), dtype=torch.float32, device=DEV)
    ws, nb = workspace(gqa.gqa_prefill_packed_workspace(p, heads, kvh, d))
    gqa.gqa_prefill_packed_lse(p, heads, kvh, d, gqa.GQA_BF16, 0.0, window, q, k, v, dpos, dseg, out,
                               lse, ws, nb)
    dq = torch.full((p, heads, d), float("nan"), dtype=bf, device=DEV)
    dk = torch.full((p, kvh, d), float("nan"), dtype=bf, device=DEV)
    dvv = torch.full((p, kvh, d), float("nan"), dtype=bf, device=DEV)
    wsb, nbb = workspace(gqa.gqa_prefill_packed_backward_workspace(p, heads, kvh, d))
    gqa.gqa_prefill_packed_backward(p, heads, kvh, d, gqa.GQA_BF16, 0.0, window, q, k, v, out, gd,
                                    lse, dpos, dseg, dq, dk, dvv, wsb, nbb)
    torch.cuda.synchronize()
    return (f64(out), f64(lse), f64(dq), f64(dk), f64(dvv)), (q64, k64, v64, g64), pos, seg


def check_grad(got, ref, what):
    assert not np.isnan(got).any(), f"{what}: NaN (an entry was never written)"
    err = np.abs(got - ref)
    bound = GRAD_TOL * (1.0 + np.abs(ref))
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (f"{what}: |err| {err[worst]:.4g} > {bound[worst]:.4g} at {worst} "
                                  f"(ref {ref[worst]:.4g})")


CASES = [
    # seed, P, heads, kv_heads, D, segment lengths [lo, hi], window
    (1, 300, 8, 2, 128, 16, 120, 0),
    (2, 300, 8, 2, 128, 16, 120, 40),
    (3, 257, 4, 4, 64, 8, 100, 0),
    (4, 520, 8, 1, 64, 30, 300, 0),
    (5, 640, 6, 2, 128, 64, 400, 0),
    (6, 520, 16, 2, 64, 30, 300, 1),
    (7, 97, 2, 1, 128, 1, 40, 0),
    (8, 1000, 32, 8, 128, 64, 600, 0),
    (9, 1, 4, 2, 128, 1, 1, 0),  # one token: one partial query tile and key tile
    (10, 31, 8, 8, 64, 5, 31, 3),  # a single partial tile, window 3
]


@pytest.mark.parametrize("seed,p,heads,kvh,d,lo,hi,window", CASES)
def test_backward_matches_oracle(seed, p, heads, kvh, d, lo, hi, window):
    print(f"[case] backward seed={seed} P={p} H={heads} KvH={kvh} D={d} W={window}", flush=True)
    (out, lse, dq, dk, dv), (q, k, v, g), pos, seg = run_pair(seed, p, heads, kvh, d, lo, hi, window)
    o = oracle.default()
    lse_ref = o.packed_lse(q, k, pos, seg, None, window)
    assert np.max(np.abs(lse - lse_ref)) <= LSE_TOL
    assert np.max(np.abs(out - o.packed(q, k, v, pos, seg, window=window))) <= 2e-2
    dq_r, dk_r, dv_r = o.packed_backward(q, k, v, g, pos, seg, None, window)
    check_grad(dq, dq_r, "dq")
    check_grad(dk, dk_r, "dk")
    check_grad(dv, dv_r, "dv")


def test_backward_llama8b_packed_sampled():
    """P = 16384, Heads 32, KvHeads 8, D 128, segments U[64, 4096] (the packed
    Llama workload). Segments are independent, so the oracle runs on one
    segment alone: the shortest one whole (dq, dk, dv), and the first 600
    tokens of the longest one (dq: those queries see only keys before them)."""
    wl = W.LLAMA8B_PACKED
    p, h, kvh, d = wl.extra["p"], wl.heads, wl.kv_heads, wl.head_dim
    print(f"[case] backward {wl.name}", flush=True)
    (out, lse, dq, dk, dv), (q, k, v, g), pos, seg = run_pair(4, p, h, kvh, d, 64, 4096, 0)
    assert not np.isnan(dk).any() and not np.isnan(dv).any() and not np.isnan(dq).any()
    o = oracle.default()
    starts = np.flatnonzero(np.r_[1, np.diff(seg)])
    ends = np.r_[starts[1:], p]
    lens = ends - starts
    si = int(np.argmin(lens))
    sl = slice(int(starts[si]), int(ends[si]))
    dq_r, dk_r, dv_r = o.packed_backward(q[sl], k[sl], v[sl], g[sl], pos[sl], seg[sl])
    check_grad(dq[sl], dq_r, f"dq segment {si}")
    check_grad(dk[sl], dk_r, f"dk segment {si}")
    check_grad(dv[sl], dv_r, f"dv segment {si}")
    li = int(np.argmax(lens))
    a = int(starts[li])
    sl = slice(a, a + 600)
    dq_r, _, _ = o.packed_backward(q[sl], k[sl], v[sl], g[sl], pos[sl], seg[sl])
    check_grad(dq[sl], dq_r, f"dq first 600 of segment {li}")
    # The longest segment whole, for KV head 0 and the query heads that read
    # it (heads 0 .. G - 1): every key's dk and dv and every query's dq of
    # that group. (KV heads are independent, so the slice is exact.)
    sl = slice(int(starts[li]), int(ends[li]))
    gq = h // kvh
    dq_r, dk_r, dv_r = o.packed_backward(q[sl][:, :gq], k[sl][:, :1], v[sl][:, :1], g[sl][:, :gq],
                                         pos[sl], seg[sl])
    print(f"[parity] backward longest segment ({int(lens[li])} tokens), KV head 0: max |err| "
          f"dk {np.max(np.abs(dk[sl][:, :1] - dk_r)):.3e} (max |ref| {np.max(np.abs(dk_r)):.3g}), "
          f"dv {np.max(np.abs(dv[sl][:, :1] - dv_r)):.3e} (max |ref| {np.max(np.abs(dv_r)):.3g})", flush=True)
    check_grad(dk[sl][:, :1], dk_r, f"dk segment {li}, KV head 0")
    check_grad(dv[sl][:, :1], dv_r, f"dv segment {li}, KV head 0")
    check_grad(dq[sl][:, :gq], dq_r, f"dq segment {li}, heads 0..{gq - 1}")


def test_backward_extreme_positions():
    """dq, dk, dv under the literal `own` mask with positions anywhere in
    int32 (differences up to 2^32 - 1), with and without a window."""
    from tests.test_gpu_prefill import extreme_position_layout
    heads, kvh, d = 8, 2, 128
    layout = extreme_position_layout(W.streams(4344))
    o = oracle.default()
    for window in (0, 37):
        print(f"[case] backward extreme positions W={window}", flush=True)
        (out, lse, dq, dk, dv), (q, k, v, g), pos, seg = run_pair(4344, 0, heads, kvh, d, 0, 0, window,
                                                                  layout=layout)
        lse_ref = o.packed_lse(q, k, pos, seg, None, window)
        assert np.max(np.abs(lse - lse_ref)) <= LSE_TOL
        rq, rk, rv = o.packed_backward(q, k, v, g, pos, seg, None, window)
        check_grad(dq, rq, "dq")
        check_grad(dk, rk, "dk")
        check_grad(dv, rv, "dv")
