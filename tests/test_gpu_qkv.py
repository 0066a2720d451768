"""GPU parity: the fused q / k / v projections + rope + cache write
(gqa_qkv_rope_write) against the oracle's Linear, rope and write_at.

Tolerance: the matrix cores sum the projection in f32, the oracle exactly.
The f32 sum of K = hidden products is within e = K 2^-24 sum_i |x_i w_i| of
the exact one (the standard summation bound), so after rounding to bf16 a
projection value differs by at most one bf16 ulp (<= 2^-7 of its magnitude)
plus e; through the rotation each output is bounded by
2^-7 (|x_lo| + |x_hi| + |y|) + 2 (e_lo + e_hi), x the oracle's unrotated pair
and y its result. Almost every value must still match bit for bit.
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import oracle
import workloads as W
from tests.gpu_common import CODE, DEV, dev, f64, host_values, i32

pytestmark = pytest.mark.gpu


def check_rotated(got, ref, pre, what, rotated=True, esum=None):
    """got, ref, pre: [n, h, D] float64 (pre = unrotated projection); esum:
    the f32 summation bound of each projection value (same shape)."""
    d = ref.shape[-1]
    half = d // 2
    esum = np.zeros_like(ref) if esum is None else esum
    if rotated:
        mag = np.concatenate([np.abs(pre[..., :half]) + np.abs(pre[..., half:])] * 2, axis=-1)
        eab = np.concatenate([esum[..., :half] + esum[..., half:]] * 2, axis=-1)
    else:
        mag = np.zeros_like(ref)
        eab = esum
    bound = 2.0 ** -7 * (mag + np.abs(ref)) + 2.0 * eab + 1e-30
    err = np.abs(got - ref)
    exact = float(np.mean(got == ref))
    worst = float(np.max(err / bound))
    print(f"[parity] {what}: bit-exact {100 * exact:.2f}%, worst err / bound {worst:.3f}",
          flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= 1.0, f"{what}: error beyond one bf16 rounding of the projection"
    assert exact >= 0.9, f"{what}: only {100 * exact:.1f}% bit-exact"


def run_case(n, hidden, heads, kvh, d, bias, rope, cache, seed, k_out=True, sel=None):
    g = W.streams(seed)
    o = oracle.default()
    xs = 1.0 / np.sqrt(hidden)
    x_t, x64 = host_values(W.normal(g["q"], (n, hidden)), "bf16")
    wq_t, wq64 = host_values(W.normal(g["k"], (heads * d, hidden)) * xs, "bf16")
    wk_t, wk64 = host_values(W.normal(g["v"], (kvh * d, hidden)) * xs, "bf16")
    wv_t, wv64 = host_values(W.normal(g["extra"], (kvh * d, hidden)) * xs, "bf16")
    b = [host_values(W.normal(g["sinks"], (f,)), "bf16") for f in (heads * d, kvh * d, kvh * d)]
    max_pos, theta = max(4096, n), 500000.0
    # distinct positions: two tokens with one cache target would race
    pos = g["index"].permutation(max(n, 700))[:n].astype(np.int32)
    tab = torch.empty((2, max_pos, d // 2), dtype=torch.bfloat16, device=DEV)
    gqa.gqa_rope_table(d, max_pos, theta, gqa.GQA_BF16, tab)
    q_out = torch.full((n, heads, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    k_o = torch.full((n, kvh, d), float("nan"), dtype=torch.bfloat16, device=DEV) if k_out else None
    v_o = torch.full((n, kvh, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    kind = {"none": gqa.GQA_CACHE_NONE, "contiguous": gqa.GQA_CACHE_CONTIGUOUS,
            "paged": gqa.GQA_CACHE_PAGED_TABLE, "slots": gqa.GQA_CACHE_PAGED_SLOTS}[cache]
    rows = g["index"].integers(0, 3, n).astype(np.int32)
    if cache == "contiguous":
        ck = torch.full((3, kvh, 2100, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        dim0, seq, table, tr, tp, slots = 3, 2100, None, 0, 0, None
    elif cache in ("paged", "slots"):
        ck = torch.full((40, kvh, 64, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        dim0, seq, tr, tp = 40, 64, 3, 12
        table = g["index"].permutation(40)[:36].reshape(3, 12).astype(np.int32)
        slots = g["index"].permutation(40 * 64)[:n].astype(np.int32) if cache == "slots" else None
    else:
        ck, dim0, seq, table, tr, tp, slots = None, 0, 0, None, 0, 0, None
    cv = torch.full_like(ck, float("nan")) if ck is not None else None
    gqa.gqa_qkv_rope_write(n, hidden, heads, kvh, d, CODE["bf16"], dev(x_t), dev(wq_t), dev(wk_t),
                           dev(wv_t), *(dev(bb[0]) if bias else None for bb in b), i32(pos),
                           tab if rope else None, max_pos, q_out, k_o, v_o, kind, ck, cv, dim0,
                           seq, i32(rows) if cache in ("contiguous", "paged") else None,
                           i32(slots) if slots is not None else None,
                           i32(table) if table is not None else None, tr, tp)
    torch.cuda.synchronize()
    idx = np.arange(n) if sel is None else sel
    bq, bk, bv = (bb[1] if bias else None for bb in b)
    qp = o.linear(x64[idx], wq64, bq).reshape(len(idx), heads, d)
    kp = o.linear(x64[idx], wk64, bk).reshape(len(idx), kvh, d)
    vp = o.linear(x64[idx], wv64, bv).reshape(len(idx), kvh, d)
    # f32 summation bounds: hidden * 2^-24 * sum_i |x_i w_i| per projection value
    ax = np.abs(x64[idx])
    eq, ek_, ev_ = (hidden * 2.0 ** -24 * o.linear(ax, np.abs(w), None, "none").reshape(len(idx), -1, d)
                    for w in (wq64, wk64, wv64))
    if rope:
        c, s = o.rope_tables(max_pos, d, theta, "bf16")
        qr = o.rope(qp, pos[idx], c, s, "bf16")
        kr = o.rope(kp, pos[idx], c, s, "bf16")
    else:
        qr, kr = qp, kp
    check_rotated(f64(q_out)[idx], qr, qp, f"q n={n} H={hidden} D={d} {cache}", rope, eq)
    check_rotated(f64(v_o)[idx], vp, vp, f"v n={n} D={d}", False, ev_)
    if k_out:
        check_rotated(f64(k_o)[idx], kr, kp, f"k n={n} D={d}", rope, ek_)
    if ck is not None and sel is None:
        # the cache holds the rotated k (and v) exactly where write_at puts them
        zero = np.zeros(ck.shape)
        ek, ev, wr = (o.write_contiguous(f64(k_o) if k_out else kr, f64(v_o), pos, zero, zero.copy(),
                                         rows=rows) if cache == "contiguous" else
                      o.write_paged(f64(k_o) if k_out else kr, f64(v_o), zero, zero.copy(),
                                    positions=pos, rows=rows if cache == "paged" else None,
                                    slots=slots, table=table))
        gk, gv = f64(ck), f64(cv)
        assert np.all(np.isnan(gk[~wr])) and np.all(np.isnan(gv[~wr])), "write outside targets"
        # v is written unrotated and k as k_out holds it: bit-exact copies
        assert np.array_equal(gv[wr], ev[wr]), "cached v differs from v_out"
        if k_out:
            assert np.array_equal(gk[wr], ek[wr]), "cached k differs from k_out"
        else:
            err = np.abs(gk[wr] - ek[wr])
            assert np.all(err <= 2.0 ** -6 * (np.abs(ek[wr]) + 1.0)), "cached k far from rope(k_proj)"


@pytest.mark.parametrize("n,hidden,heads,kvh,d,bias,rope,cache", [
    (200, 512, 8, 8, 64, True, True, "contiguous"),
    (300, 1024, 8, 2, 128, False, True, "paged"),
    (150, 2880, 64, 8, 64, True, False, "slots"),
    (129, 768, 4, 4, 64, False, True, "none"),
    (130, 512, 4, 1, 128, True, True, "contiguous"),   # kv features not a multiple of 256
])
def test_qkv_rope_write(n, hidden, heads, kvh, d, bias, rope, cache):
    print(f"[case] qkv n={n} H={hidden} heads={heads} kvh={kvh} D={d} bias={bias} rope={rope} "
          f"cache={cache}", flush=True)
    run_case(n, hidden, heads, kvh, d, bias, rope, cache, seed=2600 + n)


def test_qkv_rope_write_no_k_out():
    print("[case] qkv without k_out / with cache", flush=True)
    run_case(100, 512, 8, 2, 128, True, True, "contiguous", seed=2700, k_out=False)


@pytest.mark.parametrize("n", [2048, 16384])
def test_qkv_llama8b_sampled(n):
    """Llama-3.1-8B projections (hidden 4096, 32 / 8 heads, D 128); 24 sampled
    tokens checked against the oracle. 16384 tokens is the full prefill batch
    (64 token tiles: the XCD-banded tile order)."""
    g = W.streams(2800)
    sel = np.sort(W.sample_indices(n, 24, g["index"]))
    print(f"[case] qkv llama8b n={n} sampled", flush=True)
    run_case(n, 4096, 32, 8, 128, False, True, "none", seed=2800, sel=sel)
