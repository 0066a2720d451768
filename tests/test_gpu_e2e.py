"""GPU: whole flows of the tiny Llama example and of the gpt-oss SinkAttention
layer pair, as the pages' entries run them, against the fp64 oracle.

Tiny Llama (Linnet "examples/01-llama" page, `forward` then `decode`): the
rotary tables (theta 1e4), rope + KV write of a 128-token prompt into a
[1, 8, 512, 64] cache, causal prefill over it, then 16 decode steps, each a
rope + write of one token and `decode_rows` at its position. gpt-oss-20b
(Nest card, SinkAttention in a LayerPair): the same flow for a 4096-token
prompt and 256 decode steps into a [1, 8, 4352, 64] cache, for the sliding
layer (window 128) and the full layer, with per-head sinks.

Every output is compared with the oracle at the bf16 bar (prefill queries
sampled for the 4096-token prompt, all of them for the 128-token one, every
decode step); the cache after the last step must equal the oracle's write bit
for bit, and the slots no step wrote must still hold their poison.
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import oracle
import workloads as W
from tests.gpu_common import CODE, DEV, assert_close, bits, dev, f64, host_values, i32, workspace

pytestmark = pytest.mark.gpu


def run_flow(seed, heads, kvh, d, theta, prompt, steps, max_seq, window=0, with_sinks=False,
             prefill_sel=None):
    g = W.streams(seed)
    n = prompt + steps
    q_t, q64 = host_values(W.normal(g["q"], (n, heads, d)), "bf16")
    k_t, k64 = host_values(W.normal(g["k"], (n, kvh, d)), "bf16")
    v_t, v64 = host_values(W.normal(g["v"], (n, kvh, d)), "bf16")
    sk_t, sk64 = host_values(W.normal(g["sinks"], (heads,)), "bf16")
    sinks = dev(sk_t) if with_sinks else None
    pos = np.arange(n, dtype=np.int32)
    q, k, v = dev(q_t), dev(k_t), dev(v_t)
    bf = torch.bfloat16
    tab = torch.empty((2, max_seq, d // 2), dtype=bf, device=DEV)
    ck = torch.full((1, kvh, max_seq, d), float("nan"), dtype=bf, device=DEV)
    cv = torch.full((1, kvh, max_seq, d), float("nan"), dtype=bf, device=DEV)
    poison = bits(ck)
    dpos = i32(pos)
    gqa.gqa_rope_table(d, max_seq, theta, gqa.GQA_BF16, tab)
    # prompt: rope + write, then the causal prefill (one segment)
    gqa.gqa_rope_write_kv(prompt, heads, kvh, d, gqa.GQA_BF16, q[:prompt], k[:prompt], v[:prompt],
                          dpos[:prompt], tab, max_seq, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, 1, max_seq,
                          None, None, None, 0, 0)
    out_p = torch.empty((prompt, heads, d), dtype=bf, device=DEV)
    nb = gqa.gqa_prefill_packed_workspace(prompt, heads, kvh, d)
    ws, nb = workspace(nb)
    gqa.gqa_prefill_packed(prompt, heads, kvh, d, gqa.GQA_BF16, 0.0, window, sinks, q[:prompt],
                           k[:prompt], v[:prompt], dpos[:prompt], i32(np.zeros(prompt, np.int32)),
                           out_p, ws, nb)
    # decode steps: each writes its token, then attends the cache at its position
    out_d = torch.empty((steps, heads, d), dtype=bf, device=DEV)
    wsd, nbd = workspace(gqa.gqa_decode_rows_workspace(1, heads, kvh, d, max_seq))
    for i in range(steps):
        t = prompt + i
        gqa.gqa_rope_write_kv(1, heads, kvh, d, gqa.GQA_BF16, q[t:t + 1], k[t:t + 1], v[t:t + 1],
                              dpos[t:t + 1], tab, max_seq, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, 1, max_seq,
                              None, None, None, 0, 0)
        gqa.gqa_decode_rows(1, heads, kvh, d, gqa.GQA_BF16, 0.0, window, sinks, q[t:t + 1], ck, cv,
                            max_seq, dpos[t:t + 1], out_d[i:i + 1], wsd, nbd)
    torch.cuda.synchronize()

    o = oracle.default()
    c, s = o.rope_tables(max_seq, d, theta, "bf16")
    q64r = o.rope(q64, pos, c, s, "bf16")
    k64r = o.rope(k64, pos, c, s, "bf16")
    assert np.array_equal(f64(q), q64r), "rotated q differs from the oracle"
    ssk = sk64 if with_sinks else None
    seg = np.zeros(prompt, np.int32)
    sel = prefill_sel
    ref_p = o.packed(q64r[:prompt], k64r[:prompt], v64[:prompt], pos[:prompt], seg, window=window,
                     sinks=ssk, sel=sel)
    got_p = f64(out_p) if sel is None else f64(out_p)[sel]
    assert_close(got_p, ref_p, "bf16", f"prefill S={prompt} W={window}")
    nan_cache = np.full((1, kvh, max_seq, d), np.nan)
    ock, ocv, _ = o.write_contiguous(k64r, v64, pos, nan_cache, nan_cache.copy())
    ref_d = np.concatenate([o.decode_rows(q64r[prompt + i:prompt + i + 1], ock, ocv,
                                          pos[prompt + i:prompt + i + 1], window=window, sinks=ssk)
                            for i in range(steps)])
    assert_close(f64(out_d), ref_d, "bf16", f"{steps} decode steps W={window}")
    # the cache: written slots bit-equal to the oracle's, the rest untouched
    ref_bits = bits(torch.from_numpy(ock).to(bf))
    got = bits(ck)
    assert np.array_equal(got[:, :, :n], ref_bits[:, :, :n]), "cache k differs"
    assert np.array_equal(bits(cv)[:, :, :n], bits(torch.from_numpy(ocv).to(bf))[:, :, :n]), "cache v differs"
    assert np.array_equal(got[:, :, n:], poison[:, :, n:]), "a slot past the last step was written"


def test_tiny_llama_end_to_end():
    wl = W.TINY_LLAMA
    print(f"[case] {wl.name}: end to end", flush=True)
    run_flow(1, wl.heads, wl.kv_heads, wl.head_dim, wl.theta, wl.extra["prefill"],
             wl.extra["decode_steps"], wl.extra["max_seq"])


@pytest.mark.parametrize("window", [128, 0])
def test_gpt_oss_layer_end_to_end(window):
    wl = W.GPT_OSS_SINK
    s = wl.extra["prefill"]
    print(f"[case] {wl.name}: end to end, W={window}", flush=True)
    g = W.streams(55)
    sel = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 129, s - 1],
                                    W.sample_indices(s, 150, g["extra"])])).astype(np.int32)
    run_flow(5 + window, wl.heads, wl.kv_heads, wl.head_dim, wl.theta, s, wl.extra["decode_steps"],
             wl.extra["max_seq"], window=window, with_sinks=True, prefill_sel=sel)
