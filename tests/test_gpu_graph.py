"""GPU: the library's launches captured in a HIP graph (torch.cuda.graph) and
replayed give the eager results bit for bit.

The library allocates, synchronizes and clears nothing on its own, so a
caller may capture its calls. Each replay here follows eager work of the
program itself (restoring the rotated q/k, an unrelated torch kernel) and a
host synchronization, and every replay is compared with the eager run.
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import workloads as W
from tests.gpu_common import DEV, dev, host_values, i32, workspace

pytestmark = pytest.mark.gpu


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_graph_replay_matches_eager():
    print("[case] graph capture: decode loop (contiguous, paged, f32) + packed prefill", flush=True)
    heads, kvh, d, max_seq, steps = 16, 4, 128, 2048, 6  # 2048 slots: split decode + merge
    g = W.streams(777)
    n = 96 + steps
    q0 = dev(host_values(W.normal(g["q"], (n, heads, d)), "bf16")[0])
    k0 = dev(host_values(W.normal(g["k"], (n, kvh, d)), "bf16")[0])
    v0 = dev(host_values(W.normal(g["v"], (n, kvh, d)), "bf16")[0])
    q, k, v = q0.clone(), k0.clone(), v0.clone()
    pos = torch.arange(n, dtype=torch.int32, device=DEV)
    rows = torch.zeros(n, dtype=torch.int32, device=DEV)
    tab = torch.empty((2, max_seq, d // 2), dtype=torch.bfloat16, device=DEV)
    gqa.gqa_rope_table(d, max_seq, 500000.0, gqa.GQA_BF16, tab)
    ck = torch.zeros((1, kvh, max_seq, d), dtype=torch.bfloat16, device=DEV)
    cv = torch.zeros_like(ck)
    # Paged pool: row 0's pages scattered by a seeded table (PageSize 64).
    num_pages, pages = 40, max_seq // 64
    perm = g["index"].permutation(num_pages)[:pages].astype(np.int32)
    table = i32(perm.reshape(1, pages))
    pk = torch.zeros((num_pages, kvh, 64, d), dtype=torch.bfloat16, device=DEV)
    pvv = torch.zeros_like(pk)
    # f32 contiguous cache, written by the same steps (no rotation: a GPT-2 layer).
    q32 = dev(host_values(W.normal(g["extra"], (n, heads, d)), "f32")[0])
    k32 = q32[:, :kvh].contiguous()
    v32 = q32[:, kvh:2 * kvh].contiguous()
    ck32 = torch.zeros((1, kvh, max_seq, d), dtype=torch.float32, device=DEV)
    cv32 = torch.zeros_like(ck32)
    seg = torch.zeros(96, dtype=torch.int32, device=DEV)

    outs = [torch.empty((1, heads, d), dtype=torch.bfloat16, device=DEV) for _ in range(steps)]
    outs_p = [torch.empty((1, heads, d), dtype=torch.bfloat16, device=DEV) for _ in range(steps)]
    outs_f = [torch.empty((1, heads, d), dtype=torch.float32, device=DEV) for _ in range(steps)]
    out_pre = torch.empty((96, heads, d), dtype=torch.bfloat16, device=DEV)
    wsd, nbd = workspace(gqa.gqa_decode_rows_workspace(1, heads, kvh, d, max_seq))
    wsp, nbp = workspace(gqa.gqa_decode_paged_workspace(1, pages, heads, kvh, d))
    wsf, nbf = workspace(gqa.gqa_decode_rows_workspace(1, heads, kvh, d, max_seq))
    wspre, nbpre = workspace(gqa.gqa_prefill_packed_workspace(96, heads, kvh, d))

    def work():
        # Prefill of 96 tokens: rope + contiguous and paged writes, attention.
        gqa.gqa_rope_write_kv(96, heads, kvh, d, gqa.GQA_BF16, q[:96], k[:96], v[:96], pos[:96], tab,
                              max_seq, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, 1, max_seq, rows[:96], None,
                              None, 0, 0)
        gqa.gqa_rope_write_kv(96, heads, kvh, d, gqa.GQA_BF16, None, k0[:96], v[:96], pos[:96], None,
                              0, gqa.GQA_CACHE_PAGED_TABLE, pk, pvv, num_pages, 64, rows[:96], None,
                              table, 1, pages)
        gqa.gqa_rope_write_kv(96, heads, kvh, d, gqa.GQA_F32, None, k32[:96], v32[:96], pos[:96], None,
                              0, gqa.GQA_CACHE_CONTIGUOUS, ck32, cv32, 1, max_seq, rows[:96], None,
                              None, 0, 0)
        gqa.gqa_prefill_packed(96, heads, kvh, d, gqa.GQA_BF16, 0.0, 0, None, q[:96], k[:96], v[:96],
                               pos[:96], seg, out_pre, wspre, nbpre)
        for s in range(steps):
            i = 96 + s
            gqa.gqa_rope_write_kv(1, heads, kvh, d, gqa.GQA_BF16, q[i:i + 1], k[i:i + 1], v[i:i + 1],
                                  pos[i:i + 1], tab, max_seq, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, 1,
                                  max_seq, rows[i:i + 1], None, None, 0, 0)
            gqa.gqa_decode_rows(1, heads, kvh, d, gqa.GQA_BF16, 0.0, 0, None, q[i:i + 1], ck, cv,
                                max_seq, pos[i:i + 1], outs[s], wsd, nbd)
            gqa.gqa_rope_write_kv(1, heads, kvh, d, gqa.GQA_BF16, None, k0[i:i + 1], v[i:i + 1],
                                  pos[i:i + 1], None, 0, gqa.GQA_CACHE_PAGED_TABLE, pk, pvv,
                                  num_pages, 64, rows[i:i + 1], None, table, 1, pages)
            gqa.gqa_decode_paged(1, pages, heads, kvh, d, gqa.GQA_BF16, 0.0, 0, None, q[i:i + 1], pk,
                                 pvv, num_pages, pos[i:i + 1], table, outs_p[s], wsp, nbp)
            gqa.gqa_rope_write_kv(1, heads, kvh, d, gqa.GQA_F32, None, k32[i:i + 1], v32[i:i + 1],
                                  pos[i:i + 1], None, 0, gqa.GQA_CACHE_CONTIGUOUS, ck32, cv32, 1,
                                  max_seq, rows[i:i + 1], None, None, 0, 0)
            gqa.gqa_decode_rows(1, heads, kvh, d, gqa.GQA_F32, 0.0, 0, None, q32[i:i + 1], ck32, cv32,
                                max_seq, pos[i:i + 1], outs_f[s], wsf, nbf)

    def restore():
        # The rope pass rotates q and k in place; caches start empty again.
        q.copy_(q0)
        k.copy_(k0)
        for c in (ck, cv, pk, pvv, ck32, cv32):
            c.zero_()

    def results():
        return [x.clone() for x in [out_pre] + outs + outs_p + outs_f + [ck, pk]]

    restore()
    work()
    torch.cuda.synchronize()
    ref = results()
    assert all(torch.isfinite(x.float()).all() for x in ref)

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        for x in [out_pre] + outs + outs_p + outs_f:
            x.fill_(float("nan"))
        _ = torch.randn(4096, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = results()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert _same(a, b), f"replay {rep}: result {i} differs from the eager run"


def test_graph_replay_training_pair_matches_eager():
    print("[case] graph capture: packed forward with lse + backward", flush=True)
    heads, kvh, d = 8, 2, 128
    g = W.streams(778)
    lengths, pos_h, seg_h = W.segment_layout(700, 20, 300, g["index"])
    p = len(pos_h)
    q = dev(host_values(W.normal(g["q"], (p, heads, d)), "bf16")[0])
    k = dev(host_values(W.normal(g["k"], (p, kvh, d)), "bf16")[0])
    v = dev(host_values(W.normal(g["v"], (p, kvh, d)), "bf16")[0])
    gd = dev(host_values(W.normal(g["extra"], (p, heads, d)), "bf16")[0])
    pos, seg = i32(pos_h), i32(seg_h)
    bf = torch.bfloat16
    out = torch.empty((p, heads, d), dtype=bf, device=DEV)
    lse = torch.empty((p, heads), dtype=torch.float32, device=DEV)
    dq = torch.empty((p, heads, d), dtype=bf, device=DEV)
    dk = torch.empty((p, kvh, d), dtype=bf, device=DEV)
    dv = torch.empty((p, kvh, d), dtype=bf, device=DEV)
    wsf, nbf = workspace(gqa.gqa_prefill_packed_workspace(p, heads, kvh, d))
    wsb, nbb = workspace(gqa.gqa_prefill_packed_backward_workspace(p, heads, kvh, d))

    def work():
        gqa.gqa_prefill_packed_lse(p, heads, kvh, d, gqa.GQA_BF16, 0.0, 64, q, k, v, pos, seg, out, lse,
                                   wsf, nbf)
        gqa.gqa_prefill_packed_backward(p, heads, kvh, d, gqa.GQA_BF16, 0.0, 64, q, k, v, out, gd, lse,
                                        pos, seg, dq, dk, dv, wsb, nbb)

    def results():
        return [x.clone() for x in (out, lse, dq, dk, dv)]

    work()
    torch.cuda.synchronize()
    ref = results()
    assert all(torch.isfinite(x.float()).all() for x in ref)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (out, lse, dq, dk, dv):
            x.fill_(float("nan"))
        _ = torch.randn(4096, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(results(), ref)):
            assert _same(a, b), f"replay {rep}: result {i} differs from the eager run"


def test_graph_replay_sorted_decode_and_step_paged():
    """The launches whose dispatch order is ranked on the device (sorted decode:
    matrix-core bf16 paged rows and vector-ALU f32 contiguous rows) and the
    single-grid step_paged (decode and chunk workgroups in one launch)."""
    print("[case] graph capture: sorted paged/rows decode + step_paged", flush=True)
    g = W.streams(779)
    bf = torch.bfloat16
    # bf16 paged decode, 64 rows x 8 KV heads: one split, ranked rows.
    heads, kvh, d, num_pages = 32, 8, 128, 700
    lengths, dpos, table = W.paged_layout(64, 1, 600, num_pages, 64, g["index"], max_len=640)
    dpos = dpos.copy()
    dpos[3] = -1                                     # a row that attends nothing
    pk = dev(host_values(W.normal(g["pool_k"], (num_pages, kvh, 64, d)), "bf16")[0])
    pv = dev(host_values(W.normal(g["pool_v"], (num_pages, kvh, 64, d)), "bf16")[0])
    qd = dev(host_values(W.normal(g["q"], (64, heads, d)), "bf16")[0])
    dpos_t, table_t = i32(dpos), i32(table)
    pages = table.shape[1]
    out_d = torch.empty((64, heads, d), dtype=bf, device=DEV)
    wsd, nbd = workspace(gqa.gqa_decode_paged_workspace(64, pages, heads, kvh, d))
    # f32 contiguous decode, 32 rows x 12 heads (one head per KV head): ranked rows.
    fh, fd, fmax = 12, 64, 400
    fpos = i32(g["extra"].integers(0, fmax, 32).astype(np.int32))
    fk = dev(host_values(W.normal(g["k"], (32, fh, fmax, fd)), "f32")[0])
    fv = dev(host_values(W.normal(g["v"], (32, fh, fmax, fd)), "f32")[0])
    fq = dev(host_values(W.normal(g["q"], (32, fh, fd)), "f32")[0])
    out_f = torch.empty((32, fh, fd), dtype=torch.float32, device=DEV)
    wsf, nbf = workspace(gqa.gqa_decode_rows_workspace(32, fh, fh, fd, fmax))
    # step_paged: the last 48 positions of rows 0, 5, 9 as the chunk, all 64 rows decode.
    crow, cpos = [], []
    for r in (0, 5, 9):
        c = min(int(lengths[r]), 48)
        crow += [r] * c
        cpos += list(range(int(lengths[r]) - c, int(lengths[r])))
    p = len(cpos)
    qs = dev(host_values(W.normal(g["sinks"], (p + 64, heads, d)), "bf16")[0])
    crow_t, cpos_t = i32(np.asarray(crow, np.int32)), i32(np.asarray(cpos, np.int32))
    out_s = torch.empty((p + 64, heads, d), dtype=bf, device=DEV)
    wss, nbs = workspace(gqa.gqa_step_paged_workspace(p, 64, pages, heads, kvh, d))

    def work():
        gqa.gqa_decode_paged(64, pages, heads, kvh, d, gqa.GQA_BF16, 0.0, 0, None, qd, pk, pv,
                             num_pages, dpos_t, table_t, out_d, wsd, nbd)
        gqa.gqa_decode_rows(32, fh, fh, fd, gqa.GQA_F32, 0.0, 0, None, fq, fk, fv, fmax, fpos,
                            out_f, wsf, nbf)
        gqa.gqa_step_paged(p, 64, pages, heads, kvh, d, gqa.GQA_BF16, 0.0, 0, None, qs, crow_t,
                           cpos_t, pk, pv, num_pages, table_t, dpos_t, out_s, wss, nbs)

    outs = (out_d, out_f, out_s)
    work()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    assert all(torch.isfinite(x.float()).all() for x in ref)
    assert bool((ref[0][3] == 0).all())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        _ = torch.randn(4096, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same(a, b), f"replay {rep}: result {i} differs from the eager run"
