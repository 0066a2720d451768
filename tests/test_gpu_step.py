"""GPU parity: `step_packed` and `step_paged` -- one call over prefill tokens
and one decode token per row -- against the fp64 oracle's two parts (packed
attention + decode_rows; chunk over the paged prefix + decode_paged).
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import oracle
import workloads as W
from tests.gpu_common import CODE, DEV, assert_close, dev, f64, host_values, i32, workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("heads,kvh,d,window,use_sinks", [(32, 8, 128, 0, False),
                                                        (64, 8, 64, 128, True),
                                                        (8, 8, 64, 0, True)])
def test_step_packed(heads, kvh, d, window, use_sinks):
    print(f"[case] step_packed H={heads} KvH={kvh} D={d} W={window} sinks={use_sinks}", flush=True)
    g = W.streams(2400 + heads + d)
    batch, max_seq = 6, 700
    lengths, pos, seg = W.segment_layout(300, 20, 160, g["index"])
    p = len(pos)
    step_pos = g["index"].integers(0, max_seq - 1, batch).astype(np.int32)
    ck = W.normal(g["pool_k"], (batch, kvh, max_seq, d))
    cv = W.normal(g["pool_v"], (batch, kvh, max_seq, d))
    for b in range(batch):
        ck[b, :, step_pos[b] + 1:] = np.nan
        cv[b, :, step_pos[b] + 1:] = np.nan
    ck_t, ck64 = host_values(ck, "bf16")
    cv_t, cv64 = host_values(cv, "bf16")
    q_t, q64 = host_values(W.normal(g["q"], (batch + p, heads, d)), "bf16")
    k_t, k64 = host_values(W.normal(g["k"], (p, kvh, d)), "bf16")
    v_t, v64 = host_values(W.normal(g["v"], (p, kvh, d)), "bf16")
    sk_t, sk64 = host_values(W.normal(g["sinks"], (heads,)), "bf16")
    sinks = dev(sk_t) if use_sinks else None
    out = torch.full((batch + p, heads, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws, nb = workspace(gqa.gqa_step_packed_workspace(batch, p, heads, kvh, d, max_seq))
    gqa.gqa_step_packed(batch, p, heads, kvh, d, CODE["bf16"], 0.0, window, sinks, dev(q_t),
                        dev(k_t), dev(v_t), i32(pos), i32(seg), dev(ck_t), dev(cv_t), max_seq,
                        i32(step_pos), out, ws, nb)
    torch.cuda.synchronize()
    o = oracle.default()
    sk = sk64 if use_sinks else None
    ref_dec = o.decode_rows(q64[:batch], np.nan_to_num(ck64), np.nan_to_num(cv64), step_pos,
                            window=window, sinks=sk)
    ref_pre = o.packed(q64[batch:], k64, v64, pos, seg, window=window, sinks=sk)
    got = f64(out)
    assert_close(got[:batch], ref_dec, "bf16", "step_packed decode part")
    assert_close(got[batch:], ref_pre, "bf16", "step_packed packed part")


# Up to 16 query heads per KV head the decode tokens run in the same grid as
# the chunk (matrix-core decode workgroups placed after the first half of the
# prefill tiles); with more (G = 32 here) the decode runs as its own
# vector-ALU pass before the chunk.
@pytest.mark.parametrize("heads,kvh,d,window,use_sinks,bad_page", [
    (32, 8, 128, 0, False, False), (64, 8, 64, 0, False, False),
    (64, 8, 64, 128, True, True), (32, 2, 128, 300, False, True), (32, 1, 64, 0, True, False)])
def test_step_paged(heads, kvh, d, window, use_sinks, bad_page):
    print(f"[case] step_paged H={heads} KvH={kvh} D={d} W={window} sinks={use_sinks} "
          f"bad_page={bad_page}", flush=True)
    g = W.streams(2500 + heads + d)
    rows, num_pages = 12, 200
    lengths, dec_pos, table = W.paged_layout(rows, 40, 900, num_pages, 64, g["index"], max_len=1024)
    pk = W.normal(g["pool_k"], (num_pages, kvh, 64, d))
    pv = W.normal(g["pool_v"], (num_pages, kvh, 64, d))
    pk_t, pk64 = host_values(pk, "bf16")
    pv_t, pv64 = host_values(pv, "bf16")
    # chunk tokens: the last min(L_r, 70) positions of rows 0, 3, 5, 8 (row-contiguous)
    crow, cpos = [], []
    for r in (0, 3, 5, 8):
        c = min(int(lengths[r]), 70)
        crow += [r] * c
        cpos += list(range(int(lengths[r]) - c, int(lengths[r])))
    crow = np.asarray(crow, np.int32)
    cpos = np.asarray(cpos, np.int32)
    p = len(cpos)
    if bad_page:
        # a page outside the pool in a decode-only row and one in a chunk row:
        # both contribute no keys; row 11 attends nothing
        table = table.copy()
        table[2, 0] = num_pages
        table[5, 0] = -3
        dec_pos = dec_pos.copy()
        dec_pos[11] = -1
    q_t, q64 = host_values(W.normal(g["q"], (p + rows, heads, d)), "bf16")
    sk_t, sk64 = host_values(W.normal(g["sinks"], (heads,)), "bf16")
    sinks, sk = (dev(sk_t), sk64) if use_sinks else (None, None)
    out = torch.full((p + rows, heads, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws, nb = workspace(gqa.gqa_step_paged_workspace(p, rows, table.shape[1], heads, kvh, d))
    gqa.gqa_step_paged(p, rows, table.shape[1], heads, kvh, d, CODE["bf16"], 0.0, window, sinks,
                       dev(q_t), i32(crow), i32(cpos), dev(pk_t), dev(pv_t), num_pages, i32(table),
                       i32(dec_pos), out, ws, nb)
    torch.cuda.synchronize()
    o = oracle.default()
    ref_pre = o.prefill_paged(q64[:p], crow, cpos, pk64, pv64, table, window=window, sinks=sk)
    ref_dec = o.decode_paged(q64[p:], pk64, pv64, dec_pos, table, window=window, sinks=sk)
    got = f64(out)
    assert_close(got[:p], ref_pre, "bf16", "step_paged chunk part")
    assert_close(got[p:], ref_dec, "bf16", "step_paged decode part")
    if bad_page:
        assert np.all(got[p + 11] == 0.0)
