"""GPU: checked mode. With gqa_set_checked(1) a call validates its index
arguments on the device first and returns GQA_ERR_INDEX, enqueuing nothing
else, when a row, position, slot or page id is out of range; with valid
indices it gives exactly the unchecked result. Out-of-range indices are only
reported -- the check reads each index once and addresses nothing with it --
so no case here touches memory outside its buffers.
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import workloads as W
from tests.gpu_common import CODE, DEV, bits, dev, host_values, i32, workspace
from tests.test_gpu_decode import paged_case, run_decode_paged, run_decode_rows, contiguous_case

pytestmark = pytest.mark.gpu


@pytest.fixture
def checked():
    prev = gqa.gqa_set_checked(1)
    yield
    gqa.gqa_set_checked(prev)


def expect_index_error(fn, *args):
    with pytest.raises(gqa.GQAError) as e:
        fn(*args)
    assert e.value.status == gqa.GQA_ERR_INDEX, e.value.status


def rope_write_args(n, kvh, d, cache_kind, cache_k, cache_v, dim0, seq, pos, rows=None, slots=None,
                    table=None):
    g = W.streams(n + 7)
    k_t, _ = host_values(W.normal(g["k"], (n, kvh, d)), "bf16")
    v_t, _ = host_values(W.normal(g["v"], (n, kvh, d)), "bf16")
    tr, tp = (0, 0) if table is None else table.shape
    return (n, 8, kvh, d, CODE["bf16"], None, dev(k_t), dev(v_t), i32(pos), None, 0, cache_kind,
            cache_k, cache_v, dim0, seq, None if rows is None else i32(rows),
            None if slots is None else i32(slots), None if table is None else i32(table), tr, tp)


def test_checked_rope_write(checked):
    kvh, d, batch, max_seq, n = 2, 64, 3, 128, 10
    ck = torch.full((batch, kvh, max_seq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    cv = ck.clone()
    before = bits(ck)
    pos = np.arange(n, dtype=np.int32)
    rows = np.ones(n, dtype=np.int32)
    print("[case] checked rope_write_kv contiguous", flush=True)
    bad_rows = rows.copy()
    bad_rows[4] = batch + 2
    expect_index_error(gqa.gqa_rope_write_kv,
                       *rope_write_args(n, kvh, d, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, batch, max_seq, pos,
                                        rows=bad_rows))
    bad_pos = pos.copy()
    bad_pos[2] = max_seq
    expect_index_error(gqa.gqa_rope_write_kv,
                       *rope_write_args(n, kvh, d, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, batch, max_seq,
                                        bad_pos, rows=rows))
    torch.cuda.synchronize()
    assert np.array_equal(bits(ck), before), "a rejected call wrote the cache"
    # valid: checked and unchecked write the same bits
    gqa.gqa_rope_write_kv(*rope_write_args(n, kvh, d, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, batch, max_seq,
                                           pos, rows=rows))
    ck2, cv2 = torch.full_like(ck, float("nan")), torch.full_like(cv, float("nan"))
    prev = gqa.gqa_set_checked(0)
    gqa.gqa_rope_write_kv(*rope_write_args(n, kvh, d, gqa.GQA_CACHE_CONTIGUOUS, ck2, cv2, batch,
                                           max_seq, pos, rows=rows))
    gqa.gqa_set_checked(prev)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ck), bits(ck2)) and np.array_equal(bits(cv), bits(cv2))

    print("[case] checked rope_write_kv paged (slots, table)", flush=True)
    num_pages = 6
    pk = torch.full((num_pages, kvh, 64, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    pv = pk.clone()
    pbefore = bits(pk)
    slots = np.arange(n, dtype=np.int32) * 17
    bad_slots = slots.copy()
    bad_slots[9] = num_pages * 64
    expect_index_error(gqa.gqa_rope_write_kv,
                       *rope_write_args(n, kvh, d, gqa.GQA_CACHE_PAGED_SLOTS, pk, pv, num_pages, 64, pos,
                                        slots=bad_slots))
    table = np.array([[3, 1], [-1, 2]], dtype=np.int32)  # row 1's page 0 is missing
    trows = np.array([0] * 5 + [1] * 5, dtype=np.int32)
    tpos = np.array([0, 1, 70, 71, 72, 64, 65, 66, 3, 4], dtype=np.int32)  # row 1 writes page 0 at 3, 4
    expect_index_error(gqa.gqa_rope_write_kv,
                       *rope_write_args(n, kvh, d, gqa.GQA_CACHE_PAGED_TABLE, pk, pv, num_pages, 64, tpos,
                                        rows=trows, table=table))
    torch.cuda.synchronize()
    assert np.array_equal(bits(pk), pbefore), "a rejected call wrote the pool"
    gqa.gqa_rope_write_kv(*rope_write_args(n, kvh, d, gqa.GQA_CACHE_PAGED_SLOTS, pk, pv, num_pages, 64,
                                           pos, slots=slots))


def test_checked_decode(checked):
    heads, kvh, d = 8, 2, 64
    print("[case] checked decode_rows", flush=True)
    pos = np.array([5, 60, 127], dtype=np.int32)
    (q, ck, cv), _, _ = contiguous_case(5100, 3, heads, kvh, d, 128, pos, "bf16")
    out = run_decode_rows(q, ck, cv, pos, heads, kvh, d, "bf16")
    prev = gqa.gqa_set_checked(0)
    ref = run_decode_rows(q, ck, cv, pos, heads, kvh, d, "bf16")
    gqa.gqa_set_checked(prev)
    assert np.array_equal(bits(out), bits(ref))
    bad = pos.copy()
    bad[1] = 128
    expect_index_error(run_decode_rows, q, ck, cv, bad, heads, kvh, d, "bf16")
    bad[1] = -1
    expect_index_error(run_decode_rows, q, ck, cv, bad, heads, kvh, d, "bf16")

    print("[case] checked decode_paged", flush=True)
    lengths = np.array([100, 300, 64], dtype=np.int64)
    (q, pk, pv), _, ppos, table, _, _ = paged_case(5101, 3, heads, kvh, d, lengths, 6, 20, "bf16")
    out = run_decode_paged(q, pk, pv, ppos, table, heads, kvh, d, "bf16")
    prev = gqa.gqa_set_checked(0)
    ref = run_decode_paged(q, pk, pv, ppos, table, heads, kvh, d, "bf16")
    gqa.gqa_set_checked(prev)
    assert np.array_equal(bits(out), bits(ref))
    bad_t = table.copy()
    bad_t[1, 2] = -1                         # a page row 1 attends
    expect_index_error(run_decode_paged, q, pk, pv, ppos, bad_t, heads, kvh, d, "bf16")
    bad_t = table.copy()
    bad_t[0, 1] = 20                         # past the pool
    expect_index_error(run_decode_paged, q, pk, pv, ppos, bad_t, heads, kvh, d, "bf16")
    # a window that starts past the broken page: nothing it reads is invalid
    win_t = table.copy()
    win_t[1, 0] = -1
    run_decode_paged(q, pk, pv, ppos, win_t, heads, kvh, d, "bf16", window=100)
    expect_index_error(run_decode_paged, q, pk, pv, ppos, win_t, heads, kvh, d, "bf16")


def test_checked_prefill_cached_and_step(checked):
    heads, kvh, d = 8, 2, 64
    g = W.streams(5102)
    n, batch, max_seq = 40, 2, 256
    q_t, _ = host_values(W.normal(g["q"], (n, heads, d)), "bf16")
    k_t, _ = host_values(W.normal(g["k"], (batch, kvh, max_seq, d)), "bf16")
    ck, cv = dev(k_t), dev(k_t.clone())
    rows = np.array([0] * 20 + [1] * 20, dtype=np.int32)
    pos = np.concatenate([np.arange(100, 120), np.arange(30, 50)]).astype(np.int32)
    out = torch.full((n, heads, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws, nb = workspace(gqa.gqa_prefill_cached_workspace(n, heads, kvh, d))

    def call(rws, ps):
        gqa.gqa_prefill_cached(n, heads, kvh, d, CODE["bf16"], 0.0, 0, None, dev(q_t), i32(rws), i32(ps),
                               gqa.GQA_CACHE_CONTIGUOUS, ck, cv, batch, max_seq, None, 0, 0, out, ws, nb)
    print("[case] checked prefill_cached", flush=True)
    call(rows, pos)
    bad = rows.copy()
    bad[3] = -1
    expect_index_error(call, bad, pos)
    badp = pos.copy()
    badp[30] = max_seq + 1
    expect_index_error(call, rows, badp)

    print("[case] checked step_paged (nothing enqueued on error)", flush=True)
    lengths = np.array([200, 90], dtype=np.int64)
    (qd, pk, pv), _, ppos, table, _, _ = paged_case(5103, 2, heads, kvh, d, lengths, 4, 12, "bf16")
    p = 8
    tok_rows = np.array([0] * 4 + [1] * 4, dtype=np.int32)
    tok_pos = np.array([190, 191, 192, 193, 80, 81, 82, 83], dtype=np.int32)
    qs = torch.cat([dev(q_t[:p]), qd], 0)
    sout = torch.full((p + 2, heads, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    sws, snb = workspace(gqa.gqa_step_paged_workspace(p, 2, 4, heads, kvh, d))

    def step(tbl):
        gqa.gqa_step_paged(p, 2, 4, heads, kvh, d, CODE["bf16"], 0.0, 0, None, qs, i32(tok_rows),
                           i32(tok_pos), pk, pv, 12, i32(tbl), i32(ppos), sout, sws, snb)
    bad_t = table.copy()
    bad_t[0, 3] = 99                         # row 0's decode token reads page 3 (positions 192..199)
    expect_index_error(step, bad_t)
    torch.cuda.synchronize()
    assert torch.isnan(sout.float()).all(), "a rejected step wrote its output"
    step(table)
    torch.cuda.synchronize()
    assert torch.isfinite(sout.float()).all()
