"""GPU parity: decode over a contiguous cache (decode_rows) and through a page
table (decode_paged), against the fp64 oracle.

Caches are filled directly from the seeded generator (never by the HIP write
path) and poisoned with NaN past every row's position, so a stray read shows
up as a non-finite output. Index handling is checked exactly with mask
probes: q = 0 makes the weights uniform over the attended set, and a one-hot
value per probed key makes each output dimension 0 or not by membership.
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


def run_decode_rows(q, ck, cv, pos, heads, kvh, d, dtype, window=0, sinks=None, scale=0.0):
    batch, max_seq = ck.shape[0], ck.shape[2]
    out = torch.full((batch, heads, d), float("nan"), dtype=TORCH_DT[dtype], device=DEV)
    ws, nb = workspace(gqa.gqa_decode_rows_workspace(batch, heads, kvh, d, max_seq))
    gqa.gqa_decode_rows(batch, heads, kvh, d, CODE[dtype], scale, window, sinks, q, ck, cv,
                        max_seq, i32(pos), out, ws, nb)
    torch.cuda.synchronize()
    return out


def run_decode_paged(q, pk, pv, pos, table, heads, kvh, d, dtype, window=0, sinks=None):
    rows, pages = table.shape
    num_pages = pk.shape[0]
    out = torch.full((rows, heads, d), float("nan"), dtype=TORCH_DT[dtype], device=DEV)
    ws, nb = workspace(gqa.gqa_decode_paged_workspace(rows, pages, heads, kvh, d))
    gqa.gqa_decode_paged(rows, pages, heads, kvh, d, CODE[dtype], 0.0, window, sinks, q, pk, pv,
                         num_pages, i32(pos), i32(table), out, ws, nb)
    torch.cuda.synchronize()
    return out


def contiguous_case(seed, batch, heads, kvh, d, max_seq, pos, dtype):
    """Cache rows filled up to each row's position, NaN past it."""
    g = W.streams(seed)
    q_t, q64 = host_values(W.normal(g["q"], (batch, heads, d)), dtype)
    k_t, k64 = host_values(W.normal(g["k"], (batch, kvh, max_seq, d)), dtype)
    v_t, v64 = host_values(W.normal(g["v"], (batch, kvh, max_seq, d)), dtype)
    for b in range(batch):
        p = int(pos[b])
        if p + 1 < max_seq:
            k_t[b, :, max(p + 1, 0):] = float("nan")
            v_t[b, :, max(p + 1, 0):] = float("nan")
    k64 = k_t.to(torch.float64).numpy()
    v64 = v_t.to(torch.float64).numpy()
    return (dev(q_t), dev(k_t), dev(v_t)), (q64, k64, v64), g


# --- GPT-2 shaped MHA decode_rows, f32 (full size) ----------------------------
def test_decode_rows_gpt2_f32():
    wl = W.GPT2_DECODE_ROWS
    b, ms = wl.extra["batch"], wl.extra["max_seq"]
    print(f"[case] {wl.name}", flush=True)
    g = W.streams(2)
    pos = W.uniform_positions(b, 0, ms - 1, g["extra"])
    pos[0], pos[1] = 0, ms - 1
    dv, hv, _ = contiguous_case(2, b, wl.heads, wl.kv_heads, wl.head_dim, ms, pos, "f32")
    out = run_decode_rows(*dv, pos, wl.heads, wl.kv_heads, wl.head_dim, "f32")
    ref = oracle.default().decode_rows(*hv, pos)
    assert_close(f64(out), ref, "f32", "gpt2 decode_rows f32")


# --- one workgroup per (row, head chunk), launched longest row first ---------------
# With at most 64 rows and at least 256 (row, head chunk) units the vector-ALU
# kernel takes each row whole and ranks the rows by attended keys on the
# device. Ties, empty rows, positions past the cache, windows and sinks all
# change the ranking; 64 rows is the largest ranked batch, 65 falls back to
# split rows with a merge.
@pytest.mark.parametrize("batch,heads", [(24, 16), (64, 4), (65, 4)])
def test_decode_rows_sorted_dispatch(batch, heads):
    kvh, d, dtype, max_seq = heads, 64, "f32", 300
    print(f"[case] decode_rows sorted dispatch B={batch} H={heads} f32", flush=True)
    g = W.streams(300 + batch)
    pos = g["extra"].integers(0, max_seq, batch).astype(np.int32)
    pos[:4] = [-1, max_seq + 50, 17, 17]
    pos[4:7] = pos[7]                      # ties
    dv, hv, gg = contiguous_case(300 + batch, batch, heads, kvh, d, max_seq, pos, dtype)
    sinks_t, sinks64 = host_values(W.normal(gg["sinks"], (heads,)), dtype)
    o = oracle.default()
    for window, sk in ((0, None), (100, sinks_t), (1, None)):
        out = run_decode_rows(*dv, pos, heads, kvh, d, dtype, window=window,
                              sinks=None if sk is None else dev(sk))
        ref = o.decode_rows(*hv, pos, window=window, sinks=None if sk is None else sinks64)
        got = f64(out)
        assert np.all(got[0] == 0.0)
        assert_close(got, ref, dtype, f"sorted decode_rows B={batch} W={window}")


def test_decode_paged_sorted_dispatch():
    heads, kvh, d, dtype = 12, 12, 64, "f32"
    lengths = np.array([700, 1, 64, 65, 300, 300, 1024, 2, 128, 500] * 3, dtype=np.int64)
    rows = len(lengths)
    print(f"[case] decode_paged sorted dispatch rows={rows} f32", flush=True)
    dv, hv, pos, table, otable, g = paged_case(301, rows, heads, kvh, d, lengths, 16, 260, dtype)
    table = table.copy()
    otable = otable.copy()
    table[4, 2] = -1                       # an invalid page inside a row
    otable[4, 2] = -1
    o = oracle.default()
    for window in (0, 200):
        out = run_decode_paged(*dv, pos, table, heads, kvh, d, dtype, window=window)
        ref = o.decode_paged(hv[0], hv[1], hv[2], pos, otable, window=window)
        assert_close(f64(out), ref, dtype, f"sorted decode_paged W={window}")


# --- small and edge cases -------------------------------------------------------
# bf16 with up to 16 query heads per KV head runs on the matrix-core kernel;
# f32 and larger groups (32 here) on the vector-ALU kernel.
@pytest.mark.parametrize("heads,kvh,d,dtype", [(8, 8, 64, "bf16"), (32, 8, 128, "bf16"),
                                                (64, 8, 64, "bf16"), (16, 2, 128, "f32"),
                                                (6, 3, 64, "bf16"), (4, 4, 128, "f32"),
                                                (32, 1, 64, "bf16"), (16, 1, 128, "bf16")])
def test_decode_rows_shapes(heads, kvh, d, dtype):
    print(f"[case] decode_rows H={heads} KvH={kvh} D={d} {dtype}", flush=True)
    batch, max_seq = 7, 700
    pos = np.array([0, 1, 63, 64, 255, 256, 699], dtype=np.int32)
    dv, hv, g = contiguous_case(11 + heads, batch, heads, kvh, d, max_seq, pos, dtype)
    sinks_t, sinks64 = host_values(W.normal(g["sinks"], (heads,)), dtype)
    o = oracle.default()
    for window, sk in ((0, None), (1, None), (64, sinks_t), (300, None), (0, sinks_t)):
        out = run_decode_rows(*dv, pos, heads, kvh, d, dtype, window=window,
                              sinks=None if sk is None else dev(sk))
        ref = o.decode_rows(*hv, pos, window=window, sinks=None if sk is None else sinks64)
        assert_close(f64(out), ref, dtype, f"decode_rows W={window} sinks={sk is not None}")


def test_decode_rows_position_edges():
    """pos < 0 attends nothing (output 0); pos >= max_seq attends the whole row."""
    heads, kvh, d, dtype = 8, 4, 64, "bf16"
    batch, max_seq = 4, 130
    g = W.streams(5)
    q_t, q64 = host_values(W.normal(g["q"], (batch, heads, d)), dtype)
    k_t, k64 = host_values(W.normal(g["k"], (batch, kvh, max_seq, d)), dtype)
    v_t, v64 = host_values(W.normal(g["v"], (batch, kvh, max_seq, d)), dtype)
    pos = np.array([-1, 130, 5000, 129], dtype=np.int32)
    out = run_decode_rows(dev(q_t), dev(k_t), dev(v_t), pos, heads, kvh, d, dtype)
    ref = oracle.default().decode_rows(q64, k64, v64, pos)
    assert np.all(f64(out)[0] == 0.0)
    assert_close(f64(out), ref, dtype, "decode_rows position edges")
    out2 = run_decode_rows(dev(q_t), dev(k_t), dev(v_t), pos, heads, kvh, d, dtype, window=7)
    ref2 = oracle.default().decode_rows(q64, k64, v64, pos, window=7)
    assert_close(f64(out2), ref2, dtype, "decode_rows position edges, window 7")


# --- gpt-oss SinkAttention decode: B = 1, both layer kinds ---------------------------
@pytest.mark.parametrize("window", [128, 0])
def test_decode_rows_gpt_oss(window):
    wl = W.GPT_OSS_SINK
    ms = wl.extra["max_seq"]
    print(f"[case] {wl.name} decode, window {window}", flush=True)
    g = W.streams(5)
    sinks_t, sinks64 = host_values(W.normal(g["sinks"], (wl.heads,)), "bf16")
    for pos_v in (4096, 4200, 4351):
        pos = np.array([pos_v], dtype=np.int32)
        dv, hv, _ = contiguous_case(50 + pos_v, 1, wl.heads, wl.kv_heads, wl.head_dim, ms, pos,
                                    "bf16")
        out = run_decode_rows(*dv, pos, wl.heads, wl.kv_heads, wl.head_dim, "bf16", window=window,
                              sinks=dev(sinks_t))
        ref = oracle.default().decode_rows(*hv, pos, window=window, sinks=sinks64)
        assert_close(f64(out), ref, "bf16", f"gpt-oss decode pos {pos_v} W={window}")


# --- paged ------------------------------------------------------------------------------
def paged_case(seed, rows, heads, kvh, d, lengths, pages, num_pages, dtype, pool_seed_full=False):
    """Pool pages drawn for the used pages only; every other page is NaN, and
    so is every slot past a row's position in its last page."""
    g = W.streams(seed)
    need = -(-lengths // 64)
    perm = g["index"].permutation(num_pages).astype(np.int32)
    table = np.full((rows, pages), -1, np.int32)
    cur = 0
    for r in range(rows):
        table[r, :need[r]] = perm[cur:cur + need[r]]
        cur += int(need[r])
    pos = (lengths - 1).astype(np.int32)
    used = perm[:cur]
    pk_t = torch.full((num_pages, kvh, 64, d), float("nan"), dtype=TORCH_DT[dtype])
    pv_t = torch.full((num_pages, kvh, 64, d), float("nan"), dtype=TORCH_DT[dtype])
    kv_k, _ = host_values(W.normal(g["pool_k"], (cur, kvh, 64, d)), dtype)
    kv_v, _ = host_values(W.normal(g["pool_v"], (cur, kvh, 64, d)), dtype)
    pk_t[torch.from_numpy(used.astype(np.int64))] = kv_k
    pv_t[torch.from_numpy(used.astype(np.int64))] = kv_v
    for r in range(rows):
        last = table[r, need[r] - 1]
        off = int(lengths[r] - 1) % 64
        pk_t[last, :, off + 1:] = float("nan")
        pv_t[last, :, off + 1:] = float("nan")
    q_t, q64 = host_values(W.normal(g["q"], (rows, heads, d)), dtype)
    # Oracle view: the used pages only, renumbered (the table indirection is
    # unchanged in meaning).
    remap = np.full(num_pages, -1, np.int64)
    remap[used] = np.arange(cur)
    otable = np.where(table >= 0, remap[np.clip(table, 0, num_pages - 1)], -1).astype(np.int32)
    opk = pk_t[torch.from_numpy(used.astype(np.int64))].to(torch.float64).numpy()
    opv = pv_t[torch.from_numpy(used.astype(np.int64))].to(torch.float64).numpy()
    return (dev(q_t), dev(pk_t), dev(pv_t)), (q64, opk, opv), pos, table, otable, g


def test_decode_paged_llama8b_full():
    wl = W.LLAMA8B_PAGED
    e = wl.extra
    print(f"[case] {wl.name} (full size)", flush=True)
    g0 = W.streams(3)
    lengths, _, _ = W.paged_layout(e["rows"], e["len_lo"], e["len_hi"], e["num_pages"], 64,
                                   g0["index"])
    pages = -(-e["len_hi"] // 64)
    dv, hv, pos, table, otable, g = paged_case(3, e["rows"], wl.heads, wl.kv_heads, wl.head_dim,
                                               lengths, pages, e["num_pages"], "bf16")
    out = run_decode_paged(*dv, pos, table, wl.heads, wl.kv_heads, wl.head_dim, "bf16")
    ref = oracle.default().decode_paged(hv[0], hv[1], hv[2], pos, otable)
    assert_close(f64(out), ref, "bf16", "llama8b paged decode (64 rows)")


@pytest.mark.parametrize("heads,kvh,d,dtype", [(32, 8, 128, "bf16"), (8, 8, 64, "bf16"),
                                                (64, 8, 64, "bf16"), (12, 12, 64, "f32"),
                                                (16, 4, 128, "f32"), (64, 2, 128, "bf16")])
def test_decode_paged_shapes(heads, kvh, d, dtype):
    print(f"[case] decode_paged H={heads} KvH={kvh} D={d} {dtype}", flush=True)
    lengths = np.array([1, 2, 63, 64, 65, 128, 700, 1000, 513, 256], dtype=np.int64)
    pages = 17
    dv, hv, pos, table, otable, g = paged_case(40 + d, len(lengths), heads, kvh, d, lengths,
                                               pages, 300, dtype)
    sinks_t, sinks64 = host_values(W.normal(g["sinks"], (heads,)), dtype)
    o = oracle.default()
    for window, sk in ((0, None), (128, sinks_t), (1, None), (0, sinks_t)):
        out = run_decode_paged(*dv, pos, table, heads, kvh, d, dtype, window=window,
                               sinks=None if sk is None else dev(sk))
        ref = o.decode_paged(hv[0], hv[1], hv[2], pos, otable, window=window,
                             sinks=None if sk is None else sinks64)
        assert_close(f64(out), ref, dtype, f"decode_paged W={window} sinks={sk is not None}")


def test_decode_paged_invalid_pages_and_positions():
    """Pages with ids outside the pool contribute no keys; positions past the
    table or negative behave as the contiguous cache does."""
    heads, kvh, d, dtype = 32, 8, 128, "bf16"
    lengths = np.array([300, 300, 64, 200], dtype=np.int64)
    pages = 6
    dv, hv, pos, table, otable, g = paged_case(77, 4, heads, kvh, d, lengths, pages, 40, dtype)
    table = table.copy()
    otable = otable.copy()
    table[0, 1] = -5
    otable[0, 1] = -5
    table[1, 2] = 40            # == num_pages: out of range on the GPU
    otable[1, 2] = 10 ** 6      # out of range for the oracle's renumbered pool too
    pos = pos.copy()
    pos[2] = -1                 # nothing attended -> 0
    pos[3] = 10 ** 6            # past the table: every slot of the table (pages * 64)
    # row 3 then reads slots past its data: make those pages valid zeros-free data
    out = run_decode_paged(*dv, pos, table, heads, kvh, d, dtype)
    o = oracle.default()
    ref = o.decode_paged(hv[0], hv[1], hv[2], pos, otable)
    got = f64(out)
    assert np.all(got[2] == 0.0)
    # row 3 attends NaN-poisoned slots past its length on both sides; compare rows 0-2
    assert_close(got[:3], ref[:3], dtype, "decode_paged invalid pages")


# --- index exactness: mask probes ------------------------------------------------------
@pytest.mark.parametrize("paged", [False, True])
def test_decode_mask_probe(paged):
    """q = 0: uniform weights over the attended set. V is one-hot per probed
    key, so out[d] > 0 iff key d is attended -- exact set membership."""
    heads, kvh, d, dtype = 4, 1, 128, "bf16"
    rows = 6
    pos = np.array([0, 63, 64, 127, 130, 200], dtype=np.int32)
    windows = [0, 5]
    cap = 256
    for window in windows:
        q = torch.zeros((rows, heads, d), dtype=torch.bfloat16, device=DEV)
        k = torch.zeros((rows, kvh, cap, d), dtype=torch.bfloat16)
        v = torch.zeros((rows, kvh, cap, d), dtype=torch.bfloat16)
        # key t carries one-hot dimension (t % d) with value 1 -- probed keys:
        # only those with t in [pos - 64, pos + 63] map to distinct dims.
        for r in range(rows):
            for t in range(cap):
                if t > pos[r]:
                    k[r, :, t] = float("nan")
                    v[r, :, t] = float("nan")
                else:
                    v[r, :, t, t % d] = 1.0
        if paged:
            table = np.arange(rows * 4, dtype=np.int32).reshape(rows, 4)
            pk = k.reshape(rows, kvh, 4, 64, d).permute(0, 2, 1, 3, 4).reshape(rows * 4, kvh, 64, d)
            pv = v.reshape(rows, kvh, 4, 64, d).permute(0, 2, 1, 3, 4).reshape(rows * 4, kvh, 64, d)
            out = run_decode_paged(q, dev(pk.contiguous()), dev(pv.contiguous()), pos, table, heads,
                                   kvh, d, dtype, window=window)
        else:
            out = run_decode_rows(q, dev(k), dev(v), pos, heads, kvh, d, dtype, window=window)
        got = f64(out)
        for r in range(rows):
            lo = 0 if window == 0 else max(0, int(pos[r]) - window + 1)
            keys = np.arange(lo, int(pos[r]) + 1)
            expect = np.zeros(d)
            for t in keys:
                expect[t % d] += 1.0 / len(keys)
            for h in range(heads):
                member = got[r, h] > 0
                assert np.array_equal(member, expect > 0), f"row {r} W={window}: attended set"
                assert np.max(np.abs(got[r, h] - expect)) < 2e-2


def test_decode_deterministic():
    heads, kvh, d, dtype = 32, 8, 128, "bf16"
    lengths = np.array([4000, 17, 900], dtype=np.int64)
    dv, hv, pos, table, otable, g = paged_case(9, 3, heads, kvh, d, lengths, 63, 200, dtype)
    a = run_decode_paged(*dv, pos, table, heads, kvh, d, dtype)
    b = run_decode_paged(*dv, pos, table, heads, kvh, d, dtype)
    assert np.array_equal(bits(a), bits(b))
