"""GPU parity: chunked prefill over a cached prefix (`prefill<S>(x, pos)` with
pos > 0 over the contiguous cache, `prefill_paged` over the page pool)
against the fp64 oracle. Cache slots past each row's last written position are
poisoned with NaN; every query tile shape is exercised: one row, rows that
split a tile, interleaved rows, rows outside the cache, invalid pages.
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import oracle
import workloads as W
from tests.gpu_common import (CODE, DEV, TORCH_DT, assert_close, dev, f64, host_values, i32,
                              workspace)

pytestmark = pytest.mark.gpu


def run_cached(q, rows, pos, kind, ck, cv, heads, kvh, d, dim0, seq, table=None, window=0,
               sinks=None):
    n = q.shape[0]
    out = torch.full((n, heads, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws, nb = workspace(gqa.gqa_prefill_cached_workspace(n, heads, kvh, d))
    tr, tp = (0, 0) if table is None else table.shape
    gqa.gqa_prefill_cached(n, heads, kvh, d, CODE["bf16"], 0.0, window, sinks, q,
                           None if rows is None else i32(rows), i32(pos), kind, ck, cv, dim0, seq,
                           None if table is None else i32(table), tr, tp, out, ws, nb)
    torch.cuda.synchronize()
    return out


def chunk_layout(g, prefixes, chunks):
    """Row-contiguous chunk tokens: row r's chunk occupies positions
    prefixes[r] .. prefixes[r] + chunks[r] - 1."""
    rows = np.concatenate([np.full(c, r, np.int32) for r, c in enumerate(chunks)])
    pos = np.concatenate([np.arange(p, p + c, dtype=np.int32) for p, c in zip(prefixes, chunks)])
    return rows, pos


def contiguous_cache(g, batch, kvh, max_seq, d, last):
    """Cache with slots 0..last[r] of row r written, NaN beyond."""
    ck = W.normal(g["pool_k"], (batch, kvh, max_seq, d))
    cv = W.normal(g["pool_v"], (batch, kvh, max_seq, d))
    for r in range(batch):
        ck[r, :, last[r] + 1:] = np.nan
        cv[r, :, last[r] + 1:] = np.nan
    ck_t, ck64 = host_values(ck, "bf16")
    cv_t, cv64 = host_values(cv, "bf16")
    return dev(ck_t), dev(cv_t), ck64, cv64


def paged_from_contiguous(g, ck64, cv64, extra_pages=5):
    """Scatter a contiguous cache into a shuffled page pool; pages no row
    references are NaN."""
    batch, kvh, max_seq, d = ck64.shape
    pages = (max_seq + 63) // 64
    num_pages = batch * pages + extra_pages
    perm = g["index"].permutation(num_pages).astype(np.int32)
    table = perm[:batch * pages].reshape(batch, pages)
    pk = np.full((num_pages, kvh, 64, d), np.nan)
    pv = np.full((num_pages, kvh, 64, d), np.nan)
    for r in range(batch):
        for p in range(pages):
            n = min(64, max_seq - 64 * p)
            # slots of a referenced page past max_seq are attendable (the
            # table's capacity is whole pages): zeros there, as after a reset
            pk[table[r, p]] = 0.0
            pv[table[r, p]] = 0.0
            pk[table[r, p], :, :n] = ck64[r, :, 64 * p:64 * p + n]
            pv[table[r, p], :, :n] = cv64[r, :, 64 * p:64 * p + n]
    pk_t = torch.from_numpy(pk.astype(np.float32)).to(torch.bfloat16)
    pv_t = torch.from_numpy(pv.astype(np.float32)).to(torch.bfloat16)
    return dev(pk_t), dev(pv_t), pk, pv, table


CASES = [
    # heads, kvh, d, prefixes, chunks
    (32, 8, 128, [0, 700, 1500, 37], [200, 90, 333, 1]),
    (8, 8, 64, [128, 5, 64], [16, 59, 200]),
    (64, 8, 64, [4000, 100], [96, 31]),
    (4, 2, 128, [63, 64, 65, 0], [1, 64, 40, 130]),
]


@pytest.mark.parametrize("heads,kvh,d,prefixes,chunks", CASES)
@pytest.mark.parametrize("window,use_sinks", [(0, False), (0, True), (100, True)])
@pytest.mark.parametrize("kind", ["contiguous", "paged"])
def test_prefill_cached_rows(heads, kvh, d, prefixes, chunks, window, use_sinks, kind):
    print(f"[case] prefill_cached {kind} H={heads} KvH={kvh} D={d} prefixes={prefixes} "
          f"chunks={chunks} W={window} sinks={use_sinks}", flush=True)
    seed = 2000 + heads + d + len(prefixes)
    g = W.streams(seed)
    rows, pos = chunk_layout(g, prefixes, chunks)
    last = [p + c - 1 for p, c in zip(prefixes, chunks)]
    max_seq = max(last) + 1 + 17
    ck, cv, ck64, cv64 = contiguous_cache(g, len(prefixes), kvh, max_seq, d, last)
    q_t, q64 = host_values(W.normal(g["q"], (len(pos), heads, d)), "bf16")
    sk_t, sk64 = host_values(W.normal(g["sinks"], (heads,)), "bf16")
    sinks, sinks64 = (dev(sk_t), sk64) if use_sinks else (None, None)
    o = oracle.default()
    ref = o.prefill_cached(q64, rows, pos, np.nan_to_num(ck64), np.nan_to_num(cv64),
                           window=window, sinks=sinks64)
    if kind == "contiguous":
        out = run_cached(dev(q_t), rows, pos, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, heads, kvh, d,
                         len(prefixes), max_seq, window=window, sinks=sinks)
    else:
        pk, pv, pk64, pv64, table = paged_from_contiguous(g, ck64, cv64)
        ref_p = o.prefill_paged(q64, rows, pos, np.nan_to_num(pk64), np.nan_to_num(pv64), table,
                                window=window, sinks=sinks64)
        assert np.array_equal(ref, ref_p)
        out = run_cached(dev(q_t), rows, pos, gqa.GQA_CACHE_PAGED_TABLE, pk, pv, heads, kvh, d,
                         pk.shape[0], 64, table=table, window=window, sinks=sinks)
    assert_close(f64(out), ref, "bf16", f"prefill_cached {kind} n={len(pos)}")


def test_prefill_cached_interleaved_and_invalid():
    """Tokens of several rows interleaved in n order (query tiles with many
    rows), a row outside the cache, positions past the cache, invalid pages."""
    heads, kvh, d = 32, 8, 128
    g = W.streams(2100)
    batch, max_seq = 5, 600
    n = 150
    rows = g["index"].integers(0, batch, n).astype(np.int32)
    pos = g["index"].integers(0, max_seq, n).astype(np.int32)
    rows[7] = batch + 3      # outside the cache: output 0
    rows[8] = -1
    pos[9] = max_seq + 50    # past the cache: attends every slot of its row
    ck, cv, ck64, cv64 = contiguous_cache(g, batch, kvh, max_seq, d, [max_seq - 1] * batch)
    q_t, q64 = host_values(W.normal(g["q"], (n, heads, d)), "bf16")
    o = oracle.default()
    for window in (0, 50):
        ref = o.prefill_cached(q64, rows, pos, ck64, cv64, window=window)
        out = run_cached(dev(q_t), rows, pos, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, heads, kvh, d,
                         batch, max_seq, window=window)
        assert_close(f64(out), ref, "bf16", f"prefill_cached interleaved W={window}")
        assert np.all(f64(out)[7] == 0) and np.all(f64(out)[8] == 0)
    # paged, with invalid page ids in the table
    pk, pv, pk64, pv64, table = paged_from_contiguous(g, ck64, cv64)
    table[1, 2] = -1
    table[3, 0] = pk.shape[0] + 9
    ref = o.prefill_paged(q64, rows, pos, np.nan_to_num(pk64), np.nan_to_num(pv64), table)
    out = run_cached(dev(q_t), rows, pos, gqa.GQA_CACHE_PAGED_TABLE, pk, pv, heads, kvh, d,
                     pk.shape[0], 64, table=table)
    assert_close(f64(out), ref, "bf16", "prefill_cached paged, invalid pages")


def test_prefill_cached_single_row_tile_with_invalid_rows():
    """A query tile whose valid tokens all read one cache row, plus tokens
    whose row is -1 or past the cache: those get no keys and output 0 (the
    tile must not take the unmasked single-row path), the others match the
    oracle. Contiguous cache and paged pool."""
    heads, kvh, d = 32, 8, 128
    g = W.streams(2150)
    batch, max_seq, n = 2, 600, 40
    rows = np.ones(n, dtype=np.int32)
    pos = np.arange(500, 500 + n, dtype=np.int32)
    rows[5] = -1
    rows[12] = batch + 3
    ck, cv, ck64, cv64 = contiguous_cache(g, batch, kvh, max_seq, d, [max_seq - 1] * batch)
    q_t, q64 = host_values(W.normal(g["q"], (n, heads, d)), "bf16")
    o = oracle.default()
    for window in (0, 300):
        ref = o.prefill_cached(q64, rows, pos, ck64, cv64, window=window)
        assert np.all(ref[5] == 0) and np.all(ref[12] == 0)
        out = f64(run_cached(dev(q_t), rows, pos, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, heads, kvh, d,
                             batch, max_seq, window=window))
        assert np.all(out[5] == 0) and np.all(out[12] == 0), "a token with no row got keys"
        assert_close(out, ref, "bf16", f"prefill_cached one-row tile with invalid rows W={window}")
    pk, pv, pk64, pv64, table = paged_from_contiguous(g, ck64, cv64)
    ref = o.prefill_paged(q64, rows, pos, np.nan_to_num(pk64), np.nan_to_num(pv64), table)
    out = f64(run_cached(dev(q_t), rows, pos, gqa.GQA_CACHE_PAGED_TABLE, pk, pv, heads, kvh, d,
                         pk.shape[0], 64, table=table))
    assert np.all(out[5] == 0) and np.all(out[12] == 0), "a token with no table row got keys"
    assert_close(out, ref, "bf16", "prefill_cached paged one-row tile with invalid rows")


def test_prefill_cached_rows_null_and_empty():
    heads, kvh, d = 8, 8, 64
    g = W.streams(2200)
    max_seq = 300
    ck, cv, ck64, cv64 = contiguous_cache(g, 1, kvh, max_seq, d, [299])
    pos = np.arange(200, 300, dtype=np.int32)
    q_t, q64 = host_values(W.normal(g["q"], (len(pos), heads, d)), "bf16")
    ref = oracle.default().prefill_cached(q64, None, pos, ck64, cv64)
    out = run_cached(dev(q_t), None, pos, gqa.GQA_CACHE_CONTIGUOUS, ck, cv, heads, kvh, d, 1,
                     max_seq)
    assert_close(f64(out), ref, "bf16", "prefill_cached rows = NULL")
    # n = 0 launches nothing
    gqa.gqa_prefill_cached(0, heads, kvh, d, CODE["bf16"], 0.0, 0, None, dev(q_t), None,
                           i32(pos), gqa.GQA_CACHE_CONTIGUOUS, ck, cv, 1, max_seq, None, 0, 0,
                           dev(q_t), None, 0)


def test_prefill_cached_llama8b_paged_sampled():
    """Serving-size chunk: 8 rows of the Llama-3.1-8B paged pool, prefixes of
    1024..6144 tokens, 512-token chunks; sampled queries against the oracle."""
    heads, kvh, d = 32, 8, 128
    g = W.streams(2300)
    rows_n, chunk = 8, 512
    prefixes = g["index"].integers(1024, 6145, rows_n)
    last = prefixes + chunk - 1
    pages = int((last.max() + 64) // 64)
    num_pages = rows_n * pages + 16
    perm = g["index"].permutation(num_pages).astype(np.int32)
    table = perm[:rows_n * pages].reshape(rows_n, pages)
    pk = W.device_normal((num_pages, kvh, 64, d), 2300, "pool_k", torch.bfloat16)
    pv = W.device_normal((num_pages, kvh, 64, d), 2300, "pool_v", torch.bfloat16)
    rows, pos = chunk_layout(g, prefixes, [chunk] * rows_n)
    n = len(pos)
    q = W.device_normal((n, heads, d), 2300, "q", torch.bfloat16)
    out = run_cached(q, rows, pos, gqa.GQA_CACHE_PAGED_TABLE, pk, pv, heads, kvh, d, num_pages, 64,
                     table=table)
    sel = np.sort(W.sample_indices(n, 48, g["index"]))
    # oracle on the sampled tokens only: the pages they reach, copied to the host
    pk64 = pk.float().cpu().double().numpy()
    pv64 = pv.float().cpu().double().numpy()
    q64 = q[torch.from_numpy(sel).to(DEV)].float().cpu().double().numpy()
    ref = oracle.default().prefill_paged(q64, rows[sel], pos[sel], pk64, pv64, table)
    assert_close(f64(out)[sel], ref, "bf16", "prefill_cached llama8b paged, sampled")
