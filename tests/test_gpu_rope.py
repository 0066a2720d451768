"""GPU parity: rotary tables, rope on q/k and the KV write, against the oracle.

Tables and rotations are compared bit for bit (both sides round the exact
rotation once to T); cache writes are bit-exact, including every slot the
write must leave untouched (poisoned before the call).
"""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
import oracle
import workloads as W
from tests.gpu_common import (CODE, DEV, bits, dev, f64, host_values, i32, poison_like)

pytestmark = pytest.mark.gpu


def gpu_table(d, max_pos, theta, dtype):
    tab = torch.empty((2, max_pos, d // 2), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device=DEV)
    gqa.gqa_rope_table(d, max_pos, theta, CODE[dtype], tab)
    torch.cuda.synchronize()
    return tab


@pytest.mark.parametrize("d,max_pos,theta,dtype", [
    (64, 512, 10000.0, "bf16"), (128, 8192, 500000.0, "bf16"), (64, 4352, 500000.0, "bf16"),
    (128, 1024, 500000.0, "f32"), (64, 300, 10000.0, "f32")])
def test_rope_table(d, max_pos, theta, dtype):
    print(f"[case] rope_table D={d} S={max_pos} theta={theta} {dtype}", flush=True)
    tab = gpu_table(d, max_pos, theta, dtype)
    c, s = oracle.default().rope_tables(max_pos, d, theta, dtype)
    got_c, got_s = f64(tab[0]), f64(tab[1])
    ref_c, ref_s = c[:, :d // 2], s[:, :d // 2]
    mism = int(np.sum(got_c != ref_c) + np.sum(got_s != ref_s))
    print(f"[parity] rope_table D={d} S={max_pos}: {mism} of {2 * got_c.size} entries differ", flush=True)
    # Both sides round the f32 steps of the page's pipeline the same way and
    # cast the f32 cos / sin to T: every entry must be identical.
    assert mism == 0, f"{mism} table entries differ from the oracle"
    assert np.all(got_c[0] == 1.0) and np.all(got_s[0] == 0.0)


def _tables(d, max_pos, theta, dtype):
    """GPU table and the oracle's full [S, D] tables with identical values."""
    tab = gpu_table(d, max_pos, theta, dtype)
    c, s = oracle.default().rope_tables(max_pos, d, theta, dtype)
    assert np.array_equal(f64(tab[0]), c[:, :d // 2]) and np.array_equal(f64(tab[1]), s[:, :d // 2])
    return tab, c, s


@pytest.mark.parametrize("heads,kvh,d,dtype,n", [(8, 8, 64, "bf16", 200), (32, 8, 128, "bf16", 333),
                                                  (64, 8, 64, "bf16", 97), (12, 4, 64, "f32", 50)])
def test_rope_contiguous_write(heads, kvh, d, dtype, n):
    print(f"[case] rope_write_kv contiguous H={heads} KvH={kvh} D={d} {dtype} n={n}", flush=True)
    g = W.streams(100 + n)
    theta, max_pos = 500000.0, 512
    tab, c, s = _tables(d, max_pos, theta, dtype)
    q_t, q64 = host_values(W.normal(g["q"], (n, heads, d)), dtype)
    k_t, k64 = host_values(W.normal(g["k"], (n, kvh, d)), dtype)
    v_t, v64 = host_values(W.normal(g["v"], (n, kvh, d)), dtype)
    batch, max_seq = 4, 300
    rows = g["index"].integers(-1, batch + 1, n).astype(np.int32)       # some out of range
    pos = g["index"].integers(-2, max_seq + 3, n).astype(np.int32)       # some out of range
    # distinct targets among in-range writes (duplicates race by contract)
    seen = set()
    for t in range(n):
        key = (int(rows[t]), int(pos[t]))
        if key in seen:
            rows[t] = -1
        seen.add(key)
    q, k, v = dev(q_t), dev(k_t), dev(v_t)
    ck = poison_like((batch, kvh, max_seq, d), dtype)
    cv = poison_like((batch, kvh, max_seq, d), dtype)
    ck0, cv0 = bits(ck), bits(cv)
    gqa.gqa_rope_write_kv(n, heads, kvh, d, CODE[dtype], q, k, v, i32(pos), tab, max_pos,
                          gqa.GQA_CACHE_CONTIGUOUS, ck, cv, batch, max_seq, i32(rows), None, None,
                          0, 0)
    torch.cuda.synchronize()
    o = oracle.default()
    q_ref = o.rope(q64, pos, c, s, dtype)
    k_ref = o.rope(k64, pos, c, s, dtype)
    assert np.array_equal(f64(q), q_ref), "rotated q differs from the oracle"
    assert np.array_equal(f64(k), k_ref), "rotated k differs from the oracle"
    zk = np.zeros((batch, kvh, max_seq, d))
    ck_ref, cv_ref, wr = o.write_contiguous(k_ref, v64, pos, zk, zk, rows=rows)
    gk, gv = bits(ck), bits(cv)
    assert np.array_equal(gk[~wr], ck0[~wr]) and np.array_equal(gv[~wr], cv0[~wr]), \
        "a slot outside the write targets changed"
    assert np.array_equal(f64(ck)[wr], ck_ref[wr]), "cache_k values"
    assert np.array_equal(gv[wr], bits(torch.from_numpy(cv_ref).to(q_t.dtype))[wr]), "cache_v bits"


@pytest.mark.parametrize("mode", ["table", "slots"])
def test_rope_paged_write(mode):
    print(f"[case] rope_write_kv paged by {mode}", flush=True)
    heads, kvh, d, dtype = 32, 8, 128, "bf16"
    g = W.streams(7 if mode == "table" else 8)
    rows_n, pages, num_pages = 6, 5, 40
    tab, c, s = _tables(d, pages * 64, 500000.0, dtype)
    table = np.full((rows_n, pages), -1, np.int32)
    perm = g["index"].permutation(num_pages).astype(np.int32)
    table.flat[:rows_n * pages - 3] = perm[:rows_n * pages - 3]
    table[2, 1] = num_pages + 7  # an invalid page id
    n = 150
    if mode == "table":
        rows = g["index"].integers(-1, rows_n + 1, n).astype(np.int32)
        pos = g["index"].integers(-1, pages * 64 + 2, n).astype(np.int32)
        keyset = set()
        for t in range(n):
            kk = (int(rows[t]), int(pos[t]))
            if kk in keyset:
                rows[t] = -1
            keyset.add(kk)
        slots = None
    else:
        slots = g["index"].permutation(num_pages * 64 + 10)[:n].astype(np.int32) - 5
        pos = g["index"].integers(0, 300, n).astype(np.int32)
        rows = None
    q_t, q64 = host_values(W.normal(g["q"], (n, heads, d)), dtype)
    k_t, k64 = host_values(W.normal(g["k"], (n, kvh, d)), dtype)
    v_t, v64 = host_values(W.normal(g["v"], (n, kvh, d)), dtype)
    q, k, v = dev(q_t), dev(k_t), dev(v_t)
    pk = poison_like((num_pages, kvh, 64, d), dtype)
    pv = poison_like((num_pages, kvh, 64, d), dtype)
    pk0, pv0 = bits(pk), bits(pv)
    kind = gqa.GQA_CACHE_PAGED_TABLE if mode == "table" else gqa.GQA_CACHE_PAGED_SLOTS
    gqa.gqa_rope_write_kv(n, heads, kvh, d, CODE[dtype], q, k, v, i32(pos), tab, pages * 64, kind,
                          pk, pv, num_pages, 64, None if rows is None else i32(rows),
                          None if slots is None else i32(slots), i32(table), rows_n, pages)
    torch.cuda.synchronize()
    o = oracle.default()
    k_ref = o.rope(k64, pos, c, s, dtype)
    assert np.array_equal(f64(q), o.rope(q64, pos, c, s, dtype))
    zk = np.zeros((num_pages, kvh, 64, d))
    pk_ref, pv_ref, wr = o.write_paged(k_ref, v64, zk, zk, positions=pos, rows=rows, slots=slots,
                                       table=table if mode == "table" else None)
    assert wr.any() and not wr.all()
    gk, gv = bits(pk), bits(pv)
    assert np.array_equal(gk[~wr], pk0[~wr]) and np.array_equal(gv[~wr], pv0[~wr])
    assert np.array_equal(f64(pk)[wr], pk_ref[wr]) and np.array_equal(f64(pv)[wr], pv_ref[wr])


def test_write_without_rope_f32():
    """GPT-2: no rotary table; k and v are copied bit for bit, q untouched."""
    print("[case] rope_write_kv without rotation, f32", flush=True)
    heads, d, batch, max_seq = 12, 64, 32, 1024
    g = W.streams(21)
    n = batch
    k_t, k64 = host_values(W.normal(g["k"], (n, heads, d)), "f32")
    v_t, v64 = host_values(W.normal(g["v"], (n, heads, d)), "f32")
    pos = W.uniform_positions(n, 0, max_seq - 1, g["index"])
    k, v = dev(k_t), dev(v_t)
    ck = poison_like((batch, heads, max_seq, d), "f32")
    cv = poison_like((batch, heads, max_seq, d), "f32")
    ck0 = bits(ck)
    gqa.gqa_rope_write_kv(n, heads, heads, d, gqa.GQA_F32, None, k, v, i32(pos), None, 0,
                          gqa.GQA_CACHE_CONTIGUOUS, ck, cv, batch, max_seq,
                          i32(np.arange(n, dtype=np.int32)), None, None, 0, 0)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), bits(k_t)), "k must be untouched without a table"
    z = np.zeros((batch, heads, max_seq, d))
    ck_ref, cv_ref, wr = oracle.default().write_contiguous(k64, v64, pos, z, z,
                                                           rows=np.arange(n, dtype=np.int32))
    assert np.array_equal(f64(ck)[wr], ck_ref[wr]) and np.array_equal(f64(cv)[wr], cv_ref[wr])
    assert np.array_equal(bits(ck)[~wr], ck0[~wr])


def test_rope_rotate_only_and_empty():
    """CACHE_NONE rotates in place (packed training forward); n = 0 is a no-op."""
    heads, kvh, d = 8, 2, 64
    g = W.streams(33)
    tab, c, s = _tables(d, 128, 10000.0, "bf16")
    n = 77
    q_t, q64 = host_values(W.normal(g["q"], (n, heads, d)), "bf16")
    k_t, k64 = host_values(W.normal(g["k"], (n, kvh, d)), "bf16")
    pos = g["index"].integers(0, 128, n).astype(np.int32)
    q, k = dev(q_t), dev(k_t)
    gqa.gqa_rope_write_kv(n, heads, kvh, d, gqa.GQA_BF16, q, k, None, i32(pos), tab, 128,
                          gqa.GQA_CACHE_NONE, None, None, 0, 0, None, None, None, 0, 0)
    gqa.gqa_rope_write_kv(0, heads, kvh, d, gqa.GQA_BF16, q, k, None, i32(pos), tab, 128,
                          gqa.GQA_CACHE_NONE, None, None, 0, 0, None, None, None, 0, 0)
    torch.cuda.synchronize()
    o = oracle.default()
    assert np.array_equal(f64(q), o.rope(q64, pos, c, s, "bf16"))
    assert np.array_equal(f64(k), o.rope(k64, pos, c, s, "bf16"))
