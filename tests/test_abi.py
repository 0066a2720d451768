"""The C-ABI library without a GPU: it loads, exports every entry point that
include/gqa.h declares, and its host-side validation accepts the shapes the
pages bind and rejects what the `where` clause forbids (dry-run mode: the
library validates and returns before any HIP call)."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "decoder_attention_rope_amd", "libgqa.so")
HEADER = os.path.join(ROOT, "include", "gqa.h")


def _build_if_missing():
    """Build the library when nothing is built yet (build.py is loaded by path:
    the package itself refuses to import without the library)."""
    if os.path.exists(LIB):
        return
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_gqa_build", os.path.join(ROOT, "decoder_attention_rope_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build()


@pytest.fixture(scope="module")
def g():
    _build_if_missing()
    import decoder_attention_rope_amd as mod
    prev = mod.gqa_set_dry_run(1)
    yield mod
    mod.gqa_set_dry_run(prev)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(g):
    names = declared_functions()
    assert {"gqa_rope_write_kv", "gqa_prefill_packed", "gqa_decode_paged",
            "gqa_decode_rows"} <= set(names)
    cdll = ctypes.CDLL(g.library_path)
    missing = [n for n in names if not hasattr(cdll, n)]
    assert not missing, f"declared but not exported: {missing}"
    assert g.gqa_abi_version() == 1


def _codes(g):
    return g.GQA_ERR_INVALID_ARG, g.GQA_ERR_UNSUPPORTED, g.GQA_ERR_WORKSPACE


def _expect(g, status, fn, *args):
    if status == g.GQA_OK:
        fn(*args)
        return
    with pytest.raises(g.GQAError) as e:
        fn(*args)
    assert e.value.status == status


def _decode_rows(g, heads, kvh, d, dtype=0, batch=2, max_seq=64, window=0, ws=True, scale=0.0):
    nb = g.gqa_decode_rows_workspace(max(batch, 1), heads, kvh, d, max_seq) if ws else 0
    return (g.gqa_decode_rows, batch, heads, kvh, d, dtype, scale, window, None, 8, 8, 8, max_seq,
            8, 8, 256 if ws else None, nb)


def test_page_shapes_accepted(g):
    pages = json.load(open(os.path.join(ROOT, "tests", "golden", "page_generics.json")))
    llama, gpt2, oss, tiny = (pages["llama-3.1-8b-instruct"], pages["gpt2"], pages["gpt-oss-20b"],
                              pages["01-llama-bind"])
    shapes = [
        (llama["Heads"], llama["KvHeads"], llama["H"] // llama["Heads"], g.GQA_BF16),
        (gpt2["Heads"], gpt2["Heads"], gpt2["H"] // gpt2["Heads"], g.GQA_F32),
        (oss["Heads"], oss["KvHeads"], oss["HeadDim"], g.GQA_BF16),
        (tiny["Heads"], tiny["KvHeads"], tiny["H"] // tiny["Heads"], g.GQA_BF16),
    ]
    for heads, kvh, d, dt in shapes:
        fn, *args = _decode_rows(g, heads, kvh, d, dt)
        fn(*args)
        g.gqa_rope_write_kv(4, heads, kvh, d, dt, 8, 8, 8, 8, 8, 16, g.GQA_CACHE_CONTIGUOUS, 8, 8,
                            2, 16, None, None, None, 0, 0)
        nbp = g.gqa_decode_paged_workspace(3, 4, heads, kvh, d)
        g.gqa_decode_paged(3, 4, heads, kvh, d, dt, 0.0, oss["Window"], 8, 8, 8, 8, 10, 8, 8, 8,
                           256, nbp)
        if dt == g.GQA_BF16:
            nb = g.gqa_prefill_packed_workspace(100, heads, kvh, d)
            g.gqa_prefill_packed(100, heads, kvh, d, dt, 0.0, 0, None, 8, 8, 8, 8, 8, 8, 256, nb)
        g.gqa_rope_table(d, 64, pages["THETA"], dt, 8)
    # the workloads use the cards' shapes
    import workloads as W
    assert (W.LLAMA8B_PAGED.heads, W.LLAMA8B_PAGED.kv_heads, W.LLAMA8B_PAGED.head_dim) == \
        (llama["Heads"], llama["KvHeads"], llama["H"] // llama["Heads"])
    assert W.LLAMA8B_PAGED.extra["page_size"] == llama["PageSize"]
    assert (W.GPT2_DECODE_ROWS.heads, W.GPT2_DECODE_ROWS.head_dim) == \
        (gpt2["Heads"], gpt2["H"] // gpt2["Heads"])
    assert W.GPT2_DECODE_ROWS.extra["max_seq"] == gpt2["MaxSeq"]
    assert (W.GPT_OSS_SINK.heads, W.GPT_OSS_SINK.kv_heads, W.GPT_OSS_SINK.head_dim) == \
        (oss["Heads"], oss["KvHeads"], oss["HeadDim"])
    assert W.GPT_OSS_SINK.extra["windows"][0] == oss["Window"]
    assert (W.TINY_LLAMA.heads, W.TINY_LLAMA.kv_heads, W.TINY_LLAMA.extra["max_seq"]) == \
        (tiny["Heads"], tiny["KvHeads"], tiny["MaxSeq"])


def test_where_clause_violations(g):
    bad_arg, unsup, ws_err = _codes(g)
    cases = [
        (bad_arg, dict(heads=0, kvh=1, d=64)),
        (bad_arg, dict(heads=8, kvh=0, d=64)),
        (bad_arg, dict(heads=8, kvh=3, d=64)),     # Heads % KvHeads != 0
        (bad_arg, dict(heads=8, kvh=8, d=63)),     # odd head dim
        (unsup, dict(heads=8, kvh=8, d=96)),       # valid, not built
        (bad_arg, dict(heads=8, kvh=8, d=64, dtype=7)),
        (bad_arg, dict(heads=8, kvh=8, d=64, window=-1)),
        (bad_arg, dict(heads=8, kvh=8, d=64, batch=-1)),
        (bad_arg, dict(heads=8, kvh=8, d=64, max_seq=0)),
        (ws_err, dict(heads=8, kvh=8, d=64, ws=False)),
        (bad_arg, dict(heads=8, kvh=8, d=64, scale=float("nan"))),
        (g.GQA_OK, dict(heads=8, kvh=8, d=64, batch=0)),  # empty is fine
    ]
    for status, kw in cases:
        fn, *args = _decode_rows(g, **kw)
        _expect(g, status, fn, *args)


def test_entry_point_argument_checks(g):
    bad_arg, unsup, ws_err = _codes(g)
    # null pointers
    _expect(g, bad_arg, g.gqa_decode_paged, 2, 4, 8, 8, 64, 0, 0.0, 0, None, None, 8, 8, 10, 8, 8,
            8, 256, 10 ** 6)
    _expect(g, bad_arg, g.gqa_prefill_packed, 10, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, None, 8, 8,
            256, 10 ** 6)
    # prefill is built for bf16 only
    _expect(g, unsup, g.gqa_prefill_packed, 10, 8, 8, 64, 1, 0.0, 0, None, 8, 8, 8, 8, 8, 8, 256,
            10 ** 6)
    # workspace: too small, misaligned
    _expect(g, ws_err, g.gqa_prefill_packed, 10, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 8, 8, 8, 256,
            16)
    _expect(g, ws_err, g.gqa_prefill_packed, 10, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 8, 8, 8, 257,
            10 ** 6)
    _expect(g, g.GQA_OK, g.gqa_prefill_packed, 0, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 8, 8, 8,
            None, 0)
    # paged writes need the page size; table writes need a table
    _expect(g, bad_arg, g.gqa_rope_write_kv, 4, 8, 8, 64, 0, 8, 8, 8, 8, 8, 16,
            g.GQA_CACHE_PAGED_SLOTS, 8, 8, 10, 32, None, 8, None, 0, 0)
    _expect(g, bad_arg, g.gqa_rope_write_kv, 4, 8, 8, 64, 0, 8, 8, 8, 8, 8, 16,
            g.GQA_CACHE_PAGED_TABLE, 8, 8, 10, 64, None, None, None, 0, 0)
    _expect(g, g.GQA_OK, g.gqa_rope_write_kv, 4, 8, 8, 64, 0, 8, 8, 8, 8, 8, 16,
            g.GQA_CACHE_PAGED_TABLE, 8, 8, 10, 64, None, None, 8, 3, 2)
    _expect(g, bad_arg, g.gqa_rope_write_kv, 4, 8, 8, 64, 0, 8, 8, 8, 8, 8, 16, 9, 8, 8, 10, 64,
            None, None, None, 0, 0)
    _expect(g, bad_arg, g.gqa_rope_write_kv, -1, 8, 8, 64, 0, 8, 8, 8, 8, 8, 16,
            g.GQA_CACHE_NONE, None, None, 0, 0, None, None, None, 0, 0)
    # rope table
    _expect(g, bad_arg, g.gqa_rope_table, 64, 0, 1e4, 0, 8)
    _expect(g, bad_arg, g.gqa_rope_table, 64, 10, -1.0, 0, 8)
    _expect(g, unsup, g.gqa_rope_table, 32, 10, 1e4, 0, 8)
    # paged decode: pages * 64 must fit int32
    _expect(g, bad_arg, g.gqa_decode_paged, 2, 2 ** 26, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 10, 8,
            8, 8, 256, 10 ** 12)


def test_prefill_plan_argument_checks(g):
    bad_arg, unsup, ws_err = _codes(g)
    # the plan needs positions, segments and a workspace; q, k, v, out are not read
    _expect(g, g.GQA_OK, g.gqa_prefill_packed_plan, 10, 8, 8, 64, 0, 8, 8, 256, 10 ** 6)
    _expect(g, bad_arg, g.gqa_prefill_packed_plan, 10, 8, 8, 64, 0, None, 8, 256, 10 ** 6)
    _expect(g, bad_arg, g.gqa_prefill_packed_plan, 10, 8, 8, 64, -1, 8, 8, 256, 10 ** 6)
    _expect(g, ws_err, g.gqa_prefill_packed_plan, 10, 8, 8, 64, 0, 8, 8, 256, 16)
    _expect(g, ws_err, g.gqa_prefill_packed_plan, 10, 8, 8, 64, 0, 8, 8, 257, 10 ** 6)
    _expect(g, unsup, g.gqa_prefill_packed_plan, 10, 8, 8, 96, 0, 8, 8, 256, 10 ** 6)
    # the planned call checks what gqa_prefill_packed checks
    _expect(g, g.GQA_OK, g.gqa_prefill_packed_planned, 10, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 8, 8,
            8, 256, 10 ** 6)
    _expect(g, bad_arg, g.gqa_prefill_packed_planned, 10, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 8, 8,
            None, 256, 10 ** 6)
    _expect(g, unsup, g.gqa_prefill_packed_planned, 10, 8, 8, 64, 1, 0.0, 0, None, 8, 8, 8, 8, 8,
            8, 256, 10 ** 6)
    _expect(g, ws_err, g.gqa_prefill_packed_planned, 10, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 8, 8,
            8, None, 0)
    _expect(g, g.GQA_OK, g.gqa_prefill_packed_planned, 0, 8, 8, 64, 0, 0.0, 0, None, 8, 8, 8, 8, 8,
            8, None, 0)


def test_prefill_cached_argument_checks(g):
    bad_arg, unsup, ws_err = _codes(g)
    cont, paged = g.GQA_CACHE_CONTIGUOUS, g.GQA_CACHE_PAGED_TABLE
    nb = g.gqa_prefill_cached_workspace(10, 8, 8, 64)
    assert nb > 0 and g.gqa_prefill_cached_workspace(0, 8, 8, 64) == 0

    def call(status, n=10, dtype=0, q=8, pos=8, kind=cont, dim0=4, seq=32, table=None, trows=0,
             tpages=0, ws=256, wsb=None, window=0):
        _expect(g, status, g.gqa_prefill_cached, n, 8, 8, 64, dtype, 0.0, window, None, q, 8, pos,
                kind, 8, 8, dim0, seq, table, trows, tpages, 8, ws, nb if wsb is None else wsb)

    call(g.GQA_OK)                                           # contiguous
    call(g.GQA_OK, kind=paged, seq=64, table=8, trows=2, tpages=3)
    call(g.GQA_OK, n=0, ws=None, wsb=0)                      # empty is fine
    call(bad_arg, q=None)
    call(bad_arg, pos=None)
    call(bad_arg, window=-1)
    call(bad_arg, kind=g.GQA_CACHE_PAGED_SLOTS)             # slots address writes only
    call(bad_arg, seq=0)
    call(bad_arg, dim0=0)
    call(bad_arg, kind=paged, seq=32, table=8, trows=2, tpages=3)   # pages hold 64 slots
    call(bad_arg, kind=paged, seq=64, table=None, trows=2, tpages=3)
    call(bad_arg, kind=paged, seq=64, table=8, trows=2, tpages=2 ** 26)
    call(unsup, dtype=1)                                     # bf16 only
    call(ws_err, wsb=16)
    call(ws_err, ws=257)


def test_step_entries_argument_checks(g):
    bad_arg, unsup, ws_err = _codes(g)
    nb = g.gqa_step_packed_workspace(4, 100, 8, 8, 64, 512)
    assert nb >= g.gqa_prefill_packed_workspace(100, 8, 8, 64) + \
        g.gqa_decode_rows_workspace(4, 8, 8, 64, 512)
    sp = lambda st, batch=4, p=100, dtype=0, q=8, seg=8, cache=8, wsb=nb: _expect(  # noqa: E731
        g, st, g.gqa_step_packed, batch, p, 8, 8, 64, dtype, 0.0, 0, None, q, 8, 8, 8, seg, cache,
        cache, 512, 8, 8, 256, wsb)
    sp(g.GQA_OK)
    sp(g.GQA_OK, batch=0)
    sp(g.GQA_OK, p=0)
    sp(bad_arg, q=None)
    sp(bad_arg, seg=None)          # the packed part needs segments
    sp(bad_arg, cache=None)        # the decode part needs the cache
    sp(unsup, dtype=1)
    sp(ws_err, wsb=nb - 1)
    nbp = g.gqa_step_paged_workspace(300, 16, 128, 32, 8, 128)
    assert nbp >= g.gqa_prefill_cached_workspace(300, 32, 8, 128)
    spg = lambda st, p=300, rows=16, pages=128, table=8, wsb=nbp: _expect(  # noqa: E731
        g, st, g.gqa_step_paged, p, rows, pages, 32, 8, 128, 0, 0.0, 0, None, 8, 8, 8, 8, 8, 2000,
        table, 8, 8, 256, wsb)
    spg(g.GQA_OK)
    spg(g.GQA_OK, p=0)
    spg(bad_arg, table=None)
    spg(bad_arg, pages=0)
    spg(ws_err, wsb=16)


def test_workspace_sizes(g):
    assert g.gqa_decode_rows_workspace(0, 8, 8, 64, 10) == 0
    a = g.gqa_decode_paged_workspace(64, 128, 32, 8, 128)
    b = g.gqa_decode_paged_workspace(64, 256, 32, 8, 128)
    assert 0 < a < b
    assert g.gqa_prefill_packed_workspace(16384, 32, 8, 128) > g.gqa_prefill_packed_workspace(
        1024, 32, 8, 128) > 0


def test_training_entries_argument_checks(g):
    bad_arg, unsup, ws_err = _codes(g)
    nb_f = g.gqa_prefill_packed_workspace(100, 8, 2, 64)
    nb_b = g.gqa_prefill_packed_backward_workspace(100, 8, 2, 64)
    assert nb_b > nb_f > 0 and g.gqa_prefill_packed_backward_workspace(0, 8, 2, 64) == 0

    def fwd(status, p=100, dtype=0, lse=8, q=8, ws=256, wsb=None, window=0):
        _expect(g, status, g.gqa_prefill_packed_lse, p, 8, 2, 64, dtype, 0.0, window, q, 8, 8, 8,
                8, 8, lse, ws, nb_f if wsb is None else wsb)

    fwd(g.GQA_OK)
    fwd(g.GQA_OK, p=0, ws=None, wsb=0)
    fwd(bad_arg, lse=None)
    fwd(bad_arg, q=None)
    fwd(bad_arg, window=-1)
    fwd(unsup, dtype=1)
    fwd(ws_err, wsb=16)

    def bwd(status, p=100, dtype=0, lse=8, dout=8, dk=8, heads=8, ws=256, wsb=None, scale=0.0):
        _expect(g, status, g.gqa_prefill_packed_backward, p, heads, 2, 64, dtype, scale, 0, 8, 8, 8,
                8, dout, lse, 8, 8, 8, dk, 8, ws, nb_b if wsb is None else wsb)

    bwd(g.GQA_OK)
    bwd(g.GQA_OK, p=0, ws=None, wsb=0)
    bwd(bad_arg, lse=None)
    bwd(bad_arg, dout=None)
    bwd(bad_arg, dk=None)
    bwd(bad_arg, heads=7)          # not a multiple of kv_heads = 2
    bwd(bad_arg, scale=float("nan"))
    bwd(unsup, dtype=1)
    bwd(ws_err, wsb=16)
    bwd(ws_err, ws=257)


def test_workspace_bytes_matches_per_op_queries(g):
    for heads, kvh, d in ((32, 8, 128), (64, 8, 64), (12, 12, 64)):
        for n, rows, max_len in ((1, 1, 1), (333, 5, 64), (16384, 64, 128), (4096, 32, 1024)):
            assert g.gqa_workspace_bytes(g.GQA_OP_PREFILL_PACKED, heads, kvh, d, n, rows, max_len) == \
                g.gqa_prefill_packed_workspace(n, heads, kvh, d)
            assert g.gqa_workspace_bytes(g.GQA_OP_PREFILL_CACHED, heads, kvh, d, n, rows, max_len) == \
                g.gqa_prefill_cached_workspace(n, heads, kvh, d)
            assert g.gqa_workspace_bytes(g.GQA_OP_PREFILL_BACKWARD, heads, kvh, d, n, rows, max_len) == \
                g.gqa_prefill_packed_backward_workspace(n, heads, kvh, d)
            assert g.gqa_workspace_bytes(g.GQA_OP_DECODE_ROWS, heads, kvh, d, n, rows, max_len) == \
                g.gqa_decode_rows_workspace(rows, heads, kvh, d, max_len)
            assert g.gqa_workspace_bytes(g.GQA_OP_DECODE_PAGED, heads, kvh, d, n, rows, max_len) == \
                g.gqa_decode_paged_workspace(rows, max_len, heads, kvh, d)
            assert g.gqa_workspace_bytes(g.GQA_OP_STEP_PACKED, heads, kvh, d, n, rows, max_len) == \
                g.gqa_step_packed_workspace(rows, n, heads, kvh, d, max_len)
            assert g.gqa_workspace_bytes(g.GQA_OP_STEP_PAGED, heads, kvh, d, n, rows, max_len) == \
                g.gqa_step_paged_workspace(n, rows, max_len, heads, kvh, d)
    assert g.gqa_workspace_bytes(99, 32, 8, 128, 100, 1, 1) == 0


def test_status_names(g):
    for st in range(7):
        assert g.gqa_status_str(st) == g.gqa_status_string(st)
    assert "index" in g.gqa_status_str(g.GQA_ERR_INDEX)
    assert g.gqa_status_str(99) == "unknown status"


def test_dry_run_and_checked_mode_are_per_thread(g):
    """One thread's switches never reach another thread's calls."""
    import threading
    seen = {}

    def other():
        seen["dry"] = g.gqa_set_dry_run(0)      # this thread's own setting: off
        seen["checked"] = g.gqa_set_checked(1)  # on here only
        seen["checked_back"] = g.gqa_set_checked(0)

    prev_checked = g.gqa_set_checked(0)
    assert g.gqa_set_dry_run(1) == 1            # the fixture turned it on for this thread
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == {"dry": 0, "checked": 0, "checked_back": 1}
    assert g.gqa_set_checked(prev_checked) == 0  # unchanged by the other thread


def test_checked_mode_from_environment():
    """GQA_CHECK in the environment turns checked mode on for every thread."""
    import subprocess
    import sys
    code = ("import decoder_attention_rope_amd as g, threading; r = [g.gqa_set_checked(0)]; "
            "t = threading.Thread(target=lambda: r.append(g.gqa_set_checked(0))); t.start(); t.join(); "
            "print(r)")
    for val, want in (("1", "[1, 1]"), ("0", "[0, 0]")):
        env = dict(os.environ, GQA_CHECK=val)
        out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                             text=True, timeout=120)
        assert out.returncode == 0, out.stderr
        assert out.stdout.strip() == want, out.stdout


def test_diag_stream_read_rejects_bad_buffers(g):
    """Null pointers and sizes or addresses that are not 16-byte multiples are
    rejected before anything is enqueued."""
    cdll = ctypes.CDLL(g.library_path)
    f = cdll.gqa_diag_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 16, 64, None) == g.GQA_ERR_INVALID_ARG
    assert f(64, 16, None, None) == g.GQA_ERR_INVALID_ARG
    assert f(64, 24, 64, None) == g.GQA_ERR_INVALID_ARG
    assert f(72, 16, 64, None) == g.GQA_ERR_INVALID_ARG
    assert f(64, 0, 64, None) == g.GQA_OK
