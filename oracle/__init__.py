"""fp64 CPU oracle for grouped-query attention with rotary positions.

TEST INFRASTRUCTURE. Only the test suite, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` import this package. The product path (the HIP
library and its Python binding) never imports, links or runs it, and the two
share no code.

This module is argument marshalling over `gqa_oracle.c` (numpy arrays in,
numpy float64 arrays out). Every T-valued input is converted to float64
exactly; index tensors to int32. Citations of the pages and the readings
taken where they leave a step open live beside each C function.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIBS = {}

DT_NONE, DT_BF16, DT_F32 = -1, 0, 1
_DT_NAMES = {"none": DT_NONE, None: DT_NONE, "bf16": DT_BF16, "f32": DT_F32,
             DT_NONE: DT_NONE, DT_BF16: DT_BF16, DT_F32: DT_F32}

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)
_B = ctypes.POINTER(ctypes.c_int8)


def _dt(x):
    return _DT_NAMES[x]


def load(path=None):
    """Load (building if needed) the oracle library at `path` (default: the
    in-tree build, or ORACLE_LIBRARY from the environment)."""
    path = path or os.environ.get("ORACLE_LIBRARY") or _build.DEFAULT_LIB
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        _build.build(path)
    lib = ctypes.CDLL(path)
    c_int, c_dbl = ctypes.c_int, ctypes.c_double
    lib.orc_round.restype = c_dbl
    lib.orc_round.argtypes = [c_dbl, c_int]
    lib.orc_default_scale.restype = c_dbl
    lib.orc_default_scale.argtypes = [c_int]
    lib.orc_inv_freq.argtypes = [c_int, c_dbl, _D]
    lib.orc_rope_tables.argtypes = [c_int, c_int, c_dbl, c_int, _D, _D]
    lib.orc_rope.argtypes = [c_int, c_int, c_int, _D, _I, _D, _D, c_int, c_int, _D]
    lib.orc_write_contiguous.argtypes = [c_int, c_int, c_int, _D, _D, _I, _I, c_int, c_int,
                                         _D, _D, _B]
    lib.orc_write_paged.argtypes = [c_int, c_int, c_int, _D, _D, _I, _I, _I, _I, c_int, c_int,
                                    c_int, c_int, _D, _D, _B]
    lib.orc_forward.argtypes = [c_int, c_int, c_int, c_int, c_int, _D, _D, _D, c_dbl, c_int,
                                _D, _D]
    lib.orc_packed.argtypes = [c_int, c_int, c_int, c_int, _D, _D, _D, _I, _I, c_dbl, c_int,
                               _D, c_int, _I, _D]
    lib.orc_decode_rows.argtypes = [c_int, c_int, c_int, c_int, _D, _D, _D, c_int, _I, c_dbl,
                                    c_int, _D, _D]
    lib.orc_decode_paged.argtypes = [c_int, c_int, c_int, c_int, _D, _D, _D, c_int, c_int, _I,
                                     _I, c_int, c_dbl, c_int, _D, _D]
    lib.orc_prefill_cached.argtypes = [c_int, c_int, c_int, c_int, _D, _I, _I, c_int, _D, _D, c_int,
                                       c_dbl, c_int, _D, _D]
    lib.orc_prefill_paged.argtypes = [c_int, c_int, c_int, c_int, _D, _I, _I, _D, _D, c_int, c_int,
                                      _I, c_int, c_int, c_dbl, c_int, _D, _D]
    lib.orc_linear.argtypes = [c_int, c_int, c_int, _D, _D, _D, c_int, _D]
    lib.orc_packed_lse.argtypes = [c_int, c_int, c_int, c_int, _D, _D, _I, _I, c_dbl, c_int, _D]
    lib.orc_packed_backward.argtypes = [c_int, c_int, c_int, c_int, _D, _D, _D, _D, _I, _I, c_dbl,
                                        c_int, _D, _D, _D]
    lib.orc_num_threads.restype = c_int
    lib.orc_set_num_threads.restype = None
    lib.orc_set_num_threads.argtypes = [c_int]
    lib.orc_mutation.restype = c_int
    _LIBS[path] = lib
    return lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _pd(a):
    return None if a is None else a.ctypes.data_as(_D)


def _pi(a):
    return None if a is None else a.ctypes.data_as(_I)


class Oracle:
    """The oracle's entry points over numpy arrays. `lib_path` selects a
    library build (the default build, or a planted-mistake variant)."""

    def __init__(self, lib_path=None):
        self.lib = load(lib_path)

    # -- numerics helpers -------------------------------------------------
    def round(self, x, dtype):
        x = np.asarray(x, dtype=np.float64)
        f = self.lib.orc_round
        d = _dt(dtype)
        return np.vectorize(lambda v: f(float(v), d), otypes=[np.float64])(x)

    def default_scale(self, head_dim):
        return self.lib.orc_default_scale(int(head_dim))

    def num_threads(self):
        return self.lib.orc_num_threads()

    def set_num_threads(self, n):
        """Threads of the following calls (timing only; results do not depend on it)."""
        self.lib.orc_set_num_threads(int(n))

    def mutation(self):
        return self.lib.orc_mutation()

    # -- rotary tables and rotation ----------------------------------------
    def inv_freq(self, head_dim, theta):
        out = np.zeros(head_dim // 2, dtype=np.float64)
        self.lib.orc_inv_freq(int(head_dim), float(theta), _pd(out))
        return out

    def rope_tables(self, seq, head_dim, theta, dtype="bf16"):
        """Full [S, D] (cos, sin) tables as `tables<S, D, T>(theta)` defines."""
        c = np.zeros((seq, head_dim), dtype=np.float64)
        s = np.zeros((seq, head_dim), dtype=np.float64)
        self.lib.orc_rope_tables(int(seq), int(head_dim), float(theta), _dt(dtype), _pd(c), _pd(s))
        return c, s

    def rope(self, x, positions, cos_full, sin_full, dtype="bf16"):
        """Rotate x [n, nheads, D] at positions [n]; rounded to dtype."""
        x = _f64(x)
        n, nh, d = x.shape
        pos = _i32(positions)
        c, s = _f64(cos_full), _f64(sin_full)
        y = np.zeros_like(x)
        self.lib.orc_rope(n, nh, d, _pd(x), _pi(pos), _pd(c), _pd(s), c.shape[0], _dt(dtype), _pd(y))
        return y

    # -- cache writes --------------------------------------------------------
    def write_contiguous(self, k, v, positions, cache_k, cache_v, rows=None):
        """Returns (cache_k', cache_v', written mask); inputs are not modified."""
        k, v = _f64(k), _f64(v)
        ck, cv = _f64(cache_k).copy(), _f64(cache_v).copy()
        n, kvh, d = k.shape
        batch, _, max_seq, _ = ck.shape
        written = np.zeros(ck.shape, dtype=np.int8)
        self.lib.orc_write_contiguous(n, kvh, d, _pd(k), _pd(v), _pi(_i32(rows)), _pi(_i32(positions)),
                                      batch, max_seq, _pd(ck), _pd(cv),
                                      written.ctypes.data_as(_B))
        return ck, cv, written.astype(bool)

    def write_paged(self, k, v, pool_k, pool_v, positions=None, rows=None, slots=None,
                    table=None):
        """Pool layout [num_pages, KvHeads, page_size, D] for K and V."""
        k, v = _f64(k), _f64(v)
        pk, pv = _f64(pool_k).copy(), _f64(pool_v).copy()
        n, kvh, d = k.shape
        num_pages, _, page_size, _ = pk.shape
        tb = _i32(table)
        trows, tpages = (tb.shape if tb is not None else (0, 0))
        pos = _i32(positions) if positions is not None else np.zeros(n, dtype=np.int32)
        written = np.zeros(pk.shape, dtype=np.int8)
        self.lib.orc_write_paged(n, kvh, d, _pd(k), _pd(v), _pi(_i32(rows)), _pi(pos),
                                 _pi(_i32(slots)), _pi(tb), int(trows), int(tpages), num_pages,
                                 page_size, _pd(pk), _pd(pv), written.ctypes.data_as(_B))
        return pk, pv, written.astype(bool)

    # -- attention ------------------------------------------------------------
    def forward(self, q, k, v, scale=None, window=0, sinks=None):
        """q [B, S, Heads, D], k/v [B, S, KvHeads, D] -> [B, S, Heads, D]."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        b, s, h, d = q.shape
        kvh = k.shape[2]
        scale = self.default_scale(d) if scale is None else float(scale)
        out = np.zeros_like(q)
        self.lib.orc_forward(b, s, h, kvh, d, _pd(q), _pd(k), _pd(v), scale, int(window),
                             _pd(_f64(sinks)), _pd(out))
        return out

    def packed(self, q, k, v, positions, segments, scale=None, window=0, sinks=None, sel=None):
        """q [P, Heads, D], k/v [P, KvHeads, D] -> [P or len(sel), Heads, D]."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        p, h, d = q.shape
        kvh = k.shape[1]
        scale = self.default_scale(d) if scale is None else float(scale)
        sel = _i32(sel)
        nq = p if sel is None else sel.shape[0]
        out = np.zeros((nq, h, d), dtype=np.float64)
        self.lib.orc_packed(p, h, kvh, d, _pd(q), _pd(k), _pd(v), _pi(_i32(positions)),
                            _pi(_i32(segments)), scale, int(window), _pd(_f64(sinks)),
                            int(nq), _pi(sel), _pd(out))
        return out

    def packed_lse(self, q, k, positions, segments, scale=None, window=0):
        """Natural-log softmax denominators of packed(): [P, Heads] (-inf: no key)."""
        q, k = _f64(q), _f64(k)
        p, h, d = q.shape
        kvh = k.shape[1]
        scale = self.default_scale(d) if scale is None else float(scale)
        lse = np.zeros((p, h), dtype=np.float64)
        self.lib.orc_packed_lse(p, h, kvh, d, _pd(q), _pd(k), _pi(_i32(positions)),
                                _pi(_i32(segments)), scale, int(window), _pd(lse))
        return lse

    def packed_backward(self, q, k, v, dout, positions, segments, scale=None, window=0):
        """Gradients of sum(dout * packed(q, k, v)) -> (dq, dk, dv), shapes of q, k, v."""
        q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
        p, h, d = q.shape
        kvh = k.shape[1]
        scale = self.default_scale(d) if scale is None else float(scale)
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        self.lib.orc_packed_backward(p, h, kvh, d, _pd(q), _pd(k), _pd(v), _pd(g),
                                     _pi(_i32(positions)), _pi(_i32(segments)), scale,
                                     int(window), _pd(dq), _pd(dk), _pd(dv))
        return dq, dk, dv

    def decode_rows(self, q, cache_k, cache_v, positions, scale=None, window=0, sinks=None):
        """q [B, Heads, D], caches [B, KvHeads, MaxSeq, D] -> [B, Heads, D]."""
        q, ck, cv = _f64(q), _f64(cache_k), _f64(cache_v)
        b, h, d = q.shape
        kvh, max_seq = ck.shape[1], ck.shape[2]
        scale = self.default_scale(d) if scale is None else float(scale)
        out = np.zeros_like(q)
        self.lib.orc_decode_rows(b, h, kvh, d, _pd(q), _pd(ck), _pd(cv), max_seq,
                                 _pi(_i32(positions)), scale, int(window), _pd(_f64(sinks)),
                                 _pd(out))
        return out

    def decode_paged(self, q, pool_k, pool_v, positions, table, scale=None, window=0,
                     sinks=None):
        """q [R, Heads, D], pools [NumPages, KvHeads, PageSize, D], table [R, Pages]."""
        q, pk, pv = _f64(q), _f64(pool_k), _f64(pool_v)
        r, h, d = q.shape
        num_pages, kvh, page_size, _ = pk.shape
        tb = _i32(table)
        scale = self.default_scale(d) if scale is None else float(scale)
        out = np.zeros_like(q)
        self.lib.orc_decode_paged(r, h, kvh, d, _pd(q), _pd(pk), _pd(pv), num_pages, page_size,
                                  _pi(_i32(positions)), _pi(tb), tb.shape[1], scale, int(window),
                                  _pd(_f64(sinks)), _pd(out))
        return out

    def prefill_cached(self, q, rows, positions, cache_k, cache_v, scale=None, window=0,
                       sinks=None):
        """Chunk tokens over a contiguous cache: q [n, Heads, D]; token i reads
        cache row rows[i] (None: row 0) at slots <= positions[i]."""
        q, ck, cv = _f64(q), _f64(cache_k), _f64(cache_v)
        n, h, d = q.shape
        batch, kvh, max_seq = ck.shape[0], ck.shape[1], ck.shape[2]
        scale = self.default_scale(d) if scale is None else float(scale)
        out = np.zeros_like(q)
        self.lib.orc_prefill_cached(n, h, kvh, d, _pd(q), _pi(_i32(rows)), _pi(_i32(positions)),
                                    batch, _pd(ck), _pd(cv), max_seq, scale, int(window),
                                    _pd(_f64(sinks)), _pd(out))
        return out

    def prefill_paged(self, q, rows, positions, pool_k, pool_v, table, scale=None, window=0,
                      sinks=None):
        """Chunk tokens over a paged pool: token i reads table row rows[i]
        (None: row 0) at logical keys <= positions[i]."""
        q, pk, pv = _f64(q), _f64(pool_k), _f64(pool_v)
        n, h, d = q.shape
        num_pages, kvh, page_size, _ = pk.shape
        tb = _i32(table)
        scale = self.default_scale(d) if scale is None else float(scale)
        out = np.zeros_like(q)
        self.lib.orc_prefill_paged(n, h, kvh, d, _pd(q), _pi(_i32(rows)), _pi(_i32(positions)),
                                   _pd(pk), _pd(pv), num_pages, page_size, _pi(tb), tb.shape[0],
                                   tb.shape[1], scale, int(window), _pd(_f64(sinks)), _pd(out))
        return out

    def linear(self, x, weight, bias=None, dtype="bf16"):
        """Linear forward: x [n, in], weight [out, in], bias [out] -> [n, out] of T."""
        x, w = _f64(x), _f64(weight)
        n, fin = x.shape
        fout = w.shape[0]
        y = np.zeros((n, fout), dtype=np.float64)
        self.lib.orc_linear(n, fin, fout, _pd(x), _pd(w), _pd(_f64(bias)), _dt(dtype), _pd(y))
        return y


_DEFAULT = None


def default():
    """The oracle built from the unmodified source."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
