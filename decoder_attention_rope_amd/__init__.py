"""Python binding of the gfx950 grouped-query attention library (libgqa.so).

Argument marshalling only: each function has the name and argument order of
the C entry point declared in include/gqa.h, takes torch tensors (or raw
device addresses as ints, or None for NULL) and the current HIP stream, calls
the library through ctypes, and raises GQAError on a non-zero status. Every
step of the attention path runs in the library's kernels; there is no
fallback of any kind. Importing this module fails loudly if the library has
not been built (`python -m decoder_attention_rope_amd.build` or
`__graft_entry__.build()`).
"""
import ctypes
import os

__all__ = [
    "GQAError", "lib", "library_path",
    "GQA_OK", "GQA_ERR_INVALID_ARG", "GQA_ERR_UNSUPPORTED", "GQA_ERR_WORKSPACE", "GQA_ERR_HIP",
    "GQA_ERR_INDEX", "GQA_OP_PREFILL_PACKED", "GQA_OP_PREFILL_CACHED", "GQA_OP_PREFILL_BACKWARD",
    "GQA_OP_DECODE_ROWS", "GQA_OP_DECODE_PAGED", "GQA_OP_STEP_PACKED", "GQA_OP_STEP_PAGED",
    "GQA_BF16", "GQA_F32", "GQA_CACHE_NONE", "GQA_CACHE_CONTIGUOUS", "GQA_CACHE_PAGED_TABLE",
    "GQA_CACHE_PAGED_SLOTS", "GQA_PAGE_SIZE",
    "gqa_rope_table", "gqa_rope_write_kv", "gqa_prefill_packed", "gqa_prefill_packed_workspace",
    "gqa_prefill_packed_plan", "gqa_prefill_packed_planned",
    "gqa_prefill_cached", "gqa_prefill_cached_workspace", "gqa_step_packed",
    "gqa_step_packed_workspace", "gqa_step_paged", "gqa_step_paged_workspace",
    "gqa_qkv_rope_write", "gqa_prefill_packed_lse", "gqa_prefill_packed_backward",
    "gqa_prefill_packed_backward_workspace",
    "gqa_decode_rows", "gqa_decode_rows_workspace", "gqa_decode_paged",
    "gqa_decode_paged_workspace", "gqa_decode_paged_noalloc", "GQA_DECODE_SCRATCH_BYTES",
    "gqa_status_string", "gqa_status_str", "gqa_workspace_bytes",
    "gqa_set_dry_run", "gqa_set_checked", "gqa_abi_version", "gqa_diag_stream_read",
    "GQA_DIAG_READ_BLOCKS",
    "dtype_code",
]

GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP = 0, 1, 2, 3, 4
GQA_ERR_INDEX = 5
GQA_DECODE_SCRATCH_BYTES = 16 << 20
GQA_DIAG_READ_BLOCKS = 2048
(GQA_OP_PREFILL_PACKED, GQA_OP_PREFILL_CACHED, GQA_OP_PREFILL_BACKWARD, GQA_OP_DECODE_ROWS,
 GQA_OP_DECODE_PAGED, GQA_OP_STEP_PACKED, GQA_OP_STEP_PAGED) = range(7)
GQA_BF16, GQA_F32 = 0, 1
GQA_CACHE_NONE, GQA_CACHE_CONTIGUOUS, GQA_CACHE_PAGED_TABLE, GQA_CACHE_PAGED_SLOTS = 0, 1, 2, 3
GQA_PAGE_SIZE = 64

# The in-tree build, or another build of the same sources named by
# GQA_LIBRARY (the host-sanitizer test loads one that way).
library_path = os.environ.get("GQA_LIBRARY") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa.so")
if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build the HIP library first "
        "(python -m decoder_attention_rope_amd.build)")

lib = ctypes.CDLL(library_path)

_i32, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


def _sig(name, restype, argtypes):
    fn = getattr(lib, name)
    fn.restype = restype
    fn.argtypes = argtypes
    return fn


_rope_table = _sig("gqa_rope_table", ctypes.c_int, [_i32, _i32, _f32, _i32, _vp, _vp])
_rope_write_kv = _sig("gqa_rope_write_kv", ctypes.c_int,
                      [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp,
                       _i32, _i32, _vp, _vp, _vp, _i32, _i32, _vp])
_prefill_packed = _sig("gqa_prefill_packed", ctypes.c_int,
                       [_i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                        _vp, _vp, _sz, _vp])
_prefill_ws = _sig("gqa_prefill_packed_workspace", _sz, [_i32, _i32, _i32, _i32])
_prefill_plan = _sig("gqa_prefill_packed_plan", ctypes.c_int,
                     [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp])
_prefill_planned = _sig("gqa_prefill_packed_planned", ctypes.c_int,
                        [_i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                         _vp, _vp, _sz, _vp])
_prefill_lse = _sig("gqa_prefill_packed_lse", ctypes.c_int,
                    [_i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32] + [_vp] * 7 +
                    [_vp, _sz, _vp])
_prefill_bwd = _sig("gqa_prefill_packed_backward", ctypes.c_int,
                    [_i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32] + [_vp] * 11 +
                    [_vp, _sz, _vp])
_prefill_bwd_ws = _sig("gqa_prefill_packed_backward_workspace", _sz, [_i32, _i32, _i32, _i32])
_prefill_cached = _sig("gqa_prefill_cached", ctypes.c_int,
                       [_i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _i32, _vp,
                        _vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _sz, _vp])
_prefill_cached_ws = _sig("gqa_prefill_cached_workspace", _sz, [_i32, _i32, _i32, _i32])
_step_packed = _sig("gqa_step_packed", ctypes.c_int,
                    [_i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                     _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp])
_step_packed_ws = _sig("gqa_step_packed_workspace", _sz, [_i32, _i32, _i32, _i32, _i32, _i32])
_step_paged = _sig("gqa_step_paged", ctypes.c_int,
                   [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp,
                    _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp])
_step_paged_ws = _sig("gqa_step_paged_workspace", _sz, [_i32, _i32, _i32, _i32, _i32, _i32])
_qkv = _sig("gqa_qkv_rope_write", ctypes.c_int,
            [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
             _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _vp])
_decode_rows = _sig("gqa_decode_rows", ctypes.c_int,
                    [_i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                     _vp, _sz, _vp])
_decode_rows_ws = _sig("gqa_decode_rows_workspace", _sz, [_i32, _i32, _i32, _i32, _i32])
_decode_paged = _sig("gqa_decode_paged", ctypes.c_int,
                     [_i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _i32,
                      _vp, _vp, _vp, _vp, _sz, _vp])
_decode_paged_ws = _sig("gqa_decode_paged_workspace", _sz, [_i32, _i32, _i32, _i32, _i32])
_decode_paged_noalloc = _sig("gqa_decode_paged_noalloc", ctypes.c_int,
                             [_i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp,
                              _i32, _vp, _vp, _vp, _vp])
_status_string = _sig("gqa_status_string", ctypes.c_char_p, [_i32])
_status_str = _sig("gqa_status_str", ctypes.c_char_p, [_i32])
_workspace_bytes = _sig("gqa_workspace_bytes", _sz, [_i32] * 7)
_set_dry_run = _sig("gqa_set_dry_run", _i32, [_i32])
_set_checked = _sig("gqa_set_checked", _i32, [_i32])
_abi_version = _sig("gqa_abi_version", _i32, [])
_diag_stream_read = _sig("gqa_diag_stream_read", ctypes.c_int, [_vp, _sz, _vp, _vp])


class GQAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {gqa_status_string(status)} (status {status})")


def _ptr(x):
    """Device address of a tensor, an int address as is, None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    try:
        import torch
        if torch.cuda.is_available() and torch.cuda.is_initialized():
            return torch.cuda.current_stream().cuda_stream
    except Exception:
        pass
    return None


def _check(status, where):
    if status != GQA_OK:
        raise GQAError(status, where)


def dtype_code(torch_dtype):
    import torch
    if torch_dtype == torch.bfloat16:
        return GQA_BF16
    if torch_dtype == torch.float32:
        return GQA_F32
    raise ValueError(f"unsupported dtype {torch_dtype}")


def gqa_status_string(status):
    return _status_string(int(status)).decode()


def gqa_status_str(status):
    return _status_str(int(status)).decode()


def gqa_workspace_bytes(op, heads, kv_heads, head_dim, n_tokens, n_rows, max_len):
    return _workspace_bytes(op, heads, kv_heads, head_dim, n_tokens, n_rows, max_len)


def gqa_set_dry_run(on):
    """Dry run for calls made from the calling thread; returns the previous setting."""
    return _set_dry_run(1 if on else 0)


def gqa_set_checked(on):
    """Checked mode for calls made from the calling thread; returns the previous setting."""
    return _set_checked(1 if on else 0)


def gqa_abi_version():
    return _abi_version()


def gqa_diag_stream_read(buffer, nbytes, out, stream=None):
    """Diagnostic outside the attention path: one streaming read of nbytes at
    buffer; out holds GQA_DIAG_READ_BLOCKS 32-bit words, workgroup b's XOR of
    the words it read in out[b]."""
    _check(_diag_stream_read(_ptr(buffer), nbytes, _ptr(out), _stream(stream)), "gqa_diag_stream_read")


def gqa_rope_table(head_dim, max_pos, theta, dtype, table, stream=None):
    _check(_rope_table(head_dim, max_pos, theta, dtype, _ptr(table), _stream(stream)),
           "gqa_rope_table")


def gqa_rope_write_kv(n, heads, kv_heads, head_dim, dtype, q, k, v, positions, rope_table,
                      rope_max_pos, cache_kind, cache_k, cache_v, cache_dim0, cache_seq, rows,
                      slots, table, table_rows, table_pages, stream=None):
    _check(_rope_write_kv(n, heads, kv_heads, head_dim, dtype, _ptr(q), _ptr(k), _ptr(v),
                          _ptr(positions), _ptr(rope_table), rope_max_pos, cache_kind,
                          _ptr(cache_k), _ptr(cache_v), cache_dim0, cache_seq, _ptr(rows),
                          _ptr(slots), _ptr(table), table_rows, table_pages, _stream(stream)),
           "gqa_rope_write_kv")


def gqa_prefill_packed_workspace(p, heads, kv_heads, head_dim):
    return _prefill_ws(p, heads, kv_heads, head_dim)


def gqa_prefill_packed(p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, k, v,
                       positions, segments, out, workspace, workspace_bytes, stream=None):
    _check(_prefill_packed(p, heads, kv_heads, head_dim, dtype, scale, window, _ptr(sinks),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(segments), _ptr(out),
                           _ptr(workspace), workspace_bytes, _stream(stream)),
           "gqa_prefill_packed")


def gqa_prefill_packed_plan(p, heads, kv_heads, head_dim, window, positions, segments, workspace,
                            workspace_bytes, stream=None):
    _check(_prefill_plan(p, heads, kv_heads, head_dim, window, _ptr(positions), _ptr(segments),
                         _ptr(workspace), workspace_bytes, _stream(stream)),
           "gqa_prefill_packed_plan")


def gqa_prefill_packed_planned(p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, k, v,
                               positions, segments, out, workspace, workspace_bytes, stream=None):
    _check(_prefill_planned(p, heads, kv_heads, head_dim, dtype, scale, window, _ptr(sinks),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(segments), _ptr(out),
                            _ptr(workspace), workspace_bytes, _stream(stream)),
           "gqa_prefill_packed_planned")


def gqa_prefill_packed_lse(p, heads, kv_heads, head_dim, dtype, scale, window, q, k, v,
                           positions, segments, out, lse, workspace, workspace_bytes, stream=None):
    _check(_prefill_lse(p, heads, kv_heads, head_dim, dtype, scale, window, _ptr(q), _ptr(k),
                        _ptr(v), _ptr(positions), _ptr(segments), _ptr(out), _ptr(lse),
                        _ptr(workspace), workspace_bytes, _stream(stream)),
           "gqa_prefill_packed_lse")


def gqa_prefill_packed_backward_workspace(p, heads, kv_heads, head_dim):
    return _prefill_bwd_ws(p, heads, kv_heads, head_dim)


def gqa_prefill_packed_backward(p, heads, kv_heads, head_dim, dtype, scale, window, q, k, v, out,
                                dout, lse, positions, segments, dq, dk, dv, workspace,
                                workspace_bytes, stream=None):
    _check(_prefill_bwd(p, heads, kv_heads, head_dim, dtype, scale, window, _ptr(q), _ptr(k),
                        _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(positions),
                        _ptr(segments), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                        workspace_bytes, _stream(stream)),
           "gqa_prefill_packed_backward")


def gqa_prefill_cached_workspace(n, heads, kv_heads, head_dim):
    return _prefill_cached_ws(n, heads, kv_heads, head_dim)


def gqa_prefill_cached(n, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, rows,
                       positions, cache_kind, cache_k, cache_v, cache_dim0, cache_seq, table,
                       table_rows, table_pages, out, workspace, workspace_bytes, stream=None):
    _check(_prefill_cached(n, heads, kv_heads, head_dim, dtype, scale, window, _ptr(sinks),
                           _ptr(q), _ptr(rows), _ptr(positions), cache_kind, _ptr(cache_k),
                           _ptr(cache_v), cache_dim0, cache_seq, _ptr(table), table_rows,
                           table_pages, _ptr(out), _ptr(workspace), workspace_bytes,
                           _stream(stream)),
           "gqa_prefill_cached")


def gqa_step_packed_workspace(batch, p, heads, kv_heads, head_dim, max_seq):
    return _step_packed_ws(batch, p, heads, kv_heads, head_dim, max_seq)


def gqa_step_packed(batch, p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, k, v,
                    positions, segments, cache_k, cache_v, max_seq, step_positions, out, workspace,
                    workspace_bytes, stream=None):
    _check(_step_packed(batch, p, heads, kv_heads, head_dim, dtype, scale, window, _ptr(sinks),
                        _ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(segments), _ptr(cache_k),
                        _ptr(cache_v), max_seq, _ptr(step_positions), _ptr(out), _ptr(workspace),
                        workspace_bytes, _stream(stream)),
           "gqa_step_packed")


def gqa_step_paged_workspace(p, rows, pages, heads, kv_heads, head_dim):
    return _step_paged_ws(p, rows, pages, heads, kv_heads, head_dim)


def gqa_step_paged(p, rows, pages, heads, kv_heads, head_dim, dtype, scale, window, sinks, q,
                   token_rows, positions, pool_k, pool_v, num_pages, table, step_positions, out,
                   workspace, workspace_bytes, stream=None):
    _check(_step_paged(p, rows, pages, heads, kv_heads, head_dim, dtype, scale, window,
                       _ptr(sinks), _ptr(q), _ptr(token_rows), _ptr(positions), _ptr(pool_k),
                       _ptr(pool_v), num_pages, _ptr(table), _ptr(step_positions), _ptr(out),
                       _ptr(workspace), workspace_bytes, _stream(stream)),
           "gqa_step_paged")


def gqa_qkv_rope_write(n, hidden, heads, kv_heads, head_dim, dtype, x, w_q, w_k, w_v, b_q, b_k,
                       b_v, positions, rope_table, rope_max_pos, q_out, k_out, v_out, cache_kind,
                       cache_k, cache_v, cache_dim0, cache_seq, rows, slots, table, table_rows,
                       table_pages, stream=None):
    _check(_qkv(n, hidden, heads, kv_heads, head_dim, dtype, _ptr(x), _ptr(w_q), _ptr(w_k),
                _ptr(w_v), _ptr(b_q), _ptr(b_k), _ptr(b_v), _ptr(positions), _ptr(rope_table),
                rope_max_pos, _ptr(q_out), _ptr(k_out), _ptr(v_out), cache_kind, _ptr(cache_k),
                _ptr(cache_v), cache_dim0, cache_seq, _ptr(rows), _ptr(slots), _ptr(table),
                table_rows, table_pages, _stream(stream)),
           "gqa_qkv_rope_write")


def gqa_decode_rows_workspace(batch, heads, kv_heads, head_dim, max_seq):
    return _decode_rows_ws(batch, heads, kv_heads, head_dim, max_seq)


def gqa_decode_rows(batch, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, cache_k,
                    cache_v, max_seq, positions, out, workspace, workspace_bytes, stream=None):
    _check(_decode_rows(batch, heads, kv_heads, head_dim, dtype, scale, window, _ptr(sinks),
                        _ptr(q), _ptr(cache_k), _ptr(cache_v), max_seq, _ptr(positions),
                        _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "gqa_decode_rows")


def gqa_decode_paged_workspace(rows, pages, heads, kv_heads, head_dim):
    return _decode_paged_ws(rows, pages, heads, kv_heads, head_dim)


def gqa_decode_paged(rows, pages, heads, kv_heads, head_dim, dtype, scale, window, sinks, q,
                     pool_k, pool_v, num_pages, positions, table, out, workspace,
                     workspace_bytes, stream=None):
    _check(_decode_paged(rows, pages, heads, kv_heads, head_dim, dtype, scale, window,
                         _ptr(sinks), _ptr(q), _ptr(pool_k), _ptr(pool_v), num_pages,
                         _ptr(positions), _ptr(table), _ptr(out), _ptr(workspace),
                         workspace_bytes, _stream(stream)),
           "gqa_decode_paged")


def gqa_decode_paged_noalloc(rows, pages, heads, kv_heads, head_dim, dtype, scale, window, sinks,
                             q, pool_k, pool_v, num_pages, positions, table, out, stream=None):
    _check(_decode_paged_noalloc(rows, pages, heads, kv_heads, head_dim, dtype, scale, window,
                                 _ptr(sinks), _ptr(q), _ptr(pool_k), _ptr(pool_v), num_pages,
                                 _ptr(positions), _ptr(table), _ptr(out), _stream(stream)),
           "gqa_decode_paged_noalloc")
