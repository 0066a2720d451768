"""GPU: the paged decode entry point that allocates nothing
(gqa_decode_paged_noalloc) against gqa_decode_paged with a caller workspace,
through the C ABI: identical bits on two calls in a row, the second with a
smaller input, on plans with and without split partials, and on the plan with
the most partials the split rules allow."""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
from tests.gpu_common import CODE, DEV, TORCH_DT, bits, i32
from tests.test_gpu_decode import paged_case, run_decode_paged

pytestmark = pytest.mark.gpu


def noalloc(q, pk, pv, pos, table, heads, kvh, d, dtype, window=0, sinks=None):
    rows, pages = table.shape
    out = torch.full((rows, heads, d), float("nan"), dtype=TORCH_DT[dtype], device=DEV)
    gqa.gqa_decode_paged_noalloc(rows, pages, heads, kvh, d, CODE[dtype], 0.0, window, sinks, q, pk, pv,
                                 pk.shape[0], i32(pos), i32(table), out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("heads,kvh,d,dtype,rows,lo,hi,pages", [
    (32, 8, 128, "bf16", 2, 3000, 8000, 128),   # few rows, long contexts: several splits per row
    (64, 8, 64, "bf16", 1, 4100, 4352, 68),     # gpt-oss-shaped single row: split partials + merge
    (32, 8, 128, "bf16", 64, 512, 2048, 32),    # many rows: one split each, no partials
    (12, 12, 64, "f32", 3, 500, 1024, 16),      # vector-ALU path (f32): split partials + merge
])
def test_noalloc_matches_workspace_entry(heads, kvh, d, dtype, rows, lo, hi, pages):
    print(f"[case] decode_paged_noalloc H={heads} KvH={kvh} D={d} {dtype} rows={rows}", flush=True)
    g = np.random.default_rng(77 + rows)
    lengths = g.integers(lo, hi + 1, rows)
    num_pages = int((-(-lengths // 64)).sum()) + 8
    (q, pk, pv), _, pos, table, _, _ = paged_case(9100 + rows, rows, heads, kvh, d, lengths, pages,
                                                   num_pages, dtype)
    ref = run_decode_paged(q, pk, pv, pos, table, heads, kvh, d, dtype)
    got = noalloc(q, pk, pv, pos, table, heads, kvh, d, dtype)
    assert np.array_equal(bits(got), bits(ref)), "first call differs from the workspace entry"
    # second call in a row, smaller: fewer rows and shorter contexts
    r2 = max(1, rows // 2)
    pos2 = np.minimum(pos[:r2], pos[:r2] // 2 + 63).astype(np.int32)
    ref2 = run_decode_paged(q[:r2], pk, pv, pos2, table[:r2], heads, kvh, d, dtype)
    got2 = noalloc(q[:r2], pk, pv, pos2, table[:r2], heads, kvh, d, dtype)
    assert np.array_equal(bits(got2), bits(ref2)), "second (smaller) call differs"


def test_noalloc_largest_plan():
    """The plan with the most split partials the split rules allow: 511
    (row, KV head) units of 16 query heads with D 128 take two splits each,
    1022 x 16 partials of 130 floats (8.5 MB), inside the 16 MB array. Rows
    share a small pool through the table; bits equal to the workspace entry."""
    rows, pages, heads, kvh, d, num_pages = 511, 32, 16, 1, 128, 8
    print(f"[case] decode_paged_noalloc largest plan rows={rows} H={heads} KvH={kvh} D={d}", flush=True)
    g = np.random.default_rng(515)
    q = torch.from_numpy(g.standard_normal((rows, heads, d), dtype=np.float32)).to(DEV, torch.bfloat16)
    pk = torch.from_numpy(g.standard_normal((num_pages, kvh, 64, d), dtype=np.float32)).to(DEV, torch.bfloat16)
    pv = torch.from_numpy(g.standard_normal((num_pages, kvh, 64, d), dtype=np.float32)).to(DEV, torch.bfloat16)
    pos = g.integers(1100, pages * 64, rows).astype(np.int32)
    table = ((np.arange(rows)[:, None] + np.arange(pages)[None, :]) % num_pages).astype(np.int32)
    ref = run_decode_paged(q, pk, pv, pos, table, heads, kvh, d, "bf16")
    got = noalloc(q, pk, pv, pos, table, heads, kvh, d, "bf16")
    assert np.array_equal(bits(got), bits(ref)), "largest plan differs from the workspace entry"
    assert torch.isfinite(got.float()).all()
