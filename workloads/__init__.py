"""Seeded synthetic inputs for the attention hot path.

This module only draws numbers and index structures; it holds none of the
method's arithmetic, so both the HIP-path tests and the CPU oracle can take
their inputs from it. Values are standard normal (the Nest cards bind no
weights here, so the projected q/k/v are synthetic), index structures follow
the shapes the pages name:

* the Nest llama-3.1-8b-instruct card (Heads 32, KvHeads 8, H 4096 so
  head dim 128, MaxSeq 8192, PageSize 64, a [Rows, Pages] page table);
* the Nest gpt2 card (H 768, Heads 12, MaxSeq 1024, T f32);
* the Nest gpt-oss-20b card (Heads 64, KvHeads 8, HeadDim 64, Window 128);
* the Linnet "examples/01-llama" page (the bind line: H 512, Heads 8,
  KvHeads 8, MaxSeq 512; `packed`'s positions/segments).

Every stream comes from numpy's PCG64 seeded through SeedSequence(seed).spawn,
one child stream per role in a fixed order, so a (config, seed) pair always
yields the same tensors on every machine.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

# Child-stream roles, in spawn order.
_ROLES = ("q", "k", "v", "sinks", "index", "pool_k", "pool_v", "extra")


def streams(seed: int):
    """Independent generators for each role of one seeded instance."""
    kids = np.random.SeedSequence(int(seed)).spawn(len(_ROLES))
    return {r: np.random.Generator(np.random.PCG64(s)) for r, s in zip(_ROLES, kids)}


def normal(gen: np.random.Generator, shape) -> np.ndarray:
    """Standard-normal float32 samples."""
    return gen.standard_normal(size=shape, dtype=np.float32)


# ---------------------------------------------------------------------------
# Workload descriptions (sizes only).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    kv_heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"
    theta: Optional[float]  # None: no rotary positions
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.heads // self.kv_heads


TINY_LLAMA = Workload("tiny-llama-example prefill S=128 + 16 decode steps, MaxSeq 512",
                      8, 8, 64, "bf16", 10000.0,
                      dict(batch=1, prefill=128, decode_steps=16, max_seq=512))
GPT2_DECODE_ROWS = Workload("gpt2 MHA decode_rows f32, Batch 32, cache [32,12,1024,64]",
                            12, 12, 64, "f32", None,
                            dict(batch=32, max_seq=1024))
LLAMA8B_PAGED = Workload("llama-3.1-8b paged decode bf16, Rows 64, L~U[512,8192], pool 9000 pages",
                         32, 8, 128, "bf16", 500000.0,
                         dict(rows=64, page_size=64, len_lo=512, len_hi=8192, num_pages=9000))
LLAMA8B_PACKED = Workload("llama-3.1-8b packed prefill bf16, P=16384, segments U[64,4096]",
                          32, 8, 128, "bf16", 500000.0,
                          dict(p=16384, seg_lo=64, seg_hi=4096))
GPT_OSS_SINK = Workload("gpt-oss-20b SinkAttention bf16, prefill 4096 + 256 decode, W 128 / full",
                        64, 8, 64, "bf16", 500000.0,
                        dict(prefill=4096, decode_steps=256, windows=(128, 0), max_seq=4352))

LLAMA8B_CHUNKED = Workload("llama-3.1-8b chunked prefill over a paged prefix bf16, Rows 16, "
                           "prefix U[1024,7168], chunk 512",
                           32, 8, 128, "bf16", 500000.0,
                           dict(rows=16, pre_lo=1024, pre_hi=7168, chunk=512, num_pages=2200,
                                max_len=8192))

ALL = (TINY_LLAMA, GPT2_DECODE_ROWS, LLAMA8B_PAGED, LLAMA8B_PACKED, GPT_OSS_SINK)


# ---------------------------------------------------------------------------
# Index structures.
# ---------------------------------------------------------------------------
def segment_layout(p: int, lo: int, hi: int, gen: np.random.Generator
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Pack segments of length U[lo, hi] into one row of p tokens; the last
    one is truncated to fit. Returns (lengths, positions[p], segments[p]):
    positions restart at 0 in every segment, segment ids are 0, 1, 2, ..."""
    lengths = []
    total = 0
    while total < p:
        n = int(gen.integers(lo, hi + 1))
        n = min(n, p - total)
        lengths.append(n)
        total += n
    lengths = np.asarray(lengths, dtype=np.int64)
    segments = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    positions = (np.arange(p, dtype=np.int64) - np.repeat(starts, lengths)).astype(np.int32)
    return lengths, positions, segments


def paged_layout(rows: int, len_lo: int, len_hi: int, num_pages: int, page_size: int,
                 gen: np.random.Generator, max_len: Optional[int] = None):
    """Row lengths L_r ~ U[len_lo, len_hi]; each row takes consecutive runs of
    one seeded permutation of the page pool, ceil(L_r / page_size) pages;
    unused table entries are -1. Returns (lengths, positions = L - 1,
    table[rows, pages])."""
    lengths = gen.integers(len_lo, len_hi + 1, size=rows).astype(np.int64)
    max_len = int(max_len if max_len is not None else len_hi)
    pages = -(-max_len // page_size)
    need = -(-lengths // page_size)
    if int(need.sum()) > num_pages:
        raise ValueError("page pool too small for the drawn lengths")
    perm = gen.permutation(num_pages).astype(np.int32)
    table = np.full((rows, pages), -1, dtype=np.int32)
    cursor = 0
    for r in range(rows):
        table[r, :need[r]] = perm[cursor:cursor + need[r]]
        cursor += int(need[r])
    positions = (lengths - 1).astype(np.int32)
    return lengths, positions, table


def chunked_layout(rows: int, pre_lo: int, pre_hi: int, chunk: int, num_pages: int,
                   page_size: int, gen: np.random.Generator, max_len: int):
    """Chunked prefill over a paged prefix: row r holds a prefix of
    U[pre_lo, pre_hi] tokens and receives `chunk` new tokens at positions
    prefix_r .. prefix_r + chunk - 1; pages as in paged_layout for the total
    length. Returns (prefixes, token_rows[n], token_positions[n], table),
    tokens of one row contiguous."""
    prefixes = gen.integers(pre_lo, pre_hi + 1, size=rows).astype(np.int64)
    lengths = prefixes + chunk
    pages = -(-max_len // page_size)
    need = -(-lengths // page_size)
    if int(need.sum()) > num_pages or int(lengths.max()) > max_len:
        raise ValueError("page pool or table too small for the drawn lengths")
    perm = gen.permutation(num_pages).astype(np.int32)
    table = np.full((rows, pages), -1, dtype=np.int32)
    cursor = 0
    for r in range(rows):
        table[r, :need[r]] = perm[cursor:cursor + need[r]]
        cursor += int(need[r])
    tok_rows = np.repeat(np.arange(rows, dtype=np.int32), chunk)
    tok_pos = np.concatenate([np.arange(p, p + chunk) for p in prefixes]).astype(np.int32)
    return prefixes, tok_rows, tok_pos, table


def uniform_positions(n: int, lo: int, hi: int, gen: np.random.Generator) -> np.ndarray:
    """n positions uniform in [lo, hi]."""
    return gen.integers(lo, hi + 1, size=n).astype(np.int32)


def sample_indices(n: int, k: int, gen: np.random.Generator) -> np.ndarray:
    """k distinct sorted indices out of n (all of them if k >= n)."""
    if k >= n:
        return np.arange(n, dtype=np.int32)
    return np.sort(gen.choice(n, size=k, replace=False)).astype(np.int32)


# ---------------------------------------------------------------------------
# Device-side values for the large benchmark tensors (the 2.4 GB page pool):
# torch's seeded generator on the device, one generator per role.
# ---------------------------------------------------------------------------
_ROLE_ID = {r: i for i, r in enumerate(_ROLES)}


def device_normal(shape, seed: int, role: str, dtype, device="cuda"):
    """Standard-normal values drawn on `device` from a generator seeded by
    (seed, role), converted to `dtype` (round to nearest even)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + _ROLE_ID[role])
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)
