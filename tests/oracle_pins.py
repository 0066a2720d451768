"""Pins that tie the fp64 oracle to something other than itself.

Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle
disagrees with what the pages and the mathematics fix. The same pins run on
the normal oracle build (tests/test_oracle_pins.py) and on builds with one
planted mistake each (tests/test_oracle_mutations.py), which must fail at
least one pin.

What pins what (the pages: Linnet "examples/01-llama" page, sections Key
ideas / src/attention.linnet / src/rope.linnet; Nest cards llama-3.1-8b-
instruct and gpt-oss-20b, blocks GroupedQueryAttention and SinkAttention):
  rounding      brute-force nearest-even search over bf16 bit patterns, and
                torch's float32 -> bfloat16 conversion (a library routine)
  scale         the default scale rsqrt(f32(H / Heads)) as literal values
                (1/sqrt(D) written out and rounded once to f32 by numpy)
  inv_freq      the closed form theta^(-2i/D) of `tables`; bit for bit, the
                page's f32 pipeline redone in numpy float32 arithmetic
  tables        numpy cos/sin of the f32 angle, rounded by torch; s = 0 row;
                bit for bit at the tiny Llama, Llama-3.1-8B and gpt-oss
                table shapes, from numpy float32 angles
  rope          hand-worked rotations of basis vectors (the textbook 2-D
                rotation on the pairs (i, i + D/2)); pair-norm preservation;
                the relative-position property of rotary embeddings
  attention     torch scaled_dot_product_attention in float64 (MHA, causal,
                enable_gqa, explicit band masks); torch.softmax over logits
                with an appended sink column; one-key and q = 0 special cases;
                rows of weights summing to one
  packing       packed == each segment alone through `forward`; permuting
                tokens permutes outputs; interleaved segment ids
  decode        decode at pos == last row of a causal forward; poisoned
                slots past pos never read
  paged         paged decode == the same cache stored contiguously; pages
                with invalid ids excluded (checked with an explicit mask)
  writes        write-then-attend equals forward; out-of-range targets leave
                the cache unchanged
  linear        torch float64 F.linear rounded once to bf16; identity and
                one-hot weights select the inputs
  chunk         chunked prefill over a cached prefix: q = 0 gives the mean of
                exactly the attended slots of the right row; torch softmax
                over an explicit mask (sink as an extra logit); a chunk into
                empty rows equals `packed`; the paged form equals the same
                cache stored contiguously; invalid pages and rows excluded
"""
import numpy as np
import torch
import torch.nn.functional as F

RNG_SEED = 1234


def _rng(salt=0):
    return np.random.default_rng(RNG_SEED + salt)


def _bf16_vals(x):
    """float32 -> nearest-even bf16 values as float64 (torch's conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def _close(a, b, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= atol, f"{what}: max abs err {err:.3e} > {atol:.1e}"


# The default softmax scale of `forward`, `packed` and `decode` (Linnet
# "examples/01-llama" page, src/attention.linnet): rsqrt of the head dim cast
# to f32. 1/sqrt(D) is written out in decimal (a power of two for D = 16 and
# 64) and rounded once to f32 by numpy's cast; the attention pins use these
# values, never the oracle's own.
_SCALE = {
    8: float(np.float32(0.35355339059327376220)),
    16: 0.25,
    64: 0.125,
    128: float(np.float32(0.088388347648318440550)),
}


def _scale_ref(d):
    return _SCALE[d]


def pin_default_scale(o):
    for d, ref in _SCALE.items():
        got = o.default_scale(d)
        assert got == ref, f"default scale D={d}: {got!r} vs {ref!r}"
    assert o.default_scale(64) == 0.125
    assert o.default_scale(128) == float(np.float32(1 / np.sqrt(128)))


# ---------------------------------------------------------------------------
# Rounding
# ---------------------------------------------------------------------------
def _bf16_rne_bruteforce(x):
    """Nearest bf16 to the double x, ties to an even last bit, by comparing the
    two bf16 neighbours read off the float32 bit pattern."""
    f = np.float32(x)  # within one float32 ulp of x
    bits = int(np.array(f, dtype=np.float32).view(np.uint32))
    lo_bits = bits & 0xFFFF0000
    cands = []
    for b in (lo_bits - 0x10000, lo_bits, lo_bits + 0x10000, lo_bits + 0x20000):
        b &= 0xFFFFFFFF
        v = float(np.array(b, dtype=np.uint32).view(np.float32))
        if np.isfinite(v):
            cands.append((b, v))
    best = None
    for b, v in cands:
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and ((b >> 16) & 1) == 0):
            best = (d, v, b)
    return best[1]


def pin_rounding(o):
    rng = _rng(1)
    # float32 inputs: torch's conversion is the library reference.
    x32 = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 3,
                          np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130,
                                      3.0e38, -3.0e38, 1e-40])])
    got = o.round(x32.astype(np.float64), "bf16")
    ref = _bf16_vals(x32)
    assert np.array_equal(got, ref), "bf16 rounding differs from torch on float32 inputs"
    # double inputs (between float32 values): brute force.
    xd = rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000))
    xd = np.concatenate([xd, [1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8 - 2 ** -40]])
    got = o.round(xd, "bf16")
    ref = np.array([_bf16_rne_bruteforce(v) for v in xd])
    assert np.array_equal(got, ref), "bf16 rounding differs from brute-force nearest-even"
    # f32 rounding of doubles: numpy's float64 -> float32 cast (nearest-even).
    got = o.round(xd, "f32")
    assert np.array_equal(got, xd.astype(np.float32).astype(np.float64)), "f32 rounding"


# ---------------------------------------------------------------------------
# Rotary tables and rotation
# ---------------------------------------------------------------------------
def pin_inv_freq(o):
    for d, theta in ((64, 10000.0), (128, 500000.0), (8, 10000.0)):
        inv = o.inv_freq(d, theta)
        i = np.arange(d // 2)
        closed = theta ** (-2.0 * i / d)
        rel = np.abs(inv - closed) / closed
        assert rel.max() < 4e-6, f"inv_freq D={d}: rel err {rel.max():.2e}"
        assert inv[0] == 1.0


def pin_tables(o):
    for seq, d, theta in ((96, 64, 10000.0), (300, 128, 500000.0)):
        c, s = o.rope_tables(seq, d, theta, "bf16")
        half = d // 2
        assert np.array_equal(c[:, :half], c[:, half:]) and np.array_equal(s[:, :half], s[:, half:])
        assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
        inv = o.inv_freq(d, theta).astype(np.float32)
        ang = np.arange(seq, dtype=np.float32)[:, None] * inv[None, :]  # f32 product
        ref_c = _bf16_vals(np.cos(ang.astype(np.float64)).astype(np.float32))
        ref_s = _bf16_vals(np.sin(ang.astype(np.float64)).astype(np.float32))
        _close(c[:, :half], ref_c, 2 ** -8, "cos table")
        _close(s[:, :half], ref_s, 2 ** -8, "sin table")
        mism = np.mean(c[:, :half] != ref_c) + np.mean(s[:, :half] != ref_s)
        assert mism < 1e-3, f"table entries differing from numpy+torch: {mism}"


def _tables_f32_numpy(seq, d, theta):
    """The `tables` pipeline (Linnet "examples/01-llama" page, src/rope.linnet)
    in numpy float32 arithmetic: every product, quotient and negation is an
    IEEE float32 operation; log, exp, cos and sin are the float64 library
    values rounded once to float32 (the correctly rounded f32 result, as the
    design reads the page's f32 ops). Returns inv_freq and the bf16 cos / sin
    halves [seq, d/2] as float64."""
    import math
    f = np.float32
    log_theta = f(math.log(float(f(theta))))
    inv = np.empty(d // 2, dtype=np.float32)
    for i in range(d // 2):
        a = f(i) * f(2.0)
        b = a / f(d)
        e = (-b) * log_theta
        inv[i] = f(math.exp(float(e)))
    ang = np.arange(seq, dtype=np.float32)[:, None] * inv[None, :]
    assert ang.dtype == np.float32
    c = np.cos(ang.astype(np.float64)).astype(np.float32)
    s = np.sin(ang.astype(np.float64)).astype(np.float32)
    return inv.astype(np.float64), _bf16_vals(c), _bf16_vals(s)


def pin_tables_f32_pipeline(o):
    # The table shapes of the tiny Llama example (theta 1e4, D 64, 512 rows),
    # the Llama-3.1-8B workloads (theta 5e5, D 128, 8192 rows) and gpt-oss
    # (theta 5e5, D 64, 4352 rows): inv_freq and every bf16 entry bit for bit.
    for seq, d, theta in ((512, 64, 10000.0), (8192, 128, 500000.0), (4352, 64, 500000.0)):
        inv_ref, c_ref, s_ref = _tables_f32_numpy(seq, d, theta)
        inv = o.inv_freq(d, theta)
        assert np.array_equal(inv, inv_ref), \
            f"inv_freq D={d} theta={theta}: {int(np.sum(inv != inv_ref))} values differ from the f32 pipeline"
        c, s = o.rope_tables(seq, d, theta, "bf16")
        half = d // 2
        nc = int(np.sum(c[:, :half] != c_ref))
        ns = int(np.sum(s[:, :half] != s_ref))
        assert nc == 0 and ns == 0, f"tables {seq}x{d}: {nc} cos and {ns} sin entries differ"


def pin_rope_hand(o):
    # D = 4: pairs (0, 2) and (1, 3); inv_freq = (1, theta^-1/2).
    d, theta = 4, 10000.0
    c, s = o.rope_tables(8, d, theta, "none")
    pos = np.array([3], dtype=np.int32)
    for basis, expect in (
        (0, {0: c[3, 0], 2: s[3, 0]}),       # e0 -> cos e0 + sin e2
        (2, {0: -s[3, 0], 2: c[3, 0]}),      # e2 -> -sin e0 + cos e2
        (1, {1: c[3, 1], 3: s[3, 1]}),
        (3, {1: -s[3, 1], 3: c[3, 1]}),
    ):
        x = np.zeros((1, 1, d))
        x[0, 0, basis] = 1.0
        y = o.rope(x, pos, c, s, "none")[0, 0]
        ref = np.zeros(d)
        for k, val in expect.items():
            ref[k] = val
        _close(y, ref, 0.0, f"rope of e{basis}")
    # angle at position 3 for pair 0 is 3 rad (inv_freq[0] = 1).
    _close(c[3, 0], np.cos(3.0), 1e-7, "cos(3)")
    # position 0 is the identity, exactly, also after rounding to bf16.
    x = _bf16_vals(_rng(2).standard_normal((5, 3, 64)).astype(np.float32))
    c2, s2 = o.rope_tables(16, 64, 500000.0, "bf16")
    y = o.rope(x, np.zeros(5, np.int32), c2, s2, "bf16")
    assert np.array_equal(x, y), "rope at position 0 must be the identity"


def pin_rope_norm_and_relative(o):
    rng = _rng(3)
    d = 64
    c, s = o.rope_tables(200, d, 10000.0, "none")
    x = rng.standard_normal((20, 2, d))
    pos = rng.integers(0, 200, 20).astype(np.int32)
    y = o.rope(x, pos, c, s, "none")
    h = d // 2
    nx = x[..., :h] ** 2 + x[..., h:] ** 2
    ny = y[..., :h] ** 2 + y[..., h:] ** 2
    _close(ny / nx, np.ones_like(nx), 1e-6, "pair norms")
    # <R_m q, R_n k> depends on m - n only.
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for m, n, delta in ((5, 2, 7), (40, 40, 13), (3, 17, 50)):
        a = np.sum(o.rope(q, [m], c, s, "none") * o.rope(k, [n], c, s, "none"))
        b = np.sum(o.rope(q, [m + delta], c, s, "none") * o.rope(k, [n + delta], c, s, "none"))
        assert abs(a - b) < 1e-4 * np.linalg.norm(q) * np.linalg.norm(k), "relative position"


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def _sdpa(q, k, v, mask, scale, gqa):
    """torch SDPA in float64. q [S, H, D], k/v [S_k, KvH, D], mask [S, S_k]."""
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0)
    tv = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0)
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask),
                                         scale=scale, enable_gqa=gqa)
    return out.squeeze(0).permute(1, 0, 2).numpy()


def pin_mha_causal(o):
    rng = _rng(4)
    s, h, d = 37, 3, 16
    q, k, v = (rng.standard_normal((1, s, h, d)) for _ in range(3))
    out = o.forward(q, k, v)[0]
    mask = np.tril(np.ones((s, s), dtype=bool))
    ref = _sdpa(q[0], k[0], v[0], mask, _scale_ref(d), False)
    _close(out, ref, 1e-12, "MHA causal vs SDPA")


def pin_gqa(o):
    rng = _rng(5)
    s, h, kvh, d = 29, 8, 2, 16
    q = rng.standard_normal((1, s, h, d))
    k, v = (rng.standard_normal((1, s, kvh, d)) for _ in range(2))
    out = o.forward(q, k, v)[0]
    mask = np.tril(np.ones((s, s), dtype=bool))
    ref = _sdpa(q[0], k[0], v[0], mask, _scale_ref(d), True)
    _close(out, ref, 1e-12, "GQA vs SDPA(enable_gqa)")
    # the same by explicit broadcast_to + reshape of the KV heads
    kr = np.broadcast_to(k[0][:, :, None, :], (s, kvh, h // kvh, d)).reshape(s, h, d)
    vr = np.broadcast_to(v[0][:, :, None, :], (s, kvh, h // kvh, d)).reshape(s, h, d)
    ref2 = _sdpa(q[0], np.ascontiguousarray(kr), np.ascontiguousarray(vr), mask,
                 _scale_ref(d), False)
    _close(out, ref2, 1e-12, "GQA vs MHA on broadcast KV heads")


def pin_window(o):
    rng = _rng(6)
    s, h, kvh, d = 40, 4, 2, 8
    q = rng.standard_normal((1, s, h, d))
    k, v = (rng.standard_normal((1, s, kvh, d)) for _ in range(2))
    for w in (1, 2, 5, 17):
        out = o.forward(q, k, v, window=w)[0]
        i = np.arange(s)[:, None]
        j = np.arange(s)[None, :]
        mask = (j <= i) & (i - j < w)
        ref = _sdpa(q[0], k[0], v[0], mask, _scale_ref(d), True)
        _close(out, ref, 1e-12, f"window {w} vs SDPA band mask")
    # window 1 keeps only the query's own key: out = v exactly
    out = o.forward(q, k, v, window=1)[0]
    g = h // kvh
    for hh in range(h):
        assert np.array_equal(out[:, hh], v[0][:, hh // g]), "window 1 must return v"


def pin_sinks(o):
    rng = _rng(7)
    s, h, kvh, d = 23, 4, 2, 8
    q = rng.standard_normal((1, s, h, d))
    k, v = (rng.standard_normal((1, s, kvh, d)) for _ in range(2))
    sinks = rng.standard_normal(h)
    scale = _scale_ref(d)
    for w in (0, 6):
        out = o.forward(q, k, v, window=w, sinks=sinks)[0]
        g = h // kvh
        tq = torch.from_numpy(q[0])
        ref = np.zeros_like(out)
        for hh in range(h):
            kk = torch.from_numpy(k[0][:, hh // g])
            vv = torch.from_numpy(v[0][:, hh // g])
            logits = (tq[:, hh] @ kk.T) * scale
            i = torch.arange(s)[:, None]
            j = torch.arange(s)[None, :]
            keep = (j <= i) & ((i - j < w) if w else torch.ones_like(i - j, dtype=torch.bool))
            logits = logits.masked_fill(~keep, float("-inf"))
            full = torch.cat([logits, torch.full((s, 1), float(sinks[hh]), dtype=torch.float64)], 1)
            p = torch.softmax(full, dim=1)[:, :s]
            ref[:, hh] = (p @ vv).numpy()
        _close(out, ref, 1e-12, f"sinks (window {w}) vs softmax with a sink column")
    # one key with a sink: out = v * sigmoid(score - sink)
    out = o.forward(q[:, :1], k[:, :1], v[:, :1], sinks=sinks)[0, 0]
    for hh in range(h):
        sc = scale * np.dot(q[0, 0, hh], k[0, 0, hh // (h // kvh)])
        ref = v[0, 0, hh // (h // kvh)] / (1.0 + np.exp(sinks[hh] - sc))
        _close(out[hh], ref, 1e-14, "one key + sink")
    # a sink at -inf is no sink
    a = o.forward(q, k, v, sinks=np.full(h, -1e300))
    b = o.forward(q, k, v)
    _close(a, b, 1e-15, "sink -> -inf")


def pin_special_cases(o):
    rng = _rng(8)
    s, h, d = 19, 2, 8
    k, v = (rng.standard_normal((1, s, h, d)) for _ in range(2))
    # q = 0: uniform weights over the causal prefix
    out = o.forward(np.zeros((1, s, h, d)), k, v)[0]
    ref = np.cumsum(v[0], axis=0) / np.arange(1, s + 1)[:, None, None]
    _close(out, ref, 1e-13, "q = 0 gives the prefix mean")
    # first query sees only key 0: out = v_0
    q = rng.standard_normal((1, s, h, d)) * 10
    out = o.forward(q, k, v)[0]
    assert np.array_equal(out[0], v[0][0]), "single allowed key must return v"
    # v = 1: every output is 1 (weights sum to one)
    out = o.forward(q, k, np.ones_like(v))[0]
    _close(out, np.ones_like(out), 1e-13, "weights sum to one")


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------
def _packed_case(rng, lengths, h, kvh, d):
    p = int(sum(lengths))
    seg = np.repeat(np.arange(len(lengths)), lengths).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    pos = (np.arange(p) - np.repeat(starts, lengths)).astype(np.int32)
    q = rng.standard_normal((p, h, d))
    k, v = (rng.standard_normal((p, kvh, d)) for _ in range(2))
    return q, k, v, pos, seg, starts


def pin_packed_equals_segments(o):
    rng = _rng(9)
    lengths = [7, 1, 12, 3, 9]
    h, kvh, d = 4, 2, 8
    q, k, v, pos, seg, starts = _packed_case(rng, lengths, h, kvh, d)
    sinks = rng.standard_normal(h)
    for w, sk in ((0, None), (4, sinks)):
        out = o.packed(q, k, v, pos, seg, window=w, sinks=sk)
        for st, n in zip(starts, lengths):
            alone = o.forward(q[None, st:st + n], k[None, st:st + n], v[None, st:st + n],
                              window=w, sinks=sk)[0]
            _close(out[st:st + n], alone, 1e-13, "packed vs segment alone")
    # causal within a segment, by a library routine too
    out = o.packed(q, k, v, pos, seg)
    st, n = starts[2], lengths[2]
    ref = _sdpa(q[st:st + n], k[st:st + n], v[st:st + n], np.tril(np.ones((n, n), bool)),
                _scale_ref(d), True)
    _close(out[st:st + n], ref, 1e-12, "packed segment vs SDPA causal")
    # sampled queries give the same rows
    sel = np.array([0, 5, 20, 31], dtype=np.int32)
    _close(o.packed(q, k, v, pos, seg, sel=sel), out[sel], 0.0, "sampled queries")


def pin_packed_permutation(o):
    rng = _rng(10)
    q, k, v, pos, seg, _ = _packed_case(rng, [6, 10, 4], 2, 1, 8)
    perm = rng.permutation(q.shape[0])
    a = o.packed(q, k, v, pos, seg)
    b = o.packed(q[perm], k[perm], v[perm], pos[perm], seg[perm])
    _close(b, a[perm], 1e-13, "permuting packed tokens permutes the outputs")
    # interleaved, non-contiguous segment ids: token order is irrelevant
    seg2 = np.array([5, 9, 5, 9, 5, 9], dtype=np.int32)
    pos2 = np.array([0, 0, 1, 1, 2, 2], dtype=np.int32)
    q2, k2, v2 = q[:6], k[:6], v[:6]
    out = o.packed(q2, k2, v2, pos2, seg2)
    idx = np.array([0, 2, 4])
    alone = o.forward(q2[None, idx], k2[None, idx], v2[None, idx])[0]
    _close(out[idx], alone, 1e-13, "interleaved segment ids")


# ---------------------------------------------------------------------------
# Decode and the cache
# ---------------------------------------------------------------------------
def pin_decode_is_last_forward_row(o):
    rng = _rng(11)
    b, s_max, h, kvh, d = 3, 24, 4, 2, 8
    cache_k = np.full((b, kvh, s_max, d), np.nan)
    cache_v = np.full((b, kvh, s_max, d), np.nan)
    seqs = [rng.standard_normal((1, n, kvh, d)) for n in (1, 2, 3)]
    positions = np.array([9, 0, 16], dtype=np.int32)
    qs = rng.standard_normal((b, h, d))
    sinks = rng.standard_normal(h)
    for w, sk in ((0, None), (3, sinks)):
        kk = [rng.standard_normal((1, p + 1, kvh, d)) for p in positions]
        vv = [rng.standard_normal((1, p + 1, kvh, d)) for p in positions]
        ck, cv = cache_k.copy(), cache_v.copy()
        for r, p in enumerate(positions):
            ck, cv, _ = o.write_contiguous(kk[r][0], vv[r][0], np.arange(p + 1, dtype=np.int32),
                                           ck, cv, rows=np.full(p + 1, r, np.int32))
        out = o.decode_rows(qs, ck, cv, positions, window=w, sinks=sk)
        assert np.all(np.isfinite(out)), "decode read a poisoned slot past pos"
        for r, p in enumerate(positions):
            qq = np.zeros((1, p + 1, h, d))
            qq[0, p] = qs[r]
            ref = o.forward(qq, kk[r], vv[r], window=w, sinks=sk)[0, p]
            _close(out[r], ref, 1e-13, "decode vs last row of forward")
    del seqs


def pin_paged_equals_contiguous(o):
    rng = _rng(12)
    rows, h, kvh, d, ps = 4, 4, 2, 8, 4
    max_seq = 20
    pages = max_seq // ps
    ck = rng.standard_normal((rows, kvh, max_seq, d))
    cv = rng.standard_normal((rows, kvh, max_seq, d))
    num_pages = rows * pages + 3
    perm = rng.permutation(num_pages)
    table = perm[:rows * pages].reshape(rows, pages).astype(np.int32)
    pk = np.full((num_pages, kvh, ps, d), np.nan)
    pv = np.full((num_pages, kvh, ps, d), np.nan)
    for r in range(rows):
        for t in range(max_seq):
            pk[table[r, t // ps], :, t % ps] = ck[r, :, t]
            pv[table[r, t // ps], :, t % ps] = cv[r, :, t]
    q = rng.standard_normal((rows, h, d))
    positions = np.array([0, 7, 13, 19], dtype=np.int32)
    sinks = rng.standard_normal(h)
    for w, sk in ((0, None), (5, sinks)):
        a = o.decode_paged(q, pk, pv, positions, table, window=w, sinks=sk)
        b = o.decode_rows(q, ck, cv, positions, window=w, sinks=sk)
        assert np.array_equal(a, b), "paged decode differs from the contiguous cache"
    # a page whose id is outside the pool contributes no keys
    t2 = table.copy()
    t2[2, 1] = -1
    t2[3, 2] = num_pages + 5
    a = o.decode_paged(q, pk, pv, positions, t2)
    scale = _scale_ref(d)
    for r in range(rows):
        keep = np.arange(max_seq) <= positions[r]
        for pg in range(pages):
            if not (0 <= t2[r, pg] < num_pages):
                keep[pg * ps:(pg + 1) * ps] = False
        for hh in range(h):
            kk = torch.from_numpy(ck[r, hh // (h // kvh)])
            logits = (torch.from_numpy(q[r, hh]) @ kk.T) * scale
            logits = logits.masked_fill(~torch.from_numpy(keep), float("-inf"))
            ref = (torch.softmax(logits, 0) @ torch.from_numpy(cv[r, hh // (h // kvh)])).numpy()
            _close(a[r, hh], ref, 1e-12, "invalid page ids excluded")


def pin_writes(o):
    rng = _rng(13)
    kvh, d = 2, 4
    batch, max_seq = 3, 6
    n = 5
    k = rng.standard_normal((n, kvh, d))
    v = rng.standard_normal((n, kvh, d))
    ck0 = rng.standard_normal((batch, kvh, max_seq, d))
    cv0 = rng.standard_normal((batch, kvh, max_seq, d))
    rows = np.array([0, 2, 5, -1, 1], dtype=np.int32)      # 5 and -1 are out of range
    pos = np.array([3, 0, 1, 2, 6], dtype=np.int32)        # 6 is out of range
    ck, cv, wr = o.write_contiguous(k, v, pos, ck0, cv0, rows=rows)
    assert np.array_equal(ck[0, :, 3], k[0]) and np.array_equal(cv[2, :, 0], v[1])
    expect = np.zeros_like(wr)
    expect[0, :, 3] = True
    expect[2, :, 0] = True
    assert np.array_equal(wr, expect), "only in-range targets are written"
    assert np.array_equal(ck[~wr], ck0[~wr]) and np.array_equal(cv[~wr], cv0[~wr])
    # paged by slots and by table land where the page rules say
    num_pages, ps = 4, 2
    pk0 = rng.standard_normal((num_pages, kvh, ps, d))
    pv0 = rng.standard_normal((num_pages, kvh, ps, d))
    slots = np.array([7, 0, 8, -1, 3], dtype=np.int32)     # 8 and -1 out of range
    pk, pv, wr = o.write_paged(k, v, pk0, pv0, slots=slots)
    assert np.array_equal(pk[3, :, 1], k[0]) and np.array_equal(pv[0, :, 0], v[1])
    assert np.array_equal(pk[1, :, 1], k[4]) and wr.sum() == 3 * kvh * d
    table = np.array([[2, 0], [1, -1]], dtype=np.int32)
    trow = np.array([0, 0, 1, 1, 2], dtype=np.int32)        # row 2 out of range
    tpos = np.array([3, 0, 1, 2, 0], dtype=np.int32)        # row 1 pos 2 -> page -1
    pk, pv, wr = o.write_paged(k, v, pk0, pv0, positions=tpos, rows=trow, table=table)
    assert np.array_equal(pk[0, :, 1], k[0]) and np.array_equal(pk[2, :, 0], k[1])
    assert np.array_equal(pv[1, :, 1], v[2]) and wr.sum() == 3 * kvh * d
    # write-then-decode equals forward (prefill_slots style placement)
    s = 6
    kk = rng.standard_normal((s, kvh, d))
    vv = rng.standard_normal((s, kvh, d))
    ck, cv, _ = o.write_contiguous(kk, vv, np.arange(s, dtype=np.int32),
                                   np.full((batch, kvh, max_seq, d), np.nan),
                                   np.full((batch, kvh, max_seq, d), np.nan),
                                   rows=np.full(s, 1, np.int32))
    qq = rng.standard_normal((1, s, 2 * kvh, d))
    ref = o.forward(qq, kk[None], vv[None])[0, s - 1]
    out = o.decode_rows(np.stack([qq[0, s - 1]] * batch), ck, cv,
                        np.array([-1, s - 1, -1], dtype=np.int32))
    _close(out[1], ref, 1e-13, "prefill_slots write then decode")
    assert np.all(out[0] == 0) and np.all(out[2] == 0), "no key -> 0"


# ---------------------------------------------------------------------------
# Chunked prefill over a cached prefix
# ---------------------------------------------------------------------------
def _chunk_keep(pos, cap, window):
    """Slots a token at `pos` attends in a row of `cap` slots."""
    t = np.arange(cap)
    keep = t <= pos
    if window > 0:
        keep &= (pos - t >= 0) & (pos - t < window)
    return keep


def pin_chunk_cached(o):
    rng = _rng(14)
    batch, max_seq, h, kvh, d = 3, 24, 4, 2, 8
    g = h // kvh
    ck = rng.standard_normal((batch, kvh, max_seq, d))
    cv = rng.standard_normal((batch, kvh, max_seq, d))
    # chunk tokens of several rows, interleaved; a row outside the cache, a
    # position past the cache, a negative position
    rows = np.array([1, 0, 1, 2, 1, 0, 3, 2, -1, 0], dtype=np.int32)
    pos = np.array([5, 0, 6, 23, 7, 1, 4, 30, 2, -1], dtype=np.int32)
    n = rows.shape[0]
    scale = _scale_ref(d)
    for w, sk in ((0, None), (4, rng.standard_normal(h))):
        # q = 0: uniform weights, the mean of the attended values (closed form)
        out0 = o.prefill_cached(np.zeros((n, h, d)), rows, pos, ck, cv, window=w)
        for i in range(n):
            r = rows[i]
            keep = _chunk_keep(pos[i], max_seq, w) if 0 <= r < batch else np.zeros(max_seq, bool)
            for hh in range(h):
                ref = cv[r, hh // g][keep].mean(0) if keep.any() else np.zeros(d)
                _close(out0[i, hh], ref, 1e-13, "chunk over cache, q = 0 mean")
        # random q: softmax over an explicit mask (torch), sink as an extra logit
        q = rng.standard_normal((n, h, d))
        out = o.prefill_cached(q, rows, pos, ck, cv, window=w, sinks=sk)
        for i in range(n):
            r = rows[i]
            if not (0 <= r < batch) or not _chunk_keep(pos[i], max_seq, w).any():
                assert np.all(out[i] == 0), "no key -> 0"
                continue
            keep = torch.from_numpy(_chunk_keep(pos[i], max_seq, w))
            for hh in range(h):
                logits = (torch.from_numpy(ck[r, hh // g]) @ torch.from_numpy(q[i, hh])) * scale
                logits = logits.masked_fill(~keep, float("-inf"))
                vals = torch.from_numpy(cv[r, hh // g])
                if sk is not None:
                    logits = torch.cat([logits, torch.tensor([sk[hh]], dtype=torch.float64)])
                    vals = torch.cat([vals, torch.zeros(1, d, dtype=torch.float64)])
                ref = (torch.softmax(logits, 0) @ vals).numpy()
                _close(out[i, hh], ref, 1e-12, "chunk over cache vs explicit mask")
    # a prompt written into empty rows and attended as one chunk is `packed`
    lengths = [5, 3]
    kk = rng.standard_normal((sum(lengths), kvh, d))
    vv = rng.standard_normal((sum(lengths), kvh, d))
    qq = rng.standard_normal((sum(lengths), h, d))
    seg = np.repeat(np.arange(2, dtype=np.int32), lengths)
    ppos = np.concatenate([np.arange(L, dtype=np.int32) for L in lengths])
    ck2, cv2, _ = o.write_contiguous(kk, vv, ppos, np.full((2, kvh, 8, d), np.nan),
                                     np.full((2, kvh, 8, d), np.nan), rows=seg)
    a = o.prefill_cached(qq, seg, ppos, ck2, cv2)
    b = o.packed(qq, kk, vv, ppos, seg)
    _close(a, b, 1e-13, "chunk into empty rows == packed")


def pin_chunk_paged(o):
    rng = _rng(15)
    rows_n, h, kvh, d, ps = 3, 4, 2, 8, 4
    max_seq = 20
    pages = max_seq // ps
    ck = rng.standard_normal((rows_n, kvh, max_seq, d))
    cv = rng.standard_normal((rows_n, kvh, max_seq, d))
    num_pages = rows_n * pages + 2
    table = rng.permutation(num_pages)[:rows_n * pages].reshape(rows_n, pages).astype(np.int32)
    pk = np.full((num_pages, kvh, ps, d), np.nan)
    pv = np.full((num_pages, kvh, ps, d), np.nan)
    for r in range(rows_n):
        for t in range(max_seq):
            pk[table[r, t // ps], :, t % ps] = ck[r, :, t]
            pv[table[r, t // ps], :, t % ps] = cv[r, :, t]
    rows = np.array([2, 0, 2, 1, 0, 2], dtype=np.int32)
    pos = np.array([17, 3, 18, 9, 4, 19], dtype=np.int32)
    q = rng.standard_normal((rows.shape[0], h, d))
    for w, sk in ((0, None), (6, rng.standard_normal(h))):
        a = o.prefill_paged(q, rows, pos, pk, pv, table, window=w, sinks=sk)
        b = o.prefill_cached(q, rows, pos, ck, cv, window=w, sinks=sk)
        assert np.array_equal(a, b), "paged chunk differs from the same cache stored contiguously"
    # invalid page ids and rows outside the table contribute nothing (q = 0)
    t2 = table.copy()
    t2[2, 3] = -1
    t2[0, 0] = num_pages
    rows2 = np.concatenate([rows, np.array([3], np.int32)])
    pos2 = np.concatenate([pos, np.array([5], np.int32)])
    out0 = o.prefill_paged(np.zeros((rows2.shape[0], h, d)), rows2, pos2, pk, pv, t2)
    for i in range(rows2.shape[0]):
        r = rows2[i]
        if not (0 <= r < rows_n):
            assert np.all(out0[i] == 0), "row outside the table -> 0"
            continue
        keep = _chunk_keep(pos2[i], max_seq, 0)
        for pg in range(pages):
            if not (0 <= t2[r, pg] < num_pages):
                keep[pg * ps:(pg + 1) * ps] = False
        for hh in range(h):
            ref = cv[r, hh // (h // kvh)][keep].mean(0) if keep.any() else np.zeros(d)
            _close(out0[i, hh], ref, 1e-13, "paged chunk, invalid pages excluded")


# ---------------------------------------------------------------------------
# Linear (the q / k / v projections)
# ---------------------------------------------------------------------------
def pin_linear(o):
    rng = _rng(16)
    n, fin, fout = 7, 24, 10
    x = _bf16_vals(rng.standard_normal((n, fin)))
    w = _bf16_vals(rng.standard_normal((fout, fin)))
    b = _bf16_vals(rng.standard_normal(fout))
    # against torch's float64 F.linear, then one rounding to bf16 (torch's)
    for bias in (None, b):
        ref = F.linear(torch.from_numpy(x), torch.from_numpy(w),
                       None if bias is None else torch.from_numpy(bias))
        ref_t = ref.to(torch.bfloat16).to(torch.float64).numpy()
        got = o.linear(x, w, bias, "bf16")
        assert np.array_equal(got, ref_t), "linear differs from F.linear rounded to bf16"
        raw = o.linear(x, w, bias, "none")
        _close(raw, ref.numpy(), 1e-12, "linear before rounding")
    # identity weights return x; a one-hot row selects one input feature
    eye = np.eye(fin)
    assert np.array_equal(o.linear(x, eye, None, "bf16"), x)
    sel = np.zeros((3, fin))
    sel[0, 5] = sel[1, 0] = sel[2, fin - 1] = 1.0
    assert np.array_equal(o.linear(x, sel, None, "bf16"), x[:, [5, 0, fin - 1]])


def _torch_packed(q, k, v, positions, segments, scale, window):
    """The packed attention through torch (float64): a key mask built from
    own[i, j] and the window, F.scaled_dot_product_attention per head."""
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    pos = torch.from_numpy(positions.astype(np.int64))
    seg = torch.from_numpy(segments.astype(np.int64))
    keep = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    if window > 0:
        keep &= (pos[:, None] - pos[None, :]) < window
    g = q.shape[1] // k.shape[1]
    kx = kt.repeat_interleave(g, dim=1).permute(1, 0, 2)
    vx = vt.repeat_interleave(g, dim=1).permute(1, 0, 2)
    return qt, kt, vt, keep, kx, vx


def pin_packed_lse(o):
    rng = _rng(17)
    lengths = [5, 1, 9, 6]
    h, kvh, d = 4, 2, 8
    p = sum(lengths)
    positions = np.concatenate([np.arange(n) for n in lengths]).astype(np.int32)
    segments = np.concatenate([np.full(n, i) for i, n in enumerate(lengths)]).astype(np.int32)
    q = _bf16_vals(rng.standard_normal((p, h, d)))
    k = _bf16_vals(rng.standard_normal((p, kvh, d)))
    scale = d ** -0.5
    for window in (0, 3):
        lse = o.packed_lse(q, k, positions, segments, scale, window)
        qt, kt, _, keep, kx, _ = _torch_packed(q, k, k, positions, segments, scale, window)
        scores = scale * torch.matmul(qt.permute(1, 0, 2), kx.transpose(1, 2))
        scores = scores.masked_fill(~keep, float("-inf"))
        ref = torch.logsumexp(scores, dim=-1).permute(1, 0).numpy()
        _close(lse, ref, 1e-12, f"packed lse (window {window})")
    # a segment's first token sees only itself: lse = scale * <q, k>
    first = 5
    for hh in range(h):
        kk = hh // (h // kvh)
        assert abs(lse[first, hh] - scale * float(q[first, hh] @ k[first, kk])) < 1e-12


def pin_packed_backward(o):
    rng = _rng(18)
    lengths = [6, 1, 11, 4]
    h, kvh, d = 4, 2, 8
    p = sum(lengths)
    positions = np.concatenate([np.arange(n) for n in lengths]).astype(np.int32)
    segments = np.concatenate([np.full(n, i) for i, n in enumerate(lengths)]).astype(np.int32)
    q = rng.standard_normal((p, h, d))
    k = rng.standard_normal((p, kvh, d))
    v = rng.standard_normal((p, kvh, d))
    g = rng.standard_normal((p, h, d))
    scale = d ** -0.5
    for window in (0, 4):
        dq, dk, dv = o.packed_backward(q, k, v, g, positions, segments, scale, window)
        # torch autograd through scaled_dot_product_attention (float64)
        qt, kt, vt, keep, _, _ = _torch_packed(q, k, v, positions, segments, scale, window)
        qt.requires_grad_(True)
        kt.requires_grad_(True)
        vt.requires_grad_(True)
        grp = h // kvh
        kx = kt.repeat_interleave(grp, dim=1).permute(1, 0, 2)
        vx = vt.repeat_interleave(grp, dim=1).permute(1, 0, 2)
        out = F.scaled_dot_product_attention(qt.permute(1, 0, 2), kx, vx, attn_mask=keep, scale=scale)
        out.permute(1, 0, 2).backward(torch.from_numpy(g))
        _close(dq, qt.grad.numpy(), 1e-11, f"dq (window {window})")
        _close(dk, kt.grad.numpy(), 1e-11, f"dk (window {window})")
        _close(dv, vt.grad.numpy(), 1e-11, f"dv (window {window})")
    # central differences of the oracle's own forward at a few entries
    dq, dk, dv = o.packed_backward(q, k, v, g, positions, segments, scale, 0)
    loss = lambda qq, kk, vv: float(np.sum(g * o.packed(qq, kk, vv, positions, segments, scale)))
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            fp = loss(*(xp if a is x else a for a in args))
            fm = loss(*(xm if a is x else a for a in args))
            fd = (fp - fm) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6 * (1 + abs(fd)), f"d{name}{idx}: {grad[idx]} vs {fd}"


ALL_PINS = {
    "rounding": pin_rounding,
    "default_scale": pin_default_scale,
    "inv_freq": pin_inv_freq,
    "tables": pin_tables,
    "tables_f32_pipeline": pin_tables_f32_pipeline,
    "rope_hand": pin_rope_hand,
    "rope_norm_relative": pin_rope_norm_and_relative,
    "mha_causal": pin_mha_causal,
    "gqa": pin_gqa,
    "window": pin_window,
    "sinks": pin_sinks,
    "special_cases": pin_special_cases,
    "packed_segments": pin_packed_equals_segments,
    "packed_permutation": pin_packed_permutation,
    "decode_last_row": pin_decode_is_last_forward_row,
    "paged_contiguous": pin_paged_equals_contiguous,
    "writes": pin_writes,
    "chunk_cached": pin_chunk_cached,
    "chunk_paged": pin_chunk_paged,
    "linear": pin_linear,
    "packed_lse": pin_packed_lse,
    "packed_backward": pin_packed_backward,
}


def failing_pins(o):
    """Names of the pins this oracle build fails."""
    bad = []
    for name, fn in ALL_PINS.items():
        try:
            fn(o)
        except AssertionError:
            bad.append(name)
    return bad
