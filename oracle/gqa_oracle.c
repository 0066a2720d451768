/*
 * gqa_oracle.c -- fp64 CPU oracle for grouped-query causal attention with
 * rotary positions over a KV cache.
 *
 * TEST INFRASTRUCTURE. This file states, plainly and slowly, what the
 * attention hot path computes. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it. It shares no code, header, table or
 * helper with the HIP library, and the HIP library never loads it.
 *
 * Sources (the pages):
 *   [L] Linnet docs, "examples/01-llama": src/rope.linnet (`tables`, THETA),
 *       src/attention.linnet (`forward`, `packed`, `decode`, split_heads),
 *       and the "Key ideas" section (grouped-query attention, KV cache in
 *       state, write_at as a masked select).
 *   [N1] Nest card llama-3.1-8b-instruct, block GroupedQueryAttention
 *       (serving signatures: decode_rows, prefill_slots, prefill_packed,
 *       decode_paged, prefill_paged; generic PageSize = 64).
 *   [N3] Nest card gpt-oss-20b, block SinkAttention (`window: i32`,
 *       `param sinks: Tensor[Heads; T]`), generics Window = 128.
 *
 * Readings taken where the pages leave a step open are listed beside each
 * function and in the design notes; the short form:
 *   - grouped_attention = masked scaled-dot-product softmax attention; query
 *     head h reads KV head floor(h / (Heads/KvHeads)) (each KV head repeated
 *     for consecutive query heads by broadcast_to + reshape).
 *   - rope = rotate-half: y_lo = x_lo*c - x_hi*s, y_hi = x_hi*c + x_lo*s,
 *     evaluated exactly and rounded once to T.
 *   - window W > 0 keeps a key iff 0 <= pos_q - pos_k < W; W = 0 is no window.
 *   - a sink adds exp(sink_h) to the softmax denominator (no value vector,
 *     not multiplied by the scale).
 *   - a query with no allowed key returns 0.
 *   - write_at drops a write whose target is outside the cache.
 *   - a decode key whose page id is outside the pool contributes nothing.
 *
 * Data convention: every T-valued tensor is passed as an array of doubles
 * holding T values exactly (bf16 and f32 upcast without error). Index
 * tensors are int32. All arithmetic is fp64 unless a step of the pages is
 * written in f32, in which case it is rounded to f32 exactly where the page
 * rounds.
 *
 * Mutation hooks: ORC_MUTATE (compile-time, default 0) plants one known
 * mistake so the test suite can prove its pins catch it. A normal build
 * never defines it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORC_MUTATE
#define ORC_MUTATE 0
#endif

#define ORC_DT_NONE (-1) /* keep the value as is */
#define ORC_DT_BF16 0
#define ORC_DT_F32 1

/* ------------------------------------------------------------------------ */
/* Rounding to a binary floating-point format, round-to-nearest-even.        */
/* bf16: 8 significant bits, f32: 24; both have the f32 exponent range, so   */
/* the smallest subnormal spacing is 2^-133 (bf16) or 2^-149 (f32) and the   */
/* first value that rounds to infinity is 2^128 - half an ulp.              */
/* ------------------------------------------------------------------------ */
double orc_round(double x, int dtype) {
  if (dtype == ORC_DT_NONE) return x;
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  const int prec = (dtype == ORC_DT_BF16) ? 8 : 24;
  const int min_q = (dtype == ORC_DT_BF16) ? -133 : -149;
  int e;
  (void)frexp(x, &e); /* |x| = m * 2^e with m in [0.5, 1) */
  int q = e - prec;   /* exponent of one unit in the last place */
  if (q < min_q) q = min_q;
  double scaled = ldexp(x, -q); /* exact: a power-of-two scaling */
  double r = nearbyint(scaled); /* default rounding mode: nearest-even */
#if ORC_MUTATE == 10
  r = trunc(scaled);
#endif
  r = ldexp(r, q);
  if (fabs(r) >= 0x1p128) return copysign(INFINITY, x);
  return r;
}

static double f32(double x) { return orc_round(x, ORC_DT_F32); }

/* rsqrt(cast<f32>(H / Heads)) of `forward`, `packed` and `decode` [L], read
 * as the correctly rounded f32 value of 1/sqrt(D). */
double orc_default_scale(int head_dim) {
#if ORC_MUTATE == 15
  return 1.0 / sqrt((double)head_dim);
#else
  return f32(1.0 / sqrt(f32((double)head_dim)));
#endif
}

/* ------------------------------------------------------------------------ */
/* Rotary tables: [L], src/rope.linnet, `tables` (with THETA).               */
/* The page builds, in f32, one inverse frequency per pair of head           */
/* dimensions (theta raised to minus twice the pair index over D, written    */
/* as an exponential of a product with log theta), multiplies each by the    */
/* position to get the angle, repeats the angles for both halves of the     */
/* head dimension and casts their cosine and sine to T.                      */
/* The f32 steps, in order: i -> f32, times 2, divided by f32(D), negated,   */
/* times f32(log(f32(theta))), exp; angle = f32(s) * inv_freq (one f32      */
/* product); cos and sin of that angle in f32, then rounded to T.            */
/* Reading: each f32 operation (including exp, log, cos, sin) returns the    */
/* correctly rounded f32 result; the double-precision library value rounded */
/* to f32 stands for it. `dtype` is T (ORC_DT_NONE keeps the f32 values).   */
/* Outputs are the full [S, D] tables, halves duplicated as on the page.    */
/* ------------------------------------------------------------------------ */
void orc_inv_freq(int D, double theta, double* inv_freq /* [D/2] */) {
  const double log_theta = f32(log(f32(theta)));
#if ORC_MUTATE == 16
  for (int i = 0; i < D / 2; ++i) inv_freq[i] = f32(exp(-(2.0 * i / D) * log(theta)));
  return;
#endif
  for (int i = 0; i < D / 2; ++i) {
    double a = f32(f32((double)i) * 2.0);
#if ORC_MUTATE == 9
    double b = f32(a / f32((double)(D / 2)));
#else
    double b = f32(a / f32((double)D));
#endif
    double e = f32(-b * log_theta);
    inv_freq[i] = f32(exp(e));
  }
}

void orc_rope_tables(int S, int D, double theta, int dtype,
                     double* cos_full /* [S, D] */, double* sin_full /* [S, D] */) {
  const int half = D / 2;
  double* inv_freq = (double*)malloc(sizeof(double) * (size_t)(half > 0 ? half : 1));
  orc_inv_freq(D, theta, inv_freq);
  for (int s = 0; s < S; ++s) {
    for (int i = 0; i < half; ++i) {
      double angle = f32(f32((double)s) * inv_freq[i]);
      double c = orc_round(f32(cos(angle)), dtype);
      double sn = orc_round(f32(sin(angle)), dtype);
      cos_full[(size_t)s * D + i] = c;
      cos_full[(size_t)s * D + i + half] = c;
      sin_full[(size_t)s * D + i] = sn;
      sin_full[(size_t)s * D + i + half] = sn;
    }
  }
  free(inv_freq);
}

/* ------------------------------------------------------------------------ */
/* rope(x, cos_at, sin_at) [L]: the tables gathered at each token's          */
/* position (`packed`: cos_table[positions[p], d]; `decode`: row pos) and    */
/* applied rotate-half to every head of x:                                   */
/*   y[d]       = x[d]       * cos[d]       - x[d + D/2] * sin[d]            */
/*   y[d + D/2] = x[d + D/2] * cos[d + D/2] + x[d]       * sin[d + D/2]      */
/* evaluated in fp64 and rounded once to `dtype`. x: [n, nheads, D]; the    */
/* tables are [S, D]. A position outside [0, S) reads the nearest row (the  */
/* pages do not define that gather; the value there is unpinned).           */
/* ------------------------------------------------------------------------ */
void orc_rope(int n, int nheads, int D, const double* x, const int32_t* positions,
              const double* cos_full, const double* sin_full, int S, int dtype, double* y) {
  const int half = D / 2;
  for (int t = 0; t < n; ++t) {
    int p = positions[t];
    if (p < 0) p = 0;
    if (p >= S) p = S - 1;
    const double* c = cos_full + (size_t)p * D;
    const double* s = sin_full + (size_t)p * D;
    for (int h = 0; h < nheads; ++h) {
      const double* xi = x + ((size_t)t * nheads + h) * D;
      double* yi = y + ((size_t)t * nheads + h) * D;
      for (int d = 0; d < half; ++d) {
        double lo = xi[d], hi = xi[d + half];
#if ORC_MUTATE == 3
        double ylo = lo * c[d] + hi * s[d];
#else
        double ylo = lo * c[d] - hi * s[d];
#endif
        double yhi = hi * c[d + half] + lo * s[d + half];
        yi[d] = orc_round(ylo, dtype);
        yi[d + half] = orc_round(yhi, dtype);
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Cache writes: std.nn.cache::write_at, "a masked select" [L, KV cache in   */
/* state]; `decode` writes k and v at `pos`. Reading: a write whose target  */
/* is outside the cache is dropped and nothing else changes. `written`     */
/* (same shape as the cache, may be NULL) receives 1 where a write landed.  */
/* ------------------------------------------------------------------------ */

/* Contiguous cache [batch, kv_heads, max_seq, D] (state cache_k/cache_v).
 * Token t goes to row rows[t] (0 when rows is NULL) at position positions[t]. */
void orc_write_contiguous(int n, int kv_heads, int D, const double* k, const double* v,
                          const int32_t* rows, const int32_t* positions, int batch,
                          int max_seq, double* cache_k, double* cache_v,
                          int8_t* written) {
  for (int t = 0; t < n; ++t) {
    int row = rows ? rows[t] : 0;
    int pos = positions[t];
    if (row < 0 || row >= batch || pos < 0 || pos >= max_seq) continue;
    for (int kh = 0; kh < kv_heads; ++kh) {
      size_t dst = (((size_t)row * kv_heads + kh) * max_seq + pos) * D;
      size_t src = ((size_t)t * kv_heads + kh) * D;
      for (int d = 0; d < D; ++d) {
        if (k) cache_k[dst + d] = k[src + d];
        if (v) cache_v[dst + d] = v[src + d];
        if (written) written[dst + d] = 1;
      }
    }
  }
}

/* Paged pool [num_pages, kv_heads, page_size, D] for both K and V (the plain
 * layout; the pages fix only the [Rows, Pages] table and PageSize = 64).
 * With slots != NULL, token t goes to physical slot slots[t] = page *
 * page_size + offset (prefill_paged's `slots`). Otherwise the logical
 * position positions[t] of table row rows[t] (0 when NULL) goes to page
 * table[row, pos / page_size], offset pos % page_size (decode_paged). */
void orc_write_paged(int n, int kv_heads, int D, const double* k, const double* v,
                     const int32_t* rows, const int32_t* positions, const int32_t* slots,
                     const int32_t* table, int table_rows, int table_pages, int num_pages,
                     int page_size, double* pool_k, double* pool_v, int8_t* written) {
  for (int t = 0; t < n; ++t) {
    long page, off;
    if (slots) {
      long slot = slots[t];
      if (slot < 0 || slot >= (long)num_pages * page_size) continue;
      page = slot / page_size;
      off = slot % page_size;
    } else {
      int row = rows ? rows[t] : 0;
      long pos = positions[t];
      if (row < 0 || row >= table_rows) continue;
      if (pos < 0 || pos >= (long)table_pages * page_size) continue;
      page = table[(size_t)row * table_pages + pos / page_size];
      off = pos % page_size;
      if (page < 0 || page >= num_pages) continue;
    }
    for (int kh = 0; kh < kv_heads; ++kh) {
      size_t dst = (((size_t)page * kv_heads + kh) * page_size + off) * D;
      size_t src = ((size_t)t * kv_heads + kh) * D;
      for (int d = 0; d < D; ++d) {
        if (k) pool_k[dst + d] = k[src + d];
        if (v) pool_v[dst + d] = v[src + d];
        if (written) written[dst + d] = 1;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* grouped_attention for one query vector and one head [L]: softmax over the */
/* enumerated key set of scale * <q, k_j>, weights applied to v_j. Two      */
/* passes in fp64: the maximum, then the exponentials. A sink logit adds    */
/* exp(sink) to the denominator [N3]. An empty key set returns 0.           */
/* ------------------------------------------------------------------------ */
static void attend(int D, const double* q, int nk, const double* const* keys,
                   const double* const* vals, double scale, int has_sink, double sink,
                   double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (nk == 0) return;
  double* s = (double*)malloc(sizeof(double) * (size_t)nk);
  double m = -INFINITY;
  for (int j = 0; j < nk; ++j) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * keys[j][d];
#if ORC_MUTATE == 2
    s[j] = dot;
#else
    s[j] = scale * dot;
#endif
    if (s[j] > m) m = s[j];
  }
#if ORC_MUTATE == 6
  if (has_sink) sink = scale * sink;
#endif
  if (has_sink && sink > m) m = sink;
  double z = 0.0;
  for (int j = 0; j < nk; ++j) {
    s[j] = exp(s[j] - m);
    z += s[j];
  }
  if (has_sink) z += exp(sink - m);
  for (int j = 0; j < nk; ++j) {
    const double w = s[j] / z;
    for (int d = 0; d < D; ++d) out[d] += w * vals[j][d];
  }
  free(s);
}

/* Query head h reads KV head floor(h / G), G = Heads / KvHeads: each KV head
 * is repeated for G consecutive query heads by broadcast_to and a reshape
 * [L, Grouped-query attention]. */
static int kv_head_of(int h, int heads, int kv_heads) {
#if ORC_MUTATE == 1
  (void)heads;
  return h % kv_heads;
#else
  return h / (heads / kv_heads);
#endif
}

/* Window predicate on positions: W > 0 keeps iff 0 <= pos_q - pos_k < W. */
static int in_window(long pos_q, long pos_k, int window) {
  if (window <= 0) return 1;
  long d = pos_q - pos_k;
#if ORC_MUTATE == 5
  return d >= 0 && d <= window;
#else
  return d >= 0 && d < window;
#endif
}

/* ------------------------------------------------------------------------ */
/* `forward<B, S>` [L]: every row attends over its own S tokens with          */
/* causal_mask<S, S> (key j kept for query i iff j <= i); q, k already       */
/* rotated with tables<S> (positions 0..S-1). q: [B, S, Heads, D],           */
/* k, v: [B, S, KvHeads, D] (split_heads' layout before the permute).       */
/* ------------------------------------------------------------------------ */
void orc_forward(int B, int S, int heads, int kv_heads, int D, const double* q,
                 const double* k, const double* v, double scale, int window,
                 const double* sinks, double* out) {
  const long total = (long)B * S * heads;
#pragma omp parallel
  {
    const double** kp = (const double**)malloc(sizeof(double*) * (size_t)(S > 0 ? S : 1));
    const double** vp = (const double**)malloc(sizeof(double*) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 16)
    for (long idx = 0; idx < total; ++idx) {
      const int h = (int)(idx % heads);
      const int i = (int)((idx / heads) % S);
      const int b = (int)(idx / ((long)heads * S));
      const int kh = kv_head_of(h, heads, kv_heads);
      int nk = 0;
      for (int j = 0; j <= i; ++j) {
        if (!in_window(i, j, window)) continue;
        kp[nk] = k + (((size_t)b * S + j) * kv_heads + kh) * D;
        vp[nk] = v + (((size_t)b * S + j) * kv_heads + kh) * D;
        ++nk;
      }
      attend(D, q + (((size_t)b * S + i) * heads + h) * D, nk, kp, vp, scale,
             sinks != NULL, sinks ? sinks[h] : 0.0, out + (((size_t)b * S + i) * heads + h) * D);
    }
    free(kp);
    free(vp);
  }
}

/* ------------------------------------------------------------------------ */
/* `packed<P>` [L] (also the attention of prefill_packed [N1]): token i      */
/* attends key j iff own[i, j] = segments[i] == segments[j] &&              */
/* positions[j] <= positions[i], then the window on positions [N3].          */
/* q: [P, Heads, D]; k, v: [P, KvHeads, D]. `sel` lists the query tokens to */
/* compute (NULL: all P, nsel ignored); out rows follow sel's order:        */
/* out[r, h, :] for query sel[r].                                           */
/* ------------------------------------------------------------------------ */
void orc_packed(int P, int heads, int kv_heads, int D, const double* q, const double* k,
                const double* v, const int32_t* positions, const int32_t* segments,
                double scale, int window, const double* sinks, int nsel, const int32_t* sel,
                double* out) {
  const int nq = sel ? nsel : P;
  const long total = (long)nq * heads;
#pragma omp parallel
  {
    const double** kp = (const double**)malloc(sizeof(double*) * (size_t)(P > 0 ? P : 1));
    const double** vp = (const double**)malloc(sizeof(double*) * (size_t)(P > 0 ? P : 1));
#pragma omp for schedule(dynamic, 4)
    for (long idx = 0; idx < total; ++idx) {
      const int h = (int)(idx % heads);
      const int r = (int)(idx / heads);
      const int i = sel ? sel[r] : r;
      const int kh = kv_head_of(h, heads, kv_heads);
      int nk = 0;
      for (int j = 0; j < P; ++j) {
#if ORC_MUTATE == 4
        int own = segments[i] == segments[j] && positions[j] < positions[i];
#else
        int own = segments[i] == segments[j] && positions[j] <= positions[i];
#endif
        if (!own || !in_window(positions[i], positions[j], window)) continue;
        kp[nk] = k + ((size_t)j * kv_heads + kh) * D;
        vp[nk] = v + ((size_t)j * kv_heads + kh) * D;
        ++nk;
      }
      attend(D, q + ((size_t)i * heads + h) * D, nk, kp, vp, scale, sinks != NULL,
             sinks ? sinks[h] : 0.0, out + ((size_t)r * heads + h) * D);
    }
    free(kp);
    free(vp);
  }
}

/* ------------------------------------------------------------------------ */
/* `decode` / `decode_rows` [L, N1]: row b's query attends every slot s of    */
/* its own cache row with seen[s] = s <= positions[b] (iota over MaxSeq),   */
/* then the window on (positions[b], s). q, out: [B, Heads, D]; caches:     */
/* [B, KvHeads, max_seq, D].                                                */
/* ------------------------------------------------------------------------ */
void orc_decode_rows(int B, int heads, int kv_heads, int D, const double* q,
                     const double* cache_k, const double* cache_v, int max_seq,
                     const int32_t* positions, double scale, int window, const double* sinks,
                     double* out) {
  const long total = (long)B * heads;
#pragma omp parallel
  {
    const double** kp = (const double**)malloc(sizeof(double*) * (size_t)(max_seq > 0 ? max_seq : 1));
    const double** vp = (const double**)malloc(sizeof(double*) * (size_t)(max_seq > 0 ? max_seq : 1));
#pragma omp for schedule(dynamic, 1)
    for (long idx = 0; idx < total; ++idx) {
      const int h = (int)(idx % heads);
      const int b = (int)(idx / heads);
      const int kh = kv_head_of(h, heads, kv_heads);
      const long pos = positions[b];
      int nk = 0;
      for (int s = 0; s < max_seq; ++s) {
#if ORC_MUTATE == 7
        int seen = s < pos;
#else
        int seen = s <= pos;
#endif
        if (!seen || !in_window(pos, s, window)) continue;
        kp[nk] = cache_k + (((size_t)b * kv_heads + kh) * max_seq + s) * D;
        vp[nk] = cache_v + (((size_t)b * kv_heads + kh) * max_seq + s) * D;
        ++nk;
      }
      attend(D, q + ((size_t)b * heads + h) * D, nk, kp, vp, scale, sinks != NULL,
             sinks ? sinks[h] : 0.0, out + ((size_t)b * heads + h) * D);
    }
    free(kp);
    free(vp);
  }
}

/* ------------------------------------------------------------------------ */
/* `decode_paged<Rows, Pages>` [N1]: row r's logical key t (0 <= t <          */
/* Pages * page_size) lives at page table[r, t / page_size], offset           */
/* t % page_size of the pool [num_pages, KvHeads, page_size, D]. Key t is    */
/* attended iff t <= positions[r] and the window keeps it; a key whose page  */
/* id is outside [0, num_pages) contributes nothing.                         */
/* ------------------------------------------------------------------------ */
void orc_decode_paged(int R, int heads, int kv_heads, int D, const double* q,
                      const double* pool_k, const double* pool_v, int num_pages,
                      int page_size, const int32_t* positions, const int32_t* table,
                      int pages, double scale, int window, const double* sinks, double* out) {
  const long total = (long)R * heads;
  const long max_t = (long)pages * page_size;
#pragma omp parallel
  {
    const double** kp = (const double**)malloc(sizeof(double*) * (size_t)(max_t > 0 ? max_t : 1));
    const double** vp = (const double**)malloc(sizeof(double*) * (size_t)(max_t > 0 ? max_t : 1));
#pragma omp for schedule(dynamic, 1)
    for (long idx = 0; idx < total; ++idx) {
      const int h = (int)(idx % heads);
      const int r = (int)(idx / heads);
      const int kh = kv_head_of(h, heads, kv_heads);
      const long pos = positions[r];
      int nk = 0;
      for (long t = 0; t < max_t; ++t) {
        if (!(t <= pos) || !in_window(pos, t, window)) continue;
#if ORC_MUTATE == 8
        long page = table[(size_t)r * pages + t % pages];
        long off = t / pages;
#else
        long page = table[(size_t)r * pages + t / page_size];
        long off = t % page_size;
#endif
        if (page < 0 || page >= num_pages) continue;
        kp[nk] = pool_k + (((size_t)page * kv_heads + kh) * page_size + off) * D;
        vp[nk] = pool_v + (((size_t)page * kv_heads + kh) * page_size + off) * D;
        ++nk;
      }
      attend(D, q + ((size_t)r * heads + h) * D, nk, kp, vp, scale, sinks != NULL,
             sinks ? sinks[h] : 0.0, out + ((size_t)r * heads + h) * D);
    }
    free(kp);
    free(vp);
  }
}

/* ------------------------------------------------------------------------ */
/* `prefill<S>(x, pos)` with pos > 0 [L, N1] (reading; the page gives the    */
/* signature only): the chunk's tokens were written into their cache row at */
/* their positions (write_at, as `decode` does for one token), and each of  */
/* them attends every slot s of that row with s <= its position (`seen`),   */
/* then the window -- the prefix written by earlier calls included. Token i */
/* uses cache row rows[i] (0 when rows is NULL); a row outside [0, batch)   */
/* has no keys. q, out: [n, Heads, D]; caches [batch, KvHeads, max_seq, D]. */
/* With one token per row this is decode_rows.                              */
/* ------------------------------------------------------------------------ */
void orc_prefill_cached(int n, int heads, int kv_heads, int D, const double* q,
                        const int32_t* rows, const int32_t* positions, int batch,
                        const double* cache_k, const double* cache_v, int max_seq,
                        double scale, int window, const double* sinks, double* out) {
  const long total = (long)n * heads;
#pragma omp parallel
  {
    const double** kp = (const double**)malloc(sizeof(double*) * (size_t)(max_seq > 0 ? max_seq : 1));
    const double** vp = (const double**)malloc(sizeof(double*) * (size_t)(max_seq > 0 ? max_seq : 1));
#pragma omp for schedule(dynamic, 4)
    for (long idx = 0; idx < total; ++idx) {
      const int h = (int)(idx % heads);
      const int i = (int)(idx / heads);
      const int kh = kv_head_of(h, heads, kv_heads);
#if ORC_MUTATE == 11
      const int row = 0;
#else
      const int row = rows ? rows[i] : 0;
#endif
      const long pos = positions[i];
      int nk = 0;
      for (int s = 0; row >= 0 && row < batch && s < max_seq; ++s) {
        if (!(s <= pos) || !in_window(pos, s, window)) continue;
        kp[nk] = cache_k + (((size_t)row * kv_heads + kh) * max_seq + s) * D;
        vp[nk] = cache_v + (((size_t)row * kv_heads + kh) * max_seq + s) * D;
        ++nk;
      }
      attend(D, q + ((size_t)i * heads + h) * D, nk, kp, vp, scale, sinks != NULL,
             sinks ? sinks[h] : 0.0, out + ((size_t)i * heads + h) * D);
    }
    free(kp);
    free(vp);
  }
}

/* ------------------------------------------------------------------------ */
/* `prefill_paged<P, Rows, Pages>` [N1] (reading; signature only): token i   */
/* of table row rows[i] at logical position positions[i] attends key t      */
/* (0 <= t < pages * page_size) of that row iff t <= positions[i] and the   */
/* window keeps it, key t living at page table[row, t / page_size], offset  */
/* t % page_size (decode_paged's addressing; the chunk's own keys were      */
/* written at their `slots` beforehand). Keys on page ids outside           */
/* [0, num_pages) and rows outside [0, table_rows) contribute nothing. With */
/* one token per row this is decode_paged.                                  */
/* ------------------------------------------------------------------------ */
void orc_prefill_paged(int n, int heads, int kv_heads, int D, const double* q,
                       const int32_t* rows, const int32_t* positions, const double* pool_k,
                       const double* pool_v, int num_pages, int page_size, const int32_t* table,
                       int table_rows, int pages, double scale, int window, const double* sinks,
                       double* out) {
  const long total = (long)n * heads;
  const long max_t = (long)pages * page_size;
#pragma omp parallel
  {
    const double** kp = (const double**)malloc(sizeof(double*) * (size_t)(max_t > 0 ? max_t : 1));
    const double** vp = (const double**)malloc(sizeof(double*) * (size_t)(max_t > 0 ? max_t : 1));
#pragma omp for schedule(dynamic, 4)
    for (long idx = 0; idx < total; ++idx) {
      const int h = (int)(idx % heads);
      const int i = (int)(idx / heads);
      const int kh = kv_head_of(h, heads, kv_heads);
      const int row = rows ? rows[i] : 0;
      const long pos = positions[i];
      int nk = 0;
      for (long t = 0; row >= 0 && row < table_rows && t < max_t; ++t) {
        if (!(t <= pos) || !in_window(pos, t, window)) continue;
#if ORC_MUTATE == 12
        long page = table[(size_t)row * pages + t / page_size];
        long off = page_size - 1 - t % page_size;
#else
        long page = table[(size_t)row * pages + t / page_size];
        long off = t % page_size;
#endif
        if (page < 0 || page >= num_pages) continue;
        kp[nk] = pool_k + (((size_t)page * kv_heads + kh) * page_size + off) * D;
        vp[nk] = pool_v + (((size_t)page * kv_heads + kh) * page_size + off) * D;
        ++nk;
      }
      attend(D, q + ((size_t)i * heads + h) * D, nk, kp, vp, scale, sinks != NULL,
             sinks ? sinks[h] : 0.0, out + ((size_t)i * heads + h) * D);
    }
    free(kp);
    free(vp);
  }
}

/* ------------------------------------------------------------------------ */
/* std.nn.linear::Linear<In, Out, T> `forward` [L, N1]: param weight         */
/* [Out, In], optional param bias [Out]; y[t, o] = sum_i x[t, i] * w[o, i]  */
/* (+ b[o]) for every leading index t, a Tensor of T. Reading: the sum is   */
/* exact (fp64 here), the bias added, and the result rounded once to T.     */
/* q_proj / k_proj / v_proj of GroupedQueryAttention are three such          */
/* modules applied to the same x. x [n, in]; w [out, in]; b [out] or NULL.  */
/* ------------------------------------------------------------------------ */
void orc_linear(int n, int in, int out_f, const double* x, const double* w, const double* b,
                int dtype, double* y) {
#pragma omp parallel for schedule(static)
  for (long idx = 0; idx < (long)n * out_f; ++idx) {
    const long t = idx / out_f;
    const int o = (int)(idx % out_f);
    double acc = 0.0;
    for (int i = 0; i < in; ++i) {
#if ORC_MUTATE == 13
      acc += x[t * in + i] * w[(size_t)i * out_f + o % in];
#else
      acc += x[t * in + i] * w[(size_t)o * in + i];
#endif
    }
    if (b) acc += b[o];
    y[idx] = dtype == ORC_DT_NONE ? acc : orc_round(acc, dtype);
  }
}

/* ------------------------------------------------------------------------ */
/* Log-sum-exp of `packed<P>` [L, N1]: per query token i and head h, the     */
/* natural log of sum_j exp(scale * <q_i, k_j>) over the keys own[i, j]      */
/* keeps (the softmax denominator at reference 0); -inf for an empty set.    */
/* A training step's backward pass reads it instead of recomputing it.      */
/* lse: [P, Heads].                                                          */
/* ------------------------------------------------------------------------ */
void orc_packed_lse(int P, int heads, int kv_heads, int D, const double* q, const double* k,
                    const int32_t* positions, const int32_t* segments, double scale, int window,
                    double* lse) {
#pragma omp parallel for schedule(dynamic, 4)
  for (long idx = 0; idx < (long)P * heads; ++idx) {
    const int h = (int)(idx % heads);
    const int i = (int)(idx / heads);
    const int kh = kv_head_of(h, heads, kv_heads);
    double m = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
      double z = 0.0;
      for (int j = 0; j < P; ++j) {
        if (!(segments[i] == segments[j] && positions[j] <= positions[i]) ||
            !in_window(positions[i], positions[j], window))
          continue;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[((size_t)i * heads + h) * D + d] * k[((size_t)j * kv_heads + kh) * D + d];
        const double sj = scale * dot;
        if (pass == 0) {
          if (sj > m) m = sj;
        } else {
          z += exp(sj - m);
        }
      }
      if (pass == 1) lse[idx] = m == -INFINITY ? -INFINITY : m + log(z);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Backward of `packed<P>` (no sinks): the gradients of                     */
/* L = sum_{i,h,d} dout[i,h,d] * out[i,h,d] with respect to q, k and v,     */
/* where out[i,h] = sum_j p_ij v_j, p_ij = exp(s_ij - lse_ih),              */
/* s_ij = scale <q_ih, k_j> over the keys own[i, j] keeps. The chain rule    */
/* through the softmax gives, with dp_ij = <dout_ih, v_j> and               */
/* delta_ih = sum_j p_ij dp_ij:                                             */
/*   dv_j += p_ij dout_ih,  ds_ij = p_ij (dp_ij - delta_ih),                */
/*   dq_ih += scale sum_j ds_ij k_j,  dk_j += scale ds_ij q_ih;              */
/* a KV head's dk, dv sum over the query heads that read it (the repeat of  */
/* grouped-query attention). One thread per KV head, so the sums never race. */
/* q, dout, dq: [P, Heads, D]; k, v, dk, dv: [P, KvHeads, D].               */
/* ------------------------------------------------------------------------ */
void orc_packed_backward(int P, int heads, int kv_heads, int D, const double* q, const double* k,
                         const double* v, const double* dout, const int32_t* positions,
                         const int32_t* segments, double scale, int window, double* dq,
                         double* dk, double* dv) {
  for (long x = 0; x < (long)P * heads * D; ++x) dq[x] = 0.0;
  for (long x = 0; x < (long)P * kv_heads * D; ++x) {
    dk[x] = 0.0;
    dv[x] = 0.0;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int kh = 0; kh < kv_heads; ++kh) {
    double* s = (double*)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
    int* js = (int*)malloc(sizeof(int) * (size_t)(P > 0 ? P : 1));
    for (int h = 0; h < heads; ++h) {
      if (kv_head_of(h, heads, kv_heads) != kh) continue;
      for (int i = 0; i < P; ++i) {
        const double* qi = q + ((size_t)i * heads + h) * D;
        const double* gi = dout + ((size_t)i * heads + h) * D;
        int nk = 0;
        double m = -INFINITY;
        for (int j = 0; j < P; ++j) {
          if (!(segments[i] == segments[j] && positions[j] <= positions[i]) ||
              !in_window(positions[i], positions[j], window))
            continue;
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += qi[d] * k[((size_t)j * kv_heads + kh) * D + d];
          js[nk] = j;
          s[nk] = scale * dot;
          if (s[nk] > m) m = s[nk];
          ++nk;
        }
        if (nk == 0) continue;
        double z = 0.0;
        for (int t = 0; t < nk; ++t) {
          s[t] = exp(s[t] - m);
          z += s[t];
        }
        double delta = 0.0;
        for (int t = 0; t < nk; ++t) {
          s[t] /= z; /* p_ij */
          const double* vj = v + ((size_t)js[t] * kv_heads + kh) * D;
          double g = 0.0;
          for (int d = 0; d < D; ++d) g += gi[d] * vj[d];
          dp[t] = g;
          delta += s[t] * g;
        }
        for (int t = 0; t < nk; ++t) {
          const int j = js[t];
#if ORC_MUTATE == 14
          const double ds = s[t] * dp[t];
#else
          const double ds = s[t] * (dp[t] - delta);
#endif
          double* dkj = dk + ((size_t)j * kv_heads + kh) * D;
          double* dvj = dv + ((size_t)j * kv_heads + kh) * D;
          const double* kj = k + ((size_t)j * kv_heads + kh) * D;
          double* dqi = dq + ((size_t)i * heads + h) * D;
          for (int d = 0; d < D; ++d) {
            dvj[d] += s[t] * gi[d];
            dkj[d] += scale * ds * qi[d];
            dqi[d] += scale * ds * kj[d];
          }
        }
      }
    }
    free(s);
    free(dp);
    free(js);
  }
}

/* Threads OpenMP will use for the calls above. */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the calls that follow (timing only; results do not depend on
 * it: every parallel loop writes disjoint outputs). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_mutation(void) { return ORC_MUTATE; }
