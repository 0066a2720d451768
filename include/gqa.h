/*
 * gqa.h -- C ABI of the MI355X (gfx950) grouped-query attention library.
 *
 * The library computes grouped-query causal attention with rotary positions
 * over a KV cache, as the GroupedQueryAttention block of the Linnet
 * "examples/01-llama" page defines it (src/attention.linnet: `forward`,
 * `packed`, `decode`; src/rope.linnet: `tables`), with the serving entries of
 * the Nest llama-3.1-8b-instruct card (decode_rows, prefill_slots,
 * prefill_packed, decode_paged, prefill_paged; PageSize = 64) and the
 * sliding-window / sink-logit variant of the Nest gpt-oss-20b card
 * (SinkAttention: `window: i32`, `param sinks: Tensor[Heads; T]`).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every buffer pointer is a DEVICE pointer owned by the caller. The library
 *   keeps no pointer after a call returns, allocates no memory, holds no
 *   per-call state and never synchronizes: work is enqueued on `stream` (a
 *   hipStream_t; NULL is the default stream) and the call returns.
 * - dtype (T): GQA_BF16 or GQA_F32. q, k, v, caches, out, sinks and the rotary
 *   table all have type T. Scores, softmax statistics and accumulators are
 *   f32 on the device.
 * - Layouts are row-major, token-major for activations: q [n, heads, D],
 *   k/v [n, kv_heads, D] (the [B, S, N*D] layout before split_heads' permute).
 *   Contiguous cache: [batch, kv_heads, max_seq, D] (state cache_k/cache_v).
 *   Paged pool: [num_pages, kv_heads, GQA_PAGE_SIZE, D] for K and for V; a
 *   page table [rows, pages] of int32 page ids maps logical position t of row
 *   r to page table[r, t / 64], offset t % 64.
 * - GQA: query head h reads KV head floor(h / (heads / kv_heads)).
 * - scale: 0 selects rsqrt(f32(D)) (the pages' rsqrt(cast<f32>(H / Heads)));
 *   otherwise the given value (finite, > 0) multiplies q.k; a negative or
 *   non-finite scale is GQA_ERR_INVALID_ARG.
 * - window: 0 is no window; W > 0 keeps key position p_k for query position
 *   p_q iff 0 <= p_q - p_k < W (W keys including the query's own).
 * - sinks: NULL, or [heads] of T; exp(sinks[h]) is added to head h's softmax
 *   denominator (a logit with no value vector, not multiplied by the scale).
 * - A query with no allowed key produces 0.
 * - Errors: every call validates its arguments on the host before enqueuing
 *   anything and returns a GQA_ERR_* code without touching device memory if
 *   they are invalid (the block's `where` clause: heads > 0, kv_heads > 0,
 *   heads % kv_heads == 0, D even; here also D in {64, 128}). n == 0 is
 *   GQA_OK and enqueues nothing. A HIP launch failure returns GQA_ERR_HIP.
 *   Index values held in device memory (positions, rows, slots, table
 *   entries, segments) are not checked on the host; the kernels give every
 *   value a defined, memory-safe meaning, stated per entry point below.
 * - Checked mode (gqa_set_checked(1), or GQA_CHECK set to anything but "0"
 *   in the environment when a thread starts): before enqueuing its kernels,
 *   a call validates its index arguments on the device -- cache rows,
 *   positions (against the cache capacity and the rotary table), slots, and
 *   the page-table entries of the pages it reads or writes -- and returns
 *   GQA_ERR_INDEX, enqueuing nothing else, if any is out of range. The check
 *   waits for `stream` (checked mode synchronizes; it is for debugging) and
 *   calls in checked mode on one device take turns. Packed prefill (and its
 *   training pair) have no index constraints: any positions and segment ids
 *   are meaningful.
 * - Determinism: identical inputs give bitwise identical outputs (no float
 *   atomics; the split schedule depends only on the shapes).
 * - Thread safety: calls may be made from any host thread.
 * - Dry run: after gqa_set_dry_run(1), calls made by the same host thread
 *   validate and return without any HIP call (for hosts without a GPU).
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GQA_OK 0
#define GQA_ERR_INVALID_ARG 1 /* null pointer, negative size, violated where clause */
#define GQA_ERR_UNSUPPORTED 2 /* valid, but this dtype / head dim / op is not built */
#define GQA_ERR_WORKSPACE 3   /* workspace missing or smaller than required */
#define GQA_ERR_HIP 4         /* a HIP runtime call or kernel launch failed */
#define GQA_ERR_INDEX 5       /* checked mode: an index argument is out of range */

/* Element types. */
#define GQA_BF16 0
#define GQA_F32 1

/* Cache kinds of gqa_rope_write_kv. */
#define GQA_CACHE_NONE 0        /* rotate only */
#define GQA_CACHE_CONTIGUOUS 1  /* [batch, kv_heads, max_seq, D] */
#define GQA_CACHE_PAGED_TABLE 2 /* pool + page table, logical positions */
#define GQA_CACHE_PAGED_SLOTS 3 /* pool + physical slots */

/* PageSize generic of the GroupedQueryAttention block. */
#define GQA_PAGE_SIZE 64

/*
 * gqa_rope_table -- the rotary tables of the Linnet "examples/01-llama" page,
 * src/rope.linnet, `tables` (with THETA): per pair index i < D/2 an inverse
 * frequency theta^(-2i/D), evaluated in f32 as i -> f32, times 2, divided by
 * f32(D), negated, times f32(log(f32(theta))), exp; the angle at position s
 * is the f32 product f32(s) * inv_freq[i]; table[0, s, i] holds its cosine
 * and table[1, s, i] its sine, in f32 and then rounded to T.
 * Each f32 step is the correctly rounded f32 result (evaluated in fp64 on the
 * device and rounded), cos/sin rounded to f32 and then to T, nearest-even.
 * The page's [S, D] tables repeat every frequency in both halves of the head
 * dimension; only the first half is stored: table is [2, max_pos, D/2] of T.
 *   head_dim: D (64 or 128); max_pos: S > 0; theta > 0.
 */
int gqa_rope_table(int32_t head_dim, int32_t max_pos, float theta, int32_t dtype,
                   void* table, void* stream);

/*
 * gqa_rope_write_kv -- rope on q and k at each token's position, then the KV
 * write (`decode`: rope(q), rope(k), write_at(cache_k, k, pos),
 * write_at(cache_v, v, pos); prefill_slots / prefill_packed / prefill_paged /
 * decode_paged do the same at rows / slots / table pages).
 *   n tokens; q [n, heads, D] and k [n, kv_heads, D] are rotated IN PLACE
 *   (q may be NULL: not rotated; k may be NULL only when rope_table is NULL
 *   or cache_kind is NONE and there is nothing to rotate).
 *   Rotation (rotate-half on the pairs (i, i + D/2)) at position
 *   positions[t] with the table of gqa_rope_table:
 *     y_lo = x_lo * c - x_hi * s,  y_hi = x_hi * c + x_lo * s,
 *   evaluated exactly and rounded once to T (nearest-even). A position
 *   outside [0, rope_max_pos) reads the nearest table row.
 *   rope_table == NULL: no rotation (learned positions, as in GPT-2).
 *   v [n, kv_heads, D] is copied bit for bit into cache_v (NULL: K only).
 *   cache_kind selects the write target of token t:
 *     NONE          nothing written.
 *     CONTIGUOUS    cache[r, :, positions[t], :] with r = rows[t] (rows NULL:
 *                   0); cache_dim0 = batch, cache_seq = max_seq.
 *     PAGED_TABLE   logical position positions[t] of table row r = rows[t]
 *                   (NULL: 0): page table[r, pos / 64], offset pos % 64;
 *                   cache_dim0 = num_pages, cache_seq = 64; table is
 *                   [table_rows, table_pages].
 *     PAGED_SLOTS   physical slot slots[t] = page * 64 + offset;
 *                   cache_dim0 = num_pages, cache_seq = 64.
 *   A target outside the cache (row, position, slot or page id out of range)
 *   drops that token's write: write_at is a masked select. Two tokens with
 *   the same target race (one of them lands).
 */
int gqa_rope_write_kv(int32_t n, int32_t heads, int32_t kv_heads, int32_t head_dim,
                      int32_t dtype, void* q, void* k, const void* v,
                      const int32_t* positions, const void* rope_table, int32_t rope_max_pos,
                      int32_t cache_kind, void* cache_k, void* cache_v, int32_t cache_dim0,
                      int32_t cache_seq, const int32_t* rows, const int32_t* slots,
                      const int32_t* table, int32_t table_rows, int32_t table_pages,
                      void* stream);

/*
 * gqa_qkv_rope_write -- the q / k / v projections of GroupedQueryAttention
 * (Linnet "examples/01-llama" page, src/attention.linnet `forward` /
 * `decode`: q_proj, k_proj, v_proj are std.nn.linear::Linear, y = x W^T + b
 * as a Tensor of T) fused with the rotation and the cache write of
 * gqa_rope_write_kv: q = rope(q_proj(x)), k = rope(k_proj(x)), v = v_proj(x),
 * each projection rounded to T before the rotation, the rotation exact and
 * rounded once to T.
 *   x [n, hidden]; w_q [heads*D, hidden], w_k and w_v [kv_heads*D, hidden]
 *   (the modules' `weight` layout [Out, In]); b_q [heads*D], b_k, b_v
 *   [kv_heads*D] or NULL (no bias). q_out [n, heads, D] (required); k_out,
 *   v_out [n, kv_heads, D] or NULL. positions [n], rope_table / rope_max_pos
 *   and the cache arguments as gqa_rope_write_kv (rope_table NULL: no
 *   rotation; cache_kind NONE: no cache write).
 *   Built for T = bf16, D in {64, 128}, hidden % 64 == 0 and
 *   (heads + 2 kv_heads) * D % 128 == 0 (else GQA_ERR_UNSUPPORTED). The
 *   projection sums run in f32 on the matrix cores, so a result that lies
 *   within an f32 rounding of a bf16 rounding boundary may round the other way
 *   than the exact sum would.
 */
int gqa_qkv_rope_write(int32_t n, int32_t hidden, int32_t heads, int32_t kv_heads,
                       int32_t head_dim, int32_t dtype, const void* x, const void* w_q,
                       const void* w_k, const void* w_v, const void* b_q, const void* b_k,
                       const void* b_v, const int32_t* positions, const void* rope_table,
                       int32_t rope_max_pos, void* q_out, void* k_out, void* v_out,
                       int32_t cache_kind, void* cache_k, void* cache_v, int32_t cache_dim0,
                       int32_t cache_seq, const int32_t* rows, const int32_t* slots,
                       const int32_t* table, int32_t table_rows, int32_t table_pages,
                       void* stream);

/*
 * gqa_prefill_packed -- attention of `packed<P>` / prefill_packed: token i
 * attends key j iff segments[i] == segments[j] && positions[j] <=
 * positions[i] (the `own` mask, literal: any segment ids, any order) and the
 * window keeps it; grouped_attention then softmax-weights v.
 *   q [p, heads, D] and k, v [p, kv_heads, D] already rotated (see
 *   gqa_rope_write_kv); out [p, heads, D] of T.
 *   Built for T = bf16, D in {64, 128} and p * kv_heads * D * 2 + 4096 <
 *   2^31 (else GQA_ERR_UNSUPPORTED); bf16 matrix cores, f32 softmax.
 *   workspace: device memory of at least gqa_prefill_packed_workspace(...)
 *   bytes (tile summaries, the per-query-tile visit lists -- about
 *   ceil(p / 32) * ceil(p / 64) * 4 bytes -- and the schedule), 256-byte
 *   aligned.
 */
int gqa_prefill_packed(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                       int32_t dtype, float scale, int32_t window, const void* sinks,
                       const void* q, const void* k, const void* v,
                       const int32_t* positions, const int32_t* segments, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

size_t gqa_prefill_packed_workspace(int32_t p, int32_t heads, int32_t kv_heads,
                                    int32_t head_dim);

/*
 * gqa_prefill_packed_plan / gqa_prefill_packed_planned -- gqa_prefill_packed
 * in two calls. Which key tiles each query tile visits follows from the
 * `own` mask of `packed<P>` (the Linnet "examples/01-llama" page,
 * src/attention.linnet `packed`) alone, i.e. from positions, segments and the
 * window, which every layer of a model shares; so the plan can be built
 * once per batch, or on another stream while earlier work runs.
 *   gqa_prefill_packed_plan writes the plan (tile summaries, visit lists,
 *   costliest-first schedule) into the workspace (at least
 *   gqa_prefill_packed_workspace(p, heads, kv_heads, head_dim) bytes,
 *   256-byte aligned). It reads positions and segments [p] only.
 *   gqa_prefill_packed_planned takes the arguments of gqa_prefill_packed and
 *   only reads the workspace: it computes the same out, bit for bit, as
 *   gqa_prefill_packed, provided the workspace holds a plan built for the
 *   same p, heads, kv_heads, head_dim, window and the same positions and
 *   segments contents, and that build has finished on the device (same
 *   stream, or an event between streams). Any number of planned calls, on
 *   any q, k, v, may share one plan; nothing checks that a plan matches.
 *   Errors as gqa_prefill_packed (positions, segments, workspace checked by
 *   both calls; q, k, v, out by the planned call).
 */
int gqa_prefill_packed_plan(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                            int32_t window, const int32_t* positions, const int32_t* segments,
                            void* workspace, size_t workspace_bytes, void* stream);
int gqa_prefill_packed_planned(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                               int32_t dtype, float scale, int32_t window, const void* sinks,
                               const void* q, const void* k, const void* v,
                               const int32_t* positions, const int32_t* segments, void* out,
                               const void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_prefill_packed_lse -- gqa_prefill_packed for training: the same
 * attention (no sinks), and also each (token, head)'s natural-log softmax
 * denominator lse = ln sum_j exp(scale <q_i, k_j>) over the keys the `own`
 * mask and the window keep (-inf when there are none), which the backward
 * reads. The training entry `loss_packed` of the Linnet "examples/01-llama"
 * page's model differentiates through this attention.
 *   lse: [p, heads] f32 device memory (written); other arguments, the
 *   workspace and errors as gqa_prefill_packed.
 */
int gqa_prefill_packed_lse(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                           int32_t dtype, float scale, int32_t window, const void* q,
                           const void* k, const void* v, const int32_t* positions,
                           const int32_t* segments, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * gqa_prefill_packed_backward -- gradients of sum(dout * out) for the packed
 * attention (gqa_prefill_packed_lse, no sinks): with p_ij = exp(s_ij -
 * lse_i), s_ij = scale <q_i, k_j> over the kept keys, dp_ij = <dout_i, v_j>
 * and delta_i = <dout_i, out_i>:
 *   dv_j = sum_i p_ij dout_i, ds_ij = p_ij (dp_ij - delta_i),
 *   dq_i = scale sum_j ds_ij k_j, dk_j = scale sum_i ds_ij q_i,
 * a KV head's dk, dv summed over the query heads that read it.
 *   q, out, dout, dq [p, heads, D]; k, v, dk, dv [p, kv_heads, D] of T;
 *   lse [p, heads] f32 as written by gqa_prefill_packed_lse on the same
 *   q, k, v, positions, segments, scale and window; dq, dk, dv are written
 *   (every entry; keys no query attends get 0). Built for T = bf16, D in
 *   {64, 128}; bf16 matrix cores with f32 accumulation, one rounding to bf16.
 *   workspace: at least gqa_prefill_packed_backward_workspace(...) bytes,
 *   256-byte aligned. Errors as gqa_prefill_packed.
 */
int gqa_prefill_packed_backward(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                int32_t dtype, float scale, int32_t window, const void* q,
                                const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const int32_t* positions,
                                const int32_t* segments, void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, void* stream);

size_t gqa_prefill_packed_backward_workspace(int32_t p, int32_t heads, int32_t kv_heads,
                                             int32_t head_dim);

/*
 * gqa_prefill_cached -- chunked prefill over a cached prefix: the attention
 * of `prefill<S>(x, pos)` with pos > 0 (contiguous cache) and of
 * `prefill_paged` (paged pool) of the GroupedQueryAttention block, llama-
 * 3.1-8b-instruct card, serving signatures. Those pages give signatures
 * only; the reading taken: token i, whose k and v were already written into
 * its cache row by gqa_rope_write_kv (call it first, on the same stream),
 * attends key slot s of cache row rows[i] iff s <= positions[i] and the
 * window keeps it -- the prefix written by earlier calls included.
 *   cache_kind GQA_CACHE_CONTIGUOUS: cache_k, cache_v [cache_dim0 = batch,
 *     kv_heads, cache_seq = max_seq, D]; rows[i] is the batch row.
 *   cache_kind GQA_CACHE_PAGED_TABLE: pool_k, pool_v [cache_dim0 =
 *     num_pages, kv_heads, cache_seq = 64, D]; logical slot s of table row
 *     r is page table[r, s / 64], offset s % 64 (table [table_rows,
 *     table_pages]); rows[i] is the table row.
 *   q, out [n, heads, D] of T (q already rotated); rows, positions [n]
 *   (rows NULL: every token reads row 0). A row outside the cache / table
 *   gives no keys (output 0); keys on page ids outside [0, num_pages)
 *   contribute nothing. Built for T = bf16, D in {64, 128}. Tokens of one
 *   row kept contiguous in n order make the query tiles single-row (fast).
 *   workspace: at least gqa_prefill_cached_workspace(n, ...) bytes,
 *   256-byte aligned. Errors as gqa_prefill_packed.
 */
int gqa_prefill_cached(int32_t n, int32_t heads, int32_t kv_heads, int32_t head_dim,
                       int32_t dtype, float scale, int32_t window, const void* sinks,
                       const void* q, const int32_t* rows, const int32_t* positions,
                       int32_t cache_kind, const void* cache_k, const void* cache_v,
                       int32_t cache_dim0, int32_t cache_seq, const int32_t* table,
                       int32_t table_rows, int32_t table_pages, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

size_t gqa_prefill_cached_workspace(int32_t n, int32_t heads, int32_t kv_heads,
                                    int32_t head_dim);

/*
 * gqa_decode_rows -- `decode` / decode_rows: row b's query attends every slot
 * s of its cache row with s <= positions[b] (seen = iota(MaxSeq) <= pos) and
 * inside the window; slots past positions[b] are never read. A position at or
 * past max_seq attends the whole row; a negative position attends nothing.
 *   q [batch, heads, D]; cache_k, cache_v [batch, kv_heads, max_seq, D];
 *   positions [batch]; out [batch, heads, D].
 *   The query's own key must already be in the cache (gqa_rope_write_kv
 *   enqueued before on the same stream).
 *   workspace: at least gqa_decode_rows_workspace(...) bytes (split partials).
 */
int gqa_decode_rows(int32_t batch, int32_t heads, int32_t kv_heads, int32_t head_dim,
                    int32_t dtype, float scale, int32_t window, const void* sinks,
                    const void* q, const void* cache_k, const void* cache_v, int32_t max_seq,
                    const int32_t* positions, void* out, void* workspace,
                    size_t workspace_bytes, void* stream);

size_t gqa_decode_rows_workspace(int32_t batch, int32_t heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t max_seq);

/*
 * gqa_decode_paged -- decode_paged<Rows, Pages>: row r's logical key t,
 * 0 <= t < pages * 64, is attended iff t <= positions[r] and the window keeps
 * it; it lives at page table[r, t / 64], offset t % 64 of the pool. A page id
 * outside [0, num_pages) contributes no keys (its entries are never used to
 * address memory), so tables may carry -1 past a row's last page.
 *   q [rows, heads, D]; pool_k, pool_v [num_pages, kv_heads, 64, D];
 *   positions [rows]; table [rows, pages]; out [rows, heads, D].
 *   workspace: at least gqa_decode_paged_workspace(...) bytes.
 */
int gqa_decode_paged(int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                     int32_t head_dim, int32_t dtype, float scale, int32_t window,
                     const void* sinks, const void* q, const void* pool_k, const void* pool_v,
                     int32_t num_pages, const int32_t* positions, const int32_t* table,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);

size_t gqa_decode_paged_workspace(int32_t rows, int32_t pages, int32_t heads,
                                  int32_t kv_heads, int32_t head_dim);

/*
 * gqa_decode_paged_noalloc -- gqa_decode_paged for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments (no workspace) and the
 * same results, bit for bit, as gqa_decode_paged. The split partials live
 * in a device array the library holds, GQA_DECODE_SCRATCH_BYTES per GPU,
 * until the process ends; the call allocates and frees nothing. A call whose
 * partials would exceed that array returns GQA_ERR_WORKSPACE before touching
 * the device. The split rules keep every call far below it: a row is split
 * only while the grid has fewer than 512 workgroups (bf16 on matrix cores) or
 * 1024 (the vector-ALU kernel), so at most 16384 (query head, split) partials
 * of D + 2 floats (8.5 MB) are written, and none when each row takes one
 * split. Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialized by the caller. The array needs
 * no clearing: a call reads only partials it wrote itself. Checked mode does
 * not apply to this entry.
 */
#define GQA_DECODE_SCRATCH_BYTES (16u << 20)
int gqa_decode_paged_noalloc(int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                             int32_t head_dim, int32_t dtype, float scale, int32_t window,
                             const void* sinks, const void* q, const void* pool_k,
                             const void* pool_v, int32_t num_pages, const int32_t* positions,
                             const int32_t* table, void* out, void* stream);

/*
 * gqa_step_packed -- `step_packed<P>` of GroupedQueryAttention (llama-
 * 3.1-8b-instruct card) and SinkAttention (gpt-oss-20b card, with the
 * window): one call over `batch` decode tokens and `p` packed prefill
 * tokens, in the order of the pages' x: [1, Batch + P, H] -- the decode
 * tokens first. Signature only on the pages; the reading taken: decode token
 * b attends slots <= step_positions[b] of contiguous cache row b (as
 * gqa_decode_rows), the packed tokens attend each other under `own` (as
 * gqa_prefill_packed). Every token's k/v are written first by
 * gqa_rope_write_kv.
 *   q, out [batch + p, heads, D] of T; k, v [p, kv_heads, D] (the packed
 *   tokens, rotated); positions, segments [p]; cache_k, cache_v [batch,
 *   kv_heads, max_seq, D]; step_positions [batch]. bf16 only.
 *   workspace: gqa_step_packed_workspace(...) bytes, 256-byte aligned.
 * Both parts are validated before either is enqueued; statuses as the two
 * entries above.
 */
int gqa_step_packed(int32_t batch, int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                    int32_t dtype, float scale, int32_t window, const void* sinks, const void* q,
                    const void* k, const void* v, const int32_t* positions,
                    const int32_t* segments, const void* cache_k, const void* cache_v,
                    int32_t max_seq, const int32_t* step_positions, void* out, void* workspace,
                    size_t workspace_bytes, void* stream);

size_t gqa_step_packed_workspace(int32_t batch, int32_t p, int32_t heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t max_seq);

/*
 * gqa_step_paged -- `step_paged<P, Rows, Pages>` (llama-3.1-8b-instruct
 * card): `p` chunk tokens then one decode token for each of `rows` table
 * rows, in the order of the pages' x: [1, P + Rows, H]. Signature only; the
 * reading taken: chunk token i attends the paged row token_rows[i] at slots
 * <= positions[i], prefix included (as gqa_prefill_cached, PAGED_TABLE);
 * decode token r attends table row r at slots <= step_positions[r] (as
 * gqa_decode_paged). Every token's k/v are written first (gqa_rope_write_kv
 * with PAGED_SLOTS or PAGED_TABLE).
 *   q, out [p + rows, heads, D] of T; token_rows, positions [p]; pools
 *   [num_pages, kv_heads, 64, D]; table [rows, pages]; step_positions
 *   [rows]. bf16 only. workspace: gqa_step_paged_workspace(...) bytes,
 *   256-byte aligned.
 * With up to 16 query heads per KV head the decode tokens and the chunk run
 * as one grid (decode workgroups after the first half of the prefill tiles),
 * so the decode's cache reads overlap the chunk's matrix work; otherwise the
 * decode runs first, then the chunk.
 */
int gqa_step_paged(int32_t p, int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                   int32_t head_dim, int32_t dtype, float scale, int32_t window, const void* sinks,
                   const void* q, const int32_t* token_rows, const int32_t* positions,
                   const void* pool_k, const void* pool_v, int32_t num_pages,
                   const int32_t* table, const int32_t* step_positions, void* out,
                   void* workspace, size_t workspace_bytes, void* stream);

size_t gqa_step_paged_workspace(int32_t p, int32_t rows, int32_t pages, int32_t heads,
                                int32_t kv_heads, int32_t head_dim);

/* Human-readable name of a status code (static storage); gqa_status_str is
 * the same function. */
const char* gqa_status_string(int32_t status);
const char* gqa_status_str(int32_t status);

/*
 * gqa_workspace_bytes -- the workspace query of an operation, one entry for
 * all of them (the per-operation *_workspace functions above give the same
 * numbers). n_tokens: p (packed / backward / step prefill tokens) or n
 * (cached prefill); n_rows: decode rows (batch); max_len: max_seq
 * (contiguous decode, step_packed) or pages per table row (paged decode,
 * step_paged). Arguments an operation does not use are ignored; an unknown
 * op returns 0.
 */
#define GQA_OP_PREFILL_PACKED 0
#define GQA_OP_PREFILL_CACHED 1
#define GQA_OP_PREFILL_BACKWARD 2
#define GQA_OP_DECODE_ROWS 3
#define GQA_OP_DECODE_PAGED 4
#define GQA_OP_STEP_PACKED 5
#define GQA_OP_STEP_PAGED 6
size_t gqa_workspace_bytes(int32_t op, int32_t heads, int32_t kv_heads, int32_t head_dim,
                           int32_t n_tokens, int32_t n_rows, int32_t max_len);

/* Dry-run switch of the calling host thread; returns the previous setting. */
int32_t gqa_set_dry_run(int32_t on);

/* Checked-mode switch of the calling host thread (see the conventions
 * above); returns the previous setting. */
int32_t gqa_set_checked(int32_t on);

/* ABI version of this header. */
int32_t gqa_abi_version(void);

/*
 * gqa_diag_stream_read -- a diagnostic outside the attention path: reads
 * `bytes` of device memory at `buffer` once, in a streaming pattern
 * (nontemporal 16-byte loads, a grid-stride loop over at most
 * GQA_DIAG_READ_BLOCKS workgroups). Workgroup b stores the XOR of the 32-bit
 * words it read to out[b] (device memory, GQA_DIAG_READ_BLOCKS words; words
 * of workgroups not launched are left as they are, so a caller that zeroes
 * `out` first gets the XOR of the whole buffer by XOR-ing the words).
 * bench.py times it as the measured HBM read ceiling the decode is compared
 * with. buffer 16-byte aligned, bytes a multiple of 16 (else
 * GQA_ERR_INVALID_ARG); enqueued on `stream`, nothing allocated.
 */
#define GQA_DIAG_READ_BLOCKS 2048
int gqa_diag_stream_read(const void* buffer, size_t bytes, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
