// Packed prefill attention on bf16 matrix cores (gfx950).
//
// `packed<P>` of the Linnet "examples/01-llama" page (src/attention.linnet)
// lets token i attend key j iff own[i, j] = segments[i] == segments[j] &&
// positions[j] <= positions[i]; prefill_packed of the Nest
// llama-3.1-8b-instruct card uses the same mask, and SinkAttention of the
// Nest gpt-oss-20b card adds a window and a per-head sink logit.
//
// Design (flash-style, one pass over the keys, online softmax):
// * A workgroup owns one KV head and a tile of queries: 4 wavefronts, each
//   with 32 query tokens of one query head. With G = Heads / KvHeads >= 4 the
//   four waves are four query heads of the group over the same 32 tokens, so
//   every K/V tile staged in LDS serves four heads.
// * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//   K rows (keys) are the A operand read from LDS, Q^T the B operand held in
//   registers. In the 32x32 accumulator layout a lane owns one query column,
//   so the softmax max/sum of a query needs one cross-lane exchange (lanes l
//   and l ^ 32) per tile.
// * The key order inside a 32-key block is permuted (bits 2 and 3 of the row
//   index swapped) so that the probabilities a lane holds after the softmax
//   are exactly the B operand of the P.V product O^T = V^T P^T; no data moves
//   between lanes. V stays key-major in LDS (16-byte chunks XOR-swizzled) and
//   the A operand V^T is read with transposing 8-byte LDS reads.
// * K/V tiles of 64 keys go from memory straight into LDS (buffer loads with
//   an LDS destination, no registers), issued one tile ahead and spread over
//   the matrix steps; V is loaded one tile behind K, because a slot runs the
//   S^T of one tile next to the P.V of the previous one.
// * Tiles that cannot hold an allowed key are skipped using per-tile
//   [min, max] summaries of segments and positions; tiles in which every pair
//   is allowed skip the per-element mask, and tiles whose keys and queries all
//   lie in one segment test positions only. The exact `own` predicate is
//   evaluated everywhere else, so any segment order or id is handled.
// * Three small prep kernels compute the per-tile summaries and each query
//   tile's visited key-tile range and cost (one wavefront per tile), then
//   order the query tiles costliest first (a counting sort); workgroup index i * n_groups + g maps KV head g to the
//   round-robin XCD g % 8, keeping one head's K/V in one XCD's L2.
#include <mutex>
#include <type_traits>
#include <utility>

#include "attn_tiles.h"
#include "common.h"
#include "decode_mfma.h"
#include "internal.h"

namespace gqa {


// ---------------------------------------------------------------------------
// Prep 1: per-tile [min, max] of segments and positions, and the smallest
// position of the first and of the last segment. One wavefront per tile: key
// tiles (64 tokens) first, then query tiles (tq <= 128 tokens); each lane
// holds at most two tokens and the wavefront reduces with shuffles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_summarize_kernel(PrefillArgs a, Plan pl) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ti = blockIdx.x * 4 + wave;
  if (ti >= pl.n_kt + pl.n_qt) return;
  const bool is_k = ti < pl.n_kt;
  const int len = is_k ? kBK : pl.tq;  // at most 128: two tokens per lane
  const int lo = is_k ? ti * kBK : (ti - pl.n_kt) * pl.tq;
  const int hi = min(a.p, lo + len);
  const int t0 = lo + lane, t1 = lo + 64 + lane;
  const bool h0 = t0 < hi, h1 = t1 < min(hi, lo + len);
  const int sg0 = h0 ? (a.segments ? a.segments[t0] : 0) : 0, ps0 = h0 ? a.positions[t0] : 0;
  const int sg1 = h1 ? (a.segments ? a.segments[t1] : 0) : 0, ps1 = h1 ? a.positions[t1] : 0;
  constexpr int kMaxI = 0x7fffffff, kMinI = (int)0x80000000;
  int smin = min(h0 ? sg0 : kMaxI, h1 ? sg1 : kMaxI), smax = max(h0 ? sg0 : kMinI, h1 ? sg1 : kMinI);
  int pmin = min(h0 ? ps0 : kMaxI, h1 ? ps1 : kMaxI), pmax = max(h0 ? ps0 : kMinI, h1 ? ps1 : kMinI);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    smin = min(smin, __shfl_xor(smin, off, 64));
    smax = max(smax, __shfl_xor(smax, off, 64));
    pmin = min(pmin, __shfl_xor(pmin, off, 64));
    pmax = max(pmax, __shfl_xor(pmax, off, 64));
  }
  // Smallest positions within the first and the last segment.
  int pfirst = min((h0 && sg0 == smin) ? ps0 : kMaxI, (h1 && sg1 == smin) ? ps1 : kMaxI);
  int plast = min((h0 && sg0 == smax) ? ps0 : kMaxI, (h1 && sg1 == smax) ? ps1 : kMaxI);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    pfirst = min(pfirst, __shfl_xor(pfirst, off, 64));
    plast = min(plast, __shfl_xor(plast, off, 64));
  }
  if (lane == 0) {
    const TileSum sum{smin, smax, pmin, pmax, pfirst, plast, 0, 0};
    if (is_k) pl.ksum[ti] = sum;
    else pl.qsum[ti - pl.n_kt] = sum;
  }
}

// ---------------------------------------------------------------------------
// Prep 2: each query tile's visited key-tile range, cost and tile masks, one
// wavefront per query tile (the lanes test 64 key tiles at a time).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_scan_kernel(PrefillArgs a, Plan pl) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int qt = blockIdx.x * 4 + wave;
  if (qt >= pl.n_qt) return;
  const TileSum q = pl.qsum[qt];
  if (a.src != kSrcPacked) {
    // Cache keys: rows [seg_min, seg_max] of the cache, key tiles from the
    // window's first slot to the last slot any query may see.
    if (lane == 0) {
      const int r_lo = max(q.seg_min, 0), r_hi = min(q.seg_max, a.cache_rows - 1);
      const int last_slot = min(q.pos_max, a.cap - 1);
      const int khi = last_slot >= 0 ? last_slot / kBK : -1;
      const int klo = a.window > 0 ? max(0, q.pos_min - a.window + 1) / kBK : 0;
      const long long c = (r_hi >= r_lo && khi >= klo) ? (long long)(r_hi - r_lo + 1) * (khi - klo + 1) : 0;
      pl.qrange[qt] = make_int2(0, -1);
      pl.cost[qt] = (int)min(c, (long long)pl.max_cost);
    }
    return;
  }
  int first = pl.n_kt, last = -1, cnt = 0, nm = 0;
  int* vis = pl.vis + (size_t)qt * pl.n_kt;
  // Whether key tile g * 64 + lane can meet this query tile, is fully
  // allowed, and lies in its one segment.
  auto classify = [&](int g, const TileSum& k, bool& meet, bool& full, bool& one) {
    const int kt = g * 64 + lane;
    meet = full = one = false;
    if (kt < pl.n_kt) {
      meet = tiles_meet(q, k, a.window);
      full = meet && tiles_full(q, k, kt, a.p, a.window);
      one = meet && tiles_oneseg(q, k, kt, a.p);
    }
  };
  // The first kScanKept groups of 64 key tiles: every summary is loaded at
  // once (one memory round trip instead of one per group and pass), and the
  // classification is kept as 3 bits per group for the second pass.
  constexpr int kScanKept = 8;
  TileSum kc[kScanKept];
#pragma unroll
  for (int g = 0; g < kScanKept; ++g)
    if (g < pl.n_kg) kc[g] = pl.ksum[min(g * 64 + lane, pl.n_kt - 1)];
  uint32_t kept = 0;
  // The visit list holds the fully allowed tiles first: count them first.
  int nf = 0;
#pragma unroll
  for (int g = 0; g < kScanKept; ++g) {
    if (g < pl.n_kg) {
      bool meet, full, one;
      classify(g, kc[g], meet, full, one);
      kept |= ((meet ? 1u : 0u) | (full ? 2u : 0u) | (one ? 4u : 0u)) << (3 * g);
      nf += __builtin_popcountll(__builtin_amdgcn_ballot_w64(full));
    }
  }
  for (int g = kScanKept; g < pl.n_kg; ++g) {
    bool meet, full, one;
    classify(g, pl.ksum[min(g * 64 + lane, pl.n_kt - 1)], meet, full, one);
    nf += __builtin_popcountll(__builtin_amdgcn_ballot_w64(full));
  }
  int rank_f = 0;
  for (int g = 0; g < pl.n_kg; ++g) {
    const int kt = g * 64 + lane;
    bool meet, full, one;
    if (g < kScanKept) {
      const uint32_t b = kept >> (3 * g);
      meet = b & 1u;
      full = b & 2u;
      one = b & 4u;
    } else {
      classify(g, pl.ksum[min(kt, pl.n_kt - 1)], meet, full, one);
    }
    if (meet) {
      first = min(first, kt);
      last = max(last, kt);
      ++cnt;
    }
    const unsigned long long vm = __builtin_amdgcn_ballot_w64(meet);
    const unsigned long long fm = __builtin_amdgcn_ballot_w64(full);
    const unsigned long long om = __builtin_amdgcn_ballot_w64(one);
    if (lane < kMaskWords) {
      const unsigned long long w = lane < 2 ? vm : lane < 4 ? fm : om;
      pl.masks[((size_t)qt * pl.n_kg + g) * kMaskWords + lane] = (uint32_t)(w >> (32 * (lane & 1)));
    }
    // Visit list in walk order: the fully allowed tiles, then the others,
    // each in increasing kt (ranks by mbcnt over the ballots).
    const unsigned long long mm = vm & ~fm;
    const int rf = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(fm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)fm, 0u));
    const int rm = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0u));
    if (full) vis[rank_f + rf] = kt;
    else if (meet) vis[nf + nm + rm] = kt | ((one ? 1 : 2) << kVisMode);
    rank_f += __builtin_popcountll(fm);
    nm += __builtin_popcountll(mm);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    first = min(first, __shfl_xor(first, off, 64));
    last = max(last, __shfl_xor(last, off, 64));
    cnt += __shfl_xor(cnt, off, 64);
  }
  if (lane == 0) {
    pl.qrange[qt] = make_int2(first, last);
    pl.cost[qt] = cnt;
    pl.nfull[qt] = nf;
  }
}

// ---------------------------------------------------------------------------
// Prep 3 (one workgroup): query tiles ordered by cost, costliest first -- a
// counting sort (histogram, scan, scatter). The order among equal costs only
// affects scheduling, never results.
// ---------------------------------------------------------------------------
constexpr int kMaxCostBins = 4096;
constexpr int kTouchMinTiles = 8;  // see touch_next in prefill_body

__global__ __launch_bounds__(kPrepThreads) void prefill_order_kernel(Plan pl) {
  __shared__ int start[kMaxCostBins + 1];
  __shared__ int part[kPrepThreads];
  __shared__ int s_order[kMaxCostBins];  // the order again, for the records (n_qt <= kMaxCostBins)
  const int tid = threadIdx.x;
  const int nb = pl.max_cost + 1;  // costs 0 .. max_cost
  static_assert(kRecInts == 16 && kRecVis == 12, "record layout");
  // Exclusive scan over the bins (bin b = cost max_cost - b, so costly tiles
  // first): each thread sums a run of bins, a block scan of the run sums,
  // then the runs are rewritten as exclusive offsets.
  auto scan_bins = [&]() {
    const int per = (nb + kPrepThreads - 1) / kPrepThreads;
    const int b0 = tid * per;
    int sum = 0;
    for (int b = b0; b < min(nb, b0 + per); ++b) sum += start[b];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kPrepThreads; off <<= 1) {
      const int v = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    int run = part[tid] - sum;
    for (int b = b0; b < min(nb, b0 + per); ++b) {
      const int c = start[b];
      start[b] = run;
      run += c;
    }
    __syncthreads();
  };
  // Start record of query tile qt at slot i: its index, for packed keys the
  // numbers of fully allowed and masked tiles it visits and its first
  // kRecVis visit-list entries (zeros past the list).
  auto write_rec = [&](int i, int qt, int nf, int n, const int* e) {
    int4* rec = reinterpret_cast<int4*>(pl.rec + (size_t)i * kRecInts);
    if (pl.vis != nullptr) {
      int f[kRecVis];
#pragma unroll
      for (int w = 0; w < kRecVis; ++w) f[w] = w < n ? e[w] : 0;
      rec[0] = make_int4(qt, nf, n - nf, 0);
      rec[1] = make_int4(f[0], f[1], f[2], f[3]);
      rec[2] = make_int4(f[4], f[5], f[6], f[7]);
      rec[3] = make_int4(f[8], f[9], f[10], f[11]);
    } else {
      rec[0] = make_int4(qt, 0, 0, 0);
      rec[1] = rec[2] = rec[3] = make_int4(0, 0, 0, 0);
    }
  };
  // The list entries of query tile qt a record needs, all loads issued before
  // any is used (indices clamped into the list).
  auto load_vis = [&](int qt, int* e) {
    const int* vis = pl.vis + (size_t)qt * pl.n_kt;
#pragma unroll
    for (int w = 0; w < kRecVis; ++w) e[w] = vis[min(w, pl.n_kt - 1)];
  };

  if (pl.n_qt <= kPrepThreads && nb <= kMaxCostBins) {
    // One query tile per thread: its cost (and what its record needs) is
    // loaded once, before the sort, and the thread writes its tile's order
    // entry and record at the tile's sorted place; nothing waits on memory
    // after the sort.
    const bool mine = tid < pl.n_qt;
    const bool recs = mine && pl.rec != nullptr && pl.vis != nullptr;
    const int c = mine ? pl.cost[tid] : 0;
    const int nf = recs ? pl.nfull[tid] : 0;
    int e[kRecVis];
#pragma unroll
    for (int w = 0; w < kRecVis; ++w) e[w] = 0;
    if (recs) load_vis(tid, e);
    for (int i = tid; i < nb; i += kPrepThreads) start[i] = 0;
    __syncthreads();
    if (mine) atomicAdd(&start[pl.max_cost - c], 1);
    __syncthreads();
    scan_bins();
    if (mine) {
      const int at = atomicAdd(&start[pl.max_cost - c], 1);
      pl.order[at] = tid;
      if (pl.rec != nullptr) write_rec(at, tid, nf, c, e);
    }
    return;
  }

  const bool keep = pl.n_qt <= kMaxCostBins;
  if (nb > kMaxCostBins) {
    for (int i = tid; i < pl.n_qt; i += kPrepThreads) {
      pl.order[i] = i;
      if (keep) s_order[i] = i;
    }
  } else {
    for (int i = tid; i < nb; i += kPrepThreads) start[i] = 0;
    __syncthreads();
    for (int i = tid; i < pl.n_qt; i += kPrepThreads) atomicAdd(&start[pl.max_cost - pl.cost[i]], 1);
    __syncthreads();
    scan_bins();
    for (int i = tid; i < pl.n_qt; i += kPrepThreads) {
      const int at = atomicAdd(&start[pl.max_cost - pl.cost[i]], 1);
      pl.order[at] = i;
      if (keep) s_order[at] = i;
    }
  }
  if (pl.rec == nullptr) return;
  // Start records: the walk's first scalar loads, in one place per slot.
  __syncthreads();
  for (int i = tid; i < pl.n_qt; i += kPrepThreads) {
    const int qt = keep ? s_order[i] : pl.order[i];
    int e[kRecVis];
    const bool packed = pl.vis != nullptr;
    const int nf = packed ? pl.nfull[qt] : 0, n = packed ? pl.cost[qt] : 0;
    if (packed) load_vis(qt, e);
    write_rec(i, qt, nf, n, e);
  }
}

// ---------------------------------------------------------------------------
// LDS layouts (byte offsets; every access below is conflict-free in the
// 64-bank, 4-byte-bank LDS of gfx950, where a 16-byte access is served 16
// lanes at a time and an 8-byte access 32 lanes at a time). Tiles are filled
// by direct buffer-to-LDS loads, which place lane l's 16 bytes at
// base + 16 l, so a layout is chosen through the global address each lane
// fetches.
//   K tile [64 rows][D], row stride 2 D + 16 bytes (D / 8 + 1 chunks of 16
//          bytes; lanes that land on a row's pad chunk fetch out of range and
//          write zeros). Row r holds key kappa(r) of the tile, so lane l
//          reads row l % 32 (+32): the 16 rows of a 16-lane group start 16
//          bytes apart modulo 256.
//   V tile [64 rows][D], row stride 2 D, 16-byte chunk c of row r stored at
//          chunk c ^ vswz(r). The P.V operand is read with transposing
//          8-byte reads: a 16-lane group covers 4 keys x 16 dimensions, and
//          with the swizzle the 4 rows x 4 chunks a 32-lane half reads fall
//          on distinct banks.
//   positions, segments: 64 x 4 bytes each per tile (packed keys).
// ---------------------------------------------------------------------------
template <int D, int NKB, int NPB>
struct Lds {
  static constexpr int kStride = 2 * D + 16;     // K row stride (bytes)
  static constexpr int kChunks = D / 8 + 1;      // 16-byte chunks per K row
  static constexpr int vStride = 2 * D;          // V row stride (bytes)
  static constexpr int kBytes = kBK * kStride;   // one K tile = kChunks KiB
  static constexpr int vBytes = kBK * vStride;   // one V tile = D / 8 KiB
  static constexpr int kOff(int buf) { return buf * kBytes; }
  static constexpr int vOff(int buf) { return NKB * kBytes + buf * vBytes; }
  static constexpr int posOff(int buf) { return NKB * (kBytes + vBytes) + buf * 2 * kBK * 4; }
  static constexpr int touchOff = posOff(NPB);  // 256 bytes nobody reads (see touch_next)
  static constexpr int total = touchOff + 256;
};
// Chunk swizzle of V row r (see above).
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Wavefronts per workgroup, and how many key tiles ahead of the matrix work
// the tile loads run. Two 4-wave workgroups share a CU, so the two
// wavefronts of a SIMD belong to different workgroups and never wait on each
// other's barriers; with loads one tile ahead a workgroup's LDS (two K, two
// V and three position buffers) lets two fit. (Eight-wave workgroups alone
// on a CU with loads two tiles ahead measure slower: the two wavefronts of a
// SIMD then meet at every barrier.)
template <int GW>
constexpr int prefill_waves() { return 4; }
template <int GW>
constexpr int prefill_ahead() { return 1; }

// One workgroup of the prefill: the query tile and head group of the bid-th
// work record, in `smem_raw` (Lds<...>::total bytes, 16-byte aligned).
template <int D, int GW, int SRC>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, const Plan& pl, int bid,
                                             char* smem_raw) {
  constexpr int NW = prefill_waves<GW>();
  constexpr int AHEAD = prefill_ahead<GW>();
  constexpr int NKB = AHEAD + 1;  // K (and V) buffers
  constexpr int NPB = 4;          // position buffers (AHEAD + 2 used; a power of two)
  static_assert(AHEAD + 2 <= NPB, "position buffers");
  constexpr int SUB = NW / GW;  // query sub-tiles of 32 per workgroup
  constexpr int TQ = 32 * SUB;  // query tokens per workgroup
  constexpr int KS = D / 16;    // k-steps of QK^T over the head dim
  constexpr int MD = D / 32;    // 32-row blocks of O^T
  static_assert(TQ <= 128, "cache-row leaders fit a 128-bit mask");
  using L = Lds<D, NKB, NPB>;

  LdsByte* smem = (LdsByte*)smem_raw;

  const int G = a.heads / a.kv_heads;
  const int n_groups = a.kv_heads * pl.head_groups;
  const int wi = bid / n_groups;
  const int grp = bid % n_groups;
  const int kh = grp / pl.head_groups;
  const int hg = grp % pl.head_groups;
  // Tile indices are workgroup-uniform: keep them (and the summary loads that
  // depend on them) on the scalar unit.
  const int* rec = pl.rec + (long long)wi * kRecInts;
  const int qt = __builtin_amdgcn_readfirstlane(ld_const(rec, 0));
  // Query tile of the workgroup pl.resident indices later (-1: none).
  const int bid_next = bid + pl.resident;
  const int qt_next = pl.resident > 0 && bid_next < pl.n_qt * n_groups
                          ? __builtin_amdgcn_readfirstlane(ld_const(pl.rec + (long long)(bid_next / n_groups) * kRecInts, 0))
                          : -1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wave % GW;
  const int st = wave / GW;
  const int h = kh * G + hg * GW + hl;
  const int qn = lane & 31;
  const int hf = lane >> 5;
  const int P = a.p;
  const int q_tok = qt * TQ + st * 32 + qn;
  const bool q_valid = q_tok < P;
  const int q_ld = q_valid ? q_tok : P - 1;  // lanes past P read a real row
  const int my_pos = a.positions[q_ld];
  const int my_seg = SRC == kSrcPacked || a.segments ? a.segments[q_ld] : 0;
  // Packed keys. In one-segment tiles (mode 1) no position is negative, so
  // two differ by less than 2^31 and one unsigned compare of the difference
  // tests pos_k <= pos_q together with the window. The full predicate
  // (mode 2) compares the positions as signed values, then the unsigned
  // difference (exact once pos_k <= pos_q) against the window.
  const uint32_t wlim = a.window > 0 ? (uint32_t)a.window : 0x80000000u;
  const uint32_t wlast = a.window > 0 ? (uint32_t)a.window - 1u : 0xffffffffu;
  // Cache keys: this query sees key slots [my_lo, my_hi] of cache row my_seg
  // (empty for a row outside the cache).
  const int my_hi = (my_seg >= 0 && my_seg < a.cache_rows) ? min(my_pos, a.cap - 1) : -1;
  const int my_lo = a.window > 0 ? max(my_pos - a.window + 1, 0) : 0;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = load16(qg + ((long long)q_ld * a.heads + h) * D + ks * 16 + hf * 8);
  // These loads are retired before the loop (with the first tile's): inside
  // it the only vector loads in flight are the next tile's, so the wait
  // counters stay exact.
  auto retire_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    asm volatile("" ::"v"(my_pos), "v"(my_seg));
  };

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[md][r] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;

  // Tile loads go straight from memory into LDS, AHEAD key tiles ahead of
  // the matrix work, spread over the workgroup's wavefronts: a K tile is
  // L::kChunks 1-KiB loads (wave w the KU consecutive ones from w KU, the
  // last one wave 0), a V tile D / 8 (wave w the VU from w VU), and for
  // packed keys the positions (wave 1) and segments (wave 2) one 256-byte
  // load each. A wavefront's K (V) loads share one M0, the instruction
  // offset 1024 u moving both addresses; every buffer descriptor starts
  // kShift bytes before its tile, so that lane offsets, less those
  // instruction offsets, stay positive. Lane offsets (bytes from the tile's
  // first row, plus kShift) are fixed per wavefront; padding lanes fetch out
  // of range and write zeros.
  const int row_bytes = SRC == kSrcPacked ? a.kv_heads * D * 2 : D * 2;
  constexpr int KU = (L::kChunks - 1) / NW;  // K loads per wavefront, all waves
  constexpr int VU = (D / 8) / NW;           // V loads per wavefront
  static_assert(KU * NW == L::kChunks - 1 && VU * NW == D / 8, "loads cover the tiles");
  static_assert(1024 * (KU > VU ? KU : VU) <= kShift, "instruction offsets");
  constexpr int kOob = 0x40000000;           // past every tile's range
  int k_voff[KU + 1], v_voff[VU];
  auto k_lane_off = [&](int i) {
    const int p = 64 * i + lane;  // 16-byte chunk of the padded tile
    const int row = p / L::kChunks, ch = p - row * L::kChunks;
    return ch == D / 8 ? kOob : kappa(row) * row_bytes + ch * 16;
  };
#pragma unroll
  for (int u = 0; u < KU; ++u) k_voff[u] = k_lane_off(wave * KU + u) + kShift - 1024 * u;
  k_voff[KU] = k_lane_off(L::kChunks - 1) + kShift;
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int p = 64 * (wave * VU + u) + lane;
    const int row = p / (D / 8), ch = p % (D / 8);
    v_voff[u] = row * row_bytes + ((ch ^ vswz<D>(row)) << 4) + kShift - 1024 * u;
  }
  // Loads per wavefront per tile set, and the waits: a slot issues one K set
  // and one V set, and before its closing barrier waits for the sets the
  // previous slot issued.
  const bool extra_load = wave == 0 || (SRC == kSrcPacked && (wave == 1 || wave == 2));
  const int k_rd = qn * L::kStride + hf * 16;
  // P.V operand reads (transposing, 4 keys x 16 dimensions per 16-lane
  // group): lane l of group g = l / 16 supplies the address of key
  // 8 (g / 2) + (l % 16) / 4 (+4 for the second read), dimensions
  // 32 md + 16 (g % 2) + 4 (l % 4) .. +3; it receives 4 keys of dimension
  // 32 md + l % 32.
  int v_rd[MD];
  {
    const int vg = lane >> 4, vs = lane & 15;
    const int row = 8 * (vg >> 1) + (vs >> 2);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const int ch = 4 * md + 2 * (vg & 1) + ((vs >> 1) & 1);
      v_rd[md] = row * L::vStride + ((ch ^ vswz<D>(row)) << 4) + ((vs & 1) << 3);
    }
  }

  // A key tile: tile index kt (64 keys) of cache row r, at pool page `page`;
  // full: every pair with the query tile is allowed.
  // one: packed keys of a single segment, the query tile's (mask by
  // positions only).
  struct TileRef {
    int kt, r, page, rows, mode;  // rows: cache slots of the tile anyone may see;
                                  // mode: 0 every pair allowed, 1 / 2 masked (see soft_slice)
  };
  // Buffer resource over one operand (K or V) of a key tile: 64 key slots of
  // one cache plane, or 64 packed tokens at KV head kh; it starts kShift
  // bytes before the tile. Packed keys: the range runs to the end of the
  // operand (the host keeps p * row_bytes + kShift below 2^31), so rows past
  // p read zeros; the per-tile work is two 64-bit adds and a subtraction.
  const int tile_bytes = kBK * row_bytes;
  const int nrec0 = P * row_bytes + kShift;
  const unsigned long long kbase = reinterpret_cast<unsigned long long>(a.k) + 2ull * kh * D - kShift;
  const unsigned long long vbase = reinterpret_cast<unsigned long long>(a.v) + 2ull * kh * D - kShift;
  auto tile_src = [&](TileRef t, const void* base) {
    if constexpr (SRC != kSrcPacked) {
      const long long e0 = SRC == kSrcPaged ? ((long long)t.page * a.kv_heads + kh) * kBK * D
                                            : (((long long)t.r * a.kv_heads + kh) * a.cap + (long long)t.kt * kBK) * D;
      return raw_rsrc(static_cast<const char*>(base) + 2 * e0 - kShift, (t.rows - 1) * row_bytes + 2 * D + kShift);
    } else {
      const int off = t.kt * tile_bytes;
      const unsigned long long b = (base == a.k ? kbase : vbase) + (unsigned)off;
      i32x4 r;
      r[0] = (int)(uint32_t)b;
      r[1] = (int)(uint32_t)(b >> 32);  // device addresses are below 2^48: stride 0
      r[2] = nrec0 - off;
      r[3] = 0x00020000;
      return r;
    }
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // Load u of a K set (tile t into K buffer kb and position buffer pb). The
  // one extra load per wavefront: the last K chunk (wave 0), the key
  // positions (wave 1) or segments (wave 2) of packed keys.
  struct KSet {
    i32x4 rk, rx;
  };
  const unsigned long long x_src = reinterpret_cast<unsigned long long>(wave == 1 ? a.positions : a.segments);
  const int x_lds = wave == 1 ? 0 : kBK * 4;
  auto k_set = [&](TileRef t) {
    KSet s;
    s.rk = tile_src(t, a.k);
    if constexpr (SRC == kSrcPacked) {
      const unsigned long long b = x_src + 4u * (unsigned)(t.kt * kBK);
      s.rx[0] = (int)(uint32_t)b;
      s.rx[1] = (int)(uint32_t)(b >> 32);
      s.rx[2] = 4 * (P - t.kt * kBK);
      s.rx[3] = 0x00020000;
    } else {
      s.rx = s.rk;
    }
    return s;
  };
  // xload: this tile's key positions and segments are needed (it is masked;
  // a fully allowed tile never reads them).
  auto k_load = [&](const KSet& s, int kb, int pb, bool xload, auto uc) {
    constexpr int u = decltype(uc)::value;
    if constexpr (u < KU) {
      if constexpr (u == 0) set_lds_m0(lds0 + L::kOff(kb) + 1024 * KU * wave);
      lds_dma16_m0<1024 * u>(s.rk, k_voff[u]);
    } else {
      if (wave == 0) {
        lds_dma<16>(s.rk, lds0 + L::kOff(kb) + 1024 * (L::kChunks - 1), k_voff[KU]);
      } else if (SRC == kSrcPacked && wave < 3 && xload) {
        lds_dma<4>(s.rx, lds0 + L::posOff(pb) + x_lds, lane * 4);
      }
    }
  };
  auto v_load = [&](i32x4 rv, int vb, auto uc) {
    constexpr int u = decltype(uc)::value;
    if constexpr (u == 0) set_lds_m0(lds0 + L::vOff(vb) + 1024 * VU * wave);
    lds_dma16_m0<1024 * u>(rv, v_voff[u]);
  };
  // Wait until the tile loads of all but the last AHEAD - 1 slots have
  // landed (a slot issues KU + VU loads, one more on the waves with an extra
  // load).
  auto wait_loads = [&](bool extra) {
    constexpr int n0 = (AHEAD - 1) * (KU + VU), n1 = (AHEAD - 1) * (KU + VU + 1);
    static_assert(n1 < 16, "vmcnt field");
    if (extra) __builtin_amdgcn_s_waitcnt(0xF70 | n1);
    else __builtin_amdgcn_s_waitcnt(0xF70 | n0);
  };
  // Workgroup barrier that neither waits for the loads in flight nor lets
  // the compiler move memory accesses across it.
  auto barrier = [&]() { asm volatile("s_barrier" ::: "memory"); };

  // Packed keys: walk the query tile's visit list (fully allowed tiles
  // first; the online softmax does not depend on the order of the key
  // tiles). The first kRecVis entries come with the start record.
  const int v_n = __builtin_amdgcn_readfirstlane(ld_const(rec, 1)) + __builtin_amdgcn_readfirstlane(ld_const(rec, 2));

  // Packed keys: the workgroup pl.resident indices later will most likely
  // start when one of the workgroups running now ends. Its queries are
  // fetched into the caches by this workgroup, one 128-byte line per lane
  // (the data lands in an LDS area nobody reads), so that its start does not
  // wait on a cold read. The fetch is the first slot's last load and that
  // slot's closing wait leaves it in flight: it has two slots to land. Walks
  // shorter than kTouchMinTiles skip it (the wait would show in them).
  const int tok_next = qt_next * TQ + st * 32;
  const bool touch = SRC == kSrcPacked && AHEAD == 1 && qt_next >= 0 && tok_next < P && v_n >= kTouchMinTiles;
  auto touch_next = [&]() {
    if (touch) {
      const int grp2 = bid_next % n_groups;
      const int h2 = (grp2 / pl.head_groups) * G + (grp2 % pl.head_groups) * GW + hl;
      // Lane l: token tok_next + l % 32, line l / 32 of its 2 D-byte row;
      // the range ends at the end of q (lanes past it read nothing).
      const long long row = (long long)a.heads * D * 2;
      const long long left = (long long)(P - tok_next) * row - (long long)h2 * D * 2;
      const i32x4 rq = raw_rsrc(static_cast<const char*>(a.q) + (tok_next * (long long)a.heads + h2) * D * 2,
                                (int)(left < (1ll << 30) ? left : (1ll << 30)));
      constexpr int kLine2 = D * 2 > 128 ? 128 : 0;
      lds_dma<4>(rq, (uint32_t)(uintptr_t)smem + L::touchOff, (int)((lane & 31) * row + (lane >> 5) * kLine2));
    }
  };
  // The first slot's closing wait: the same, less the query fetch issued
  // last (loads complete in issue order, so the next slot's wait covers it).
  auto wait_loads_first = [&](bool extra) {
    static_assert(AHEAD == 1, "one load left in flight");
    if (touch) __builtin_amdgcn_s_waitcnt(0xF70 | 1);
    else wait_loads(extra);
  };
  const int* visq = pl.vis + (long long)qt * pl.n_kt;
  int v_i = 0;

  // Cache keys. Once per workgroup: the distinct cache rows of the query
  // tile's tokens, each with the smallest and largest position among them
  // (a row's token is its leader if no earlier token of the tile has the same
  // row; leaders are flagged in a 128-bit mask, so the walk is deterministic).
  // A row's key tiles run from the window's first slot to its largest
  // position; loads past that position return zeros (slots nobody sees may
  // hold anything). When the tile holds one row, the key tiles [f_lo, f_hi]
  // are fully allowed for every query. Phase 0 walks those, phase 1 the
  // rest; tiles on invalid pages are skipped (they hold no keys).
  __shared__ int sTokRow[SRC == kSrcPacked ? 1 : TQ];
  __shared__ int sTokLo[SRC == kSrcPacked ? 1 : TQ];
  __shared__ int sTokHi[SRC == kSrcPacked ? 1 : TQ];
  __shared__ unsigned long long sLead[2];
  __shared__ int sBad;
  unsigned long long lead0 = 0, lead1 = 0;
  bool any_bad = false;
  if constexpr (SRC != kSrcPacked) {
    const int t = qt * TQ + tid;
    const bool tok = tid < TQ && t < P;
    const int trow = tok ? (a.segments ? a.segments[t] : 0) : -1;
    const int tpos = tok ? a.positions[t] : 0;
    const bool row_ok = tok && trow >= 0 && trow < a.cache_rows;
    if (tid < TQ) {
      sTokRow[tid] = row_ok ? trow : -1;
      sTokLo[tid] = tpos;
    }
    if (tid == 0) sBad = 0;
    __syncthreads();
    // A token whose row is outside the cache has no keys: its tile may not
    // take the unmasked single-row path.
    if (tok && !row_ok) sBad = 1;
    bool lead = row_ok;
    int lo = tpos, hi = tpos;
    if (row_ok) {
      for (int u = 0; u < TQ; ++u) {
        const int ru = sTokRow[u];
        if (ru != trow) continue;
        if (u < tid) lead = false;
        lo = min(lo, sTokLo[u]);
        hi = max(hi, sTokLo[u]);
      }
    }
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(lead);
    __syncthreads();
    if (tid < TQ) {
      sTokLo[tid] = lo;
      sTokHi[tid] = hi;
    }
    if (lane == 0 && wave < 2) sLead[wave] = bal;
    __syncthreads();
    lead0 = sLead[0];
    lead1 = TQ > 64 ? sLead[1] : 0ull;
    any_bad = sBad != 0;
  }
  const int n_lead = __builtin_popcountll(lead0) + __builtin_popcountll(lead1);
  const bool c_single = n_lead == 1 && !any_bad;
  // Walk state: current leader token u, its row, key-tile range, last slot.
  int c_phase = 0, c_u = -1, c_row = 0, c_klo = 0, c_khi = -1, c_last = -1, c_kt = 0;
  int c_flo = 0, c_fhi = -1;
  auto next_row = [&]() {
    // Next leader after c_u (bit scans over the two 64-bit halves).
    const int from = c_u + 1;
    int u = -1;
    if (from < 64) {
      const unsigned long long m = from == 0 ? lead0 : (lead0 >> from) << from;
      if (m) u = __builtin_ctzll(m);
    }
    if (u < 0 && from < 128) {
      const int f1 = max(from - 64, 0);
      const unsigned long long m = f1 == 0 ? lead1 : (f1 >= 64 ? 0ull : (lead1 >> f1) << f1);
      if (m) u = 64 + __builtin_ctzll(m);
    }
    c_u = u < 0 ? 128 : u;
    if (u < 0) return false;
    c_row = __builtin_amdgcn_readfirstlane(sTokRow[u]);
    const int lo = __builtin_amdgcn_readfirstlane(sTokLo[u]);
    const int hi = __builtin_amdgcn_readfirstlane(sTokHi[u]);
    c_last = min(hi, a.cap - 1);
    c_khi = c_last >= 0 ? c_last / kBK : -1;
    c_klo = a.window > 0 ? max(0, lo - a.window + 1) / kBK : 0;
    c_flo = max(c_klo, a.window > 0 ? (max(hi - a.window + 1, 0) + kBK - 1) / kBK : 0);
    c_fhi = min(c_khi, c_single ? (min(lo, a.cap - 1) + 1) / kBK - 1 : -1);
    return true;
  };
  // Page id of key tile kt of table row r (a scalar load: the walk runs
  // while tile loads are in flight, and a vector load would wait for them).
  auto page_of = [&](int r, int kt) {
    return kt < a.table_pages ? ld_const(a.table, (long long)r * a.table_pages + kt) : -1;
  };
  bool c_started = false;
  auto cache_next = [&](int& phase) {
    TileRef t{-1, 0, 0, 0, 2};
    if (!c_started) {
      c_started = true;
      c_phase = c_single ? 0 : 1;
      if (next_row()) c_kt = c_phase == 0 ? c_flo : c_klo;
    }
    for (;;) {
      if (c_u >= 128) break;
      if (c_phase == 0) {
        if (c_kt > c_fhi) {
          // Phase 1 restarts the single row, skipping the full range.
          c_phase = 1;
          c_kt = c_klo;
          continue;
        }
      } else {
        if (c_kt > c_khi) {
          if (!next_row()) break;
          c_kt = c_klo;
          continue;
        }
        if (c_single && c_kt >= c_flo && c_kt <= c_fhi) {
          c_kt = c_fhi + 1;
          continue;
        }
      }
      const int kt = c_kt++;
      int page = 0;
      if constexpr (SRC == kSrcPaged) {
        page = page_of(c_row, kt);
        if (page < 0 || page >= a.num_pages) continue;
      }
      t = TileRef{kt, c_row, page, min(kBK, c_last - kt * kBK + 1), 2};
      break;
    }
    phase = c_phase;
    t.kt = __builtin_amdgcn_readfirstlane(t.kt);
    t.mode = __builtin_amdgcn_readfirstlane(phase == 0 ? 0 : 2);
    t.r = __builtin_amdgcn_readfirstlane(t.r);
    t.page = __builtin_amdgcn_readfirstlane(t.page);
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    return t;
  };

  // Software pipeline over 32-key halves of the key tiles. Half-slot j
  // issues the S^T MFMAs of half j, the P.V MFMAs of half j - 2 (alternating,
  // so the S^T accumulator chain never waits on itself) and, in the shadow of
  // those MFMAs, the softmax of half j - 1. A slot is the two half-slots of
  // key tile T: it reads K of tile T and V of tile T - 1 and issues the loads
  // of K (and positions) of tile T + AHEAD and V of tile T + AHEAD - 1, so
  // AHEAD + 1 K and V buffers and AHEAD + 2 position buffers rotate. On gfx950 a SIMD overlaps an MFMA
  // with vector instructions issued in its shadow, so each step issues one
  // MFMA followed by a slice of vector work, and a scheduling fence keeps
  // that order; every slice's inputs were produced a step or more earlier.
  // Matrix operands are read from LDS four steps ahead through a ring of
  // registers. The O rescales of the lazy softmax (rare) close a half-slot
  // whose softmax moved the reference.
  constexpr int C = D / 16;        // S^T MFMAs (and P.V MFMAs) per half
  static_assert(KS == C && 2 * MD == C, "step counts");
  constexpr int HS = 2 * C;        // matrix steps per half-slot
  constexpr int NSOFT = 14;        // softmax slices per half
  constexpr int NLOAD = KU + 1 + VU;  // load steps at the start of a slot
  static_assert(NLOAD < HS, "loads (and the query fetch after them) fit the first half-slot");
  u32x4 pw[4];                     // P of the halves of parity 0 and 1 (bf16)
  f32x16 s[2];                     // S^T of the halves of parity 0 and 1
  bf16x8 ring[4];
  float tmax = kNegInf, m_use = 0.f, alpha = 1.f;
  float xa0 = 0.f, xa1 = 0.f, ea0 = 0.f, ea1 = 0.f, psa = 0.f, psb = 0.f;

  // Operand of slot step g: half-slot h = g / HS, step i = g % HS; even
  // steps are S^T MFMAs (K rows of half h of tile T), odd ones P.V MFMAs
  // (V^T of keys of half h of tile T - 1, two transposing reads).
  // kb: this lane's K row of the slot's K buffer; vb[md]: its V^T read
  // address for block md of the slot's V buffer (per-slot VGPR bases, so
  // every read below takes a small immediate offset).
  auto operand = [&](const LdsByte* kb, const uint32_t* vb, auto gc) {
    constexpr int g = decltype(gc)::value;
    constexpr int h = g / HS, i = g % HS;
    if constexpr (i % 2 == 0) {
      return lds_ld<bf16x8>(kb + h * 32 * L::kStride + (i / 2) * 32);
    } else {
      constexpr int j = i / 2, kk = j / MD, md = j % MD;
      typedef __attribute__((address_space(3))) bf16x4 LdsV4;
      const LdsByte* p = smem + vb[md] + 16 * (2 * h + kk) * L::vStride;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsV4*)p);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsV4*)(p + 4 * L::vStride));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto mfma_at = [&](auto gc, const bf16x8& op) {
    constexpr int g = decltype(gc)::value;
    constexpr int h = g / HS, i = g % HS;
    if constexpr (i % 2 == 0) {
      constexpr int ks = i / 2;
      if constexpr (ks == 0)
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, __builtin_bit_cast(bf16x8, qf[ks]), f32x16{}, 0, 0, 0);
      else
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, __builtin_bit_cast(bf16x8, qf[ks]), s[h], 0, 0, 0);
    } else {
      constexpr int j = i / 2, kk = j / MD, md = j % MD;
      o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, __builtin_bit_cast(bf16x8, pw[2 * h + kk]), o[md], 0, 0, 0);
    }
  };

  // Slice c (0 <= c < NSOFT) of the mask and online-softmax update of the
  // 32-key half hb of a tile (accumulator s[hb]):
  //   0, 1   mask (when masked) rows 8c .. 8c + 7 and fold them into the max
  //   2      combine the two lane halves' maxima
  //   3      move the lazy reference
  //   4 .. 13  probabilities as a three-stage pipeline over the 8 row pairs
  //          (slice 4 + k: pack pair k - 2 to bf16 and add it to the sums,
  //          exponentiate pair k - 1, scale pair k), so no instruction waits
  //          on one issued in the same slice.
  // mode: 0 every pair allowed, 1 packed keys of the query tile's one
  // segment (positions and the window decide), 2 the full predicate.
  auto soft_slice = [&](const LdsByte* pb, int lo_j, int hi_j, int n_j, auto hbc, auto cc, int mode) {
    constexpr int hb = decltype(hbc)::value;
    constexpr int c = decltype(cc)::value;
    if constexpr (c < 2) {
      if (__builtin_expect(mode != 0, 0)) {
        // The literal own predicate (and the window) per element; rows
        // 8c .. 8c + 7 are the 8 consecutive keys jb + 8 hf + e.
        constexpr int jb = 32 * hb + 16 * c;
        if constexpr (SRC == kSrcPacked) {
          const LdsByte* pp = pb + (jb + 8 * hf) * 4;
          if (mode == 1) {
            // Every key and query of the two tiles is in one segment and the
            // key tile holds 64 real keys.
#pragma unroll
            for (int q4 = 0; q4 < 2; ++q4) {
              const u32x4 kp = lds_ld<u32x4>(pp + 16 * q4);
#pragma unroll
              for (int e4 = 0; e4 < 4; ++e4) {
                const int e = 4 * q4 + e4;
                s[hb][8 * c + e] = ((uint32_t)my_pos - kp[e4] < wlim) ? s[hb][8 * c + e] : kNegInf;
              }
            }
          } else {
          // Keys past P (zeros in LDS) are excluded by index: e < e_end.
          const int e_end = n_j - jb - 8 * hf;
#pragma unroll
          for (int q4 = 0; q4 < 2; ++q4) {
            const u32x4 kp = lds_ld<u32x4>(pp + 16 * q4), ksg = lds_ld<u32x4>(pp + kBK * 4 + 16 * q4);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int e = 4 * q4 + e4;
              const bool ok = ((int)ksg[e4] == my_seg) & ((int)kp[e4] <= my_pos) &
                              ((uint32_t)my_pos - kp[e4] <= wlast) & (e < e_end);
              s[hb][8 * c + e] = ok ? s[hb][8 * c + e] : kNegInf;
            }
          }
          }
        } else {
          // Key slot kt * 64 + jb + 8 hf + e of the tile's row is visible
          // for e in [e_lo, e_hi].
          const int e_lo = lo_j - jb - 8 * hf, e_hi = hi_j - jb - 8 * hf;
#pragma unroll
          for (int e = 0; e < 8; ++e) s[hb][8 * c + e] = ((e >= e_lo) & (e <= e_hi)) ? s[hb][8 * c + e] : kNegInf;
        }
      }
      const float m0 = vmax3(s[hb][8 * c], s[hb][8 * c + 1], s[hb][8 * c + 2]);
      const float m1 = vmax3(s[hb][8 * c + 3], s[hb][8 * c + 4], s[hb][8 * c + 5]);
      const float m2 = c == 0 ? vmax(s[hb][8 * c + 6], s[hb][8 * c + 7]) : vmax3(s[hb][8 * c + 6], s[hb][8 * c + 7], tmax);
      tmax = vmax3(m0, m1, m2);
      // Keep this slice's work in its step (the compiler would merge it
      // into the next slice, past the mask branch).
      asm volatile("" : "+v"(tmax));
    } else if constexpr (c == 2) {
      // Online softmax in the log2 domain. scale > 0, so the row max of the
      // scaled scores is the scaled row max of the raw ones.
      tmax = pair_max(tmax) * a.scale_log2;
      asm volatile("" : "+v"(tmax));
    } else if constexpr (c == 3) {
      // m_run is the lazy reference (see kLazyMaxLog2).
      const float m_new = (tmax > m_run + kLazyMaxLog2) ? tmax : m_run;
      m_use = (m_new == kNegInf) ? 0.f : m_new;
      alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      asm volatile("" : "+v"(m_use), "+v"(alpha), "+v"(m_run));
    } else {
      constexpr int k = c - 4;
      if constexpr (k >= 2) {
        constexpr int r = 2 * (k - 2);
        pw[2 * hb + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(ea0, ea1);
        psa = k == 2 ? ea0 : psa + ea0;
        psb = k == 2 ? ea1 : psb + ea1;
        // Materialize here: without the anchors the compiler sinks this work
        // past the rescale branch, next to its use, out of the MFMA shadow.
        asm volatile("" ::"v"(pw[2 * hb + (r >> 3)][(r & 7) >> 1]));
        asm volatile("" : "+v"(psa), "+v"(psb));
      }
      if constexpr (k >= 1 && k <= 8) {
        ea0 = fast_exp2(xa0);
        ea1 = fast_exp2(xa1);
        asm volatile("" : "+v"(ea0), "+v"(ea1));
      }
      if constexpr (k <= 7) {
        constexpr int r = 2 * k;
        xa0 = __builtin_fmaf(s[hb][r], a.scale_log2, -m_use);
        xa1 = __builtin_fmaf(s[hb][r + 1], a.scale_log2, -m_use);
        asm volatile("" : "+v"(xa0), "+v"(xa1));
      }
      if constexpr (k == 9) {
        l_run = l_run * alpha + (psa + psb);
        asm volatile("" : "+v"(l_run));
      }
    }
  };

  // Rescale O only when some lane's reference moved.
  auto rescale = [&](float f) {
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(f != 1.f) != 0, 0)) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= f;
    }
  };

  // The key tiles in visiting order: phase 0 (every pair allowed) first,
  // then phase 1 (masked); the online softmax does not depend on the order.
  auto valid = [&](TileRef t) { return t.kt >= 0; };
  int wphase = 0;
  auto gen = [&]() {
    TileRef t{-1, 0, 0, 0, 2};
    if constexpr (SRC == kSrcPacked) {
      if (v_i < v_n) {
        const int* e = v_i < kRecVis ? rec + 4 : visq;
        const int ent = __builtin_amdgcn_readfirstlane(ld_const(e, v_i));
        t.kt = ent & ((1 << kVisMode) - 1);
        t.mode = ent >> kVisMode;
        ++v_i;
      }
    } else {
      t = cache_next(wphase);
      t.mode = wphase == 0 ? 0 : 2;
    }
    return t;
  };

  // One slot (T = its index). DO_S: key tile t exists (its S^T and the
  // softmax of its first half run, the loads of tiles kn (K) and vn (V) are
  // issued, and the walk finds the tile after kn, t_gen); DO_PREV: tile tp
  // (the previous one) exists (the softmax of its second half and its P.V
  // run). Unless `masked`, every pair of both tiles is allowed (a uniform
  // branch: one loop body serves both kinds of slot).
  TileRef t_gen{-1, 0, 0, 0, 2};
  auto mode_of = [](TileRef t) { return t.mode; };
  auto slot = [&](int mode_t, int mode_p, auto dosc, auto doprevc, TileRef t, TileRef tp, TileRef kn, TileRef vn, int T) {
    constexpr bool DO_S = decltype(dosc)::value;
    constexpr bool DO_PREV = decltype(doprevc)::value;
    const unsigned Tu = T;
    uint32_t kb_off = L::kOff(Tu % NKB) + k_rd;
    asm volatile("" : "+v"(kb_off));
    const LdsByte* kb = smem + kb_off;
    uint32_t vb[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      vb[md] = L::vOff((Tu + NKB - 1) % NKB) + v_rd[md];
      asm volatile("" : "+v"(vb[md]));
    }
    const LdsByte* pb_t = smem + L::posOff(Tu % NPB);
    const LdsByte* pb_p = smem + L::posOff((Tu + NPB - 1) % NPB);
    // Cache keys: this lane's visible slots relative to each tile; packed
    // keys: the real keys of each tile.
    const int lo_t = my_lo - t.kt * kBK;
    const int hi_t = (t.r == my_seg ? my_hi : -1) - t.kt * kBK;
    const int lo_p = my_lo - tp.kt * kBK;
    const int hi_p = (tp.r == my_seg ? my_hi : -1) - tp.kt * kBK;
    const int n_t = P - t.kt * kBK, n_p = P - tp.kt * kBK;
    const KSet ks = k_set(kn);
    const i32x4 rv = tile_src(vn, a.v);
    auto has_mfma = [](auto gc) {
      constexpr int i = decltype(gc)::value % HS;
      return std::integral_constant<bool, (i % 2 == 0) ? DO_S : DO_PREV>{};
    };
    static_for<4>([&](auto gc) {
      if constexpr (decltype(has_mfma(gc))::value) ring[decltype(gc)::value] = operand(kb, vb, gc);
    });
    static_for<2 * HS>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      constexpr int h = g / HS, i = g % HS;
      if constexpr (decltype(has_mfma(gc))::value) mfma_at(gc, ring[g & 3]);
      if constexpr (g + 4 < 2 * HS) {
        using gn = std::integral_constant<int, g + 4>;
        if constexpr (decltype(has_mfma(gn{}))::value) ring[(g + 4) & 3] = operand(kb, vb, gn{});
      }
      if constexpr (DO_S && h == 0 && i < NLOAD) {
        if constexpr (i <= KU) k_load(ks, (Tu + AHEAD) % NKB, (Tu + AHEAD) % NPB, AHEAD >= 2 || kn.mode != 0, std::integral_constant<int, i>{});
        else v_load(rv, (Tu + AHEAD - 1) % NKB, std::integral_constant<int, i - KU - 1>{});
      }
      if constexpr (SRC == kSrcPacked && DO_S && !DO_PREV && h == 0 && i == NLOAD) touch_next();
      if constexpr (DO_S && h == 1 && i == 0) t_gen = gen();
      // Half-slot 0 runs the softmax of tile tp's second half, half-slot 1
      // that of tile t's first half; slice c sits at step 2 + c (HS - 2) / NSOFT,
      // clear of the latency of the S^T MFMAs it reads.
      constexpr bool soft = h == 0 ? DO_PREV : DO_S;
      if constexpr (soft) {
        static_for<NSOFT>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr (2 + c * (HS - 2) / NSOFT == i)
            soft_slice(h == 0 ? pb_p : pb_t, h == 0 ? lo_p : lo_t, h == 0 ? hi_p : hi_t, h == 0 ? n_p : n_t,
                       std::integral_constant<int, 1 - h>{}, cc, h == 0 ? mode_p : mode_t);
        });
      }
      if constexpr (soft && i == HS - 1) rescale(alpha);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (DO_S) {
      // The loads of the previous slot have landed (this slot's may fly on).
      if constexpr (SRC == kSrcPacked && !DO_PREV) wait_loads_first(extra_load);
      else wait_loads(extra_load);
      barrier();
    }
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  static_assert(AHEAD == 1 || AHEAD == 2, "tile look-ahead");
  TileRef cur = gen();
  if (valid(cur)) {
    // The tiles after cur: n1, and n2 when the loads run two tiles ahead.
    TileRef n1 = gen();
    TileRef n2 = AHEAD >= 2 ? gen() : cur;
    auto or_cur = [&](TileRef x, TileRef c) { return valid(x) ? x : c; };
    // Tiles whose K and V a slot loads (a tile past the end loads cur again,
    // into a buffer nobody reads, which keeps the wait counts exact).
    auto kn_of = [&]() { return AHEAD >= 2 ? or_cur(n2, cur) : or_cur(n1, cur); };
    auto vn_of = [&]() { return AHEAD >= 2 ? or_cur(n1, cur) : cur; };
    auto shift = [&](TileRef& prev) {
      prev = cur;
      cur = n1;
      if constexpr (AHEAD >= 2) {
        n1 = n2;
        n2 = t_gen;
      } else {
        n1 = t_gen;
      }
    };
    // Prologue: K of the first AHEAD tiles and V of the first AHEAD - 1.
    {
      const KSet k0 = k_set(cur);
      static_for<KU + 1>([&](auto uc) { k_load(k0, 0, 0, AHEAD >= 2 || cur.mode != 0, uc); });
      if constexpr (AHEAD >= 2) {
        const KSet k1 = k_set(or_cur(n1, cur));
        static_for<KU + 1>([&](auto uc) { k_load(k1, 1, 1, true, uc); });
        const i32x4 r0 = tile_src(cur, a.v);
        static_for<VU>([&](auto uc) { v_load(r0, 0, uc); });
      }
      retire_q();
      wait_loads(extra_load);
      barrier();
    }
    slot(mode_of(cur), 0, T_{}, F_{}, cur, cur, kn_of(), vn_of(), 0);
    TileRef prev;
    shift(prev);
    int T = 1;
    // Each half-slot masks by the mode of the tile whose softmax it runs.
    while (valid(cur)) {
      slot(mode_of(cur), mode_of(prev), T_{}, T_{}, cur, prev, kn_of(), vn_of(), T);
      shift(prev);
      ++T;
    }
    // Drain: the last tile's second half and its P.V.
    slot(0, mode_of(prev), F_{}, T_{}, prev, prev, prev, prev, T);
  }
  // No tile load may still be writing this workgroup's LDS when it exits.
  __builtin_amdgcn_s_waitcnt(0xF70);

  // Normalize; the sink logit joins the denominator.
  const float l_tot = pair_sum(l_run);
  float f = 1.f, den = l_tot;
  if (a.sinks != nullptr) {
    const float s2 = bf16_to_f32(static_cast<const uint16_t*>(a.sinks)[h]) * kLog2e;
    const float M = fmaxf(m_run, s2);
    f = fast_exp2(m_run - M);
    den = l_tot * f + fast_exp2(s2 - M);
  }
  const float inv = den > 0.f ? f / den : 0.f;
  if (a.lse != nullptr && q_valid && hf == 0) {
    // Natural-log softmax denominator at reference 0 (no sink).
    constexpr float kLn2 = 0.6931471805599453f;
    a.lse[(long long)q_tok * a.heads + h] = l_tot > 0.f ? (m_use + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
  }
  if (q_valid) {
    uint16_t* og = static_cast<uint16_t*>(a.out) + ((long long)q_tok * a.heads + h) * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(o[md][4 * g] * inv, o[md][4 * g + 1] * inv);
        w[1] = pack_bf16x2(o[md][4 * g + 2] * inv, o[md][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(og + 32 * md + 8 * g + 4 * hf) = w;
      }
  }
}

template <int D, int GW, int SRC>
__global__ __launch_bounds__(64 * prefill_waves<GW>(), 8 / prefill_waves<GW>()) void prefill_kernel(PrefillArgs a, Plan pl) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Lds<D, prefill_ahead<GW>() + 1, 4>::total];
  prefill_body<D, GW, SRC>(a, pl, blockIdx.x, smem_raw);
}

// One step of step_paged in a single grid: the first n_dec workgroups each
// decode one (decode row, KV head) over its whole key range -- one split, so
// they write the output themselves -- and the rest are the chunk's prefill
// workgroups in their usual order. The decode shares take workgroup ids
// [dec0, dec0 + n_dec): the costliest prefill tiles (the first in their
// order) start before them, and they stream the cache (each wavefront loading
// its next chunk while it computes the current one) while the remaining
// prefill tiles keep the matrix cores busy, finishing long before the grid's
// tail. Measured alternatives were slower: the decode shares first or last in
// the grid, and rows split into 1024- or 2048-key pieces (more workgroups
// plus a merge pass).
template <int D, int GW>
__global__ __launch_bounds__(64 * prefill_waves<GW>(), 8 / prefill_waves<GW>()) void step_paged_kernel(PrefillArgs a, Plan pl, DecodeArgs d, int n_dec, int dec0) {
  constexpr int NW = prefill_waves<GW>();
  constexpr int kPre = Lds<D, prefill_ahead<GW>() + 1, 4>::total;
  constexpr int kDec = decode_mfma_lds_bytes<D, NW>();
  __shared__ __attribute__((aligned(16))) char smem_raw[kPre > kDec ? kPre : kDec];
  const int bid = blockIdx.x;
  if (bid >= dec0 && bid < dec0 + n_dec) {
    const int db = bid - dec0;
    decode_mfma_body<D, true, NW, false, true>(d, 0, db % d.kv_heads, db / d.kv_heads, smem_raw);
    return;
  }
  prefill_body<D, GW, kSrcPaged>(a, pl, bid < dec0 ? bid : bid - n_dec, smem_raw);
}

// ---------------------------------------------------------------------------
static int group_width(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1; }

size_t prefill_plan_bytes(int p) {
  const size_t n_kt = (size_t)(p + kBK - 1) / kBK;
  const size_t n_qt = (size_t)(p + 31) / 32;  // the smallest query tile
  const size_t n_kg = (n_kt + 63) / 64;
  return align256(n_kt * sizeof(TileSum)) + align256(n_qt * sizeof(TileSum)) +
         align256(n_qt * sizeof(int2)) + 2 * align256(n_qt * sizeof(int)) +
         align256(n_qt * n_kg * kMaskWords * sizeof(uint32_t)) + align256(n_qt * kRecInts * sizeof(int)) +
         align256(n_qt * sizeof(int)) + align256(n_qt * n_kt * sizeof(int));
}

size_t prefill_workspace_bytes(int p, int heads, int kv_heads, int head_dim) {
  (void)heads;
  (void)kv_heads;
  (void)head_dim;
  return prefill_plan_bytes(p);
}

template <int D, int GW>
static void launch_main(const PrefillArgs& a, const Plan& pl, hipStream_t stream) {
  const int n_groups = a.kv_heads * pl.head_groups;
  const dim3 grid(pl.n_qt * n_groups), block(64 * prefill_waves<GW>());
  if (a.src == kSrcContiguous) prefill_kernel<D, GW, kSrcContiguous><<<grid, block, 0, stream>>>(a, pl);
  else if (a.src == kSrcPaged) prefill_kernel<D, GW, kSrcPaged><<<grid, block, 0, stream>>>(a, pl);
  else prefill_kernel<D, GW, kSrcPacked><<<grid, block, 0, stream>>>(a, pl);
}

// Compute units of the current device (queried once per device; 0 if the
// query fails).
static int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// The plan's shape and its arrays' places in the workspace (host only).
static void prefill_layout(const PrefillArgs& a, Plan& pl, int waves) {
  const int G = a.heads / a.kv_heads;
  pl.gw = group_width(G);
  pl.head_groups = G / pl.gw;
  if (waves <= 0) waves = pl.gw == 4 ? prefill_waves<4>() : pl.gw == 2 ? prefill_waves<2>() : prefill_waves<1>();
  pl.tq = 32 * (waves / pl.gw);
  // Cache keys need no key-tile summaries or masks.
  pl.n_kt = a.src == kSrcPacked ? (a.p + kBK - 1) / kBK : 0;
  pl.n_qt = (a.p + pl.tq - 1) / pl.tq;
  pl.max_cost = a.src == kSrcPacked ? pl.n_kt : min(kMaxCostBins - 1, a.cap / kBK + 1);
  pl.resident = 2 * device_cu_count();  // two forward workgroups per CU
  const size_t n_kt_b = align256((size_t)pl.n_kt * sizeof(TileSum));
  const size_t n_qt_max = (size_t)(a.p + 31) / 32;
  const size_t q_b = align256(n_qt_max * sizeof(TileSum));
  const size_t r_b = align256(n_qt_max * sizeof(int2));
  char* ws = static_cast<char*>(a.ws);
  pl.ksum = reinterpret_cast<TileSum*>(ws);
  pl.qsum = reinterpret_cast<TileSum*>(ws + n_kt_b);
  pl.qrange = reinterpret_cast<int2*>(ws + n_kt_b + q_b);
  pl.order = reinterpret_cast<int*>(ws + n_kt_b + q_b + r_b);
  pl.cost = reinterpret_cast<int*>(ws + n_kt_b + q_b + r_b + align256(n_qt_max * sizeof(int)));
  pl.n_kg = (pl.n_kt + 63) / 64;
  pl.masks = reinterpret_cast<uint32_t*>(ws + n_kt_b + q_b + r_b + 2 * align256(n_qt_max * sizeof(int)));
  const size_t n_kg_max = ((a.p + kBK - 1) / kBK + 63) / 64;
  pl.rec = reinterpret_cast<int*>(reinterpret_cast<char*>(pl.masks) +
                                  align256(n_qt_max * n_kg_max * kMaskWords * sizeof(uint32_t)));
  pl.nfull = reinterpret_cast<int*>(reinterpret_cast<char*>(pl.rec) + align256(n_qt_max * kRecInts * sizeof(int)));
  const size_t n_kt_max = (size_t)(a.p + kBK - 1) / kBK;
  pl.vis = a.src == kSrcPacked
               ? reinterpret_cast<int*>(reinterpret_cast<char*>(pl.nfull) + align256(n_qt_max * sizeof(int)))
               : nullptr;
  (void)n_kt_max;
}

hipError_t prefill_prepare(const PrefillArgs& a, Plan& pl, hipStream_t stream, int waves) {
  prefill_layout(a, pl, waves);
  const int n_tiles = pl.n_kt + pl.n_qt;
  prefill_summarize_kernel<<<dim3((n_tiles + 3) / 4), dim3(256), 0, stream>>>(a, pl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_scan_kernel<<<dim3((pl.n_qt + 3) / 4), dim3(256), 0, stream>>>(a, pl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_order_kernel<<<1, kPrepThreads, 0, stream>>>(pl);
  return hipGetLastError();
}

hipError_t prefill_order(const Plan& pl, hipStream_t stream) {
  prefill_order_kernel<<<1, kPrepThreads, 0, stream>>>(pl);
  return hipGetLastError();
}

hipError_t prefill_summarize(const PrefillArgs& a, const Plan& pl, hipStream_t stream) {
  const int n_tiles = pl.n_kt + pl.n_qt;
  prefill_summarize_kernel<<<dim3((n_tiles + 3) / 4), dim3(256), 0, stream>>>(a, pl);
  return hipGetLastError();
}

template <int D, int GW>
static void launch_step(const PrefillArgs& a, const Plan& pl, const DecodeArgs& d,
                        hipStream_t stream) {
  const int n_groups = a.kv_heads * pl.head_groups;
  const int n_dec = d.rows * d.kv_heads;
  const int n_pre = pl.n_qt * n_groups;
  // The decode shares follow half the prefill tiles, at most three
  // workgroups per compute unit of them (1.5 residencies of two per CU).
  const int cus = device_cu_count();
  const int cap = 3 * (cus > 0 ? cus : 256);
  const int dec0 = n_pre / 2 < cap ? n_pre / 2 : cap;
  const dim3 grid(n_dec + n_pre), block(64 * prefill_waves<GW>());
  step_paged_kernel<D, GW><<<grid, block, 0, stream>>>(a, pl, d, n_dec, dec0);
}

hipError_t launch_prefill_step(const PrefillArgs& a, DecodeArgs d, hipStream_t stream) {
  d.split_len = d.cap;
  d.nsplit = 1;
  d.ws = nullptr;
  Plan pl;
  const hipError_t e = prefill_prepare(a, pl, stream);
  if (e != hipSuccess) return e;
  if (a.head_dim == 64) {
    if (pl.gw == 4) launch_step<64, 4>(a, pl, d, stream);
    else if (pl.gw == 2) launch_step<64, 2>(a, pl, d, stream);
    else launch_step<64, 1>(a, pl, d, stream);
  } else {
    if (pl.gw == 4) launch_step<128, 4>(a, pl, d, stream);
    else if (pl.gw == 2) launch_step<128, 2>(a, pl, d, stream);
    else launch_step<128, 1>(a, pl, d, stream);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_plan(const PrefillArgs& a, hipStream_t stream) {
  Plan pl;
  return prefill_prepare(a, pl, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream, bool planned) {
  Plan pl;
  if (planned) {
    prefill_layout(a, pl, 0);
  } else {
    const hipError_t e = prefill_prepare(a, pl, stream);
    if (e != hipSuccess) return e;
  }
  if (a.head_dim == 64) {
    if (pl.gw == 4) launch_main<64, 4>(a, pl, stream);
    else if (pl.gw == 2) launch_main<64, 2>(a, pl, stream);
    else launch_main<64, 1>(a, pl, stream);
  } else {
    if (pl.gw == 4) launch_main<128, 4>(a, pl, stream);
    else if (pl.gw == 2) launch_main<128, 2>(a, pl, stream);
    else launch_main<128, 1>(a, pl, stream);
  }
  return hipGetLastError();
}

}  // namespace gqa
