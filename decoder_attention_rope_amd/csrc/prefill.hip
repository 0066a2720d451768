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
//   between lanes. V is written to LDS transposed (dimension-major, XOR
//   swizzled) while it is staged, so the A operand V^T is one 16-byte LDS
//   read per lane.
// * K/V tiles of 64 keys are double-buffered in LDS: the global loads of the
//   next tile are in flight while the current tile is on the matrix cores.
// * Tiles that cannot hold an allowed key are skipped using per-tile
//   [min, max] summaries of segments and positions; tiles in which every pair
//   is allowed skip the per-element mask. The exact `own` predicate is
//   evaluated everywhere else, so any segment order or id is handled.
// * Three small prep kernels compute the per-tile summaries and each query
//   tile's visited key-tile range and cost (one wavefront per tile), then
//   order the query tiles costliest first (a counting sort); workgroup index i * n_groups + g maps KV head g to the
//   round-robin XCD g % 8, keeping one head's K/V in one XCD's L2.
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"

namespace gqa {

namespace {
constexpr int kBK = 64;       // keys per tile
constexpr int kPrepThreads = 1024;
constexpr float kNegInf = -__builtin_huge_valf();

struct TileSum {
  int seg_min, seg_max, pos_min, pos_max;
};

struct Plan {
  TileSum* ksum;   // [n_kt]
  TileSum* qsum;   // [n_qt]
  int2* qrange;    // [n_qt] first / last key tile to visit
  int* order;      // [n_qt] query tiles, costliest first
  int* cost;       // [n_qt] key tiles each query tile visits
  uint32_t* masks; // [n_qt][n_kg][4]: per group of 64 key tiles, a 64-bit
                   // "visit" mask then a 64-bit "every pair allowed" mask
  int n_kt, n_qt, n_kg, tq, head_groups, gw;
  int max_cost;    // costs are clamped to [0, max_cost] for the ordering
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Read-only views through the constant address space: the prep kernels wrote
// these arrays before this kernel started and nothing writes them during it,
// so workgroup-uniform reads may use scalar loads (they then stay out of the
// vector-memory wait counter that tracks the K/V tile loads).
typedef __attribute__((address_space(4))) const int ConstInt;
__device__ __forceinline__ int ld_const(const int* p, long long i) { return ((ConstInt*)p)[i]; }
__device__ __forceinline__ TileSum ld_const(const TileSum* p, int i) {
  const int* b = reinterpret_cast<const int*>(p + i);
  return TileSum{ld_const(b, 0), ld_const(b, 1), ld_const(b, 2), ld_const(b, 3)};
}

__device__ __forceinline__ bool tiles_meet(const TileSum& q, const TileSum& k, int window) {
  if (k.seg_max < q.seg_min || k.seg_min > q.seg_max) return false;
  if (k.pos_min > q.pos_max) return false;
  if (window > 0 && (long long)q.pos_min - (long long)k.pos_max >= window) return false;
  return true;
}

// Every (query, key) pair of the two tiles is allowed: one segment on both
// sides, every key position at or below every query position, all inside the
// window, and key tile kt holds 64 real keys.
__device__ __forceinline__ bool tiles_full(const TileSum& q, const TileSum& k, int kt, int p, int window) {
  return (kt + 1) * kBK <= p && q.seg_min == q.seg_max && k.seg_min == k.seg_max &&
         k.seg_min == q.seg_min && k.pos_max <= q.pos_min &&
         (window <= 0 || (long long)q.pos_max - (long long)k.pos_min < window);
}

}  // namespace

// ---------------------------------------------------------------------------
// Prep 1: per-tile [min, max] of segments and positions. One wavefront per
// tile: key tiles (64 tokens) first, then query tiles (tq tokens); lanes read
// consecutive tokens and reduce with shuffles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_summarize_kernel(PrefillArgs a, Plan pl) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ti = blockIdx.x * 4 + wave;
  if (ti >= pl.n_kt + pl.n_qt) return;
  const bool is_k = ti < pl.n_kt;
  const int len = is_k ? kBK : pl.tq;
  const int lo = is_k ? ti * kBK : (ti - pl.n_kt) * pl.tq;
  const int hi = min(a.p, lo + len);
  int smin = 0x7fffffff, smax = (int)0x80000000, pmin = 0x7fffffff, pmax = (int)0x80000000;
  for (int t = lo + lane; t < hi; t += 64) {
    const int sg = a.segments ? a.segments[t] : 0, ps = a.positions[t];
    smin = min(smin, sg);
    smax = max(smax, sg);
    pmin = min(pmin, ps);
    pmax = max(pmax, ps);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    smin = min(smin, __shfl_xor(smin, off, 64));
    smax = max(smax, __shfl_xor(smax, off, 64));
    pmin = min(pmin, __shfl_xor(pmin, off, 64));
    pmax = max(pmax, __shfl_xor(pmax, off, 64));
  }
  if (lane == 0) {
    const TileSum sum{smin, smax, pmin, pmax};
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
  int first = pl.n_kt, last = -1, cnt = 0;
  for (int g = 0; g < pl.n_kg; ++g) {
    const int kt = g * 64 + lane;
    bool meet = false, full = false;
    if (kt < pl.n_kt) {
      const TileSum k = pl.ksum[kt];
      meet = tiles_meet(q, k, a.window);
      full = meet && tiles_full(q, k, kt, a.p, a.window);
    }
    if (meet) {
      first = min(first, kt);
      last = max(last, kt);
      ++cnt;
    }
    const unsigned long long vm = __builtin_amdgcn_ballot_w64(meet);
    const unsigned long long fm = __builtin_amdgcn_ballot_w64(full);
    if (lane < 4) {
      const unsigned long long w = lane < 2 ? vm : fm;
      pl.masks[((size_t)qt * pl.n_kg + g) * 4 + lane] = (uint32_t)(w >> (32 * (lane & 1)));
    }
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
  }
}

// ---------------------------------------------------------------------------
// Prep 3 (one workgroup): query tiles ordered by cost, costliest first -- a
// counting sort (histogram, scan, scatter). The order among equal costs only
// affects scheduling, never results.
// ---------------------------------------------------------------------------
constexpr int kMaxCostBins = 4096;

__global__ __launch_bounds__(kPrepThreads) void prefill_order_kernel(Plan pl) {
  __shared__ int start[kMaxCostBins + 1];
  __shared__ int part[kPrepThreads];
  const int tid = threadIdx.x;
  const int nb = pl.max_cost + 1;  // costs 0 .. max_cost
  if (nb > kMaxCostBins) {
    for (int i = tid; i < pl.n_qt; i += kPrepThreads) pl.order[i] = i;
    return;
  }
  for (int i = tid; i < nb; i += kPrepThreads) start[i] = 0;
  __syncthreads();
  for (int i = tid; i < pl.n_qt; i += kPrepThreads) atomicAdd(&start[pl.max_cost - pl.cost[i]], 1);
  __syncthreads();
  // Exclusive scan over bins (bin b = cost max_cost - b, so costly tiles first):
  // each thread sums a run of bins, a block scan of the run sums, then the
  // runs are rewritten as exclusive offsets.
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
  for (int i = tid; i < pl.n_qt; i += kPrepThreads)
    pl.order[atomicAdd(&start[pl.max_cost - pl.cost[i]], 1)] = i;
}

// ---------------------------------------------------------------------------
// LDS layouts (byte offsets; every access below is conflict-free in the
// 64-bank, 4-byte-bank LDS of gfx950, where a 16-byte access is served 16
// lanes at a time and an 8-byte access 32 lanes at a time).
//   K tile   [64 rows][D], row stride 2 D + 16 bytes. Key r of the tile sits
//            in row kappa(r), so lane l reads row l % 32 (+32): the 16 rows
//            of a 16-lane group start 16 bytes apart modulo 256.
//   V^T tile [D rows][64 keys], row stride 144 bytes: the 16 rows a 16-lane
//            group reads start 16 bytes apart modulo 256, and the staging
//            threads of a 32-lane group write 16 key groups of 2 dimension
//            rows whose starts differ by 128 bytes modulo 256.
// With padded (not XOR-swizzled) rows every read address is one per-lane
// base plus a compile-time offset.
// ---------------------------------------------------------------------------
// Lanes l and l ^ 32 own the two key halves of one query column; these
// combine their values (one cross-half lane swap, no LDS round trip).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N - 1, unrolled at
// compile time (every index below selects registers, so none may be a
// runtime value).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Key row feeding accumulator row m of a 32-key block: bits 2 and 3 swapped.
__device__ __forceinline__ int kappa(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D>
struct Lds {
  static constexpr int kStride = 2 * D + 16;       // K row stride (bytes)
  static constexpr int vStride = 2 * kBK + 16;     // V^T row stride (bytes)
  static constexpr int kBytes = kBK * kStride;     // one K tile
  static constexpr int vBytes = D * vStride;       // one V^T tile
  static constexpr int kOff(int buf) { return buf * kBytes; }
  static constexpr int vOff(int buf) { return 2 * kBytes + buf * vBytes; }
  static constexpr int posOff(int buf) { return 2 * kBytes + 2 * vBytes + buf * 2 * kBK * 4; }
  static constexpr int segOff(int buf) { return posOff(buf) + kBK * 4; }
  static constexpr int total = posOff(2);
};

typedef __attribute__((address_space(3))) char LdsByte;
template <typename T>
__device__ __forceinline__ T lds_ld(const LdsByte* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_st(LdsByte* p, const T& v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}

// Buffer resource over one key tile of a [P, kv_heads, D] tensor, starting at
// head kh of the tile's first token and covering exactly its n_rows valid
// rows: loads past them return zeros (dword 3 = raw, untyped 32-bit access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, long long elem_off,
                                                            int n_rows, int row_bytes, int tail_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(base) + 2 * elem_off), (short)0,
      (n_rows - 1) * row_bytes + tail_bytes, 0x00020000);
}

template <int D, int GW, int SRC>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a, Plan pl) {
  constexpr int SUB = 4 / GW;   // query sub-tiles of 32 per workgroup
  constexpr int TQ = 32 * SUB;  // query tokens per workgroup
  constexpr int KS = D / 16;    // k-steps of QK^T over the head dim
  constexpr int MD = D / 32;    // 32-row blocks of O^T
  constexpr int LPR = D / 8;    // 16-byte chunks per key row
  constexpr int RPT = D / 32;   // key rows staged per thread
  constexpr int NA = kBK / RPT; // key groups of RPT rows
  static_assert(LPR * NA == 256, "staging covers the tile");
  using L = Lds<D>;

  __shared__ __attribute__((aligned(16))) char smem_raw[L::total];
  LdsByte* smem = (LdsByte*)smem_raw;

  const int G = a.heads / a.kv_heads;
  const int n_groups = a.kv_heads * pl.head_groups;
  const int wi = blockIdx.x / n_groups;
  const int grp = blockIdx.x % n_groups;
  const int kh = grp / pl.head_groups;
  const int hg = grp % pl.head_groups;
  // Tile indices are workgroup-uniform: keep them (and the summary loads that
  // depend on them) on the scalar unit.
  const int qt = __builtin_amdgcn_readfirstlane(ld_const(pl.order, wi));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  // Packed keys: positions are token positions in [0, 2^31), so the
  // difference of two fits in 32 bits and an unsigned compare tests
  // pos_k <= pos_q together with the window. Keys past P carry position
  // INT_MIN, which fails it.
  const uint32_t wlim = a.window > 0 ? (uint32_t)a.window : 0x80000000u;
  // Cache keys: this query sees key slots [my_lo, my_hi] of cache row my_seg
  // (empty for a row outside the cache).
  const int my_hi = (my_seg >= 0 && my_seg < a.cache_rows) ? min(my_pos, a.cap - 1) : -1;
  const int my_lo = a.window > 0 ? max(my_pos - a.window + 1, 0) : 0;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = load16(qg + ((long long)q_ld * a.heads + h) * D + ks * 16 + hf * 8);
  // Retire these loads before the loop: inside it the only vector loads in
  // flight are the next tile's, so the wait counters stay exact.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  asm volatile("" ::"v"(my_pos), "v"(my_seg));

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[md][r] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;

  int2 rng = make_int2(ld_const(reinterpret_cast<const int*>(pl.qrange), 2LL * qt),
                       ld_const(reinterpret_cast<const int*>(pl.qrange), 2LL * qt + 1));
  rng.x = __builtin_amdgcn_readfirstlane(rng.x);
  rng.y = __builtin_amdgcn_readfirstlane(rng.y);

  // Staging. K: thread (c, ar) loads 16-byte chunk c of key rows
  // ar * RPT + i (LPR consecutive lanes cover a row). V: thread (av, cv) with
  // the key group fastest, so the transposed LDS writes spread over the banks.
  const int row_bytes = SRC == kSrcPacked ? a.kv_heads * D * 2 : D * 2;
  const int kc = tid % LPR, ka = tid / LPR;
  const int va = tid % NA, vc = tid / NA;
  int k_goff[RPT], v_goff[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    k_goff[i] = (ka * RPT + i) * row_bytes + kc * 16;
    v_goff[i] = (va * RPT + i) * row_bytes + vc * 16;
  }
  const int k_wr = kappa(ka * RPT) * L::kStride + kc * 16;
  const int v_wr = 8 * vc * L::vStride + va * RPT * 2;
  const int k_rd = qn * L::kStride + hf * 16;
  const int v_rd = qn * L::vStride + hf * 16;
  u32x4 kreg[RPT], vreg[RPT];
  int pos_reg = 0, seg_reg = 0, staged_rows = 0;

  // A key tile: tile index kt (64 keys) of cache row r, at pool page `page`.
  struct TileRef {
    int kt, r, page, rows;  // rows: cache slots of the tile anyone may see
  };
  auto load_tile = [&](TileRef t) {
    const int kt = t.kt;
    if constexpr (SRC != kSrcPacked) {
      // 64 key slots of one cache plane (contiguous rows of D elements).
      const int n_rows = t.rows;
      const long long e0 = SRC == kSrcPaged
                               ? ((long long)t.page * a.kv_heads + kh) * kBK * D
                               : (((long long)t.r * a.kv_heads + kh) * a.cap + (long long)kt * kBK) * D;
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(a.k, e0, n_rows, row_bytes, 2 * D);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(a.v, e0, n_rows, row_bytes, 2 * D);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_goff[i], 0, 0);
        vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_goff[i], 0, 0);
      }
      return;
    }
    const int n_rows = min(kBK, P - kt * kBK);
    const long long e0 = (long long)kt * kBK * a.kv_heads * D + (long long)kh * D;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(a.k, e0, n_rows, row_bytes, 2 * D);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(a.v, e0, n_rows, row_bytes, 2 * D);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_goff[i], 0, 0);
      vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_goff[i], 0, 0);
    }
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.positions + (long long)kt * kBK), (short)0, 4 * n_rows, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.segments + (long long)kt * kBK), (short)0, 4 * n_rows, 0x00020000);
    const int lo = (tid & (kBK - 1)) * 4;
    pos_reg = __builtin_amdgcn_raw_buffer_load_b32(rp, lo, 0, 0);
    seg_reg = __builtin_amdgcn_raw_buffer_load_b32(rs, lo, 0, 0);
    staged_rows = n_rows;
  };

  // Walk the visited key tiles with the prepared masks: scalar bit scans,
  // one scalar load per group of 64 key tiles. Phase 0 visits the tiles in
  // which every pair is allowed, phase 1 the others (the online softmax does
  // not depend on the order of the key tiles), so each phase runs one
  // specialized loop body.
  int vis_g = -1;
  unsigned long long vis_m = 0, full_m = 0;
  auto next_in = [&](int kt, int phase) {
    while (kt <= rng.y) {
      const int g = kt >> 6;
      if (g != vis_g) {
        const int* w = reinterpret_cast<const int*>(pl.masks) + ((long long)qt * pl.n_kg + g) * 4;
        vis_m = (unsigned long long)(uint32_t)ld_const(w, 0) | ((unsigned long long)(uint32_t)ld_const(w, 1) << 32);
        full_m = (unsigned long long)(uint32_t)ld_const(w, 2) | ((unsigned long long)(uint32_t)ld_const(w, 3) << 32);
        vis_g = g;
      }
      const unsigned long long m = (phase == 0 ? full_m : (vis_m & ~full_m)) >> (kt & 63);
      if (m != 0) return __builtin_amdgcn_readfirstlane(kt + (int)__builtin_ctzll(m));
      kt = (g + 1) << 6;
    }
    return rng.y + 1;
  };
  auto advance = [&](int kt, int& phase) {
    int r = next_in(kt, phase);
    if (r > rng.y && phase == 0) {
      phase = 1;
      r = next_in(rng.x, 1);
    }
    return r;
  };

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
  unsigned long long lead0 = 0, lead1 = 0;
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
    __syncthreads();
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
  }
  const int n_lead = __builtin_popcountll(lead0) + __builtin_popcountll(lead1);
  const bool c_single = n_lead == 1;
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
  // Page ids of 64 consecutive key tiles of one table row, one per lane.
  int tab_row = -1, tab_base = 0, tab_v = -1;
  auto page_of = [&](int r, int kt) {
    if (r != tab_row || kt < tab_base || kt >= tab_base + 64) {
      tab_row = r;
      tab_base = kt & ~63;
      const int idx = tab_base + lane;
      tab_v = idx < a.table_pages ? a.table[(long long)r * a.table_pages + idx] : -1;
    }
    return __builtin_amdgcn_readlane(tab_v, kt - tab_base);
  };
  bool c_started = false;
  auto cache_next = [&](int& phase) {
    TileRef t{-1, 0, 0, 0};
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
      t = TileRef{kt, c_row, page, min(kBK, c_last - kt * kBK + 1)};
      break;
    }
    phase = c_phase;
    t.kt = __builtin_amdgcn_readfirstlane(t.kt);
    t.r = __builtin_amdgcn_readfirstlane(t.r);
    t.page = __builtin_amdgcn_readfirstlane(t.page);
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    return t;
  };

  // One tile is 4 C matrix steps in four blocks (C = D / 16):
  //   block 0  S^T for keys 0..31        (one accumulator chain)
  //   block 1  S^T for keys 32..63       with the softmax of keys 0..31
  //   block 2  P.V of keys 0..31         with the softmax of keys 32..63
  //   block 3  P.V of keys 32..63        with the staging of the next tile
  // On gfx950 a SIMD overlaps an MFMA with vector instructions of the same
  // wavefront issued in its shadow (not with another wave's), so each step
  // issues one MFMA followed by a slice of vector work, and a scheduling
  // fence keeps that order. Matrix operands are read from LDS four steps
  // ahead through a ring of registers. The O rescales of the lazy softmax
  // (rare) sit between blocks 1 and 2 and between blocks 2 and 3.
  constexpr int C = D / 16;
  static_assert(KS == C && 2 * MD == C, "step counts");
  u32x4 pw[4];
  f32x16 s[2];
  bf16x8 ring[4];
  float tmax = kNegInf, m_use = 0.f, alpha = 1.f, psum = 0.f;

  // Operand of matrix step st (0 <= st < 4 C) of the tile in kb / vb.
  auto operand = [&](const LdsByte* kb, const LdsByte* vb, auto stc) {
    constexpr int st = decltype(stc)::value;
    if constexpr (st < 2 * C) {
      constexpr int hb = st / C, ks = st % C;
      return lds_ld<bf16x8>(kb + hb * 32 * L::kStride + ks * 32);
    } else {
      constexpr int hb = (st - 2 * C) / C, j = (st - 2 * C) % C;
      constexpr int ks = 2 * hb + j / MD, md = j % MD;
      return lds_ld<bf16x8>(vb + 32 * md * L::vStride + ks * 32);
    }
  };
  auto mfma_step = [&](auto stc, const bf16x8& op) {
    constexpr int st = decltype(stc)::value;
    if constexpr (st < 2 * C) {
      constexpr int hb = st / C, ks = st % C;
      if constexpr (ks == 0)
        s[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, __builtin_bit_cast(bf16x8, qf[ks]), f32x16{}, 0, 0, 0);
      else
        s[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, __builtin_bit_cast(bf16x8, qf[ks]), s[hb], 0, 0, 0);
    } else {
      constexpr int hb = (st - 2 * C) / C, j = (st - 2 * C) % C;
      constexpr int ks = 2 * hb + j / MD, md = j % MD;
      o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, __builtin_bit_cast(bf16x8, pw[ks]), o[md], 0, 0, 0);
    }
  };

  // Slice c (0 <= c < C) of the mask and online-softmax update of one 32-key
  // half (accumulator s[hb]): slice 0 masks and takes the row max, slice 1
  // moves the lazy reference, slices 2 .. C - 1 turn pairs of scores into
  // bf16 probabilities (pw[2 hb], pw[2 hb + 1], the B operands of P.V).
  auto soft_slice = [&](const LdsByte* pb, int lo_j, int hi_j, auto hbc, auto cc, auto fullc) {
    constexpr bool full = decltype(fullc)::value;
    constexpr int hb = decltype(hbc)::value;
    constexpr int c = decltype(cc)::value;
    if constexpr (c == 0) {
      if constexpr (!full) {
        // The literal own predicate (and the window) per element.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 32 * hb + 16 * (r >> 3) + 8 * hf + (r & 7);
          bool ok;
          if constexpr (SRC == kSrcPacked) {
            const int kp = lds_ld<int>(pb + j * 4);
            const int ksg = lds_ld<int>(pb + kBK * 4 + j * 4);
            ok = (ksg == my_seg) & ((uint32_t)my_pos - (uint32_t)kp < wlim);
          } else {
            // Key slot kt * 64 + j of the tile's row.
            ok = (j >= lo_j) & (j <= hi_j);
          }
          s[hb][r] = ok ? s[hb][r] : kNegInf;
        }
      }
      tmax = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[hb][r]);
    } else if constexpr (c == 1) {
      // Online softmax in the log2 domain. scale > 0, so the row max of the
      // scaled scores is the scaled row max of the raw ones; m_run is the
      // lazy reference (see kLazyMaxLog2).
      tmax = pair_max(tmax) * a.scale_log2;
      const float m_new = (tmax > m_run + kLazyMaxLog2) ? tmax : m_run;
      m_use = (m_new == kNegInf) ? 0.f : m_new;
      alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      psum = 0.f;
    } else {
      constexpr int q0 = 8 * (c - 2) / (C - 2), q1 = 8 * (c - 1) / (C - 2);
      static_for<q1 - q0>([&](auto qc) {
        constexpr int r = 2 * (q0 + decltype(qc)::value);
        const float p0 = fast_exp2(__builtin_fmaf(s[hb][r], a.scale_log2, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s[hb][r + 1], a.scale_log2, -m_use));
        psum += p0 + p1;
        pw[2 * hb + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
        // Materialize here: without the anchor the compiler sinks this work
        // past the rescale branch, next to its use, out of the MFMA shadow.
        asm volatile("" ::"v"(pw[2 * hb + (r >> 3)][(r & 7) >> 1]));
      });
      if constexpr (c == C - 1) l_run = l_run * alpha + psum;
    }
  };

  // Rescale O only when some lane's reference moved.
  auto rescale = [&](float f) {
    if (__builtin_amdgcn_ballot_w64(f != 1.f) != 0) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= f;
    }
  };

  // Slice c of staging the next tile (registers -> LDS buffer nb).
  auto store_slice = [&](int nb, auto cc) {
    constexpr int c = decltype(cc)::value;
    LdsByte* kbw = smem + nb * L::kBytes;
    LdsByte* vbw = smem + 2 * L::kBytes + nb * L::vBytes;
    if constexpr (c == 0) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) lds_st(kbw + k_wr + i * L::kStride, kreg[i]);
    }
    constexpr int e0 = (c == 0 || c == C - 1) ? 0 : 8 * (c - 1) / (C - 2);
    constexpr int e1 = (c == 0 || c == C - 1) ? 0 : 8 * c / (C - 2);
    static_for<e1 - e0>([&](auto ec) {
      constexpr int e = e0 + decltype(ec)::value;
      constexpr int w = e >> 1;
      LdsByte* dst = vbw + v_wr + e * L::vStride;
      if (RPT == 4) {
        u32x2 pk;
        pk[0] = (e & 1) ? pack_hi16(vreg[0][w], vreg[1 % RPT][w]) : pack_lo16(vreg[0][w], vreg[1 % RPT][w]);
        pk[1] = (e & 1) ? pack_hi16(vreg[2 % RPT][w], vreg[3 % RPT][w])
                        : pack_lo16(vreg[2 % RPT][w], vreg[3 % RPT][w]);
        lds_st(dst, pk);
      } else {
        lds_st(dst, (e & 1) ? pack_hi16(vreg[0][w], vreg[1 % RPT][w]) : pack_lo16(vreg[0][w], vreg[1 % RPT][w]));
      }
    });
    if (SRC == kSrcPacked && c == C - 1 && tid < kBK) {
      // Applied here, once the loads have landed, not at issue time.
      LdsByte* pbw = smem + L::posOff(nb);
      lds_st(pbw + tid * 4, tid < staged_rows ? pos_reg : (int)0x80000000);
      lds_st(pbw + kBK * 4 + tid * 4, seg_reg);
    }
  };

  // The first tile, then the iteration: phase 0 (every pair allowed) and
  // phase 1 (masked) tiles in turn.
  auto first_tile = [&](int& phase) {
    if constexpr (SRC == kSrcPacked) {
      phase = 0;
      return TileRef{advance(rng.x, phase), 0, 0, 0};
    } else {
      return cache_next(phase);
    }
  };
  auto next_tile = [&](TileRef cur, int& phase) {
    if constexpr (SRC == kSrcPacked) {
      return TileRef{advance(cur.kt + 1, phase), 0, 0, 0};
    } else {
      return cache_next(phase);
    }
  };
  auto valid = [&](TileRef t) { return SRC == kSrcPacked ? t.kt <= rng.y : t.kt >= 0; };

  int phase = 0;
  TileRef cur = first_tile(phase);
  int buf = 0;
  if (valid(cur)) {
    load_tile(cur);
    static_for<C>([&](auto cc) { store_slice(0, cc); });
  }
  __syncthreads();

  // One tile from LDS buffer buf (every pair allowed when FULL). The next
  // tile's global loads fly during the whole tile; its LDS buffer (buf ^ 1)
  // was last read before the previous barrier. When there is no next tile
  // the staging writes stale registers into that buffer, which nothing
  // reads again.
  auto tile = [&](auto fullc, TileRef t) {
    const LdsByte* kb = smem + buf * L::kBytes + k_rd;
    const LdsByte* vb = smem + 2 * L::kBytes + buf * L::vBytes + v_rd;
    const LdsByte* pb = smem + L::posOff(buf);
    // Cache keys: this lane's visible slots relative to the tile.
    const int lo_j = my_lo - t.kt * kBK;
    const int hi_j = (t.r == my_seg ? my_hi : -1) - t.kt * kBK;
    static_for<4>([&](auto stc) { ring[decltype(stc)::value] = operand(kb, vb, stc); });
    static_for<4 * C>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      if constexpr (st == 2 * C || st == 3 * C) rescale(alpha);
      mfma_step(stc, ring[st & 3]);
      if constexpr (st + 4 < 4 * C) ring[st & 3] = operand(kb, vb, std::integral_constant<int, st + 4>{});
      if constexpr (st >= C && st < 2 * C)
        soft_slice(pb, lo_j, hi_j, std::integral_constant<int, 0>{}, std::integral_constant<int, st - C>{}, fullc);
      if constexpr (st >= 2 * C && st < 3 * C)
        soft_slice(pb, lo_j, hi_j, std::integral_constant<int, 1>{}, std::integral_constant<int, st - 2 * C>{},
                   fullc);
      if constexpr (st >= 3 * C) store_slice(buf ^ 1, std::integral_constant<int, st - 3 * C>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    __syncthreads();
    buf ^= 1;
  };
  while (valid(cur) && phase == 0) {
    int nphase = phase;
    const TileRef nxt = next_tile(cur, nphase);
    if (valid(nxt)) load_tile(nxt);
    tile(std::true_type{}, cur);
    cur = nxt;
    phase = nphase;
  }
  while (valid(cur)) {
    int nphase = 1;
    const TileRef nxt = next_tile(cur, nphase);
    if (valid(nxt)) load_tile(nxt);
    tile(std::false_type{}, cur);
    cur = nxt;
  }

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

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static int group_width(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1; }

size_t prefill_workspace_bytes(int p, int heads, int kv_heads, int head_dim) {
  (void)heads;
  (void)kv_heads;
  (void)head_dim;
  const size_t n_kt = (size_t)(p + kBK - 1) / kBK;
  const size_t n_qt = (size_t)(p + 31) / 32;  // the smallest query tile
  const size_t n_kg = (n_kt + 63) / 64;
  return align256(n_kt * sizeof(TileSum)) + align256(n_qt * sizeof(TileSum)) +
         align256(n_qt * sizeof(int2)) + 2 * align256(n_qt * sizeof(int)) +
         align256(n_qt * n_kg * 4 * sizeof(uint32_t));
}

template <int D, int GW>
static void launch_main(const PrefillArgs& a, const Plan& pl, hipStream_t stream) {
  const int n_groups = a.kv_heads * pl.head_groups;
  const dim3 grid(pl.n_qt * n_groups), block(256);
  if (a.src == kSrcContiguous) prefill_kernel<D, GW, kSrcContiguous><<<grid, block, 0, stream>>>(a, pl);
  else if (a.src == kSrcPaged) prefill_kernel<D, GW, kSrcPaged><<<grid, block, 0, stream>>>(a, pl);
  else prefill_kernel<D, GW, kSrcPacked><<<grid, block, 0, stream>>>(a, pl);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.heads / a.kv_heads;
  Plan pl;
  pl.gw = group_width(G);
  pl.head_groups = G / pl.gw;
  pl.tq = 32 * (4 / pl.gw);
  // Cache keys need no key-tile summaries or masks.
  pl.n_kt = a.src == kSrcPacked ? (a.p + kBK - 1) / kBK : 0;
  pl.n_qt = (a.p + pl.tq - 1) / pl.tq;
  pl.max_cost = a.src == kSrcPacked ? pl.n_kt : min(kMaxCostBins - 1, a.cap / kBK + 1);
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

  const int n_tiles = pl.n_kt + pl.n_qt;
  prefill_summarize_kernel<<<dim3((n_tiles + 3) / 4), dim3(256), 0, stream>>>(a, pl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_scan_kernel<<<dim3((pl.n_qt + 3) / 4), dim3(256), 0, stream>>>(a, pl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_order_kernel<<<1, kPrepThreads, 0, stream>>>(pl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
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
