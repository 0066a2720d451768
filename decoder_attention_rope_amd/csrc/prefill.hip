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
#include "common.h"
#include "internal.h"

namespace gqa {

namespace {
constexpr int kBK = 64;       // keys per tile
constexpr int kPrepThreads = 1024;
constexpr float kNegInf = -__builtin_huge_valf();
#ifndef GQA_PREFILL_SETPRIO
#define GQA_PREFILL_SETPRIO 0
#endif

struct TileSum {
  int seg_min, seg_max, pos_min, pos_max;
};

struct Plan {
  TileSum* ksum;  // [n_kt]
  TileSum* qsum;  // [n_qt]
  int2* qrange;   // [n_qt] first / last key tile to visit
  int* order;     // [n_qt] query tiles, costliest first
  int* cost;      // [n_qt] key tiles each query tile visits
  int n_kt, n_qt, tq, head_groups, gw;
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
    const int sg = a.segments[t], ps = a.positions[t];
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
// Prep 2: each query tile's visited key-tile range and cost, one wavefront per
// query tile (the lanes test 64 key tiles at a time and reduce).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_scan_kernel(PrefillArgs a, Plan pl) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int qt = blockIdx.x * 4 + wave;
  if (qt >= pl.n_qt) return;
  const TileSum q = pl.qsum[qt];
  int first = pl.n_kt, last = -1, cnt = 0;
  for (int kt = lane; kt < pl.n_kt; kt += 64) {
    if (tiles_meet(q, pl.ksum[kt], a.window)) {
      first = min(first, kt);
      last = max(last, kt);
      ++cnt;
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
  const int nb = pl.n_kt + 1;  // costs 0 .. n_kt
  if (nb > kMaxCostBins) {
    for (int i = tid; i < pl.n_qt; i += kPrepThreads) pl.order[i] = i;
    return;
  }
  for (int i = tid; i < nb; i += kPrepThreads) start[i] = 0;
  __syncthreads();
  for (int i = tid; i < pl.n_qt; i += kPrepThreads) atomicAdd(&start[pl.n_kt - pl.cost[i]], 1);
  __syncthreads();
  // Exclusive scan over bins (bin b = cost n_kt - b, so costly tiles first):
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
    pl.order[atomicAdd(&start[pl.n_kt - pl.cost[i]], 1)] = i;
}

// ---------------------------------------------------------------------------
// LDS layouts.
//   K tile  [64 keys][D]: 16-byte granule g of row r stored at granule
//           g ^ swk(r); the rows a group of lanes reads at once land in
//           distinct bank groups.
//   V^T tile [D][64 keys]: granule g (8 keys) of row d stored at g ^ swv(d).
// ---------------------------------------------------------------------------
// Key row feeding accumulator row m of a 32-key block: bits 2 and 3 swapped.
__device__ __forceinline__ int kappa(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// K granule swizzle. D = 128 (16 granules per row): kappa of the row's low 4
// bits, so the 16 rows that 16 consecutive lanes read for one operand hit 16
// distinct granules (and any 8 consecutive lanes 8 distinct granules mod 8).
// D = 64 (8 granules): the 8 rows of 8 consecutive lanes hit 8 granules.
template <int D>
__device__ __forceinline__ int swk(int row) {
  return D == 128 ? kappa(row & 15) : ((row & 3) | ((row >> 1) & 4));
}
__device__ __forceinline__ int swv(int d) { return (d + (d >> 3)) & 7; }
template <int D, int GW>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a, Plan pl) {
  constexpr int SUB = 4 / GW;   // query sub-tiles of 32 per workgroup
  constexpr int TQ = 32 * SUB;  // query tokens per workgroup
  constexpr int KS = D / 16;    // k-steps of QK^T over the head dim
  constexpr int MD = D / 32;    // 32-row blocks of O^T
  constexpr int LPR = D / 8;    // staging threads per key row (16 B each)
  constexpr int RPT = D / 32;   // key rows staged per thread
  static_assert(LPR * (kBK / RPT) == 256, "staging covers the tile");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBK * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * kBK];
  __shared__ __attribute__((aligned(16))) int sPos[2][kBK];
  __shared__ __attribute__((aligned(16))) int sSeg[2][kBK];

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
  const int my_seg = a.segments[q_ld];
  const int window = a.window;

  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* vg = static_cast<const uint16_t*>(a.v);

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
  const TileSum qs = ld_const(pl.qsum, qt);

  // Staging of one K/V tile: thread (c, ar) loads 16-byte chunk c of key rows
  // ar * RPT .. ar * RPT + RPT - 1 (LPR threads cover a row, so a wavefront
  // reads whole rows).
  const int sc_c = tid % LPR;
  const int sc_a = tid / LPR;
  u32x4 kreg[RPT], vreg[RPT];
  int pos_reg = 0, seg_reg = 0;

  auto load_tile = [&](int kt) {
    // Keys past P read row P - 1 (a real row); the mask drops them and
    // their probability is exactly 0.
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int key = min(kt * kBK + sc_a * RPT + i, P - 1);
      const long long off = ((long long)key * a.kv_heads + kh) * D + sc_c * 8;
      kreg[i] = load16(kg + off);
      vreg[i] = load16(vg + off);
    }
    const int pkey = min(kt * kBK + (tid & (kBK - 1)), P - 1);
    pos_reg = a.positions[pkey];
    seg_reg = a.segments[pkey];
  };

  auto store_tile = [&](int buf) {
    uint16_t* k_s = sK[buf];
    uint16_t* v_s = sV[buf];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = sc_a * RPT + i;
      store16(k_s + row * D + ((sc_c ^ swk<D>(row)) * 8), kreg[i]);
    }
    const int key0 = sc_a * RPT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = sc_c * 8 + e;
      const int w = e >> 1;
      uint16_t* dst = v_s + d * kBK + ((((key0 >> 3) ^ swv(d)) << 3) | (key0 & 7));
      if (RPT == 4) {
        u32x2 pk;
        pk[0] = (e & 1) ? pack_hi16(vreg[0][w], vreg[1 % RPT][w]) : pack_lo16(vreg[0][w], vreg[1 % RPT][w]);
        pk[1] = (e & 1) ? pack_hi16(vreg[2 % RPT][w], vreg[3 % RPT][w])
                        : pack_lo16(vreg[2 % RPT][w], vreg[3 % RPT][w]);
        *reinterpret_cast<u32x2*>(dst) = pk;
      } else {
        *reinterpret_cast<uint32_t*>(dst) =
            (e & 1) ? pack_hi16(vreg[0][w], vreg[1 % RPT][w]) : pack_lo16(vreg[0][w], vreg[1 % RPT][w]);
      }
    }
    if (tid < kBK) {
      sPos[buf][tid] = pos_reg;
      sSeg[buf][tid] = seg_reg;
    }
  };

  auto visit = [&](int kt) { return tiles_meet(qs, ld_const(pl.ksum, kt), window); };
  auto next_visit = [&](int kt) {
    while (kt <= rng.y && !visit(kt)) ++kt;
    return __builtin_amdgcn_readfirstlane(kt);
  };

  // S^T = K Q^T over the tile's 64 keys (two independent accumulator chains,
  // interleaved so consecutive matrix ops do not depend on each other).
  u32x4 pw[4];
  f32x16 s[2];
  auto qk = [&](int buf) {
    const uint16_t* k_s = sK[buf];
    const int row0 = kappa(qn), row1 = kappa(qn) + 32;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
    // Matrix bursts run at raised wave priority, so the other wavefront on
    // the SIMD fills the gaps with its softmax instead of competing.
    if (GQA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(
          k_s + row0 * D + (((2 * ks + hf) ^ swk<D>(row0)) * 8));
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(
          k_s + row1 * D + (((2 * ks + hf) ^ swk<D>(row1)) * 8));
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, __builtin_bit_cast(bf16x8, qf[ks]), s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, __builtin_bit_cast(bf16x8, qf[ks]), s[1], 0, 0, 0);
    }
    if (GQA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };

  // Mask, online-softmax update; leaves the bf16 probabilities in pw (the B
  // operand of the P.V product) and rescales the O accumulator.
  auto softmax = [&](int buf, int kt) {
    const TileSum ks_ = ld_const(pl.ksum, kt);
    const bool full = (kt + 1) * kBK <= P && qs.seg_min == qs.seg_max &&
                      ks_.seg_min == ks_.seg_max && ks_.seg_min == qs.seg_min &&
                      ks_.pos_max <= qs.pos_min &&
                      (window <= 0 || (long long)qs.pos_max - (long long)ks_.pos_min < window);
    if (!full) {
      // The literal own predicate (and the window) per element, branch-free.
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 32 * mb + 16 * (r >> 3) + 8 * hf + (r & 7);
          const int kp = sPos[buf][j];
          const int ksg = sSeg[buf][j];
          const bool ok = (kt * kBK + j < P) & (ksg == my_seg) & (kp <= my_pos) &
                          ((window <= 0) | ((uint32_t)my_pos - (uint32_t)kp < (uint32_t)window));
          s[mb][r] = ok ? s[mb][r] : kNegInf;
        }
      }
    }
    // Online softmax in the log2 domain. scale > 0, so the row max of the
    // scaled scores is the scaled row max of the raw ones.
    float tmax = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[mb][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * a.scale_log2;
    // m_run is the lazy reference (see kLazyMaxLog2).
    const float m_new = (tmax > m_run + kLazyMaxLog2) ? tmax : m_run;
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[mb][r], a.scale_log2, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s[mb][r + 1], a.scale_log2, -m_use));
        psum += p0 + p1;
        pw[2 * mb + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // Rescale O only when some lane's reference moved.
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= alpha;
    }
  };

  // O^T += V^T P^T over the tile's 64 keys (MD independent chains).
  auto pv = [&](int buf) {
    const uint16_t* v_s = sV[buf];
    if (GQA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 av[MD];
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int d = 32 * md + qn;
        av[md] = *reinterpret_cast<const bf16x8*>(v_s + d * kBK + (((2 * ks + hf) ^ swv(d)) * 8));
      }
#pragma unroll
      for (int md = 0; md < MD; ++md)
        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[md], __builtin_bit_cast(bf16x8, pw[ks]),
                                                        o[md], 0, 0, 0);
    }
    if (GQA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };

  int cur = next_visit(rng.x);
  if (cur <= rng.y) {
    load_tile(cur);
    store_tile(0);
  }
  __syncthreads();
  int buf = 0;
  while (cur <= rng.y) {
    const int nxt = next_visit(cur + 1);
    qk(buf);
    // The next tile's global loads fly during the softmax and P.V; its LDS
    // buffer was last read before the previous barrier.
    if (nxt <= rng.y) load_tile(nxt);
    softmax(buf, cur);
    pv(buf);
    if (nxt <= rng.y) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    cur = nxt;
  }

  // Normalize; the sink logit joins the denominator.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
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
  return align256(n_kt * sizeof(TileSum)) + align256(n_qt * sizeof(TileSum)) +
         align256(n_qt * sizeof(int2)) + 2 * align256(n_qt * sizeof(int));
}

template <int D, int GW>
static void launch_main(const PrefillArgs& a, const Plan& pl, hipStream_t stream) {
  const int n_groups = a.kv_heads * pl.head_groups;
  prefill_kernel<D, GW><<<dim3(pl.n_qt * n_groups), dim3(256), 0, stream>>>(a, pl);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int G = a.heads / a.kv_heads;
  Plan pl;
  pl.gw = group_width(G);
  pl.head_groups = G / pl.gw;
  pl.tq = 32 * (4 / pl.gw);
  pl.n_kt = (a.p + kBK - 1) / kBK;
  pl.n_qt = (a.p + pl.tq - 1) / pl.tq;
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
