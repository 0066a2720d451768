// Backward of the packed prefill attention on bf16 matrix cores (gfx950).
//
// `packed<P>` of the Linnet "examples/01-llama" page (src/attention.linnet)
// is trained through the model's `loss_packed` entry (the same page's model
// source): token i attends key j iff segments[i] == segments[j] &&
// positions[j] <= positions[i] (and the window). The gradients of
// sum(dout * out) follow from the chain rule through the softmax: with
// p_ij = exp(s_ij - lse_i), s_ij = scale <q_i, k_j>, dp_ij = <dout_i, v_j>
// and delta_i = <dout_i, out_i> (= sum_j p_ij dp_ij):
//   dv_j = sum_i p_ij dout_i,   ds_ij = p_ij (dp_ij - delta_i),
//   dq_i = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i,
// a KV head's dk, dv summed over the query heads that read it.
//
// Design: the forward stores lse (natural-log softmax denominators), so the
// backward never renormalizes. Three kernels after the forward's prepared
// walk:
// * delta: one pass over out and dout (and lse, rewritten in base-2 units).
// * dQ, one workgroup per query tile and group of query heads, as the
//   forward: for each visited key tile, S^T = K Q^T and dP^T = V dO^T on the
//   32x32x16 bf16 MFMA (K and V rows the A operands, q and dout in
//   registers), P and dS in the accumulator layout (a lane owns one query),
//   then dQ^T += K^T dS^T with K^T read from the same LDS tile by transposing
//   8-byte reads (the key order inside a 32-key block is permuted as in the
//   forward, so dS packs straight into the B operand).
// * dK / dV, one workgroup per key tile and KV head, in producer / consumer
//   wavefront pairs: a producer owns 32 keys (K^T and V^T as B operands in
//   registers) and every other (query tile, head) pair; S = Q K^T and
//   dP = dO V^T put a lane on one key, and it passes P and dS through LDS.
//   Its consumer accumulates dV^T += dO^T P and dK^T += Q^T dS with dO^T
//   and Q^T read transposed from LDS. The consumers of a key half add their
//   sums at the end.
// Query, dout, K and V tiles go from memory straight into LDS (row r of a
// 32-row block holding entity kappa(r)), ahead of the matrix work, in
// unpadded rows with XOR-swizzled 16-byte chunks (they are read both
// row-wise and transposed).
#include "attn_tiles.h"
#include "common.h"
#include "internal.h"

namespace gqa {

namespace {
constexpr float kLog2eB = 1.4426950408889634f;

// Swizzled LDS tile of rows of D bf16 values (the dK/dV kernel's Q and dout
// tiles, the dQ kernel's K and V tiles): row stride 2 D bytes, 16-byte chunk
// c of row r stored at chunk c ^ swz(r). Rows are read two ways: 16 lanes
// reading one chunk of 16 consecutive rows (row-wise operands of S and dP),
// and 32 lanes reading 4
// consecutive rows (aligned to 4) x 64 bytes (transposing reads); swz makes
// both touch every bank once (D = 128: one row is one pass over the 64
// banks; D = 64: two rows are).
template <int D>
struct ST {
  static constexpr int kStride = 2 * D;
  static constexpr int kChunks = D / 8;
  static constexpr int loads(int rows) { return rows * kChunks / 64; }
  static constexpr int bytes(int rows) { return rows * kStride; }
  __device__ static __forceinline__ int swz(int r) {
    return D >= 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};
// Source offset of slot p (16-byte LDS chunk) of a swizzled tile whose row r
// holds row kappa(r) of a [*, row_bytes] tensor; rows at or past `rows`
// fetch out of range.
template <int D>
__device__ __forceinline__ int swz_off(int p, int rows, int row_bytes) {
  const int row = p / ST<D>::kChunks, pc = p % ST<D>::kChunks;
  const int src = kappa(row);
  return src >= rows ? 0x40000000 : src * row_bytes + ((pc ^ ST<D>::swz(row)) << 4);
}
// A^T operand (32 dimension rows x 16 entity columns) of a transposed
// product: two transposing reads of 4 entities each. Lane l of group
// g = l / 16 supplies the address of LDS row 4 (g / 2) + (l % 16) / 4 (+8 for
// the second read), dimensions 32 md + 16 (g % 2) + 4 (l % 4) .. +3; rows
// hold entities kappa(row), which keeps every group of 4 entities in 4
// consecutive rows. Step kk adds 16 rows, which leaves swz unchanged, so the
// per-lane offsets are computed once.
template <int D>
__device__ __forceinline__ void swz_tr_offs(int lane, int (*off)[2]) {
  constexpr int MD = D / 32;
  const int g = lane >> 4, s = lane & 15;
  const int r0 = 4 * (g >> 1) + (s >> 2);
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    const int c = 4 * md + 2 * (g & 1) + ((s & 3) >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = r0 + 8 * h;
      off[md][h] = r * ST<D>::kStride + ((c ^ ST<D>::swz(r)) << 4) + 8 * (s & 1);
    }
  }
}
template <int D>
__device__ __forceinline__ bf16x8 swz_tr_operand(const LdsByte* tile, const int (*off)[2], int kk, int md) {
  const LdsByte* p = tile + 16 * kk * ST<D>::kStride;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p + off[md][0]));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p + off[md][1]));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Workgroup barrier that neither waits for loads in flight nor lets the
// compiler move memory accesses across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0xF70); }

}  // namespace

// ---------------------------------------------------------------------------
// delta[i, h] = <dout[i, h, :], out[i, h, :]> in f32; D / 8 lanes per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a, float* delta, float* lse2) {
  const int cpr = a.head_dim / 8;  // 16-byte chunks per row (8 or 16)
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)a.p * a.heads * cpr;
  float acc = 0.f;
  if (idx < total) {
    const u32x4 o = load16(static_cast<const uint16_t*>(a.out) + idx * 8);
    const u32x4 g = load16(static_cast<const uint16_t*>(a.dout) + idx * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(bf16_to_f32((uint16_t)(o[w] & 0xffff)), bf16_to_f32((uint16_t)(g[w] & 0xffff)), acc);
      acc = __builtin_fmaf(bf16_to_f32((uint16_t)(o[w] >> 16)), bf16_to_f32((uint16_t)(g[w] >> 16)), acc);
    }
  }
  for (int off = 1; off < cpr; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (idx < total && (threadIdx.x & (cpr - 1)) == 0) {
    delta[idx / cpr] = acc;
    lse2[idx / cpr] = a.lse[idx / cpr] * kLog2eB;  // lse in base-2 units, for the dK/dV kernel
  }
}

// ---------------------------------------------------------------------------
// Per key tile, the first and last 32-token query tile that can meet it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_krange_kernel(BwdArgs a, Plan qp, const TileSum* ksum,
                                                         int2* krange, int* kcost, int n_kt) {
  const int kt = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (kt >= n_kt) return;
  const TileSum k = ksum[kt];
  int first = qp.n_qt, last = -1;
  for (int qt = lane; qt < qp.n_qt; qt += 64) {
    if (tiles_meet(qp.qsum[qt], k, a.window)) {
      first = min(first, qt);
      last = max(last, qt);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    first = min(first, __shfl_xor(first, off, 64));
    last = max(last, __shfl_xor(last, off, 64));
  }
  if (lane == 0) {
    krange[kt] = make_int2(first, last);
    kcost[kt] = last >= first ? last - first + 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per query tile and group of query heads (the forward's
// prepared walk and workgroup shape).
// ---------------------------------------------------------------------------
template <int D, int GW>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a, Plan pl, const float* delta) {
  constexpr int SUB = 4 / GW, TQ = 32 * SUB, KS = D / 16, MD = D / 32;
  using SKT = ST<D>;
  constexpr int kTile = SKT::bytes(kBK);  // K and V tiles swizzled (K is also read transposed)
  constexpr int kOffV = 2 * kTile, kOffP = 4 * kTile;
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * kTile + 2 * 512];
  LdsByte* smem = (LdsByte*)smem_raw;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int G = a.heads / a.kv_heads;
  const int n_groups = a.kv_heads * pl.head_groups;
  const int wi = blockIdx.x / n_groups, grp = blockIdx.x % n_groups;
  const int kh = grp / pl.head_groups, hg = grp % pl.head_groups;
  const int qt = __builtin_amdgcn_readfirstlane(ld_const(pl.order, wi));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = kh * G + hg * GW + wave % GW;
  const int qn = lane & 31, hf = lane >> 5;
  const int P = a.p;
  const int q_tok = qt * TQ + (wave / GW) * 32 + qn;
  const bool q_valid = q_tok < P;
  const int q_ld = q_valid ? q_tok : P - 1;
  const int my_pos = a.positions[q_ld], my_seg = a.segments[q_ld];
  // The `own` predicate on signed positions, then the window on the
  // unsigned difference (exact once pos_k <= pos_q).
  const uint32_t wlast = a.window > 0 ? (uint32_t)a.window - 1u : 0xffffffffu;
  const float scale_log2 = a.scale * kLog2eB;
  const float lse2 = a.lse[(long long)q_ld * a.heads + h] * kLog2eB;
  const float dlt = delta[(long long)q_ld * a.heads + h];

  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((long long)q_ld * a.heads + h) * D;
  const uint16_t* gg = static_cast<const uint16_t*>(a.dout) + ((long long)q_ld * a.heads + h) * D;
  u32x4 qf[KS], gf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = load16(qg + ks * 16 + hf * 8);
    gf[ks] = load16(gg + ks * 16 + hf * 8);
  }
  f32x16 dq[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[md][r] = 0.f;

  const int row_bytes = a.kv_heads * D * 2;
  // Row-wise reads: row qn (+32 hb), chunk 2 ks + hf stored at 2 ks ^ k_xc.
  const int k_row = qn * SKT::kStride;
  const int k_xc = hf ^ SKT::swz(qn);
  int t_offs[MD][2];
  swz_tr_offs<D>(lane, t_offs);
  // Tile loads of key tile kt into buffer b: K and V (SKT::loads(64) each) and
  // the positions / segments, spread over the 4 wavefronts.
  auto load_tile = [&](int kt, int b) {
    const int n_rows = min(kBK, P - kt * kBK);
    const long long e0 = (long long)kt * kBK * a.kv_heads * D + (long long)kh * D;
    const int nrec = (n_rows - 1) * row_bytes + 2 * D;
    const i32x4 rk = raw_rsrc(static_cast<const uint16_t*>(a.k) + e0, nrec);
    const i32x4 rv = raw_rsrc(static_cast<const uint16_t*>(a.v) + e0, nrec);
    for (int i = wave; i < SKT::loads(kBK); i += 4) {
      const int off = swz_off<D>(64 * i + lane, kBK, row_bytes);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + b * kTile + 1024 * i);
      lds_dma<16>(rk, dst, off);
      lds_dma<16>(rv, dst + kOffV, off);
    }
    if (wave == 3) {
      lds_dma<4>(raw_rsrc(a.positions + (long long)kt * kBK, 4 * n_rows), lds0 + kOffP + b * 512, lane * 4);
      lds_dma<4>(raw_rsrc(a.segments + (long long)kt * kBK, 4 * n_rows), lds0 + kOffP + b * 512 + 256, lane * 4);
    }
  };

  // The visited key tiles in order (both phases of the walk), with their
  // every-pair-allowed bit.
  const int2 rng = make_int2(__builtin_amdgcn_readfirstlane(ld_const(reinterpret_cast<const int*>(pl.qrange), 2LL * qt)),
                             __builtin_amdgcn_readfirstlane(ld_const(reinterpret_cast<const int*>(pl.qrange), 2LL * qt + 1)));
  auto next_visit = [&](int kt, bool& full) {
    while (kt <= rng.y) {
      const int g = kt >> 6;
      const int* w = reinterpret_cast<const int*>(pl.masks) + ((long long)qt * pl.n_kg + g) * kMaskWords;
      const unsigned long long vis = (unsigned long long)(uint32_t)ld_const(w, 0) |
                                     ((unsigned long long)(uint32_t)ld_const(w, 1) << 32);
      const unsigned long long fm = (unsigned long long)(uint32_t)ld_const(w, 2) |
                                    ((unsigned long long)(uint32_t)ld_const(w, 3) << 32);
      const unsigned long long m = vis >> (kt & 63);
      if (m != 0) {
        const int r = __builtin_amdgcn_readfirstlane(kt + (int)__builtin_ctzll(m));
        full = ((fm >> (r & 63)) & 1ull) != 0;
        return r;
      }
      kt = (g + 1) << 6;
    }
    return rng.y + 1;
  };

  bool full = false;
  int kt = next_visit(rng.x, full);
  int b = 0;
  if (kt <= rng.y) {
    load_tile(kt, 0);
    wait_all_loads();
    wg_barrier();
  }
  while (kt <= rng.y) {
    bool nfull = false;
    const int nkt = next_visit(kt + 1, nfull);
    if (nkt <= rng.y) load_tile(nkt, b ^ 1);
    const LdsByte* kb = smem + b * kTile;
    const LdsByte* vb = smem + kOffV + b * kTile;
    const LdsByte* pb = smem + kOffP + b * 512;
    const int n_j = P - kt * kBK;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ko = k_row + hb * 32 * SKT::kStride + (((2 * ks) ^ k_xc) << 4);
        const bf16x8 ak = lds_ld<bf16x8>(kb + ko);
        const bf16x8 av = lds_ld<bf16x8>(vb + ko);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, __builtin_bit_cast(bf16x8, qf[ks]), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, gf[ks]), dp, 0, 0, 0);
      }
      // Register r of this lane holds key j = 32 hb + 16 (r / 8) + 8 hf + r % 8.
      // Keys come in runs of four: their positions and segments are read
      // 16 bytes at a time (a masked tile only). One copy of this code for
      // fully-allowed tiles and one for masked tiles, so the branch on
      // `full` is taken once per half tile rather than once per element.
      // The element work runs in fenced phases of 16 independent
      // operations (the compiler otherwise chains it element by element and
      // waits out each result's latency).
      u32x4 dsw[2];
      auto ds_of = [&](auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        u32x4 kpw[4] = {}, ksw[4] = {};
        if constexpr (!FULL) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j0 = 32 * hb + 16 * (c >> 1) + 8 * hf + 4 * (c & 1);
            kpw[c] = lds_ld<u32x4>(pb + j0 * 4);
            ksw[c] = lds_ld<u32x4>(pb + 256 + j0 * 4);
          }
        }
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], scale_log2, -lse2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fast_exp2(x[r]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!FULL) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 32 * hb + 16 * (r >> 3) + 8 * hf + (r & 7);
            const uint32_t kp = kpw[r >> 2][r & 3], kq = ksw[r >> 2][r & 3];
            const bool ok = ((int)kq == my_seg) & ((int)kp <= my_pos) & ((uint32_t)my_pos - kp <= wlast) & (j < n_j);
            x[r] = ok ? x[r] : 0.f;
          }
        }
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = dp[r] - dlt;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] *= x[r];  // x is 0 where masked; dP and delta are finite
#pragma unroll
        for (int r = 0; r < 16; r += 2) dsw[r >> 3][(r & 7) >> 1] = pack_bf16x2(t[r], t[r + 1]);
      };
      if (full) ds_of(std::true_type{});
      else ds_of(std::false_type{});
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const bf16x8 at = swz_tr_operand<D>(kb + hb * 32 * SKT::kStride, t_offs, kk, md);
          dq[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, __builtin_bit_cast(bf16x8, dsw[kk]), dq[md], 0, 0, 0);
        }
    }
    wait_all_loads();
    wg_barrier();
    kt = nkt;
    full = nfull;
    b ^= 1;
  }
  wait_all_loads();

  if (q_valid) {
    uint16_t* og = static_cast<uint16_t*>(a.dq) + ((long long)q_tok * a.heads + h) * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(dq[md][4 * g] * a.scale, dq[md][4 * g + 1] * a.scale);
        w[1] = pack_bf16x2(dq[md][4 * g + 2] * a.scale, dq[md][4 * g + 3] * a.scale);
        *reinterpret_cast<u32x2*>(og + 32 * md + 8 * g + 4 * hf) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK / dV: one workgroup per key tile and KV head, 8 wavefronts in producer /
// consumer pairs. Wave w owns keys 32 (w & 1) .. +31 of the tile and the
// (query tile, head) pairs of parity (w >> 1) & 1. A producer (w >= 4) holds
// K^T and V^T of its keys in registers and forms S = Q K^T, dP = dO V^T,
// P and dS = P (dP - delta) for each pair, passing P and dS (bf16) through
// LDS. Its consumer (w - 4, on the same SIMD) takes them one step later and
// accumulates dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
// transposed from that step's stage. Pairs are visited two at a time, both
// staged in LDS (a ring of three stages). The consumers also stage the
// pairs (each one its parity's pair and half of its tiles) and classify
// them, so a producer's step holds only its matrix and softmax work.
// ---------------------------------------------------------------------------
// How a producer forms P for a staged pair: no element allowed (P = dS = 0),
// every element allowed, one segment and non-negative positions (one unsigned
// compare of the position difference per element), or the full mask.
enum : int { kPairSkip = 0, kPairFull = 1, kPairOneSeg = 2, kPairMasked = 3 };

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a, Plan qp, const TileSum* ksum,
                                                         const int2* krange, const int* korder,
                                                         const float* delta, const float* lse2) {
  constexpr int KS = D / 16, MD = D / 32;
  using SQT = ST<D>;
  constexpr int qTile = SQT::bytes(32);            // one Q or dout tile (32 queries, swizzled)
  constexpr int NLD = SQT::loads(32) / 2;          // 16-byte loads of a tile per consumer half
  // Q, dout, then lse, delta, positions, segments (256 bytes each: a 64-lane
  // load writes its 32 values and 32 zeros).
  constexpr int pairBytes = 2 * qTile + 4 * 256;
  constexpr int stageBytes = 2 * pairBytes;
  // After three stages, P and dS of the producers: two buffers of 4 slots
  // (key half, pair parity) of 4 x 64 lanes x 16 bytes (P halves, then dS
  // halves; piece c of lane l at 1024 c + 16 l, so each access covers the
  // banks once); then one code word per (stage, slot).
  constexpr int pOff = 3 * stageBytes;
  constexpr int pBufBytes = 4 * 64 * 64;
  constexpr int codeOff = pOff + 2 * pBufBytes;
  constexpr int combineBytes = 2 * 2 * MD * 16 * 64 * 4;
  constexpr int ldsBytes = codeOff + 32 > combineBytes ? codeOff + 32 : combineBytes;
  __shared__ __attribute__((aligned(16))) char smem_raw[ldsBytes];
  LdsByte* smem = (LdsByte*)smem_raw;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // Key tiles costliest first (the most query tiles to visit), so the long
  // ones do not start last; workgroup i * kv_heads + kh takes KV head kh.
  const int kt = __builtin_amdgcn_readfirstlane(ld_const(korder, blockIdx.x / a.kv_heads));
  const int kh = blockIdx.x % a.kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wave & 1, hp = (wave >> 1) & 1;
  const int qn = lane & 31, hf = lane >> 5;
  const int P = a.p, G = a.heads / a.kv_heads;
  const int key = kt * kBK + 32 * kb + qn;
  const bool k_valid = key < P;
  const int key_ld = k_valid ? key : P - 1;

  const int2 rng = make_int2(__builtin_amdgcn_readfirstlane(krange[kt].x), __builtin_amdgcn_readfirstlane(krange[kt].y));
  const int n_pairs = rng.y >= rng.x ? (rng.y - rng.x + 1) * G : 0;
  const int n_steps = (n_pairs + 1) / 2;
  // This lane's first piece of P and dS in slot (kb, hp) of buffer pbuf.
  auto p_slot = [&](int pbuf) { return pOff + pbuf * pBufBytes + (2 * hp + kb) * 4096 + lane * 16; };
  auto code_at = [&](int b, int slot) { return codeOff + 4 * (2 * b + slot); };

  // Producer: this lane's key as the B operand of S and dP (K^T and V^T
  // columns, dimensions 16 ks + 8 hf ..).
  auto produce = [&]() {
    const int pos_k = a.positions[key_ld], seg_k = a.segments[key_ld];
    const uint32_t wlast = a.window > 0 ? (uint32_t)a.window - 1u : 0xffffffffu;
    // One-segment pairs: positions are non-negative, so an unsigned
    // difference at most this bound means order and window both hold.
    const uint32_t wl_one = a.window > 0 ? (uint32_t)a.window - 1u : 0x7fffffffu;
    const float scale_log2 = a.scale * kLog2eB;
    const uint16_t* kg = static_cast<const uint16_t*>(a.k) + ((long long)key_ld * a.kv_heads + kh) * D;
    const uint16_t* vg = static_cast<const uint16_t*>(a.v) + ((long long)key_ld * a.kv_heads + kh) * D;
    u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = load16(kg + ks * 16 + hf * 8);
      vf[ks] = load16(vg + ks * 16 + hf * 8);
    }
    // A-operand reads of the Q and dout tiles: row qn, chunk 2 ks + hf
    // stored at (2 ks + hf) ^ swz(qn) = 2 ks ^ (hf ^ swz(qn)).
    const int q_row = qn * SQT::kStride;
    const int q_xc = hf ^ SQT::swz(qn);

    if (n_steps > 0) wg_barrier();  // the first stage
    int b = 0;  // stage of this step
    for (int step = 0; step < n_steps; ++step) {
      const int bn = b == 2 ? 0 : b + 1;
      const int code = __builtin_amdgcn_readfirstlane(lds_ld<int>(smem + code_at(b, hp)));
      const LdsByte* pbase = smem + b * stageBytes + hp * pairBytes;
      const LdsByte* qb = pbase;
      const LdsByte* gb = pbase + qTile;
      const LdsByte* misc = pbase + 2 * qTile;  // lse, delta, positions, segments
      // S = Q K^T and dP = dO V^T; the Q and dout operands of a k-step are
      // read from LDS two k-steps ahead of its MFMAs (a ring of three), and
      // a scheduling fence keeps that order.
      f32x16 s = {}, dp = {};
      bf16x8 ra[3][2];
      auto ld_ks = [&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        const int qo = q_row + (((2 * ks) ^ q_xc) << 4);
        ra[ks % 3][0] = lds_ld<bf16x8>(qb + qo);
        ra[ks % 3][1] = lds_ld<bf16x8>(gb + qo);
      };
      ld_ks(std::integral_constant<int, 0>{});
      if constexpr (KS > 1) ld_ks(std::integral_constant<int, 1>{});
      static_for<KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + 2 < KS) ld_ks(std::integral_constant<int, ks + 2>{});
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[ks % 3][0], __builtin_bit_cast(bf16x8, kf[ks]), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[ks % 3][1], __builtin_bit_cast(bf16x8, vf[ks]), dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      // Register r of this lane holds query iq = 16 (r / 8) + 8 hf + r % 8
      // of the tile and this lane's key; lse and delta of those queries
      // come as four 16-byte reads each.
      float lse_r[16], dl_r[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int iq0 = 16 * (c >> 1) + 8 * hf + 4 * (c & 1);
        const u32x4 lw = lds_ld<u32x4>(misc + iq0 * 4), dw = lds_ld<u32x4>(misc + 256 + iq0 * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lse_r[4 * c + e] = __uint_as_float(lw[e]);
          dl_r[4 * c + e] = __uint_as_float(dw[e]);
        }
      }
      // P and dS in bf16, two 16-query halves each, to LDS; one copy of this
      // code per pair class, chosen once per pair. Rows past the end of a
      // partial query tile were staged as zeros (q, dout, lse, delta), so
      // their P is finite and their dout and q columns add nothing; keys
      // past the end only feed their own (unwritten) columns of dK and dV.
      u32x4 pp[2] = {}, pds[2] = {};
      auto p_ds = [&](auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
        int qpos_r[16], qseg_r[16];
        if constexpr (MODE != kPairFull) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int iq0 = 16 * (c >> 1) + 8 * hf + 4 * (c & 1);
            const u32x4 pw = lds_ld<u32x4>(misc + 512 + iq0 * 4);
            u32x4 sw = {};
            if constexpr (MODE == kPairMasked) sw = lds_ld<u32x4>(misc + 768 + iq0 * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              qpos_r[4 * c + e] = (int)pw[e];
              qseg_r[4 * c + e] = (int)sw[e];
            }
          }
        }
        // In phases of 16 independent operations each (fenced, so the
        // compiler does not fold them back into per-element chains that
        // wait out each result's latency): P from S, whose MFMAs were issued
        // first, then dS, which needs dP.
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], scale_log2, -lse_r[r]);  // lse * log2(e)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fast_exp2(x[r]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MODE == kPairOneSeg) {
          // Allowed iff 0 <= d <= wl_one for d = qpos - pos_k (both
          // non-negative, so neither d nor wl_one - d overflows when d >= 0):
          // the sign of d | (wl_one - d) is the mask.
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int d = qpos_r[r] - pos_k;
            const int m = (d | ((int)wl_one - d)) >> 31;
            x[r] = __int_as_float(__float_as_int(x[r]) & ~m);
          }
        } else if constexpr (MODE == kPairMasked) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            x[r] = (qseg_r[r] == seg_k) & (pos_k <= qpos_r[r]) & ((uint32_t)qpos_r[r] - (uint32_t)pos_k <= wlast)
                       ? x[r]
                       : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) pp[r >> 3][(r & 7) >> 1] = pack_bf16x2(x[r], x[r + 1]);
        __builtin_amdgcn_sched_barrier(0);
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = dp[r] - dl_r[r];
        __builtin_amdgcn_sched_barrier(0);
        // p is 0 where masked; dP and delta are finite
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] *= x[r];
#pragma unroll
        for (int r = 0; r < 16; r += 2) pds[r >> 3][(r & 7) >> 1] = pack_bf16x2(t[r], t[r + 1]);
      };
      if (code == kPairFull) p_ds(std::integral_constant<int, kPairFull>{});
      else if (code == kPairOneSeg) p_ds(std::integral_constant<int, kPairOneSeg>{});
      else if (code == kPairMasked) p_ds(std::integral_constant<int, kPairMasked>{});
      const int po = p_slot(step & 1);
      lds_st(smem + po, pp[0]);
      lds_st(smem + po + 1024, pp[1]);
      lds_st(smem + po + 2048, pds[0]);
      lds_st(smem + po + 3072, pds[1]);
      wg_barrier();
      b = bn;
    }
    wait_all_loads();
    wg_barrier();
    wg_barrier();  // the consumers' sums
  };

  // Consumer: stages the pairs one step ahead and accumulates one step
  // behind its producer.
  auto consume = [&]() {
    f32x16 dk[MD], dv[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[md][r] = 0.f;
        dv[md][r] = 0.f;
      }
    int t_offs[MD][2];
    swz_tr_offs<D>(lane, t_offs);
    // dV^T += dO^T P and dK^T += Q^T dS for the pair staged at pbase, P and
    // dS from P buffer pbuf: MFMA j (kk = j / 2 MD, md = (j / 2) % MD, dV
    // for even j, dK for odd) takes its transposed operand from a ring of
    // four read three MFMAs ahead.
    auto accumulate = [&](const LdsByte* pbase, int pbuf) {
      const LdsByte* qb = pbase;
      const LdsByte* gb = pbase + qTile;
      const int po = p_slot(pbuf);
      const u32x4 pp[2] = {lds_ld<u32x4>(smem + po), lds_ld<u32x4>(smem + po + 1024)};
      const u32x4 pds[2] = {lds_ld<u32x4>(smem + po + 2048), lds_ld<u32x4>(smem + po + 3072)};
      constexpr int NJ = 4 * MD;
      bf16x8 rt[4];
      auto tr_j = [&](auto jc) {
        constexpr int j = decltype(jc)::value, kk = j / (2 * MD), md = (j / 2) % MD;
        rt[j & 3] = swz_tr_operand<D>((j & 1) ? qb : gb, t_offs, kk, md);
      };
      tr_j(std::integral_constant<int, 0>{});
      tr_j(std::integral_constant<int, 1>{});
      tr_j(std::integral_constant<int, 2>{});
      static_for<NJ>([&](auto jc) {
        constexpr int j = decltype(jc)::value, kk = j / (2 * MD), md = (j / 2) % MD;
        if constexpr (j + 3 < NJ) tr_j(std::integral_constant<int, j + 3>{});
        if constexpr (j & 1)
          dk[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rt[j & 3], __builtin_bit_cast(bf16x8, pds[kk]), dk[md], 0, 0, 0);
        else
          dv[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rt[j & 3], __builtin_bit_cast(bf16x8, pp[kk]), dv[md], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // Staging: this wave loads half kb of the pair of parity hp (Q and dout
    // loads kb NLD .. +NLD - 1 of each tile; lse and delta for half 0,
    // positions and segments for half 1); half 0 also writes the pair's
    // code (classify).
    // Lane offsets of the tile loads: row r of the LDS tile holds query
    // kappa(r); rows past a partial tile's end lie past the descriptor's
    // range and load zeros.
    const int row_bytes = a.heads * D * 2;
    int voff[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int p = 64 * (kb * NLD + j) + lane;
      const int row = p / SQT::kChunks, pc = p % SQT::kChunks;
      voff[j] = kappa(row) * row_bytes + ((pc ^ SQT::swz(row)) << 4);
    }
    const int moff = lane >= 32 ? 0x40000000 : kb == 0 ? lane * a.heads * 4 : lane * 4;
    const TileSum ks_sum = ld_const(ksum, kt);
    // The pair of this parity for the step being staged: index np, query
    // tile rng.x + lq, head kh G + lh (lq = np / G, lh = np % G, advanced
    // two pairs at a time).
    int np = hp, lq = G == 1 ? hp : 0, lh = G == 1 ? 0 : hp;
    int st_qt = 0;
    bool st_valid = false;
    auto stage = [&](int b) {
      // A slot past the last pair stages the last pair again (its code
      // makes the producer's P zero), so every step has the same body.
      const bool valid = np < n_pairs;
      int sq = lq, sh = lh;
      if (!valid) {
        if (sh == 0) {
          sq -= 1;
          sh = G - 1;
        } else {
          sh -= 1;
        }
      }
      const int qt = rng.x + sq, h = kh * G + sh;
      const int n_rows = min(32, P - qt * 32);
      const uint32_t base = lds0 + b * stageBytes + hp * pairBytes;
      const long long r0 = (long long)qt * 32 * a.heads + h;
      const int nrec = (n_rows - 1) * row_bytes + 2 * D;
      const i32x4 rq = raw_rsrc(static_cast<const uint16_t*>(a.q) + r0 * D, nrec);
      const i32x4 rg = raw_rsrc(static_cast<const uint16_t*>(a.dout) + r0 * D, nrec);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const uint32_t dst = base + 1024 * (kb * NLD + j);
        lds_dma<16>(rq, dst, voff[j]);
        lds_dma<16>(rg, dst + qTile, voff[j]);
      }
      const uint32_t mdst = base + 2 * qTile + 512 * kb;
      if (kb == 0) {
        const int nm = 4 * ((n_rows - 1) * a.heads + 1);
        lds_dma<4>(raw_rsrc(lse2 + r0, nm), mdst, moff);
        lds_dma<4>(raw_rsrc(delta + r0, nm), mdst + 256, moff);
      } else {
        lds_dma<4>(raw_rsrc(a.positions + (long long)qt * 32, 4 * n_rows), mdst, moff);
        lds_dma<4>(raw_rsrc(a.segments + (long long)qt * 32, 4 * n_rows), mdst + 256, moff);
      }
      st_qt = qt;
      st_valid = valid;
      np += 2;
      lh += 2;
      while (lh >= G) {
        lh -= G;
        ++lq;
      }
    };
    // The code of the pair staged last (half-0 waves; after this wave's
    // matrix work, so the scalar load's wait holds up no LDS reads).
    auto classify = [&](int b) {
      if (kb != 0) return;
      int code = kPairSkip;
      if (st_valid) {
        const TileSum q_sum = ld_const(qp.qsum, st_qt);
        if (tiles_meet(q_sum, ks_sum, a.window))
          code = tiles_full(q_sum, ks_sum, kt, P, a.window) && (st_qt + 1) * 32 <= P ? kPairFull
                 : tiles_oneseg(q_sum, ks_sum, kt, P)                                ? kPairOneSeg
                                                                                     : kPairMasked;
      }
      lds_st(smem + code_at(b, hp), code);
    };

    // Stages form a ring of three: step s of the producers reads stage
    // s % 3 and this wave stage (s - 1) % 3, while the pairs of step s + 1
    // load into stage (s + 1) % 3, last read in step s - 1. P and dS of step
    // s sit in P buffer s % 2.
    if (n_steps > 0) {
      stage(0);
      classify(0);
      wait_all_loads();
      wg_barrier();
    }
    int b = 0;
    for (int step = 0; step < n_steps; ++step) {
      const int bn = b == 2 ? 0 : b + 1, bp = b == 0 ? 2 : b - 1;
      if (step + 1 < n_steps) stage(bn);
      if (step > 0) accumulate(smem + bp * stageBytes + hp * pairBytes, (step - 1) & 1);
      if (step + 1 < n_steps) classify(bn);
      wait_all_loads();
      wg_barrier();
      b = bn;
    }
    // The last pair (its stage is the last one read: nothing loads into it
    // any more).
    if (n_steps > 0) {
      const int bp = b == 0 ? 2 : b - 1;
      accumulate(smem + bp * stageBytes + hp * pairBytes, (n_steps - 1) & 1);
    }
    wait_all_loads();
    wg_barrier();

    // The two parity consumers of a key half add their sums: the odd-pair
    // one puts its sums in LDS, the even-pair one reads, adds and writes.
    LdsByte* cb = smem + kb * (2 * MD * 16 * 64 * 4);
    if (hp == 1) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          lds_st(cb + ((md * 16 + r) * 64 + lane) * 4, dk[md][r]);
          lds_st(cb + (((MD + md) * 16 + r) * 64 + lane) * 4, dv[md][r]);
        }
    }
    wg_barrier();
    if (hp == 0 && k_valid) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dk[md][r] += lds_ld<float>(cb + ((md * 16 + r) * 64 + lane) * 4);
          dv[md][r] += lds_ld<float>(cb + (((MD + md) * 16 + r) * 64 + lane) * 4);
        }
      uint16_t* dkg = static_cast<uint16_t*>(a.dk) + ((long long)key * a.kv_heads + kh) * D;
      uint16_t* dvg = static_cast<uint16_t*>(a.dv) + ((long long)key * a.kv_heads + kh) * D;
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 wk, wv;
          wk[0] = pack_bf16x2(dk[md][4 * g] * a.scale, dk[md][4 * g + 1] * a.scale);
          wk[1] = pack_bf16x2(dk[md][4 * g + 2] * a.scale, dk[md][4 * g + 3] * a.scale);
          wv[0] = pack_bf16x2(dv[md][4 * g], dv[md][4 * g + 1]);
          wv[1] = pack_bf16x2(dv[md][4 * g + 2], dv[md][4 * g + 3]);
          *reinterpret_cast<u32x2*>(dkg + 32 * md + 8 * g + 4 * hf) = wk;
          *reinterpret_cast<u32x2*>(dvg + 32 * md + 8 * g + 4 * hf) = wv;
        }
    }
  };
  if (wave >= 4) produce();
  else consume();
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
size_t prefill_bwd_workspace_bytes(int p, int heads) {
  const size_t n_kt = (size_t)(p + kBK - 1) / kBK;
  const size_t n_q32 = (size_t)(p + 31) / 32;
  return prefill_plan_bytes(p) + align256(n_q32 * sizeof(TileSum)) + align256(n_kt * sizeof(int2)) +
         2 * align256(n_kt * sizeof(int)) + 2 * align256((size_t)p * heads * sizeof(float));
}

template <int D>
static hipError_t launch_bwd_main(const BwdArgs& a, const Plan& pl, const Plan& qp, const int2* krange,
                                  const int* korder, const float* delta, const float* lse2, hipStream_t stream) {
  const int n_groups = a.kv_heads * pl.head_groups;
  const dim3 gq(pl.n_qt * n_groups), blk(256);
  if (pl.gw == 4) bwd_dq_kernel<D, 4><<<gq, blk, 0, stream>>>(a, pl, delta);
  else if (pl.gw == 2) bwd_dq_kernel<D, 2><<<gq, blk, 0, stream>>>(a, pl, delta);
  else bwd_dq_kernel<D, 1><<<gq, blk, 0, stream>>>(a, pl, delta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dkdv_kernel<D><<<dim3(pl.n_kt * a.kv_heads), dim3(512), 0, stream>>>(a, qp, pl.ksum, krange, korder, delta, lse2);
  return hipGetLastError();
}

hipError_t launch_prefill_bwd(const BwdArgs& a, hipStream_t stream) {
  PrefillArgs pa{};
  pa.p = a.p;
  pa.heads = a.heads;
  pa.kv_heads = a.kv_heads;
  pa.head_dim = a.head_dim;
  pa.window = a.window;
  pa.positions = a.positions;
  pa.segments = a.segments;
  pa.ws = a.ws;
  pa.src = kSrcPacked;
  Plan pl;
  // The dQ kernel walks 4-wave query tiles (32 tokens of each head).
  hipError_t e = prefill_prepare(pa, pl, stream, 4);
  if (e != hipSuccess) return e;
  char* ws = static_cast<char*>(a.ws) + prefill_plan_bytes(a.p);
  const size_t n_q32 = (size_t)(a.p + 31) / 32;
  // Summaries of 32-token query tiles (the key-side walk's unit).
  Plan qp = pl;
  qp.tq = 32;
  qp.n_qt = (int)n_q32;
  qp.n_kt = 0;
  qp.qsum = reinterpret_cast<TileSum*>(ws);
  ws += align256(n_q32 * sizeof(TileSum));
  int2* krange = reinterpret_cast<int2*>(ws);
  ws += align256((size_t)pl.n_kt * sizeof(int2));
  // Key-tile costs and their costliest-first order (the prefill's counting
  // sort over key tiles instead of query tiles).
  Plan kp = pl;
  kp.rec = nullptr;
  kp.n_qt = pl.n_kt;
  kp.cost = reinterpret_cast<int*>(ws);
  ws += align256((size_t)pl.n_kt * sizeof(int));
  kp.order = reinterpret_cast<int*>(ws);
  ws += align256((size_t)pl.n_kt * sizeof(int));
  kp.max_cost = (int)n_q32;
  float* delta = reinterpret_cast<float*>(ws);
  ws += align256((size_t)a.p * a.heads * sizeof(float));
  float* lse2 = reinterpret_cast<float*>(ws);
  e = prefill_summarize(pa, qp, stream);
  if (e != hipSuccess) return e;
  bwd_krange_kernel<<<dim3((pl.n_kt + 3) / 4), dim3(256), 0, stream>>>(a, qp, pl.ksum, krange, kp.cost, pl.n_kt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = prefill_order(kp, stream);
  if (e != hipSuccess) return e;
  const long long chunks = (long long)a.p * a.heads * (a.head_dim / 8);
  bwd_delta_kernel<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream>>>(a, delta, lse2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.head_dim == 64 ? launch_bwd_main<64>(a, pl, qp, krange, kp.order, delta, lse2, stream)
                          : launch_bwd_main<128>(a, pl, qp, krange, kp.order, delta, lse2, stream);
}

}  // namespace gqa
