// Fused q / k / v projections + rope + KV write on bf16 matrix cores (gfx950).
//
// GroupedQueryAttention of the Linnet "examples/01-llama" page
// (src/attention.linnet, `forward` / `decode`) computes q_proj, k_proj and
// v_proj -- std.nn.linear::Linear modules, y = x W^T (+ b) as a Tensor of T --
// then rotates q and k (`rope`, rotate-half) and writes k and v into the
// caches (write_at); the Nest llama-3.1-8b-instruct card lists the same
// modules. Here the three projections are one GEMM over the concatenated
// output features [q | k | v], and its epilogue rounds to T, rotates and
// writes straight to q_out / the caches: the projections' outputs never make
// a separate trip through HBM.
//
// Design:
// * Workgroup tile: 128 tokens x 128 output features (one head at D = 128,
//   two at D = 64), 4 waves of 64 x 64, K slabs of 64. Both operands are
//   K-contiguous rows (x [n, hidden], weight [out, hidden]), so each is one
//   16-byte read per lane in the layout of v_mfma_f32_32x32x16_bf16's A / B
//   operands; 4 independent accumulators per wave.
// * K / W slabs are staged through LDS with a padded row stride (144 bytes):
//   the 16 rows a 16-lane group reads land in distinct bank groups. Double
//   buffered; the next slab's global loads fly during the current slab.
// * Epilogue: accumulators + bias, rounded to bf16, go through LDS so a thread
//   holds both halves (d, d + D/2) of a head chunk; the rotation is the
//   exact value rounded once to T (the same helper as the rope pass).
#include <type_traits>
#include <utility>

#include "attn_tiles.h"
#include "common.h"
#include "internal.h"
#include "rope_common.h"

#ifndef GQA_QKV_LARGE_TILES
#define GQA_QKV_LARGE_TILES 1
#endif

namespace gqa {

namespace {
constexpr int kBM = 128;            // tokens per workgroup tile
constexpr int kBN = 128;            // output features per workgroup tile
constexpr int kSK = 64;             // hidden (K) per slab
constexpr int kRow = kSK * 2 + 16;  // LDS row stride of a staged slab (bytes)
constexpr int kSlab = kBM * kRow;   // one operand slab
constexpr int kOutRow = kBN * 2 + 16;  // LDS row stride of the output tile

typedef __attribute__((address_space(3))) char LdsB;
template <typename T>
__device__ __forceinline__ T lds_get(const LdsB* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_put(LdsB* p, const T& v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}
// Calls f(std::integral_constant<int, i>) for i = 0 .. N - 1 (register
// indices below must be compile-time constants).
template <typename F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}
}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void qkv_kernel(QkvArgs a) {
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * kSlab];
  LdsB* smem = (LdsB*)smem_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int f0 = blockIdx.x * kBN;  // first output feature of the tile
  const int m0 = blockIdx.y * kBM;  // first token of the tile
  const int H = a.hidden;
  const int qf = a.heads * D, kf = a.kv_heads * D;

  // Staging: thread tid owns chunks tid + 256 i (i < 4) of each 128 x 64 slab:
  // row = chunk / 8, 16-byte column chunk = chunk % 8 (8 lanes per row).
  const int s_col = tid & 7;
  const uint16_t* wrow[4];
  int a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 3) + 32 * i;
    a_off[i] = ((m0 + row) * H + s_col * 8) * 2;  // bytes from x
    const int f = f0 + row;
    const uint16_t* w = f < qf ? static_cast<const uint16_t*>(a.wq) + (long long)f * H
                        : f < qf + kf ? static_cast<const uint16_t*>(a.wk) + (long long)(f - qf) * H
                                      : static_cast<const uint16_t*>(a.wv) + (long long)(f - qf - kf) * H;
    wrow[i] = w + s_col * 8;
  }
  u32x4 ra[4], rb[4];
  auto load_slab = [&](int k0) {
    // Rows of x past n read zeros (the buffer range ends at the last row).
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const uint16_t*>(a.x) + k0), (short)0,
        (int)(((long long)a.n * H - k0) * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, a_off[i], 0, 0);
      rb[i] = load16(wrow[i] + k0);
    }
  };
  auto store_slab = [&](int buf) {
    LdsB* sa = smem + buf * 2 * kSlab;
    LdsB* sb = sa + kSlab;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      lds_put(sa + row * kRow + s_col * 16, ra[i]);
      lds_put(sb + row * kRow + s_col * 16, rb[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Operand reads: lane l supplies row l % 32 of its 32-row block, k chunk
  // 2 ks + l / 32 of the slab.
  const int rd = (lane & 31) * kRow + (lane >> 5) * 16;
  const int n_slabs = H / kSK;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int t = 0; t < n_slabs; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_slabs) load_slab((t + 1) * kSK);
    const LdsB* sa = smem + buf * 2 * kSlab + (wm * 64) * kRow + rd;
    const LdsB* sb = smem + buf * 2 * kSlab + kSlab + (wn * 64) * kRow + rd;
    // Operands of k-step ks + 1 are read while the MFMAs of ks run (a ring
    // of two sets), each step fenced so the order holds.
    bf16x8 op[2][4];
    auto ld_ks = [&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      bf16x8* o = op[ks & 1];
      o[0] = lds_get<bf16x8>(sa + ks * 32);
      o[1] = lds_get<bf16x8>(sa + 32 * kRow + ks * 32);
      o[2] = lds_get<bf16x8>(sb + ks * 32);
      o[3] = lds_get<bf16x8>(sb + 32 * kRow + ks * 32);
    };
    ld_ks(std::integral_constant<int, 0>{});
    unroll<kSK / 16>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      if constexpr (ks + 1 < kSK / 16) ld_ks(std::integral_constant<int, ks + 1>{});
      const bf16x8* o = op[ks & 1];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[0], o[2], acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[0], o[3], acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[1], o[2], acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[1], o[3], acc[1][1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (t + 1 < n_slabs) store_slab(buf ^ 1);
    __syncthreads();
  }

  // Epilogue 1: + bias, round to bf16, into the output tile [128 tokens][128
  // features] in LDS (the slabs are no longer needed). Accumulator register r
  // of lane l in block (i, j): token 8 (r / 4) + 4 (l / 32) + r % 4, feature
  // l % 32.
  LdsB* so = smem;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = wn * 64 + j * 32 + (lane & 31);
    const int f = f0 + col;
    const void* bsrc = f < qf ? a.bq : f < qf + kf ? a.bk : a.bv;
    const int bidx = f < qf ? f : f < qf + kf ? f - qf : f - qf - kf;
    const float bf = bsrc ? bf16_to_f32(static_cast<const uint16_t*>(bsrc)[bidx]) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        lds_put(so + row * kOutRow + col * 2, f32_to_bf16(acc[i][j][r] + bf));
      }
  }
  __syncthreads();

  // Epilogue 2: per (token, head chunk pair) job, rotate and write. Jobs:
  // 128 tokens x (128 / D) heads x (D / 16) chunk pairs = 1024.
  constexpr int HPT = kBN / D;      // heads per tile
  constexpr int CPH = D / 16;       // chunk pairs per head (8 elements each half)
  const bool rotate = a.wr.rope_table != nullptr;
#pragma unroll
  for (int it = 0; it < kBM * HPT * CPH / 256; ++it) {
    const int job = tid + 256 * it;
    const int cp = job % CPH;
    const int hh = (job / CPH) % HPT;
    const int tl = job / (CPH * HPT);
    const int t = m0 + tl;
    if (t >= a.n) continue;
    const int fh = f0 + hh * D;  // first feature of the head
    const int d0 = cp * 8;
    u32x4 lo = lds_get<u32x4>(so + tl * kOutRow + (hh * D + d0) * 2);
    u32x4 hi = lds_get<u32x4>(so + tl * kOutRow + (hh * D + D / 2 + d0) * 2);
    const bool is_v = fh >= qf + kf;
    if (rotate && !is_v) {
      int p = a.wr.positions[t];
      p = p < 0 ? 0 : (p >= a.wr.rope_max_pos ? a.wr.rope_max_pos - 1 : p);
      const uint16_t* tab = static_cast<const uint16_t*>(a.wr.rope_table);
      const u32x4 cw = load16(tab + (long long)p * (D / 2) + d0);
      const u32x4 sw = load16(tab + ((long long)a.wr.rope_max_pos + p) * (D / 2) + d0);
      rotate_chunk<uint16_t>(lo, hi, cw, sw);
    }
    if (fh < qf) {
      uint16_t* dst = static_cast<uint16_t*>(a.q_out) + ((long long)t * a.heads + fh / D) * D;
      store16(dst + d0, lo);
      store16(dst + D / 2 + d0, hi);
      continue;
    }
    const int kh = (is_v ? fh - qf - kf : fh - qf) / D;
    uint16_t* own = static_cast<uint16_t*>(is_v ? a.v_out : a.k_out);
    if (own != nullptr) {
      uint16_t* dst = own + ((long long)t * a.kv_heads + kh) * D;
      store16(dst + d0, lo);
      store16(dst + D / 2 + d0, hi);
    }
    const long long off = a.wr.cache_kind != 0 ? cache_offset(a.wr, t, kh) : -1;
    if (off >= 0) {
      uint16_t* c = static_cast<uint16_t*>(is_v ? a.wr.cache_v : a.wr.cache_k) + off;
      if (is_v ? a.wr.cache_v != nullptr : true) {
        store16(c + d0, lo);
        store16(c + D / 2 + d0, hi);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-tile variant, used when the q, k and v feature blocks are multiples of
// 256 (every model these entries serve): 256 tokens x 256 features per
// workgroup of 4 wavefronts, each wavefront 128 x 128 (4 x 4 blocks of
// 32 x 32, 256 accumulator registers), one wavefront per SIMD. Per 16-wide
// k-step a wavefront reads 8 operand vectors from LDS for 16 MFMAs, half the
// LDS bytes per MFMA of the 128 x 128 tile, and the reads of the next k-step
// are interleaved with the first half of the current one's MFMAs. Slabs of
// 32 hidden columns go straight from memory into LDS (buffer loads with an
// LDS destination, no register staging) into a ring of buffers, issued
// GQA_QKV_AHEAD slabs ahead of their use, with one barrier per slab; each
// slab row holds its 16-byte chunks XOR-swizzled by row so that operand reads
// are free of bank conflicts.
// Tiles are handed out so that the 32 workgroups resident on one XCD share 8
// token tiles and 4 feature tiles: their slabs are L2 hits.
#ifndef GQA_QKV_AHEAD
#define GQA_QKV_AHEAD 1
#endif
#ifndef GQA_QKV_BK
#define GQA_QKV_BK 64
#endif
#ifndef GQA_QKV_BUFS
#define GQA_QKV_BUFS 2
#endif
namespace {
constexpr int kGM = 256;                  // tokens per tile
constexpr int kGN = 256;                  // features per tile
constexpr int kGK = GQA_QKV_BK;           // hidden columns per slab (32 or 64)
constexpr int kGRow = kGK * 2;            // bytes per slab row
constexpr int kGGran = kGRow / 16;        // 16-byte chunks per slab row (4 or 8)
constexpr int kGSlab = kGM * kGRow;       // bytes of one operand slab
constexpr int kGBufs = GQA_QKV_BUFS;      // slab ring (x and weights per slot)
// Swizzle of slab row r: chunk c is stored at granule c ^ qkv_sw(r). The
// LDS of gfx950 has 64 4-byte banks and serves a 16-byte read 16 lanes at a
// time; those lanes read 16 consecutive rows at one chunk, which with the
// swizzle land in 16 distinct 16-byte bank groups (a 128-byte row puts rows r
// and r + 1 half a bank period apart, a 64-byte row a quarter).
__device__ __forceinline__ int qkv_sw(int r) { return kGGran == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
constexpr int kGAhead = GQA_QKV_AHEAD;    // slabs in flight ahead of the one in use
static_assert(kGAhead >= 1 && kGAhead < kGBufs, "ring");
constexpr int kGOutRow = kGN * 2 + 16;    // LDS row stride of the output tile
constexpr int kGLds = kGBufs * 2 * kGSlab > kGM * kGOutRow ? kGBufs * 2 * kGSlab : kGM * kGOutRow;
constexpr int kGDma = kGSlab / 1024 / 4;  // 1 KiB loads per wavefront per operand slab
}  // namespace

template <int D>
__global__ __launch_bounds__(256) void qkv256_kernel(QkvArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kGLds];
  LdsB* smem = (LdsB*)smem_raw;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // Tile of this workgroup. Workgroup L runs on XCD L % 8; with 8 | tiles_m
  // each XCD takes a band of tiles_m / 8 token tiles, walked 8 token tiles
  // at a time across every feature tile.
  const int L = blockIdx.x;
  int tm, tn;
  if (tiles_m % 8 == 0) {
    const int xcd = L % 8, i = L / 8;
    const int band = tiles_m / 8;           // token tiles per XCD
    const int grp = i / (8 * tiles_n);      // groups of 8 token tiles
    const int j = i % (8 * tiles_n);
    tm = xcd * band + grp * 8 + j % 8;
    tn = j / 8;
    if (band % 8 != 0) {                    // bands not a multiple of 8: plain order
      tm = xcd * band + i / tiles_n;
      tn = i % tiles_n;
    }
  } else {
    tm = L / tiles_n;
    tn = L % tiles_n;
  }
  const int m0 = tm * kGM, f0 = tn * kGN;
  const int H = a.hidden;
  const int qf = a.heads * D, kf = a.kv_heads * D;
  const long long K2 = 2LL * H;  // bytes per operand row

  // DMA lanes: load u of this wavefront (instruction j = kGDma wave + u)
  // fills LDS bytes [1024 j, 1024 j + 1024) of a slab, lane l the granule
  // l % kGGran of row (1024 j + 16 l) / kGRow, with global chunk
  // (l % kGGran) ^ qkv_sw(row).
  int voff[kGDma];
#pragma unroll
  for (int u = 0; u < kGDma; ++u) {
    const int j = wave * kGDma + u;
    const int row = (1024 * j + 16 * lane) / kGRow;
    voff[u] = (int)(row * K2) + (((lane % kGGran) ^ qkv_sw(row)) * 16);
  }
  const uint16_t* xb = static_cast<const uint16_t*>(a.x) + (long long)m0 * H;
  const int x_rows = min(a.n - m0, kGM);
  const uint16_t* wb = f0 < qf        ? static_cast<const uint16_t*>(a.wq) + (long long)f0 * H
                       : f0 < qf + kf ? static_cast<const uint16_t*>(a.wk) + (long long)(f0 - qf) * H
                                      : static_cast<const uint16_t*>(a.wv) + (long long)(f0 - qf - kf) * H;
  const int n_slabs = H / kGK;
  // Slab t into ring slot t % kGBufs (x, then the weights); nothing past the
  // last slab.
  auto issue_slab = [&](int t) __attribute__((always_inline)) {
    if (t >= n_slabs) return;
    const int k0 = t * kGK;
    const i32x4 rx = raw_rsrc(xb + k0, (int)(x_rows * K2 - 2LL * k0));
    const i32x4 rw = raw_rsrc(wb + k0, (int)(kGN * K2 - 2LL * k0));
    const uint32_t bx = lds0 + (t % kGBufs) * 2 * kGSlab;
#pragma unroll
    for (int u = 0; u < kGDma; ++u) lds_dma<16>(rx, bx + (wave * kGDma + u) * 1024, voff[u]);
#pragma unroll
    for (int u = 0; u < kGDma; ++u) lds_dma<16>(rw, bx + kGSlab + (wave * kGDma + u) * 1024, voff[u]);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Operand (row r, 16-byte chunk c) of a slab sits at r * kGRow + ((c ^
  // qkv_sw(r)) * 16); lane l reads row l % 32 of its 32-row block (qkv_sw of
  // which depends on l % 32 only), chunk 2 ks + l / 32.
  const int lr = lane & 31;
  const int lh = lane >> 5;
  auto ld_ks = [&](int t, int ks, bf16x8* o) __attribute__((always_inline)) {
    const LdsB* sx = smem + (t % kGBufs) * 2 * kGSlab + (wm * 128 + lr) * kGRow;
    const LdsB* sw = sx + kGSlab + (wn - wm) * 128 * kGRow;
    const int g = ((2 * ks + lh) ^ qkv_sw(lr)) * 16;
    // In the order the MFMAs consume them: x block 0, the weight blocks,
    // then x blocks 1-3.
    o[0] = lds_get<bf16x8>(sx + g);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[4 + j] = lds_get<bf16x8>(sw + j * 32 * kGRow + g);
#pragma unroll
    for (int i = 1; i < 4; ++i) o[i] = lds_get<bf16x8>(sx + i * 32 * kGRow + g);
  };
  auto mfma16 = [&](const bf16x8* o) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[i], o[4 + j], acc[i][j], 0, 0, 0);
  };
  // One k-step: the 16 MFMAs of `cur` with the 8 operand reads of the next
  // step between its first 8 (one read per MFMA), so the reads have the last
  // 8 MFMAs (256 cycles) to land before the next step needs them.
  auto step = [&](const bf16x8* cur, int nt, int nks, bf16x8* nxt) __attribute__((always_inline)) {
    ld_ks(nt, nks, nxt);
    mfma16(cur);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);    // 8 MFMA
    __builtin_amdgcn_sched_barrier(0);
  };
  bf16x8 opa[8], opb[8];
#pragma unroll
  for (int t = 0; t < kGAhead; ++t) issue_slab(t);
  // Slab 0 landed: the kGAhead - 1 later slabs' loads may still be in flight
  // (all of them were issued only if there are that many slabs).
  if (n_slabs >= kGAhead) {
    if constexpr (kGAhead == 3) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(4 * kGDma) : "memory");
    else if constexpr (kGAhead == 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * kGDma) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  ld_ks(0, 0, opa);
  for (int t = 0; t < n_slabs; ++t) {
    // Ring slot (t + kGAhead) % kGBufs last held slab t - 1, which every
    // wavefront finished reading before the previous barrier.
    issue_slab(t + kGAhead);
    if constexpr (kGK == 64) {
      step(opa, t, 1, opb);
      step(opb, t, 2, opa);
      step(opa, t, 3, opb);
    } else {
      step(opa, t, 1, opb);
    }
    // Slab t + 1 landed (every wavefront's part; up to kGAhead - 1 later
    // slabs may still be in flight), and every read of slab t is done.
    if (t + kGAhead < n_slabs) {
      if constexpr (kGAhead == 3) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(4 * kGDma) : "memory");
      else if constexpr (kGAhead == 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * kGDma) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // (After the last slab this reads a stale slot, which nothing uses.)
    step(opb, t + 1, 0, opa);
  }

  // Epilogue 1: + bias, round to bf16, into the output tile [256 tokens][256
  // features] in LDS. Register r of lane l in block (i, j): token
  // 8 (r / 4) + 4 (l / 32) + r % 4 of the block, feature l % 32.
  LdsB* so = smem;
  const void* bsrc = f0 < qf ? a.bq : f0 < qf + kf ? a.bk : a.bv;
  const int bofs = f0 < qf ? f0 : f0 < qf + kf ? f0 - qf : f0 - qf - kf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = wn * 128 + j * 32 + lr;
    const float bf = bsrc ? bf16_to_f32(static_cast<const uint16_t*>(bsrc)[bofs + col]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        lds_put(so + row * kGOutRow + col * 2, f32_to_bf16(acc[i][j][r] + bf));
      }
  }
  __syncthreads();

  // Epilogue 2: rotate and write. Thread tid owns head tid % 16 / CPH of the
  // tile and its chunk pair tid % CPH (8 dimensions of each half) for the
  // tokens tid / 16 + 16 k. The tile is all q, all k or all v features. Work
  // goes in groups of 8 tokens whose position, table and cache-index loads
  // are all issued before any is used, so a group costs one round trip per
  // level of indirection rather than one per token.
  constexpr int HPT = kGN / D;  // heads per tile
  constexpr int CPH = D / 16;   // chunk pairs per head
  static_assert(HPT * CPH == 16, "16 jobs per token");
  const int hh = (tid % 16) / CPH;
  const int d0 = (tid % CPH) * 8;
  const int fh = f0 + hh * D;  // first feature of the head
  const bool is_q = f0 < qf;
  const bool is_v = f0 >= qf + kf;
  const bool rot = a.wr.rope_table != nullptr && !is_v;
  const int kh = is_q ? 0 : (is_v ? fh - qf - kf : fh - qf) / D;
  const uint16_t* tab = static_cast<const uint16_t*>(a.wr.rope_table);
  uint16_t* own = static_cast<uint16_t*>(is_q ? a.q_out : is_v ? a.v_out : a.k_out);
  const int own_heads = is_q ? a.heads : a.kv_heads;
  const int own_h = is_q ? fh / D : kh;
  uint16_t* cache = static_cast<uint16_t*>(is_v ? a.wr.cache_v : a.wr.cache_k);
  const bool to_cache = !is_q && a.wr.cache_kind != 0 && cache != nullptr;
#pragma unroll 1
  for (int g0 = 0; g0 < 16; g0 += 8) {
    int tk[8];
    u32x4 lo[8], hi[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tl = tid / 16 + 16 * (g0 + u);
      tk[u] = m0 + tl;
      lo[u] = lds_get<u32x4>(so + tl * kGOutRow + (hh * D + d0) * 2);
      hi[u] = lds_get<u32x4>(so + tl * kGOutRow + (hh * D + D / 2 + d0) * 2);
    }
    if (rot) {
      int p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = tk[u] < a.n ? a.wr.positions[tk[u]] : 0;
      u32x4 cw[8], sw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pc = p[u] < 0 ? 0 : (p[u] >= a.wr.rope_max_pos ? a.wr.rope_max_pos - 1 : p[u]);
        cw[u] = load16(tab + (long long)pc * (D / 2) + d0);
        sw[u] = load16(tab + ((long long)a.wr.rope_max_pos + pc) * (D / 2) + d0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) rotate_chunk<uint16_t>(lo[u], hi[u], cw[u], sw[u]);
    }
    long long off[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) off[u] = to_cache && tk[u] < a.n ? cache_offset(a.wr, tk[u], kh) : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (tk[u] >= a.n) continue;
      if (own != nullptr) {
        uint16_t* dst = own + ((long long)tk[u] * own_heads + own_h) * D;
        store16(dst + d0, lo[u]);
        store16(dst + D / 2 + d0, hi[u]);
      }
      if (off[u] >= 0) {
        store16(cache + off[u] + d0, lo[u]);
        store16(cache + off[u] + D / 2 + d0, hi[u]);
      }
    }
  }
}

hipError_t launch_qkv(const QkvArgs& a, hipStream_t stream) {
  const int qf = a.heads * a.head_dim, kf = a.kv_heads * a.head_dim;
  const int features = qf + 2 * kf;
  // (Lane offsets into a tile's rows are 32-bit: 256 rows of the hidden size.)
  if (GQA_QKV_LARGE_TILES && qf % kGN == 0 && kf % kGN == 0 && (long long)kGM * 2 * a.hidden < (1LL << 31)) {
    const int tiles_m = (a.n + kGM - 1) / kGM, tiles_n = features / kGN;
    const dim3 grid(tiles_m * tiles_n), block(256);
    if (a.head_dim == 64) qkv256_kernel<64><<<grid, block, 0, stream>>>(a, tiles_m, tiles_n);
    else qkv256_kernel<128><<<grid, block, 0, stream>>>(a, tiles_m, tiles_n);
    return hipGetLastError();
  }
  const dim3 grid(features / kBN, (a.n + kBM - 1) / kBM), block(256);
  if (a.head_dim == 64) qkv_kernel<64><<<grid, block, 0, stream>>>(a);
  else qkv_kernel<128><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gqa
