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
//   holds both halves (d, d + D/2) of a head chunk; the rotation is exact in
//   fp64 and rounded once to T (the same helper as the rope pass).
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"
#include "rope_common.h"

namespace gqa {

namespace {
constexpr int kBM = 128;            // tokens per workgroup tile
constexpr int kBN = 128;            // output features per workgroup tile
constexpr int kBK = 64;             // hidden (K) per slab
constexpr int kRow = kBK * 2 + 16;  // LDS row stride of a staged slab (bytes)
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
  const int n_slabs = H / kBK;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int t = 0; t < n_slabs; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_slabs) load_slab((t + 1) * kBK);
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
    unroll<kBK / 16>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      if constexpr (ks + 1 < kBK / 16) ld_ks(std::integral_constant<int, ks + 1>{});
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

hipError_t launch_qkv(const QkvArgs& a, hipStream_t stream) {
  const int features = (a.heads + 2 * a.kv_heads) * a.head_dim;
  const dim3 grid(features / kBN, (a.n + kBM - 1) / kBM), block(256);
  if (a.head_dim == 64) qkv_kernel<64><<<grid, block, 0, stream>>>(a);
  else qkv_kernel<128><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gqa
