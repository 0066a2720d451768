// Split-K decode attention on bf16 matrix cores (gfx950), contiguous or paged.
//
// Same result as decode.hip -- `decode` / decode_rows / decode_paged of the
// Linnet "examples/01-llama" page and the Nest llama-3.1-8b-instruct card,
// with SinkAttention's window (Nest gpt-oss-20b card) -- for bf16 caches, head
// dims 64 / 128 and up to 16 query heads per KV head. Decode is HBM-bound
// (about 2 flops per byte at G = 4), so the kernel is shaped for memory-level
// parallelism with few instructions per byte:
// * A workgroup of NW wavefronts owns one (row, KV head, split of keys); its
//   wavefronts take 32-key chunks round-robin, each keeping its own online
//   softmax state, combined once at the end. Long splits and many resident
//   wavefronts (<= 128 VGPRs: 4 per SIMD) keep the page streams few and deep.
// * Every chunk's 16 loads (8 for K, 8 for V, 16 bytes per lane, nontemporal)
//   are issued at once, unconditionally: addresses are clamped into the
//   split's key range and out-of-range keys are masked afterwards by
//   selection. No branch guards a load, so the compiler's wait counters stay
//   precise, and poisoned slots past a row's position never reach the result.
// * Each load instruction of a wavefront reads whole cache rows (contiguous
//   runs of 256 or 128 bytes): measured on the paged pattern, nontemporal
//   loads of whole rows stream ~20% faster than loads shaped like the matrix
//   operands (64 bytes from each of 16 rows).
// * K is therefore staged through a wavefront-private LDS tile (XOR-swizzled
//   16-byte granules) and read back as the A operand of S^T = K Q^T on
//   v_mfma_f32_16x16x32_bf16; the G query heads (padded to 16) are the B
//   operand, staged once per workgroup in LDS.
// * The key order inside a chunk is permuted so the probabilities a lane holds
//   after the softmax are exactly the A operand of O = P V.
// * V is written transposed into the same LDS tile once K has been read and
//   read back as the B operand. Only the issuing wavefront touches its tile
//   (LDS operations of one wavefront execute in order), so no workgroup
//   barrier is needed inside the loop.
// * The split length is chosen per call: as long as possible while the grid
//   still fills the chip. With a single split per (row, KV head) the kernel
//   also normalizes (and adds the sink) and writes the output directly.
// * With one split and at most 64 rows the workgroups take the rows in order
//   of decreasing key count, ranked on the device from the positions: only
//   one workgroup fits a CU at D = 128, so the grid runs in rounds, and
//   starting the longest rows first keeps the last round short.
// * A chunk whose page id is out of range contributes nothing.
// The merge of the split partials (and the sink term) is shared with the
// vector-ALU path in decode.hip.
#include "common.h"
#include "internal.h"

namespace gqa {

namespace {
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kChunk = 32;  // keys per chunk (half a page)
#ifndef GQA_DECODE_TARGET_WGS
#define GQA_DECODE_TARGET_WGS 512
#endif
#ifndef GQA_DECODE_WAVES
#define GQA_DECODE_WAVES 8
#endif
#ifndef GQA_DECODE_MIN_WAVES_PER_SIMD
#define GQA_DECODE_MIN_WAVES_PER_SIMD 3
#endif
constexpr int kWaves = GQA_DECODE_WAVES;  // wavefronts per workgroup

// Chunk row m of the QK block mb holds key 8 * (m / 4) + 4 * mb + m % 4.
__device__ __forceinline__ int chunk_row_key(int mb, int m) {
  return 8 * (m >> 2) + 4 * mb + (m & 3);
}
// Swizzle of the 16-byte granule (8 keys) in row d of a V^T tile.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }
// Swizzle of the 16-byte granule in key row k of a K tile: the 8 rows that 8
// consecutive lanes read for one operand (k = 0-3 and 8-11, +4, +16) land in 8
// distinct bank groups.
__device__ __forceinline__ int kt_swz(int k) { return (k & 3) | ((k >> 1) & 4); }
}  // namespace

#ifndef GQA_DECODE_SORTED_WAVES
#define GQA_DECODE_SORTED_WAVES 8
#endif
constexpr int kWavesSorted = GQA_DECODE_SORTED_WAVES;  // ... with sorted dispatch

template <int D, bool PAGED, int NW, bool SORTED>
__global__ __launch_bounds__(64 * NW, NW == kWaves ? GQA_DECODE_MIN_WAVES_PER_SIMD : 1) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;               // 32-wide k-steps of QK over the head dim
  constexpr int NB = D / 16;               // 16-wide d-blocks of O
  constexpr int VROWS = D == 128 ? 8 : 4;  // V rows loaded per lane per chunk
  constexpr int VC = D / 8;                // 16-byte column chunks per V row
  // NW wavefront-private tiles of 32 x D bf16 (K [32 keys][D], then V^T
  // [D][32 keys]), reused at the end for the cross-wavefront combine
  // [NW][16][D + 2] floats; then Q [16][D].
  constexpr int kTileBytes = NW * D * kChunk * 2;
  constexpr int kRedBytes = NW * 16 * (D + 2) * 4;
  constexpr int kMainBytes = kTileBytes > kRedBytes ? kTileBytes : kRedBytes;
  __shared__ __attribute__((aligned(16))) char smem[kMainBytes + 16 * D * 2];
  uint16_t* q_s = reinterpret_cast<uint16_t*>(smem + kMainBytes);

  const int split = blockIdx.x;
  const int kh = blockIdx.y;
  // Sorted dispatch (one split, at most 64 rows): workgroups start in
  // blockIdx order, so ranking the rows by attended keys makes the longest
  // start first.
  const int r = SORTED ? __builtin_amdgcn_readfirstlane(row_of_rank(a.positions, a.rows, a.cap, a.window, blockIdx.z))
                       : blockIdx.z;
  const int G = a.heads / a.kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform in a scalar register, so chunk indices and page-table reads
  // stay on the scalar unit.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15;  // MFMA column / row within 16
  const int lg = lane >> 4;  // lane group 0..3

  int lo, hi;
  decode_key_range(a.positions[r], a.cap, a.window, lo, hi);
  const int t0 = max(lo, split * a.split_len);
  const int t1 = min(hi + 1, (split + 1) * a.split_len);
  if (t0 >= t1) {
    // No keys in this split. The merge never reads a split outside [lo, hi];
    // with a single split this workgroup owns the output, which is 0.
    if (a.nsplit == 1) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + ((long long)r * a.heads + kh * G) * D;
      for (int x = tid; x < G * D; x += 64 * NW) out[x] = 0;
    }
    return;
  }

  // Stage the G query heads (zero rows up to 16) in LDS.
  const int h0 = kh * G;
  for (int x = tid; x < 16 * D / 8; x += 64 * NW) {
    const int hh = x / (D / 8);
    const int c8 = x % (D / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (hh < G)
      v = load16(static_cast<const uint16_t*>(a.q) + ((long long)r * a.heads + h0 + hh) * D + c8 * 8);
    store16(q_s + hh * D + c8 * 8, v);
  }
  __syncthreads();

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v);
  uint16_t* my_vt = reinterpret_cast<uint16_t*>(smem) + wave * D * kChunk;
  const int vc = lane % VC;
  const int vg = lane / VC;

  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int c_begin = t0 / kChunk;
  const int c_end = (t1 + kChunk - 1) / kChunk;
  for (int c = c_begin + wave; c < c_end; c += NW) {
    const int tb = c * kChunk;
    // Offset of key 0 of the chunk: page table for paged caches.
    long long row0;
    if (PAGED) {
      const int page = a.table[(long long)r * a.pages + tb / kPageSize];
      if (page < 0 || page >= a.num_pages) continue;  // no keys from this page
      row0 = (((long long)page * a.kv_heads + kh) * kPageSize + tb % kPageSize) * D;
    } else {
      row0 = (((long long)r * a.kv_heads + kh) * a.cap + tb) * D;
    }
    // Keys outside [t0, t1) read a clamped in-range row and are masked below.
    auto key_row = [&](int key) {
      const int t = min(max(tb + key, t0), t1 - 1);
      return (long long)(t - tb) * D;
    };
    const uint16_t* kr = kbase + row0;
    const uint16_t* vr_ = vbase + row0;
    // Whole-row loads: lane (vc, vg) reads 16 bytes at column 8 vc of rows
    // vg * VROWS + i, for K and for V.
    u32x4 kx[VROWS], vx[VROWS];
#pragma unroll
    for (int i = 0; i < VROWS; ++i) kx[i] = load16_stream(kr + key_row(vg * VROWS + i) + vc * 8);
#pragma unroll
    for (int i = 0; i < VROWS; ++i) vx[i] = load16_stream(vr_ + key_row(vg * VROWS + i) + vc * 8);
    // K -> LDS tile [32 keys][D], granule g of key k at g ^ kt_swz(k).
#pragma unroll
    for (int i = 0; i < VROWS; ++i) {
      const int k = vg * VROWS + i;
      store16(my_vt + k * D + ((vc ^ kt_swz(k)) * 8), kx[i]);
    }
    __builtin_amdgcn_wave_barrier();

    // S^T = K Q^T for the chunk's 32 keys: two 16-key blocks.
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int k = chunk_row_key(mb, ln);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 kv = load16(my_vt + k * D + (((4 * kk + lg) ^ kt_swz(k)) * 8));
        const u32x4 qv = load16(q_s + ln * D + kk * 32 + lg * 8);
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                        __builtin_bit_cast(bf16x8, qv), s[mb], 0,
                                                        0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const bool full = tb >= t0 && tb + kChunk <= t1;
    // Lane (head ln, group lg) holds keys 8 lg + 4 mb + i.
    float tmax = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!full) {
          const int t = tb + 8 * lg + 4 * mb + i;
          s[mb][i] = ((t >= t0) & (t < t1)) ? s[mb][i] : kNegInf;
        }
        tmax = fmaxf(tmax, s[mb][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * a.scale_log2;
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float p[8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[4 * mb + i] = fast_exp2(__builtin_fmaf(s[mb][i], a.scale_log2, -m_use));
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    m_run = m_new;
    u32x4 pa;
#pragma unroll
    for (int j = 0; j < 4; ++j) pa[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
    // O rows are heads 4 lg + i; their alphas live in lanes 4 lg + i.
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * lg + i, 64);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb][i] *= ai;
      }
    }
    // Zero the V rows of masked keys (their clamped loads read a real row).
    if (!full) {
#pragma unroll
      for (int i = 0; i < VROWS; ++i) {
        const int t = tb + vg * VROWS + i;
        if (!((t >= t0) & (t < t1))) vx[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    // V^T into this wavefront's LDS tile [D][32 keys].
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = vc * 8 + e;
      const int w = e >> 1;
      const int sh = (e & 1) * 16;
      if (VROWS == 8) {
        u32x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pk[j] = ((vx[2 * j][w] >> sh) & 0xffffu) |
                  (((vx[(2 * j + 1) % VROWS][w] >> sh) & 0xffffu) << 16);
        store16(my_vt + d * kChunk + ((vg ^ vt_swz(d)) * 8), pk);
      } else {
        u32x2 pk;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          pk[j] = ((vx[2 * j][w] >> sh) & 0xffffu) | (((vx[2 * j + 1][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(my_vt + d * kChunk + (((vg >> 1) ^ vt_swz(d)) * 8) +
                                  (vg & 1) * 4) = pk;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // O += P V: B operand lane (n = d % 16, g) = V^T[16 nb + n][8 g ..].
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int d = nb * 16 + ln;
      const u32x4 vb = load16(my_vt + d * kChunk + ((lg ^ vt_swz(d)) * 8));
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                      __builtin_bit_cast(bf16x8, vb), o[nb], 0, 0,
                                                      0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Combine the wavefronts' states in LDS (reusing the V^T tiles).
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [NW][16][D + 2]
  constexpr int RS = D + 2;
  if (lg == 0) {
    red[(wave * 16 + ln) * RS + 0] = m_run;
    red[(wave * 16 + ln) * RS + 1] = l_run;
  }
  // o[nb][i] is head 4 lg + i, dimension 16 nb + ln.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * lg + i;
    if (hh < G) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[(wave * 16 + hh) * RS + 2 + nb * 16 + ln] = o[nb][i];
    }
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 64 * NW) {
    const int hh = x / D;
    const int d = x % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red[(w * 16 + hh) * RS]);
    float acc = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red[(w * 16 + hh) * RS];
      const float sc = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      acc += sc * red[(w * 16 + hh) * RS + 2 + d];
      den += sc * red[(w * 16 + hh) * RS + 1];
    }
    if (a.nsplit == 1) {
      // The only split: normalize here; the sink joins the denominator.
      if (a.sinks != nullptr) {
        const float s2 = bf16_to_f32(static_cast<const uint16_t*>(a.sinks)[h0 + hh]) * kLog2e;
        const float Ms = fmaxf(M, s2);
        const float f = (M == kNegInf) ? 0.f : fast_exp2(M - Ms);
        acc *= f;
        den = den * f + fast_exp2(s2 - Ms);
      }
      static_cast<uint16_t*>(a.out)[((long long)r * a.heads + h0 + hh) * D + d] =
          f32_to_bf16(den > 0.f ? acc / den : 0.f);
    } else {
      float* part = a.ws + (((long long)r * a.heads + h0 + hh) * a.nsplit + split) * (D + 2);
      part[2 + d] = acc;
      if (d == 0) {
        part[0] = M;
        part[1] = den;
      }
    }
  }
}

bool decode_mfma_supported(const DecodeArgs& a) {
  const int G = a.heads / a.kv_heads;
  return a.dtype == kDtypeBf16 && (a.head_dim == 64 || a.head_dim == 128) && G <= 16;
}

// Longest split (a multiple of the page size) that still gives about
// GQA_DECODE_TARGET_WGS workgroups, at least 1024 keys.
int decode_mfma_split_len(int rows, int kv_heads, int cap) {
  const long long units = (long long)rows * kv_heads;
  long long nsplit = (GQA_DECODE_TARGET_WGS + units - 1) / units;
  const long long max_split = (cap + 1023) / 1024;
  if (nsplit > max_split) nsplit = max_split;
  if (nsplit < 1) nsplit = 1;
  long long len = (cap + nsplit - 1) / nsplit;
  len = (len + kPageSize - 1) / kPageSize * kPageSize;
  return (int)len;
}

template <int D, bool PAGED>
static void launch_mfma_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.nsplit, a.kv_heads, a.rows);
  if (a.nsplit == 1 && a.rows <= kSortMaxRows)
    decode_mfma_kernel<D, PAGED, kWavesSorted, true><<<grid, dim3(64 * kWavesSorted), 0, stream>>>(a);
  else
    decode_mfma_kernel<D, PAGED, kWaves, false><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) {
    if (a.paged) launch_mfma_t<128, true>(a, stream);
    else launch_mfma_t<128, false>(a, stream);
  } else {
    if (a.paged) launch_mfma_t<64, true>(a, stream);
    else launch_mfma_t<64, false>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace gqa
