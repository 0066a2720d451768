// Device body of the matrix-core split-K decode (the design is described in
// decode_mfma.hip): shared by the decode kernel and by the combined step
// kernel, whose workgroups run either a decode share or a prefill tile.
#pragma once

#include "common.h"
#include "internal.h"

namespace gqa {

constexpr float kDecNegInf = -__builtin_huge_valf();
constexpr int kDecChunk = 32;  // keys per chunk (half a page)

// Chunk row m of the QK block mb holds key 8 * (m / 4) + 4 * mb + m % 4.
__device__ __forceinline__ int dec_chunk_row_key(int mb, int m) {
  return 8 * (m >> 2) + 4 * mb + (m & 3);
}
// Swizzle of the 16-byte granule (8 keys) in row d of a V^T tile.
__device__ __forceinline__ int dec_vt_swz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }
// Swizzle of the 16-byte granule in key row k of a K tile: the 8 rows that 8
// consecutive lanes read for one operand (k = 0-3 and 8-11, +4, +16) land in 8
// distinct bank groups.
__device__ __forceinline__ int dec_kt_swz(int k) { return (k & 3) | ((k >> 1) & 4); }

// LDS of one workgroup of NW wavefronts: NW wavefront-private tiles of 32 x D
// bf16 (K [32 keys][D], then V^T [D][32 keys]), reused at the end for the
// cross-wavefront combine [NW][16][D + 2] floats; then Q [16][D].
template <int D, int NW>
constexpr int decode_mfma_main_bytes() {
  return NW * D * kDecChunk * 2 > NW * 16 * (D + 2) * 4 ? NW * D * kDecChunk * 2 : NW * 16 * (D + 2) * 4;
}
template <int D, int NW>
constexpr int decode_mfma_lds_bytes() {
  return decode_mfma_main_bytes<D, NW>() + 16 * D * 2;
}

// One workgroup's share of the decode: (row, KV head, split of keys) for NW
// wavefronts, in `smem` (decode_mfma_lds_bytes<D, NW>() bytes, 16-byte
// aligned). Every thread of the workgroup calls it.
template <int D, bool PAGED, int NW, bool SORTED, bool PF = false>
__device__ __forceinline__ void decode_mfma_body(const DecodeArgs& a, int split, int kh, int rz,
                                                 char* smem) {
  constexpr int KK = D / 32;               // 32-wide k-steps of QK over the head dim
  constexpr int NB = D / 16;               // 16-wide d-blocks of O
  constexpr int VROWS = D == 128 ? 8 : 4;  // V rows loaded per lane per chunk
  constexpr int VC = D / 8;                // 16-byte column chunks per V row
  constexpr int kMainBytes = decode_mfma_main_bytes<D, NW>();
  constexpr int kChunk = kDecChunk;
  uint16_t* q_s = reinterpret_cast<uint16_t*>(smem + kMainBytes);
  // Sorted dispatch (one split, at most 64 rows): workgroups start in
  // blockIdx order, so ranking the rows by attended keys makes the longest
  // start first.
  const int r = SORTED ? __builtin_amdgcn_readfirstlane(row_of_rank(a.positions, a.rows, a.cap, a.window, rz))
                       : rz;
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
  float m_run = kDecNegInf, l_run = 0.f;

  const int c_begin = t0 / kChunk;
  const int c_end = (t1 + kChunk - 1) / kChunk;
  // Chunk c's K and V rows, 16 bytes per lane each: lane (vc, vg) reads
  // column 8 vc of rows vg * VROWS + i. Keys outside [t0, t1) read a clamped
  // in-range row and are masked when the chunk is processed.
  auto chunk_row0 = [&](int c, bool& ok) -> long long {
    const int tb = c * kChunk;
    ok = true;
    if (PAGED) {
      int page = a.table[(long long)r * a.pages + tb / kPageSize];
      if (page < 0 || page >= a.num_pages) {  // no keys from this page
        ok = false;
        page = 0;                              // a real page, read and masked
      }
      return (((long long)page * a.kv_heads + kh) * kPageSize + tb % kPageSize) * D;
    }
    return (((long long)r * a.kv_heads + kh) * a.cap + tb) * D;
  };
  auto load_rows = [&](const uint16_t* base, int c, long long row0, u32x4* x) {
    const int tb = c * kChunk;
#pragma unroll
    for (int i = 0; i < VROWS; ++i) {
      const int t = min(max(tb + vg * VROWS + i, t0), t1 - 1);
      x[i] = load16_stream(base + row0 + (long long)(t - tb) * D + vc * 8);
    }
  };
  // Fold chunk c (rows already in kx, vx) into the running state. With
  // c_next >= 0 the rows of chunk c_next are loaded into kx (vx) as soon as
  // chunk c's K (V) has gone to LDS, so a wavefront always has a chunk's
  // loads in flight while it computes; ok_next says whether c_next's page
  // is valid.
  auto process_chunk = [&](int c, u32x4* kx, u32x4* vx, bool ok, int c_next, bool& ok_next) {
    const int tb = c * kChunk;
    // K -> LDS tile [32 keys][D], granule g of key k at g ^ dec_kt_swz(k).
#pragma unroll
    for (int i = 0; i < VROWS; ++i) {
      const int k = vg * VROWS + i;
      store16(my_vt + k * D + ((vc ^ dec_kt_swz(k)) * 8), kx[i]);
    }
    long long row0_next = 0;
    if (c_next >= 0) {
      row0_next = chunk_row0(c_next, ok_next);
      load_rows(kbase, c_next, row0_next, kx);
    }
    __builtin_amdgcn_wave_barrier();

    // S^T = K Q^T for the chunk's 32 keys: two 16-key blocks.
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int k = dec_chunk_row_key(mb, ln);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 kv = load16(my_vt + k * D + (((4 * kk + lg) ^ dec_kt_swz(k)) * 8));
        const u32x4 qv = load16(q_s + ln * D + kk * 32 + lg * 8);
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                        __builtin_bit_cast(bf16x8, qv), s[mb], 0,
                                                        0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const bool full = ok && tb >= t0 && tb + kChunk <= t1;
    // Lane (head ln, group lg) holds keys 8 lg + 4 mb + i.
    float tmax = kDecNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!full) {
          const int t = tb + 8 * lg + 4 * mb + i;
          s[mb][i] = (ok & (t >= t0) & (t < t1)) ? s[mb][i] : kDecNegInf;
        }
        tmax = fmaxf(tmax, s[mb][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * a.scale_log2;
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kDecNegInf) ? 0.f : m_new;
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
        if (!(ok & (t >= t0) & (t < t1))) vx[i] = u32x4{0u, 0u, 0u, 0u};
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
        store16(my_vt + d * kChunk + ((vg ^ dec_vt_swz(d)) * 8), pk);
      } else {
        u32x2 pk;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          pk[j] = ((vx[2 * j][w] >> sh) & 0xffffu) | (((vx[2 * j + 1][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(my_vt + d * kChunk + (((vg >> 1) ^ dec_vt_swz(d)) * 8) +
                                  (vg & 1) * 4) = pk;
      }
    }
    if (c_next >= 0) load_rows(vbase, c_next, row0_next, vx);
    __builtin_amdgcn_wave_barrier();
    // O += P V: B operand lane (n = d % 16, g) = V^T[16 nb + n][8 g ..].
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int d = nb * 16 + ln;
      const u32x4 vb = load16(my_vt + d * kChunk + ((lg ^ dec_vt_swz(d)) * 8));
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                      __builtin_bit_cast(bf16x8, vb), o[nb], 0, 0,
                                                      0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  if (PF) {
    // Loads of the next chunk overlap the current chunk's work. Past the
    // end, the last chunk is loaded again and never processed.
    u32x4 kx[VROWS], vx[VROWS];
    int c = c_begin + wave;
    bool ok;
    const long long row0 = chunk_row0(min(c, c_end - 1), ok);
    load_rows(kbase, min(c, c_end - 1), row0, kx);
    load_rows(vbase, min(c, c_end - 1), row0, vx);
    for (; c < c_end; c += NW) {
      bool ok_next;
      process_chunk(c, kx, vx, ok, min(c + NW, c_end - 1), ok_next);
      ok = ok_next;
    }
  } else {
    for (int c = c_begin + wave; c < c_end; c += NW) {
      u32x4 kx[VROWS], vx[VROWS];
      bool ok, unused;
      const long long row0 = chunk_row0(c, ok);
      if (!ok) continue;  // no keys from this page
      load_rows(kbase, c, row0, kx);
      load_rows(vbase, c, row0, vx);
      process_chunk(c, kx, vx, true, -1, unused);
    }
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
    float M = kDecNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red[(w * 16 + hh) * RS]);
    float acc = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red[(w * 16 + hh) * RS];
      const float sc = (mw == kDecNegInf) ? 0.f : fast_exp2(mw - M);
      acc += sc * red[(w * 16 + hh) * RS + 2 + d];
      den += sc * red[(w * 16 + hh) * RS + 1];
    }
    if (a.nsplit == 1) {
      // The only split: normalize here; the sink joins the denominator.
      if (a.sinks != nullptr) {
        const float s2 = bf16_to_f32(static_cast<const uint16_t*>(a.sinks)[h0 + hh]) * kLog2e;
        const float Ms = fmaxf(M, s2);
        const float f = (M == kDecNegInf) ? 0.f : fast_exp2(M - Ms);
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

}  // namespace gqa
