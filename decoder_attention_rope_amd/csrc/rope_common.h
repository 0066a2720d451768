// Rotation and cache addressing shared by the rope + KV-write pass and the
// fused projection kernel.
//
// `rope` of the Linnet "examples/01-llama" page (src/attention.linnet) pairs
// dimension i with i + D/2 (rotate-half); the rotation of T values by T table
// entries is the exact value rounded once to T (bf16: an f32 fma of exact
// products, fp64 for the rare f32 results on a bf16 midpoint; f32: fp64,
// where the f32 x f32 products are exact). write_at ("a masked select", section Key
// ideas) drops a write whose target is outside the cache; the serving entries
// of the Nest llama-3.1-8b-instruct card address the cache by row and
// position, by table page, or by physical slot.
#pragma once

#include "common.h"
#include "internal.h"

namespace gqa {

template <typename T>
__device__ __forceinline__ void rotate_chunk(u32x4& lo, u32x4& hi, const u32x4& cw,
                                             const u32x4& sw);

// bf16: 8 elements per 16-byte chunk. A product of two bf16 values is exact
// in f32, so fma(a, b, c * d) is the exact a b + c d rounded once to f32.
// Rounding that f32 to bf16 (nearest-even) gives the correctly rounded
// result unless the f32 value sits exactly on a bf16 midpoint (low 16 bits
// 0x8000): a bf16 midpoint is itself an f32 value, so the first rounding can
// land on one but never cross one. Only then is the value recomputed in fp64
// and rounded once.
__device__ __forceinline__ uint16_t rot_bf16(float a, float b, float c, float d) {
  const float y = __builtin_fmaf(a, b, c * d);
  if ((__float_as_uint(y) & 0xffffu) != 0x8000u) return f32_to_bf16(y);
  return f64_to_bf16((double)a * (double)b + (double)c * (double)d);
}

template <>
__device__ __forceinline__ void rotate_chunk<uint16_t>(u32x4& lo, u32x4& hi, const u32x4& cw,
                                                       const u32x4& sw) {
  float xl[8], xh[8], c[8], s[8];
  Elem<uint16_t>::to_f32(lo, xl);
  Elem<uint16_t>::to_f32(hi, xh);
  Elem<uint16_t>::to_f32(cw, c);
  Elem<uint16_t>::to_f32(sw, s);
  uint16_t yl[8], yh[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    yl[e] = rot_bf16(xl[e], c[e], -xh[e], s[e]);
    yh[e] = rot_bf16(xh[e], c[e], xl[e], s[e]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = (uint32_t)yl[2 * i] | ((uint32_t)yl[2 * i + 1] << 16);
    hi[i] = (uint32_t)yh[2 * i] | ((uint32_t)yh[2 * i + 1] << 16);
  }
}

// f32: 4 elements per chunk.
template <>
__device__ __forceinline__ void rotate_chunk<float>(u32x4& lo, u32x4& hi, const u32x4& cw,
                                                    const u32x4& sw) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double xl = (double)__uint_as_float(lo[e]);
    const double xh = (double)__uint_as_float(hi[e]);
    const double c = (double)__uint_as_float(cw[e]);
    const double s = (double)__uint_as_float(sw[e]);
    lo[e] = __float_as_uint((float)(xl * c - xh * s));
    hi[e] = __float_as_uint((float)(xh * c + xl * s));
  }
}

// Element offset of token t / kv head kh in the cache, or -1 when write_at
// masks the write out.
__device__ __forceinline__ long long cache_offset(const RopeWriteArgs& a, int t, int kh) {
  const int D = a.head_dim;
  switch (a.cache_kind) {
    case 1: {  // contiguous [batch, kv_heads, max_seq, D]
      const int row = a.rows ? a.rows[t] : 0;
      const int pos = a.positions[t];
      if (row < 0 || row >= a.cache_dim0 || pos < 0 || pos >= a.cache_seq) return -1;
      return (((long long)row * a.kv_heads + kh) * a.cache_seq + pos) * D;
    }
    case 2: {  // paged, logical position through the table
      const int row = a.rows ? a.rows[t] : 0;
      const long long pos = a.positions[t];
      if (row < 0 || row >= a.table_rows) return -1;
      if (pos < 0 || pos >= (long long)a.table_pages * kPageSize) return -1;
      const int page = a.table[(long long)row * a.table_pages + pos / kPageSize];
      if (page < 0 || page >= a.cache_dim0) return -1;
      return (((long long)page * a.kv_heads + kh) * kPageSize + pos % kPageSize) * D;
    }
    case 3: {  // paged, physical slot
      const long long slot = a.slots[t];
      if (slot < 0 || slot >= (long long)a.cache_dim0 * kPageSize) return -1;
      return (((slot / kPageSize) * a.kv_heads + kh) * kPageSize + slot % kPageSize) * D;
    }
    default:
      return -1;
  }
}

}  // namespace gqa
