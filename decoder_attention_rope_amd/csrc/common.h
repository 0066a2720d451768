// Device-side helpers shared by the gfx950 kernels of the attention library:
// bf16 <-> f32 conversion, exact rounding of fp64 results to T, wavefront
// shuffles, and the MFMA operand vector types. Nothing here is visible
// through the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPageSize = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// bf16 storage is raw 16-bit patterns (uint16_t); arithmetic is f32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN. One
// v_cvt_pk_bf16_f32: the hardware converter rounds every finite and infinite
// f32 exactly as the integer nearest-even formula
// (u + 0x7fff + ((u >> 16) & 1)) >> 16 does (checked over all 2^32 patterns),
// so results compared bit for bit are unchanged. The empty asm keeps the f32
// value opaque: otherwise the compiler folds a preceding fp64 -> f32
// conversion into one fp64 -> bf16 rounding, which differs from rounding
// through f32 (the rotary tables depend on the two steps).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  asm("" : "+v"(f));
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two f32 -> packed bf16 with one v_cvt_pk_bf16_f32 (nearest-even, as
// f32_to_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Interleave the low (high) 16-bit halves of two words: a's half in the low
// 16 bits of the result, b's in the high 16 (one v_perm_b32).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Online softmax with a lazy reference: the reference max moves only when a
// new score exceeds it by more than 2^kLazyMaxLog2 (scores in log2 units), so
// the running output rarely needs rescaling. Probabilities stay below
// 2^kLazyMaxLog2, far inside the f32 and bf16 ranges, and the output and the
// denominator share the reference, so the normalized result is unchanged.
constexpr float kLazyMaxLog2 = 8.0f;

// 2^x on the transcendental unit (v_exp_f32); the attention kernels only
// evaluate it for x <= 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp64 -> f32 with round-to-odd: truncate toward zero, then force the last
// bit to 1 when inexact. A second rounding of that value to any format with
// at most 22 significant bits (bf16 has 8) is then the correctly rounded
// (nearest-even) result of the original fp64 value.
__device__ __forceinline__ float f64_to_f32_round_odd(double x) {
  float f = (float)x;
  double back = (double)f;
  if (back != x && !__builtin_isnan(x)) {
    uint32_t u = __float_as_uint(f);
    if (__builtin_fabs(back) > __builtin_fabs(x)) u -= 1u;  // step toward zero
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f;
}

// fp64 -> bf16, nearest-even, exactly (single rounding).
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  return f32_to_bf16(f64_to_f32_round_odd(x));
}

// ---------------------------------------------------------------------------
// Element traits: 16-byte vectors of T and their f32 view.
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16
  static constexpr int kPer16B = 8;
  __device__ __forceinline__ static void to_f32(const u32x4& w, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_lo(w[i]);
      out[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ __forceinline__ static void to_f32(const u32x4& w, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming load (nontemporal hint): for data read once, such as the KV cache
// in decode.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// Wavefront (64-lane) reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Key range [lo, hi] a decode query at `pos` attends in a cache of `cap`
// logical slots: seen = slot <= pos, window W > 0 keeps pos - slot < W.
// Empty when hi < lo.
__device__ __forceinline__ void decode_key_range(int pos, int cap, int window, int& lo,
                                                 int& hi) {
  hi = pos < cap - 1 ? pos : cap - 1;
  long long l = 0;
  if (window > 0) {
    long long w0 = (long long)pos - (long long)window + 1;
    l = w0 > 0 ? w0 : 0;
  }
  lo = (int)(l < (long long)cap ? l : (long long)cap);
}

// Largest batch the decode kernels rank on the device (one row per lane).
constexpr int kSortMaxRows = 64;

// Row of rank k when rows (at most 64) are ordered by the number of keys they
// attend, longest first (ties by row index). Every wavefront of the caller
// computes it on its own: lane l holds row l's key count and counts the rows
// ahead of it.
__device__ __forceinline__ int row_of_rank(const int32_t* positions, int rows, int cap, int window,
                                           int k) {
  const int lane = threadIdx.x & 63;
  int n = -1;  // lanes past the last row never match
  if (lane < rows) {
    int lo, hi;
    decode_key_range(positions[lane], cap, window, lo, hi);
    n = hi >= lo ? hi - lo + 1 : 0;
  }
  int rank = 0;
  for (int j = 0; j < rows; ++j) {
    const int nj = __builtin_amdgcn_readlane(n, j);
    rank += (nj > n) | ((nj == n) & (j < lane));
  }
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < rows && rank == k);
  return (int)__builtin_ctzll(hit);
}

}  // namespace gqa
