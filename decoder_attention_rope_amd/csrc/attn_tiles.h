// Tile machinery shared by the packed-prefill attention kernels (forward and
// backward) on gfx950: key-tile summaries and the prepared walk, LDS access
// helpers, lane-pair reductions, direct buffer-to-LDS loads.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "internal.h"

namespace gqa {

constexpr int kBK = 64;       // keys per tile
constexpr int kPrepThreads = 1024;
constexpr int kMaskWords = 6;  // 32-bit words per (query tile, group of 64 key tiles)
constexpr int kRecInts = 16;   // ints per start record (64 bytes)
constexpr int kRecVis = 12;    // visit-list entries copied into a start record
constexpr int kVisMode = 24;   // visit-list entry: kt | mode << kVisMode
constexpr float kNegInf = -__builtin_huge_valf();
// Bytes by which a tile's buffer descriptor starts before the tile (see the
// shared-M0 loads in the prefill kernel); the host keeps every packed
// operand's range, p * row bytes + kShift, below 2^31.
constexpr int kShift = 4096;

// Per tile of tokens: [min, max] of segments and positions, and the smallest
// position among the tokens of segment seg_min (pos_first) and of segment
// seg_max (pos_last).
struct TileSum {
  int seg_min, seg_max, pos_min, pos_max, pos_first, pos_last, pad0, pad1;
};

struct Plan {
  TileSum* ksum;   // [n_kt]
  TileSum* qsum;   // [n_qt]
  int2* qrange;    // [n_qt] first / last key tile to visit
  int* order;      // [n_qt] query tiles, costliest first
  int* cost;       // [n_qt] key tiles each query tile visits
  uint32_t* masks; // [n_qt][n_kg][kMaskWords]: per group of 64 key tiles,
                   // 64-bit masks "visit", "every pair allowed" and "one
                   // segment" (see tiles_oneseg)
  int* rec;        // [n_qt][kRecInts] or null: per ordered slot i, the start
                   // of its walk in one record -- query tile order[i], the
                   // numbers of fully allowed and of masked key tiles it
                   // visits, and its first kRecVis visit-list entries
  int* vis;        // [n_qt][n_kt] or null (packed keys): per query tile the
                   // key tiles it visits, in walk order, as entries
                   // kt | mode << kVisMode (mode 0: every pair allowed, 1: one
                   // segment, positions decide, 2: the full predicate); the
                   // fully allowed tiles first, then the others, each in
                   // increasing kt
  int* nfull;      // [n_qt] fully allowed tiles in each visit list
  int n_kt, n_qt, n_kg, tq, head_groups, gw;
  int max_cost;    // costs are clamped to [0, max_cost] for the ordering
  int resident;    // forward workgroups resident at once on the device (0: unknown)
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Read-only views through the constant address space: the prep kernels wrote
// these arrays before this kernel started and nothing writes them during it,
// so workgroup-uniform reads may use scalar loads (they then stay out of the
// vector-memory wait counter that tracks the K/V tile loads).
typedef __attribute__((address_space(4))) const int ConstInt;
__device__ __forceinline__ int ld_const(const int* p, long long i) { return ((ConstInt*)p)[i]; }
__device__ __forceinline__ TileSum ld_const(const TileSum* p, int i) {
  const int* b = reinterpret_cast<const int*>(p + i);
  return TileSum{ld_const(b, 0), ld_const(b, 1), ld_const(b, 2), ld_const(b, 3), ld_const(b, 4), ld_const(b, 5), 0, 0};
}

// Whether a query tile and a key tile may hold an allowed pair (a superset
// test: the walk visits these, the per-element mask is exact). When the two
// tiles can share only the key tile's first (or last) segment, only that
// segment's keys count: a key tile that straddles the end of a segment is
// not visited by the segment's early queries.
__device__ __forceinline__ bool tiles_meet(const TileSum& q, const TileSum& k, int window) {
  if (k.seg_max < q.seg_min || k.seg_min > q.seg_max) return false;
  // Plain values first: a conditional between two fields of one struct
  // would select an address and keep the struct in memory.
  const int p_first = k.pos_first, p_last = k.pos_last, p_min = k.pos_min;
  const int kp = q.seg_max == k.seg_min ? p_first : q.seg_min == k.seg_max ? p_last : p_min;
  if (kp > q.pos_max) return false;
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

// Both tiles lie in one and the same segment, key tile kt holds 64 real
// keys and no position is negative: a pair is then allowed iff its
// positions (and the window) allow it, so the per-element mask may skip the
// segment compare, and two positions differ by less than 2^31, so one
// unsigned compare of their difference tests order and window together.
__device__ __forceinline__ bool tiles_oneseg(const TileSum& q, const TileSum& k, int kt, int p) {
  return (kt + 1) * kBK <= p && q.seg_min == q.seg_max && k.seg_min == k.seg_max && k.seg_min == q.seg_min &&
         q.pos_min >= 0 && k.pos_min >= 0;
}

// Maximum of floats without the canonicalizing moves fmaxf needs (v_maximum3
// on gfx950); a NaN input propagates.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Lanes l and l ^ 32 own the two key halves of one query column; these
// combine their values (one cross-half lane swap, no LDS round trip).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

typedef __attribute__((address_space(3))) char LdsByte;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T lds_ld(const LdsByte* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_st(LdsByte* p, const T& v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}

// Raw buffer descriptor (base, num_records bytes, untyped 32-bit access) as
// four scalar registers, for the asm loads below.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int num_records) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)p;
  r[1] = (int)((p >> 32) & 0xffff);
  r[2] = num_records;
  r[3] = 0x00020000;
  return r;
}
// Direct buffer-to-LDS load: BYTES (4 or 16) per lane from base + voffset,
// written at LDS byte address lds + BYTES * lane (zeros for lanes out of
// range). Issued as asm so that the compiler's wait-counter bookkeeping
// leaves these loads alone: the kernel waits for them explicitly, a tile or
// two after issue, and an automatic wait before each LDS read would drain
// them at once.
template <int BYTES>
__device__ __forceinline__ void lds_dma(i32x4 rsrc, uint32_t lds, int voffset) {
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voffset), "s"(rsrc) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voffset), "s"(rsrc) : "memory", "m0");
}


// Direct buffer-to-LDS load through the current M0: BYTES = 16 per lane from
// base + voffset + OFF, written at LDS byte address M0 + OFF + 16 * lane (the
// instruction offset moves both addresses). set_lds_m0 writes M0 (and the
// wait state an LDS DMA needs after an M0 write); nothing else in the
// kernels that use these touches M0.
__device__ __forceinline__ void set_lds_m0(uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" :: "s"(lds) : "memory", "m0");
}
template <int OFF>
__device__ __forceinline__ void lds_dma16_m0(i32x4 rsrc, int voffset) {
  static_assert(OFF >= 0 && OFF < 4096, "instruction offset");
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%2 lds" :: "v"(voffset), "s"(rsrc), "i"(OFF) : "memory");
}

// The prepared walk of a packed prefill (summaries, per query tile the key
// tiles to visit and which of them need no mask, the costliest-first order),
// built by three small kernels into the workspace; and its size. Query tiles
// hold 32 tokens per wavefront of a head group: `waves` wavefronts per
// workgroup (0: the forward kernel's own count).
hipError_t prefill_prepare(const PrefillArgs& a, Plan& pl, hipStream_t stream, int waves = 0);
// Summaries of pl's query tiles (pl.tq tokens) and, if pl.n_kt > 0, key tiles.
hipError_t prefill_summarize(const PrefillArgs& a, const Plan& pl, hipStream_t stream);
size_t prefill_plan_bytes(int p);
// pl.order[0 .. pl.n_qt) = the indices 0 .. pl.n_qt - 1 by pl.cost (each in
// [0, pl.max_cost]), costliest first (one workgroup; identity order when
// max_cost is too large for its bins).
hipError_t prefill_order(const Plan& pl, hipStream_t stream);

}  // namespace gqa
