// Rotary tables and the fused rope + KV-write pass (gfx950).
//
// `tables<S, D, T>(theta)` of rope.linnet (Linnet "examples/01-llama" page)
// computes inv_freq, the angles and cos/sin in f32 and casts them to T; the
// rotation `rope` pairs dimension i with i + D/2 (the page repeats each
// frequency in both halves of the head dimension). `decode` rotates q and k
// at `pos` and writes k and v into the caches with write_at, a masked
// select; the serving entries of the Nest llama-3.1-8b-instruct card do the
// same at rows / slots / table pages.
//
// The pass is HBM-bound: one thread owns one 16-byte chunk of the low half of
// a head and the matching chunk of the high half, so every load and store is
// a full 16-byte vector and the rotation needs no cross-lane traffic. The
// rotation is the exact value rounded once to T (rope_common.h).
#include "common.h"
#include "internal.h"
#include "rope_common.h"

namespace gqa {

// ---------------------------------------------------------------------------
// Table: [2, max_pos, D/2] of T, entry (c, s, i) = cos / sin of f32(s) *
// inv_freq[i]. Each f32 step of the page's pipeline is evaluated in fp64 and
// rounded to f32 (a product or quotient of two f32 values rounded through
// fp64 is the correctly rounded f32 result).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void rope_table_kernel(int head_dim, int max_pos, float theta, T* table) {
  const int half = head_dim / 2;
  const long long total = (long long)max_pos * half;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int s = (int)(idx / half);
  const int i = (int)(idx % half);
  const float a = (float)i * 2.0f;                              // exact
  const float b = (float)((double)a / (double)(float)head_dim);  // f32 quotient
  const float lt = (float)log((double)theta);                   // f32 log
  const float e = (float)(-(double)b * (double)lt);             // f32 product
  const float inv = (float)exp((double)e);                      // f32 exp
  const float ang = (float)((double)(float)s * (double)inv);    // f32 product
  const float c = (float)cos((double)ang);
  const float sn = (float)sin((double)ang);
  Elem<T>::store1(table + idx, c);
  Elem<T>::store1(table + total + idx, sn);
}

// ---------------------------------------------------------------------------
// Fused rotate + write.
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void rope_write_kernel(RopeWriteArgs a) {
  constexpr int EPC = Elem<T>::kPer16B;  // elements per 16-byte chunk
  const int D = a.head_dim;
  const int half = D / 2;
  const int cph = half / EPC;  // chunks per half head
  const int slots_per_token = (a.heads + a.kv_heads) * cph;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.n * slots_per_token) return;
  const int t = (int)(idx / slots_per_token);
  const int rem = (int)(idx % slots_per_token);
  const int hs = rem / cph;  // head slot: q heads first, then kv heads
  const int c = rem % cph;
  const int d0 = c * EPC;
  const bool is_q = hs < a.heads;
  const bool rotate = a.rope_table != nullptr;

  u32x4 cw, sw;
  if (rotate) {
    int p = a.positions[t];
    p = p < 0 ? 0 : (p >= a.rope_max_pos ? a.rope_max_pos - 1 : p);
    const T* tab = static_cast<const T*>(a.rope_table);
    cw = load16(tab + (long long)p * half + d0);
    sw = load16(tab + ((long long)a.rope_max_pos + p) * half + d0);
  }

  if (is_q) {
    if (!rotate || a.q == nullptr) return;
    T* base = static_cast<T*>(a.q) + ((long long)t * a.heads + hs) * D;
    u32x4 lo = load16(base + d0), hi = load16(base + half + d0);
    rotate_chunk<T>(lo, hi, cw, sw);
    store16(base + d0, lo);
    store16(base + half + d0, hi);
    return;
  }

  const int kh = hs - a.heads;
  const long long src = ((long long)t * a.kv_heads + kh) * D;
  long long dst = -1;
  if (a.cache_kind != 0) dst = cache_offset(a, t, kh);
  if (a.k != nullptr) {
    T* kb = static_cast<T*>(a.k) + src;
    u32x4 lo = load16(kb + d0), hi = load16(kb + half + d0);
    if (rotate) {
      rotate_chunk<T>(lo, hi, cw, sw);
      store16(kb + d0, lo);
      store16(kb + half + d0, hi);
    }
    if (dst >= 0) {
      T* ck = static_cast<T*>(a.cache_k) + dst;
      store16(ck + d0, lo);
      store16(ck + half + d0, hi);
    }
  }
  if (dst >= 0 && a.v != nullptr && a.cache_v != nullptr) {
    const T* vb = static_cast<const T*>(a.v) + src;
    T* cv = static_cast<T*>(a.cache_v) + dst;
    store16(cv + d0, load16(vb + d0));
    store16(cv + half + d0, load16(vb + half + d0));
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_rope_table(int head_dim, int max_pos, float theta, int dtype, void* table,
                             hipStream_t stream) {
  const long long total = (long long)max_pos * (head_dim / 2);
  const int block = 256;
  const long long grid = (total + block - 1) / block;
  if (dtype == kDtypeBf16)
    rope_table_kernel<uint16_t><<<dim3((unsigned)grid), dim3(block), 0, stream>>>(
        head_dim, max_pos, theta, static_cast<uint16_t*>(table));
  else
    rope_table_kernel<float><<<dim3((unsigned)grid), dim3(block), 0, stream>>>(
        head_dim, max_pos, theta, static_cast<float*>(table));
  return hipGetLastError();
}

hipError_t launch_rope_write(const RopeWriteArgs& a, hipStream_t stream) {
  const int epc = a.dtype == kDtypeBf16 ? 8 : 4;
  const long long items = (long long)a.n * (a.heads + a.kv_heads) * (a.head_dim / 2 / epc);
  const int block = 256;
  const long long grid = (items + block - 1) / block;
  if (a.dtype == kDtypeBf16)
    rope_write_kernel<uint16_t><<<dim3((unsigned)grid), dim3(block), 0, stream>>>(a);
  else
    rope_write_kernel<float><<<dim3((unsigned)grid), dim3(block), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace gqa
