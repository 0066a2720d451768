// Split-K decode attention over a contiguous cache or a paged pool (gfx950).
//
// `decode` of the Linnet "examples/01-llama" page (src/attention.linnet)
// attends every cached slot s with s <= pos; decode_rows takes one position
// per row and decode_paged addresses the cache through a [Rows, Pages] page
// table with PageSize 64 (Nest llama-3.1-8b-instruct card, block
// GroupedQueryAttention). The softmax over a row's keys is split into
// independent ranges of `split_len` tokens; each workgroup reduces one range
// for the G query heads that share one KV head (so every K/V byte is read
// once per KV head, not once per query head) and writes a partial
// (max, sum, weighted V); a merge kernel rescales and combines the partials,
// adding the sink term of SinkAttention (Nest gpt-oss-20b card) to the
// denominator. Splitting by ranges reaches exactly the softmax over the union
// (up to rounding order).
//
// This generic kernel runs on the vector ALUs: a token's row of D elements is
// spread over D*sizeof(T)/16 lanes that each load one 16-byte chunk (so a
// wavefront reads whole rows, coalesced), dot products are finished with
// butterfly shuffles, and the split's scores live in LDS between the QK and
// PV phases (one exp per score). It serves f32, contiguous caches and every
// head-group size.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace gqa {

namespace {
constexpr int kSplitLen = 256;
constexpr int kBlock = 256;
constexpr float kNegInf = -__builtin_huge_valf();
}  // namespace

template <typename T, int D, bool PAGED>
__device__ __forceinline__ const T* row_ptr(const DecodeArgs& a, const void* base, int r, int kh,
                                            int t) {
  if (PAGED) {
    const int page = a.table[(long long)r * a.pages + t / kPageSize];
    if (page < 0 || page >= a.num_pages) return nullptr;
    return static_cast<const T*>(base) +
           (((long long)page * a.kv_heads + kh) * kPageSize + t % kPageSize) * D;
  }
  return static_cast<const T*>(base) + (((long long)r * a.kv_heads + kh) * a.cap + t) * D;
}

template <typename T, int D, int GC, bool PAGED>
__global__ __launch_bounds__(kBlock) void decode_split_kernel(DecodeArgs a) {
  constexpr int EPL = Elem<T>::kPer16B;  // elements per lane per token
  constexpr int LPT = D / EPL;           // lanes per token
  constexpr int TPP = kBlock / LPT;      // tokens per pass of the block
  __shared__ float sc[GC][kSplitLen];
  __shared__ float red[4][GC][D];
  __shared__ float stat[GC][2];

  const int split = blockIdx.x;
  const int r = blockIdx.z;
  const int G = a.heads / a.kv_heads;
  const int nchunks = G / GC;
  const int kh = blockIdx.y / nchunks;
  const int h0 = kh * G + (blockIdx.y % nchunks) * GC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int lo, hi;
  decode_key_range(a.positions[r], a.cap, a.window, lo, hi);
  const int t0 = max(lo, split * a.split_len);
  const int t1 = min(hi + 1, (split + 1) * a.split_len);
  if (t0 >= t1) return;  // the merge never reads a split outside [lo, hi]
  const int n = t1 - t0;

  const int sub = tid % LPT;
  const int tk = tid / LPT;

  float qr[GC][EPL];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    const T* qp = static_cast<const T*>(a.q) + ((long long)r * a.heads + h0 + h) * D + sub * EPL;
    Elem<T>::to_f32(load16(qp), qr[h]);
  }

  // Phase 1: scaled scores (log2 domain) of every key of the split. The
  // loads of UNR passes are issued before any of them is used, so that many
  // memory round trips overlap.
  constexpr int UNR = 8;
  for (int base = 0; base < n; base += TPP * UNR) {
    u32x4 raw[UNR];
    bool valid[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + u * TPP + tk;
      const T* kp = i < n ? row_ptr<T, D, PAGED>(a, a.k, r, kh, t0 + i) : nullptr;
      valid[u] = kp != nullptr;
      raw[u] = valid[u] ? load16(kp + sub * EPL) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + u * TPP + tk;
      float dot[GC];
#pragma unroll
      for (int h = 0; h < GC; ++h) dot[h] = 0.f;
      if (valid[u]) {
        float x[EPL];
        Elem<T>::to_f32(raw[u], x);
#pragma unroll
        for (int h = 0; h < GC; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) dot[h] += qr[h][e] * x[e];
      }
#pragma unroll
      for (int off = LPT / 2; off >= 1; off >>= 1)
#pragma unroll
        for (int h = 0; h < GC; ++h) dot[h] += __shfl_xor(dot[h], off, 64);
      if (sub == 0 && i < n) {
#pragma unroll
        for (int h = 0; h < GC; ++h) sc[h][i] = valid[u] ? dot[h] * a.scale_log2 : kNegInf;
      }
    }
  }
  __syncthreads();

  // Phase 2: per-head max, exponentials and their sum.
  for (int h = wave; h < GC; h += 4) {
    float m = kNegInf;
    for (int i = lane; i < n; i += 64) m = fmaxf(m, sc[h][i]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float p = (m == kNegInf) ? 0.f : exp2f(sc[h][i] - m);
      sc[h][i] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      stat[h][0] = m;
      stat[h][1] = l;
    }
  }
  __syncthreads();

  // Phase 3: probability-weighted values.
  float acc[GC][EPL];
#pragma unroll
  for (int h = 0; h < GC; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  for (int base = 0; base < n; base += TPP * UNR) {
    u32x4 raw[UNR];
    bool valid[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + u * TPP + tk;
      // Keys of invalid pages were never scored.
      const T* vp = i < n ? row_ptr<T, D, PAGED>(a, a.v, r, kh, t0 + i) : nullptr;
      valid[u] = vp != nullptr;
      raw[u] = valid[u] ? load16(vp + sub * EPL) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (valid[u]) {
        const int i = base + u * TPP + tk;
        float x[EPL];
        Elem<T>::to_f32(raw[u], x);
#pragma unroll
        for (int h = 0; h < GC; ++h) {
          const float p = sc[h][i];
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] += p * x[e];
        }
      }
    }
  }
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][h][sub * EPL + e] = acc[h][e];
  }
  __syncthreads();

  for (int x = tid; x < GC * D; x += kBlock) {
    const int h = x / D;
    const int d = x % D;
    float* part = a.ws + (((long long)r * a.heads + h0 + h) * a.nsplit + split) * (D + 2);
    part[2 + d] = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
    if (d == 0) {
      part[0] = stat[h][0];
      part[1] = stat[h][1];
    }
  }
}

// Combine the split partials of one (row, KV head): the G query heads' split
// weights exp2(m_s - M) go to LDS, then every (head, dimension) output is one
// coalesced pass over the splits. The sink logit joins the denominator here.
constexpr int kMergeMaxW = 4096;

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float w[kMergeMaxW];
  __shared__ float inv_l[64];
  const int kh = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int G = a.heads / a.kv_heads;
  const int h0 = kh * G;
  int lo, hi;
  decode_key_range(a.positions[r], a.cap, a.window, lo, hi);
  int s_first = 0, ns = 0;
  if (hi >= lo) {
    s_first = lo / a.split_len;
    ns = hi / a.split_len - s_first + 1;
  }
  const bool has_sink = a.sinks != nullptr;
  auto part = [&](int h, int s) {
    return a.ws + (((long long)r * a.heads + h0 + h) * a.nsplit + s_first + s) * (D + 2);
  };
  auto sink2 = [&](int h) {
    return has_sink ? Elem<T>::load1(static_cast<const T*>(a.sinks) + h0 + h) * kLog2e : kNegInf;
  };
  T* out = static_cast<T*>(a.out) + ((long long)r * a.heads + h0) * D;
  if (G * ns > kMergeMaxW || G > 64) {
    // Serial fallback for very long caches: one thread per output.
    for (int x = tid; x < G * D; x += blockDim.x) {
      const int h = x / D, d = x % D;
      float M = sink2(h);
      for (int s = 0; s < ns; ++s) M = fmaxf(M, part(h, s)[0]);
      float num = 0.f, den = (has_sink && M != kNegInf) ? fast_exp2(sink2(h) - M) : 0.f;
      for (int s = 0; s < ns; ++s) {
        const float ms = part(h, s)[0];
        if (ms == kNegInf) continue;
        const float ws = fast_exp2(ms - M);
        num += ws * part(h, s)[2 + d];
        den += ws * part(h, s)[1];
      }
      Elem<T>::store1(out + (long long)h * D + d, den > 0.f ? num / den : 0.f);
    }
    return;
  }
  for (int x = tid; x < G * ns; x += blockDim.x) w[x] = part(x / ns, x % ns)[0];
  __syncthreads();
  if (tid < G) {
    float M = sink2(tid);
    for (int s = 0; s < ns; ++s) M = fmaxf(M, w[tid * ns + s]);
    float L = (has_sink && M != kNegInf) ? fast_exp2(sink2(tid) - M) : 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = w[tid * ns + s];
      const float ws = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
      w[tid * ns + s] = ws;
      L += ws * part(tid, s)[1];
    }
    inv_l[tid] = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += blockDim.x) {
    const int h = x / D, d = x % D;
    float acc = 0.f;
    const float* ws = w + h * ns;
    for (int s = 0; s < ns; ++s) {
      const float wt = ws[s];
      if (wt != 0.f) acc += wt * part(h, s)[2 + d];
    }
    Elem<T>::store1(out + (long long)h * D + d, acc * inv_l[h]);
  }
}

// Vector-ALU split plan; its 256-key splits are the shortest of both paths,
// so its workspace bound covers the matrix-core path too.
void decode_plan(int rows, int heads, int kv_heads, int head_dim, int dtype, int paged, int cap,
                 int* split_len, int* nsplit, size_t* ws_bytes) {
  (void)kv_heads;
  (void)dtype;
  (void)paged;
  const int sl = kSplitLen;
  const int ns = cap > 0 ? (cap + sl - 1) / sl : 1;
  if (split_len) *split_len = sl;
  if (nsplit) *nsplit = ns;
  if (ws_bytes) *ws_bytes = (size_t)rows * heads * ns * (head_dim + 2) * sizeof(float);
}

template <typename T, int D, bool PAGED>
static hipError_t launch_split_t(const DecodeArgs& a, int gc, hipStream_t stream) {
  const int G = a.heads / a.kv_heads;
  dim3 grid(a.nsplit, a.kv_heads * (G / gc), a.rows);
  switch (gc) {
    case 8:
      decode_split_kernel<T, D, 8, PAGED><<<grid, kBlock, 0, stream>>>(a);
      break;
    case 4:
      decode_split_kernel<T, D, 4, PAGED><<<grid, kBlock, 0, stream>>>(a);
      break;
    case 2:
      decode_split_kernel<T, D, 2, PAGED><<<grid, kBlock, 0, stream>>>(a);
      break;
    default:
      decode_split_kernel<T, D, 1, PAGED><<<grid, kBlock, 0, stream>>>(a);
      break;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.heads / a.kv_heads;
  const int gc = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  hipError_t e = a.paged ? launch_split_t<T, D, true>(a, gc, stream)
                         : launch_split_t<T, D, false>(a, gc, stream);
  if (e != hipSuccess) return e;
  decode_merge_kernel<T, D><<<dim3(a.kv_heads, a.rows), 256, 0, stream>>>(a);
  return hipGetLastError();
}

// Bytes of split partials the launch below will write for `a` (0 when the
// matrix-core path covers each row with one split and writes the output
// itself).
size_t decode_partials_bytes(const DecodeArgs& a) {
  int nsplit;
  if (decode_mfma_supported(a)) {
    const int sl = decode_mfma_split_len(a.rows, a.kv_heads, a.cap);
    nsplit = (a.cap + sl - 1) / sl;
    if (nsplit == 1) return 0;
  } else {
    decode_plan(a.rows, a.heads, a.kv_heads, a.head_dim, a.dtype, a.paged, a.cap, nullptr, &nsplit,
                nullptr);
  }
  return (size_t)a.rows * a.heads * nsplit * (a.head_dim + 2) * sizeof(float);
}

// Scratch of the entry point that allocates nothing: the split partials live
// in this module array (each GPU the library runs on holds its own copy for
// the life of the process). In host code the name `scratch` is only a
// stand-in: its device address, per device, comes from hipGetSymbolAddress
// on the first call made with that device current, and only that address is
// handed to kernels. Calls that overlap on one GPU share it and race.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = static_cast<float*>(p);
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_decode(DecodeArgs a, hipStream_t stream) {
  if (decode_mfma_supported(a)) {
    // Matrix-core split kernel, then (with more than one split) the merge.
    a.split_len = decode_mfma_split_len(a.rows, a.kv_heads, a.cap);
    a.nsplit = (a.cap + a.split_len - 1) / a.split_len;
    hipError_t e = launch_decode_mfma(a, stream);
    if (e != hipSuccess) return e;
    if (a.nsplit == 1) return hipSuccess;  // the split kernel wrote the output
    if (a.head_dim == 64)
      decode_merge_kernel<uint16_t, 64><<<dim3(a.kv_heads, a.rows), 256, 0, stream>>>(a);
    else
      decode_merge_kernel<uint16_t, 128><<<dim3(a.kv_heads, a.rows), 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  decode_plan(a.rows, a.heads, a.kv_heads, a.head_dim, a.dtype, a.paged, a.cap, &a.split_len,
              &a.nsplit, nullptr);
  if (a.dtype == kDtypeBf16) {
    return a.head_dim == 64 ? launch_decode_t<uint16_t, 64>(a, stream)
                            : launch_decode_t<uint16_t, 128>(a, stream);
  }
  return a.head_dim == 64 ? launch_decode_t<float, 64>(a, stream)
                          : launch_decode_t<float, 128>(a, stream);
}

}  // namespace gqa
