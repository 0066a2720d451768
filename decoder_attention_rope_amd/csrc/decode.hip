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
// This generic kernel runs on the vector ALUs and serves f32, and bf16 with
// more query heads per KV head than the matrix-core kernel takes. It makes
// one pass over the keys with an online softmax in registers:
// * A workgroup of NW wavefronts owns one (row, KV head, head chunk, split of
//   keys); its wavefronts take chunks of CK keys round-robin. A key row of D
//   elements is spread over LPT = D * sizeof(T) / 16 lanes that each load one
//   16-byte chunk, so every load instruction of a wavefront reads 64 / LPT
//   whole, consecutive rows (1 KB).
// * A chunk's K and V loads (UNR per lane each, nontemporal) are all issued
//   before any is used, unconditionally: addresses are clamped into the
//   split's key range and keys outside it are masked afterwards.
// * Dot products are finished with DPP butterflies inside each 16-lane row,
//   so all LPT lanes of a key hold the same score bit for bit; each lane then
//   keeps the running max, sum and weighted V of its key slot for its EPL
//   dimensions. Slots and wavefronts are combined once, at the end.
// * With a single split per (row, head chunk) the workgroup also normalizes,
//   adds the sink and writes the output; otherwise it writes a partial for
//   the merge kernel below.
// * Rows are split only when there are too few (row, head chunk) units to
//   fill the chip. With enough units and at most 64 rows, every unit is one
//   workgroup of up to 16 wavefronts and the workgroups map to rows in order
//   of decreasing key count (ranked on the device from the positions):
//   workgroups start in blockIdx order, so the longest rows start first and
//   the short ones fill the gaps, with no merge pass.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace gqa {

namespace {
constexpr int kSplitLen = 256;
constexpr float kNegInf = -__builtin_huge_valf();
}  // namespace

// Sum over the LPT lanes of each key slot (LPT = 8, 16 or 32), left in every
// one of them. Inside a 16-lane row the butterfly runs on DPP (quad swaps,
// then the half-row and row mirrors); the step across rows is a shuffle.
// Every lane adds the same two values in either order, so all lanes of a
// slot end with identical bits.
template <int CTRL>
__device__ __forceinline__ float dpp_get(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int LPT>
__device__ __forceinline__ float slot_sum(float v) {
  v += dpp_get<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_get<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_get<0x141>(v);  // row_half_mirror
  if (LPT >= 16) v += dpp_get<0x140>(v);  // row_mirror
  if (LPT >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

#ifndef GQA_DECODE_VEC_TARGET_WGS
#define GQA_DECODE_VEC_TARGET_WGS 1024
#endif
#ifndef GQA_DECODE_VEC_LOADS
#define GQA_DECODE_VEC_LOADS 8
#endif
#ifndef GQA_DECODE_VEC_SORT_UNITS
#define GQA_DECODE_VEC_SORT_UNITS 256
#endif
constexpr int kVecLoads = GQA_DECODE_VEC_LOADS;  // K (and V) loads per lane per chunk, at most
constexpr int kVecWaves = 8;         // wavefronts per workgroup with split rows
constexpr int kVecWavesSorted = 16;  // ... with one workgroup per row and head chunk

template <typename T, int D, int GC, bool PAGED, int NW, bool SORTED>
__global__ __launch_bounds__(64 * NW) void decode_vec_kernel(DecodeArgs a) {
  constexpr int EPL = Elem<T>::kPer16B;       // elements per lane per key row
  constexpr int LPT = D / EPL;                // lanes per key row
  constexpr int TPW = 64 / LPT;               // key rows per load instruction
  constexpr int UNR = TPW * kVecLoads <= kPageSize ? kVecLoads : kPageSize / TPW;
  constexpr int CK = TPW * UNR;               // keys per chunk (inside one page)
  constexpr int RS = D + 2;
  __shared__ float red[NW][GC][RS];

  const int split = blockIdx.x;
  // Sorted dispatch (one split): workgroups are launched in blockIdx order,
  // so the longest rows start first and shorter ones fill in behind them.
  const int r = SORTED ? __builtin_amdgcn_readfirstlane(row_of_rank(a.positions, a.rows, a.cap, a.window, blockIdx.z)) : blockIdx.z;
  const int G = a.heads / a.kv_heads;
  const int nchunks = G / GC;
  const int kh = blockIdx.y / nchunks;
  const int h0 = kh * G + (blockIdx.y % nchunks) * GC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % LPT;  // 16-byte column of the key row
  const int tk = lane / LPT;   // key slot within a load instruction

  int lo, hi;
  decode_key_range(a.positions[r], a.cap, a.window, lo, hi);
  const int t0 = max(lo, split * a.split_len);
  const int t1 = min(hi + 1, (split + 1) * a.split_len);
  if (t0 >= t1) {
    // No keys in this split. The merge never reads a split outside [lo, hi];
    // with a single split this workgroup owns the output, which is 0.
    if (a.nsplit == 1) {
      T* out = static_cast<T*>(a.out) + ((long long)r * a.heads + h0) * D;
      for (int x = tid; x < GC * D; x += 64 * NW) Elem<T>::store1(out + x, 0.f);
    }
    return;
  }

  float qr[GC][EPL];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    const T* qp = static_cast<const T*>(a.q) + ((long long)r * a.heads + h0 + h) * D + sub * EPL;
    Elem<T>::to_f32(load16(qp), qr[h]);
  }
  float m_run[GC], l_run[GC], acc[GC][EPL];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const T* kbase = static_cast<const T*>(a.k);
  const T* vbase = static_cast<const T*>(a.v);
  const int c_begin = t0 / CK;
  const int c_end = (t1 + CK - 1) / CK;
  for (int c = c_begin + wave; c < c_end; c += NW) {
    const int tb = c * CK;
    long long row0;  // element offset of key tb
    if (PAGED) {
      const int page = a.table[(long long)r * a.pages + tb / kPageSize];
      if (page < 0 || page >= a.num_pages) continue;  // no keys from this page
      row0 = (((long long)page * a.kv_heads + kh) * kPageSize + tb % kPageSize) * D;
    } else {
      row0 = (((long long)r * a.kv_heads + kh) * a.cap + tb) * D;
    }
    // Key u * TPW + tk of the chunk; keys outside [t0, t1) read a clamped
    // in-range row and are masked below.
    u32x4 kx[UNR], vx[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = min(max(tb + u * TPW + tk, t0), t1 - 1);
      kx[u] = load16_stream(kbase + row0 + (long long)(t - tb) * D + sub * EPL);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = min(max(tb + u * TPW + tk, t0), t1 - 1);
      vx[u] = load16_stream(vbase + row0 + (long long)(t - tb) * D + sub * EPL);
    }
    // Keep all 2 * UNR loads in flight together: without this fence the
    // scheduler sinks each load to just before its first use, which leaves
    // only a few in flight per wavefront.
    __builtin_amdgcn_sched_barrier(0);
    const bool full = tb >= t0 && tb + CK <= t1;
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      float s[UNR];
      float cmax = kNegInf;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float x[EPL];
        Elem<T>::to_f32(kx[u], x);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = __builtin_fmaf(qr[h][e], x[e], d);
        d = slot_sum<LPT>(d) * a.scale_log2;
        if (!full) {
          const int t = tb + u * TPW + tk;
          d = ((t >= t0) & (t < t1)) ? d : kNegInf;
        }
        s[u] = d;
        cmax = fmaxf(cmax, d);
      }
      const float m_new = fmaxf(m_run[h], cmax);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[h] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float p = fast_exp2(s[u] - m_use);
        psum += p;
        float x[EPL];
        Elem<T>::to_f32(vx[u], x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = __builtin_fmaf(p, x[e], acc[h][e]);
      }
      l_run[h] = l_run[h] * alpha + psum;
      m_run[h] = m_new;
    }
  }

  // Combine the TPW key slots of the wavefront (lanes sub + LPT * tk).
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    float M = m_run[h];
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float f = (m_run[h] == kNegInf) ? 0.f : fast_exp2(m_run[h] - M);
    float l = l_run[h] * f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      l += __shfl_xor(l, off, 64);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);
    }
    if (tk == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][h][2 + sub * EPL + e] = acc[h][e];
      if (sub == 0) {
        red[wave][h][0] = M;
        red[wave][h][1] = l;
      }
    }
  }
  __syncthreads();

  // Combine the wavefronts: one thread per (head, dimension).
  for (int x = tid; x < GC * D; x += 64 * NW) {
    const int h = x / D;
    const int d = x % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red[w][h][0]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red[w][h][0];
      const float sc = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      num += sc * red[w][h][2 + d];
      den += sc * red[w][h][1];
    }
    if (a.nsplit == 1) {
      // The only split: normalize here; the sink joins the denominator.
      if (a.sinks != nullptr) {
        const float s2 = Elem<T>::load1(static_cast<const T*>(a.sinks) + h0 + h) * kLog2e;
        const float Ms = fmaxf(M, s2);
        const float f = (M == kNegInf) ? 0.f : fast_exp2(M - Ms);
        num *= f;
        den = den * f + fast_exp2(s2 - Ms);
      }
      Elem<T>::store1(static_cast<T*>(a.out) + ((long long)r * a.heads + h0 + h) * D + d,
                      den > 0.f ? num / den : 0.f);
    } else {
      float* part = a.ws + (((long long)r * a.heads + h0 + h) * a.nsplit + split) * RS;
      part[2 + d] = num;
      if (d == 0) {
        part[0] = M;
        part[1] = den;
      }
    }
  }
}

// Combine the split partials of one (row, query head) in one wavefront: lane
// l owns dimensions l (and l + 64 for D = 128). Splits are visited in groups
// of kMergeGroup whose partials are all loaded at once -- before the row's
// key range is known, so those loads do not wait for the position -- and
// splits outside the range (never written by this call) are then dropped by
// selection. Each group is folded into a running (max, denominator,
// numerator) with rescaling. The sink logit starts the running state: max =
// sink, denominator 2^0 = 1.
constexpr int kMergeGroup = 8;

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int DPL = D / 64;  // dimensions per lane
  constexpr int NG = kMergeGroup;
  const int lane = threadIdx.x & 63;
  const int rh = blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, query head)
  if (rh >= a.rows * a.heads) return;
  const int r = rh / a.heads;
  const int h = rh % a.heads;
  const float* part = a.ws + (long long)rh * a.nsplit * (D + 2);
  float ms[NG], ls[NG], xs[NG][DPL];
  auto load_group = [&](int s0) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const float* p = part + (long long)min(s0 + i, a.nsplit - 1) * (D + 2);
      ms[i] = p[0];
      ls[i] = p[1];
#pragma unroll
      for (int j = 0; j < DPL; ++j) xs[i][j] = p[2 + lane + 64 * j];
    }
  };
  // The first group, the position and the sink are all in flight together.
  load_group(0);
  const int pos = a.positions[r];
  const float sink = a.sinks != nullptr ? Elem<T>::load1(static_cast<const T*>(a.sinks) + h) : 0.f;
  __builtin_amdgcn_sched_barrier(0);
  int lo, hi;
  decode_key_range(pos, a.cap, a.window, lo, hi);
  // Splits [s_lo, s_hi] hold the row's keys (none when hi < lo).
  const int s_lo = hi >= lo ? lo / a.split_len : 1;
  const int s_hi = hi >= lo ? hi / a.split_len : 0;
  float M = kNegInf, den = 0.f, num[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) num[j] = 0.f;
  if (a.sinks != nullptr) {
    M = sink * kLog2e;
    den = 1.f;
  }
  for (int s0 = 0;;) {
    bool ok[NG];
    float gmax = M;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      ok[i] = s0 + i >= s_lo && s0 + i <= s_hi && ms[i] != kNegInf;
      gmax = ok[i] ? fmaxf(gmax, ms[i]) : gmax;
    }
    if (gmax != kNegInf) {
      const float f = (M == kNegInf) ? 0.f : fast_exp2(M - gmax);
      den *= f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) num[j] *= f;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const float w = fast_exp2(ms[i] - gmax);
        den = ok[i] ? __builtin_fmaf(w, ls[i], den) : den;
#pragma unroll
        for (int j = 0; j < DPL; ++j) num[j] = ok[i] ? __builtin_fmaf(w, xs[i][j], num[j]) : num[j];
      }
      M = gmax;
    }
    s0 += NG;
    if (s0 >= a.nsplit) break;
    load_group(s0);
  }
  T* out = static_cast<T*>(a.out) + (long long)rh * D;
#pragma unroll
  for (int j = 0; j < DPL; ++j) Elem<T>::store1(out + lane + 64 * j, den > 0.f ? num[j] / den : 0.f);
}

static hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream) {
  const int waves = a.rows * a.heads;
  dim3 grid((waves + 3) / 4);
  if (a.dtype == kDtypeBf16) {
    if (a.head_dim == 64) decode_merge_kernel<uint16_t, 64><<<grid, 256, 0, stream>>>(a);
    else decode_merge_kernel<uint16_t, 128><<<grid, 256, 0, stream>>>(a);
  } else {
    if (a.head_dim == 64) decode_merge_kernel<float, 64><<<grid, 256, 0, stream>>>(a);
    else decode_merge_kernel<float, 128><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

// Workspace bound of both decode paths: neither splits a row into pieces
// shorter than kSplitLen keys, so at most ceil(cap / kSplitLen) partials of
// D + 2 floats per (row, query head) are ever written.
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

// Query heads per workgroup of the vector kernel: as many as divide G, up to
// 8 for f32 and 4 for bf16 (whose K and V rows take twice the registers per
// 16-byte load once widened).
static int decode_vec_heads(const DecodeArgs& a) {
  const int G = a.heads / a.kv_heads;
  const int most = a.dtype == kDtypeBf16 ? 4 : 8;
  int gc = 1;
  while (gc * 2 <= most && G % (gc * 2) == 0) gc *= 2;
  return gc;
}

// Split length of the vector kernel: the whole cache (sorted dispatch) when
// at most 64 rows give at least GQA_DECODE_VEC_SORT_UNITS (row, head chunk)
// units; otherwise the longest length (a multiple of the page size) that
// still gives about GQA_DECODE_VEC_TARGET_WGS workgroups, never under
// kSplitLen keys.
static int decode_vec_split_len(const DecodeArgs& a) {
  const long long units = (long long)a.rows * a.heads / decode_vec_heads(a);
  if (a.rows <= kSortMaxRows && units >= GQA_DECODE_VEC_SORT_UNITS)
    return (a.cap + kPageSize - 1) / kPageSize * kPageSize;  // one split, sorted dispatch
  long long nsplit = (GQA_DECODE_VEC_TARGET_WGS + units - 1) / units;
  const long long max_split = (a.cap + kSplitLen - 1) / kSplitLen;
  if (nsplit > max_split) nsplit = max_split;
  if (nsplit < 1) nsplit = 1;
  long long len = (a.cap + nsplit - 1) / nsplit;
  len = (len + kPageSize - 1) / kPageSize * kPageSize;
  return (int)(len > 0 ? len : kPageSize);
}

// Wavefronts per workgroup: 8 with split rows; with sorted dispatch 16 where
// the head chunk's state fits 128 registers (f32 up to 2 heads, bf16 1).
template <typename T, int GC, bool SORTED>
constexpr int vec_waves() {
  return SORTED && GC * Elem<T>::kPer16B <= 8 ? kVecWavesSorted : kVecWaves;
}

template <typename T, int D, int GC, bool PAGED, bool SORTED>
static void launch_vec_gc(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  constexpr int NW = vec_waves<T, GC, SORTED>();
  decode_vec_kernel<T, D, GC, PAGED, NW, SORTED><<<grid, dim3(64 * NW), 0, stream>>>(a);
}

template <typename T, int D, bool PAGED, bool SORTED>
static hipError_t launch_vec_t(const DecodeArgs& a, int gc, hipStream_t stream) {
  const int G = a.heads / a.kv_heads;
  dim3 grid(a.nsplit, a.kv_heads * (G / gc), a.rows);
  switch (gc) {
    case 8:
      if constexpr (sizeof(T) == 4) launch_vec_gc<T, D, 8, PAGED, SORTED>(a, grid, stream);
      break;
    case 4:
      launch_vec_gc<T, D, 4, PAGED, SORTED>(a, grid, stream);
      break;
    case 2:
      launch_vec_gc<T, D, 2, PAGED, SORTED>(a, grid, stream);
      break;
    default:
      launch_vec_gc<T, D, 1, PAGED, SORTED>(a, grid, stream);
      break;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int gc = decode_vec_heads(a);
  hipError_t e;
  if (a.nsplit == 1 && a.rows <= kSortMaxRows)
    e = a.paged ? launch_vec_t<T, D, true, true>(a, gc, stream)
                : launch_vec_t<T, D, false, true>(a, gc, stream);
  else
    e = a.paged ? launch_vec_t<T, D, true, false>(a, gc, stream)
                : launch_vec_t<T, D, false, false>(a, gc, stream);
  if (e != hipSuccess || a.nsplit == 1) return e;  // one split: the output is written
  return launch_merge(a, stream);
}

// Bytes of split partials the launch below will write for `a` (0 when each
// row is covered by one split and the kernel writes the output itself).
size_t decode_partials_bytes(const DecodeArgs& a) {
  const int sl = decode_mfma_supported(a) ? decode_mfma_split_len(a.rows, a.kv_heads, a.cap)
                                          : decode_vec_split_len(a);
  const int nsplit = (a.cap + sl - 1) / sl;
  if (nsplit == 1) return 0;
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
    return launch_merge(a, stream);
  }
  a.split_len = decode_vec_split_len(a);
  a.nsplit = (a.cap + a.split_len - 1) / a.split_len;
  if (a.dtype == kDtypeBf16) {
    return a.head_dim == 64 ? launch_decode_t<uint16_t, 64>(a, stream)
                            : launch_decode_t<uint16_t, 128>(a, stream);
  }
  return a.head_dim == 64 ? launch_decode_t<float, 64>(a, stream)
                          : launch_decode_t<float, 128>(a, stream);
}

}  // namespace gqa
