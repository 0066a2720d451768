// Diagnostic kernel outside the attention path: a streaming read of a device
// buffer, timed by bench.py as the measured HBM read ceiling that the decode
// is compared with (the published 8 TB/s is not reachable by any read).
//
// Every lane reads 16-byte chunks with nontemporal loads in a grid-stride
// loop, 8 loads in flight per lane; the XOR of all words a workgroup read is
// folded into one 32-bit word (so the loads cannot be dropped) and stored to
// out[blockIdx.x] -- a plain store per workgroup, no atomics on one address.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gqa.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kBlocks = GQA_DIAG_READ_BLOCKS;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, long long n16,
                                                               uint32_t* out) {
  const long long stride = (long long)gridDim.x * kThreads * kUnroll;
  uint32_t acc = 0;
  for (long long i = (long long)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n16; i += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long long j = i + (long long)u * kThreads;
      v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

extern "C" int gqa_diag_stream_read(const void* buffer, size_t bytes, void* out, void* stream) {
  if (buffer == nullptr || out == nullptr || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buffer) % 16 != 0)
    return GQA_ERR_INVALID_ARG;
  if (bytes == 0) return GQA_OK;
  const long long n16 = (long long)(bytes / 16);
  const long long per_block = (long long)kThreads * kUnroll;
  const int blocks = (int)((n16 + per_block - 1) / per_block < kBlocks ? (n16 + per_block - 1) / per_block : kBlocks);
  stream_read_kernel<<<blocks, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buffer), n16, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}
