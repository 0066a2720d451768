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
#include "decode_mfma.h"
#include "internal.h"

namespace gqa {

namespace {
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
}  // namespace

#ifndef GQA_DECODE_SORTED_WAVES
#define GQA_DECODE_SORTED_WAVES 8
#endif
constexpr int kWavesSorted = GQA_DECODE_SORTED_WAVES;  // ... with sorted dispatch

template <int D, bool PAGED, int NW, bool SORTED>
__global__ __launch_bounds__(64 * NW, NW == kWaves ? GQA_DECODE_MIN_WAVES_PER_SIMD : 1) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[decode_mfma_lds_bytes<D, NW>()];
  decode_mfma_body<D, PAGED, NW, SORTED, false>(a, blockIdx.x, blockIdx.y, blockIdx.z, smem);
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
