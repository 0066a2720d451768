// Checked mode: device-side validation of the index arguments of a call
// (rows, positions, slots, page-table entries) before its kernels run.
//
// Every index value already has a defined, memory-safe meaning in the
// kernels (a write outside the cache is dropped, a page id outside the pool
// contributes no keys, ...), following `write_at` as a masked select (Linnet
// "examples/01-llama" page, Key ideas, KV cache in state). Checked mode turns
// those cases into an error instead: one thread per token counts the values
// outside their range; the host reads the count back (this synchronizes the
// stream, which checked mode documents) and returns GQA_ERR_INDEX without
// enqueuing the call's own kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"
#include "internal.h"

namespace gqa {

// Violation counter of the check kernels: one int per device, module
// storage (nothing is allocated). Calls in checked mode take a host lock
// around their use of it.
static __device__ int g_index_violations;

__global__ __launch_bounds__(256) void index_zero_kernel(int* count) { *count = 0; }

__global__ __launch_bounds__(256) void index_check_kernel(IndexCheck c, int* count) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= c.n) return;
  int bad = 0;
  const int r = c.rows != nullptr ? c.rows[t] : (c.row_is_token ? t : 0);
  bool row_ok = true;
  if (c.rows_hi > 0) {
    row_ok = r >= 0 && r < c.rows_hi;
    bad += !row_ok;
  }
  const int p = c.positions != nullptr ? c.positions[t] : 0;
  bool pos_ok = true;
  if (c.positions != nullptr && c.pos_hi > 0) {
    pos_ok = p >= 0 && p < c.pos_hi;
    bad += !pos_ok;
  }
  if (c.positions != nullptr && c.rope_hi > 0) bad += !(p >= 0 && p < c.rope_hi);
  if (c.slots != nullptr) {
    const int s = c.slots[t];
    bad += !(s >= 0 && s < c.slots_hi);
  }
  if (c.table_mode != 0 && row_ok && pos_ok && r >= 0 && r < c.table_rows && p >= 0) {
    // Pages the call reads (mode 2: every page of the attended key range)
    // or writes (mode 1: the page of position p).
    const int last = p / kPageSize;
    int first = last;
    if (c.table_mode == 2) {
      const long long lo = c.window > 0 ? (long long)p - c.window + 1 : 0;
      first = (int)((lo > 0 ? lo : 0) / kPageSize);
    }
    for (int pg = first; pg <= last && pg < c.table_pages; ++pg) {
      const int id = c.table[(long long)r * c.table_pages + pg];
      bad += !(id >= 0 && id < c.num_pages);
    }
  }
  if (bad != 0) atomicAdd(count, bad);
}

hipError_t index_check(const IndexCheck* checks, int n_checks, hipStream_t stream, int* violations) {
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  *violations = 0;
  int* count = nullptr;
  hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&count), HIP_SYMBOL(g_index_violations));
  if (e != hipSuccess) return e;
  index_zero_kernel<<<1, 1, 0, stream>>>(count);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i < n_checks; ++i) {
    if (checks[i].n <= 0) continue;
    index_check_kernel<<<dim3((checks[i].n + 255) / 256), dim3(256), 0, stream>>>(checks[i], count);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int h = 0;
  e = hipMemcpyAsync(&h, count, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *violations = h;
  return hipSuccess;
}

}  // namespace gqa
