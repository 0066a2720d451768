// C ABI of the attention library: host-side validation (the `where` clause of
// the GroupedQueryAttention block on the Linnet "examples/01-llama" page,
// plus what this build supports) and dispatch to the kernel launchers. No
// C++ exception crosses this boundary; nothing here allocates or
// synchronizes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>

#include "gqa.h"
#include "internal.h"

namespace {

// Per calling thread: one thread's dry run or checked mode never changes
// another thread's calls. Checked mode starts on when GQA_CHECK is set to
// anything but "0" in the environment.
thread_local int32_t g_dry_run = 0;
int32_t env_checked() {
  const char* e = std::getenv("GQA_CHECK");
  return (e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0')) ? 1 : 0;
}
thread_local int32_t g_checked = env_checked();

// Checked mode: run the index checks; GQA_ERR_INDEX if any value is out of
// its range (nothing else is enqueued then).
int run_checks(const gqa::IndexCheck* c, int n, void* stream) {
  int bad = 0;
  const hipError_t e = gqa::index_check(c, n, static_cast<hipStream_t>(stream), &bad);
  if (e != hipSuccess) return GQA_ERR_HIP;
  return bad != 0 ? GQA_ERR_INDEX : GQA_OK;
}

int clamp_i32(long long x) { return x > 0x7fffffffLL ? 0x7fffffff : (int)x; }

// What each call's index arguments must satisfy in checked mode.
gqa::IndexCheck check_rope_write(int n, const int32_t* positions, const void* rope_table,
                                 int rope_max_pos, int cache_kind, int dim0, int seq,
                                 const int32_t* rows, const int32_t* slots, const int32_t* table,
                                 int table_rows, int table_pages) {
  gqa::IndexCheck c{};
  c.n = n;
  c.positions = positions;
  if (rope_table != nullptr) c.rope_hi = rope_max_pos;
  if (cache_kind == GQA_CACHE_CONTIGUOUS) {
    c.rows = rows;
    c.rows_hi = dim0;
    c.pos_hi = seq;
  } else if (cache_kind == GQA_CACHE_PAGED_TABLE) {
    c.rows = rows;
    c.rows_hi = table_rows;
    c.pos_hi = clamp_i32((long long)table_pages * GQA_PAGE_SIZE);
    c.table = table;
    c.table_rows = table_rows;
    c.table_pages = table_pages;
    c.num_pages = dim0;
    c.table_mode = 1;
  } else if (cache_kind == GQA_CACHE_PAGED_SLOTS) {
    c.slots = slots;
    c.slots_hi = clamp_i32((long long)dim0 * GQA_PAGE_SIZE);
  }
  return c;
}

gqa::IndexCheck check_decode_rows(int batch, int max_seq, const int32_t* positions) {
  gqa::IndexCheck c{};
  c.n = batch;
  c.positions = positions;
  c.pos_hi = max_seq;
  return c;
}

gqa::IndexCheck check_paged_keys(int n, const int32_t* rows, bool row_is_token,
                                 const int32_t* positions, const int32_t* table, int table_rows,
                                 int table_pages, int num_pages, int window) {
  gqa::IndexCheck c{};
  c.n = n;
  c.rows = rows;
  c.row_is_token = row_is_token ? 1 : 0;
  c.rows_hi = table_rows;
  c.positions = positions;
  c.pos_hi = clamp_i32((long long)table_pages * GQA_PAGE_SIZE);
  c.table = table;
  c.table_rows = table_rows;
  c.table_pages = table_pages;
  c.num_pages = num_pages;
  c.table_mode = 2;
  c.window = window;
  return c;
}
constexpr float kLog2e = 1.4426950408889634f;

bool supported_dim(int32_t d) { return d == 64 || d == 128; }
bool valid_dtype(int32_t t) { return t == GQA_BF16 || t == GQA_F32; }

// where Heads > 0, KvHeads > 0, Heads % KvHeads == 0, (H / Heads) % 2 == 0.
int check_heads(int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype) {
  if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0) return GQA_ERR_INVALID_ARG;
  if (head_dim <= 0 || head_dim % 2 != 0) return GQA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return GQA_ERR_INVALID_ARG;
  if (!supported_dim(head_dim)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

float effective_scale_log2(float scale, int32_t head_dim) {
  // rsqrt(cast<f32>(H / Heads)) as the correctly rounded f32 value.
  const float s = scale != 0.0f ? scale : (float)(1.0 / std::sqrt((double)head_dim));
  return s * kLog2e;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

}  // namespace

extern "C" {

int32_t gqa_abi_version(void) { return 1; }

int32_t gqa_set_dry_run(int32_t on) {
  const int32_t prev = g_dry_run;
  g_dry_run = on ? 1 : 0;
  return prev;
}

int32_t gqa_set_checked(int32_t on) {
  const int32_t prev = g_checked;
  g_checked = on ? 1 : 0;
  return prev;
}

const char* gqa_status_string(int32_t status) {
  switch (status) {
    case GQA_OK:
      return "ok";
    case GQA_ERR_INVALID_ARG:
      return "invalid argument";
    case GQA_ERR_UNSUPPORTED:
      return "unsupported dtype / head dim / operation";
    case GQA_ERR_WORKSPACE:
      return "workspace missing or too small";
    case GQA_ERR_HIP:
      return "HIP runtime error";
    case GQA_ERR_INDEX:
      return "index argument out of range (checked mode)";
    default:
      return "unknown status";
  }
}

const char* gqa_status_str(int32_t status) { return gqa_status_string(status); }

int gqa_rope_table(int32_t head_dim, int32_t max_pos, float theta, int32_t dtype, void* table,
                   void* stream) {
  if (head_dim <= 0 || head_dim % 2 != 0 || max_pos <= 0 || !valid_dtype(dtype))
    return GQA_ERR_INVALID_ARG;
  if (!(theta > 0.0f) || !std::isfinite(theta)) return GQA_ERR_INVALID_ARG;
  if (table == nullptr) return GQA_ERR_INVALID_ARG;
  if (!supported_dim(head_dim)) return GQA_ERR_UNSUPPORTED;
  if (g_dry_run) return GQA_OK;
  return hip_status(gqa::launch_rope_table(head_dim, max_pos, theta, dtype, table,
                                           static_cast<hipStream_t>(stream)));
}

int gqa_rope_write_kv(int32_t n, int32_t heads, int32_t kv_heads, int32_t head_dim,
                      int32_t dtype, void* q, void* k, const void* v,
                      const int32_t* positions, const void* rope_table, int32_t rope_max_pos,
                      int32_t cache_kind, void* cache_k, void* cache_v, int32_t cache_dim0,
                      int32_t cache_seq, const int32_t* rows, const int32_t* slots,
                      const int32_t* table, int32_t table_rows, int32_t table_pages,
                      void* stream) {
  if (n < 0) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (cache_kind < GQA_CACHE_NONE || cache_kind > GQA_CACHE_PAGED_SLOTS) return GQA_ERR_INVALID_ARG;
  if (rope_table != nullptr && rope_max_pos <= 0) return GQA_ERR_INVALID_ARG;
  const bool needs_pos = rope_table != nullptr || cache_kind == GQA_CACHE_CONTIGUOUS ||
                         cache_kind == GQA_CACHE_PAGED_TABLE;
  if (needs_pos && positions == nullptr) return GQA_ERR_INVALID_ARG;
  if (cache_kind != GQA_CACHE_NONE) {
    if (k == nullptr || cache_k == nullptr) return GQA_ERR_INVALID_ARG;
    if (v != nullptr && cache_v == nullptr) return GQA_ERR_INVALID_ARG;
    if (cache_dim0 <= 0) return GQA_ERR_INVALID_ARG;
    if (cache_kind == GQA_CACHE_CONTIGUOUS && cache_seq <= 0) return GQA_ERR_INVALID_ARG;
    if (cache_kind != GQA_CACHE_CONTIGUOUS && cache_seq != GQA_PAGE_SIZE)
      return GQA_ERR_INVALID_ARG;
    if (cache_kind == GQA_CACHE_PAGED_TABLE &&
        (table == nullptr || table_rows <= 0 || table_pages <= 0))
      return GQA_ERR_INVALID_ARG;
    if (cache_kind == GQA_CACHE_PAGED_SLOTS && slots == nullptr) return GQA_ERR_INVALID_ARG;
  } else if (rope_table == nullptr || (q == nullptr && k == nullptr)) {
    return GQA_ERR_INVALID_ARG;  // nothing to do is a caller error
  }
  if (n == 0 || g_dry_run) return GQA_OK;
  if (g_checked) {
    const gqa::IndexCheck c = check_rope_write(n, positions, rope_table, rope_max_pos, cache_kind,
                                               cache_dim0, cache_seq, rows, slots, table,
                                               table_rows, table_pages);
    st = run_checks(&c, 1, stream);
    if (st != GQA_OK) return st;
  }
  gqa::RopeWriteArgs a;
  a.n = n;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.v = v;
  a.positions = positions;
  a.rope_table = rope_table;
  a.rope_max_pos = rope_max_pos;
  a.cache_kind = cache_kind;
  a.cache_k = cache_k;
  a.cache_v = cache_v;
  a.cache_dim0 = cache_dim0;
  a.cache_seq = cache_seq;
  a.rows = rows;
  a.slots = slots;
  a.table = table;
  a.table_rows = table_rows;
  a.table_pages = table_pages;
  return hip_status(gqa::launch_rope_write(a, static_cast<hipStream_t>(stream)));
}

size_t gqa_prefill_packed_workspace(int32_t p, int32_t heads, int32_t kv_heads,
                                    int32_t head_dim) {
  if (p <= 0) return 0;
  return gqa::prefill_workspace_bytes(p, heads, kv_heads, head_dim);
}

// What a packed prefill call launches: plan and attention, the plan alone,
// or the attention alone on a plan already in the workspace.
enum class PackedPart { kAll, kPlan, kPlanned };

static int prefill_packed_impl(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                               int32_t dtype, float scale, int32_t window, const void* sinks,
                               const void* q, const void* k, const void* v,
                               const int32_t* positions, const int32_t* segments, void* out,
                               void* workspace, size_t workspace_bytes, void* stream, bool launch,
                               PackedPart part = PackedPart::kAll) {
  if (p < 0 || window < 0) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (!std::isfinite(scale) || scale < 0.0f) return GQA_ERR_INVALID_ARG;
  if (positions == nullptr || segments == nullptr) return GQA_ERR_INVALID_ARG;
  if (part != PackedPart::kPlan && (q == nullptr || k == nullptr || v == nullptr || out == nullptr))
    return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  // Each KV head's K (and V) is addressed through one 32-bit buffer range.
  if ((long long)p * kv_heads * head_dim * 2 + 4096 >= (1LL << 31)) return GQA_ERR_UNSUPPORTED;
  if (p == 0) return GQA_OK;
  const size_t need = gqa::prefill_workspace_bytes(p, heads, kv_heads, head_dim);
  if (workspace == nullptr || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GQA_ERR_WORKSPACE;
  if (!launch) return GQA_OK;
  gqa::PrefillArgs a{};
  a.p = p;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.scale_log2 = effective_scale_log2(scale, head_dim);
  a.window = window;
  a.sinks = sinks;
  a.q = q;
  a.k = k;
  a.v = v;
  a.positions = positions;
  a.segments = segments;
  a.out = out;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.src = gqa::kSrcPacked;
  if (part == PackedPart::kPlan) return hip_status(gqa::launch_prefill_plan(a, static_cast<hipStream_t>(stream)));
  return hip_status(gqa::launch_prefill(a, static_cast<hipStream_t>(stream), part == PackedPart::kPlanned));
}

int gqa_prefill_packed_plan(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                            int32_t window, const int32_t* positions, const int32_t* segments,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_packed_impl(p, heads, kv_heads, head_dim, GQA_BF16, 0.0f, window, nullptr, nullptr,
                             nullptr, nullptr, positions, segments, nullptr, workspace, workspace_bytes,
                             stream, !g_dry_run, PackedPart::kPlan);
}

int gqa_prefill_packed_planned(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                               int32_t dtype, float scale, int32_t window, const void* sinks,
                               const void* q, const void* k, const void* v,
                               const int32_t* positions, const int32_t* segments, void* out,
                               const void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_packed_impl(p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, k, v,
                             positions, segments, out, const_cast<void*>(workspace), workspace_bytes,
                             stream, !g_dry_run, PackedPart::kPlanned);
}

int gqa_prefill_packed(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                       int32_t dtype, float scale, int32_t window, const void* sinks,
                       const void* q, const void* k, const void* v,
                       const int32_t* positions, const int32_t* segments, void* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_packed_impl(p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, k, v,
                             positions, segments, out, workspace, workspace_bytes, stream,
                             !g_dry_run);
}

int gqa_prefill_packed_lse(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                           int32_t dtype, float scale, int32_t window, const void* q, const void* k,
                           const void* v, const int32_t* positions, const int32_t* segments,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (lse == nullptr) return GQA_ERR_INVALID_ARG;
  const int st = prefill_packed_impl(p, heads, kv_heads, head_dim, dtype, scale, window, nullptr, q, k,
                                     v, positions, segments, out, workspace, workspace_bytes, stream,
                                     false);
  if (st != GQA_OK || p == 0 || g_dry_run) return st;
  gqa::PrefillArgs a{};
  a.p = p;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.scale_log2 = effective_scale_log2(scale, head_dim);
  a.window = window;
  a.q = q;
  a.k = k;
  a.v = v;
  a.positions = positions;
  a.segments = segments;
  a.out = out;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.src = gqa::kSrcPacked;
  a.lse = lse;
  return hip_status(gqa::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

size_t gqa_prefill_packed_backward_workspace(int32_t p, int32_t heads, int32_t kv_heads,
                                             int32_t head_dim) {
  (void)kv_heads;
  (void)head_dim;
  if (p <= 0 || heads <= 0) return 0;
  return gqa::prefill_bwd_workspace_bytes(p, heads);
}

int gqa_prefill_packed_backward(int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                int32_t dtype, float scale, int32_t window, const void* q,
                                const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const int32_t* positions,
                                const int32_t* segments, void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (p < 0 || window < 0) return GQA_ERR_INVALID_ARG;
  const int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (!std::isfinite(scale) || scale < 0.0f) return GQA_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr ||
      lse == nullptr || positions == nullptr || segments == nullptr || dq == nullptr ||
      dk == nullptr || dv == nullptr)
    return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (p == 0) return GQA_OK;
  const size_t need = gqa::prefill_bwd_workspace_bytes(p, heads);
  if (workspace == nullptr || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GQA_ERR_WORKSPACE;
  if (g_dry_run) return GQA_OK;
  gqa::BwdArgs a{};
  a.p = p;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.scale = scale != 0.0f ? scale : (float)(1.0 / std::sqrt((double)head_dim));
  a.window = window;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.positions = positions;
  a.segments = segments;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  return hip_status(gqa::launch_prefill_bwd(a, static_cast<hipStream_t>(stream)));
}

size_t gqa_prefill_cached_workspace(int32_t n, int32_t heads, int32_t kv_heads,
                                    int32_t head_dim) {
  if (n <= 0) return 0;
  return gqa::prefill_workspace_bytes(n, heads, kv_heads, head_dim);
}

static int prefill_cached_impl(int32_t n, int32_t heads, int32_t kv_heads, int32_t head_dim,
                               int32_t dtype, float scale, int32_t window, const void* sinks,
                               const void* q, const int32_t* rows, const int32_t* positions,
                               int32_t cache_kind, const void* cache_k, const void* cache_v,
                               int32_t cache_dim0, int32_t cache_seq, const int32_t* table,
                               int32_t table_rows, int32_t table_pages, void* out,
                               void* workspace, size_t workspace_bytes, void* stream,
                               bool launch, bool check,
                               const gqa::DecodeArgs* with_decode = nullptr) {
  if (n < 0 || window < 0) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (!std::isfinite(scale) || scale < 0.0f) return GQA_ERR_INVALID_ARG;
  if (q == nullptr || positions == nullptr || cache_k == nullptr || cache_v == nullptr ||
      out == nullptr)
    return GQA_ERR_INVALID_ARG;
  if (cache_kind != GQA_CACHE_CONTIGUOUS && cache_kind != GQA_CACHE_PAGED_TABLE)
    return GQA_ERR_INVALID_ARG;
  if (cache_dim0 <= 0) return GQA_ERR_INVALID_ARG;
  if (cache_kind == GQA_CACHE_CONTIGUOUS && cache_seq <= 0) return GQA_ERR_INVALID_ARG;
  if (cache_kind == GQA_CACHE_PAGED_TABLE) {
    if (cache_seq != GQA_PAGE_SIZE || table == nullptr || table_rows <= 0 || table_pages <= 0)
      return GQA_ERR_INVALID_ARG;
    if ((long long)table_pages * GQA_PAGE_SIZE > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;
  }
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (n == 0) return GQA_OK;
  const size_t need = gqa::prefill_workspace_bytes(n, heads, kv_heads, head_dim);
  if (workspace == nullptr || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GQA_ERR_WORKSPACE;
  if (!launch) return GQA_OK;
  if (check) {
    gqa::IndexCheck c{};
    if (cache_kind == GQA_CACHE_CONTIGUOUS) {
      c.n = n;
      c.rows = rows;
      c.rows_hi = cache_dim0;
      c.positions = positions;
      c.pos_hi = cache_seq;
    } else {
      c = check_paged_keys(n, rows, false, positions, table, table_rows, table_pages, cache_dim0,
                           window);
    }
    st = run_checks(&c, 1, stream);
    if (st != GQA_OK) return st;
  }
  gqa::PrefillArgs a{};
  a.p = n;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.scale_log2 = effective_scale_log2(scale, head_dim);
  a.window = window;
  a.sinks = sinks;
  a.q = q;
  a.k = cache_k;
  a.v = cache_v;
  a.positions = positions;
  a.segments = rows;
  a.out = out;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  if (cache_kind == GQA_CACHE_CONTIGUOUS) {
    a.src = gqa::kSrcContiguous;
    a.cache_rows = cache_dim0;
    a.cap = cache_seq;
  } else {
    a.src = gqa::kSrcPaged;
    a.cache_rows = table_rows;
    a.cap = table_pages * GQA_PAGE_SIZE;
    a.table = table;
    a.table_pages = table_pages;
    a.num_pages = cache_dim0;
  }
  if (with_decode != nullptr)
    return hip_status(gqa::launch_prefill_step(a, *with_decode, static_cast<hipStream_t>(stream)));
  return hip_status(gqa::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

int gqa_prefill_cached(int32_t n, int32_t heads, int32_t kv_heads, int32_t head_dim,
                       int32_t dtype, float scale, int32_t window, const void* sinks,
                       const void* q, const int32_t* rows, const int32_t* positions,
                       int32_t cache_kind, const void* cache_k, const void* cache_v,
                       int32_t cache_dim0, int32_t cache_seq, const int32_t* table,
                       int32_t table_rows, int32_t table_pages, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return prefill_cached_impl(n, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, rows,
                             positions, cache_kind, cache_k, cache_v, cache_dim0, cache_seq, table,
                             table_rows, table_pages, out, workspace, workspace_bytes, stream,
                             !g_dry_run, g_checked != 0);
}

static size_t decode_ws(int rows, int heads, int kv_heads, int head_dim, int dtype, int paged,
                        int cap) {
  size_t ws = 0;
  gqa::decode_plan(rows, heads, kv_heads, head_dim, dtype, paged, cap, nullptr, nullptr, &ws);
  return ws;
}

size_t gqa_decode_rows_workspace(int32_t batch, int32_t heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t max_seq) {
  if (batch <= 0 || heads <= 0 || max_seq <= 0) return 0;
  // The plan does not depend on dtype for the contiguous cache.
  return decode_ws(batch, heads, kv_heads, head_dim, GQA_F32, 0, max_seq);
}

size_t gqa_decode_paged_workspace(int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                                  int32_t head_dim) {
  if (rows <= 0 || pages <= 0 || heads <= 0) return 0;
  if ((long long)pages * GQA_PAGE_SIZE > 0x7fffffffLL) return 0;
  const size_t a = decode_ws(rows, heads, kv_heads, head_dim, GQA_BF16, 1, pages * GQA_PAGE_SIZE);
  const size_t b = decode_ws(rows, heads, kv_heads, head_dim, GQA_F32, 1, pages * GQA_PAGE_SIZE);
  return a > b ? a : b;
}

static int decode_common(gqa::DecodeArgs& a, size_t workspace_bytes, void* workspace,
                         hipStream_t stream, bool launch) {
  const size_t need =
      decode_ws(a.rows, a.heads, a.kv_heads, a.head_dim, a.dtype, a.paged, a.cap);
  if (workspace == nullptr || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GQA_ERR_WORKSPACE;
  if (!launch) return GQA_OK;
  a.ws = static_cast<float*>(workspace);
  return hip_status(gqa::launch_decode(a, stream));
}

static int decode_rows_impl(int32_t batch, int32_t heads, int32_t kv_heads, int32_t head_dim,
                    int32_t dtype, float scale, int32_t window, const void* sinks,
                    const void* q, const void* cache_k, const void* cache_v, int32_t max_seq,
                    const int32_t* positions, void* out, void* workspace,
                    size_t workspace_bytes, void* stream, bool launch, bool check) {
  if (batch < 0 || window < 0 || max_seq <= 0) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (!std::isfinite(scale) || scale < 0.0f) return GQA_ERR_INVALID_ARG;
  if (q == nullptr || cache_k == nullptr || cache_v == nullptr || positions == nullptr ||
      out == nullptr)
    return GQA_ERR_INVALID_ARG;
  if (batch == 0) return GQA_OK;
  if (launch && check) {
    const gqa::IndexCheck c = check_decode_rows(batch, max_seq, positions);
    st = run_checks(&c, 1, stream);
    if (st != GQA_OK) return st;
  }
  gqa::DecodeArgs a{};
  a.rows = batch;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.scale_log2 = effective_scale_log2(scale, head_dim);
  a.window = window;
  a.sinks = sinks;
  a.q = q;
  a.k = cache_k;
  a.v = cache_v;
  a.positions = positions;
  a.table = nullptr;
  a.paged = 0;
  a.cap = max_seq;
  a.pages = 0;
  a.num_pages = 0;
  a.out = out;
  return decode_common(a, workspace_bytes, workspace, static_cast<hipStream_t>(stream), launch);
}

int gqa_decode_rows(int32_t batch, int32_t heads, int32_t kv_heads, int32_t head_dim,
                    int32_t dtype, float scale, int32_t window, const void* sinks,
                    const void* q, const void* cache_k, const void* cache_v, int32_t max_seq,
                    const int32_t* positions, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_rows_impl(batch, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, cache_k,
                          cache_v, max_seq, positions, out, workspace, workspace_bytes, stream,
                          !g_dry_run, g_checked != 0);
}

static gqa::DecodeArgs paged_decode_args(int32_t rows, int32_t pages, int32_t heads,
                                         int32_t kv_heads, int32_t head_dim, int32_t dtype,
                                         float scale, int32_t window, const void* sinks,
                                         const void* q, const void* pool_k, const void* pool_v,
                                         int32_t num_pages, const int32_t* positions,
                                         const int32_t* table, void* out) {
  gqa::DecodeArgs a{};
  a.rows = rows;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.scale_log2 = effective_scale_log2(scale, head_dim);
  a.window = window;
  a.sinks = sinks;
  a.q = q;
  a.k = pool_k;
  a.v = pool_v;
  a.positions = positions;
  a.table = table;
  a.paged = 1;
  a.cap = pages * GQA_PAGE_SIZE;
  a.pages = pages;
  a.num_pages = num_pages;
  a.out = out;
  return a;
}

static int decode_paged_impl(int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                     int32_t head_dim, int32_t dtype, float scale, int32_t window,
                     const void* sinks, const void* q, const void* pool_k, const void* pool_v,
                     int32_t num_pages, const int32_t* positions, const int32_t* table,
                     void* out, void* workspace, size_t workspace_bytes, void* stream, bool launch,
                     bool check, bool noalloc = false) {
  if (rows < 0 || pages <= 0 || num_pages <= 0 || window < 0) return GQA_ERR_INVALID_ARG;
  if ((long long)pages * GQA_PAGE_SIZE > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (!std::isfinite(scale) || scale < 0.0f) return GQA_ERR_INVALID_ARG;
  if (q == nullptr || pool_k == nullptr || pool_v == nullptr || positions == nullptr ||
      table == nullptr || out == nullptr)
    return GQA_ERR_INVALID_ARG;
  if (rows == 0) return GQA_OK;
  if (launch && check) {
    const gqa::IndexCheck c =
        check_paged_keys(rows, nullptr, true, positions, table, rows, pages, num_pages, window);
    st = run_checks(&c, 1, stream);
    if (st != GQA_OK) return st;
  }
  gqa::DecodeArgs a = paged_decode_args(rows, pages, heads, kv_heads, head_dim, dtype, scale, window,
                                        sinks, q, pool_k, pool_v, num_pages, positions, table, out);
  if (noalloc) {
    // The split partials go to the library's own device array.
    if (gqa::decode_partials_bytes(a) > gqa::kDecodeScratchBytes) return GQA_ERR_WORKSPACE;
    if (!launch) return GQA_OK;
    float* ptr = nullptr;
    if (gqa::decode_scratch(&ptr) != hipSuccess) return GQA_ERR_HIP;
    a.ws = ptr;
    return hip_status(gqa::launch_decode(a, static_cast<hipStream_t>(stream)));
  }
  return decode_common(a, workspace_bytes, workspace, static_cast<hipStream_t>(stream), launch);
}

int gqa_decode_paged(int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                     int32_t head_dim, int32_t dtype, float scale, int32_t window,
                     const void* sinks, const void* q, const void* pool_k, const void* pool_v,
                     int32_t num_pages, const int32_t* positions, const int32_t* table,
                     void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_paged_impl(rows, pages, heads, kv_heads, head_dim, dtype, scale, window, sinks, q,
                           pool_k, pool_v, num_pages, positions, table, out, workspace,
                           workspace_bytes, stream, !g_dry_run, g_checked != 0);
}

int gqa_decode_paged_noalloc(int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                             int32_t head_dim, int32_t dtype, float scale, int32_t window,
                             const void* sinks, const void* q, const void* pool_k,
                             const void* pool_v, int32_t num_pages, const int32_t* positions,
                             const int32_t* table, void* out, void* stream) {
  return decode_paged_impl(rows, pages, heads, kv_heads, head_dim, dtype, scale, window, sinks, q,
                           pool_k, pool_v, num_pages, positions, table, out, nullptr, 0, stream,
                           !g_dry_run, false, true);
}


// ---------------------------------------------------------------------------
// step_packed / step_paged (llama-3.1-8b-instruct and gpt-oss-20b cards,
// serving signatures): one call over prefill tokens and one decode token per
// row, in the token order of the pages' types. Both parts write their k/v
// first (gqa_rope_write_kv); here each part runs its attention kernels on the
// same stream, out of one caller workspace (the prefill part's bytes, then the
// decode part's, each 256-byte aligned).
// ---------------------------------------------------------------------------
static size_t align_up_256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t gqa_step_packed_workspace(int32_t batch, int32_t p, int32_t heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t max_seq) {
  if (batch < 0 || p < 0) return 0;
  const size_t a = p > 0 ? align_up_256(gqa_prefill_packed_workspace(p, heads, kv_heads, head_dim)) : 0;
  const size_t b = batch > 0 ? gqa_decode_rows_workspace(batch, heads, kv_heads, head_dim, max_seq) : 0;
  return a + b;
}

int gqa_step_packed(int32_t batch, int32_t p, int32_t heads, int32_t kv_heads, int32_t head_dim,
                    int32_t dtype, float scale, int32_t window, const void* sinks, const void* q,
                    const void* k, const void* v, const int32_t* positions,
                    const int32_t* segments, const void* cache_k, const void* cache_v,
                    int32_t max_seq, const int32_t* step_positions, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (batch < 0 || p < 0) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (q == nullptr || out == nullptr) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  const size_t need = gqa_step_packed_workspace(batch, p, heads, kv_heads, head_dim, max_seq);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GQA_ERR_WORKSPACE;
  const size_t row = (size_t)heads * head_dim * 2;  // bytes of one token's q / out (bf16)
  const size_t pre_ws = p > 0 ? align_up_256(gqa_prefill_packed_workspace(p, heads, kv_heads, head_dim)) : 0;
  char* ws = static_cast<char*>(workspace);
  // Validate both parts before enqueuing either (dry-run validation first).
  const bool launch = !g_dry_run;
  int s1 = p > 0 ? prefill_packed_impl(p, heads, kv_heads, head_dim, dtype, scale, window, sinks,
                                      static_cast<const char*>(q) + batch * row, k, v, positions,
                                      segments, static_cast<char*>(out) + batch * row, ws,
                                      pre_ws, stream, false)
                 : GQA_OK;
  int s2 = batch > 0 ? decode_rows_impl(batch, heads, kv_heads, head_dim, dtype, scale, window,
                                        sinks, q, cache_k, cache_v, max_seq, step_positions, out,
                                        ws == nullptr ? nullptr : ws + pre_ws,
                                        workspace_bytes - pre_ws, stream, false, false)
                     : GQA_OK;
  if (s1 != GQA_OK) return s1;
  if (s2 != GQA_OK) return s2;
  if (!launch) return GQA_OK;
  if (g_checked && batch > 0) {
    // The packed part's positions and segments take any value.
    const gqa::IndexCheck c = check_decode_rows(batch, max_seq, step_positions);
    st = run_checks(&c, 1, stream);
    if (st != GQA_OK) return st;
  }
  if (batch > 0) {
    s2 = decode_rows_impl(batch, heads, kv_heads, head_dim, dtype, scale, window, sinks, q, cache_k,
                          cache_v, max_seq, step_positions, out, ws + pre_ws,
                          workspace_bytes - pre_ws, stream, true, false);
    if (s2 != GQA_OK) return s2;
  }
  if (p > 0)
    return prefill_packed_impl(p, heads, kv_heads, head_dim, dtype, scale, window, sinks,
                               static_cast<const char*>(q) + batch * row, k, v, positions, segments,
                               static_cast<char*>(out) + batch * row, ws, pre_ws, stream, true);
  return GQA_OK;
}

size_t gqa_step_paged_workspace(int32_t p, int32_t rows, int32_t pages, int32_t heads,
                                int32_t kv_heads, int32_t head_dim) {
  if (p < 0 || rows < 0) return 0;
  const size_t a = p > 0 ? align_up_256(gqa_prefill_cached_workspace(p, heads, kv_heads, head_dim)) : 0;
  const size_t b = rows > 0 ? gqa_decode_paged_workspace(rows, pages, heads, kv_heads, head_dim) : 0;
  return a + b;
}

int gqa_step_paged(int32_t p, int32_t rows, int32_t pages, int32_t heads, int32_t kv_heads,
                   int32_t head_dim, int32_t dtype, float scale, int32_t window, const void* sinks,
                   const void* q, const int32_t* token_rows, const int32_t* positions,
                   const void* pool_k, const void* pool_v, int32_t num_pages,
                   const int32_t* table, const int32_t* step_positions, void* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (p < 0 || rows < 0) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (q == nullptr || out == nullptr) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (rows <= 0 && p > 0) return GQA_ERR_INVALID_ARG;  // the table has `rows` rows
  const size_t need = gqa_step_paged_workspace(p, rows, pages, heads, kv_heads, head_dim);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GQA_ERR_WORKSPACE;
  const size_t row = (size_t)heads * head_dim * 2;
  const size_t pre_ws = p > 0 ? align_up_256(gqa_prefill_cached_workspace(p, heads, kv_heads, head_dim)) : 0;
  char* ws = static_cast<char*>(workspace);
  const bool launch = !g_dry_run;
  int s1 = p > 0 ? prefill_cached_impl(p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q,
                                       token_rows, positions, GQA_CACHE_PAGED_TABLE, pool_k, pool_v,
                                       num_pages, GQA_PAGE_SIZE, table, rows, pages, out, ws,
                                       pre_ws, stream, false, false)
                 : GQA_OK;
  int s2 = rows > 0 ? decode_paged_impl(rows, pages, heads, kv_heads, head_dim, dtype, scale, window,
                                        sinks, static_cast<const char*>(q) + p * row, pool_k,
                                        pool_v, num_pages, step_positions, table,
                                        static_cast<char*>(out) + p * row,
                                        ws == nullptr ? nullptr : ws + pre_ws,
                                        workspace_bytes - pre_ws, stream, false, false)
                    : GQA_OK;
  if (s1 != GQA_OK) return s1;
  if (s2 != GQA_OK) return s2;
  if (!launch) return GQA_OK;
  if (g_checked) {
    gqa::IndexCheck c[2];
    int nc = 0;
    if (p > 0)
      c[nc++] = check_paged_keys(p, token_rows, false, positions, table, rows, pages, num_pages,
                                 window);
    if (rows > 0)
      c[nc++] = check_paged_keys(rows, nullptr, true, step_positions, table, rows, pages, num_pages,
                                 window);
    st = run_checks(c, nc, stream);
    if (st != GQA_OK) return st;
  }
  if (p > 0 && rows > 0) {
    // Decode tokens and chunk tokens in one grid when the decode runs on
    // matrix cores: its workgroups stream the cache beside the prefill tiles.
    const gqa::DecodeArgs d = paged_decode_args(
        rows, pages, heads, kv_heads, head_dim, dtype, scale, window, sinks,
        static_cast<const char*>(q) + p * row, pool_k, pool_v, num_pages, step_positions, table,
        static_cast<char*>(out) + p * row);
    if (gqa::decode_mfma_supported(d))
      return prefill_cached_impl(p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q,
                                 token_rows, positions, GQA_CACHE_PAGED_TABLE, pool_k, pool_v,
                                 num_pages, GQA_PAGE_SIZE, table, rows, pages, out, ws, pre_ws,
                                 stream, true, false, &d);
  }
  if (rows > 0) {
    s2 = decode_paged_impl(rows, pages, heads, kv_heads, head_dim, dtype, scale, window, sinks,
                           static_cast<const char*>(q) + p * row, pool_k, pool_v, num_pages,
                           step_positions, table, static_cast<char*>(out) + p * row, ws + pre_ws,
                           workspace_bytes - pre_ws, stream, true, false);
    if (s2 != GQA_OK) return s2;
  }
  if (p > 0)
    return prefill_cached_impl(p, heads, kv_heads, head_dim, dtype, scale, window, sinks, q,
                               token_rows, positions, GQA_CACHE_PAGED_TABLE, pool_k, pool_v,
                               num_pages, GQA_PAGE_SIZE, table, rows, pages, out, ws, pre_ws,
                               stream, true, false);
  return GQA_OK;
}

int gqa_qkv_rope_write(int32_t n, int32_t hidden, int32_t heads, int32_t kv_heads,
                       int32_t head_dim, int32_t dtype, const void* x, const void* w_q,
                       const void* w_k, const void* w_v, const void* b_q, const void* b_k,
                       const void* b_v, const int32_t* positions, const void* rope_table,
                       int32_t rope_max_pos, void* q_out, void* k_out, void* v_out,
                       int32_t cache_kind, void* cache_k, void* cache_v, int32_t cache_dim0,
                       int32_t cache_seq, const int32_t* rows, const int32_t* slots,
                       const int32_t* table, int32_t table_rows, int32_t table_pages,
                       void* stream) {
  if (n < 0 || hidden <= 0) return GQA_ERR_INVALID_ARG;
  int st = check_heads(heads, kv_heads, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (x == nullptr || w_q == nullptr || w_k == nullptr || w_v == nullptr || q_out == nullptr)
    return GQA_ERR_INVALID_ARG;
  if (cache_kind < GQA_CACHE_NONE || cache_kind > GQA_CACHE_PAGED_SLOTS) return GQA_ERR_INVALID_ARG;
  if (rope_table != nullptr && (rope_max_pos <= 0 || positions == nullptr)) return GQA_ERR_INVALID_ARG;
  if (cache_kind != GQA_CACHE_NONE) {
    if (cache_k == nullptr || cache_dim0 <= 0) return GQA_ERR_INVALID_ARG;
    if (cache_kind == GQA_CACHE_CONTIGUOUS && (cache_seq <= 0 || positions == nullptr))
      return GQA_ERR_INVALID_ARG;
    if (cache_kind != GQA_CACHE_CONTIGUOUS && cache_seq != GQA_PAGE_SIZE) return GQA_ERR_INVALID_ARG;
    if (cache_kind == GQA_CACHE_PAGED_TABLE &&
        (table == nullptr || table_rows <= 0 || table_pages <= 0 || positions == nullptr))
      return GQA_ERR_INVALID_ARG;
    if (cache_kind == GQA_CACHE_PAGED_SLOTS && slots == nullptr) return GQA_ERR_INVALID_ARG;
  }
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  // Tiles: K slabs of 64 hidden features, 128 output features per tile.
  if (hidden % 64 != 0 || ((long long)(heads + 2 * kv_heads) * head_dim) % 128 != 0)
    return GQA_ERR_UNSUPPORTED;
  if (((long long)n + 128) * hidden * 2 > 0x7fffffffLL) return GQA_ERR_UNSUPPORTED;
  if (n == 0 || g_dry_run) return GQA_OK;
  if (g_checked) {
    const gqa::IndexCheck c = check_rope_write(n, positions, rope_table, rope_max_pos, cache_kind,
                                               cache_dim0, cache_seq, rows, slots, table,
                                               table_rows, table_pages);
    st = run_checks(&c, 1, stream);
    if (st != GQA_OK) return st;
  }
  gqa::QkvArgs a{};
  a.n = n;
  a.hidden = hidden;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.x = x;
  a.wq = w_q;
  a.wk = w_k;
  a.wv = w_v;
  a.bq = b_q;
  a.bk = b_k;
  a.bv = b_v;
  a.q_out = q_out;
  a.k_out = k_out;
  a.v_out = v_out;
  a.wr.n = n;
  a.wr.heads = heads;
  a.wr.kv_heads = kv_heads;
  a.wr.head_dim = head_dim;
  a.wr.dtype = dtype;
  a.wr.positions = positions;
  a.wr.rope_table = rope_table;
  a.wr.rope_max_pos = rope_max_pos;
  a.wr.cache_kind = cache_kind;
  a.wr.cache_k = cache_k;
  a.wr.cache_v = cache_v;
  a.wr.cache_dim0 = cache_dim0;
  a.wr.cache_seq = cache_seq;
  a.wr.rows = rows;
  a.wr.slots = slots;
  a.wr.table = table;
  a.wr.table_rows = table_rows;
  a.wr.table_pages = table_pages;
  return hip_status(gqa::launch_qkv(a, static_cast<hipStream_t>(stream)));
}

size_t gqa_workspace_bytes(int32_t op, int32_t heads, int32_t kv_heads, int32_t head_dim,
                           int32_t n_tokens, int32_t n_rows, int32_t max_len) {
  switch (op) {
    case GQA_OP_PREFILL_PACKED:
      return gqa_prefill_packed_workspace(n_tokens, heads, kv_heads, head_dim);
    case GQA_OP_PREFILL_CACHED:
      return gqa_prefill_cached_workspace(n_tokens, heads, kv_heads, head_dim);
    case GQA_OP_PREFILL_BACKWARD:
      return gqa_prefill_packed_backward_workspace(n_tokens, heads, kv_heads, head_dim);
    case GQA_OP_DECODE_ROWS:
      return gqa_decode_rows_workspace(n_rows, heads, kv_heads, head_dim, max_len);
    case GQA_OP_DECODE_PAGED:
      return gqa_decode_paged_workspace(n_rows, max_len, heads, kv_heads, head_dim);
    case GQA_OP_STEP_PACKED:
      return gqa_step_packed_workspace(n_rows, n_tokens, heads, kv_heads, head_dim, max_len);
    case GQA_OP_STEP_PAGED:
      return gqa_step_paged_workspace(n_tokens, n_rows, max_len, heads, kv_heads, head_dim);
    default:
      return 0;
  }
}

}  // extern "C"
