// Launcher interface between the C ABI (gqa_api.cpp) and the kernels. Host
// code only: argument structs passed by value to kernels, and the launchers
// each kernel file provides. All pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

constexpr int kDtypeBf16 = 0;
constexpr int kDtypeF32 = 1;

struct RopeWriteArgs {
  int n, heads, kv_heads, head_dim, dtype;
  void* q;
  void* k;
  const void* v;
  const int32_t* positions;
  const void* rope_table;
  int rope_max_pos;
  int cache_kind;  // 0 none, 1 contiguous, 2 paged table, 3 paged slots
  void* cache_k;
  void* cache_v;
  int cache_dim0;  // batch (contiguous) or num_pages (paged)
  int cache_seq;   // max_seq (contiguous) or page size (paged)
  const int32_t* rows;
  const int32_t* slots;
  const int32_t* table;
  int table_rows, table_pages;
};

// One decode call, contiguous or paged.
struct DecodeArgs {
  int rows;          // batch rows / table rows
  int heads, kv_heads, head_dim, dtype;
  float scale_log2;  // scale * log2(e)
  int window;
  const void* sinks;  // [heads] of T or null
  const void* q;      // [rows, heads, D]
  const void* k;      // contiguous [rows, kvh, cap, D] or pool [num_pages, kvh, 64, D]
  const void* v;
  const int32_t* positions;  // [rows]
  const int32_t* table;      // [rows, pages] or null (contiguous)
  int paged;
  int cap;        // max_seq (contiguous) or pages * 64 (paged)
  int pages;      // table width (paged)
  int num_pages;  // pool size (paged)
  void* out;      // [rows, heads, D]
  float* ws;      // split partials
  int split_len;  // tokens per split
  int nsplit;     // splits per row
};

// Keys of the prefill: the packed tokens themselves, or a cache the tokens
// (and an earlier prefix) were written into.
enum PrefillSource { kSrcPacked = 0, kSrcContiguous = 1, kSrcPaged = 2 };

struct PrefillArgs {
  int p, heads, kv_heads, head_dim, dtype;
  float scale_log2;
  int window;
  const void* sinks;
  const void* q;
  const void* k;         // packed k [p, kv_heads, D], or cache_k / pool_k
  const void* v;
  const int32_t* positions;
  const int32_t* segments;  // packed: segment ids; cache: cache / table row (may be null = 0)
  void* out;
  void* ws;
  size_t ws_bytes;
  int src;               // PrefillSource
  int cache_rows;        // cache: batch (contiguous) or table rows (paged)
  int cap;               // cache: key slots per row (max_seq, or table_pages * 64)
  const int32_t* table;  // paged: [cache_rows, table_pages]
  int table_pages;
  int num_pages;
  float* lse;            // optional [p, heads]: natural-log softmax denominators
};

// Fused projections: x [n, hidden] times the q / k / v weights ([features,
// hidden] each), + optional biases, rounded to bf16, rotated and written
// (q to q_out, k / v to k_out / v_out and the cache described by wr, whose
// q / k / v fields are unused).
struct QkvArgs {
  int n, hidden, heads, kv_heads, head_dim;
  const void* x;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* bq;
  const void* bk;
  const void* bv;
  void* q_out;
  void* k_out;
  void* v_out;
  RopeWriteArgs wr;
};
hipError_t launch_qkv(const QkvArgs& a, hipStream_t stream);

hipError_t launch_rope_table(int head_dim, int max_pos, float theta, int dtype, void* table,
                             hipStream_t stream);
hipError_t launch_rope_write(const RopeWriteArgs& a, hipStream_t stream);

// Decode: split length / split count the launcher will use, the workspace
// bytes that needs, and the launch itself.
void decode_plan(int rows, int heads, int kv_heads, int head_dim, int dtype, int paged, int cap,
                 int* split_len, int* nsplit, size_t* ws_bytes);
hipError_t launch_decode(DecodeArgs a, hipStream_t stream);
// The entry point that allocates nothing: its split partials live in a
// module array of kDecodeScratchBytes per GPU; decode_scratch returns that
// array's device address on the current device, decode_partials_bytes what
// a launch needs of it.
constexpr size_t kDecodeScratchBytes = 16u << 20;
size_t decode_partials_bytes(const DecodeArgs& a);
hipError_t decode_scratch(float** ptr);
bool decode_mfma_supported(const DecodeArgs& a);
int decode_mfma_split_len(int rows, int kv_heads, int cap);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);

size_t prefill_workspace_bytes(int p, int heads, int kv_heads, int head_dim);
// The prefill (plan, then attention; with `planned` the attention alone, on
// the plan a launch_prefill_plan of the same p, heads, kv_heads, window,
// positions and segments left in a.ws).
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream, bool planned = false);
hipError_t launch_prefill_plan(const PrefillArgs& a, hipStream_t stream);
// A cached paged prefill and a one-split matrix-core paged decode (bf16,
// G <= 16, same head dim) in one grid; `d` needs no workspace.
hipError_t launch_prefill_step(const PrefillArgs& a, DecodeArgs d, hipStream_t stream);

// Backward of the packed prefill (bf16): dq [p, heads, D], dk / dv
// [p, kv_heads, D] from q, k, v, the forward's out and lse, and dout.
struct BwdArgs {
  int p, heads, kv_heads, head_dim;
  float scale;  // softmax scale (natural)
  int window;
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;  // [p, heads], natural log
  const int32_t* positions;
  const int32_t* segments;
  void* dq;
  void* dk;
  void* dv;
  void* ws;
  size_t ws_bytes;
};
size_t prefill_bwd_workspace_bytes(int p, int heads);
hipError_t launch_prefill_bwd(const BwdArgs& a, hipStream_t stream);

// Checked mode: one validation pass over n tokens' index arguments. A field
// left null / 0 is not checked.
struct IndexCheck {
  int n;
  const int32_t* rows;       // rows[t] in [0, rows_hi) (null: row 0, or t if row_is_token)
  int rows_hi;
  int row_is_token;
  const int32_t* positions;  // positions[t] in [0, pos_hi) (cache) and [0, rope_hi) (rotary table)
  int pos_hi, rope_hi;
  const int32_t* slots;      // slots[t] in [0, slots_hi)
  int slots_hi;
  const int32_t* table;      // [table_rows, table_pages] page ids in [0, num_pages)
  int table_rows, table_pages, num_pages;
  int table_mode;            // 1: the page of positions[t]; 2: the pages of its key range
  int window;
};
// Runs the checks on `stream`, waits for them, and returns the number of
// values found outside their range in *violations.
hipError_t index_check(const IndexCheck* checks, int n_checks, hipStream_t stream, int* violations);

}  // namespace gqa
