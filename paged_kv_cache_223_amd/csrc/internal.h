// Internal declarations shared by the C ABI (api.cpp) and the HIP launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pkv.h"

namespace pkv {

void set_error(const char* fmt, ...);
int hip_status(hipError_t e, const char* what);

inline int elem_bytes(int dt) { return dt == PKV_F32 ? 4 : dt == PKV_BF16 ? 2 : 1; }

// Context-split plan shared by the workspace query and the decode call.  A work
// item is (sequence, context split, KV head); a split covers `split_tokens`
// consecutive logical tokens (a multiple of 256).  The split length aims at
// kTargetItems items for the batch's upper-bound token count, between
// kMinSplit and kMaxSplit tokens so that no item runs much longer than the rest.
struct SplitPlan {
  int split_tokens;
  int max_splits;  // splits of the longest admissible sequence
};

constexpr int kTargetItems = 2048;
constexpr int kMinSplit = 256;
constexpr int kMaxSplit = 2048;

inline SplitPlan plan_splits(int B, int H_kv, int max_ctx) {
  long long total = (long long)B * H_kv * (max_ctx > 0 ? max_ctx : 1);
  long long s = (total + kTargetItems - 1) / kTargetItems;
  s = (s + 255) / 256 * 256;
  if (s < kMinSplit) s = kMinSplit;
  if (s > kMaxSplit) s = kMaxSplit;
  SplitPlan p;
  p.split_tokens = (int)s;
  p.max_splits = max_ctx > 0 ? (int)((max_ctx + s - 1) / s) : 1;
  return p;
}

// The matrix-core path plans one round of 4-wave workgroups (at most this many
// per CU) and launches up to that many plus B * H_kv pieces, each owning one
// partial slot of 16 heads.
constexpr int kMaxGroupsPerCU = 4;

// Workspace layout, large enough for either path:
//   [matrix path: one 64-bit arrival counter per (sequence, KV head) segment][pad to 256]
//   [partial outputs fp32: max(vector path B*H_q*max_splits*D,
//                              matrix path (CUs*4 + B*H_kv) pieces*16 heads*D)][pad to 256]
//   [partial (max, sum) fp32: the same count of rows * 2]
// A counter word is 0 between calls, or holds (call token << 32 | pieces arrived) while its
// segment's pieces finish; a word whose upper half is not the call's token counts as empty, so
// the workspace needs no initialisation.
struct WorkspaceLayout {
  size_t ctr, o, ml, total;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// paths: 1 = vector path only, 2 = matrix-core path only, 3 = either (what a caller's workspace covers)
inline WorkspaceLayout workspace_layout(int B, int H_q, int H_kv, int D, const SplitPlan& p, int num_cus,
                                        int paths = 3) {
  const size_t vec_rows = (paths & 1) && p.max_splits > 1 ? (size_t)B * H_q * p.max_splits : 0;
  const size_t mfma_rows = (paths & 2) ? ((size_t)num_cus * kMaxGroupsPerCU + (size_t)B * H_kv) * 16 : 0;
  const size_t rows = vec_rows > mfma_rows ? vec_rows : mfma_rows;
  WorkspaceLayout w;
  w.ctr = 0;
  w.o = (paths & 2) ? align256((size_t)B * H_kv * sizeof(unsigned long long)) : 0;
  w.ml = w.o + align256(rows * D * sizeof(float));
  w.total = w.ml + rows * 2 * sizeof(float);
  return w;
}

inline size_t workspace_bytes_for(int B, int H_q, int H_kv, int D, const SplitPlan& p, int num_cus,
                                  int paths = 3) {
  return workspace_layout(B, H_q, H_kv, D, p, num_cus, paths).total;
}

struct DecodeArgs {
  float* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* new_k;            // fused step: the step's K rows [B][H_kv][D] bf16 (null: plain decode)
  const void* new_v;            // fused step: the step's V rows [B][H_kv][D] bf16
  const int64_t* new_slots;     // fused step: slot of sequence b's new token ([B]; < 0: none)
  const int32_t* sink_lens;      // optional [B]: attend t < sink_lens[b] ...
  const int32_t* window_starts;  // optional [B]: ... or t >= window_starts[b] (both null: every t < n)
  const float* k_scale;
  const float* v_scale;
  float* ws_o;   // [B][H_q][max_splits][D] split partial outputs (unnormalised)
  float* ws_ml;  // [B][H_q][max_splits][2]  split running max (log2 units) and sum
  unsigned long long* ws_ctr;  // matrix path: arrival counter per segment (see WorkspaceLayout)
  unsigned int call_token;     // nonzero, different on consecutive calls of the process
  int B, H_q, H_kv, G, D, NB, bs;
  int max_blocks;    // table row stride
  int len_cap;       // min(max_context_len, max_blocks * bs)
  int split_tokens;
  int max_splits;
  float scale_log2;  // scale * log2(e)
  int q_dtype, kv_dtype;
  int num_cus;       // compute units of the device (sizes the matrix-core launch)
  long long sum_len_hint;  // caller's sum of context_lens (< 0: unknown); picks single-piece mode
  int single_piece;        // set by the launcher: one piece per segment, no partials
  int speculate;           // set by the launcher: the length sum says every length is len_cap, so a
                           // workgroup may load its likely segment's first chunk before its plan
};

// Scratch of pkv_paged_attn_decode_noalloc: a file-scope device array in paged_decode.hip, one copy
// per device, holding the decode's partials for callers that cannot allocate.  static_scratch looks
// up its address on the current device (once per device) and returns it with its size.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr);

// Kernel launchers (matrix-core path: paged_decode.hip; vector path and its split merge:
// decode_vector.hip).  Return hipError_t of the launch.
bool decode_fast_path_supported(int q_dtype, int kv_dtype, int G, int D, int bs);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_vector(const DecodeArgs& a, hipStream_t s);
hipError_t launch_split_merge(const DecodeArgs& a, hipStream_t s);

// kv_append.hip
struct AppendArgs {
  const void* k;
  const void* v;
  const int64_t* slots;
  void* k_pool;
  void* v_pool;
  const float* k_scale;
  const float* v_scale;
  int T, H_kv, D, bs;
  long long n_slots;  // NB * bs
  int src_dtype, pool_dtype;
};
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);

// paged prefill (causal chunked multi-query attention)
struct PrefillArgs {
  float* out;                  // [T][H_q][D]
  const void* q;               // [T][H_q][D] bf16
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* context_lens;  // [B]
  const int32_t* query_start;   // [B + 1]
  const float* k_scale;
  const float* v_scale;
  int B, T, H_q, H_kv, G, D, NB, bs, max_blocks, len_cap;
  float scale_log2;
  int kv_dtype;
  int items;           // B * H_kv * groups_per_seq work items
  int groups_per_seq;  // tile groups that cover the longest chunk
  int nw;              // waves per workgroup: 12, or 8 where 12 would leave CUs without work
};
int prefill_wg_tokens(int G, int nw);  // query tokens one workgroup of nw waves covers
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

// whole-block moves of both pools: pool -> pool (copy-on-write pairs),
// pool -> staging records (swap-out gather), staging -> pool (swap-in scatter)
enum BlockMove { kMovePairs = 0, kMoveGather = 1, kMoveScatter = 2 };
struct CopyBlocksArgs {
  void* k_pool;
  void* v_pool;
  const int32_t* src;  // device [n_pairs]: source blocks (pairs, gather)
  const int32_t* dst;  // device [n_pairs]: target blocks (pairs, scatter)
  void* staging;       // gather / scatter: [n_pairs][2 (K, V)][block bytes], device or mapped host memory
  int32_t n_pairs;
  int32_t NB;
  long long block_units;  // 16-byte units per block of one pool (H_kv * D * bs * elem / 16)
  long long tiles;        // copy tiles per block of one pool
};
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
hipError_t launch_block_move(const CopyBlocksArgs& a, BlockMove mode, hipStream_t s);

// stream.hip
size_t stream_read_blocks(size_t bytes);
hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

}  // namespace pkv
