// C ABI entry points: argument validation, launch planning, error reporting.
// Every check happens on the host before any launch; see pkv.h for contracts.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <random>

#include "internal.h"

namespace pkv {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  set_error("%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return PKV_ERR_HIP;
}

static bool valid_dtype(int dt) { return dt == PKV_F32 || dt == PKV_BF16 || dt == PKV_FP8_E4M3; }

// compute units of the current device (256 on MI355X when no device is visible,
// e.g. when only sizes are queried on a host without a GPU)
static int current_num_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return cus;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_err; }

int pkv_abi_version(void) { return 2; }

int pkv_kv_append(const void* k, const void* v, int src_dtype, const int64_t* slot_mapping, int32_t T,
                  void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs, int32_t H_kv, int32_t D,
                  const float* k_scale, const float* v_scale, void* stream) {
  g_err[0] = 0;
  if (T < 0 || NB <= 0 || bs <= 0 || bs > 256 || H_kv <= 0 || D <= 0) {
    set_error("kv_append: bad sizes T=%d NB=%d bs=%d H_kv=%d D=%d", T, NB, bs, H_kv, D);
    return PKV_ERR_INVALID_ARG;
  }
  if (D % 16 != 0 || D > 512) {
    set_error("kv_append: D=%d must be a multiple of 16 and <= 512", D);
    return PKV_ERR_UNSUPPORTED;
  }
  if (!valid_dtype(src_dtype) || !valid_dtype(pool_dtype)) {
    set_error("kv_append: unknown dtype (src %d, pool %d)", src_dtype, pool_dtype);
    return PKV_ERR_INVALID_ARG;
  }
  const bool ok_pair = (src_dtype == pool_dtype) || (src_dtype == PKV_BF16 && pool_dtype == PKV_FP8_E4M3);
  if (!ok_pair) {
    set_error("kv_append: unsupported conversion %d -> %d", src_dtype, pool_dtype);
    return PKV_ERR_UNSUPPORTED;
  }
  if (T == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) {
    set_error("kv_append: null pointer");
    return PKV_ERR_INVALID_ARG;
  }
  if (src_dtype == PKV_BF16 && pool_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) {
    set_error("kv_append: quantising to E4M3 needs k_scale and v_scale");
    return PKV_ERR_INVALID_ARG;
  }
  if ((long long)T * H_kv * (D / 8) > (long long)0x7FFFFFFF * 256) {
    set_error("kv_append: T too large for one launch");
    return PKV_ERR_INVALID_ARG;
  }
  AppendArgs a{k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale, T, H_kv, D, bs, (long long)NB * bs,
               src_dtype, pool_dtype};
  return hip_status(launch_kv_append(a, (hipStream_t)stream), "kv_append launch");
}

// shared validation of the block moves; fills `a` (without the index arrays)
static int block_move_args(const char* what, void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs,
                           int32_t H_kv, int32_t D, int32_t n, CopyBlocksArgs& a) {
  if (n < 0 || NB <= 0 || bs <= 0 || bs > 256 || H_kv <= 0 || D <= 0) {
    set_error("%s: bad sizes n=%d NB=%d bs=%d H_kv=%d D=%d", what, n, NB, bs, H_kv, D);
    return PKV_ERR_INVALID_ARG;
  }
  if (!valid_dtype(pool_dtype)) {
    set_error("%s: unknown dtype %d", what, pool_dtype);
    return PKV_ERR_INVALID_ARG;
  }
  if (D % 16 != 0 || D > 512) {
    set_error("%s: D=%d must be a multiple of 16 and <= 512", what, D);
    return PKV_ERR_UNSUPPORTED;
  }
  if (n > 0 && (!k_pool || !v_pool)) {
    set_error("%s: null pool", what);
    return PKV_ERR_INVALID_ARG;
  }
  const int elem = pool_dtype == PKV_F32 ? 4 : pool_dtype == PKV_BF16 ? 2 : 1;
  a = CopyBlocksArgs{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.n_pairs = n;
  a.NB = NB;
  a.block_units = (long long)H_kv * D * bs * elem / 16;
  a.tiles = (a.block_units + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll);
  if ((long long)n * 2 * a.tiles > 0x7FFFFFFFLL) {
    set_error("%s: too many blocks for one launch", what);
    return PKV_ERR_INVALID_ARG;
  }
  return PKV_OK;
}

int pkv_copy_blocks(void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs, int32_t H_kv, int32_t D,
                    const int32_t* src, const int32_t* dst, int32_t n_pairs, void* stream) {
  g_err[0] = 0;
  CopyBlocksArgs a;
  const int st = block_move_args("copy_blocks", k_pool, v_pool, pool_dtype, NB, bs, H_kv, D, n_pairs, a);
  if (st != PKV_OK || n_pairs == 0) return st;
  if (!src || !dst) {
    set_error("copy_blocks: null pointer");
    return PKV_ERR_INVALID_ARG;
  }
  a.src = src;
  a.dst = dst;
  return hip_status(launch_block_move(a, kMovePairs, (hipStream_t)stream), "copy_blocks launch");
}

// Device address of a staging buffer: device memory as is, pinned host memory through its
// mapping.  Pageable (unregistered) host memory is refused: a kernel must never touch it.
static int staging_device_ptr(const char* what, const void* p, void** dev_ptr) {
  hipPointerAttribute_t attr{};
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess || attr.type == hipMemoryTypeUnregistered) {
    (void)hipGetLastError();
    set_error("%s: staging %p is neither device memory nor pinned host memory", what, p);
    return PKV_ERR_INVALID_ARG;
  }
  if (attr.type == hipMemoryTypeHost) {
    if (!attr.devicePointer) {
      set_error("%s: pinned staging %p has no device mapping", what, p);
      return PKV_ERR_INVALID_ARG;
    }
    *dev_ptr = (char*)attr.devicePointer + ((const char*)p - (const char*)attr.hostPointer);
  } else {
    *dev_ptr = (void*)p;
  }
  return PKV_OK;
}

size_t pkv_block_record_bytes(int pool_dtype, int32_t bs, int32_t H_kv, int32_t D) {
  g_err[0] = 0;
  if (!valid_dtype(pool_dtype) || bs <= 0 || H_kv <= 0 || D <= 0) {
    set_error("block_record_bytes: bad arguments");
    return 0;
  }
  const size_t elem = pool_dtype == PKV_F32 ? 4 : pool_dtype == PKV_BF16 ? 2 : 1;
  return 2 * (size_t)H_kv * D * bs * elem;
}

int pkv_gather_blocks(const void* k_pool, const void* v_pool, int pool_dtype, int32_t NB, int32_t bs, int32_t H_kv,
                      int32_t D, const int32_t* blocks, int32_t n, void* staging, void* stream) {
  g_err[0] = 0;
  CopyBlocksArgs a;
  const int st = block_move_args("gather_blocks", (void*)k_pool, (void*)v_pool, pool_dtype, NB, bs, H_kv, D, n, a);
  if (st != PKV_OK || n == 0) return st;
  if (!blocks || !staging || ((uintptr_t)staging & 15u)) {
    set_error("gather_blocks: null pointer or staging not 16-byte aligned");
    return PKV_ERR_INVALID_ARG;
  }
  a.src = blocks;
  const int ps = staging_device_ptr("gather_blocks", staging, &a.staging);
  if (ps != PKV_OK) return ps;
  return hip_status(launch_block_move(a, kMoveGather, (hipStream_t)stream), "gather_blocks launch");
}

int pkv_scatter_blocks(void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs, int32_t H_kv, int32_t D,
                       const int32_t* blocks, int32_t n, const void* staging, void* stream) {
  g_err[0] = 0;
  CopyBlocksArgs a;
  const int st = block_move_args("scatter_blocks", k_pool, v_pool, pool_dtype, NB, bs, H_kv, D, n, a);
  if (st != PKV_OK || n == 0) return st;
  if (!blocks || !staging || ((uintptr_t)staging & 15u)) {
    set_error("scatter_blocks: null pointer or staging not 16-byte aligned");
    return PKV_ERR_INVALID_ARG;
  }
  a.dst = blocks;
  const int ps = staging_device_ptr("scatter_blocks", staging, &a.staging);
  if (ps != PKV_OK) return ps;
  return hip_status(launch_block_move(a, kMoveScatter, (hipStream_t)stream), "scatter_blocks launch");
}

size_t pkv_decode_workspace_bytes_gqa(int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t max_context_len,
                                      int32_t bs) {
  g_err[0] = 0;
  if (B < 0 || H_q <= 0 || H_kv <= 0 || D <= 0 || max_context_len < 0 || bs <= 0) {
    set_error("decode_workspace_bytes: bad sizes");
    return 0;
  }
  return workspace_bytes_for(B, H_q, H_kv, D, plan_splits(B, H_kv, max_context_len), current_num_cus());
}

// Without H_kv: the largest size over every KV head count that divides H_q, so the result
// serves a decode call with any of them.
size_t pkv_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t D, int32_t max_context_len, int32_t bs) {
  g_err[0] = 0;
  if (B < 0 || H_q <= 0 || D <= 0 || max_context_len < 0 || bs <= 0) {
    set_error("decode_workspace_bytes: bad sizes");
    return 0;
  }
  const int cus = current_num_cus();
  size_t best = 0;
  for (int32_t h = 1; h <= H_q; ++h) {
    if (H_q % h) continue;
    const size_t n = workspace_bytes_for(B, H_q, h, D, plan_splits(B, h, max_context_len), cus);
    best = n > best ? n : best;
  }
  return best;
}

static std::atomic<int> g_decode_path{PKV_DECODE_PATH_AUTO};

int pkv_set_decode_path(int path) {
  g_err[0] = 0;
  if (path != PKV_DECODE_PATH_AUTO && path != PKV_DECODE_PATH_VECTOR) {
    set_error("set_decode_path: unknown path %d", path);
    return PKV_ERR_INVALID_ARG;
  }
  return g_decode_path.exchange(path);
}

static std::atomic<int> g_prefill_waves{0};  // 0: automatic; 8 or 12: forced

int pkv_set_prefill_waves(int nw) {
  g_err[0] = 0;
  if (nw != 0 && nw != 8 && nw != 12) {
    set_error("set_prefill_waves: unknown workgroup size %d (0, 8 or 12)", nw);
    return PKV_ERR_INVALID_ARG;
  }
  return g_prefill_waves.exchange(nw);
}

// the matrix-core path runs where it is supported unless the vector path is forced
static bool use_matrix_path(int q_dtype, int kv_dtype, int G, int D, int bs) {
  return g_decode_path.load() == PKV_DECODE_PATH_AUTO && decode_fast_path_supported(q_dtype, kv_dtype, G, D, bs);
}

static int decode_impl(float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t max_context_len, const int32_t* sink_lens, const int32_t* window_starts, int32_t B,
                       int32_t H_q, int32_t H_kv, int32_t D, int32_t NB, int32_t bs, float scale,
                       const float* k_scale, const float* v_scale, void* workspace, size_t workspace_bytes,
                       void* stream, const void* new_k = nullptr, const void* new_v = nullptr,
                       const int64_t* new_slots = nullptr, int64_t sum_len_hint = -1, bool check_only = false,
                       bool static_ws = false) {
  if (B < 0 || H_q <= 0 || H_kv <= 0 || NB <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0) {
    set_error("decode: bad sizes B=%d H_q=%d H_kv=%d NB=%d max_blocks=%d max_context_len=%d", B, H_q, H_kv, NB,
              max_blocks_per_seq, max_context_len);
    return PKV_ERR_INVALID_ARG;
  }
  if (H_q % H_kv != 0) {
    set_error("decode: H_q=%d is not a multiple of H_kv=%d", H_q, H_kv);
    return PKV_ERR_INVALID_ARG;
  }
  if (!(D == 64 || D == 128 || D == 256) || !(bs == 8 || bs == 16 || bs == 32)) {
    set_error("decode: unsupported D=%d / bs=%d (D in {64,128,256}, bs in {8,16,32})", D, bs);
    return PKV_ERR_UNSUPPORTED;
  }
  if (!(q_dtype == PKV_F32 || q_dtype == PKV_BF16) || !valid_dtype(kv_dtype)) {
    set_error("decode: unsupported dtypes q=%d kv=%d", q_dtype, kv_dtype);
    return PKV_ERR_UNSUPPORTED;
  }
  if (!std::isfinite(scale)) {
    set_error("decode: scale is not finite");
    return PKV_ERR_INVALID_ARG;
  }
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) {
    set_error("decode: null pointer");
    return PKV_ERR_INVALID_ARG;
  }
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) {
    set_error("decode: E4M3 KV needs k_scale and v_scale");
    return PKV_ERR_INVALID_ARG;
  }
  const SplitPlan plan = plan_splits(B, H_kv, max_context_len);
  const int num_cus = current_num_cus();
  const int G = H_q / H_kv;
  const bool fast = use_matrix_path(q_dtype, kv_dtype, G, D, bs);
  // a caller's workspace is sized for either path; the static scratch only for the path that runs
  const int paths = static_ws ? (fast ? 2 : 1) : 3;
  const size_t need = workspace_bytes_for(B, H_q, H_kv, D, plan, num_cus, paths);
  if (static_ws) {  // the library's own scratch (pkv_paged_attn_decode_noalloc)
    if (need > kStaticScratchBytes) {
      set_error("decode_noalloc: these sizes need %zu bytes of scratch, more than the %zu of the library's static "
                "scratch; call pkv_paged_attn_decode with a workspace", need, kStaticScratchBytes);
      return PKV_ERR_INVALID_ARG;
    }
  } else if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))) {
    set_error("decode: workspace needs %zu bytes, 256-byte aligned (got %zu at %p)", need, workspace_bytes,
              workspace);
    return PKV_ERR_INVALID_ARG;
  }
  const long long items = fast ? (long long)num_cus * kMaxGroupsPerCU + (long long)B * H_kv
                               : (long long)B * plan.max_splits * H_q;
  if (items > 0x7FFFFFFFLL) {
    set_error("decode: launch too large (%lld work items)", items);
    return PKV_ERR_INVALID_ARG;
  }
  if (check_only) return PKV_OK;
  if (static_ws) {
    const int st = hip_status(static_scratch(&workspace), "decode_noalloc: static scratch lookup");
    if (st != PKV_OK) return st;
    workspace_bytes = kStaticScratchBytes;
  }
  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.sink_lens = sink_lens;
  a.window_starts = window_starts;
  a.new_k = new_k;
  a.new_v = new_v;
  a.new_slots = new_slots;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  if (need > 0) {
    const WorkspaceLayout wl = workspace_layout(B, H_q, H_kv, D, plan, num_cus, paths);
    a.ws_o = (float*)((char*)workspace + wl.o);
    a.ws_ml = (float*)((char*)workspace + wl.ml);
    a.ws_ctr = (unsigned long long*)((char*)workspace + wl.ctr);
    // a different odd token per call; the count starts at a per-process random value, so that a
    // word another process left in reused memory is not taken for this process's first calls
    static std::atomic<unsigned int> calls{(unsigned int)std::random_device{}()};
    a.call_token = (calls.fetch_add(1) << 1) | 1u;
  }
  a.B = B;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.G = G;
  a.D = D;
  a.NB = NB;
  a.bs = bs;
  a.max_blocks = max_blocks_per_seq;
  const long long cap = (long long)max_blocks_per_seq * bs;
  a.len_cap = (int)(cap < max_context_len ? cap : max_context_len);
  a.split_tokens = plan.split_tokens;
  a.max_splits = plan.max_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.num_cus = num_cus;
  // A length sum above B * len_cap is impossible (every length is cut to len_cap): the hint is then
  // taken as unknown rather than as a reason to keep every segment whole.
  a.sum_len_hint = sum_len_hint > (long long)B * a.len_cap ? -1 : sum_len_hint;
  hipStream_t s = (hipStream_t)stream;
  if (fast) return hip_status(launch_decode_mfma(a, s), "decode launch");
  const int st = hip_status(launch_decode_vector(a, s), "decode launch");
  if (st != PKV_OK || plan.max_splits <= 1) return st;
  return hip_status(launch_split_merge(a, s), "split merge launch");
}

int pkv_paged_attn_decode(float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                          int kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H_q, int32_t H_kv,
                          int32_t D, int32_t NB, int32_t bs, float scale, const float* k_scale,
                          const float* v_scale, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, nullptr, nullptr, B, H_q, H_kv, D, NB, bs, scale, k_scale, v_scale, workspace,
                     workspace_bytes, stream);
}

int pkv_paged_attn_decode_noalloc(float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                                  int kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H_q,
                                  int32_t H_kv, int32_t D, int32_t NB, int32_t bs, float scale,
                                  const float* k_scale, const float* v_scale, void* stream) {
  g_err[0] = 0;
  return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, nullptr, nullptr, B, H_q, H_kv, D, NB, bs, scale, k_scale, v_scale, nullptr, 0,
                     stream, nullptr, nullptr, nullptr, -1, false, true);
}

int pkv_paged_attn_decode_hinted(float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                                 int kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len, int64_t sum_context_lens,
                                 int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t NB, int32_t bs, float scale,
                                 const float* k_scale, const float* v_scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  g_err[0] = 0;
  return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, nullptr, nullptr, B, H_q, H_kv, D, NB, bs, scale, k_scale, v_scale, workspace,
                     workspace_bytes, stream, nullptr, nullptr, nullptr, sum_context_lens);
}

int pkv_paged_attn_decode_window(float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                                 int kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len, const int32_t* sink_lens,
                                 const int32_t* window_starts, int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                 int32_t NB, int32_t bs, float scale, const float* k_scale, const float* v_scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, sink_lens, window_starts, B, H_q, H_kv, D, NB, bs, scale, k_scale, v_scale,
                     workspace, workspace_bytes, stream);
}

int pkv_paged_prefill(float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      const int32_t* query_start, int32_t max_query_len, int32_t B, int32_t T, int32_t H_q,
                      int32_t H_kv, int32_t D, int32_t NB, int32_t bs, float scale, const float* k_scale,
                      const float* v_scale, void* stream) {
  g_err[0] = 0;
  if (B < 0 || T < 0 || H_q <= 0 || H_kv <= 0 || NB <= 0 || max_blocks_per_seq <= 0 || max_query_len < 0) {
    set_error("prefill: bad sizes B=%d T=%d H_q=%d H_kv=%d NB=%d max_blocks=%d max_query_len=%d", B, T, H_q, H_kv,
              NB, max_blocks_per_seq, max_query_len);
    return PKV_ERR_INVALID_ARG;
  }
  if (H_q % H_kv != 0) {
    set_error("prefill: H_q=%d is not a multiple of H_kv=%d", H_q, H_kv);
    return PKV_ERR_INVALID_ARG;
  }
  const int G = H_q / H_kv;
  if (!(D == 64 || D == 128) || !(bs == 8 || bs == 16 || bs == 32) || 16 % G != 0 || q_dtype != PKV_BF16 ||
      !(kv_dtype == PKV_BF16 || kv_dtype == PKV_FP8_E4M3)) {
    set_error("prefill: unsupported D=%d bs=%d G=%d q=%d kv=%d (D 64/128, bs 8/16/32, G in {1,2,4,8,16}, bf16 q, "
              "bf16/E4M3 KV)", D, bs, G, q_dtype, kv_dtype);
    return PKV_ERR_UNSUPPORTED;
  }
  if (!std::isfinite(scale)) {
    set_error("prefill: scale is not finite");
    return PKV_ERR_INVALID_ARG;
  }
  if (B == 0 || T == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start) {
    set_error("prefill: null pointer");
    return PKV_ERR_INVALID_ARG;
  }
  if (kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) {
    set_error("prefill: E4M3 KV needs k_scale and v_scale");
    return PKV_ERR_INVALID_ARG;
  }
  // 12-wave workgroups (48 query tokens at G = 8) share each staged K/V chunk among the most
  // columns; where they would leave compute units without a work item (small batches or small
  // GQA groups: 384 tokens per workgroup at G = 1), 8-wave ones cut the queries finer.  (At 1.4
  // items per CU, G = 2 on 4 x 2048 queries, the 12-wave ones were still 2.5 % faster.)
  const int forced = g_prefill_waves.load();
  int nw = forced ? forced : 12;
  long long groups = ((long long)max_query_len + prefill_wg_tokens(G, nw) - 1) / prefill_wg_tokens(G, nw);
  if (!forced && (long long)B * H_kv * groups < (long long)current_num_cus()) {
    nw = 8;
    groups = ((long long)max_query_len + prefill_wg_tokens(G, nw) - 1) / prefill_wg_tokens(G, nw);
  }
  const long long items = (long long)B * H_kv * groups;
  if (items > 0x7FFFFFF0LL) {
    set_error("prefill: launch too large (%lld work items)", items);
    return PKV_ERR_INVALID_ARG;
  }
  PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.B = B;
  a.T = T;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.G = G;
  a.D = D;
  a.NB = NB;
  a.bs = bs;
  a.max_blocks = max_blocks_per_seq;
  const long long cap = (long long)max_blocks_per_seq * bs;
  a.len_cap = (int)(cap < 0x7FFFFFFF ? cap : 0x7FFFFFFF);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.kv_dtype = kv_dtype;
  a.items = (int)items;
  a.groups_per_seq = (int)groups;
  a.nw = nw;
  return hip_status(launch_prefill(a, (hipStream_t)stream), "prefill launch");
}

int pkv_decode_step(float* out, const void* q, int q_dtype, const void* k_new, const void* v_new, int src_dtype,
                    const int64_t* new_slots, void* k_pool, void* v_pool, int kv_dtype, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                    int64_t sum_context_lens, int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t NB,
                    int32_t bs, float scale, const float* k_scale, const float* v_scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const bool fused = B > 0 && H_kv > 0 && H_q % H_kv == 0 && (kv_dtype == PKV_BF16 || kv_dtype == PKV_FP8_E4M3) &&
                     src_dtype == PKV_BF16 && use_matrix_path(q_dtype, kv_dtype, H_q / H_kv, D, bs);
  if (!fused) {  // the two calls, in order, on the stream; the decode's arguments are checked first
    int st = decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq, context_lens,
                         max_context_len, nullptr, nullptr, B, H_q, H_kv, D, NB, bs, scale, k_scale, v_scale,
                         workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, sum_context_lens, true);
    if (st != PKV_OK) return st;
    st = pkv_kv_append(k_new, v_new, src_dtype, new_slots, B, k_pool, v_pool, kv_dtype, NB, bs, H_kv, D, k_scale,
                       v_scale, stream);
    if (st != PKV_OK) return st;
    return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, nullptr, nullptr, B, H_q, H_kv, D, NB, bs, scale, k_scale, v_scale,
                       workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, sum_context_lens);
  }
  if (!k_new || !v_new || !new_slots) {
    set_error("decode_step: null new-token pointer");
    return PKV_ERR_INVALID_ARG;
  }
  if (NB <= 0 || bs <= 0 || (long long)NB * bs > 0x7FFFFFFFFFFFLL) {
    set_error("decode_step: bad pool size NB=%d bs=%d", NB, bs);
    return PKV_ERR_INVALID_ARG;
  }
  return decode_impl(out, q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, nullptr, nullptr, B, H_q, H_kv, D, NB, bs, scale, k_scale, v_scale, workspace,
                     workspace_bytes, stream, k_new, v_new, new_slots, sum_context_lens);
}

size_t pkv_stream_read_sink_floats(size_t bytes) { return stream_read_blocks(bytes); }

int pkv_stream_read(const void* src, size_t bytes, float* sink, void* stream) {
  g_err[0] = 0;
  if (!src || !sink || bytes % 16 != 0) {
    set_error("stream_read: null pointer or size not a multiple of 16");
    return PKV_ERR_INVALID_ARG;
  }
  if (bytes == 0) return PKV_OK;
  return hip_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream), "stream_read launch");
}

int pkv_copy(void* dst, const void* src, size_t bytes, void* stream) {
  g_err[0] = 0;
  if (!src || !dst || bytes % 16 != 0) {
    set_error("copy: null pointer or size not a multiple of 16");
    return PKV_ERR_INVALID_ARG;
  }
  if (bytes == 0) return PKV_OK;
  return hip_status(launch_copy(dst, src, bytes, (hipStream_t)stream), "copy launch");
}

}  // extern "C"
