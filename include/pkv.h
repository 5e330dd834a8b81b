/*
 * pkv.h — C ABI of the paged-KV decode-attention library for AMD MI355X (gfx950).
 *
 * The method ("KV Cache Fragmentation" field guide, defragging.ai, section
 * "Definition"; "Paged Attention and KV Cache Fragmentation",
 * inferenceengineering.co, section "How PagedAttention maps an OS concept onto
 * GPU memory"): the KV cache lives in one pool of fixed-size physical blocks;
 * each sequence owns a block table mapping its logical block j to a physical
 * block; blocks are taken only as a sequence grows, returned when it finishes,
 * and may be shared by several sequences (a common prefix, a fork).  The
 * attention kernel walks the table.
 *
 * Groups of calls:
 *   pkv_kv_append          scatter this step's K/V rows into their slots
 *   pkv_copy_blocks        copy whole blocks (copy-on-write of shared blocks)
 *   pkv_gather_blocks / pkv_scatter_blocks  pack blocks into / unpack from a
 *                          contiguous staging buffer (swap-out / swap-in)
 *   pkv_paged_attn_decode  one query token per sequence attends over its paged KV
 *   pkv_paged_attn_decode_hinted  the same, given the host's sum of the context
 *                          lengths (skips the partial results when nothing is cut)
 *   pkv_paged_attn_decode_window  the same, attending only sink tokens and a
 *                          recent window (StreamingLLM; with pkv_seq_streaming_evict)
 *   pkv_paged_prefill      causal attention of a chunk of new tokens per sequence
 *                          (prompt or chunked prefill) over the same pools
 *   pkv_decode_step        kv_append of one new token per sequence, then the
 *                          decode, fused into the decode launch where it can be
 *   pkv_alloc_* / pkv_seq_* host-side fixed-block free-list allocator
 *
 * ---------------------------------------------------------------------------
 * Conventions
 *   - Every call returns an int status (PKV_OK or a negative PKV_ERR_*);
 *     pkv_last_error() returns a thread-local message for the last failure.
 *   - Device pointers are owned by the caller (e.g. torch tensors), must be
 *     contiguous in the layouts below and live on the current HIP device.
 *     The library never allocates device memory: scratch for the decode's
 *     split-context partials is passed in as `workspace`.
 *   - Device calls are asynchronous on the caller's stream (`stream` is a
 *     hipStream_t passed as void*; NULL = the null stream) and never
 *     synchronize.  Scalar arguments are validated on the host before any
 *     launch; an invalid call launches nothing.  Device-resident contents
 *     (slots, block ids, lengths) are not validated for meaning, but the
 *     kernels never read or write outside the buffers described here:
 *     an out-of-range slot is skipped, an out-of-range block id is read as
 *     block 0, a length beyond the table or beyond max_context_len is cut to
 *     it.  Such inputs are caller errors with unspecified results.
 *   - The allocator object is host memory only and is not thread-safe.
 *
 * Element types (PKV_*): fp32, bf16, and OCP FP8 E4M3FN (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, max 448).
 * An E4M3 pool carries one fp32 scale per KV head for K and one for V
 * (real value = code value * scale), device arrays of H_kv floats.
 *
 * Pool layout.  NB physical blocks of bs tokens; inside a block every KV
 * head owns a contiguous tile (D = head dim, X = 16 bytes / element size):
 *     K pool  [NB][H_kv][D/X][bs][X]
 *     V pool  [NB][H_kv][D][bs]
 * Token position p of a sequence with table row T lives at slot
 * s = T[p / bs] * bs + p % bs (block s / bs, offset s % bs).
 * GQA: query head h reads KV head h / (H_q / H_kv).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,   /* bad pointer, size, shape or id */
  PKV_ERR_UNSUPPORTED = -2,   /* valid but not implemented (dtype / bs / D / G combination) */
  PKV_ERR_OUT_OF_BLOCKS = -3, /* the pool cannot hold the request; allocator state unchanged */
  PKV_ERR_UNKNOWN_SEQ = -4,   /* sequence id not present */
  PKV_ERR_SHARED_BLOCK = -5,  /* growth would write into a shared, partly filled block */
  PKV_ERR_HIP = -6            /* the HIP runtime reported an error (message has details) */
};

enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 };

/*
 * Design (not on the pages): error text and versioning of this library.
 * pkv_last_error: thread-local text of the last error set by a call on this
 * thread ("" if none).  pkv_abi_version: bumped on incompatible changes (2:
 * pkv_decode_workspace_bytes takes no H_kv).
 */
const char* pkv_last_error(void);
int pkv_abi_version(void);

/*
 * pkv_kv_append — write T tokens' K and V rows into their slots.
 * ("Paged Attention and KV Cache Fragmentation", section "How PagedAttention
 * maps an OS concept onto GPU memory": a sequence's new tokens go into the
 * blocks its table maps them to.)
 *
 *   k, v           device, [T][H_kv][D] of src_dtype, row-major
 *   slot_mapping   device int64 [T]; slot < 0 = padding, skipped;
 *                  slot >= NB*bs is skipped (caller error); duplicate slots
 *                  within one call are a caller error (unspecified winner)
 *   k_pool, v_pool device, layouts above, pool_dtype
 *   k_scale, v_scale device fp32 [H_kv], required iff pool_dtype = E4M3
 *   Supported (src -> pool): F32->F32, BF16->BF16, E4M3->E4M3 (copy),
 *   BF16->E4M3 (quantise: y = fp32(x) / scale[h] with IEEE fp32 division,
 *   then round to nearest even E4M3; |y| >= 448 and +-inf saturate to +-448,
 *   NaN becomes 0x7F with the input's sign).
 *   D must be a multiple of 16 and <= 512; bs in 1..256.
 */
int pkv_kv_append(const void* k, const void* v, int src_dtype, const int64_t* slot_mapping,
                  int32_t T, void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs,
                  int32_t H_kv, int32_t D, const float* k_scale, const float* v_scale,
                  void* stream);

/*
 * pkv_copy_blocks — for i in 0..n_pairs-1, physical block dst[i] of both pools
 * becomes a copy of block src[i]: every head, every token slot, bit for bit.
 * ("Paged Attention and KV Cache Fragmentation", section "How PagedAttention
 * maps an OS concept onto GPU memory": sharers of a block diverge only where
 * their content differs; the copy gives a diverging sequence its own block.)
 * Use it with the pairs pkv_seq_append_slots_cow reports, before the
 * pkv_kv_append that writes the new tokens, on the same stream.
 *
 *   k_pool, v_pool device, layouts above, pool_dtype
 *   src, dst       device int32 [n_pairs]; a pair with an id outside [0, NB)
 *                  is skipped (caller error); src == dst is a no-op.  A block
 *                  that is the dst of one pair and the src or dst of another
 *                  is a caller error (the pairs run concurrently).
 *   D must be a multiple of 16 and <= 512; bs in 1..256.
 */
int pkv_copy_blocks(void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs, int32_t H_kv,
                    int32_t D, const int32_t* src, const int32_t* dst, int32_t n_pairs, void* stream);

/*
 * Swap staging ("Paged Attention and KV Cache Fragmentation", section
 * "Offloading paged KV blocks to CPU DRAM and NVMe": blocks move between HBM
 * and host memory, and the paged layout scatters them into many small
 * transfers).  A staging buffer holds n records of
 * pkv_block_record_bytes(...) bytes; record i is block blocks[i]'s K block
 * (every head) followed by its V block, raw bytes in pool layout.
 *
 * pkv_gather_blocks: record i <- block blocks[i].  pkv_scatter_blocks: block
 * blocks[i] <- record i.  `staging` is device memory (then one
 * hipMemcpyAsync moves it to or from the host) or pinned, mapped host memory
 * (hipHostMalloc; the kernel reads or writes it directly); 16-byte aligned,
 * owned by the caller.  Pageable host memory is refused (PKV_ERR_INVALID_ARG),
 * checked with hipPointerGetAttributes before the launch.  blocks: device int32 [n]; an id outside [0, NB) skips
 * its record (caller error).  Repeated ids in one scatter are a caller error.
 * Use with pkv_seq_swap_out / pkv_seq_swap_in.  D must be a multiple of 16 and
 * <= 512; bs in 1..256.  pkv_block_record_bytes returns 0 for bad arguments.
 */
size_t pkv_block_record_bytes(int pool_dtype, int32_t bs, int32_t H_kv, int32_t D);
int pkv_gather_blocks(const void* k_pool, const void* v_pool, int pool_dtype, int32_t NB, int32_t bs,
                      int32_t H_kv, int32_t D, const int32_t* blocks, int32_t n, void* staging,
                      void* stream);
int pkv_scatter_blocks(void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs, int32_t H_kv,
                       int32_t D, const int32_t* blocks, int32_t n, const void* staging, void* stream);

/*
 * Design (not on the pages): the decode's scratch.  A sequence whose context
 * is cut into several pieces keeps per-piece partial results (the unnormalised
 * output and the running max and sum of every query head) until they are
 * merged (by the segment's last piece on the matrix-core path, by a second
 * small launch on the vector path), plus one arrival counter per segment; the
 * caller owns that memory.
 *
 * pkv_decode_workspace_bytes — bytes of scratch pkv_paged_attn_decode (and the
 * hinted, window and step variants) needs for a batch of B sequences with H_q
 * query heads of dimension D, contexts of at most max_context_len tokens and
 * block size bs, whatever the KV head count H_kv (a divisor of H_q).  0 is
 * possible.  pkv_decode_workspace_bytes_gqa gives the exact, smaller figure for
 * one H_kv.  Both return 0 and set the last error for invalid sizes; the decode
 * call must receive at least the figure for its own arguments.
 */
size_t pkv_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t D, int32_t max_context_len, int32_t bs);
size_t pkv_decode_workspace_bytes_gqa(int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                      int32_t max_context_len, int32_t bs);

/*
 * pkv_paged_attn_decode — one query token per sequence attends over its paged KV.
 * For sequence b with n = context_lens[b] and query head h (KV head g):
 *     out[b][h] = sum_{t<n} softmax_t(scale * <q[b][h], K_b[g][t]>) V_b[g][t]
 * where K_b, V_b are the sequence's tokens in logical order reached through
 * block_tables[b].  ("KV Cache Fragmentation" field guide, section
 * "Definition": the cache is cut into fixed-size pages and the attention
 * kernel follows the per-request table from logical to physical pages;
 * "Paged Attention and KV Cache Fragmentation", sections "How PagedAttention
 * maps an OS concept onto GPU memory" and "The non-contiguous memory layout
 * PagedAttention introduces and its overhead": every attention step goes
 * through the block table, and paging moves where the bytes live, not what
 * attention computes.)  Each (sequence, KV head) segment runs an online
 * softmax over its tokens without writing scores to memory; when a segment is
 * cut into several pieces their partial results are merged before the call's
 * work ends (in the same launch on the matrix-core path).
 * n = 0 gives a zero row.  context_lens counts the token appended this step.
 *
 *   out            device fp32 [B][H_q][D]
 *   q              device [B][H_q][D], q_dtype F32 or BF16
 *   k_pool, v_pool device, kv_dtype, layouts above
 *   block_tables   device int32 [B][max_blocks_per_seq]; entries past
 *                  ceil(n/bs) are ignored (may be -1)
 *   context_lens   device int32 [B]
 *   max_context_len host hint >= max(context_lens) (sizes the launch without
 *                  a device->host read); lengths above it are cut to it
 *   scale          softmax scale (e.g. 1/sqrt(D)), applied to q.k in fp32
 *   k_scale, v_scale device fp32 [H_kv], required iff kv_dtype = E4M3
 *   workspace      device scratch of >= pkv_decode_workspace_bytes(...) bytes,
 *                  256-byte aligned (may be NULL when that size is 0); its
 *                  contents need no initialisation and are overwritten.
 *                  (A segment's arrival counter carries a 32-bit token of
 *                  the call that set it and is cleared by the call's last
 *                  piece; arbitrary bytes match a call's token with a
 *                  chance of 2^-32 per counter, zero-filled memory never.)
 *                  Calls that share a workspace must be ordered (one stream,
 *                  or synchronised); concurrent calls on one workspace race.
 *   Requires H_q % H_kv == 0, D in {64, 128, 256}, bs in {8, 16, 32}.
 *   bf16 q with bf16/E4M3 KV, H_q/H_kv <= 16 and D in {64, 128} take the
 *   matrix-core path; other supported combinations (fp32 q or KV, larger
 *   groups, and D = 256, a head size beyond the layers the pages discuss)
 *   take a vector path.  All accumulation is fp32.
 */
int pkv_paged_attn_decode(float* out, const void* q, int q_dtype, const void* k_pool,
                          const void* v_pool, int kv_dtype, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t max_context_len, int32_t B, int32_t H_q, int32_t H_kv,
                          int32_t D, int32_t NB, int32_t bs, float scale, const float* k_scale,
                          const float* v_scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Design (not on the pages): which decode kernel runs.  The decode variants
 * (plain, noalloc, hinted, step, window) pick the matrix-core path for the
 * combinations listed under pkv_paged_attn_decode and the vector path for the
 * rest.  pkv_set_decode_path(PKV_DECODE_PATH_VECTOR) sends every later call in
 * the process to the vector path, to compare the two on one batch;
 * PKV_DECODE_PATH_AUTO restores the default choice.  Results agree within
 * the decode's tolerance, not bit for bit.  The setting is process-wide; it
 * returns the previous setting, or PKV_ERR_INVALID_ARG for another value.  A
 * decode already enqueued is not affected.
 */
enum pkv_decode_path { PKV_DECODE_PATH_AUTO = 0, PKV_DECODE_PATH_VECTOR = 1 };
int pkv_set_decode_path(int path);

/*
 * Design (not on the pages): the prefill's workgroup size.  pkv_paged_prefill
 * runs 12-wave workgroups, or 8-wave ones (finer query tiles) when 12-wave
 * ones would give the device fewer work items than it has compute units.
 * pkv_set_prefill_waves(8 or 12) forces one size for every later call in the
 * process, to test and compare the two; 0 restores the automatic choice.
 * Each wave computes the same 32 columns either way, so the results are the
 * same bits, except for bf16 V beyond fp16's range: the workgroups that hold
 * such keys run again with bf16 V, and the two sizes cut the queries into
 * different workgroups.  Returns the previous setting, or
 * PKV_ERR_INVALID_ARG for another value.  A prefill already enqueued is not
 * affected.
 */
int pkv_set_prefill_waves(int nw);

/*
 * pkv_paged_attn_decode_noalloc — pkv_paged_attn_decode without a workspace
 * argument.  Design, for the callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels keep their partials in the library's static scratch instead:
 * a device array of 32 MiB that every device running the library holds until
 * the process ends.  The call itself allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).
 *   Sizes whose scratch need (pkv_decode_workspace_bytes_gqa) exceeds 32 MiB
 *   are refused with PKV_ERR_INVALID_ARG before anything is launched; use
 *   pkv_paged_attn_decode with a workspace for those.
 *   Every call on a device shares that device's scratch and leaves its last
 *   contents there: calls that overlap on one device (several streams or
 *   threads) race.  Nothing in the scratch needs to start at zero.
 *   Other arguments, results and errors as pkv_paged_attn_decode.
 */
int pkv_paged_attn_decode_noalloc(float* out, const void* q, int q_dtype, const void* k_pool,
                                  const void* v_pool, int kv_dtype, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t B, int32_t H_q, int32_t H_kv,
                                  int32_t D, int32_t NB, int32_t bs, float scale, const float* k_scale,
                                  const float* v_scale, void* stream);

/*
 * pkv_paged_attn_decode_hinted — pkv_paged_attn_decode with the host's sum of
 * the context lengths, for callers whose allocator holds the lengths (the sum
 * is the same hint pkv_decode_step takes):
 *   sum_context_lens  the sum of context_lens[b] over the batch, or -1 if
 *     unknown (then the call is pkv_paged_attn_decode).  It only chooses the
 *     work split: when it shows that the planned split keeps every (sequence,
 *     KV head) segment whole, the call runs one piece per segment and skips
 *     the partial results and their merge.  A value above B * min(max_context_len,
 *     max_blocks_per_seq * bs) cannot be a sum of lengths and is taken as -1.
 *     A wrong value keeps the result within the decode's tolerance; it gives
 *     the same bits as the unhinted call only when it leaves the split
 *     unchanged (an overestimate can keep long segments whole, which changes
 *     the order of the reduction and unbalances the work).
 * (Design, not on the pages: the host's allocator knows the lengths, so the
 * sum costs no device read.)
 *   other arguments, errors and ownership as pkv_paged_attn_decode.
 */
int pkv_paged_attn_decode_hinted(float* out, const void* q, int q_dtype, const void* k_pool,
                                 const void* v_pool, int kv_dtype, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, int64_t sum_context_lens, int32_t B,
                                 int32_t H_q, int32_t H_kv, int32_t D, int32_t NB, int32_t bs,
                                 float scale, const float* k_scale, const float* v_scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_decode_step — one decode step: the same result (output and pools) as
 *     pkv_kv_append(k_new, v_new, src_dtype, new_slots, T = B, ...);
 *     pkv_paged_attn_decode(...);
 * where sequence b's new token is its last position: context_lens[b] counts
 * it and new_slots[b] is the slot of position context_lens[b] - 1 (or < 0:
 * the sequence appends nothing this step).
 *   k_new, v_new   device [B][H_kv][D] of src_dtype; new_slots device int64 [B]
 *   others         as pkv_paged_attn_decode / pkv_kv_append
 * With bf16 q and bf16 source rows into bf16 or E4M3 pools on the
 * matrix-core path, the append runs inside the decode launch: the piece that
 * reads position n - 1 takes the new token from k_new/v_new (as the append
 * stores it: the bits of a bf16 pool, the codes of x / scale of an E4M3 pool,
 * encoded as pkv_kv_append encodes them) and stores it into the pool after its
 * reads, saving the append launch.  Other combinations issue the two calls.
 * ("Paged Attention and KV Cache Fragmentation", section "Quantization as a
 * way to stretch paged memory further", for the one-byte codes.)  In the fused form, a new_slots[b] that is not the slot
 * of position n - 1 (or a sequence with n = 0) is a caller error: the token is
 * then stored (when its position's piece exists) but not attended.
 *   sum_context_lens  host hint: the sum of context_lens[b] over the batch, as
 *     the caller's allocator knows it, or -1 if unknown; as for
 *     pkv_paged_attn_decode_hinted (a wrong value keeps the result within
 *     the decode's tolerance, bit-identical only when the split is unchanged).
 * ("Paged Attention and KV Cache Fragmentation", section "How PagedAttention
 * maps an OS concept onto GPU memory": each step appends the new token into
 * the block its table maps it to, then attends over the whole sequence.)
 */
int pkv_decode_step(float* out, const void* q, int q_dtype, const void* k_new, const void* v_new,
                    int src_dtype, const int64_t* new_slots, void* k_pool, void* v_pool, int kv_dtype,
                    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t max_context_len, int64_t sum_context_lens, int32_t B, int32_t H_q, int32_t H_kv,
                    int32_t D, int32_t NB, int32_t bs, float scale, const float* k_scale, const float* v_scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attn_decode_window — pkv_paged_attn_decode over part of each
 * sequence: sequence b attends the positions t < n with t < sink_lens[b] or
 * t >= window_starts[b] (positions in its current table).  A row that attends
 * nothing is zero.  ("Paged Attention and KV Cache Fragmentation", section
 * "A fragmentation problem that paging itself creates: block-level eviction
 * mismatch": StreamingLLM keeps a few attention-sink tokens at the start and
 * a window of recent tokens.)
 *
 *   sink_lens, window_starts  device int32 [B], each may be NULL (= 0 for
 *                  every sequence); a negative sink length counts as 0.  With
 *                  sink_lens NULL, window_starts is a per-sequence start
 *                  offset.  Both NULL: identical to pkv_paged_attn_decode.
 * The positions between the two ranges are read from the table like any
 * other (their blocks must be valid) but weigh nothing, NaN included; evict
 * their whole blocks (pkv_seq_streaming_evict) so that they are not read.
 * Other arguments, workspace included, as pkv_paged_attn_decode.
 */
int pkv_paged_attn_decode_window(float* out, const void* q, int q_dtype, const void* k_pool,
                                 const void* v_pool, int kv_dtype, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, const int32_t* sink_lens,
                                 const int32_t* window_starts, int32_t B, int32_t H_q, int32_t H_kv,
                                 int32_t D, int32_t NB, int32_t bs, float scale, const float* k_scale,
                                 const float* v_scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * pkv_paged_prefill — causal chunked prefill over the paged pools.  The last
 * C_b = query_start[b+1] - query_start[b] tokens of sequence b (whose K/V are
 * already appended, so context_lens[b] = n_b counts them) are its queries:
 * query i, at row query_start[b] + i of q and out, sits at position
 * p = n_b - C_b + i and attends positions 0..p:
 *     out[r][h] = sum_{t<=p} softmax_t(scale * <q[r][h], K_b[g][t]>) V_b[g][t]
 * ("Paged Attention and KV Cache Fragmentation", section "How PagedAttention
 * maps an OS concept onto GPU memory": a prompt is written into the blocks a
 * sequence takes as it grows and attends over them through its table.)
 *
 *   out            device fp32 [T][H_q][D]; rows of no sequence are not written
 *   q              device bf16 [T][H_q][D]
 *   query_start    device int32 [B+1], non-decreasing, query_start[B] <= T
 *   max_query_len  host hint >= max C_b (sizes the launch); queries past it
 *                  are not computed
 *   others         as pkv_paged_attn_decode
 * Requires bf16 q, bf16 or E4M3 KV, D in {64, 128}, bs in {8, 16, 32} and
 * G = H_q / H_kv in {1, 2, 4, 8, 16} (else PKV_ERR_UNSUPPORTED).  No workspace.
 * Device contents are clamped as for the decode; a sequence whose rows leave
 * [0, T) is skipped, and one with C_b > n_b gets zero rows (caller errors).
 */
int pkv_paged_prefill(float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                      int kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, const int32_t* query_start, int32_t max_query_len,
                      int32_t B, int32_t T, int32_t H_q, int32_t H_kv, int32_t D, int32_t NB, int32_t bs,
                      float scale, const float* k_scale, const float* v_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Host allocator: fixed-size blocks, LIFO free list, per-block refcounts.
 * ("Paged Attention and KV Cache Fragmentation", section "How PagedAttention
 * maps an OS concept onto GPU memory": new blocks only as a sequence grows,
 * freed the moment it finishes; every block has the same size so a freed
 * block always fits; shared prefixes point at the same physical blocks.
 * "KV Cache Fragmentation" field guide, section "Why it matters": cheap forks.)
 *
 * Semantics (deterministic, so block ids are reproducible):
 *   - the free list is a stack; initially the first pops return
 *     initial_free_order[0], [1], ... (NULL = 0, 1, ..., NB-1);
 *   - append of n tokens to a sequence of length L takes
 *     ceil((L+n)/bs) - ceil(L/bs) blocks, popped in logical order;
 *     it is all-or-nothing: on PKV_ERR_OUT_OF_BLOCKS nothing changes;
 *     if L % bs != 0, n > 0 and the last block is shared (refcount > 1)
 *     it fails with PKV_ERR_SHARED_BLOCK and nothing changes;
 *   - append with copy-on-write (pkv_seq_append_slots_cow) handles that case
 *     instead: the sequence first takes a fresh block for its last logical
 *     block (popped before any growth block), the shared block's refcount
 *     goes down by one, and the pair (shared, fresh) is reported for
 *     pkv_copy_blocks.  The fresh block counts towards the all-or-nothing
 *     need.  In every other case it behaves as pkv_seq_append_slots and
 *     reports no pair;
 *   - fork: the child (a new id) gets the parent's blocks and length, and
 *     each of those blocks' refcount goes up by one;
 *   - free: the sequence's blocks are visited last to first, refcount goes
 *     down, blocks reaching zero are pushed on the free list;
 *   - swap-out: the sequence's blocks are returned in logical order (save
 *     their contents with pkv_gather_blocks first, or before any later
 *     append or swap-in can reuse them) and released as by free, but the
 *     sequence and its length stay.  A swapped-out sequence holds no blocks
 *     and cannot grow, fork or appear in pkv_block_tables (INVALID_ARG);
 *     free forgets it;
 *   - swap-in: ceil(len/bs) fresh blocks, all-or-nothing (OUT_OF_BLOCKS
 *     changes nothing), popped in logical order and returned; restore the
 *     contents with pkv_scatter_blocks;
 *   - evict_blocks(first, count): full logical blocks [first, first+count)
 *     leave the sequence; its table closes the gap, its length drops by
 *     count*bs, the blocks are released last to first as by free.  A range
 *     that is not made of full blocks of a resident sequence: INVALID_ARG;
 *   - streaming_evict(S, W): if len <= S + W nothing changes and the decode
 *     attends everything (sink_len = window_start = 0).  Otherwise it evicts
 *     blocks [ceil(S/bs), (len-W)/bs) (none if empty) and returns sink_len = S
 *     and window_start = len - W - evicted*bs: with these, the decode attends
 *     exactly the first S and the last W tokens the sequence had before.
 * -------------------------------------------------------------------------*/
typedef struct pkv_allocator pkv_allocator;

int pkv_alloc_create(int32_t NB, int32_t bs, const int32_t* initial_free_order /* host, NB, or NULL */,
                     pkv_allocator** out);
void pkv_alloc_destroy(pkv_allocator* a);
int32_t pkv_alloc_num_free(const pkv_allocator* a);
int pkv_seq_add(pkv_allocator* a, int64_t seq); /* PKV_ERR_INVALID_ARG if seq exists */
/* slots_out: host int64 [n] (may be NULL when n == 0) receives the new tokens' slots. */
int pkv_seq_append_slots(pkv_allocator* a, int64_t seq, int32_t n, int64_t* slots_out);
/* copy_src, copy_dst: host int32 [1] receive the pair, n_copies (host) its count, 0 or 1. */
int pkv_seq_append_slots_cow(pkv_allocator* a, int64_t seq, int32_t n, int64_t* slots_out,
                             int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies);
int pkv_seq_fork(pkv_allocator* a, int64_t parent, int64_t child);
int pkv_seq_free(pkv_allocator* a, int64_t seq);
/* blocks_out: host int32 [max_blocks]; *n_out (host) = blocks written.  INVALID_ARG if the
 * sequence is already swapped out (swap_out) / not swapped out (swap_in) or needs more than
 * max_blocks entries. */
int pkv_seq_swap_out(pkv_allocator* a, int64_t seq, int32_t* blocks_out, int32_t max_blocks,
                     int32_t* n_out);
int pkv_seq_swap_in(pkv_allocator* a, int64_t seq, int32_t* blocks_out, int32_t max_blocks,
                    int32_t* n_out);
int pkv_seq_evict_blocks(pkv_allocator* a, int64_t seq, int32_t first, int32_t count);
/* outputs: host int32 scalars */
int pkv_seq_streaming_evict(pkv_allocator* a, int64_t seq, int32_t sink_tokens, int32_t window_tokens,
                            int32_t* sink_len_out, int32_t* window_start_out, int32_t* evicted_out);
int pkv_seq_len(const pkv_allocator* a, int64_t seq, int32_t* len_out);
/* table_out: host int32 [n][max_blocks], padded with -1; lens_out: host int32 [n].
 * PKV_ERR_INVALID_ARG if a sequence holds more than max_blocks blocks. */
int pkv_block_tables(const pkv_allocator* a, const int64_t* seqs, int32_t n, int32_t max_blocks,
                     int32_t* table_out, int32_t* lens_out);
/* Refcount of a physical block (0 = free); -1 for an id outside the pool. */
int32_t pkv_block_refcount(const pkv_allocator* a, int32_t block);

/* ---------------------------------------------------------------------------
 * Measurement helpers.  Design, not on the pages and not part of the method.
 * pkv_stream_read: reads `bytes` (multiple of 16) from `src` with the
 * library's load pattern and writes one fp32 per workgroup to `sink`
 * (device, >= pkv_stream_read_sink_floats(bytes) floats): a read-bandwidth
 * ceiling for the decode kernels.  pkv_copy: dst[0:bytes) = src[0:bytes),
 * a plain copy of known size used to calibrate memory counters.
 * -------------------------------------------------------------------------*/
size_t pkv_stream_read_sink_floats(size_t bytes);
int pkv_stream_read(const void* src, size_t bytes, float* sink, void* stream);
int pkv_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
