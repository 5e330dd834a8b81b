// Host-side fixed-block free-list allocator with refcounted shared blocks.
//
// "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
// section "How PagedAttention maps an OS concept onto GPU memory": blocks are
// all the same size, so any freed block fits any later need and there is no
// external fragmentation; a sequence takes blocks only as it grows and gives
// them back when it finishes; sequences with a common prefix, or beam-search
// branches, point at the same physical blocks.  "KV Cache Fragmentation"
// field guide (defragging.ai), section "Why it matters": sharing makes forks
// cheap.  Section "Offloading paged KV blocks to CPU DRAM and NVMe": blocks of
// a sequence that is not running move to host memory and come back later
// (swap-out / swap-in).  Section "A fragmentation problem that paging itself
// creates: block-level eviction mismatch": eviction of whole blocks keeps the
// paged structure; StreamingLLM keeps sink tokens plus a recent window.  Exact
// semantics (LIFO order, all-or-nothing appends, the shared partial-block rule,
// copy-on-write appends, reverse-order frees, swaps, block eviction) are
// spelled out in pkv.h.

#include <stdint.h>

#include <unordered_map>
#include <vector>

#include "internal.h"

struct pkv_allocator {
  int32_t NB = 0;
  int32_t bs = 0;
  std::vector<int32_t> stack;  // free list, top = back
  std::vector<int32_t> rc;     // refcount per physical block
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
    bool swapped = false;  // swapped out: keeps its length, holds no blocks
  };
  std::unordered_map<int64_t, Seq> seqs;
};

using pkv::set_error;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// release a sequence's blocks last to first (a block reaching refcount 0 goes on the free list)
static void release_blocks(pkv_allocator* a, const std::vector<int32_t>& blocks) {
  for (auto r = blocks.rbegin(); r != blocks.rend(); ++r)
    if (--a->rc[*r] == 0) a->stack.push_back(*r);
}

extern "C" {

int pkv_alloc_create(int32_t NB, int32_t bs, const int32_t* initial_free_order, pkv_allocator** out) {
  if (!out || NB <= 0 || bs <= 0) {
    set_error("alloc_create: bad arguments NB=%d bs=%d", NB, bs);
    return PKV_ERR_INVALID_ARG;
  }
  *out = nullptr;
  auto* a = new pkv_allocator();
  a->NB = NB;
  a->bs = bs;
  a->rc.assign(NB, 0);
  a->stack.resize(NB);
  if (initial_free_order) {
    std::vector<char> seen(NB, 0);
    for (int32_t i = 0; i < NB; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= NB || seen[b]) {
        set_error("alloc_create: initial_free_order is not a permutation of 0..NB-1 (entry %d = %d)", i, b);
        delete a;
        return PKV_ERR_INVALID_ARG;
      }
      seen[b] = 1;
      a->stack[NB - 1 - i] = b;  // first pop returns initial_free_order[0]
    }
  } else {
    for (int32_t i = 0; i < NB; ++i) a->stack[NB - 1 - i] = i;
  }
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_allocator* a) { delete a; }

int32_t pkv_alloc_num_free(const pkv_allocator* a) { return a ? (int32_t)a->stack.size() : -1; }

int pkv_seq_add(pkv_allocator* a, int64_t seq) {
  if (!a) return PKV_ERR_INVALID_ARG;
  if (a->seqs.count(seq)) {
    set_error("seq_add: sequence %lld already exists", (long long)seq);
    return PKV_ERR_INVALID_ARG;
  }
  a->seqs.emplace(seq, pkv_allocator::Seq{});
  return PKV_OK;
}

// Shared body of the two appends.  With `cow`, a shared partly filled last
// block is replaced by a fresh one (popped before the growth blocks) and the
// pair (old, new) is reported; without it, that case is refused.
static int append_impl(pkv_allocator* a, int64_t seq, int32_t n, int64_t* slots_out, bool cow,
                       int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    set_error("append_slots: unknown sequence %lld", (long long)seq);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  if (n < 0 || (n > 0 && !slots_out)) {
    set_error("append_slots: bad n=%d or null output", n);
    return PKV_ERR_INVALID_ARG;
  }
  auto& s = it->second;
  if (s.swapped) {
    set_error("append_slots: sequence %lld is swapped out", (long long)seq);
    return PKV_ERR_INVALID_ARG;
  }
  const int64_t L = s.len, bs = a->bs;
  if (L + n > (int64_t)0x7FFFFFFF) {
    set_error("append_slots: length would exceed 2^31-1");
    return PKV_ERR_INVALID_ARG;
  }
  const bool shared_tail = n > 0 && L % bs != 0 && a->rc[s.blocks.back()] > 1;
  if (shared_tail && !cow) {
    set_error("append_slots: sequence %lld would grow into shared block %d", (long long)seq, s.blocks.back());
    return PKV_ERR_SHARED_BLOCK;
  }
  const int64_t need = ceil_div(L + n, bs) - ceil_div(L, bs) + (shared_tail ? 1 : 0);
  if (need > (int64_t)a->stack.size()) {
    set_error("append_slots: need %lld blocks, %zu free", (long long)need, a->stack.size());
    return PKV_ERR_OUT_OF_BLOCKS;
  }
  if (cow) *n_copies = 0;
  if (shared_tail) {
    const int32_t old = s.blocks.back(), fresh = a->stack.back();
    a->stack.pop_back();
    a->rc[old] -= 1;
    a->rc[fresh] = 1;
    s.blocks.back() = fresh;
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *n_copies = 1;
  }
  const int64_t grow = need - (shared_tail ? 1 : 0);
  for (int64_t i = 0; i < grow; ++i) {
    const int32_t b = a->stack.back();
    a->stack.pop_back();
    a->rc[b] = 1;
    s.blocks.push_back(b);
  }
  for (int64_t p = L; p < L + n; ++p) slots_out[p - L] = (int64_t)s.blocks[p / bs] * bs + p % bs;
  s.len = L + n;
  return PKV_OK;
}

int pkv_seq_append_slots(pkv_allocator* a, int64_t seq, int32_t n, int64_t* slots_out) {
  return append_impl(a, seq, n, slots_out, false, nullptr, nullptr, nullptr);
}

int pkv_seq_append_slots_cow(pkv_allocator* a, int64_t seq, int32_t n, int64_t* slots_out, int32_t* copy_src,
                             int32_t* copy_dst, int32_t* n_copies) {
  if (!copy_src || !copy_dst || !n_copies) {
    set_error("append_slots_cow: null copy output");
    return PKV_ERR_INVALID_ARG;
  }
  return append_impl(a, seq, n, slots_out, true, copy_src, copy_dst, n_copies);
}

int pkv_seq_fork(pkv_allocator* a, int64_t parent, int64_t child) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) {
    set_error("fork: unknown parent %lld", (long long)parent);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  if (a->seqs.count(child)) {
    set_error("fork: child %lld already exists", (long long)child);
    return PKV_ERR_INVALID_ARG;
  }
  if (it->second.swapped) {
    set_error("fork: parent %lld is swapped out", (long long)parent);
    return PKV_ERR_INVALID_ARG;
  }
  pkv_allocator::Seq c = it->second;  // copy before emplace (rehash may move it)
  for (int32_t b : c.blocks) a->rc[b] += 1;
  a->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_seq_free(pkv_allocator* a, int64_t seq) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    set_error("free: unknown sequence %lld", (long long)seq);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  release_blocks(a, it->second.blocks);
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_seq_swap_out(pkv_allocator* a, int64_t seq, int32_t* blocks_out, int32_t max_blocks, int32_t* n_out) {
  if (!a || !n_out || max_blocks < 0 || (max_blocks > 0 && !blocks_out)) {
    set_error("swap_out: bad arguments");
    return PKV_ERR_INVALID_ARG;
  }
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    set_error("swap_out: unknown sequence %lld", (long long)seq);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  auto& s = it->second;
  if (s.swapped || (int64_t)s.blocks.size() > max_blocks) {
    set_error("swap_out: sequence %lld is swapped out already or holds more than %d blocks", (long long)seq,
              max_blocks);
    return PKV_ERR_INVALID_ARG;
  }
  for (size_t j = 0; j < s.blocks.size(); ++j) blocks_out[j] = s.blocks[j];
  *n_out = (int32_t)s.blocks.size();
  release_blocks(a, s.blocks);
  s.blocks.clear();
  s.swapped = true;
  return PKV_OK;
}

int pkv_seq_swap_in(pkv_allocator* a, int64_t seq, int32_t* blocks_out, int32_t max_blocks, int32_t* n_out) {
  if (!a || !n_out || max_blocks < 0 || (max_blocks > 0 && !blocks_out)) {
    set_error("swap_in: bad arguments");
    return PKV_ERR_INVALID_ARG;
  }
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    set_error("swap_in: unknown sequence %lld", (long long)seq);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  auto& s = it->second;
  const int64_t need = ceil_div(s.len, a->bs);
  if (!s.swapped || need > max_blocks) {
    set_error("swap_in: sequence %lld is not swapped out or needs more than %d blocks", (long long)seq,
              max_blocks);
    return PKV_ERR_INVALID_ARG;
  }
  if (need > (int64_t)a->stack.size()) {
    set_error("swap_in: need %lld blocks, %zu free", (long long)need, a->stack.size());
    return PKV_ERR_OUT_OF_BLOCKS;
  }
  for (int64_t j = 0; j < need; ++j) {
    const int32_t b = a->stack.back();
    a->stack.pop_back();
    a->rc[b] = 1;
    s.blocks.push_back(b);
    blocks_out[j] = b;
  }
  *n_out = (int32_t)need;
  s.swapped = false;
  return PKV_OK;
}

int pkv_seq_evict_blocks(pkv_allocator* a, int64_t seq, int32_t first, int32_t count) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    set_error("evict_blocks: unknown sequence %lld", (long long)seq);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  auto& s = it->second;
  const int64_t full = s.len / a->bs;
  if (s.swapped || first < 0 || count < 0 || (int64_t)first + count > full) {
    set_error("evict_blocks: blocks [%d, %d) are not full blocks of resident sequence %lld", first,
              first + count, (long long)seq);
    return PKV_ERR_INVALID_ARG;
  }
  const std::vector<int32_t> gone(s.blocks.begin() + first, s.blocks.begin() + first + count);
  release_blocks(a, gone);
  s.blocks.erase(s.blocks.begin() + first, s.blocks.begin() + first + count);
  s.len -= (int64_t)count * a->bs;
  return PKV_OK;
}

int pkv_seq_streaming_evict(pkv_allocator* a, int64_t seq, int32_t sink_tokens, int32_t window_tokens,
                            int32_t* sink_len_out, int32_t* window_start_out, int32_t* evicted_out) {
  if (!a || !sink_len_out || !window_start_out || !evicted_out || sink_tokens < 0 || window_tokens < 0) {
    set_error("streaming_evict: bad arguments");
    return PKV_ERR_INVALID_ARG;
  }
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    set_error("streaming_evict: unknown sequence %lld", (long long)seq);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  if (it->second.swapped) {
    set_error("streaming_evict: sequence %lld is swapped out", (long long)seq);
    return PKV_ERR_INVALID_ARG;
  }
  const int64_t L = it->second.len, bs = a->bs;
  if (L <= (int64_t)sink_tokens + window_tokens) {  // everything is kept and attended
    *sink_len_out = 0;
    *window_start_out = 0;
    *evicted_out = 0;
    return PKV_OK;
  }
  const int64_t first = ceil_div(sink_tokens, bs);
  int64_t count = (L - window_tokens) / bs - first;
  if (count < 0) count = 0;
  if (count > 0) {  // the blocks strictly between the sink blocks and the window's first block
    const int st = pkv_seq_evict_blocks(a, seq, (int32_t)first, (int32_t)count);
    if (st != PKV_OK) return st;
  }
  *sink_len_out = sink_tokens;
  *window_start_out = (int32_t)(L - window_tokens - count * bs);
  *evicted_out = (int32_t)count;
  return PKV_OK;
}

int pkv_seq_len(const pkv_allocator* a, int64_t seq, int32_t* len_out) {
  if (!a || !len_out) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) {
    set_error("seq_len: unknown sequence %lld", (long long)seq);
    return PKV_ERR_UNKNOWN_SEQ;
  }
  *len_out = (int32_t)it->second.len;
  return PKV_OK;
}

int pkv_block_tables(const pkv_allocator* a, const int64_t* seqs, int32_t n, int32_t max_blocks,
                     int32_t* table_out, int32_t* lens_out) {
  if (!a || n < 0 || max_blocks <= 0 || (n > 0 && (!seqs || !table_out || !lens_out))) {
    set_error("block_tables: bad arguments");
    return PKV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {  // validate first: no partial output on error
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) {
      set_error("block_tables: unknown sequence %lld", (long long)seqs[i]);
      return PKV_ERR_UNKNOWN_SEQ;
    }
    if (it->second.swapped) {
      set_error("block_tables: sequence %lld is swapped out", (long long)seqs[i]);
      return PKV_ERR_INVALID_ARG;
    }
    if ((int64_t)it->second.blocks.size() > max_blocks) {
      set_error("block_tables: sequence %lld holds %zu blocks > max_blocks %d", (long long)seqs[i],
                it->second.blocks.size(), max_blocks);
      return PKV_ERR_INVALID_ARG;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = a->seqs.find(seqs[i])->second;
    int32_t* row = table_out + (size_t)i * max_blocks;
    int32_t j = 0;
    for (; j < (int32_t)s.blocks.size(); ++j) row[j] = s.blocks[j];
    for (; j < max_blocks; ++j) row[j] = -1;
    lens_out[i] = (int32_t)s.len;
  }
  return PKV_OK;
}

int32_t pkv_block_refcount(const pkv_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->NB) return -1;
  return a->rc[block];
}

}  // extern "C"
