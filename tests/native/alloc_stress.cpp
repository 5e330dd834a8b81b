// Randomised stress of the host block allocator through its C API, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_allocator_sanitized.py
// (host code only).  Every operation is drawn at random, invalid ones included
// (unknown sequences, negative or oversized counts, swapped sequences), and the
// allocator's state is checked after each one through the API alone:
//   free blocks + blocks in use == NB, and each block's refcount equals the
//   number of resident sequences whose table holds it;
//   a resident sequence holds ceil(len / bs) blocks, a swapped-out one none.
// Exit status 0 on success, 1 with a message on the first violation.
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <cstdlib>
#include <memory>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"

namespace pkv {
void set_error(const char*, ...) {}  // the library's error text is not needed here
}

static int fail(const char* what, long step) {
  fprintf(stderr, "violation at step %ld: %s\n", step, what);
  return 1;
}

int run(int NB, int bs, unsigned seed, long steps) {
  std::mt19937 rng(seed);
  std::vector<int32_t> order(NB);
  for (int i = 0; i < NB; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_allocator* a = nullptr;
  if (pkv_alloc_create(NB, bs, order.data(), &a) != PKV_OK) return fail("create", -1);
  std::unique_ptr<pkv_allocator, void (*)(pkv_allocator*)> guard(a, pkv_alloc_destroy);
  const int kSeqs = 12;
  std::set<int64_t> live, swapped;
  std::vector<int64_t> slots(4 * NB + 8);
  std::vector<int32_t> blocks(NB + 8), table(kSeqs * (NB + 1));
  std::vector<int32_t> lens(kSeqs);
  auto pick = [&](int hi) { return (int)(rng() % (unsigned)hi); };
  long ok[11] = {0};
  for (long step = 0; step < steps; ++step) {
    const int64_t s = pick(kSeqs + 2) - 1;  // -1 and kSeqs are never added
    const int op = pick(11);
    int st = PKV_OK;
    switch (op) {
      case 0:
        st = pkv_seq_add(a, s);
        if (st == PKV_OK) live.insert(s);
        break;
      case 1: {
        const int n = pick(3 * bs + 2) - 1;
        st = pkv_seq_append_slots(a, s, n, n > 0 ? slots.data() : nullptr);
        break;
      }
      case 2: {
        const int n = pick(3 * bs + 2) - 1;
        int32_t cs = -1, cd = -1, nc = -1;
        st = pkv_seq_append_slots_cow(a, s, n, n > 0 ? slots.data() : nullptr, &cs, &cd, &nc);
        if (st == PKV_OK && (nc < 0 || nc > 1)) return fail("cow copy count", step);
        break;
      }
      case 3: {
        const int64_t c = pick(kSeqs + 1);
        st = pkv_seq_fork(a, s, c);
        if (st == PKV_OK) live.insert(c);
        break;
      }
      case 4:
        st = pkv_seq_free(a, s);
        if (st == PKV_OK) {
          live.erase(s);
          swapped.erase(s);
        }
        break;
      case 5: {
        int32_t n = -1;
        st = pkv_seq_swap_out(a, s, blocks.data(), pick(NB + 2), &n);
        if (st == PKV_OK) swapped.insert(s);
        break;
      }
      case 6: {
        int32_t n = -1;
        st = pkv_seq_swap_in(a, s, blocks.data(), pick(NB + 2), &n);
        if (st == PKV_OK) swapped.erase(s);
        break;
      }
      case 7:
        st = pkv_seq_evict_blocks(a, s, pick(6) - 1, pick(5) - 1);
        break;
      case 8: {
        int32_t sl = -1, ws = -1, ev = -1;
        st = pkv_seq_streaming_evict(a, s, pick(3 * bs), pick(4 * bs), &sl, &ws, &ev);
        break;
      }
      case 9: {
        int32_t len = -1;
        st = pkv_seq_len(a, s, &len);
        break;
      }
      default: {
        const int64_t q[2] = {s, (int64_t)pick(kSeqs)};
        st = pkv_block_tables(a, q, 2, pick(NB + 2), table.data(), lens.data());
        break;
      }
    }
    if (st > 0 || st < PKV_ERR_HIP) return fail("status out of range", step);
    ok[op] += st == PKV_OK;
    // ---- invariants through the API
    std::vector<int32_t> holders(NB, 0);
    int32_t held = 0;
    for (int64_t q : live) {
      int32_t len = -1;
      if (pkv_seq_len(a, q, &len) != PKV_OK || len < 0) return fail("live sequence has no length", step);
      const int nb = (len + bs - 1) / bs;
      int32_t lq = -1;
      const int tst = pkv_block_tables(a, &q, 1, NB + 1, table.data(), &lq);
      if (swapped.count(q)) {
        if (tst == PKV_OK) return fail("swapped sequence appears in a table", step);
        continue;
      }
      if (tst != PKV_OK || lq != len) return fail("table of a resident sequence", step);
      for (int j = 0; j < NB + 1; ++j) {
        const int32_t b = table[j];
        if (j < nb) {
          if (b < 0 || b >= NB) return fail("table entry out of the pool", step);
          ++holders[b];
        } else if (b != -1) {
          return fail("table padding", step);
        }
      }
      held += nb;
    }
    int32_t in_use = 0, rc_sum = 0;
    for (int b = 0; b < NB; ++b) {
      const int32_t rc = pkv_block_refcount(a, b);
      if (rc < 0) return fail("refcount", step);
      if (rc != holders[b]) return fail("refcount differs from the holders", step);
      in_use += rc > 0;
      rc_sum += rc;
    }
    if (rc_sum != held) return fail("blocks held", step);
    if (pkv_alloc_num_free(a) + in_use != NB) return fail("free + in use != NB", step);
  }
  if (pkv_block_refcount(a, -1) != -1 || pkv_block_refcount(a, NB) != -1) return fail("refcount range", steps);
  // every operation must have succeeded often enough for the script to exercise it
  printf("NB %d bs %d successes:", NB, bs);
  for (int i = 0; i < 11; ++i) printf(" %ld", ok[i]);
  printf("\n");
  for (int i = 0; i < 11; ++i)
    if (ok[i] < steps / 500) return fail("an operation rarely succeeds", steps);
  return 0;
}

int main(int argc, char** argv) {
  const long steps = argc > 1 ? atol(argv[1]) : 20000;
  int rc = 0;
  rc |= run(48, 4, 1u, steps);
  rc |= run(17, 1, 2u, steps);
  rc |= run(96, 16, 3u, steps);
  if (rc == 0) printf("alloc_stress ok: %ld steps x 3 allocators\n", steps);
  return rc;
}
