"""Fixed-block free-list allocator with refcounted shared blocks (reference model).

"Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
section "How PagedAttention maps an OS concept onto GPU memory": every block
has the same size, so a freed block always fits any later need; blocks are
taken only as a sequence actually grows and returned the moment it finishes;
requests that share a prefix (or beam-search branches) point at the same
physical blocks.  "KV Cache Fragmentation" field guide (defragging.ai),
section "Why it matters": sharing makes forks cheap.

Readings where the pages are silent (the product allocator reproduces them
bit for bit):
  * the free list is a LIFO stack; with initial order o, the first pops return
    o[0], o[1], ... ;
  * append of n tokens needs ceil((len+n)/bs) - ceil(len/bs) new blocks, popped
    in logical order; it is all-or-nothing;
  * a sequence whose last, partly filled block is shared (refcount > 1) cannot
    grow in place (the shared block would be written for every sharer);
  * fork: the child gets the parent's block list and length, each block's
    refcount goes up by one;
  * free: logical blocks are visited last to first, refcount goes down, a block
    reaching zero is pushed, so the next pops return the freed sequence's blocks
    in their original logical order.

Copy-on-write append (PA, same section: sharers point at one physical block
and only diverge where their content differs; FG "Why it matters": cheap
forks for beam search and branching conversations).  `append_slots_cow` is
append_slots except where the last block is shared and partly filled: the
growing sequence first takes a fresh block for that logical position (popped
before any growth block), the old block loses one reference, and the pair
(old, new) is returned so that the caller copies the block's contents before
writing the new tokens.  The fresh block counts towards the all-or-nothing
block need.

Swap (PA, section "Offloading paged KV blocks to CPU DRAM and NVMe": blocks of
a sequence that is not running move to host memory and come back later).
`swap_out` returns the sequence's blocks in logical order (the caller saves
their contents) and releases them as `free` does, but keeps the sequence and
its length; a swapped-out sequence holds no blocks and cannot grow, fork or
appear in a block table.  `swap_in` takes ceil(len / bs) fresh blocks,
all-or-nothing, popped in logical order, and returns them (the caller restores
the contents into them).

Whole-block eviction (PA, section "A fragmentation problem that paging itself
creates: block-level eviction mismatch": evicting whole blocks keeps the paged
structure that token-level eviction breaks; StreamingLLM keeps a few sink
tokens at the start plus a window of recent tokens).  `evict_blocks` removes
full logical blocks [first, first + count) from a sequence: the table closes
the gap, the length drops by count * bs, the blocks are released as by free.
`streaming_evict(seq, S, W)` evicts the whole blocks strictly between the
blocks holding the first S tokens and the block holding token len - W, and
returns the sink length and window start the decode must use in the
compacted positions, so that it attends exactly the first S and the last W
tokens of the sequence as it was before the eviction.
"""
from __future__ import annotations

from enum import IntEnum


class Status(IntEnum):
    OK = 0
    INVALID_ARG = -1
    UNSUPPORTED = -2
    OUT_OF_BLOCKS = -3
    UNKNOWN_SEQ = -4
    SHARED_BLOCK = -5


def _ceil_div(a, b):
    return -(-a // b)


class AllocModel:
    def __init__(self, NB: int, bs: int, initial_free_order=None):
        if NB <= 0 or bs <= 0:
            raise ValueError("NB and bs must be positive")
        order = list(range(NB)) if initial_free_order is None else [int(x) for x in initial_free_order]
        if sorted(order) != list(range(NB)):
            raise ValueError("initial_free_order must be a permutation of 0..NB-1")
        self.NB, self.bs = NB, bs
        self.stack = order[::-1]  # top of stack = end of list = order[0]
        self.rc = [0] * NB
        self.blocks = {}
        self.lens = {}
        self.swapped = set()

    def num_free(self) -> int:
        return len(self.stack)

    def seq_add(self, seq) -> int:
        if seq in self.blocks:
            return Status.INVALID_ARG
        self.blocks[seq] = []
        self.lens[seq] = 0
        return Status.OK

    def append_slots(self, seq, n):
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ, None
        if n < 0 or seq in self.swapped:
            return Status.INVALID_ARG, None
        blocks, L, bs = self.blocks[seq], self.lens[seq], self.bs
        if n > 0 and L % bs != 0 and self.rc[blocks[-1]] > 1:
            return Status.SHARED_BLOCK, None
        need = _ceil_div(L + n, bs) - _ceil_div(L, bs)
        if need > len(self.stack):
            return Status.OUT_OF_BLOCKS, None
        for _ in range(need):
            blk = self.stack.pop()
            self.rc[blk] = 1
            blocks.append(blk)
        slots = [blocks[p // bs] * bs + p % bs for p in range(L, L + n)]
        self.lens[seq] = L + n
        return Status.OK, slots

    def append_slots_cow(self, seq, n):
        """(status, slots, copies): copies is a list of (src_block, dst_block) pairs (0 or 1)."""
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ, None, None
        if n < 0 or seq in self.swapped:
            return Status.INVALID_ARG, None, None
        blocks, L, bs = self.blocks[seq], self.lens[seq], self.bs
        cow = n > 0 and L % bs != 0 and self.rc[blocks[-1]] > 1
        need = _ceil_div(L + n, bs) - _ceil_div(L, bs) + (1 if cow else 0)
        if need > len(self.stack):
            return Status.OUT_OF_BLOCKS, None, None
        copies = []
        if cow:
            old, new = blocks[-1], self.stack.pop()
            self.rc[old] -= 1
            self.rc[new] = 1
            blocks[-1] = new
            copies.append((old, new))
        st, slots = self.append_slots(seq, n)
        assert st == Status.OK
        return Status.OK, slots, copies

    def fork(self, parent, child) -> int:
        if parent not in self.blocks:
            return Status.UNKNOWN_SEQ
        if child in self.blocks or parent in self.swapped:
            return Status.INVALID_ARG
        self.blocks[child] = list(self.blocks[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.blocks[child]:
            self.rc[blk] += 1
        return Status.OK

    def free(self, seq) -> int:
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ
        for blk in reversed(self.blocks[seq]):
            self.rc[blk] -= 1
            if self.rc[blk] == 0:
                self.stack.append(blk)
        del self.blocks[seq]
        del self.lens[seq]
        self.swapped.discard(seq)
        return Status.OK

    def swap_out(self, seq):
        """(status, blocks): the sequence's blocks in logical order, then released."""
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ, None
        if seq in self.swapped:
            return Status.INVALID_ARG, None
        blocks = list(self.blocks[seq])
        for blk in reversed(blocks):
            self.rc[blk] -= 1
            if self.rc[blk] == 0:
                self.stack.append(blk)
        self.blocks[seq] = []
        self.swapped.add(seq)
        return Status.OK, blocks

    def swap_in(self, seq):
        """(status, blocks): fresh blocks for the whole sequence, in logical order."""
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ, None
        if seq not in self.swapped:
            return Status.INVALID_ARG, None
        need = _ceil_div(self.lens[seq], self.bs)
        if need > len(self.stack):
            return Status.OUT_OF_BLOCKS, None
        blocks = []
        for _ in range(need):
            blk = self.stack.pop()
            self.rc[blk] = 1
            blocks.append(blk)
        self.blocks[seq] = blocks
        self.swapped.discard(seq)
        return Status.OK, list(blocks)

    def _release(self, blocks):
        for blk in reversed(blocks):
            self.rc[blk] -= 1
            if self.rc[blk] == 0:
                self.stack.append(blk)

    def evict_blocks(self, seq, first, count) -> int:
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ
        full = self.lens[seq] // self.bs
        if seq in self.swapped or first < 0 or count < 0 or first + count > full:
            return Status.INVALID_ARG
        blocks = self.blocks[seq]
        self._release(blocks[first:first + count])
        self.blocks[seq] = blocks[:first] + blocks[first + count:]
        self.lens[seq] -= count * self.bs
        return Status.OK

    def streaming_evict(self, seq, sink_tokens, window_tokens):
        """(status, sink_len, window_start, evicted_blocks)."""
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ, None, None, None
        if seq in self.swapped or sink_tokens < 0 or window_tokens < 0:
            return Status.INVALID_ARG, None, None, None
        L, bs = self.lens[seq], self.bs
        if L <= sink_tokens + window_tokens:
            return Status.OK, 0, 0, 0  # everything is kept and attended
        first = _ceil_div(sink_tokens, bs)
        count = max((L - window_tokens) // bs - first, 0)
        if count:  # the blocks strictly between the sink blocks and the window's first block
            st = self.evict_blocks(seq, first, count)
            assert st == Status.OK
        return Status.OK, sink_tokens, L - window_tokens - count * bs, count

    def seq_len(self, seq):
        if seq not in self.blocks:
            return Status.UNKNOWN_SEQ, None
        return Status.OK, self.lens[seq]

    def block_tables(self, seqs, max_blocks):
        import numpy as np
        table = np.full((len(seqs), max_blocks), -1, np.int32)
        lens = np.zeros(len(seqs), np.int32)
        for i, s in enumerate(seqs):
            if s not in self.blocks:
                return Status.UNKNOWN_SEQ, None, None
            if s in self.swapped:
                return Status.INVALID_ARG, None, None
            blocks = self.blocks[s]
            if len(blocks) > max_blocks:
                return Status.INVALID_ARG, None, None
            table[i, :len(blocks)] = blocks
            lens[i] = self.lens[s]
        return Status.OK, table, lens

    def refcount(self, blk) -> int:
        return self.rc[blk]
