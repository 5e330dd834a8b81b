"""KV-cache byte arithmetic and allocation-waste accounting.

* Per-token footprint of a decoder-only model, "Fragmentation" lesson
  (klaylearn, The KV Cache 03.06), section "Notes": b_tok = 2 * L * H_kv * d_h * s
  (2 for K and V, L layers, H_kv KV heads, head dim d_h, s bytes per scalar); a
  request of length T stored contiguously needs T * b_tok bytes.
* The memory bill in "Paged Attention and KV Cache Fragmentation"
  (inferenceengineering.co), opening section: batch x sequence length x layers
  x 2 x hidden dimension x bytes per value.
* Waste: "KV Cache Fragmentation" field guide (defragging.ai), section
  "Definition" and "Paged Attention and KV Cache Fragmentation", section "The
  two fragmentation modes that previous systems failed to solve": a contiguous
  max-length reservation per request leaves the unfilled part idle, while a
  paged cache only loses the unfilled tail of each sequence's last block
  (section "How PagedAttention maps an OS concept onto GPU memory").
"""
from __future__ import annotations

import numpy as np


def bytes_per_token(L: int, H_kv: int, d_h: int, s: float) -> float:
    return 2 * L * H_kv * d_h * s


def request_bytes(T: int, L: int, H_kv: int, d_h: int, s: float) -> float:
    return T * bytes_per_token(L, H_kv, d_h, s)


def memory_bill(batch: int, seq_len: int, layers: int, hidden: int, s: float) -> float:
    return batch * seq_len * layers * 2 * hidden * s


def kv_bytes_logical(context_lens, H_kv: int, d: int, s: float) -> int:
    """K+V bytes one decode call reads when every sequence reads its own tokens."""
    return int(sum(int(n) for n in context_lens) * H_kv * d * 2 * s)


def kv_bytes_unique(block_tables, context_lens, bs: int, H_kv: int, d: int, s: float) -> int:
    """K+V bytes of the distinct physical blocks the batch touches: for every physical
    block, the token positions in it that at least one sequence attends to."""
    used = {}
    for row, n in zip(block_tables, context_lens):
        n = int(n)
        for j in range(-(-n // bs)):
            blk = int(row[j])
            used[blk] = max(used.get(blk, 0), min(bs, n - j * bs))
    return int(sum(used.values()) * H_kv * d * 2 * s)


def paged_waste(context_lens, bs: int) -> float:
    """Fraction of allocated token slots left empty when each sequence holds ceil(n/bs) blocks."""
    n = np.asarray(context_lens, np.int64)
    alloc = (-(-n // bs) * bs).sum()
    return float(1.0 - n.sum() / alloc)


def contiguous_waste(context_lens, reserve: int) -> float:
    """Fraction left empty when each sequence reserves `reserve` contiguous token slots."""
    n = np.asarray(context_lens, np.int64)
    assert (n <= reserve).all()
    return float(1.0 - n.sum() / (len(n) * reserve))
