"""Paged KV pool, slot scatter and gather-then-attend decode (fp64 reference).

What the method computes ("KV Cache Fragmentation" field guide, defragging.ai,
section "Definition"; "Paged Attention and KV Cache Fragmentation",
inferenceengineering.co, section "How PagedAttention maps an OS concept onto
GPU memory"): the KV cache is cut into fixed-size physical blocks, each
holding a fixed number of tokens' keys and values for every attention head; a
sequence sees its cache as one logical run of tokens, and a per-sequence
block table maps logical block j to the physical block that holds it.  Paging
changes where the bytes live, not what attention computes: the decode output
of a sequence is ordinary softmax attention of its one query token over its
n logical tokens.

Pool layout (a design choice of this library; the pages fix none).  Both pools
hold NB physical blocks; inside a block every KV head has its own contiguous
tile of bs tokens:

  K pool  [NB, H_kv, d // X, bs, X]   X = 16 bytes / element size
  V pool  [NB, H_kv, d, bs]

i.e. a K tile stores, for each 16-byte group of the head dimension, the bs
tokens one after another, and a V tile stores each head-dimension column as a
run of bs tokens.  Element storage: fp32 values, bf16 bit patterns (uint16) or
E4M3FN codes (uint8, with one fp32 scale per KV head for K and one for V;
real value = code value * scale).

Slots: token position p of a sequence lives at slot = table[p // bs] * bs + p % bs.

GQA ("Fragmentation" lesson, klaylearn, navigation "MHA, MQA, GQA"): the
pages name the grouping only.  Reading taken: query head h uses KV head
h // (H_q / H_kv), i.e. contiguous groups.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, e4m3_decode, e4m3_encode

_ELEM = {"f32": 4, "bf16": 2, "e4m3": 1}
_STORE = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}


def lanes_per_16b(dtype: str) -> int:
    """X: elements per 16-byte group of the K layout."""
    return 16 // _ELEM[dtype]


def pool_shapes(NB: int, H_kv: int, d: int, bs: int, dtype: str):
    X = lanes_per_16b(dtype)
    assert d % X == 0
    return (NB, H_kv, d // X, bs, X), (NB, H_kv, d, bs)


def empty_pools(NB, H_kv, d, bs, dtype):
    ks, vs = pool_shapes(NB, H_kv, d, bs, dtype)
    return np.zeros(ks, _STORE[dtype]), np.zeros(vs, _STORE[dtype])


def to_f64(x, dtype: str) -> np.ndarray:
    """Exact fp64 values of stored elements (E4M3 codes are decoded without their scale)."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "e4m3":
        return e4m3_decode(x)
    raise ValueError(dtype)


def _convert_rows(x, src: str, dst: str, scale):
    """Source rows [T, H, d] -> pool storage; the only arithmetic is the fp8 quantisation:
    y = fp32(x) / scale_h as an IEEE fp32 division, then round-to-nearest-even E4M3FN."""
    if src == dst:
        return np.asarray(x, _STORE[dst])
    if src == "bf16" and dst == "e4m3":
        x32 = bf16_bits_to_f64(x).astype(np.float32)  # exact
        y = x32 / np.asarray(scale, np.float32)[None, :, None]  # fp32 / fp32, correctly rounded
        return e4m3_encode(y.astype(np.float32))
    raise ValueError(f"unsupported append {src} -> {dst}")


def ref_append(k_pool, v_pool, k, v, src_dtype: str, slots, bs: int, pool_dtype: str,
               k_scale=None, v_scale=None):
    """Write token t's K/V rows to slot slots[t] (slots < 0 are padding and skipped).
    Returns new pools; the inputs are not modified."""
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    slots = np.asarray(slots, np.int64)
    keep = slots >= 0
    if not keep.any():
        return kp, vp
    NB, H, dX, bs_, X = kp.shape
    assert bs_ == bs
    kr = _convert_rows(np.asarray(k)[keep], src_dtype, pool_dtype, k_scale)
    vr = _convert_rows(np.asarray(v)[keep], src_dtype, pool_dtype, v_scale)
    blk = slots[keep] // bs
    off = slots[keep] % bs
    assert blk.max() < NB
    T = kr.shape[0]
    kp[blk, :, :, off, :] = kr.reshape(T, H, dX, X)
    vp[blk, :, :, off] = vr
    return kp, vp


def gather_sequence(k_pool, v_pool, kv_dtype, table_row, n, bs, k_scale=None, v_scale=None):
    """Walk the block table: the sequence's first n tokens as contiguous fp64 [H_kv, n, d]."""
    NB, H, dX, bs_, X = k_pool.shape
    d = dX * X
    nblk = -(-n // bs)
    ids = np.asarray(table_row[:nblk], np.int64)
    assert ((ids >= 0) & (ids < NB)).all(), "block table entry outside the pool"
    kb = to_f64(k_pool[ids], kv_dtype)  # [nblk, H, d/X, bs, X]
    vb = to_f64(v_pool[ids], kv_dtype)  # [nblk, H, d, bs]
    K = np.ascontiguousarray(kb.transpose(1, 0, 3, 2, 4).reshape(H, nblk * bs, d)[:, :n])
    V = np.ascontiguousarray(vb.transpose(1, 0, 3, 2).reshape(H, nblk * bs, d)[:, :n])
    if kv_dtype == "e4m3":  # real = code value * per-KV-head scale (exact in fp64)
        K = K * np.asarray(k_scale, np.float32).astype(np.float64)[:, None, None]
        V = V * np.asarray(v_scale, np.float32).astype(np.float64)[:, None, None]
    return K, V


def attended(n, sink_len=0, window_start=0):
    """Logical positions a decode attends: t < n with t < sink_len or t >= window_start.

    "Paged Attention and KV Cache Fragmentation", section "A fragmentation problem that paging
    itself creates: block-level eviction mismatch": StreamingLLM keeps a few attention-sink tokens
    at the start plus a window of recent tokens and drops the rest.  With sink_len = 0 the window
    start is a plain per-sequence start offset; with window_start <= sink_len nothing is dropped."""
    t = np.arange(n)
    return (t < sink_len) | (t >= window_start)


def ref_decode(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens, scale, bs,
               k_scale=None, v_scale=None, rows=None, sink_lens=None, window_starts=None):
    """Paged decode attention, gather-then-attend, fp64.

    q [B, H_q, d] (fp32 values or bf16 bits); returns fp64 [B, H_q, d].
    For sequence b with n = context_lens[b] > 0 and query head h (KV head g = h // G):
        s_t = scale * <q[b,h], K_b[g, t]>,  t in A_b
        o[b,h] = sum_t exp(s_t - max s) V_b[g, t] / sum_t exp(s_t - max s)
    where A_b = attended(n, sink_lens[b], window_starts[b]) (all t < n when both are None).
    An empty A_b (n = 0 among others) gives a zero row.  `rows` optionally restricts the work
    to some batch entries (other rows are left zero).
    """
    q64 = to_f64(q, q_dtype)
    B, H_q, d = q64.shape
    H_kv = k_pool.shape[1]
    G = H_q // H_kv
    assert G * H_kv == H_q
    s64 = float(np.float32(scale))
    out = np.zeros((B, H_q, d), np.float64)
    for b in (range(B) if rows is None else rows):
        n = int(context_lens[b])
        keep = attended(n, 0 if sink_lens is None else int(sink_lens[b]),
                        0 if window_starts is None else int(window_starts[b]))
        if not keep.any():
            continue
        K, V = gather_sequence(k_pool, v_pool, kv_dtype, block_tables[b], n, bs, k_scale, v_scale)
        K, V = K[:, keep], V[:, keep]
        for h in range(H_q):
            g = h // G
            s = s64 * (K[g] @ q64[b, h])
            w = np.exp(s - s.max())
            out[b, h] = (w @ V[g]) / w.sum()
    return out


def ref_prefill(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens, query_start, scale, bs,
                k_scale=None, v_scale=None, seqs=None, rows=None):
    """Paged prefill (chunked multi-query attention) over the same pools, fp64.

    The last C_b = query_start[b+1] - query_start[b] tokens of sequence b (n_b = context_lens[b]
    tokens, their K/V already appended) are its queries, packed in q [T, H_q, d] at rows
    query_start[b] ... query_start[b+1]-1.  Query i sits at position p = n_b - C_b + i and attends
    causally: s_t = scale * <q_i, K_b[g, t]> for t <= p, o_i = softmax(s) V_b[g, :p+1].
    Returns fp64 [T, H_q, d].  `seqs` (sequences) or `rows` (packed query rows) optionally restrict
    the work; other rows stay zero.

    "Paged Attention and KV Cache Fragmentation", section "How PagedAttention maps an OS concept
    onto GPU memory": a sequence's blocks are taken as it grows; the prompt (or each chunk of
    it) is written into them and attends over everything before it through the same table."""
    q64 = to_f64(q, q_dtype)
    T, H_q, d = q64.shape
    H_kv = k_pool.shape[1]
    G = H_q // H_kv
    assert G * H_kv == H_q
    s64 = float(np.float32(scale))
    qs = np.asarray(query_start, np.int64)
    out = np.zeros((T, H_q, d), np.float64)
    for b in (range(len(qs) - 1) if seqs is None else seqs):
        n, r0, C = int(context_lens[b]), int(qs[b]), int(qs[b + 1] - qs[b])
        assert 0 <= C <= n
        if C == 0:
            continue
        wanted = [i for i in range(C) if rows is None or r0 + i in rows]
        if not wanted:
            continue
        K, V = gather_sequence(k_pool, v_pool, kv_dtype, block_tables[b], n, bs, k_scale, v_scale)
        for i in wanted:
            p = n - C + i
            for h in range(H_q):
                g = h // G
                s = s64 * (K[g, :p + 1] @ q64[r0 + i, h])
                w = np.exp(s - s.max())
                out[r0 + i, h] = (w @ V[g, :p + 1]) / w.sum()
    return out


__all__ = ["pool_shapes", "lanes_per_16b", "empty_pools", "to_f64", "ref_append",
           "gather_sequence", "ref_decode", "attended", "ref_prefill"]


def ref_copy_blocks(k_pool, v_pool, pairs):
    """Copy-on-write block copy: for each (src, dst) pair in order, physical block dst of
    both pools becomes an exact copy of block src (every head, every token slot).

    "Paged Attention and KV Cache Fragmentation", section "How PagedAttention maps an OS
    concept onto GPU memory": sharers of a block diverge only where their content differs;
    the copy gives the diverging sequence its own block holding the shared tokens.
    Returns new arrays; the inputs are not modified."""
    k, v = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    for src, dst in pairs:
        k[dst] = k[src]
        v[dst] = v[src]
    return k, v


def ref_gather_blocks(k_pool, v_pool, blocks):
    """Swap-out staging: record i of the result holds physical block blocks[i] as raw bytes,
    its K tile of every head followed by its V tile of every head ([n, 2, block bytes], uint8).

    "Paged Attention and KV Cache Fragmentation", section "Offloading paged KV blocks to CPU
    DRAM and NVMe": blocks move between HBM and host memory, and the scattered paged layout
    turns that into many small transfers; gathering the blocks into one contiguous buffer
    makes it one large transfer."""
    ids = np.asarray(blocks, np.int64)
    nbytes = k_pool[0].nbytes  # one block of one pool (K and V blocks have the same size)
    kb = np.ascontiguousarray(k_pool[ids]).view(np.uint8).reshape(len(ids), nbytes)
    vb = np.ascontiguousarray(v_pool[ids]).view(np.uint8).reshape(len(ids), nbytes)
    return np.stack([kb, vb], axis=1)


def ref_scatter_blocks(k_pool, v_pool, blocks, staging):
    """Swap-in: physical block blocks[i] of both pools takes the bytes of record i of a staging
    buffer laid out as ref_gather_blocks makes it.  Returns new pools; inputs unchanged."""
    k, v = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    st = np.asarray(staging, np.uint8)
    for i, b in enumerate(np.asarray(blocks, np.int64)):
        k[b] = st[i, 0].view(k.dtype).reshape(k.shape[1:])
        v[b] = st[i, 1].view(v.dtype).reshape(v.shape[1:])
    return k, v

