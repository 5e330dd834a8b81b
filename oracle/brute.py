"""A second decode oracle in pure Python, for tiny inputs only.

It shares nothing with `paged.ref_decode` beyond the format decoders: it walks
the block table token by token with explicit flat-index arithmetic over the
pool layout (see `paged` for the layout), forms the softmax weights without
subtracting the maximum, and sums with math.fsum.  Agreement of the two on
small cases pins the numpy gather (reshape/transpose) and the numpy softmax.

Method: "KV Cache Fragmentation" field guide (defragging.ai), section
"Definition" — the attention kernel walks the per-request table that maps
logical positions to physical pages.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import bf16_bits_to_f64, e4m3_decode_table


def _scalar_decoder(dtype):
    if dtype == "f32":
        return lambda x: float(np.float32(x))
    if dtype == "bf16":
        return lambda x: float(bf16_bits_to_f64(np.uint16(x)))
    table = e4m3_decode_table()
    return lambda x: float(table[int(x)])


def brute_decode(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens, scale, bs,
                 k_scale=None, v_scale=None, sink_lens=None, window_starts=None):
    qd = _scalar_decoder(q_dtype)
    kd = _scalar_decoder(kv_dtype)
    q = np.asarray(q)
    B, H_q, d = q.shape
    kflat = np.asarray(k_pool).reshape(-1)
    vflat = np.asarray(v_pool).reshape(-1)
    NB, H_kv = k_pool.shape[0], k_pool.shape[1]
    X = k_pool.shape[4]
    G = H_q // H_kv
    sc = float(np.float32(scale))
    out = [[[0.0] * d for _ in range(H_q)] for _ in range(B)]
    for b in range(B):
        n = int(context_lens[b])
        sink = 0 if sink_lens is None else int(sink_lens[b])
        wst = 0 if window_starts is None else int(window_starts[b])
        for h in range(H_q):
            g = h // G
            ks = float(np.float32(k_scale[g])) if kv_dtype == "e4m3" else 1.0
            vs = float(np.float32(v_scale[g])) if kv_dtype == "e4m3" else 1.0
            qv = [qd(q[b, h, i]) for i in range(d)]
            weights, vrows = [], []
            for t in range(n):
                if sink <= t < wst:  # dropped by the sink + window rule
                    continue
                blk = int(block_tables[b][t // bs])
                assert 0 <= blk < NB
                off = t % bs
                krow, vrow = [], []
                for i in range(d):
                    # K[blk, g, i // X, off, i % X] and V[blk, g, i, off] in row-major order
                    kidx = (((blk * H_kv + g) * (d // X) + i // X) * bs + off) * X + i % X
                    vidx = ((blk * H_kv + g) * d + i) * bs + off
                    krow.append(kd(kflat[kidx]) * ks)
                    vrow.append(kd(vflat[vidx]) * vs)
                s = sc * math.fsum(a * c for a, c in zip(qv, krow))
                weights.append(math.exp(s))
                vrows.append(vrow)
            if weights:
                den = math.fsum(weights)
                out[b][h] = [math.fsum(w * vr[i] for w, vr in zip(weights, vrows)) / den
                             for i in range(d)]
    return np.array(out, dtype=np.float64)


def brute_prefill(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens, query_start, scale, bs,
                  k_scale=None, v_scale=None):
    """Causal chunked prefill, token by token in pure Python (see paged.ref_prefill): query i of
    sequence b sits at position n_b - C_b + i and attends positions 0 .. that position."""
    qd = _scalar_decoder(q_dtype)
    kd = _scalar_decoder(kv_dtype)
    q = np.asarray(q)
    T, H_q, d = q.shape
    kflat = np.asarray(k_pool).reshape(-1)
    vflat = np.asarray(v_pool).reshape(-1)
    NB, H_kv = k_pool.shape[0], k_pool.shape[1]
    X = k_pool.shape[4]
    G = H_q // H_kv
    sc = float(np.float32(scale))
    out = np.zeros((T, H_q, d))
    for b in range(len(query_start) - 1):
        n = int(context_lens[b])
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        for r in range(r0, r1):
            pos = n - (r1 - r0) + (r - r0)
            for h in range(H_q):
                g = h // G
                ks = float(np.float32(k_scale[g])) if kv_dtype == "e4m3" else 1.0
                vs = float(np.float32(v_scale[g])) if kv_dtype == "e4m3" else 1.0
                qv = [qd(q[r, h, i]) for i in range(d)]
                weights, vrows = [], []
                for t in range(pos + 1):
                    blk = int(block_tables[b][t // bs])
                    off = t % bs
                    krow = [kd(kflat[(((blk * H_kv + g) * (d // X) + i // X) * bs + off) * X + i % X]) * ks
                            for i in range(d)]
                    vrows.append([kd(vflat[((blk * H_kv + g) * d + i) * bs + off]) * vs for i in range(d)])
                    weights.append(math.exp(sc * math.fsum(a * c for a, c in zip(qv, krow))))
                den = math.fsum(weights)
                out[r, h] = [math.fsum(w * vr[i] for w, vr in zip(weights, vrows)) / den for i in range(d)]
    return out

