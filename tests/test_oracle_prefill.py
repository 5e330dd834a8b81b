"""Pins of the causal chunked prefill oracle (CPU only).

Library pin: torch's scaled_dot_product_attention in fp64 on the unpaged data, with its causal
flag (a whole prompt) or an explicit causal mask offset by the earlier context (a later chunk).
Cross-pins: the chunk's last query equals the decode of the whole sequence; one chunk equals two;
a pure-Python brute force agrees on tiny cases.
"""
import numpy as np
import pytest
import torch

from oracle import (brute_prefill, empty_pools, gather_sequence, ref_append, ref_decode, ref_prefill)


def _paged(rng, lens, H_kv, d, bs, dtype="f32", NB=None):
    """Pools holding sequences of the given lengths at scattered blocks, plus tables and rows."""
    nblk = [-(-n // bs) for n in lens]
    NB = NB or sum(nblk) + 5
    perm = rng.permutation(NB)
    tab = np.full((len(lens), max(nblk)), -1, np.int32)
    rows, slots, at = [], [], 0
    for b, n in enumerate(lens):
        tab[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += nblk[b]
        rows.append((rng.standard_normal((n, H_kv, d)).astype(np.float32),
                     rng.standard_normal((n, H_kv, d)).astype(np.float32)))
        slots.append(tab[b, np.arange(n) // bs].astype(np.int64) * bs + np.arange(n) % bs)
    kp, vp = empty_pools(NB, H_kv, d, bs, dtype)
    kp[:] = np.nan
    vp[:] = np.nan
    kp, vp = ref_append(kp, vp, np.concatenate([r[0] for r in rows]), np.concatenate([r[1] for r in rows]),
                        "f32", np.concatenate(slots), bs, dtype)
    return kp, vp, tab, rows


@pytest.mark.parametrize("G,bs,lens,chunks", [(1, 16, [40, 17], [40, 17]), (4, 8, [64, 100, 5], [20, 100, 1]),
                                               (8, 3, [31, 9], [7, 9]), (2, 32, [129], [64])])
def test_prefill_equals_torch_sdpa_in_fp64(G, bs, lens, chunks):
    rng = np.random.default_rng(G * 10 + bs)
    H_kv, d = 2, 16
    H_q = G * H_kv
    kp, vp, tab, rows = _paged(rng, lens, H_kv, d, bs)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), H_q, d)).astype(np.float32)
    out = ref_prefill(q, "f32", kp, vp, "f32", tab, np.array(lens, np.int32), qs, 0.3, bs)
    for b, (n, C) in enumerate(zip(lens, chunks)):
        K = torch.from_numpy(rows[b][0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)  # [H_q, n, d]
        V = torch.from_numpy(rows[b][1].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
        Q = torch.from_numpy(q[qs[b]:qs[b + 1]].astype(np.float64)).permute(1, 0, 2)  # [H_q, C, d]
        scale = float(np.float32(0.3))
        if C == n:
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
        else:
            pos = torch.arange(n - C, n)[:, None]
            mask = torch.arange(n)[None, :] <= pos  # [C, n]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        assert np.allclose(out[qs[b]:qs[b + 1]], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_last_query_of_a_chunk_is_the_decode_and_one_chunk_equals_two():
    rng = np.random.default_rng(3)
    H_kv, G, d, bs = 2, 4, 16, 8
    lens = [50, 23, 8]
    kp, vp, tab, rows = _paged(rng, lens, H_kv, d, bs)
    C = [50, 23, 8]
    qs = np.concatenate([[0], np.cumsum(C)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), H_kv * G, d)).astype(np.float32)
    full = ref_prefill(q, "f32", kp, vp, "f32", tab, np.array(lens, np.int32), qs, 0.2, bs)
    last = np.stack([q[qs[b + 1] - 1] for b in range(3)])
    dec = ref_decode(last, "f32", kp, vp, "f32", tab, np.array(lens, np.int32), 0.2, bs)
    for b in range(3):
        assert np.allclose(full[qs[b + 1] - 1], dec[b], rtol=1e-13, atol=1e-13)
    # the same prompts prefilled in two chunks: the first call sees only the first part
    first = [30, 10, 8]
    qs1 = np.concatenate([[0], np.cumsum(first)]).astype(np.int32)
    q1 = np.concatenate([q[qs[b]:qs[b] + first[b]] for b in range(3)])
    o1 = ref_prefill(q1, "f32", kp, vp, "f32", tab, np.array(first, np.int32), qs1, 0.2, bs)
    second = [lens[b] - first[b] for b in range(3)]
    qs2 = np.concatenate([[0], np.cumsum(second)]).astype(np.int32)
    q2 = np.concatenate([q[qs[b] + first[b]:qs[b + 1]] for b in range(3)])
    o2 = ref_prefill(q2, "f32", kp, vp, "f32", tab, np.array(lens, np.int32), qs2, 0.2, bs)
    for b in range(3):
        got = np.concatenate([o1[qs1[b]:qs1[b + 1]], o2[qs2[b]:qs2[b + 1]]])
        assert np.allclose(got, full[qs[b]:qs[b + 1]], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_prefill_agrees(seed):
    rng = np.random.default_rng(70 + seed)
    bs, H_kv, G, d = [1, 3, 16, 4][seed], [1, 2][seed % 2], [1, 2, 4][seed % 3], 4
    lens = [int(x) for x in rng.integers(1, 20, 3)]
    chunks = [int(rng.integers(0, n + 1)) for n in lens]
    kp, vp, tab, rows = _paged(rng, lens, H_kv, d, bs)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), H_kv * G, d)).astype(np.float32)
    a = ref_prefill(q, "f32", kp, vp, "f32", tab, np.array(lens, np.int32), qs, 0.4, bs)
    b = brute_prefill(q, "f32", kp, vp, "f32", tab, np.array(lens, np.int32), qs, 0.4, bs)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_first_token_of_a_prompt_returns_its_value():
    rng = np.random.default_rng(9)
    kp, vp, tab, rows = _paged(rng, [12], 1, 8, 4)
    q = rng.standard_normal((12, 2, 8)).astype(np.float32)
    out = ref_prefill(q, "f32", kp, vp, "f32", tab, np.array([12], np.int32), np.array([0, 12], np.int32), 1.0, 4)
    assert np.array_equal(out[0, 0], rows[0][1][0, 0].astype(np.float64))
    assert np.array_equal(out[0, 1], rows[0][1][0, 0].astype(np.float64))
