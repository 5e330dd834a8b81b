"""Pins of whole-block eviction, the StreamingLLM sink + window rule and the masked decode
(oracle side, CPU only).

"Paged Attention and KV Cache Fragmentation", section "A fragmentation problem that paging
itself creates: block-level eviction mismatch": eviction of whole blocks keeps the paged
structure; StreamingLLM keeps a few attention-sink tokens at the start plus a window of recent
tokens and drops the rest.

The decisive pin streams tokens into a sequence, evicts with the sink + window rule as it grows,
and compares the masked decode over the compacted table with textbook softmax attention over
exactly the first S and the last W tokens of the whole history, computed from the rows directly
(no pool, no table).
"""
import copy

import numpy as np
import pytest

from oracle import AllocModel, Status, brute_decode, empty_pools, ref_append, ref_decode
from oracle.paged import attended
from test_oracle_alloc import _check_invariants


def test_worked_example_streaming_evict():
    # hand-derived: bs 4, 23 tokens in blocks [0..5]; keep 4 sinks and the last 8 tokens
    m = AllocModel(10, 4)
    m.seq_add(0)
    m.append_slots(0, 23)
    assert m.streaming_evict(0, 4, 8) == (Status.OK, 4, 7, 2)
    assert m.blocks[0] == [0, 3, 4, 5] and m.lens[0] == 15
    assert m.stack[-2:] == [2, 1]  # released last to first: the next pops return 1, 2
    assert list(np.nonzero(attended(15, 4, 7))[0]) == [0, 1, 2, 3] + list(range(7, 15))
    # nothing to drop while the sequence is short
    m.seq_add(1)
    m.append_slots(1, 12)
    assert m.streaming_evict(1, 4, 8) == (Status.OK, 0, 0, 0)
    # no sinks: the window start is a plain start offset inside the first kept block
    m.seq_add(2)
    m.append_slots(2, 10)  # blocks 1, 2, 6
    assert m.streaming_evict(2, 0, 5) == (Status.OK, 0, 1, 1)
    assert m.lens[2] == 6
    # the sinks end inside the only (partial) block: nothing to evict, the rest is masked
    m.seq_add(3)
    m.append_slots(3, 3)
    assert m.streaming_evict(3, 2, 0) == (Status.OK, 2, 3, 0)
    assert list(np.nonzero(attended(3, 2, 3))[0]) == [0, 1]
    _check_invariants(m)


def test_evict_blocks_rules():
    m = AllocModel(8, 4)
    m.seq_add(0)
    m.append_slots(0, 14)  # 3 full blocks + 2 tokens
    m.fork(0, 1)
    before = copy.deepcopy((m.stack, m.rc, m.blocks, m.lens))
    assert m.evict_blocks(0, 2, 2) == Status.INVALID_ARG  # block 3 is partly filled
    assert m.evict_blocks(0, -1, 1) == Status.INVALID_ARG
    assert m.evict_blocks(0, 0, -1) == Status.INVALID_ARG
    assert m.evict_blocks(7, 0, 1) == Status.UNKNOWN_SEQ
    assert copy.deepcopy((m.stack, m.rc, m.blocks, m.lens)) == before
    assert m.evict_blocks(0, 1, 2) == Status.OK
    assert m.blocks[0] == [0, 3] and m.lens[0] == 6
    assert m.rc[1] == m.rc[2] == 1 and m.blocks[1] == [0, 1, 2, 3]  # the fork still holds them
    assert m.evict_blocks(0, 0, 0) == Status.OK
    m.swap_out(1)
    assert m.evict_blocks(1, 0, 1) == Status.INVALID_ARG
    _check_invariants(m)


def test_closed_forms_of_the_mask():
    rng = np.random.default_rng(1)
    H, d, bs, n = 1, 8, 4, 11
    k, v = rng.standard_normal((n, H, d)).astype(np.float32), rng.standard_normal((n, H, d)).astype(np.float32)
    kp, vp = ref_append(*empty_pools(3, H, d, bs, "f32"), k, v, "f32", np.arange(n), bs, "f32")
    q = rng.standard_normal((3, H, d)).astype(np.float32)
    tab = np.tile(np.arange(3, dtype=np.int32), (3, 1))
    lens = np.array([n, n, n], np.int32)
    out = ref_decode(q, "f32", kp, vp, "f32", tab, lens, 0.5, bs,
                     sink_lens=np.array([0, 0, 5], np.int32), window_starts=np.array([n - 1, n, 7], np.int32))
    assert np.array_equal(out[0, 0], v[n - 1, 0].astype(np.float64))  # one attended token: its value
    assert not out[1].any()  # nothing attended: zero row
    # sinks 0..4 and window 7..10 with equal keys reduce to the mean of those values
    kp2, vp2 = ref_append(*empty_pools(3, H, d, bs, "f32"), np.repeat(k[:1], n, 0), v, "f32", np.arange(n), bs, "f32")
    o2 = ref_decode(q, "f32", kp2, vp2, "f32", tab, lens, 0.5, bs, sink_lens=np.array([0, 0, 5], np.int32),
                    window_starts=np.array([0, 0, 7], np.int32))
    sel = [0, 1, 2, 3, 4, 7, 8, 9, 10]
    assert np.allclose(o2[2, 0], v[sel, 0].astype(np.float64).mean(0), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_agrees_with_masks(seed):
    rng = np.random.default_rng(40 + seed)
    bs, H_kv, G, d = [1, 2, 3, 16, 4, 8][seed], [1, 2][seed % 2], [1, 2, 4][seed % 3], 8
    B, NB = 3, 40
    lens = rng.integers(1, 30, B).astype(np.int32)
    mb = int(max(-(-lens // bs)))
    tab = np.stack([rng.permutation(NB)[:mb] for _ in range(B)]).astype(np.int32)
    kp, vp = empty_pools(NB, H_kv, d, bs, "f32")
    kp[:] = rng.standard_normal(kp.shape)
    vp[:] = rng.standard_normal(vp.shape)
    q = rng.standard_normal((B, H_kv * G, d)).astype(np.float32)
    sinks = rng.integers(0, 6, B).astype(np.int32)
    wins = np.array([int(rng.integers(0, n + 1)) for n in lens], np.int32)
    a = ref_decode(q, "f32", kp, vp, "f32", tab, lens, 0.3, bs, sink_lens=sinks, window_starts=wins)
    b = brute_decode(q, "f32", kp, vp, "f32", tab, lens, 0.3, bs, sink_lens=sinks, window_starts=wins)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def _textbook(q, K, V, scale):
    """softmax(scale * K q) V for one head, fp64, straight from the selected rows."""
    s = float(np.float32(scale)) * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


@pytest.mark.parametrize("bs,S,W,G", [(4, 4, 8, 1), (16, 4, 64, 2), (8, 0, 20, 4), (2, 3, 5, 1), (16, 20, 33, 2)])
def test_streaming_evict_attends_exactly_the_sinks_and_the_window(bs, S, W, G):
    rng = np.random.default_rng(bs * 131 + S * 7 + W)
    H_kv, d, NB = 2, 16, 64
    H_q = H_kv * G
    m = AllocModel(NB, bs, rng.permutation(NB))
    kp, vp = empty_pools(NB, H_kv, d, bs, "f32")
    kp[:] = np.nan
    vp[:] = np.nan
    m.seq_add(0)
    hist_k, hist_v = [], []
    sink_len, win = 0, 0
    for step in range(12):
        n_new = int(rng.integers(1, 3 * bs))
        st, slots = m.append_slots(0, n_new)
        assert st == Status.OK
        k = rng.standard_normal((n_new, H_kv, d)).astype(np.float32)
        v = rng.standard_normal((n_new, H_kv, d)).astype(np.float32)
        kp, vp = ref_append(kp, vp, k, v, "f32", slots, bs, "f32")
        hist_k.append(k)
        hist_v.append(v)
        if step % 3 == 2:  # evict every few steps, so the window slides over many appends
            st, sink_len, win, freed = m.streaming_evict(0, S, W)
            assert st == Status.OK
            for b in range(NB):  # released blocks nobody holds are poisoned
                if m.rc[b] == 0:
                    kp[b] = np.nan
                    vp[b] = np.nan
        _check_invariants(m)
        hk, hv = np.concatenate(hist_k), np.concatenate(hist_v)
        L = len(hk)
        keep = np.zeros(L, bool)
        if step % 3 == 2 and L > S + W:
            keep[:S] = True
            keep[L - W:] = True
        elif step % 3 == 2:
            keep[:] = True
        else:
            continue
        q = rng.standard_normal((1, H_q, d)).astype(np.float32)
        tab = np.array([m.blocks[0]], np.int32)
        out = ref_decode(q, "f32", kp, vp, "f32", tab, np.array([m.lens[0]], np.int32), 0.25, bs,
                         sink_lens=np.array([sink_len], np.int32), window_starts=np.array([win], np.int32))
        for h in range(H_q):
            g = h // G
            ref = _textbook(q[0, h].astype(np.float64), hk[keep, g].astype(np.float64),
                            hv[keep, g].astype(np.float64), 0.25)
            assert np.allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)
        # the blocks kept are no more than the sinks' blocks plus the window's blocks (+1 straddling)
        assert len(m.blocks[0]) <= -(-S // bs) + -(-W // bs) + 2
