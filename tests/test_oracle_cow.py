"""Pins of the copy-on-write append and the block copy (oracle side, CPU only).

"Paged Attention and KV Cache Fragmentation", section "How PagedAttention maps an OS
concept onto GPU memory": sequences that share a prefix or are beam-search branches
point at the same physical blocks and diverge only where their content differs.
"KV Cache Fragmentation" field guide, section "Why it matters": forks are cheap.

The decisive pin replays random fork / append / free scripts with real token rows through
the scatter and the block copy, and checks that every live sequence still holds exactly the
rows it was given: a copy in the wrong direction, a missed copy, a copy after the write or a
write into a block another sequence still reads all fail it.
"""
import copy

import numpy as np
import pytest

from oracle import AllocModel, Status, empty_pools, gather_sequence, ref_append, ref_copy_blocks
from test_oracle_alloc import _check_invariants


def test_worked_example_fork_then_diverge():
    # hand-derived: bs 4, identity free order
    m = AllocModel(8, 4)
    m.seq_add("a")
    assert m.append_slots_cow("a", 6) == (Status.OK, [0, 1, 2, 3, 4, 5], [])
    assert m.fork("a", "b") == Status.OK
    assert m.rc[:2] == [2, 2]
    # b grows into the shared, partly filled block 1: it takes block 2 and copies 1 -> 2
    assert m.append_slots_cow("b", 1) == (Status.OK, [10], [(1, 2)])
    assert m.blocks["b"] == [0, 2] and m.rc[:3] == [2, 1, 1]
    # a now owns block 1 alone and grows in place
    assert m.append_slots_cow("a", 3) == (Status.OK, [6, 7, 12], [])
    assert m.blocks["a"] == [0, 1, 3]
    # a full shared last block needs no copy: new tokens start a new block
    m.seq_add("c")
    m.append_slots_cow("c", 4)
    m.fork("c", "d")
    st, slots, copies = m.append_slots_cow("d", 2)
    assert st == Status.OK and copies == [] and m.blocks["d"][0] == m.blocks["c"][0]
    _check_invariants(m)


def test_cow_block_counts_towards_the_all_or_nothing_need():
    m = AllocModel(3, 4)
    m.seq_add(0)
    m.append_slots_cow(0, 6)  # blocks 0, 1; one free
    m.fork(0, 1)
    before = copy.deepcopy((m.stack, m.rc, m.blocks, m.lens))
    # growth alone would need 1 block (free: 1), but the copy needs one more
    assert m.append_slots_cow(1, 3)[0] == Status.OUT_OF_BLOCKS
    assert copy.deepcopy((m.stack, m.rc, m.blocks, m.lens)) == before
    assert m.append_slots_cow(1, 2) == (Status.OK, [10, 11], [(1, 2)])
    # zero tokens never copy
    m.fork(1, 2)
    assert m.append_slots_cow(2, 0) == (Status.OK, [], [])


def test_plain_append_still_refuses_and_cow_append_matches_it_when_nothing_is_shared():
    rng = np.random.default_rng(7)
    a, b = AllocModel(64, 8, rng.permutation(64)), None
    b = copy.deepcopy(a)
    for i in range(6):
        a.seq_add(i)
        b.seq_add(i)
    for _ in range(200):
        s, n = int(rng.integers(6)), int(rng.integers(0, 5))
        ra = a.append_slots(s, n)
        rb = b.append_slots_cow(s, n)
        assert ra[0] == rb[0] and ra[1] == rb[1] and rb[2] in (None, [])
    a.fork(0, 99)
    if a.lens[0] % 8:
        assert a.append_slots(99, 1)[0] == Status.SHARED_BLOCK


def test_copy_blocks_copies_whole_blocks_in_order():
    rng = np.random.default_rng(3)
    k, v = empty_pools(6, 2, 32, 4, "bf16")
    k[:] = rng.integers(0, 1 << 16, k.shape, dtype=np.uint16)
    v[:] = rng.integers(0, 1 << 16, v.shape, dtype=np.uint16)
    k2, v2 = ref_copy_blocks(k, v, [(1, 4), (4, 5)])
    assert (k2[4] == k[1]).all() and (v2[4] == v[1]).all()
    assert (k2[5] == k[1]).all() and (v2[5] == v[1]).all()  # pairs apply in order
    for blk in (0, 1, 2, 3):
        assert (k2[blk] == k[blk]).all() and (v2[blk] == v[blk]).all()
    assert not (k2 is k)


@pytest.mark.parametrize("bs,seed", [(1, 0), (2, 1), (4, 2), (8, 3), (16, 4)])
def test_random_beam_scripts_keep_every_sequence_content(bs, seed):
    rng = np.random.default_rng(100 + seed)
    H, d, NB = 2, 16, 96
    m = AllocModel(NB, bs, rng.permutation(NB))
    kp, vp = empty_pools(NB, H, d, bs, "f32")
    kp[:] = np.nan
    vp[:] = np.nan
    content = {}  # seq -> (K rows [n, H, d], V rows)
    next_id = 0

    def new_rows(n):
        return rng.standard_normal((n, H, d)).astype(np.float32), rng.standard_normal((n, H, d)).astype(np.float32)

    for _ in range(400):
        live = sorted(content)
        op = rng.random()
        if op < 0.15 or not live:
            m.seq_add(next_id)
            content[next_id] = (np.zeros((0, H, d), np.float32), np.zeros((0, H, d), np.float32))
            next_id += 1
        elif op < 0.35:
            p = live[int(rng.integers(len(live)))]
            assert m.fork(p, next_id) == Status.OK
            content[next_id] = content[p]
            next_id += 1
        elif op < 0.5:
            s = live[int(rng.integers(len(live)))]
            m.free(s)
            del content[s]
        else:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(1, 2 * bs + 2))
            st, slots, copies = m.append_slots_cow(s, n)
            if st == Status.OUT_OF_BLOCKS:
                continue
            assert st == Status.OK
            kp, vp = ref_copy_blocks(kp, vp, copies)  # the copy first, then the new tokens
            kr, vr = new_rows(n)
            kp, vp = ref_append(kp, vp, kr, vr, "f32", slots, bs, "f32")
            content[s] = (np.concatenate([content[s][0], kr]), np.concatenate([content[s][1], vr]))
        _check_invariants(m)
        for s, (kr, vr) in content.items():
            n = m.lens[s]
            assert n == kr.shape[0]
            if n == 0:
                continue
            K, V = gather_sequence(kp, vp, "f32", m.blocks[s], n, bs)
            assert np.array_equal(K, kr.transpose(1, 0, 2).astype(np.float64))
            assert np.array_equal(V, vr.transpose(1, 0, 2).astype(np.float64))
