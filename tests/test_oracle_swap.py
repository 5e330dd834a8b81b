"""Pins of block swap-out / swap-in (oracle side, CPU only).

"Paged Attention and KV Cache Fragmentation", section "Offloading paged KV blocks to CPU DRAM
and NVMe": blocks of sequences that are not running move to host memory and come back later;
the paged layout scatters them, so they are gathered into one contiguous buffer on the way
out and scattered into fresh blocks on the way in.

The main pin replays random scripts of add / append (copy-on-write) / fork / free / swap-out /
swap-in with real rows, saving each swapped sequence's gathered staging buffer and restoring it
into whatever blocks swap-in hands out; every live, resident sequence must keep exactly its rows.
"""
import copy

import numpy as np
import pytest

from oracle import (AllocModel, Status, empty_pools, gather_sequence, ref_append, ref_copy_blocks,
                    ref_gather_blocks, ref_scatter_blocks)
from oracle.paged import to_f64
from test_oracle_alloc import _check_invariants

POISON = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}  # NaN in each format


def test_worked_example_swap_out_and_back_into_other_blocks():
    # hand-derived, bs 4, identity free order (stack top = 0)
    m = AllocModel(6, 4)
    m.seq_add("a")
    m.append_slots("a", 6)  # blocks [0, 1]
    m.seq_add("b")
    m.append_slots("b", 3)  # block [2]
    assert m.swap_out("a") == (Status.OK, [0, 1])
    assert m.num_free() == 5 and m.lens["a"] == 6 and m.blocks["a"] == []
    assert m.append_slots("b", 5) == (Status.OK, [11, 0, 1, 2, 3])  # b grows into block 0
    assert m.swap_in("a") == (Status.OK, [1, 3])
    assert m.blocks["a"] == [1, 3] and m.rc[1] == m.rc[3] == 1
    _check_invariants(m)


def test_swapped_sequence_rules_and_atomic_swap_in():
    m = AllocModel(4, 4)
    m.seq_add(0)
    m.append_slots(0, 9)  # 3 blocks
    m.fork(0, 1)
    assert m.swap_out(0)[0] == Status.OK
    assert m.rc[:3] == [1, 1, 1]  # the fork still holds them
    assert m.swap_out(0)[0] == Status.INVALID_ARG
    assert m.append_slots(0, 1)[0] == Status.INVALID_ARG
    assert m.append_slots_cow(0, 1)[0] == Status.INVALID_ARG
    assert m.fork(0, 2) == Status.INVALID_ARG
    assert m.block_tables([0], 4)[0] == Status.INVALID_ARG
    assert m.swap_in(1)[0] == Status.INVALID_ARG  # not swapped out
    assert m.swap_in(9)[0] == Status.UNKNOWN_SEQ
    before = copy.deepcopy((m.stack, m.rc, m.blocks, m.lens, m.swapped))
    assert m.swap_in(0)[0] == Status.OUT_OF_BLOCKS  # needs 3, one free
    assert copy.deepcopy((m.stack, m.rc, m.blocks, m.lens, m.swapped)) == before
    m.free(1)
    assert m.swap_in(0) == (Status.OK, [0, 1, 2])
    assert m.seq_len(0) == (Status.OK, 9)
    m.swap_out(0)
    assert m.free(0) == Status.OK and m.num_free() == 4
    _check_invariants(m)


def test_gather_record_layout_hand_example():
    # fp32 pools, NB 3, one head, d 4 (X = 4), bs 2: a K block is 8 floats, a V block 8 floats
    k, v = empty_pools(3, 1, 4, 2, "f32")
    for b in range(3):
        k[b] = (100 * b + np.arange(8, dtype=np.float32)).reshape(k.shape[1:])
        v[b] = (-100 * b - np.arange(8, dtype=np.float32)).reshape(v.shape[1:])
    st = ref_gather_blocks(k, v, [2, 0])
    assert st.shape == (2, 2, 32) and st.dtype == np.uint8
    assert np.array_equal(st[0, 0].view(np.float32), 200 + np.arange(8, dtype=np.float32))
    assert np.array_equal(st[0, 1].view(np.float32), -200 - np.arange(8, dtype=np.float32))
    assert np.array_equal(st[1, 0].view(np.float32), np.arange(8, dtype=np.float32))
    k2, v2 = ref_scatter_blocks(np.zeros_like(k), np.zeros_like(v), [1, 2], st)
    assert np.array_equal(k2[1], k[2]) and np.array_equal(v2[2], v[0]) and not k2[0].any()


@pytest.mark.parametrize("bs,seed,dtype", [(1, 0, "f32"), (3, 1, "f32"), (4, 2, "bf16"), (16, 3, "e4m3"),
                                           (8, 4, "bf16")])
def test_random_scripts_with_swaps_keep_every_sequence_content(bs, seed, dtype):
    rng = np.random.default_rng(500 + seed)
    H, d, NB = 2, 16, 80
    m = AllocModel(NB, bs, rng.permutation(NB))
    kp, vp = empty_pools(NB, H, d, bs, dtype)
    bits = kp.dtype
    kp[:] = POISON[dtype]
    vp[:] = POISON[dtype]
    content = {}   # seq -> (K rows, V rows) in pool storage format
    staged = {}    # swapped-out seq -> staging buffer
    next_id = 0

    def rows(n):
        if dtype == "f32":
            r = lambda: rng.standard_normal((n, H, d)).astype(np.float32)
        else:
            r = lambda: rng.integers(0, 0x7F if dtype == "e4m3" else 0x7F00, (n, H, d), dtype=bits)
        return r(), r()

    n_swaps = 0
    for _ in range(500):
        live = sorted(content)
        resident = [s for s in live if s not in m.swapped]
        op = rng.random()
        if op < 0.1 or not live:
            m.seq_add(next_id)
            content[next_id] = (np.zeros((0, H, d), kp.dtype), np.zeros((0, H, d), kp.dtype))
            next_id += 1
        elif op < 0.2 and resident:
            p = resident[int(rng.integers(len(resident)))]
            m.fork(p, next_id)
            content[next_id] = content[p]
            next_id += 1
        elif op < 0.3:
            s = live[int(rng.integers(len(live)))]
            m.free(s)
            del content[s]
            staged.pop(s, None)
        elif op < 0.45 and resident:
            s = resident[int(rng.integers(len(resident)))]
            st, blocks = m.swap_out(s)
            assert st == Status.OK
            staged[s] = ref_gather_blocks(kp, vp, blocks)
            n_swaps += 1
            # released blocks nobody else holds may be reused: poison them so a wrong restore shows
            for b in blocks:
                if m.rc[b] == 0:
                    kp[b] = POISON[dtype]
                    vp[b] = POISON[dtype]
        elif op < 0.6 and staged:
            s = sorted(staged)[int(rng.integers(len(staged)))]
            st, blocks = m.swap_in(s)
            if st == Status.OUT_OF_BLOCKS:
                continue
            assert st == Status.OK
            kp, vp = ref_scatter_blocks(kp, vp, blocks, staged.pop(s))
        elif resident:
            s = resident[int(rng.integers(len(resident)))]
            n = int(rng.integers(1, 2 * bs + 2))
            st, slots, copies = m.append_slots_cow(s, n)
            if st == Status.OUT_OF_BLOCKS:
                continue
            assert st == Status.OK
            kp, vp = ref_copy_blocks(kp, vp, copies)
            kr, vr = rows(n)
            kp, vp = ref_append(kp, vp, kr, vr, dtype, slots, bs, dtype, np.ones(H, np.float32),
                                np.ones(H, np.float32))
            content[s] = (np.concatenate([content[s][0], kr]), np.concatenate([content[s][1], vr]))
        _check_invariants(m)
        for s, (kr, vr) in content.items():
            if s in m.swapped or m.lens[s] == 0:
                continue
            n = m.lens[s]
            K, V = gather_sequence(kp, vp, dtype, m.blocks[s], n, bs, np.ones(H), np.ones(H))
            assert np.array_equal(K, to_f64(kr, dtype).transpose(1, 0, 2))
            assert np.array_equal(V, to_f64(vr, dtype).transpose(1, 0, 2))
    assert n_swaps >= 10
