"""Pins of the allocator model: the invariants of fixed-size paging, brute-force capacity
checks, LIFO order and error atomicity."""
import copy

import numpy as np
import pytest

from oracle import AllocModel, Status


def _ceil(a, b):
    return -(-a // b)


def _check_invariants(m: AllocModel):
    live = {b for b in range(m.NB) if m.rc[b] > 0}
    assert m.num_free() + len(live) == m.NB
    assert len(set(m.stack)) == len(m.stack) and not (set(m.stack) & live)
    swapped = getattr(m, "swapped", set())  # swapped-out sequences keep their length, hold no blocks
    assert sum(_ceil(m.lens[s], m.bs) for s in m.blocks if s not in swapped) == sum(m.rc)
    for s, blocks in m.blocks.items():
        assert len(blocks) == (0 if s in swapped else _ceil(m.lens[s], m.bs))
    # refcount = number of sequences holding the block
    held = {}
    for blocks in m.blocks.values():
        for b in blocks:
            held[b] = held.get(b, 0) + 1
    assert all(m.rc[b] == held.get(b, 0) for b in range(m.NB))


def _snapshot(m):
    return copy.deepcopy((m.stack, m.rc, m.blocks, m.lens))


def test_pops_follow_initial_order_and_free_restores_logical_order():
    m = AllocModel(8, 4, [5, 1, 7, 0, 2, 6, 3, 4])
    m.seq_add("a")
    st, slots = m.append_slots("a", 9)
    assert st == Status.OK and m.blocks["a"] == [5, 1, 7]
    assert slots == [20, 21, 22, 23, 4, 5, 6, 7, 28]
    m.free("a")
    m.seq_add("b")
    _, slots = m.append_slots("b", 12)
    assert m.blocks["b"] == [5, 1, 7]


def test_growth_takes_blocks_only_at_block_boundaries():
    m = AllocModel(4, 16)
    m.seq_add(1)
    for n in range(1, 49):
        free_before = m.num_free()
        st, slots = m.append_slots(1, 1)
        assert st == Status.OK
        assert free_before - m.num_free() == (1 if (n - 1) % 16 == 0 else 0)
        assert slots[0] == m.blocks[1][(n - 1) // 16] * 16 + (n - 1) % 16


def test_out_of_blocks_is_atomic_and_exactly_at_capacity():
    m = AllocModel(5, 4)
    m.seq_add(0)
    assert m.append_slots(0, 6)[0] == Status.OK  # 2 blocks, 3 free
    snap = _snapshot(m)
    assert m.append_slots(0, 2 + 12 + 1)[0] == Status.OUT_OF_BLOCKS  # needs 4
    assert _snapshot(m) == snap
    assert m.append_slots(0, 2 + 12)[0] == Status.OK  # needs exactly 3
    assert m.num_free() == 0


def test_fork_shares_blocks_and_refuses_growth_into_shared_partial_block():
    m = AllocModel(10, 4)
    m.seq_add("p")
    m.append_slots("p", 6)
    assert m.fork("p", "c") == Status.OK
    assert m.blocks["c"] == m.blocks["p"] and all(m.rc[b] == 2 for b in m.blocks["p"])
    snap = _snapshot(m)
    assert m.append_slots("c", 1)[0] == Status.SHARED_BLOCK
    assert _snapshot(m) == snap
    assert m.append_slots("c", 0)[0] == Status.OK
    # a full shared prefix can be extended: the next token opens a fresh private block
    m2 = AllocModel(10, 4)
    m2.seq_add("p")
    m2.append_slots("p", 8)
    m2.fork("p", "c")
    st, slots = m2.append_slots("c", 1)
    assert st == Status.OK and m2.rc[m2.blocks["c"][-1]] == 1 and slots[0] // 4 == m2.blocks["c"][-1]
    m2.free("p")
    assert all(m2.rc[b] == 1 for b in m2.blocks["c"])


def test_error_codes():
    m = AllocModel(4, 4)
    assert m.append_slots("x", 1)[0] == Status.UNKNOWN_SEQ
    assert m.free("x") == Status.UNKNOWN_SEQ
    assert m.fork("x", "y") == Status.UNKNOWN_SEQ
    m.seq_add("x")
    assert m.seq_add("x") == Status.INVALID_ARG
    assert m.fork("x", "x") == Status.INVALID_ARG
    assert m.append_slots("x", -1)[0] == Status.INVALID_ARG
    m.append_slots("x", 9)
    assert m.block_tables(["x"], 2)[0] == Status.INVALID_ARG
    st, t, lens = m.block_tables(["x"], 4)
    assert st == Status.OK and t[0, 3] == -1 and lens[0] == 9
    with pytest.raises(ValueError):
        AllocModel(3, 4, [0, 1, 1])


@pytest.mark.parametrize("seed", range(5))
def test_random_ops_keep_invariants_and_never_fragment(seed):
    rng = np.random.default_rng(seed)
    NB, bs = 37, [1, 4, 16, 8, 3][seed]
    m = AllocModel(NB, bs, rng.permutation(NB))
    live, nid = [], 0
    for _ in range(3000):
        r = rng.random()
        if r < 0.35 or not live:
            m.seq_add(nid)
            live.append(nid)
            nid += 1
        elif r < 0.7:
            s = live[rng.integers(len(live))]
            n = int(rng.integers(0, 3 * bs + 2))
            L = m.lens[s]
            need = _ceil(L + n, bs) - _ceil(L, bs)
            shared = n > 0 and L % bs and m.rc[m.blocks[s][-1]] > 1
            snap = _snapshot(m)
            st, _ = m.append_slots(s, n)
            if shared:
                assert st == Status.SHARED_BLOCK and _snapshot(m) == snap
            else:
                # a freed block always fits: success iff enough blocks are free, wherever they are
                assert (st == Status.OK) == (need <= len(snap[0]))
                if st != Status.OK:
                    assert _snapshot(m) == snap
        elif r < 0.8:
            s = live[rng.integers(len(live))]
            m.fork(s, nid)
            live.append(nid)
            nid += 1
        else:
            s = live.pop(rng.integers(len(live)))
            m.free(s)
        _check_invariants(m)
    for s in live:
        m.free(s)
    assert m.num_free() == NB and sum(m.rc) == 0
