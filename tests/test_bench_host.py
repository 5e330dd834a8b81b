"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic bytes of a decode
call, the allocator-waste figure, and the refusal of more than one GPU.

The byte figures are those the pages fix for the 70B shape (Paged Attention and KV Cache
Fragmentation, section "Quantization as a way to stretch paged memory further": 2 x 80 layers x
8 KV heads x 128 dims x s bytes per token): per layer and token, K and V of 8 heads of 128 bf16
values are 4096 bytes.  The workload shares one 2048-token prefix among 16 of 32 sequences, so a
call reads 32 x 8192 - 15 x 2048 = 231424 distinct tokens.
"""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _shared_prefix_tables(B=32, ctx=8192, prefix=2048, n_shared=16, bs=16, seed=5):
    """Block tables of B sequences of ctx tokens; the first n_shared hold the same prefix blocks."""
    rng = np.random.default_rng(seed)
    nb, npre = ctx // bs, prefix // bs
    need = n_shared * (nb - npre) + npre + (B - n_shared) * nb
    ids = rng.permutation(need).astype(np.int32)
    pre, rest = ids[:npre], ids[npre:]
    tables, o = [], 0
    for b in range(B):
        if b < n_shared:
            row = np.concatenate([pre, rest[o:o + nb - npre]])
            o += nb - npre
        else:
            row = rest[o:o + nb]
            o += nb
        tables.append(row)
    return np.stack(tables), np.full(B, ctx, np.int32), need


def test_70b_decode_bytes_count_shared_blocks_once():
    tables, lens, need = _shared_prefix_tables()
    by = bench.algorithmic_bytes(tables, lens, 16, 32, 64, 8, 128, 2, 2, 32, 2)
    assert need == 14464
    assert by["kv_logical"] == 32 * 8192 * 4096 == 1_073_741_824
    assert by["kv_unique"] == (32 * 8192 - 15 * 2048) * 4096 == 947_912_704
    # q (bf16) + fp32 output + one 4-byte table entry per used block + lengths
    other = 32 * 64 * 128 * 2 + 32 * 64 * 128 * 4 + 32 * 512 * 4 + 32 * 4
    assert by["decode"] == 947_912_704 + other
    # this step's 32 rows: bf16 K and V read from the source and written to the pools, plus slots
    assert by["append"] == 32 * 8 * 128 * 2 * (2 + 2) + 32 * 8


def test_partial_last_block_counts_only_attended_tokens():
    # two sequences sharing a 20-token prefix (block 0 full, block 1 holds 4 shared tokens);
    # one reads block 1 to token 20, the other to token 30: block 1 counts 14 tokens once
    tables = np.array([[0, 1, -1], [0, 1, 2]], np.int32)
    lens = np.array([20, 40], np.int32)
    by = bench.algorithmic_bytes(tables, lens, 16, 2, 4, 4, 64, 2, 2, 0, 2)
    per_tok = 4 * 64 * 2 * 2
    assert by["kv_unique"] == (16 + 16 + 8) * per_tok
    assert by["kv_logical"] == 60 * per_tok
    w = bench.block_waste(tables, lens, 16)
    assert w == {"blocks_in_use": 3, "slots": 48, "tokens": 40, "internal_frac": round(1 - 40 / 48, 6)}


def test_70b_blocks_are_full():
    tables, lens, need = _shared_prefix_tables()
    w = bench.block_waste(tables, lens, 16)
    assert w["blocks_in_use"] == need and w["internal_frac"] == 0.0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_steps_per_graph_keeps_the_input_rotation():
    assert bench.steps_per_graph(1, 1) == 1 and bench.steps_per_graph(1, 2) == 1
    assert bench.steps_per_graph(20, 1) == 20 and bench.steps_per_graph(20, 2) == 20
    assert bench.steps_per_graph(7, 2) == 8 and bench.steps_per_graph(2, 3) == 3
    for gs in range(2, 30):
        for n in range(1, 5):
            r = bench.steps_per_graph(gs, n)
            assert r % n == 0 and gs <= r < gs + n
