"""Pins of the oracle's byte arithmetic and waste accounting against figures the pages print."""
import os

import numpy as np

import oracle
import workloads
from tests.oracle_cases import materialize_with_model

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _figures():
    figs = {}
    for line in open(os.path.join(GOLD, "pages_figures.txt")):
        line = line.split("|")[0].split("#")[0].strip()
        if line:
            key, val, _unit = line.split()
            figs[key] = float(val)
    return figs


def test_per_token_footprint_llama70b():
    # 2 (K and V) * 80 layers * 8 KV heads * 128 head dim * 2 bytes
    assert oracle.bytes_per_token(80, 8, 128, 2) == 327_680
    assert oracle.bytes_per_token(1, 1, 1, 1) == 2


def test_128k_footprints_match_printed_figures():
    f = _figures()
    for s, key, exact in ((2, "llama70b_128k_bf16_GB", 42_949_672_960),
                          (1, "llama70b_128k_fp8_GB", 21_474_836_480),
                          (0.5, "llama70b_128k_nvfp4_GB", 10_737_418_240)):
        b = oracle.request_bytes(131_072, 80, 8, 128, s)
        assert b == exact
        assert round(b / 1e9, 1) == f[key]  # decimal GB, one decimal as printed
        assert b / 2**30 == 20 * s  # exactly 40 / 20 / 10 GiB


def test_8k_bill_reading_uses_the_hidden_dimension():
    """The opening section's "something like 20 GB" and "past 640 GB" come out of its own bill
    formula with the model's hidden dimension (64 heads x 128): 21.5 GB and 687 GB.  With the
    8 KV heads of the quantisation section the same request is only 2.7 GB, so the two
    sections disagree; both readings are kept."""
    f = _figures()
    one = oracle.memory_bill(1, 8192, 80, 64 * 128, 2)
    assert one == 21_474_836_480
    assert abs(one / 1e9 - f["llama70b_8k_one_request_GB"]) / f["llama70b_8k_one_request_GB"] < 0.1
    many = oracle.memory_bill(32, 8192, 80, 64 * 128, 2)
    assert many / 1e9 > f["llama70b_8k_32_requests_GB"]
    assert round(many / 1e9, 1) == 687.2
    gqa = oracle.request_bytes(8192, 80, 8, 128, 2)
    assert round(gqa / 1e9, 2) == 2.68


def test_long_context_layer_bytes():
    # 4 sequences x 131072 tokens x 8 KV heads x 128 x 2 (K,V) x 2 bytes, one layer
    assert oracle.kv_bytes_logical([131072] * 4, 8, 128, 2) == 2_147_483_648


def test_shared_prefix_workload_unique_and_logical_bytes():
    case = workloads.llama70b_bf16()
    mat = materialize_with_model(case)
    assert oracle.kv_bytes_logical(mat.context_lens, 8, 128, 2) == 1_073_741_824
    # 14464 distinct blocks of 16 tokens: 128 prefix + 16 x 384 + 16 x 512
    assert oracle.kv_bytes_unique(mat.block_tables, mat.context_lens, 16, 8, 128, 2) == 947_912_704
    assert oracle.kv_bytes_unique(mat.block_tables, mat.context_lens, 16, 8, 128, 2) == 14464 * 16 * 8 * 128 * 4


def test_unique_bytes_counts_partial_blocks_by_use():
    table = np.array([[5, 2], [5, -1]], np.int32)
    # seq0: 20 tokens (block 5 full, block 2 holds 4); seq1: 7 tokens of block 5
    assert oracle.kv_bytes_unique(table, [20, 7], 16, 1, 1, 1) == (16 + 4) * 2
    assert oracle.kv_bytes_logical([20, 7], 1, 1, 1) == 27 * 2


def test_waste_contrast_reproduces_the_pages_shape():
    """Paged allocation loses only last-block tails (pages: under 4 %); a contiguous
    max-length reservation loses most of the slab (pages: 60-80 %)."""
    f = _figures()
    case = workloads.mixed_fp8(bs=16, churn_ops=0)
    lens = case.context_lens
    # mean decode length of the synthetic stand-in for ShareGPT
    dec = np.random.default_rng(5).geometric(1 / f["sharegpt_mean_decode_tokens"], 200_000)
    assert abs(dec.mean() / f["sharegpt_mean_decode_tokens"] - 1) < 0.01
    for bs in (8, 16, 32):
        w = oracle.paged_waste(lens, bs)
        assert w < f["paged_waste_max_pct"] / 100
        # brute force: at most bs-1 empty slots per sequence
        assert w * (-(-lens // bs) * bs).sum() < len(lens) * bs
    capped = np.minimum(lens, 4096)
    w4k = oracle.contiguous_waste(capped, 4096)
    assert f["prior_waste_low_pct"] / 100 <= w4k <= f["prior_waste_high_pct"] / 100 + 0.05
    assert oracle.contiguous_waste(np.minimum(lens, 8192), 8192) > f["prior_waste_high_pct"] / 100
