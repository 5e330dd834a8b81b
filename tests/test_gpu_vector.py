"""GPU parity of the vector decode path on the shapes the matrix-core path takes by default.

pkv_set_decode_path(PKV_DECODE_PATH_VECTOR) sends every decode to the vector kernels (one wave
per group of up to four query heads of one KV head, bf16 pair dot products for bf16 q against
bf16 or E4M3 KV).  Each case is checked against the fp64 oracle at the decode's tolerance (per-row
relative error 2e-3 with bf16 / fp32 KV, 2e-2 with E4M3 KV), including ragged lengths, empty
sequences, NaN-poisoned pools, pieces and their merge, sink + window masks, and the two-call
step.  The setting is restored after every test."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_223_amd as pkv
import workloads
from tests.gpu_helpers import DEV, decode, device_inputs, tol
from tests.oracle_cases import materialize_with_model, oracle_decode, oracle_pools, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def vector_path():
    prev = pkv.set_decode_path(pkv.DECODE_PATH_VECTOR)
    yield
    pkv.set_decode_path(prev)


def _run(case, sinks=None, wins=None):
    mat = materialize_with_model(case)
    kp, vp = oracle_pools(case, mat)
    dev = device_inputs(case, mat, kp, vp)
    if sinks is None:
        got = decode(case, dev)
    else:
        out = pkv.paged_attn_decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["block_tables"],
                                    dev["context_lens"], float(case.scale), dev["k_scale"], dev["v_scale"],
                                    case.max_context_len, sink_lens=torch.from_numpy(sinks).to(DEV),
                                    window_starts=torch.from_numpy(wins).to(DEV))
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
    if sinks is None:
        ref = oracle_decode(case, mat, kp, vp)
    else:
        ref = oracle.ref_decode(case.q, case.spec.q_dtype, kp, vp, case.spec.kv_dtype, mat.block_tables,
                                mat.context_lens, case.scale, case.bs, case.k_scale, case.v_scale,
                                sink_lens=sinks, window_starts=wins)
    err = row_rel_err(got, ref)
    print(f"vector path {case.spec.name} bs={case.bs} B={case.B} max row rel err {err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= tol(case), err
    return got, mat


# (name, B, H_q, H_kv, D, bs, kv dtype, q dtype, lengths): every head-group size of the vector
# kernel (1, 2, 4 and a partial last group), both KV types with bf16 q, D 64 and 128, every
# block size, one-step and many-step segments, empty sequences
SHAPES = [
    ("v_g1_d128_bs16", 4, 8, 8, 128, 16, "bf16", "bf16", [1, 63, 64, 1500]),
    ("v_g2_d128_bs16", 4, 16, 8, 128, 16, "bf16", "bf16", [65, 700, 0, 2049]),
    ("v_g2_d64_bs8", 3, 8, 4, 64, 8, "bf16", "bf16", [1, 40, 513]),
    ("v_g4_d128_bs32", 3, 16, 4, 128, 32, "bf16", "bf16", [33, 4000, 96]),
    ("v_g8_d128_bs16", 2, 64, 8, 128, 16, "bf16", "bf16", [900, 5]),
    ("v_g3_d64_bs16", 2, 6, 2, 64, 16, "bf16", "bf16", [64, 129]),
    ("v_g1_e4m3_bs16", 3, 8, 8, 128, 16, "e4m3", "bf16", [2, 300, 1100]),
    ("v_g2_e4m3_d64_bs32", 3, 8, 4, 64, 32, "e4m3", "bf16", [31, 32, 600]),
    ("v_g8_e4m3_bs16", 2, 64, 8, 128, 16, "e4m3", "bf16", [17, 2500]),
    ("v_g16_e4m3_bs8", 2, 32, 2, 128, 8, "e4m3", "bf16", [77, 1030]),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=[c[0] for c in SHAPES])
def test_vector_path_shapes(cfg):
    name, B, H_q, H_kv, d, bs, kvd, qd, lens = cfg
    got, _ = _run(workloads.custom(name, B, H_q, H_kv, d, bs, kvd, qd, lens, seed=3000 + len(name)))
    for b, n in enumerate(lens):
        if n == 0:
            assert (got[b] == 0).all()


WORKLOADS = {
    "llama70b_small": lambda: workloads.llama70b_bf16(B=4, ctx=600, prefix=256),
    "llama8b_small_nan": lambda: workloads.llama8b_bf16(B=5, lo=1, hi=300, fill="nan"),
    "long_pieces": lambda: workloads.long128k_bf16(B=2, ctx=9000),
    "fp8_bs16": lambda: workloads.mixed_fp8(bs=16, B=8, churn_ops=200, max_prompt=1500),
    "fp8_bs32_nan": lambda: workloads.mixed_fp8(bs=32, B=8, churn_ops=200, max_prompt=1500, fill="nan"),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_vector_path_workloads(name):
    _run(WORKLOADS[name]())


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_vector_path_sinks_and_windows(kv):
    lens = [700, 1, 33, 2000, 64, 95, 1500, 3, 800, 31]
    case = workloads.custom(f"vw_{kv}", 10, 32, 8, 128, 16, kv, "bf16", lens, 90)
    rng = np.random.default_rng(6)
    sinks, wins = [], []
    for i, n in enumerate(lens):  # plain windows, sinks + windows, nothing masked, everything masked
        kind = i % 4
        s = [0, int(rng.integers(1, 40)), 0, 0][kind]
        w = [int(rng.integers(0, n + 1)), int(rng.integers(0, n + 1)), 0, n + 5][kind]
        sinks.append(s)
        wins.append(w)
    sinks, wins = np.array(sinks, np.int32), np.array(wins, np.int32)
    got, mat = _run(case, sinks, wins)
    for b in range(case.B):
        if not oracle.attended(int(mat.context_lens[b]), int(sinks[b]), int(wins[b])).any():
            assert not got[b].any()


def test_vector_and_matrix_paths_agree():
    """The same batch through both paths: each within the oracle tolerance, and within twice that
    of each other."""
    case = workloads.llama70b_bf16(B=6, ctx=1200, prefix=256)
    mat = materialize_with_model(case)
    kp, vp = oracle_pools(case, mat)
    dev = device_inputs(case, mat, kp, vp)
    vec = decode(case, dev)
    pkv.set_decode_path(pkv.DECODE_PATH_AUTO)
    mfma = decode(case, dev)
    ref = oracle_decode(case, mat, kp, vp)
    assert row_rel_err(vec, ref) <= 2e-3 and row_rel_err(mfma, ref) <= 2e-3
    assert row_rel_err(vec, mfma) <= 4e-3
