"""Pins of the oracle's paged decode: a pure-Python second oracle, torch's SDPA in fp64 on the
unpaged data, closed forms, and the invariants paging implies."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.formats import e4m3_decode
from tests.oracle_cases import materialize_with_model, oracle_decode, oracle_pools

STORE = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}


def _bf16(x):
    return workloads.round_bf16(np.asarray(x, np.float32))


def _rand_store(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return _bf16(x)
    codes = rng.integers(0, 254, size=shape)
    return (codes + (codes >= 0x7F)).astype(np.uint8)


def _tables_from_order(order, lens, bs, max_blocks):
    t = np.full((len(lens), max_blocks), -1, np.int32)
    pos = 0
    for b, n in enumerate(lens):
        nb = -(-n // bs)
        t[b, :nb] = order[pos:pos + nb]
        pos += nb
    return t


def _logical(rng, lens, H, d, dtype):
    return [(_rand_store(rng, (n, H, d), dtype), _rand_store(rng, (n, H, d), dtype)) for n in lens]


def _place(logical, table, NB, H, d, bs, dtype, rng=None, fill=None):
    """Lay logical rows out in pools through `table` (using the oracle's own scatter)."""
    ks, vs = oracle.pool_shapes(NB, H, d, bs, dtype)
    if rng is not None:
        kp, vp = _rand_store(rng, ks, dtype), _rand_store(rng, vs, dtype)
    else:
        kp, vp = oracle.empty_pools(NB, H, d, bs, dtype)
    if fill is not None:
        kp[...] = fill
        vp[...] = fill
    for b, (k, v) in enumerate(logical):
        n = k.shape[0]
        p = np.arange(n)
        slots = table[b][p // bs].astype(np.int64) * bs + p % bs
        kp, vp = oracle.ref_append(kp, vp, k, v, dtype, slots, bs, dtype)
    return kp, vp


def _qrows(rng, B, H_q, d, dtype):
    q = rng.standard_normal((B, H_q, d)).astype(np.float32)
    return q if dtype == "f32" else _bf16(q)


def _q64(q, dtype):
    return oracle.paged.to_f64(q, dtype)


def _scales(rng, H, dtype):
    if dtype != "e4m3":
        return None, None
    return (rng.uniform(0.001, 0.02, H).astype(np.float32), rng.uniform(0.001, 0.02, H).astype(np.float32))


# -------------------------------------------------------------------- second oracle
def test_brute_matches_numpy_on_tiny_workload():
    case = workloads.tiny_f32()
    mat = materialize_with_model(case)
    kp, vp = oracle_pools(case, mat)
    ref = oracle_decode(case, mat, kp, vp)
    brute = oracle.brute_decode(case.q, "f32", kp, vp, "f32", mat.block_tables, mat.context_lens,
                                case.scale, case.bs)
    np.testing.assert_allclose(ref, brute, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_brute_matches_numpy_random_tiny(seed, dtype):
    rng = np.random.default_rng([77, seed, len(dtype)])
    bs = [1, 2, 3, 16][seed % 4]
    G = [1, 2, 4][seed % 3]
    H_kv, d = 2, 16
    B = 3
    lens = rng.integers(1, 41, size=B).tolist()
    if seed == 5:
        lens[1] = 0
    NB = sum(-(-n // bs) for n in lens) + 5
    order = rng.permutation(NB)
    table = _tables_from_order(order, lens, bs, max(1, -(-max(lens) // bs)))
    ks, vs = oracle.pool_shapes(NB, H_kv, d, bs, dtype)
    kp, vp = _rand_store(rng, ks, dtype), _rand_store(rng, vs, dtype)
    qd = "f32" if dtype == "f32" else "bf16"
    q = _qrows(rng, B, H_kv * G, d, qd)
    k_s, v_s = _scales(rng, H_kv, dtype)
    scale = np.float32(1 / math.sqrt(d))
    a = oracle.ref_decode(q, qd, kp, vp, dtype, table, lens, scale, bs, k_s, v_s)
    b = oracle.brute_decode(q, qd, kp, vp, dtype, table, lens, scale, bs, k_s, v_s)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# -------------------------------------------------------------------- library pin
def _sdpa64(q64, K64, V64, scale):
    qt = torch.from_numpy(q64)[None, None, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K64))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(V64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(scale))[0, 0, 0].numpy()


def _expect_sdpa(case, b):
    """torch SDPA in fp64 over sequence b's *unpaged* logical data (from the generator)."""
    spec = case.spec
    k, v = case.logical_kv(b)
    if spec.kv_dtype == "f32":
        K, V = k.astype(np.float64), v.astype(np.float64)
    elif spec.kv_dtype == "bf16":
        K, V = oracle.bf16_bits_to_f64(k), oracle.bf16_bits_to_f64(v)
    else:  # quantise with torch's own fp8 cast (in range: scale = amax / 448)
        def q8(x, s):
            x32 = torch.from_numpy(workloads.bf16_bits_as_f32(x))
            y = (x32 / torch.from_numpy(s)[None, :, None]).to(torch.float8_e4m3fn)
            return y.to(torch.float64).numpy() * s.astype(np.float64)[None, :, None]
        K, V = q8(k, case.k_scale), q8(v, case.v_scale)
    q64 = _q64(case.q, spec.q_dtype)
    G = spec.H_q // spec.H_kv
    out = np.zeros((spec.H_q, spec.d))
    for h in range(spec.H_q):
        out[h] = _sdpa64(q64[b, h], K[:, h // G], V[:, h // G], case.scale)
    return out


@pytest.mark.parametrize("make", [
    lambda: workloads.tiny_f32(),
    lambda: workloads.llama8b_bf16(B=3, lo=1, hi=300),
    lambda: workloads.llama70b_bf16(B=4, ctx=160, prefix=64),
    lambda: workloads.long128k_bf16(B=2, ctx=200),
    lambda: workloads.mixed_fp8(bs=8, B=3, churn_ops=40, max_prompt=200),
])
def test_append_then_decode_matches_sdpa_on_unpaged_data(make):
    case = make()
    mat = materialize_with_model(case)
    kp, vp = oracle_pools(case, mat)
    got = oracle_decode(case, mat, kp, vp)
    for b in range(case.B):
        np.testing.assert_allclose(got[b], _expect_sdpa(case, b), rtol=1e-10, atol=1e-12)


# -------------------------------------------------------------------- closed forms
def _single(q64, Krows, Vrows, bs=4, dtype="f32", scale=0.125):
    """Decode one sequence (one head) holding the given fp32 rows."""
    n, d = Krows.shape
    NB = -(-n // bs) + 2
    table = np.arange(NB - 1, -1, -1, dtype=np.int32)[None, :]
    kp, vp = _place([(Krows[:, None, :].astype(np.float32), Vrows[:, None, :].astype(np.float32))],
                    table, NB, 1, d, bs, dtype)
    return oracle.ref_decode(q64[None, None, :].astype(np.float32), "f32", kp, vp, dtype, table,
                             [n], np.float32(scale), bs)[0, 0]


def test_closed_form_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    k, v, q = (rng.standard_normal((1, 16)).astype(np.float32) for _ in range(3))
    assert (_single(q[0], k, v) == v[0].astype(np.float64)).all()


def test_closed_form_zero_query_averages_values():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((23, 8)).astype(np.float32)
    V = rng.standard_normal((23, 8)).astype(np.float32)
    np.testing.assert_allclose(_single(np.zeros(8, np.float32), K, V), V.astype(np.float64).mean(0),
                               rtol=1e-13, atol=1e-15)
    # scale = 0 has the same effect
    q = rng.standard_normal(8).astype(np.float32)
    np.testing.assert_allclose(_single(q, K, V, scale=0.0), V.astype(np.float64).mean(0), rtol=1e-13, atol=1e-15)


def test_closed_form_equal_keys_average_and_equal_values_return_value():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(8).astype(np.float32)
    K = np.repeat(rng.standard_normal((1, 8)).astype(np.float32), 19, axis=0)
    V = rng.standard_normal((19, 8)).astype(np.float32)
    np.testing.assert_allclose(_single(q, K, V), V.astype(np.float64).mean(0), rtol=1e-13, atol=1e-15)
    K2 = rng.standard_normal((19, 8)).astype(np.float32)
    c = rng.standard_normal((1, 8)).astype(np.float32)
    np.testing.assert_allclose(_single(q, K2, np.repeat(c, 19, axis=0)), c[0].astype(np.float64), rtol=1e-14)


def test_closed_form_dominant_score_selects_its_value():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((30, 8)).astype(np.float32) * 0.01
    V = rng.standard_normal((30, 8)).astype(np.float32)
    q = np.zeros(8, np.float32)
    q[0] = 1.0
    K[17, 0] = 2000.0  # score gap of 250 at scale 1/8
    np.testing.assert_allclose(_single(q, K, V), V[17].astype(np.float64), rtol=1e-12)


def test_closed_form_two_tokens_logistic_weights():
    # n = 2: o = v0 + sigmoid(s1 - s0) (v1 - v0)
    q = np.array([1.0, 0, 0, 0], np.float32)
    K = np.array([[0.5, 0, 0, 0], [2.5, 0, 0, 0]], np.float32)
    V = np.array([[1, 0, 0, 0], [0, 1, 0, 0]], np.float32)
    w1 = 1.0 / (1.0 + math.exp(-(2.5 - 0.5) * 0.125))
    np.testing.assert_allclose(_single(q, K, V, scale=0.125), [1 - w1, w1, 0, 0], rtol=1e-14)


# -------------------------------------------------------------------- invariants
@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_invariant_physical_placement(dtype):
    rng = np.random.default_rng(11)
    bs, H, G, d = 4, 2, 2, 16
    lens = [1, 9, 16, 30]
    NB = sum(-(-n // bs) for n in lens) + 7
    logical = _logical(rng, lens, H, d, dtype)
    qd = "f32" if dtype == "f32" else "bf16"
    q = _qrows(rng, len(lens), H * G, d, qd)
    ks_, vs_ = _scales(rng, H, dtype)
    mb = -(-max(lens) // bs)
    t_id = _tables_from_order(np.arange(NB), lens, bs, mb)
    t_perm = _tables_from_order(rng.permutation(NB), lens, bs, mb)
    outs = []
    for t in (t_id, t_perm):
        kp, vp = _place(logical, t, NB, H, d, bs, dtype, rng=rng)  # unused slots: noise
        outs.append(oracle.ref_decode(q, qd, kp, vp, dtype, t, lens, np.float32(0.25), bs, ks_, vs_))
    assert (outs[0] == outs[1]).all()


def test_invariant_shared_prefix_equals_private_copies():
    rng = np.random.default_rng(12)
    bs, H, d = 4, 2, 8
    prefix = _logical(rng, [12], H, d, "bf16")[0]
    tails = _logical(rng, [5, 9, 0], H, d, "bf16")
    logical = [(np.concatenate([prefix[0], k]), np.concatenate([prefix[1], v])) for k, v in tails]
    lens = [k.shape[0] for k, _ in logical]
    q = _qrows(rng, 3, H, d, "bf16")
    # private copies
    NB = 40
    t_priv = _tables_from_order(rng.permutation(NB), lens, bs, 6)
    kp, vp = _place(logical, t_priv, NB, H, d, bs, "bf16", rng=rng)
    priv = oracle.ref_decode(q, "bf16", kp, vp, "bf16", t_priv, lens, np.float32(0.3), bs)
    # one physical copy of the 3 prefix blocks, shared by all three tables
    order = rng.permutation(NB)
    shared = order[:3]
    t_sh = np.full((3, 6), -1, np.int32)
    pos = 3
    for b, n in enumerate(lens):
        nb = -(-n // bs)
        t_sh[b, :3] = shared
        t_sh[b, 3:nb] = order[pos:pos + nb - 3]
        pos += nb - 3
    kp2, vp2 = _place(logical, t_sh, NB, H, d, bs, "bf16", rng=rng)
    sh = oracle.ref_decode(q, "bf16", kp2, vp2, "bf16", t_sh, lens, np.float32(0.3), bs)
    assert (priv == sh).all()


def test_invariant_block_size_does_not_change_the_result():
    rng = np.random.default_rng(13)
    H, d = 2, 16
    lens = [3, 31, 64]
    logical = _logical(rng, lens, H, d, "bf16")
    q = _qrows(rng, 3, H * 2, d, "bf16")
    outs = []
    for bs in (1, 8, 16, 32):
        NB = sum(-(-n // bs) for n in lens) + 3
        t = _tables_from_order(rng.permutation(NB), lens, bs, -(-max(lens) // bs))
        kp, vp = _place(logical, t, NB, H, d, bs, "bf16", rng=rng)
        outs.append(oracle.ref_decode(q, "bf16", kp, vp, "bf16", t, lens, np.float32(0.25), bs))
    for o in outs[1:]:
        assert (o == outs[0]).all()


def test_invariant_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(14)
    bs, H_kv, G, d = 8, 2, 4, 16
    lens = [5, 40]
    logical = _logical(rng, lens, H_kv, d, "bf16")
    rep = [(np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)) for k, v in logical]
    q = _qrows(rng, 2, H_kv * G, d, "bf16")
    NB = 12
    t = _tables_from_order(rng.permutation(NB), lens, bs, 5)
    kp, vp = _place(logical, t, NB, H_kv, d, bs, "bf16")
    kr, vr = _place(rep, t, NB, H_kv * G, d, bs, "bf16")
    gqa = oracle.ref_decode(q, "bf16", kp, vp, "bf16", t, lens, np.float32(0.25), bs)
    mha = oracle.ref_decode(q, "bf16", kr, vr, "bf16", t, lens, np.float32(0.25), bs)
    assert (gqa == mha).all()


def test_unused_slots_and_table_padding_are_never_read():
    rng = np.random.default_rng(15)
    bs, H, d = 8, 1, 16
    lens = [3, 17, 0]
    logical = _logical(rng, lens, H, d, "f32")
    NB = 9
    t = _tables_from_order(rng.permutation(NB), lens, bs, 4)
    kp, vp = _place(logical, t, NB, H, d, bs, "f32", fill=np.nan)
    q = _qrows(rng, 3, H, d, "f32")
    out = oracle.ref_decode(q, "f32", kp, vp, "f32", t, lens, np.float32(0.25), bs)
    assert np.isfinite(out).all()
    assert (out[2] == 0).all()  # empty context -> zero row
    assert (t[:, -1] == -1).all()
