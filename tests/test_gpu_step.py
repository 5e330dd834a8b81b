"""The fused decode step (pkv_decode_step) against kv_append followed by the decode, from the same
pools: the output and the pools are identical bit for bit (the fused piece takes the new token's
operands from the step's rows, the same bits the append stores, and keeps the reduction order), and
the output matches the oracle.  Covers the fused form (bf16 pools, several block sizes, a sequence
without a new token, a captured graph) and the two-launch form (E4M3 pools)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_223_amd as pkv
import workloads
from tests.gpu_helpers import DEV, from_dev, src_dtype, to_dev
from tests.oracle_cases import materialize_with_model, oracle_decode, oracle_pools, row_rel_err

pytestmark = pytest.mark.gpu


def _pre_step_pools(case, mat):
    """Device pools holding everything but the step's tokens (NaN / 0x7F elsewhere)."""
    spec = case.spec
    kvd = {"bf16": pkv.BF16, "e4m3": pkv.FP8_E4M3, "f32": pkv.F32}[spec.kv_dtype]
    ks, vs = pkv.pool_shapes(case.NB, spec.H_kv, spec.d, case.bs, kvd)
    if spec.kv_dtype == "e4m3":
        kp = torch.full(ks, 0x7F, dtype=torch.uint8, device=DEV)
        vp = torch.full(vs, 0x7F, dtype=torch.uint8, device=DEV)
    else:
        kp = torch.full(ks, float("nan"), dtype=torch.bfloat16, device=DEV)
        vp = torch.full(vs, float("nan"), dtype=torch.bfloat16, device=DEV)
    k_s = None if case.k_scale is None else torch.from_numpy(case.k_scale).to(DEV)
    v_s = None if case.v_scale is None else torch.from_numpy(case.v_scale).to(DEV)
    sd = src_dtype(case)
    for i in range(0, len(mat.slots), 65536):
        pkv.kv_append(to_dev(mat.k_src[i:i + 65536], sd), to_dev(mat.v_src[i:i + 65536], sd),
                      torch.from_numpy(np.ascontiguousarray(mat.slots[i:i + 65536])).to(DEV), kp, vp, k_s, v_s)
    torch.cuda.synchronize()
    return kp, vp, k_s, v_s


def _both_ways(case, mat, drop=()):
    """(unfused out, unfused pools, fused out, fused pools); sequences in `drop` append nothing."""
    slots = mat.step_slots.copy()
    lens = mat.context_lens.copy()
    for b in drop:
        slots[b] = -1
        lens[b] -= 1
    q = to_dev(case.q, "bf16")
    sk, sv = to_dev(mat.step_k.reshape(case.B, case.spec.H_kv, case.spec.d), "bf16"), \
        to_dev(mat.step_v.reshape(case.B, case.spec.H_kv, case.spec.d), "bf16")
    tab = torch.from_numpy(mat.block_tables).to(DEV)
    ln = torch.from_numpy(lens).to(DEV)
    sl = torch.from_numpy(slots).to(DEV)
    res = []
    for fused in (False, True):
        kp, vp, k_s, v_s = _pre_step_pools(case, mat)
        if fused:
            out = pkv.decode_step(q, sk, sv, sl, kp, vp, tab, ln, float(case.scale), k_s, v_s, case.max_context_len)
        else:
            pkv.kv_append(sk, sv, sl, kp, vp, k_s, v_s)
            out = pkv.paged_attn_decode(q, kp, vp, tab, ln, float(case.scale), k_s, v_s, case.max_context_len)
        torch.cuda.synchronize()
        res += [out.cpu().numpy(), from_dev(kp), from_dev(vp)]
    return res, lens


def _with_step(case):
    """A custom case whose last token of every sequence is this step's append."""
    steps = []
    for op in list(case.ops):
        if op[0] == "append":
            _, sid, n, (key, start) = op
            case.ops.remove(op)
            if n > 1:
                case.ops.append(("append", sid, n - 1, (key, start)))
            steps.append(("append", sid, 1, (key, start + n - 1)))
    case.step_ops = steps
    return case


CASES = {
    "llama70b_B6_ctx700": lambda: workloads.llama70b_bf16(B=6, ctx=700, prefix=256),
    "llama70b_B3_ctx33": lambda: workloads.llama70b_bf16(B=3, ctx=33, prefix=16),
    "e4m3": lambda: _with_step(workloads.custom("step_e4m3", 4, 64, 8, 128, 16, "e4m3", "bf16",
                                                [300, 17, 1, 128], 91)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_step_equals_append_then_decode_bitwise(name):
    print(f"decode step {name}", flush=True)
    case = CASES[name]()
    mat = materialize_with_model(case)
    (o0, k0, v0, o1, k1, v1), lens = _both_ways(case, mat)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))
    kp, vp = oracle_pools(case, mat)
    ref = oracle_decode(case, mat, kp, vp)
    tol = 2e-2 if case.spec.kv_dtype == "e4m3" else 2e-3
    assert row_rel_err(o1.astype(np.float64), ref) <= tol


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_fused_step_block_sizes_and_a_sequence_without_a_token(bs, kv):
    print(f"fused step bs={bs} {kv}", flush=True)
    case = _with_step(workloads.custom(f"step_bs{bs}_{kv}", 5, 32, 8, 128, bs, kv, "bf16", [1, 40, 97, 500, 33], 92))
    mat = materialize_with_model(case)
    (o0, k0, v0, o1, k1, v1), lens = _both_ways(case, mat, drop=(2,))
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("H_q,H_kv,D,bs", [(32, 2, 64, 8), (4, 4, 128, 32), (16, 8, 64, 16), (48, 3, 128, 16)])
def test_fused_step_head_shapes(H_q, H_kv, D, bs, kv):
    """Head dims 64 and 128 with GQA groups of 16, 1, 2 and 16 (3 KV heads): the fused step's
    operand injection and pool store follow each layout; the result equals append + decode and
    the oracle's."""
    print(f"fused step H_q={H_q} H_kv={H_kv} D={D} bs={bs} {kv}", flush=True)
    case = _with_step(workloads.custom(f"step_{H_q}_{H_kv}_{D}_{bs}_{kv}", 4, H_q, H_kv, D, bs, kv, "bf16",
                                       [3, 70, 257, 1000], 94 + H_q + D))
    mat = materialize_with_model(case)
    (o0, k0, v0, o1, k1, v1), lens = _both_ways(case, mat)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))
    kp, vp = oracle_pools(case, mat)
    assert row_rel_err(o1.astype(np.float64), oracle_decode(case, mat, kp, vp)) <= (2e-2 if kv == "e4m3" else 2e-3)


def test_fused_e4m3_step_saturated_and_subnormal_codes():
    """E4M3 pools, new tokens far outside the scales' range (codes saturate at 448) and far inside
    it (subnormal codes and zeros), and one with a NaN element: the fused step writes the same
    codes as kv_append and attends them in the same way, bit for bit (NaN payloads included)."""
    case = _with_step(workloads.custom("step_e4m3_extremes", 4, 32, 8, 128, 16, "e4m3", "bf16", [9, 64, 130, 700], 95))
    mat = materialize_with_model(case)
    as_f32 = lambda bits: (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    sk = as_f32(mat.step_k).reshape(case.B, 8, 128).copy()
    sv = as_f32(mat.step_v).reshape(case.B, 8, 128).copy()
    sk[0] *= 1e3      # saturates
    sv[1] *= 3e3
    sk[2] *= 1e-4     # subnormal codes and zeros
    sv[2] *= 1e-5
    sk[3, 5, 17] = np.nan
    mat.step_k = workloads.round_bf16(sk.reshape(mat.step_k.shape))
    mat.step_v = workloads.round_bf16(sv.reshape(mat.step_v.shape))
    (o0, k0, v0, o1, k1, v1), lens = _both_ways(case, mat)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))


def test_fused_full_70b_step_and_graph_replay():
    case = workloads.llama70b_bf16()
    mat = materialize_with_model(case)
    (o0, k0, v0, o1, k1, v1), lens = _both_ways(case, mat)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    # replays of a captured fused step equal the eager result
    kp, vp, _, _ = _pre_step_pools(case, mat)
    q = to_dev(case.q, "bf16")
    sk = to_dev(mat.step_k.reshape(case.B, 8, 128), "bf16")
    sv = to_dev(mat.step_v.reshape(case.B, 8, 128), "bf16")
    tab, ln = torch.from_numpy(mat.block_tables).to(DEV), torch.from_numpy(mat.context_lens).to(DEV)
    sl = torch.from_numpy(mat.step_slots).to(DEV)
    out = torch.empty((case.B, 64, 128), dtype=torch.float32, device=DEV)
    ws = pkv.decode_workspace(case.B, 64, 128, case.max_context_len, case.bs, H_kv=8, device=DEV)
    pkv.decode_step(q, sk, sv, sl, kp, vp, tab, ln, float(case.scale), max_context_len=case.max_context_len, out=out, workspace=ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.decode_step(q, sk, sv, sl, kp, vp, tab, ln, float(case.scale), max_context_len=case.max_context_len, out=out,
                        workspace=ws)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), o1.view(np.uint32))
    # with the batch's length sum the plan is the same one piece per segment and the merge
    # launch is skipped: the result is the same, bit for bit, also from a captured graph
    hint = int(mat.context_lens.astype(np.int64).sum())
    kp, vp, _, _ = _pre_step_pools(case, mat)
    pkv.decode_step(q, sk, sv, sl, kp, vp, tab, ln, float(case.scale), max_context_len=case.max_context_len, out=out, workspace=ws,
                    sum_context_lens=hint)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), o1.view(np.uint32))
    assert np.array_equal(from_dev(kp), k1) and np.array_equal(from_dev(vp), v1)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        pkv.decode_step(q, sk, sv, sl, kp, vp, tab, ln, float(case.scale), max_context_len=case.max_context_len, out=out,
                        workspace=ws, sum_context_lens=hint)
    for _ in range(3):
        out.zero_()
        g2.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), o1.view(np.uint32))


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_length_hint_only_chooses_the_split(kv):
    """A batch of very mixed lengths: a hint of 0, or one above B * max_context_len (no sum of
    lengths can be that large, so it is ignored), leaves the planned split unchanged (same bits);
    the largest possible hint still gives the oracle's result."""
    print(f"length hint {kv}", flush=True)
    case = _with_step(workloads.custom(f"hint_{kv}", 6, 32, 8, 128, 16, kv, "bf16", [5000, 30, 1, 700, 2049, 64],
                                       93 + len(kv)))
    mat = materialize_with_model(case)
    q = to_dev(case.q, "bf16")
    sk = to_dev(mat.step_k.reshape(case.B, 8, 128), "bf16")
    sv = to_dev(mat.step_v.reshape(case.B, 8, 128), "bf16")
    tab, ln = torch.from_numpy(mat.block_tables).to(DEV), torch.from_numpy(mat.context_lens).to(DEV)
    sl = torch.from_numpy(mat.step_slots).to(DEV)
    outs = {}
    for hint in (-1, 0, 10 ** 12, case.B * case.max_context_len):
        kp, vp, k_s, v_s = _pre_step_pools(case, mat)
        outs[hint] = pkv.decode_step(q, sk, sv, sl, kp, vp, tab, ln, float(case.scale), k_s, v_s,
                                     case.max_context_len, sum_context_lens=hint).cpu().numpy()
    assert np.array_equal(outs[-1].view(np.uint32), outs[0].view(np.uint32))
    assert np.array_equal(outs[-1].view(np.uint32), outs[10 ** 12].view(np.uint32))
    kp, vp = oracle_pools(case, mat)
    ref = oracle_decode(case, mat, kp, vp)
    tol = 2e-2 if kv == "e4m3" else 2e-3
    for hint, o in outs.items():
        assert np.isfinite(o).all()
        assert row_rel_err(o.astype(np.float64), ref) <= tol, hint


@pytest.mark.parametrize("name", ["uniform", "lying_mixed", "lying_empty"])
def test_uniform_length_sum_loads_early(name):
    """A length sum equal to B * max_context_len lets each workgroup load its likely segment's first
    chunk before its plan (sequences of at most 8 chunks always run in single-piece mode).  With
    every length at the maximum the output equals, bit for bit, the same single-piece step without
    the early loads (sum - 1); a sum that lies about uneven lengths (or a sequence with no tokens,
    which shifts every later segment) still gives the oracle's result and the same bits as without
    the early loads."""
    print(f"early loads {name}", flush=True)
    if name == "uniform":
        case = workloads.llama70b_bf16(B=6, ctx=200, prefix=64)
    elif name == "lying_mixed":
        case = _with_step(workloads.custom("early_mixed", 6, 64, 8, 128, 16, "bf16", "bf16",
                                           [256, 30, 1, 200, 129, 64], 97))
    else:
        case = _with_step(workloads.custom("early_empty", 4, 64, 8, 128, 16, "bf16", "bf16", [200, 1, 200, 200], 98))
    mat = materialize_with_model(case)
    drop = (1,) if name == "lying_empty" else ()
    slots, lens = mat.step_slots.copy(), mat.context_lens.copy()
    for b in drop:  # sequence 1 appends nothing and holds no tokens
        slots[b], lens[b] = -1, 0
    q = to_dev(case.q, "bf16")
    sk = to_dev(mat.step_k.reshape(case.B, 8, 128), "bf16")
    sv = to_dev(mat.step_v.reshape(case.B, 8, 128), "bf16")
    tab, ln = torch.from_numpy(mat.block_tables).to(DEV), torch.from_numpy(lens).to(DEV)
    sl = torch.from_numpy(slots).to(DEV)
    mcl = int(lens.max())
    early = case.B * mcl  # claims every length is the maximum
    outs = {}
    for hint in (early, early - 1):
        kp, vp, k_s, v_s = _pre_step_pools(case, mat)
        outs[hint] = pkv.decode_step(q, sk, sv, sl, kp, vp, tab, ln, float(case.scale), k_s, v_s, mcl,
                                     sum_context_lens=hint).cpu().numpy()
    assert np.array_equal(outs[early].view(np.uint32), outs[early - 1].view(np.uint32))
    if name == "uniform":
        assert int(lens.sum()) == early
    mat.context_lens = lens
    kp, vp = oracle_pools(case, mat)
    ref = oracle_decode(case, mat, kp, vp)
    got = outs[early].astype(np.float64)
    for b in drop:
        assert (got[b] == 0).all()
    keep = [b for b in range(case.B) if b not in drop]
    assert row_rel_err(got[keep], ref[keep]) <= 2e-3


def test_blocks_past_4_gib_of_pool():
    """The same step with its blocks moved near the top of pools larger than 4 GiB (byte offsets
    past 2^32): the fused step's output and pool stores, copy_blocks, the swap gather and the
    prefill give the same bits as in the small pools, and kv_append stores rows there exactly."""
    case = workloads.llama70b_bf16(B=3, ctx=900, prefix=256)
    mat = materialize_with_model(case)
    (o0, k0, v0, o1, k1, v1), lens = _both_ways(case, mat)
    kp, vp, _, _ = _pre_step_pools(case, mat)
    blk_bytes = kp[0].numel() * kp.element_size()
    big_nb = (5 << 30) // blk_bytes + 64  # each pool just over 5 GiB
    used = np.unique(mat.block_tables[mat.block_tables >= 0])
    used = used[used < case.NB]
    remap = np.full(case.NB, -1, np.int64)
    remap[used] = big_nb - 1 - np.arange(len(used))  # the top blocks of the big pools, reversed
    assert remap[used].min() * blk_bytes > (4 << 30)
    print(f"big pools: {big_nb} blocks of {blk_bytes} B, blocks used from {int(remap[used].min())}", flush=True)
    kb = torch.zeros((big_nb,) + tuple(kp.shape[1:]), dtype=kp.dtype, device=DEV)
    vb = torch.zeros((big_nb,) + tuple(vp.shape[1:]), dtype=vp.dtype, device=DEV)
    src = torch.from_numpy(used).to(DEV)
    dst = torch.from_numpy(remap[used]).to(DEV)
    kb.index_copy_(0, dst, kp.index_select(0, src))
    vb.index_copy_(0, dst, vp.index_select(0, src))
    tab = mat.block_tables.copy()
    tab[tab >= 0] = remap[tab[tab >= 0]]
    slots = mat.step_slots.copy()
    slots = remap[slots // case.bs] * case.bs + slots % case.bs
    q = to_dev(case.q, "bf16")
    sk = to_dev(mat.step_k.reshape(case.B, 8, 128), "bf16")
    sv = to_dev(mat.step_v.reshape(case.B, 8, 128), "bf16")
    ln = torch.from_numpy(mat.context_lens).to(DEV)
    out = pkv.decode_step(q, sk, sv, torch.from_numpy(slots).to(DEV), kb, vb, torch.from_numpy(tab).to(DEV), ln,
                          float(case.scale), max_context_len=case.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), o1.view(np.uint32))
    assert np.array_equal(from_dev(kb.index_select(0, dst)), k1[used])
    assert np.array_equal(from_dev(vb.index_select(0, dst)), v1[used])
    # copy_blocks between two high blocks, then the gather of a few high blocks into staging
    a, b = int(remap[used[0]]), int(big_nb - 1 - len(used) - 5)
    pkv.copy_blocks(kb, vb, torch.tensor([a], dtype=torch.int32, device=DEV),
                    torch.tensor([b], dtype=torch.int32, device=DEV))
    st = pkv.gather_blocks(kb, vb, torch.tensor([b, a], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    rec = st.cpu().numpy().reshape(2, 2, -1)
    kraw = from_dev(kb.index_select(0, torch.tensor([a], device=DEV))).reshape(1, -1).view(np.uint8)
    vraw = from_dev(vb.index_select(0, torch.tensor([a], device=DEV))).reshape(1, -1).view(np.uint8)
    assert np.array_equal(rec[0, 0], kraw[0]) and np.array_equal(rec[1, 0], kraw[0])
    assert np.array_equal(rec[0, 1], vraw[0]) and np.array_equal(rec[1, 1], vraw[0])
    # prefill of each sequence's last 5 tokens over the big pools equals that over the small ones
    kp2, vp2, _, _ = _pre_step_pools(case, mat)
    pkv.kv_append(sk, sv, torch.from_numpy(mat.step_slots).to(DEV), kp2, vp2)
    qp = torch.randn((case.B * 5, 64, 128), device=DEV).to(torch.bfloat16)
    qs = torch.arange(0, case.B * 5 + 1, 5, dtype=torch.int32, device=DEV)
    small = pkv.paged_prefill(qp, kp2, vp2, torch.from_numpy(mat.block_tables).to(DEV), ln, qs, float(case.scale), 5)
    big = pkv.paged_prefill(qp, kb, vb, torch.from_numpy(tab).to(DEV), ln, qs, float(case.scale), 5)
    torch.cuda.synchronize()
    assert torch.equal(small.view(torch.int32), big.view(torch.int32))
    # kv_append of a block's worth of rows into a free block past 4 GiB
    c = int(big_nb - 1 - len(used) - 9)
    rows_k = torch.randn((case.bs, 8, 128), device=DEV).to(torch.bfloat16)
    rows_v = torch.randn((case.bs, 8, 128), device=DEV).to(torch.bfloat16)
    hs = torch.arange(c * case.bs, (c + 1) * case.bs, dtype=torch.int64, device=DEV)
    pkv.kv_append(rows_k, rows_v, hs, kb, vb)
    torch.cuda.synchronize()
    vt = from_dev(vb[c])  # [H_kv][D][bs]
    assert np.array_equal(vt.transpose(2, 0, 1), from_dev(rows_v))
    kt = from_dev(kb[c])  # [H_kv][D/8][bs][8]
    assert np.array_equal(kt.transpose(2, 0, 1, 3).reshape(case.bs, 8, 128), from_dev(rows_k))
    del kb, vb
    torch.cuda.empty_cache()
