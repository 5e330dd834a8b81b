"""Test plumbing: turn a seeded workload into oracle-side inputs and expected outputs."""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def materialize_with_model(case: workloads.Case) -> workloads.Materialized:
    alloc = oracle.AllocModel(case.NB, case.bs, case.initial_free_order)
    return workloads.materialize(case, alloc)


def src_dtype(case) -> str:
    return "f32" if case.spec.kv_dtype == "f32" else "bf16"


def oracle_pools(case, mat, include_step=True):
    """Pools holding every stored token (and the step's tokens unless include_step=False)."""
    spec = case.spec
    ks, vs = oracle.pool_shapes(case.NB, spec.H_kv, spec.d, case.bs, spec.kv_dtype)
    kp = workloads.initial_pool_fill(case, "k", ks)
    vp = workloads.initial_pool_fill(case, "v", vs)
    kp, vp = oracle.ref_append(kp, vp, mat.k_src, mat.v_src, src_dtype(case), mat.slots, case.bs,
                               spec.kv_dtype, case.k_scale, case.v_scale)
    if include_step and len(mat.step_slots):
        kp, vp = oracle.ref_append(kp, vp, mat.step_k, mat.step_v, src_dtype(case), mat.step_slots,
                                   case.bs, spec.kv_dtype, case.k_scale, case.v_scale)
    return kp, vp


def oracle_pools_for_rows(case, mat, rows):
    """Zero pools holding only the tokens stored in blocks that `rows` reference (enough for
    the oracle to decode those rows at full size without quantising the whole batch)."""
    spec = case.spec
    used = set()
    for b in rows:
        nb = -(-int(mat.context_lens[b]) // case.bs)
        used.update(int(x) for x in mat.block_tables[b, :nb])
    used = np.array(sorted(used), np.int64)
    kp, vp = oracle.empty_pools(case.NB, spec.H_kv, spec.d, case.bs, spec.kv_dtype)
    for k, v, s in ((mat.k_src, mat.v_src, mat.slots), (mat.step_k, mat.step_v, mat.step_slots)):
        if not len(s):
            continue
        keep = np.isin(np.asarray(s) // case.bs, used)
        kp, vp = oracle.ref_append(kp, vp, k[keep], v[keep], src_dtype(case), s[keep], case.bs, spec.kv_dtype,
                                   case.k_scale, case.v_scale)
    return kp, vp


def oracle_decode(case, mat, kp, vp, rows=None):
    spec = case.spec
    return oracle.ref_decode(case.q, spec.q_dtype, kp, vp, spec.kv_dtype, mat.block_tables,
                             mat.context_lens, case.scale, case.bs, case.k_scale, case.v_scale, rows=rows)


def row_rel_err(out, ref):
    """Per (b, h) row: max |o - o_ref| / max |o_ref|; rows with an all-zero reference use
    the absolute error.  Returns the max over rows."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(rel.max()) if rel.size else 0.0
