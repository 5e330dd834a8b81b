"""GPU kv_append is bit-exact against the oracle's scatter (and its E4M3 quantisation)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_223_amd as pkv
import workloads
from tests.gpu_helpers import DEV, from_dev, src_dtype, to_dev
from tests.oracle_cases import materialize_with_model, oracle_pools

pytestmark = pytest.mark.gpu


def _gpu_pools(case, mat, include_step=True, chunk=65536):
    spec = case.spec
    ks, vs = oracle.pool_shapes(case.NB, spec.H_kv, spec.d, case.bs, spec.kv_dtype)
    kp = to_dev(workloads.initial_pool_fill(case, "k", ks), spec.kv_dtype)
    vp = to_dev(workloads.initial_pool_fill(case, "v", vs), spec.kv_dtype)
    sd = src_dtype(case)
    k_s = None if case.k_scale is None else torch.from_numpy(case.k_scale).to(DEV)
    v_s = None if case.v_scale is None else torch.from_numpy(case.v_scale).to(DEV)
    parts = [(mat.k_src, mat.v_src, mat.slots)]
    if include_step:
        parts.append((mat.step_k, mat.step_v, mat.step_slots))
    for k, v, s in parts:
        for i in range(0, len(s), chunk):
            pkv.kv_append(to_dev(k[i:i + chunk], sd), to_dev(v[i:i + chunk], sd),
                          torch.from_numpy(np.ascontiguousarray(s[i:i + chunk])).to(DEV), kp, vp, k_s, v_s)
    torch.cuda.synchronize()
    return from_dev(kp), from_dev(vp)


CASES = {
    "tiny_f32": lambda: workloads.tiny_f32(),
    "llama8b_small": lambda: workloads.llama8b_bf16(B=6, lo=1, hi=700),
    "llama70b_small_step": lambda: workloads.llama70b_bf16(B=4, ctx=600, prefix=256),
    "fp8_bs8_quantise": lambda: workloads.mixed_fp8(bs=8, B=6, churn_ops=100, max_prompt=900),
    "fp8_bs32_quantise_nan": lambda: workloads.mixed_fp8(bs=32, B=6, churn_ops=100, max_prompt=900, fill="nan"),
    "llama70b_full_step": lambda: workloads.llama70b_bf16(),
}


@pytest.mark.parametrize("name", list(CASES))
def test_kv_append_bit_exact(name):
    case = CASES[name]()
    mat = materialize_with_model(case)
    kp_ref, vp_ref = oracle_pools(case, mat)
    kp, vp = _gpu_pools(case, mat)
    assert kp.dtype == kp_ref.dtype and kp.shape == kp_ref.shape
    if case.spec.kv_dtype == "f32":  # compare bits (NaN poison included)
        kp, kp_ref, vp, vp_ref = (x.view(np.uint32) for x in (kp, kp_ref, vp, vp_ref))
    assert (kp == kp_ref).all()
    assert (vp == vp_ref).all()


def test_e4m3_copy_and_padding_slots():
    """E4M3 -> E4M3 copies codes; slots < 0 and slots past the pool are skipped."""
    rng = np.random.default_rng(3)
    NB, H, d, bs, T = 5, 2, 64, 8, 12
    ks, vs = oracle.pool_shapes(NB, H, d, bs, "e4m3")
    k0 = rng.integers(0, 256, ks).astype(np.uint8)
    v0 = rng.integers(0, 256, vs).astype(np.uint8)
    k = rng.integers(0, 256, (T, H, d)).astype(np.uint8)
    v = rng.integers(0, 256, (T, H, d)).astype(np.uint8)
    slots = rng.permutation(NB * bs)[:T].astype(np.int64)
    slots[[2, 7]] = -1
    slots[5] = NB * bs + 3  # outside the pool: skipped
    kp, vp = to_dev(k0, "e4m3"), to_dev(v0, "e4m3")
    pkv.kv_append(to_dev(k, "e4m3"), to_dev(v, "e4m3"), torch.from_numpy(slots).to(DEV), kp, vp)
    torch.cuda.synchronize()
    keep = (slots >= 0) & (slots < NB * bs)
    kr, vr = oracle.ref_append(k0, v0, k[keep], v[keep], "e4m3", slots[keep], bs, "e4m3")
    assert (from_dev(kp) == kr).all() and (from_dev(vp) == vr).all()


@pytest.mark.parametrize("scale", [1.0, 0.0173, 3.7e-3, 5e4])
def test_e4m3_quantise_every_bf16_pattern(scale):
    """All 65536 bf16 bit patterns (NaNs, infinities, subnormals included) through the
    bf16 -> E4M3 append, against the oracle's encoder."""
    H, d, bs = 1, 128, 16
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, H, d)
    T = bits.shape[0]
    NB = T // bs
    ks, vs = oracle.pool_shapes(NB, H, d, bs, "e4m3")
    slots = np.arange(T, dtype=np.int64)[::-1].copy()
    sc = np.array([scale], np.float32)
    kp = torch.zeros(ks, dtype=torch.uint8, device=DEV)
    vp = torch.zeros(vs, dtype=torch.uint8, device=DEV)
    flipped = bits[::-1].copy()
    pkv.kv_append(to_dev(bits, "bf16"), to_dev(flipped, "bf16"), torch.from_numpy(slots).to(DEV), kp, vp,
                  torch.from_numpy(sc).to(DEV), torch.from_numpy(sc).to(DEV))
    torch.cuda.synchronize()
    kr, vr = oracle.ref_append(np.zeros(ks, np.uint8), np.zeros(vs, np.uint8), bits, flipped, "bf16", slots, bs,
                               "e4m3", sc, sc)
    assert (from_dev(kp) == kr).all()
    assert (from_dev(vp) == vr).all()
