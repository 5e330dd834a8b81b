"""GPU: the allocation-free decode entry (pkv_paged_attn_decode_noalloc, partials in the library's
static scratch) called through the C ABI gives the bits of pkv_paged_attn_decode with a caller's
workspace, and the oracle's result, on two calls in a row with the second batch smaller (so the
second call runs over whatever the first left in the scratch)."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_223_amd as pkv
import workloads
from tests.gpu_helpers import DEV, device_inputs, tol
from tests.oracle_cases import materialize_with_model, oracle_decode, oracle_pools, row_rel_err

pytestmark = pytest.mark.gpu

KV = {"bf16": pkv.BF16, "e4m3": pkv.FP8_E4M3, "f32": pkv.F32}


def _call(case, dev, noalloc):
    """One decode through the C ABI; returns the fp32 output as numpy."""
    spec = case.spec
    B, H_q, H_kv, D = case.B, spec.H_q, spec.H_kv, spec.d
    kp, vp = dev["k_pool"], dev["v_pool"]
    tab, lens = dev["block_tables"], dev["context_lens"]
    out = torch.full((B, H_q, D), float("nan"), dtype=torch.float32, device=DEV)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = (ptr(out), ptr(dev["q"]), KV[spec.q_dtype], ptr(kp), ptr(vp), KV[spec.kv_dtype], ptr(tab),
              tab.shape[1], ptr(lens), case.max_context_len, B, H_q, H_kv, D, case.NB, case.bs,
              ctypes.c_float(float(case.scale)), ptr(dev["k_scale"]), ptr(dev["v_scale"]))
    if noalloc:
        st = pkv.lib.pkv_paged_attn_decode_noalloc(*common, stream)
    else:
        need = pkv.decode_workspace_bytes(B, H_q, D, case.max_context_len, case.bs, H_kv)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
        st = pkv.lib.pkv_paged_attn_decode(*common, ptr(ws), ws.numel(), stream)
    assert st == pkv.OK, pkv.last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy()


PAIRS = {
    # segments cut into pieces (the piece merge reads the scratch)
    "long_bf16": (lambda: workloads.long128k_bf16(B=3, ctx=9000), lambda: workloads.long128k_bf16(B=1, ctx=2500)),
    # mixed lengths, E4M3 pools
    "mix_e4m3": (lambda: workloads.mixed_fp8(bs=16, B=40, churn_ops=300, max_prompt=6000),
                 lambda: workloads.mixed_fp8(bs=16, B=9, churn_ops=100, max_prompt=2000)),
    # vector path (fp32 q): fixed context splits and their merge
    "vector_f32q": (lambda: workloads.custom("noalloc_vec_a", 3, 8, 2, 128, 16, "bf16", "f32", [5000, 700, 3000], 77),
                    lambda: workloads.custom("noalloc_vec_b", 2, 8, 2, 128, 16, "bf16", "f32", [1300, 40], 78)),
}


@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_matches_workspace_call(name):
    for i, make in enumerate(PAIRS[name]):
        case = make()
        print(f"noalloc {name} call {i}: B={case.B} max len {case.max_context_len}", flush=True)
        mat = materialize_with_model(case)
        kp, vp = oracle_pools(case, mat)
        dev = device_inputs(case, mat, kp, vp)
        got = _call(case, dev, noalloc=True)
        want = _call(case, dev, noalloc=False)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name
        ref = oracle_decode(case, mat, kp, vp)
        assert row_rel_err(got.astype(np.float64), ref) <= tol(case)
