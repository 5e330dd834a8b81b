"""CPU checks of the C ABI: the library loads, exports every symbol pkv.h declares, and
rejects invalid arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_223_amd as pkv

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 18
    lib = ctypes.CDLL(pkv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pkv.SIGNATURES)


def test_abi_version():
    assert pkv.lib.pkv_abi_version() == 2


def _prototypes():
    """name -> list of parameter types (names dropped, whitespace normalised) from pkv.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"\b(pkv_[a-z0-9_]+)\s*\(([^()]*)\)\s*;", text):
        params = [" ".join(p.split()) for p in m.group(2).split(",")]
        types = []
        for p in params:
            if p == "void":
                continue
            t = re.sub(r"\s*\b[A-Za-z_][A-Za-z0-9_]*$", "", p)  # drop the parameter name
            types.append(t.replace(" *", "*"))
        protos[m.group(1)] = types
    return protos


# The calls of the boundary as the hot-path contract lists them (types in order).
CONTRACT = {
    "pkv_kv_append": "const void* k, const void* v, int src_dtype, const int64_t* slot_mapping, int32_t T, "
                     "void* k_pool, void* v_pool, int pool_dtype, int32_t NB, int32_t bs, int32_t H_kv, int32_t d, "
                     "const float* k_scale, const float* v_scale, void* stream",
    "pkv_decode_workspace_bytes": "int32_t B, int32_t H_q, int32_t d, int32_t max_context_len, int32_t bs",
    "pkv_paged_attn_decode": "float* out, const void* q, int q_dtype, const void* k_pool, const void* v_pool, "
                             "int kv_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq, "
                             "const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H_q, "
                             "int32_t H_kv, int32_t d, int32_t NB, int32_t bs, float scale, const float* k_scale, "
                             "const float* v_scale, void* workspace, size_t workspace_bytes, void* stream",
    "pkv_alloc_create": "int32_t NB, int32_t bs, const int32_t* initial_free_order, pkv_allocator** out",
    "pkv_alloc_destroy": "pkv_allocator* a",
    "pkv_alloc_num_free": "const pkv_allocator* a",
    "pkv_seq_add": "pkv_allocator* a, int64_t seq",
    "pkv_seq_append_slots": "pkv_allocator* a, int64_t seq, int32_t n, int64_t* slots_out",
    "pkv_seq_fork": "pkv_allocator* a, int64_t parent, int64_t child",
    "pkv_seq_free": "pkv_allocator* a, int64_t seq",
    "pkv_seq_len": "const pkv_allocator* a, int64_t seq, int32_t* len",
    "pkv_block_tables": "const pkv_allocator* a, const int64_t* seqs, int32_t n, int32_t max_blocks, "
                        "int32_t* table_out, int32_t* lens_out",
    "pkv_block_refcount": "const pkv_allocator* a, int32_t block",
}


def test_contract_signatures():
    protos = _prototypes()
    for name, params in CONTRACT.items():
        want = [re.sub(r"\s*\b[A-Za-z_][A-Za-z0-9_]*$", "", " ".join(p.split())).replace(" *", "*")
                for p in params.split(",")]
        assert protos[name] == want, (name, protos[name], want)
    assert len(pkv.SIGNATURES["pkv_kv_append"][1]) == 15
    assert len(pkv.SIGNATURES["pkv_paged_attn_decode"][1]) == 22
    assert len(pkv.SIGNATURES["pkv_decode_workspace_bytes"][1]) == 5


def test_python_contract_signatures():
    """The binding's names and argument order as the contract gives them."""
    import inspect
    want = {
        "kv_append": ["k", "v", "slot_mapping", "k_pool", "v_pool", "k_scale", "v_scale"],
        "paged_attn_decode": ["q", "k_pool", "v_pool", "block_tables", "context_lens", "scale", "k_scale", "v_scale",
                              "max_context_len"],
    }
    for fn, names in want.items():
        ps = list(inspect.signature(getattr(pkv, fn)).parameters.values())
        assert [p.name for p in ps[:len(names)]] == names, fn
        for p in ps[len(names):]:
            assert p.kind is inspect.Parameter.KEYWORD_ONLY or p.default is not inspect.Parameter.empty
        for p in ps:
            if p.name in ("k_scale", "v_scale", "max_context_len"):
                assert p.default is None, (fn, p.name)
    assert [p for p in inspect.signature(pkv.Allocator).parameters] == ["NB", "bs", "initial_free_order"]


def test_every_call_cites_a_passage_or_says_design():
    """Each declaration sits under a multi-line comment block that names the page passage
    defining the operation, or says that the call is a design of this library."""
    lines = open(HEADER).read().splitlines()
    cites = ("Paged Attention and KV Cache Fragmentation", "KV Cache Fragmentation", "Design")
    block, doc, inside = [], "", False
    seen = set()
    for ln in lines:
        st = ln.strip()
        if not inside and (st == "/*" or st.startswith("/* ---")):  # a documentation block opens
            inside, block = True, [st]
            continue
        if inside:
            block.append(st)
            if "*/" in st:
                inside, doc = False, " ".join(block)
            continue
        for name in re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", ln):
            if name in pkv.SIGNATURES and name not in seen:
                seen.add(name)
                assert any(c in doc for c in cites), name
    assert seen == set(pkv.SIGNATURES)


def test_status_and_dtype_codes_match_header():
    text = open(HEADER).read()
    for name, val in [("PKV_OK", 0), ("PKV_ERR_INVALID_ARG", -1), ("PKV_ERR_UNSUPPORTED", -2),
                      ("PKV_ERR_OUT_OF_BLOCKS", -3), ("PKV_ERR_UNKNOWN_SEQ", -4), ("PKV_ERR_SHARED_BLOCK", -5),
                      ("PKV_ERR_HIP", -6), ("PKV_F32", 0), ("PKV_BF16", 1), ("PKV_FP8_E4M3", 2),
                      ("PKV_DECODE_PATH_AUTO", pkv.DECODE_PATH_AUTO),
                      ("PKV_DECODE_PATH_VECTOR", pkv.DECODE_PATH_VECTOR)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name
    import oracle
    import workloads
    assert workloads.STATUS_OUT_OF_BLOCKS == pkv.ERR_OUT_OF_BLOCKS == int(oracle.Status.OUT_OF_BLOCKS)
    for s in oracle.Status:
        assert int(s) == getattr(pkv, "OK" if s.name == "OK" else "ERR_" + s.name)


def test_decode_path_setting_round_trips_and_rejects_unknown_values():
    assert pkv.set_decode_path(pkv.DECODE_PATH_VECTOR) == pkv.DECODE_PATH_AUTO
    try:
        assert pkv.lib.pkv_set_decode_path(7) == pkv.ERR_INVALID_ARG
        assert "unknown path" in pkv.last_error()
        with pytest.raises(pkv.PkvError):
            pkv.set_decode_path(-1)
    finally:  # a refused value leaves the setting as it was
        assert pkv.set_decode_path(pkv.DECODE_PATH_AUTO) == pkv.DECODE_PATH_VECTOR
    assert pkv.set_decode_path(pkv.DECODE_PATH_AUTO) == pkv.DECODE_PATH_AUTO


def test_prefill_waves_setting_round_trips_and_rejects_unknown_values():
    assert pkv.set_prefill_waves(12) == 0
    try:
        assert pkv.set_prefill_waves(8) == 12
        assert pkv.lib.pkv_set_prefill_waves(4) == pkv.ERR_INVALID_ARG
        assert "unknown workgroup size" in pkv.last_error()
        with pytest.raises(pkv.PkvError):
            pkv.set_prefill_waves(-1)
    finally:  # a refused value leaves the setting as it was
        assert pkv.set_prefill_waves(0) == 8
    assert pkv.set_prefill_waves(0) == 0


# dummy non-null device pointers: every call below must fail validation before touching them
P = ctypes.c_void_p(0x1000)


def _decode(hinted=None, **kw):
    a = dict(out=P, q=P, q_dtype=pkv.BF16, k=P, v=P, kv=pkv.BF16, tab=P, mb=4, lens=P, mcl=64, B=2, H_q=8, H_kv=2,
             D=128, NB=16, bs=16, scale=0.1, ks=None, vs=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    if hinted is not None:  # the same call with a length-sum hint
        return pkv.lib.pkv_paged_attn_decode_hinted(a["out"], a["q"], a["q_dtype"], a["k"], a["v"], a["kv"], a["tab"],
                                                    a["mb"], a["lens"], a["mcl"], hinted, a["B"], a["H_q"],
                                                    a["H_kv"], a["D"], a["NB"], a["bs"], a["scale"], a["ks"], a["vs"],
                                                    a["ws"], a["wsb"], a["stream"])
    return pkv.lib.pkv_paged_attn_decode(a["out"], a["q"], a["q_dtype"], a["k"], a["v"], a["kv"], a["tab"], a["mb"],
                                         a["lens"], a["mcl"], a["B"], a["H_q"], a["H_kv"], a["D"], a["NB"], a["bs"],
                                         a["scale"], a["ks"], a["vs"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(H_q=6, H_kv=4), pkv.ERR_INVALID_ARG),
    (dict(D=96), pkv.ERR_UNSUPPORTED),
    (dict(bs=12), pkv.ERR_UNSUPPORTED),
    (dict(q_dtype=pkv.FP8_E4M3), pkv.ERR_UNSUPPORTED),
    (dict(kv=7), pkv.ERR_UNSUPPORTED),
    (dict(NB=0), pkv.ERR_INVALID_ARG),
    (dict(mb=0), pkv.ERR_INVALID_ARG),
    (dict(B=-1), pkv.ERR_INVALID_ARG),
    (dict(mcl=-5), pkv.ERR_INVALID_ARG),
    (dict(scale=float("nan")), pkv.ERR_INVALID_ARG),
    (dict(out=None), pkv.ERR_INVALID_ARG),
    (dict(tab=None), pkv.ERR_INVALID_ARG),
    (dict(kv=pkv.FP8_E4M3), pkv.ERR_INVALID_ARG),  # scales missing
    (dict(), pkv.ERR_INVALID_ARG),  # needs a workspace, none given
    (dict(mcl=100000, ws=ctypes.c_void_p(0x1008), wsb=1 << 40), pkv.ERR_INVALID_ARG),  # misaligned
])
def test_decode_rejects_bad_arguments_before_launch(kw, status):
    assert _decode(**kw) == status
    assert pkv.last_error()
    for hint in (-1, 0, 128, 2 ** 63 - 1):  # the hinted entry checks the same arguments
        assert _decode(hinted=hint, **kw) == status
        assert pkv.last_error()


def test_decode_empty_batch_is_a_no_op():
    assert _decode(B=0) == pkv.OK
    assert _decode(hinted=0, B=0) == pkv.OK


def _step(**kw):
    a = dict(out=P, q=P, q_dtype=pkv.BF16, kn=P, vn=P, src=pkv.BF16, slots=P, k=P, v=P, kv=pkv.BF16, tab=P, mb=4,
             lens=P, mcl=64, hint=-1, B=2, H_q=8, H_kv=2, D=128, NB=16, bs=16, scale=0.1, ks=None, vs=None, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return pkv.lib.pkv_decode_step(a["out"], a["q"], a["q_dtype"], a["kn"], a["vn"], a["src"], a["slots"], a["k"],
                                   a["v"], a["kv"], a["tab"], a["mb"], a["lens"], a["mcl"], a["hint"], a["B"],
                                   a["H_q"], a["H_kv"], a["D"], a["NB"], a["bs"], a["scale"], a["ks"], a["vs"],
                                   a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(H_q=6, H_kv=4), pkv.ERR_INVALID_ARG),  # two-call route: refused before the append runs
    (dict(D=96), pkv.ERR_UNSUPPORTED),
    (dict(kv=pkv.FP8_E4M3), pkv.ERR_INVALID_ARG),  # two-call route, scales missing
    (dict(kn=None), pkv.ERR_INVALID_ARG),  # fused route
    (dict(out=None), pkv.ERR_INVALID_ARG),
    (dict(), pkv.ERR_INVALID_ARG),  # needs a workspace, none given
    (dict(hint=1 << 40), pkv.ERR_INVALID_ARG),  # the hint does not lift any check
])
def test_decode_step_rejects_bad_arguments_before_launch(kw, status):
    # the dummy pointers would fail any launch (HIP error); the status shows nothing was launched
    assert _step(**kw) == status
    assert pkv.last_error()


def test_decode_step_empty_batch_is_a_no_op():
    assert _step(B=0) == pkv.OK
    assert _step(B=0, kv=pkv.FP8_E4M3, ks=P, vs=P) == pkv.OK


def _decode_window(**kw):
    a = dict(out=P, q=P, q_dtype=pkv.BF16, k=P, v=P, kv=pkv.BF16, tab=P, mb=4, lens=P, mcl=64, sinks=P, wins=P, B=2,
             H_q=8, H_kv=2, D=128, NB=16, bs=16, scale=0.1, ks=None, vs=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return pkv.lib.pkv_paged_attn_decode_window(
        a["out"], a["q"], a["q_dtype"], a["k"], a["v"], a["kv"], a["tab"], a["mb"], a["lens"], a["mcl"], a["sinks"],
        a["wins"], a["B"], a["H_q"], a["H_kv"], a["D"], a["NB"], a["bs"], a["scale"], a["ks"], a["vs"], a["ws"],
        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(H_q=6, H_kv=4), pkv.ERR_INVALID_ARG),
    (dict(D=96), pkv.ERR_UNSUPPORTED),
    (dict(bs=12), pkv.ERR_UNSUPPORTED),
    (dict(out=None), pkv.ERR_INVALID_ARG),
    (dict(), pkv.ERR_INVALID_ARG),  # needs a workspace, none given
])
def test_decode_window_rejects_bad_arguments_before_launch(kw, status):
    assert _decode_window(**kw) == status
    assert _decode_window(sinks=None, wins=None, **kw) == status


def test_decode_window_empty_batch_is_a_no_op():
    assert _decode_window(B=0) == pkv.OK


def test_workspace_size_covers_both_paths():
    small = pkv.decode_workspace_bytes(4, 64, 128, 200, 16, H_kv=8)
    assert small > 0 and small % 4 == 0  # the matrix-core path always keeps its partial slots
    big = pkv.decode_workspace_bytes(4096, 64, 128, 131072, 32, H_kv=8)  # vector-path splits dominate
    assert big > small
    assert pkv.decode_workspace_bytes(-1, 64, 128, 10, 16, H_kv=8) == 0 and pkv.last_error()
    assert pkv.decode_workspace_bytes(-1, 64, 128, 10, 16) == 0 and pkv.last_error()


def test_workspace_size_without_h_kv_bounds_every_divisor():
    """The contract's query takes no KV head count: its figure is the largest over every H_kv
    that divides H_q, so it serves any of them."""
    for B, H_q, D, mcl, bs in ((4, 64, 128, 200, 16), (4096, 64, 128, 131072, 32), (256, 32, 128, 20000, 8),
                               (3, 6, 64, 77, 8)):
        bound = pkv.decode_workspace_bytes(B, H_q, D, mcl, bs)
        exact = [pkv.decode_workspace_bytes(B, H_q, D, mcl, bs, H_kv=h) for h in range(1, H_q + 1) if H_q % h == 0]
        assert bound == max(exact) and min(exact) > 0


def _append(**kw):
    a = dict(k=P, v=P, src=pkv.BF16, slots=P, T=4, kp=P, vp=P, pool=pkv.BF16, NB=8, bs=16, H=2, D=128, ks=None,
             vs=None, stream=None)
    a.update(kw)
    return pkv.lib.pkv_kv_append(a["k"], a["v"], a["src"], a["slots"], a["T"], a["kp"], a["vp"], a["pool"], a["NB"],
                                 a["bs"], a["H"], a["D"], a["ks"], a["vs"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), pkv.ERR_INVALID_ARG),
    (dict(D=40), pkv.ERR_UNSUPPORTED),
    (dict(src=pkv.F32, pool=pkv.BF16), pkv.ERR_UNSUPPORTED),
    (dict(src=pkv.FP8_E4M3, pool=pkv.BF16), pkv.ERR_UNSUPPORTED),
    (dict(pool=pkv.FP8_E4M3), pkv.ERR_INVALID_ARG),  # quantising needs scales
    (dict(slots=None), pkv.ERR_INVALID_ARG),
    (dict(bs=0), pkv.ERR_INVALID_ARG),
    (dict(src=9), pkv.ERR_INVALID_ARG),
])
def test_append_rejects_bad_arguments_before_launch(kw, status):
    assert _append(**kw) == status


def test_append_zero_tokens_is_a_no_op():
    assert _append(T=0, k=None, v=None, slots=None) == pkv.OK


def _copy_blocks(**kw):
    a = dict(kp=P, vp=P, pool=pkv.BF16, NB=8, bs=16, H=2, D=128, src=P, dst=P, n=3, stream=None)
    a.update(kw)
    return pkv.lib.pkv_copy_blocks(a["kp"], a["vp"], a["pool"], a["NB"], a["bs"], a["H"], a["D"], a["src"],
                                   a["dst"], a["n"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), pkv.ERR_INVALID_ARG),
    (dict(NB=0), pkv.ERR_INVALID_ARG),
    (dict(bs=300), pkv.ERR_INVALID_ARG),
    (dict(pool=5), pkv.ERR_INVALID_ARG),
    (dict(D=40), pkv.ERR_UNSUPPORTED),
    (dict(src=None), pkv.ERR_INVALID_ARG),
    (dict(vp=None), pkv.ERR_INVALID_ARG),
])
def test_copy_blocks_rejects_bad_arguments_before_launch(kw, status):
    assert _copy_blocks(**kw) == status
    assert pkv.last_error()


def test_copy_blocks_zero_pairs_is_a_no_op():
    assert _copy_blocks(n=0, src=None, dst=None) == pkv.OK


def test_cow_append_needs_its_copy_outputs():
    a = pkv.Allocator(4, 4)
    a.seq_add(0)
    out = (ctypes.c_int64 * 2)()
    c = ctypes.c_int32()
    assert pkv.lib.pkv_seq_append_slots_cow(a._h, 0, 2, out, None, ctypes.byref(c), ctypes.byref(c)) == \
        pkv.ERR_INVALID_ARG
    assert pkv.lib.pkv_seq_append_slots_cow(a._h, 7, 2, out, ctypes.byref(c), ctypes.byref(c), ctypes.byref(c)) == \
        pkv.ERR_UNKNOWN_SEQ


def _move(fn, **kw):
    a = dict(kp=P, vp=P, pool=pkv.BF16, NB=8, bs=16, H=2, D=128, blocks=P, n=3, staging=P, stream=None)
    a.update(kw)
    return fn(a["kp"], a["vp"], a["pool"], a["NB"], a["bs"], a["H"], a["D"], a["blocks"], a["n"], a["staging"],
              a["stream"])


@pytest.mark.parametrize("which", ["pkv_gather_blocks", "pkv_scatter_blocks"])
@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), pkv.ERR_INVALID_ARG),
    (dict(bs=0), pkv.ERR_INVALID_ARG),
    (dict(pool=9), pkv.ERR_INVALID_ARG),
    (dict(D=24), pkv.ERR_UNSUPPORTED),
    (dict(blocks=None), pkv.ERR_INVALID_ARG),
    (dict(staging=None), pkv.ERR_INVALID_ARG),
    (dict(staging=ctypes.c_void_p(0x1008)), pkv.ERR_INVALID_ARG),  # not 16-byte aligned
    (dict(kp=None), pkv.ERR_INVALID_ARG),
])
def test_block_moves_reject_bad_arguments_before_launch(which, kw, status):
    assert _move(getattr(pkv.lib, which), **kw) == status
    assert pkv.last_error()


def test_block_moves_zero_blocks_are_no_ops_and_record_size():
    assert _move(pkv.lib.pkv_gather_blocks, n=0, blocks=None, staging=None) == pkv.OK
    assert _move(pkv.lib.pkv_scatter_blocks, n=0, blocks=None, staging=None) == pkv.OK
    assert pkv.lib.pkv_block_record_bytes(pkv.BF16, 16, 8, 128) == 2 * 8 * 128 * 16 * 2
    assert pkv.lib.pkv_block_record_bytes(pkv.FP8_E4M3, 32, 8, 128) == 2 * 8 * 128 * 32
    assert pkv.lib.pkv_block_record_bytes(pkv.BF16, 0, 8, 128) == 0


def test_swap_calls_check_their_outputs():
    a = pkv.Allocator(8, 4)
    a.seq_add(0)
    a.append_slots(0, 9)  # 3 blocks
    n = ctypes.c_int32()
    buf = (ctypes.c_int32 * 2)()
    assert pkv.lib.pkv_seq_swap_out(a._h, 0, buf, 2, ctypes.byref(n)) == pkv.ERR_INVALID_ARG  # too small
    assert a.seq_len(0) == (pkv.OK, 9) and a.num_free() == 5  # nothing changed
    assert pkv.lib.pkv_seq_swap_out(a._h, 0, buf, 2, None) == pkv.ERR_INVALID_ARG
    assert pkv.lib.pkv_seq_swap_in(a._h, 5, buf, 2, ctypes.byref(n)) == pkv.ERR_UNKNOWN_SEQ


def _prefill(**kw):
    a = dict(out=P, q=P, q_dtype=pkv.BF16, k=P, v=P, kv=pkv.BF16, tab=P, mb=4, lens=P, qs=P, mq=64, B=2, T=100,
             H_q=8, H_kv=2, D=128, NB=16, bs=16, scale=0.1, ks=None, vs=None, stream=None)
    a.update(kw)
    return pkv.lib.pkv_paged_prefill(a["out"], a["q"], a["q_dtype"], a["k"], a["v"], a["kv"], a["tab"], a["mb"],
                                     a["lens"], a["qs"], a["mq"], a["B"], a["T"], a["H_q"], a["H_kv"], a["D"],
                                     a["NB"], a["bs"], a["scale"], a["ks"], a["vs"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(H_q=6, H_kv=4), pkv.ERR_INVALID_ARG),
    (dict(H_q=6, H_kv=2), pkv.ERR_UNSUPPORTED),   # G = 3 does not divide 16
    (dict(D=256), pkv.ERR_UNSUPPORTED),
    (dict(bs=4), pkv.ERR_UNSUPPORTED),
    (dict(q_dtype=pkv.F32), pkv.ERR_UNSUPPORTED),
    (dict(kv=pkv.F32), pkv.ERR_UNSUPPORTED),
    (dict(T=-1), pkv.ERR_INVALID_ARG),
    (dict(mq=-2), pkv.ERR_INVALID_ARG),
    (dict(scale=float("inf")), pkv.ERR_INVALID_ARG),
    (dict(qs=None), pkv.ERR_INVALID_ARG),
    (dict(kv=pkv.FP8_E4M3), pkv.ERR_INVALID_ARG),  # scales missing
])
def test_prefill_rejects_bad_arguments_before_launch(kw, status):
    assert _prefill(**kw) == status
    assert pkv.last_error()


def test_prefill_empty_is_a_no_op():
    assert _prefill(B=0) == pkv.OK
    assert _prefill(T=0) == pkv.OK



def _decode_noalloc(**kw):
    a = dict(out=P, q=P, q_dtype=pkv.BF16, k=P, v=P, kv=pkv.BF16, tab=P, mb=4, lens=P, mcl=64, B=2, H_q=8, H_kv=2,
             D=128, NB=16, bs=16, scale=0.1, ks=None, vs=None, stream=None)
    a.update(kw)
    return pkv.lib.pkv_paged_attn_decode_noalloc(a["out"], a["q"], a["q_dtype"], a["k"], a["v"], a["kv"], a["tab"],
                                                 a["mb"], a["lens"], a["mcl"], a["B"], a["H_q"], a["H_kv"], a["D"],
                                                 a["NB"], a["bs"], a["scale"], a["ks"], a["vs"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(H_q=6, H_kv=4), pkv.ERR_INVALID_ARG),
    (dict(D=96), pkv.ERR_UNSUPPORTED),
    (dict(bs=12), pkv.ERR_UNSUPPORTED),
    (dict(q=None), pkv.ERR_INVALID_ARG),
    (dict(kv=pkv.FP8_E4M3), pkv.ERR_INVALID_ARG),  # E4M3 without scales
    (dict(scale=float("nan")), pkv.ERR_INVALID_ARG),
    (dict(B=0), pkv.OK),  # nothing to do: no launch, no scratch lookup
])
def test_noalloc_decode_checks_arguments_on_the_host(kw, status):
    assert _decode_noalloc(**kw) == status


def test_noalloc_decode_refuses_sizes_beyond_its_scratch():
    """A batch whose partials need more than the 32 MiB static scratch is refused before any
    launch, with a message that names the workspace call."""
    B, H_q, H_kv, D, mcl, bs = 8192, 64, 8, 128, 131072, 16
    assert pkv.decode_workspace_bytes(B, H_q, D, mcl, bs, H_kv) > 32 << 20
    assert _decode_noalloc(B=B, H_q=H_q, H_kv=H_kv, D=D, mcl=mcl, bs=bs, mb=mcl // bs, NB=1 << 20) == \
        pkv.ERR_INVALID_ARG
    msg = pkv.last_error()
    assert "static" in msg and "workspace" in msg, msg
    # matrix-core path only (what the noalloc call sizes for these shapes): the 70B and 128K layers
    # and the E4M3 mix fit, well inside the limit
    for B, H_kv in ((32, 8), (4, 8), (256, 8)):
        assert (256 * 4 + B * H_kv) * 16 * (128 + 2) * 4 + 256 <= 32 << 20
