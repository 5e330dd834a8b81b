"""paged_kv_cache_223_amd — paged-KV decode attention for AMD MI355X (gfx950).

Thin ctypes binding over libpkv.so (C ABI in include/pkv.h).  This module
only marshals arguments: it checks shapes and dtypes of torch tensors, passes
their device pointers and the current HIP stream, and turns status codes into
exceptions.  Every step of the computation runs in the library's HIP kernels;
if the library is not built, importing this package fails.

    kv_append(k, v, slot_mapping, k_pool, v_pool, k_scale=None, v_scale=None)
    paged_attn_decode(q, k_pool, v_pool, block_tables, context_lens, scale,
                      k_scale=None, v_scale=None, max_context_len=None) -> out
    Allocator(NB, bs, initial_free_order=None)

A max_context_len of None is taken as block_tables.shape[1] * block size, the
longest context the table can describe (no device read).

Pool layout (see pkv.h): K [NB, H_kv, D // X, bs, X], V [NB, H_kv, D, bs],
X = 16 bytes / element size; E4M3 pools are uint8 (or float8_e4m3fn) tensors.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# torch ships its own HIP runtime (libamdhip64.so.7).  It must be the one libpkv.so binds to:
# loading torch first makes the dynamic loader satisfy libpkv's libamdhip64.so.7 dependency
# with torch's already-loaded copy, so device pointers and stream handles mean the same
# thing on both sides.  (Loading libpkv first would pull in a second runtime.)
import torch  # noqa: E402,F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_OUT_OF_BLOCKS, ERR_UNKNOWN_SEQ, ERR_SHARED_BLOCK, ERR_HIP = \
    0, -1, -2, -3, -4, -5, -6
F32, BF16, FP8_E4M3 = 0, 1, 2
ELEM_BYTES = {F32: 4, BF16: 2, FP8_E4M3: 1}
DECODE_PATH_AUTO, DECODE_PATH_VECTOR = 0, 1

# every symbol include/pkv.h declares: name -> (restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_abi_version": (ctypes.c_int, []),
    "pkv_set_decode_path": (ctypes.c_int, [ctypes.c_int]),
    "pkv_set_prefill_waves": (ctypes.c_int, [ctypes.c_int]),
    "pkv_kv_append": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _I32, _P, _P, ctypes.c_int, _I32, _I32, _I32,
                                     _I32, _P, _P, _P]),
    "pkv_copy_blocks": (ctypes.c_int, [_P, _P, ctypes.c_int, _I32, _I32, _I32, _I32, _P, _P, _I32, _P]),
    "pkv_block_record_bytes": (_SZ, [ctypes.c_int, _I32, _I32, _I32]),
    "pkv_gather_blocks": (ctypes.c_int, [_P, _P, ctypes.c_int, _I32, _I32, _I32, _I32, _P, _I32, _P, _P]),
    "pkv_scatter_blocks": (ctypes.c_int, [_P, _P, ctypes.c_int, _I32, _I32, _I32, _I32, _P, _I32, _P, _P]),
    "pkv_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "pkv_decode_workspace_bytes_gqa": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_attn_decode": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _I32, _P, _I32,
                                             _I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P, _P,
                                             _SZ, _P]),
    "pkv_paged_attn_decode_noalloc": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _I32, _P, _I32,
                                                     _I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P,
                                                     _P]),
    "pkv_paged_attn_decode_hinted": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _I32, _P, _I32,
                                                    ctypes.c_int64, _I32, _I32, _I32, _I32, _I32, _I32,
                                                    ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "pkv_paged_attn_decode_window": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _I32, _P,
                                                    _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                                    ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "pkv_decode_step": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P, _P, ctypes.c_int, _P,
                                       _I32, _P, _I32, ctypes.c_int64, _I32, _I32, _I32, _I32, _I32, _I32,
                                       ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "pkv_paged_prefill": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _I32, _P, _P, _I32, _I32,
                                         _I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P, _P]),
    "pkv_alloc_create": (ctypes.c_int, [_I32, _I32, _P, ctypes.POINTER(_P)]),
    "pkv_alloc_destroy": (None, [_P]),
    "pkv_alloc_num_free": (_I32, [_P]),
    "pkv_seq_add": (ctypes.c_int, [_P, _I64]),
    "pkv_seq_append_slots": (ctypes.c_int, [_P, _I64, _I32, _P]),
    "pkv_seq_append_slots_cow": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P, _P]),
    "pkv_seq_fork": (ctypes.c_int, [_P, _I64, _I64]),
    "pkv_seq_free": (ctypes.c_int, [_P, _I64]),
    "pkv_seq_swap_out": (ctypes.c_int, [_P, _I64, _P, _I32, _P]),
    "pkv_seq_swap_in": (ctypes.c_int, [_P, _I64, _P, _I32, _P]),
    "pkv_seq_evict_blocks": (ctypes.c_int, [_P, _I64, _I32, _I32]),
    "pkv_seq_streaming_evict": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "pkv_seq_len": (ctypes.c_int, [_P, _I64, _P]),
    "pkv_block_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "pkv_block_refcount": (_I32, [_P, _I32]),
    "pkv_stream_read_sink_floats": (_SZ, [_SZ]),
    "pkv_stream_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "pkv_copy": (ctypes.c_int, [_P, _P, _SZ, _P]),
}


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                p = line.split()[-1] if line.strip() else ""
                if "libamdhip64.so" in p:
                    paths.add(os.path.realpath(p))
    except OSError:
        pass
    return paths


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_cache_223_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(rts)}); import torch before anything that "
                          "loads /opt/rocm's libamdhip64, so that libpkv.so shares torch's runtime")
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pkv status {status}: {msg}")
        self.status = status


def last_error() -> str:
    return (lib.pkv_last_error() or b"").decode()


def _check(st: int):
    if st != OK:
        raise PkvError(st, last_error())


def set_decode_path(path: int) -> int:
    """Process-wide decode kernel choice (DECODE_PATH_AUTO or DECODE_PATH_VECTOR); returns the previous one."""
    st = lib.pkv_set_decode_path(int(path))
    if st < 0:
        raise PkvError(st, last_error())
    return st


def set_prefill_waves(nw: int) -> int:
    """Process-wide prefill workgroup size (0 = automatic, 8 or 12 waves); returns the previous one."""
    st = lib.pkv_set_prefill_waves(int(nw))
    if st < 0:
        raise PkvError(st, last_error())
    return st


# ---------------------------------------------------------------------------
# device ops
# ---------------------------------------------------------------------------
def _torch():
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def pool_shapes(NB: int, H_kv: int, D: int, bs: int, kv_dtype: int):
    X = 16 // ELEM_BYTES[kv_dtype]
    if D % X:
        raise ValueError(f"D={D} is not a multiple of {X}")
    return (NB, H_kv, D // X, bs, X), (NB, H_kv, D, bs)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dev(*ts):
    """Every tensor on the current GPU (the calls launch on its current stream), contiguous."""
    cur = None
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensor is not on a GPU")
            if cur is None:
                cur = _torch().cuda.current_device()
            if t.device.index != cur:
                raise ValueError(f"tensor is on cuda:{t.device.index}, the current device is cuda:{cur}")
            if not t.is_contiguous():
                raise ValueError("tensor is not contiguous")


def _pool_dims(k_pool, v_pool):
    kv = dtype_code(k_pool)
    if dtype_code(v_pool) != kv:
        raise TypeError("k_pool and v_pool dtypes differ")
    if k_pool.dim() != 5 or v_pool.dim() != 4:
        raise ValueError("k_pool must be [NB, H_kv, D/X, bs, X] and v_pool [NB, H_kv, D, bs]")
    NB, H_kv, DX, bs, X = k_pool.shape
    D = DX * X
    if X != 16 // ELEM_BYTES[kv] or tuple(v_pool.shape) != (NB, H_kv, D, bs):
        raise ValueError(f"pool shapes {tuple(k_pool.shape)} / {tuple(v_pool.shape)} do not match the layout")
    return kv, NB, H_kv, D, bs


def kv_append(k, v, slot_mapping, k_pool, v_pool, k_scale=None, v_scale=None):
    """Write k[t], v[t] ([T, H_kv, D]) into slot slot_mapping[t] (int64; < 0 skipped)."""
    torch = _torch()
    _dev(k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    src = dtype_code(k)
    if dtype_code(v) != src or k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (H_kv, D):
        raise ValueError("k and v must both be [T, H_kv, D] of one dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (k.shape[0],):
        raise ValueError("slot_mapping must be int64 [T]")
    for s in (k_scale, v_scale):
        if s is not None and (s.dtype != torch.float32 or s.shape != (H_kv,)):
            raise ValueError("scales must be fp32 [H_kv]")
    _check(lib.pkv_kv_append(_ptr(k), _ptr(v), src, _ptr(slot_mapping), k.shape[0], _ptr(k_pool), _ptr(v_pool),
                             kv, NB, bs, H_kv, D, _ptr(k_scale), _ptr(v_scale), _stream()))


def copy_blocks(k_pool, v_pool, src, dst):
    """Block dst[i] of both pools becomes a copy of block src[i] (int32 device tensors [n])."""
    torch = _torch()
    _dev(k_pool, v_pool, src, dst)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.dim() != 1 or src.shape != dst.shape:
        raise ValueError("src and dst must be int32 [n] of one length")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    _check(lib.pkv_copy_blocks(_ptr(k_pool), _ptr(v_pool), kv, NB, bs, H_kv, D, _ptr(src), _ptr(dst),
                               src.shape[0], _stream()))


def _staging_ok(t):
    return t.is_cuda or t.is_pinned()


def gather_blocks(k_pool, v_pool, blocks, out=None, pinned=False):
    """Pack blocks[i] (int32 device tensor [n]) of both pools into record i of a staging buffer
    (uint8 [n, 2, block bytes]: K block then V block).  `out` may be a device tensor or a pinned
    host tensor (written directly by the kernel); without it one is allocated, pinned host memory
    if `pinned`, else on the pools' device."""
    torch = _torch()
    _dev(k_pool, v_pool, blocks)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    if blocks.dtype != torch.int32 or blocks.dim() != 1 or not blocks.is_contiguous():
        raise ValueError("blocks must be a contiguous int32 [n] tensor")
    n, rec = blocks.shape[0], int(lib.pkv_block_record_bytes(kv, bs, H_kv, D))
    if out is None:
        out = (torch.empty((n, 2, rec // 2), dtype=torch.uint8, pin_memory=True) if pinned
               else torch.empty((n, 2, rec // 2), dtype=torch.uint8, device=k_pool.device))
    if out.dtype != torch.uint8 or tuple(out.shape) != (n, 2, rec // 2) or not out.is_contiguous() \
            or not _staging_ok(out):
        raise ValueError(f"staging must be a contiguous uint8 [{n}, 2, {rec // 2}] device or pinned tensor")
    _check(lib.pkv_gather_blocks(_ptr(k_pool), _ptr(v_pool), kv, NB, bs, H_kv, D, _ptr(blocks), n, _ptr(out),
                                 _stream()))
    return out


def scatter_blocks(k_pool, v_pool, blocks, staging):
    """Unpack record i of `staging` (as gather_blocks makes it; device or pinned host) into block
    blocks[i] (int32 device tensor [n]) of both pools."""
    torch = _torch()
    _dev(k_pool, v_pool, blocks)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    if blocks.dtype != torch.int32 or blocks.dim() != 1 or not blocks.is_contiguous():
        raise ValueError("blocks must be a contiguous int32 [n] tensor")
    n, rec = blocks.shape[0], int(lib.pkv_block_record_bytes(kv, bs, H_kv, D))
    if staging.dtype != torch.uint8 or tuple(staging.shape) != (n, 2, rec // 2) or not staging.is_contiguous() \
            or not _staging_ok(staging):
        raise ValueError(f"staging must be a contiguous uint8 [{n}, 2, {rec // 2}] device or pinned tensor")
    _check(lib.pkv_scatter_blocks(_ptr(k_pool), _ptr(v_pool), kv, NB, bs, H_kv, D, _ptr(blocks), n,
                                  _ptr(staging), _stream()))


def decode_workspace_bytes(B: int, H_q: int, D: int, max_context_len: int, bs: int, H_kv: int | None = None) -> int:
    """Scratch bytes of a decode call (pkv_decode_workspace_bytes; with H_kv, the exact figure
    for that KV head count, pkv_decode_workspace_bytes_gqa)."""
    if H_kv is None:
        return int(lib.pkv_decode_workspace_bytes(B, H_q, D, max_context_len, bs))
    return int(lib.pkv_decode_workspace_bytes_gqa(B, H_q, H_kv, D, max_context_len, bs))


def decode_workspace(B: int, H_q: int, D: int, max_context_len: int, bs: int, H_kv: int | None = None,
                     device="cuda"):
    """A workspace for these sizes (zero-filled once; the library needs no initialisation, and
    zeros rule out even the 2^-32 chance of a stray arrival-counter token)."""
    n = decode_workspace_bytes(B, H_q, D, max_context_len, bs, H_kv)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _max_context_len(max_context_len, block_tables, bs: int) -> int:
    """The host's bound on the batch's context lengths; None: what the table can describe."""
    return int(block_tables.shape[1]) * int(bs) if max_context_len is None else int(max_context_len)


_ws_cache = {}


def _cached_workspace(device, need: int):
    """Workspace reused by calls that pass none, one per (device, stream): calls on one stream run
    in order, so they may share it; calls on different streams get their own.  It is allocated
    while that stream is current, so torch's allocator orders its eventual reuse on that stream."""
    torch = _torch()
    key = (device.type, device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def paged_attn_decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, k_scale=None, v_scale=None,
                      max_context_len: int | None = None, *, out=None, workspace=None, sink_lens=None,
                      window_starts=None, sum_context_lens: int = -1):
    """Decode attention of one query token per sequence over its paged KV; fp32 [B, H_q, D].
    max_context_len: host bound on context_lens (None: block_tables.shape[1] * block size).
    With sink_lens and/or window_starts (int32 [B]) sequence b attends only t < sink_lens[b] or
    t >= window_starts[b] (pkv_paged_attn_decode_window).  sum_context_lens: the host's sum of
    context_lens (-1 unknown); it only chooses the work split (pkv_paged_attn_decode_hinted)."""
    torch = _torch()
    _dev(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, workspace, sink_lens, window_starts)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [B, H_q, D]")
    B, H_q, _ = q.shape
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    for t in (context_lens, sink_lens, window_starts):
        if t is not None and (t.dtype != torch.int32 or t.shape != (B,)):
            raise ValueError("context_lens, sink_lens and window_starts must be int32 [B]")
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, H_q, D):
        raise ValueError("out must be fp32 [B, H_q, D]")
    max_context_len = _max_context_len(max_context_len, block_tables, bs)
    need = decode_workspace_bytes(B, H_q, D, max_context_len, bs, H_kv)
    if workspace is None and need:
        workspace = _cached_workspace(q.device, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if sink_lens is None and window_starts is None and sum_context_lens >= 0:
        _check(lib.pkv_paged_attn_decode_hinted(
            _ptr(out), _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), kv, _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), int(max_context_len), int(sum_context_lens), B, H_q, H_kv,
            D, NB, bs, float(scale), _ptr(k_scale), _ptr(v_scale), _ptr(workspace), ws_bytes, _stream()))
    elif sink_lens is None and window_starts is None:
        _check(lib.pkv_paged_attn_decode(
            _ptr(out), _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), kv, _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), int(max_context_len), B, H_q, H_kv, D, NB, bs,
            float(scale), _ptr(k_scale), _ptr(v_scale), _ptr(workspace), ws_bytes, _stream()))
    else:
        _check(lib.pkv_paged_attn_decode_window(
            _ptr(out), _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), kv, _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), int(max_context_len), _ptr(sink_lens), _ptr(window_starts),
            B, H_q, H_kv, D, NB, bs, float(scale), _ptr(k_scale), _ptr(v_scale), _ptr(workspace), ws_bytes,
            _stream()))
    return out


def paged_attn_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale: float, k_scale=None,
                              v_scale=None, max_context_len: int | None = None, *, out):
    """paged_attn_decode with its partials in the library's static scratch (32 MiB per device):
    for callers that cannot allocate, so `out` (fp32 [B, H_q, D]) must be given.  Calls that
    overlap on one device race on that scratch."""
    torch = _torch()
    _dev(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [B, H_q, D]")
    B, H_q, _ = q.shape
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H_q, D):
        raise ValueError("out must be fp32 [B, H_q, D]")
    max_context_len = _max_context_len(max_context_len, block_tables, bs)
    _check(lib.pkv_paged_attn_decode_noalloc(
        _ptr(out), _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), kv, _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), max_context_len, B, H_q, H_kv, D, NB, bs, float(scale), _ptr(k_scale), _ptr(v_scale),
        _stream()))
    return out


def decode_step(q, k_new, v_new, new_slots, k_pool, v_pool, block_tables, context_lens, scale: float,
                k_scale=None, v_scale=None, max_context_len: int | None = None, *, out=None, workspace=None,
                sum_context_lens: int = -1):
    """kv_append(k_new, v_new, new_slots) then paged_attn_decode, fused into one launch where possible.
    k_new, v_new: [B, H_kv, D] (sequence b's token at its last position); new_slots: int64 [B].
    max_context_len as for paged_attn_decode.  sum_context_lens: the host's sum of context_lens
    (-1 unknown); it only chooses the work split."""
    torch = _torch()
    _dev(q, k_new, v_new, new_slots, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, workspace)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [B, H_q, D]")
    B, H_q, _ = q.shape
    src = dtype_code(k_new)
    if dtype_code(v_new) != src or tuple(k_new.shape) != (B, H_kv, D) or tuple(v_new.shape) != (B, H_kv, D):
        raise ValueError("k_new and v_new must both be [B, H_kv, D] of one dtype")
    if new_slots.dtype != torch.int64 or new_slots.shape != (B,):
        raise ValueError("new_slots must be int64 [B]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, H_q, D):
        raise ValueError("out must be fp32 [B, H_q, D]")
    max_context_len = _max_context_len(max_context_len, block_tables, bs)
    need = decode_workspace_bytes(B, H_q, D, max_context_len, bs, H_kv)
    if workspace is None and need:
        workspace = _cached_workspace(q.device, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_decode_step(_ptr(out), _ptr(q), dtype_code(q), _ptr(k_new), _ptr(v_new), src, _ptr(new_slots),
                               _ptr(k_pool), _ptr(v_pool), kv, _ptr(block_tables), block_tables.shape[1],
                               _ptr(context_lens), int(max_context_len), int(sum_context_lens), B, H_q, H_kv, D,
                               NB, bs, float(scale), _ptr(k_scale), _ptr(v_scale), _ptr(workspace), ws_bytes,
                               _stream()))
    return out


def paged_prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale: float, max_query_len: int,
                  k_scale=None, v_scale=None, out=None):
    """Causal prefill of the last C_b tokens of each sequence (K/V already appended); q bf16 [T, H_q, D]
    packed by query_start (int32 [B+1]); returns fp32 [T, H_q, D]."""
    torch = _torch()
    _dev(q, k_pool, v_pool, block_tables, context_lens, query_start, k_scale, v_scale, out)
    kv, NB, H_kv, D, bs = _pool_dims(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [T, H_q, D]")
    T, H_q, _ = q.shape
    B = block_tables.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    if query_start.dtype != torch.int32 or query_start.shape != (B + 1,):
        raise ValueError("query_start must be int32 [B + 1]")
    if out is None:
        out = torch.empty((T, H_q, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (T, H_q, D):
        raise ValueError("out must be fp32 [T, H_q, D]")
    _check(lib.pkv_paged_prefill(_ptr(out), _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), kv,
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), _ptr(query_start),
                                 int(max_query_len), B, T, H_q, H_kv, D, NB, bs, float(scale), _ptr(k_scale),
                                 _ptr(v_scale), _stream()))
    return out


def stream_read(src, sink=None):
    """Read all of `src` (bytes multiple of 16) once; returns the per-workgroup sink."""
    torch = _torch()
    _dev(src)
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(int(lib.pkv_stream_read_sink_floats(nbytes)), dtype=torch.float32, device=src.device)
    _check(lib.pkv_stream_read(_ptr(src), nbytes, _ptr(sink), _stream()))
    return sink


def copy_(dst, src):
    _dev(dst, src)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check(lib.pkv_copy(_ptr(dst), _ptr(src), nbytes, _stream()))


# ---------------------------------------------------------------------------
# host allocator
# ---------------------------------------------------------------------------
class Allocator:
    """Fixed-block free-list allocator with refcounted shared blocks (host only).

    Methods return the C status code (0 = OK) like the C ABI, so scripts can react
    to PKV_ERR_OUT_OF_BLOCKS; append_slots and block_tables also return arrays.
    """

    def __init__(self, NB: int, bs: int, initial_free_order=None):
        self.NB, self.bs = int(NB), int(bs)
        self._lib = lib  # kept for __del__, which may run after module globals are cleared
        self._h = ctypes.c_void_p()
        order = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if order.shape != (self.NB,):
                raise ValueError("initial_free_order must have NB entries")
        _check(lib.pkv_alloc_create(self.NB, self.bs, order.ctypes.data if order is not None else None,
                                    ctypes.byref(self._h)))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pkv_alloc_destroy(h)
            self._h = None

    def num_free(self) -> int:
        return int(lib.pkv_alloc_num_free(self._h))

    def seq_add(self, seq) -> int:
        return int(lib.pkv_seq_add(self._h, int(seq)))

    def append_slots(self, seq, n: int):
        out = np.empty(max(int(n), 0), np.int64)
        st = int(lib.pkv_seq_append_slots(self._h, int(seq), int(n), out.ctypes.data if n > 0 else None))
        return st, (out if st == OK else None)

    def append_slots_cow(self, seq, n: int):
        """(status, slots, copies): copies is a list of (src_block, dst_block) pairs (0 or 1) to run
        through copy_blocks before the new tokens are appended."""
        out = np.empty(max(int(n), 0), np.int64)
        src, dst, cnt = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        st = int(lib.pkv_seq_append_slots_cow(self._h, int(seq), int(n), out.ctypes.data if n > 0 else None,
                                              ctypes.byref(src), ctypes.byref(dst), ctypes.byref(cnt)))
        if st != OK:
            return st, None, None
        return st, out, ([(src.value, dst.value)] if cnt.value else [])

    def fork(self, parent, child) -> int:
        return int(lib.pkv_seq_fork(self._h, int(parent), int(child)))

    def free(self, seq) -> int:
        return int(lib.pkv_seq_free(self._h, int(seq)))

    def swap_out(self, seq):
        """(status, blocks): the sequence's blocks in logical order, now released."""
        return self._swap(lib.pkv_seq_swap_out, seq)

    def swap_in(self, seq):
        """(status, blocks): fresh blocks for the swapped-out sequence, in logical order."""
        return self._swap(lib.pkv_seq_swap_in, seq)

    def _swap(self, fn, seq):
        st, n = self.seq_len(seq)
        if st != OK:
            return st, None
        cap = max(-(-n // self.bs), 1)
        out = np.empty(cap, np.int32)
        cnt = ctypes.c_int32()
        st = int(fn(self._h, int(seq), out.ctypes.data, cap, ctypes.byref(cnt)))
        return st, (out[:cnt.value].copy() if st == OK else None)

    def evict_blocks(self, seq, first: int, count: int) -> int:
        return int(lib.pkv_seq_evict_blocks(self._h, int(seq), int(first), int(count)))

    def streaming_evict(self, seq, sink_tokens: int, window_tokens: int):
        """(status, sink_len, window_start, evicted_blocks) for paged_attn_decode's masks."""
        sl, ws, ev = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        st = int(lib.pkv_seq_streaming_evict(self._h, int(seq), int(sink_tokens), int(window_tokens),
                                             ctypes.byref(sl), ctypes.byref(ws), ctypes.byref(ev)))
        return (st, sl.value, ws.value, ev.value) if st == OK else (st, None, None, None)

    def seq_len(self, seq):
        n = ctypes.c_int32()
        st = int(lib.pkv_seq_len(self._h, int(seq), ctypes.byref(n)))
        return st, (n.value if st == OK else None)

    def block_tables(self, seqs, max_blocks: int):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        table = np.empty((len(s), int(max_blocks)), np.int32)
        lens = np.empty(len(s), np.int32)
        st = int(lib.pkv_block_tables(self._h, s.ctypes.data, len(s), int(max_blocks), table.ctypes.data,
                                      lens.ctypes.data))
        return st, (table if st == OK else None), (lens if st == OK else None)

    def refcount(self, block: int) -> int:
        return int(lib.pkv_block_refcount(self._h, int(block)))


__all__ = ["lib", "LIB_PATH", "PkvError", "last_error", "kv_append", "copy_blocks", "gather_blocks",
           "scatter_blocks", "paged_attn_decode", "paged_attn_decode_noalloc", "paged_prefill", "decode_step",
           "decode_workspace_bytes",
           "decode_workspace",
           "pool_shapes", "dtype_code", "stream_read", "copy_", "Allocator", "SIGNATURES",
           "set_decode_path", "DECODE_PATH_AUTO", "DECODE_PATH_VECTOR", "set_prefill_waves",
           "F32", "BF16", "FP8_E4M3"]
