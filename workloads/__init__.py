"""Seeded synthetic workloads for paged-KV decode attention.

This module only draws random numbers and lays out bookkeeping: it holds none
of the method's arithmetic (no attention, no scatter into a pool, no fp8
encoding, no allocator logic).  Both the CPU oracle and the GPU path take
their inputs from here.

The five workloads follow the shapes the pages discuss: a Llama-3-8B-like
layer, a Llama-3.1-70B-like layer (the footprint arithmetic in "Paged
Attention and KV Cache Fragmentation", section "Quantization as a way to
stretch paged memory further" uses its 80 layers, 8 KV heads and head_dim
128), a 128K-token long-context case, and a mixed-length fp8 batch whose
decode lengths follow the ShareGPT mean of about 415 tokens quoted in the
same page's section "The two fragmentation modes that previous systems failed
to solve".  ShareGPT itself is not available; a geometric distribution with
that mean stands in for it.

Block tables are never written here.  A workload is an *allocation script*
(add / append / fork / free operations on sequences) plus per-sequence
logical token contents.  Any allocator implementing the small interface used
by :func:`materialize` turns the script into slots and block tables, so the
oracle's allocator model and the product allocator can be driven by the very
same script.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Status code an allocator returns when the pool cannot satisfy an append.
# (Value fixed by the C ABI; the churn driver reacts to it.)
STATUS_OK = 0
STATUS_OUT_OF_BLOCKS = -3


@dataclass(frozen=True)
class Spec:
    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    bs: int
    kv_dtype: str  # "f32" | "bf16" | "e4m3"
    q_dtype: str  # "f32" | "bf16"
    seed: int
    desc: str


SPECS = {
    "tiny_f32": Spec("tiny_f32", 4, 4, 4, 64, 16, "f32", "f32", 1001,
                     "tiny fp32: 4 seqs, lens {1,17,33,64}, H_q=H_kv=4, d=64, bs=16, pool of 32 blocks"),
    "llama8b_bf16": Spec("llama8b_bf16", 64, 32, 8, 128, 16, "bf16", "bf16", 1002,
                         "Llama-3-8B-shaped layer: H_q=32, H_kv=8, d=128, bf16, bs=16, batch 64, lens U[128,4096]"),
    "llama70b_bf16": Spec("llama70b_bf16", 32, 64, 8, 128, 16, "bf16", "bf16", 1003,
                          "Llama-3.1-70B-shaped layer: H_q=64, H_kv=8, d=128, bf16, bs=16, batch 32 at 8192, "
                          "16 seqs share a 2048-token prefix, plus 1 appended token per seq"),
    "long128k_bf16": Spec("long128k_bf16", 4, 64, 8, 128, 32, "bf16", "bf16", 1004,
                          "long context: H_q=64, H_kv=8, d=128, bf16, bs=32, batch 4 at 131072, scattered tables"),
    "mixed_fp8": Spec("mixed_fp8", 256, 32, 8, 128, 16, "e4m3", "bf16", 1005,
                      "mixed fp8 KV: e4m3 with per-head fp32 scales, H_q=32, H_kv=8, d=128, batch 256, "
                      "log-normal prompts (median 512) + geometric decode (mean 415), alloc/free churn"),
}


# ----------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------
_Q, _K, _V, _LEN, _TAB, _CHURN, _FILL = range(1, 8)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng([seed, *key])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 samples -> bf16 bit patterns (uint16), round-to-nearest-even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


# ----------------------------------------------------------------------------
# workload description
# ----------------------------------------------------------------------------
@dataclass
class Case:
    spec: Spec
    bs: int
    B: int
    NB: int
    initial_free_order: np.ndarray  # int32 [NB]
    ops: list  # allocation script, see materialize()
    step_ops: list  # the timed step's appends (one token per seq) or []
    seqs: list  # sequence ids of the batch, in batch order
    context_lens: np.ndarray  # int32 [B], after step_ops
    streams: dict  # data stream key -> length (tokens)
    seq_sources: dict  # seq id -> list of (stream key, stream start, logical start, n)
    q: np.ndarray  # [B, H_q, d] fp32 values or bf16 bits (uint16)
    scale: np.float32
    fill: str  # "noise" | "nan": contents of pool slots nobody writes
    k_scale: np.ndarray | None = None  # fp32 [H_kv] (e4m3 only)
    v_scale: np.ndarray | None = None
    _stream_cache: dict = field(default_factory=dict, repr=False)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.B else 0

    @property
    def max_blocks(self) -> int:
        return max(1, -(-self.max_context_len // self.bs))

    def stream_kv(self, key):
        """(K, V) source rows of a data stream: [n, H_kv, d] as fp32 (f32) or bf16 bits."""
        if key not in self._stream_cache:
            self._stream_cache[key] = _gen_stream(self.spec, key, self.streams[key])
        return self._stream_cache[key]

    def logical_kv(self, b: int):
        """Full logical K/V rows [n_b, H_kv, d] of batch entry b (source dtype)."""
        sid = self.seqs[b]
        ks, vs = [], []
        for key, s0, _l0, n in self.seq_sources[sid]:
            k, v = self.stream_kv(key)
            ks.append(k[s0:s0 + n])
            vs.append(v[s0:s0 + n])
        return np.concatenate(ks), np.concatenate(vs)


def _src_dtype(spec: Spec) -> str:
    return "f32" if spec.kv_dtype == "f32" else "bf16"


def _stream_key_id(key) -> int:
    if key == "prefix":
        return 1 << 20
    return int(key)


def _gen_stream(spec: Spec, key, n: int):
    kid = _stream_key_id(key)
    shape = (n, spec.H_kv, spec.d)
    k = _normal(_rng(spec.seed, _K, kid), shape)
    v = _normal(_rng(spec.seed, _V, kid), shape)
    if _src_dtype(spec) == "bf16":
        return round_bf16(k), round_bf16(v)
    return k, v


def _gen_q(spec: Spec, B: int):
    q = _normal(_rng(spec.seed, _Q), (B, spec.H_q, spec.d))
    return q if spec.q_dtype == "f32" else round_bf16(q)


def _blocks(n: int, bs: int) -> int:
    # plain bookkeeping for sizing the pool (not an allocator decision)
    return -(-n // bs)


def _plain_case(spec, bs, lens, NB, fill, seqs=None, step=False):
    """Sequences allocated one after another, each with its own data stream."""
    B = len(lens)
    seqs = list(range(B)) if seqs is None else seqs
    ops, step_ops, streams, sources = [], [], {}, {}
    for b, n in enumerate(lens):
        sid = seqs[b]
        pre = n - 1 if step else n
        ops.append(("add", sid))
        if pre > 0:
            ops.append(("append", sid, pre, (sid, 0)))
        if step:
            step_ops.append(("append", sid, 1, (sid, pre)))
        streams[sid] = n
        sources[sid] = [(sid, 0, 0, n)]
    order = _rng(spec.seed, _TAB).permutation(NB).astype(np.int32)
    return Case(spec=spec, bs=bs, B=B, NB=NB, initial_free_order=order, ops=ops, step_ops=step_ops,
                seqs=seqs, context_lens=np.asarray(lens, np.int32), streams=streams, seq_sources=sources,
                q=_gen_q(spec, B), scale=np.float32(1.0 / math.sqrt(spec.d)), fill=fill)


def tiny_f32(fill="noise"):
    """Workload 1: lens {1,17,33,64}, a 32-block pool handed out in a seeded random order."""
    spec = SPECS["tiny_f32"]
    return _plain_case(spec, spec.bs, [1, 17, 33, 64], 32, fill)


def llama8b_bf16(B=None, lo=128, hi=4096, fill="noise"):
    """Workload 2: lens uniform on [lo, hi], pool 1.2x the total need, shuffled free list."""
    spec = SPECS["llama8b_bf16"]
    B = spec.B if B is None else B
    lens = _rng(spec.seed, _LEN).integers(lo, hi + 1, size=B).tolist()
    need = sum(_blocks(n, spec.bs) for n in lens)
    return _plain_case(spec, spec.bs, lens, math.ceil(1.2 * need), fill)


def llama70b_bf16(B=None, ctx=8192, prefix=2048, n_shared=None, fill="noise"):
    """Workload 3: batch at one context length; the first half of the batch forks from one
    refcounted prefix (same physical blocks); every sequence then appends one token (the step)."""
    spec = SPECS["llama70b_bf16"]
    bs = spec.bs
    B = spec.B if B is None else B
    n_shared = B // 2 if n_shared is None else n_shared
    assert prefix % bs == 0 and prefix < ctx
    ops, step_ops, streams, sources = [], [], {}, {}
    parent = 1 << 30
    if n_shared:
        ops += [("add", parent), ("append", parent, prefix, ("prefix", 0))]
        streams["prefix"] = prefix
        for b in range(n_shared):
            ops.append(("fork", parent, b))
        ops.append(("free", parent))
    for b in range(B):
        if b < n_shared:
            ops.append(("append", b, ctx - 1 - prefix, (b, 0)))
            streams[b] = ctx - prefix
            sources[b] = [("prefix", 0, 0, prefix), (b, 0, prefix, ctx - prefix)]
            step_ops.append(("append", b, 1, (b, ctx - 1 - prefix)))
        else:
            ops += [("add", b), ("append", b, ctx - 1, (b, 0))]
            streams[b] = ctx
            sources[b] = [(b, 0, 0, ctx)]
            step_ops.append(("append", b, 1, (b, ctx - 1)))
    need = (prefix // bs if n_shared else 0) + n_shared * _blocks(ctx - prefix, bs) \
        + (B - n_shared) * _blocks(ctx, bs)
    NB = math.ceil(1.2 * need)
    order = _rng(spec.seed, _TAB).permutation(NB).astype(np.int32)
    return Case(spec=spec, bs=bs, B=B, NB=NB, initial_free_order=order, ops=ops, step_ops=step_ops,
                seqs=list(range(B)), context_lens=np.full(B, ctx, np.int32), streams=streams,
                seq_sources=sources, q=_gen_q(spec, B), scale=np.float32(1.0 / math.sqrt(spec.d)), fill=fill)


def long128k_bf16(B=None, ctx=131072, fill="noise"):
    """Workload 4: a few very long sequences over a fully scattered table."""
    spec = SPECS["long128k_bf16"]
    B = spec.B if B is None else B
    need = B * _blocks(ctx, spec.bs)
    return _plain_case(spec, spec.bs, [ctx] * B, math.ceil(1.2 * need), fill)


def _mixed_lengths(rng, B, max_prompt=16384):
    prompt = np.clip(np.rint(rng.lognormal(mean=math.log(512.0), sigma=1.0, size=B)), 1, max_prompt)
    decode = rng.geometric(1.0 / 415.0, size=B)
    return (prompt + decode).astype(np.int64).tolist()


def mixed_fp8(bs=16, B=None, churn_ops=4096, max_prompt=16384, fill="noise", stream_cache=None):
    """Workload 5: e4m3 KV with per-KV-head scales; mixed lengths; the measured batch is
    allocated from a free list scrambled by seeded alloc/free churn.  Token contents are
    drawn per logical token, so bs 8 / 16 / 32 see the same data: cases of several block sizes
    may share one `stream_cache` dict (the drawn rows are then kept, not drawn again)."""
    spec = SPECS["mixed_fp8"]
    B = spec.B if B is None else B
    lens = _mixed_lengths(_rng(spec.seed, _LEN), B, max_prompt)
    need = sum(_blocks(n, bs) for n in lens)
    NB = math.ceil(1.3 * need)
    seqs = list(range(B))
    streams = {b: n for b, n in enumerate(lens)}
    sources = {b: [(b, 0, 0, n)] for b, n in enumerate(lens)}
    ops = [("churn", churn_ops, bs, max_prompt)]
    for b, n in enumerate(lens):
        ops += [("add", b), ("append", b, n, (b, 0))]
    order = _rng(spec.seed, _TAB).permutation(NB).astype(np.int32)
    case = Case(spec=spec, bs=bs, B=B, NB=NB, initial_free_order=order, ops=ops, step_ops=[],
                seqs=seqs, context_lens=np.asarray(lens, np.int32), streams=streams, seq_sources=sources,
                q=_gen_q(spec, B), scale=np.float32(1.0 / math.sqrt(spec.d)), fill=fill)
    if stream_cache is not None:
        case._stream_cache = stream_cache
    # per-KV-head scales amax/448 over the fp32 values of the stored bf16 samples
    amax_k = np.zeros(spec.H_kv, np.float32)
    amax_v = np.zeros(spec.H_kv, np.float32)
    for b in range(B):
        k, v = case.stream_kv(b)
        amax_k = np.maximum(amax_k, np.abs(bf16_bits_as_f32(k)).max(axis=(0, 2)))
        amax_v = np.maximum(amax_v, np.abs(bf16_bits_as_f32(v)).max(axis=(0, 2)))
    case.k_scale = (amax_k / np.float32(448.0)).astype(np.float32)
    case.v_scale = (amax_v / np.float32(448.0)).astype(np.float32)
    if stream_cache is None:
        case._stream_cache.clear()
    return case


def length_mix(kind: str, seed: int) -> np.ndarray:
    """Seeded context lengths of extra batches for timing the decode's work split on length
    mixes other than the five workloads' (int32 [B]):
      u4k   64 sequences, uniform on [128, 4096]
      u8k   48 sequences, uniform on [1, 8192]
      mix   256 sequences, log-normal prompt (median 512, sigma 1, at most 16384) + geometric
            decode (mean 415), the E4M3 workload's distribution
      uni   32 sequences of 8192 tokens (the seed only places the blocks)"""
    rng = _rng(seed, _LEN)
    if kind == "u4k":
        lens = rng.integers(128, 4097, size=64)
    elif kind == "u8k":
        lens = rng.integers(1, 8193, size=48)
    elif kind == "mix":
        lens = np.asarray(_mixed_lengths(rng, 256))
    elif kind == "uni":
        lens = np.full(32, 8192)
    else:
        raise ValueError(kind)
    return np.asarray(lens, np.int32)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Reinterpret bf16 bit patterns as fp32 (used only to size the fp8 scales of the inputs)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def custom(name, B, H_q, H_kv, d, bs, kv_dtype, q_dtype, lens, seed, fill="noise", NB=None):
    """A one-off workload of given shapes and lengths (test coverage beyond the five above)."""
    spec = Spec(name, B, H_q, H_kv, d, bs, kv_dtype, q_dtype, seed, "custom")
    assert len(lens) == B
    need = sum(_blocks(n, bs) for n in lens)
    case = _plain_case(spec, bs, list(lens), NB if NB is not None else need + 3, fill)
    if kv_dtype == "e4m3":
        amax_k = np.zeros(H_kv, np.float32)
        amax_v = np.zeros(H_kv, np.float32)
        for b in range(B):
            k, v = case.stream_kv(b)
            if len(k):
                amax_k = np.maximum(amax_k, np.abs(bf16_bits_as_f32(k)).max(axis=(0, 2)))
                amax_v = np.maximum(amax_v, np.abs(bf16_bits_as_f32(v)).max(axis=(0, 2)))
        case.k_scale = np.maximum(amax_k, np.float32(1e-3)) / np.float32(448.0)
        case.v_scale = np.maximum(amax_v, np.float32(1e-3)) / np.float32(448.0)
    return case


@dataclass
class BeamScript:
    """A seeded beam-search allocation script plus the rows every append writes.

    ops: ("add", sid) | ("append", sid, rows_index) | ("fork", parent, child) | ("free", sid)
         | ("decode", sids, q_index).  An append is meant to run as a copy-on-write append:
    allocator append with copy-on-write, then the reported block copies, then the scatter of
    rows[rows_index] into the returned slots."""
    name: str
    H_q: int
    H_kv: int
    d: int
    bs: int
    kv_dtype: str
    NB: int
    scale: float
    ops: list
    rows: list          # (k bf16 bits [n, H_kv, d], v bf16 bits [n, H_kv, d])
    qs: list            # bf16 bits [len(sids), H_q, d]
    k_scale: np.ndarray = None
    v_scale: np.ndarray = None


def beam_search(seed=1006, bs=16, prompts=3, width=4, steps=6, prompt_lo=17, prompt_hi=300, H_q=8, H_kv=2, d=128,
                kv_dtype="bf16", reselect=0.35):
    """Beam-search-shaped sharing ("KV Cache Fragmentation" field guide, section "Why it
    matters": cheap forks for beam search; "Paged Attention and KV Cache Fragmentation",
    section "How PagedAttention maps an OS concept onto GPU memory": branches share blocks
    until they diverge).  Each prompt is prefilled once and forked into `width` beams; every
    step appends one token to every beam; with probability `reselect` per prompt and step a
    random beam is dropped and a random survivor is forked in its place, so partly filled
    blocks keep being shared and copied on write.  All beams are decoded after every step."""
    rng = _rng(seed, 0)
    data = _rng(seed, 1)
    ops, rows, qs = [], [], []
    sid = 0

    def new_rows(n):
        k = round_bf16(data.standard_normal((n, H_kv, d), dtype=np.float32))
        v = round_bf16(data.standard_normal((n, H_kv, d), dtype=np.float32))
        rows.append((k, v))
        return len(rows) - 1

    beams = []
    for _ in range(prompts):
        n = int(rng.integers(prompt_lo, prompt_hi + 1))
        ops.append(("add", sid))
        ops.append(("append", sid, new_rows(n)))
        group = [sid]
        sid += 1
        for _ in range(width - 1):
            ops.append(("fork", group[0], sid))
            group.append(sid)
            sid += 1
        beams.append(group)
    for _ in range(steps):
        for group in beams:
            for b in group:
                ops.append(("append", b, new_rows(1)))
            if rng.random() < reselect and len(group) > 1:
                drop = group.pop(int(rng.integers(len(group))))
                ops.append(("free", drop))
                parent = group[int(rng.integers(len(group)))]
                ops.append(("fork", parent, sid))
                group.append(sid)
                sid += 1
        live = [b for g in beams for b in g]
        qs.append(round_bf16(data.standard_normal((len(live), H_q, d), dtype=np.float32)))
        ops.append(("decode", live, len(qs) - 1))
    NB = prompts * width * (-(-(prompt_hi + steps) // bs) + 2)
    script = BeamScript(f"beam_search_bs{bs}_{kv_dtype}", H_q, H_kv, d, bs, kv_dtype, NB,
                        float(np.float32(1.0 / math.sqrt(d))), ops, rows, qs)
    if kv_dtype == "e4m3":
        amax_k = np.max([np.abs(bf16_bits_as_f32(k)).max(axis=(0, 2)) for k, _ in rows], axis=0)
        amax_v = np.max([np.abs(bf16_bits_as_f32(v)).max(axis=(0, 2)) for _, v in rows], axis=0)
        script.k_scale = (np.maximum(amax_k, np.float32(1e-3)) / np.float32(448.0)).astype(np.float32)
        script.v_scale = (np.maximum(amax_v, np.float32(1e-3)) / np.float32(448.0)).astype(np.float32)
    return script


BUILDERS = {
    "tiny_f32": tiny_f32,
    "llama8b_bf16": llama8b_bf16,
    "llama70b_bf16": llama70b_bf16,
    "long128k_bf16": long128k_bf16,
    "mixed_fp8": mixed_fp8,
}


# ----------------------------------------------------------------------------
# driving an allocator with a script
# ----------------------------------------------------------------------------
def drive_churn(alloc, rng, n_ops: int, max_prompt: int):
    """Seeded alloc/free churn: each op, with probability 1/2, adds a sequence of a freshly
    drawn length (when the pool refuses it, a random live sequence is freed instead);
    otherwise a random live sequence is freed.  All churn sequences are freed at the end."""
    live = []
    sid = 1 << 40
    for _ in range(n_ops):
        if rng.random() < 0.5:
            n = _mixed_lengths(rng, 1, max_prompt)[0]
            sid += 1
            _check(alloc.seq_add(sid))
            st, _ = alloc.append_slots(sid, n)
            if st == STATUS_OUT_OF_BLOCKS:
                _check(alloc.free(sid))
                if live:
                    _check(alloc.free(live.pop(int(rng.integers(len(live))))))
            else:
                _check(st)
                live.append(sid)
        elif live:
            _check(alloc.free(live.pop(int(rng.integers(len(live))))))
    for s in live:
        _check(alloc.free(s))


def _check(st):
    if st != STATUS_OK:
        raise RuntimeError(f"allocator returned status {st} while replaying a workload script")


@dataclass
class Materialized:
    """What an allocator made of a script: the K/V rows to store and where."""
    k_src: np.ndarray  # [T, H_kv, d] source dtype
    v_src: np.ndarray
    slots: np.ndarray  # int64 [T]
    step_k: np.ndarray  # the step's rows [B_step, H_kv, d]
    step_v: np.ndarray
    step_slots: np.ndarray  # int64 [B_step]
    block_tables: np.ndarray  # int32 [B, max_blocks], -1 padded
    context_lens: np.ndarray  # int32 [B]


def materialize(case: Case, alloc) -> Materialized:
    """Replay the case's script on `alloc` and collect slots and tables.

    `alloc` must provide seq_add(seq), append_slots(seq, n) -> (status, int64 slots),
    fork(parent, child), free(seq) and block_tables(seqs, max_blocks) -> (status, table, lens).
    """
    ks, vs, ss = [], [], []

    def run(ops, out_k, out_v, out_s):
        for op in ops:
            kind = op[0]
            if kind == "add":
                _check(alloc.seq_add(op[1]))
            elif kind == "append":
                _, sid, n, (key, start) = op
                st, slots = alloc.append_slots(sid, n)
                _check(st)
                k, v = case.stream_kv(key)
                out_k.append(k[start:start + n])
                out_v.append(v[start:start + n])
                out_s.append(np.asarray(slots, np.int64))
            elif kind == "fork":
                _check(alloc.fork(op[1], op[2]))
            elif kind == "free":
                _check(alloc.free(op[1]))
            elif kind == "churn":
                _, n_ops, bs, max_prompt = op
                drive_churn(alloc, _rng(case.spec.seed, _CHURN, bs), n_ops, max_prompt)
            else:
                raise ValueError(kind)

    run(case.ops, ks, vs, ss)
    sk, sv, sslots = [], [], []
    run(case.step_ops, sk, sv, sslots)
    H, d = case.spec.H_kv, case.spec.d
    src = np.float32 if _src_dtype(case.spec) == "f32" else np.uint16

    def cat(parts, shape_tail, dt):
        return np.concatenate(parts) if parts else np.zeros((0, *shape_tail), dt)

    st, table, lens = alloc.block_tables(case.seqs, case.max_blocks)
    _check(st)
    return Materialized(
        k_src=cat(ks, (H, d), src), v_src=cat(vs, (H, d), src), slots=cat(ss, (), np.int64),
        step_k=cat(sk, (H, d), src), step_v=cat(sv, (H, d), src), step_slots=cat(sslots, (), np.int64),
        block_tables=np.asarray(table, np.int32), context_lens=np.asarray(lens, np.int32))


def initial_pool_fill(case: Case, which: str, pool_shape) -> np.ndarray:
    """Contents of pool slots that no append writes: N(0,1) noise, or NaN poison.

    Returned in the pool's storage dtype (fp32 values, bf16 bits, or e4m3 codes).
    For e4m3 the noise is uniform over the finite codes and the poison is code 0x7F (NaN).
    """
    spec = case.spec
    rng = _rng(spec.seed, _FILL, 0 if which == "k" else 1)
    n = int(np.prod(pool_shape))
    if spec.kv_dtype == "e4m3":
        if case.fill == "nan":
            return np.full(pool_shape, 0x7F, np.uint8)
        codes = rng.integers(0, 254, size=n, dtype=np.int64)
        codes = codes + (codes >= 0x7F)  # skip 0x7F; 0xFF is never drawn
        return codes.astype(np.uint8).reshape(pool_shape)
    if case.fill == "nan":
        vals = np.full(n, np.nan, np.float32)
    else:
        vals = _normal(rng, n)
    if spec.kv_dtype == "f32":
        return vals.reshape(pool_shape)
    return round_bf16(vals).reshape(pool_shape)
