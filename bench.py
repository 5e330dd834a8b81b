#!/usr/bin/env python3
"""Paged-KV decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: kv_append of this step's token
for every sequence, then paged decode attention of every sequence's query over its paged
KV (piece kernel + piece merge); with one new token per sequence the two run as one fused
pkv_decode_step call (--unfused issues them separately).  The default workload is a
Llama-3.1-70B-shaped layer: 32 sequences at 8192 tokens (16 of them share one refcounted
2048-token prefix), H_q 64, H_kv 8, head dim 128, bf16 KV, 16-token blocks scattered by
the allocator.  Inputs are synthetic and resident in HBM before the timed region.  A
workload with less than 1 GB of KV rotates through copies of its inputs (--sets).

Prints one JSON line.  `value` = algorithmic bytes of the step / step time in GB/s
(KV counted once per distinct physical block).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV GB/s (% of HBM peak) and sequences/s per layer"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
KERNEL_SOURCE = [os.path.join(ROOT, "paged_kv_cache_223_amd", "csrc", f) for f in ("paged_decode.hip", "decode_common.h", "tile_ops.h", "wave_scan.h", "e4m3_encode.h")]
COUNTERS = os.path.join(ROOT, "profiles", "decode_counters.json")
PREFILL_SOURCE = [os.path.join(ROOT, "paged_kv_cache_223_amd", "csrc", f) for f in ("prefill.hip", "tile_ops.h")]
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_counters.json")

WORKLOADS = {
    "llama70b": ("llama70b_bf16", {}),
    "llama8b": ("llama8b_bf16", {}),
    "long128k": ("long128k_bf16", {}),
    "fp8_bs8": ("mixed_fp8", {"bs": 8}),
    "fp8_bs16": ("mixed_fp8", {"bs": 16}),
    "fp8_bs32": ("mixed_fp8", {"bs": 32}),
}
# timed after the headline workload by the default invocation
OTHER_CONFIGS = ("llama8b", "long128k", "fp8_bs8", "fp8_bs16", "fp8_bs32")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama70b", choices=sorted(WORKLOADS))
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run the library's plain copy kernel over MIB MiB, 5 times (calibrates the "
                        "FETCH_SIZE / WRITE_SIZE memory counters against a known byte count) and exit")
    p.add_argument("--eager", action="store_true",
                   help="launch the step's kernels one by one instead of replaying a captured HIP graph")
    p.add_argument("--identity-tables", action="store_true",
                   help="lay every sequence out contiguously (identity block order) instead of scattered")
    p.add_argument("--op", default="step", choices=["step", "copy_blocks", "swap", "prefill", "mixes", "paths"],
                   help="step: the decode step (default); copy_blocks: copy-on-write block copies alone; "
                        "swap: swap-out / swap-in of scattered blocks to and from pinned host memory; "
                        "prefill: causal chunked prefill over the paged pools; mixes: decode call time on "
                        "seeded length mixes beyond the five workloads")
    p.add_argument("--prior", type=int, default=2048, help="earlier tokens per sequence (--op prefill)")
    p.add_argument("--chunk", type=int, default=2048, help="new tokens per sequence (--op prefill)")
    p.add_argument("--seqs", type=int, default=4, help="sequences (--op prefill)")
    p.add_argument("--prefill-kv", default="bf16", choices=["bf16", "e4m3"], help="KV pool type (--op prefill)")
    p.add_argument("--prefill-hq", type=int, default=64, choices=[8, 16, 32, 64, 128],
                   help="query heads over 8 KV heads (--op prefill; 64 = the 70B layer, G = 8)")
    p.add_argument("--prefill-d", type=int, default=128, choices=[64, 128], help="head dim (--op prefill)")
    p.add_argument("--prefill-waves", type=int, default=0, choices=[0, 8, 12],
                   help="prefill workgroup size (--op prefill; 0 = the library's automatic choice)")
    p.add_argument("--blocks", type=int, default=4096, help="blocks moved per swap call (--op swap)")
    p.add_argument("--pairs", type=int, default=4096, help="block pairs per copy_blocks call (--op copy_blocks)")
    p.add_argument("--unfused", action="store_true",
                   help="issue the step as kv_append + decode instead of the fused pkv_decode_step")
    p.add_argument("--no-length-hint", action="store_true",
                   help="do not pass the batch's length sum to the decode call (pkv_decode_step or "
                        "pkv_paged_attn_decode_hinted); the merge is then always launched")
    p.add_argument("--only", action="store_true",
                   help="time the named workload only (by default the 70B workload is followed by the other "
                        "configurations: " + ", ".join(OTHER_CONFIGS) + ", and the tiny fp32 one)")
    p.add_argument("--extra-steps", type=int, default=100, help="timed steps of each other configuration")
    p.add_argument("--extra-warmup", type=int, default=10, help="warm-up steps of each other configuration")
    p.add_argument("--extra-cpu-seconds", type=float, default=4.0,
                   help="budget of each other configuration's oracle baseline sample")
    p.add_argument("--sets", type=int, default=0,
                   help="independent copies of the inputs the steps rotate through (0 = enough for 1 GB of "
                        "KV, so the 256 MB last-level cache cannot hold the working set)")
    p.add_argument("--graph-steps", type=int, default=20,
                   help="consecutive steps captured in one HIP graph for the timed replays (rounded up to a "
                        "multiple of the input sets; 1 = one graph per step)")
    return p.parse_args()


# ----------------------------------------------------------------------------- byte accounting
def algorithmic_bytes(tables, lens, bs, B, H_q, H_kv, D, s_kv, s_q, T_append, s_src):
    """Bytes the step must move at minimum.

    decode: K and V of every distinct physical block the batch touches (the token positions
    some sequence attends to), q, the fp32 output, the used table entries, the lengths and the
    fp8 scales.  append: this step's K/V rows read and written, plus their slots.
    """
    used = {}
    logical_tok = 0
    tab_entries = 0
    for row, n in zip(tables, lens):
        n = int(n)
        logical_tok += n
        nb = -(-n // bs)
        tab_entries += nb
        for j in range(nb):
            blk = int(row[j])
            used[blk] = max(used.get(blk, 0), min(bs, n - j * bs))
    per_tok = H_kv * D * 2 * s_kv
    kv_unique = sum(used.values()) * per_tok
    kv_logical = logical_tok * per_tok
    other = B * H_q * D * s_q + B * H_q * D * 4 + tab_entries * 4 + B * 4 + (2 * H_kv * 4 if s_kv == 1 else 0)
    append = T_append * H_kv * D * 2 * (s_src + s_kv) + T_append * 8
    return dict(kv_unique=kv_unique, kv_logical=kv_logical, decode=kv_unique + other,
                decode_logical=kv_logical + other, append=append)


def source_hash(paths):
    """Hash of C++/HIP sources with comments and whitespace removed, so that the counters
    taken on a kernel stay valid across comment-only edits."""
    text = "".join(open(p).read() for p in paths)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(workload, counters=COUNTERS, sources=KERNEL_SOURCE):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on the
    current kernel source and this workload; else None."""
    try:
        rec = json.load(open(counters))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("code_sha256_16") != source_hash(sources):
        return None
    return ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode path is not sharded "
              "across GPUs in this build.", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_223_amd as pkv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            pkv.copy_(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)
        return
    if args.op == "copy_blocks":
        bench_copy_blocks(args, torch, pkv, dev)
        return
    if args.op == "swap":
        bench_swap(args, torch, pkv, dev)
        return
    if args.op == "prefill":
        bench_prefill(args, torch, pkv, dev)
        return
    if args.op == "mixes":
        bench_mixes(args, torch, pkv, dev)
        return
    if args.op == "paths":
        bench_paths(args, torch, pkv, dev)
        return
    shared = {}  # drawn K/V rows shared by the E4M3 workload's block sizes (the same logical data)
    res = bench_decode(args.workload, args, torch, pkv, dev, args.steps, args.warmup, args.cpu_seconds,
                       headline=True, shared=shared)
    if not args.only and args.workload == "llama70b":
        # the other configurations, each with its own (shorter) timing and oracle baseline; `value`
        # and `config` stay on the headline workload
        res["other_configs"] = {}
        for w in OTHER_CONFIGS:
            res["other_configs"][w] = bench_decode(w, args, torch, pkv, dev, args.extra_steps, args.extra_warmup,
                                                   args.extra_cpu_seconds, headline=False, shared=shared)
        shared.clear()
        res["other_configs"]["tiny_f32"] = bench_tiny(args, torch, pkv, dev)
    print(json.dumps(res), flush=True)


def _build_case(wkey, shared):
    import workloads
    wname, kw = WORKLOADS[wkey]
    if wname == "mixed_fp8":
        kw = dict(kw, stream_cache=shared.setdefault("mixed_fp8", {}))
    return workloads.BUILDERS[wname](**kw)


def bench_decode(wkey, args, torch, pkv, dev, steps, warmup, cpu_seconds, headline, shared):
    """One decode workload: setup, eager per-call timing, graph-replayed steps, roofline, oracle
    baseline.  Returns the JSON object (the headline form carries the whole line's keys)."""
    import workloads

    t_setup = time.time()
    case = _build_case(wkey, shared)
    if args.identity_tables:
        case.initial_free_order = np.arange(case.NB, dtype=np.int32)
    spec = case.spec
    mat = workloads.materialize(case, pkv.Allocator(case.NB, case.bs, case.initial_free_order))
    kvd = {"bf16": pkv.BF16, "e4m3": pkv.FP8_E4M3, "f32": pkv.F32}[spec.kv_dtype]
    ks, vs = pkv.pool_shapes(case.NB, spec.H_kv, spec.d, case.bs, kvd)
    pool_dt = {"bf16": torch.bfloat16, "e4m3": torch.uint8, "f32": torch.float32}[spec.kv_dtype]
    k_pool = torch.zeros(ks, dtype=pool_dt, device=dev)
    v_pool = torch.zeros(vs, dtype=pool_dt, device=dev)

    def up(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sd = "f32" if spec.kv_dtype == "f32" else "bf16"
    k_scale = None if case.k_scale is None else torch.from_numpy(case.k_scale).to(dev)
    v_scale = None if case.v_scale is None else torch.from_numpy(case.v_scale).to(dev)
    CH = 65536
    for i in range(0, len(mat.slots), CH):  # prefill the pools through the library's own append
        pkv.kv_append(up(mat.k_src[i:i + CH], sd), up(mat.v_src[i:i + CH], sd),
                      torch.from_numpy(mat.slots[i:i + CH]).to(dev), k_pool, v_pool, k_scale, v_scale)
    step_k, step_v = up(mat.step_k, sd), up(mat.step_v, sd)
    step_slots = torch.from_numpy(mat.step_slots).to(dev)
    q = up(case.q, spec.q_dtype)
    tables = torch.from_numpy(mat.block_tables).to(dev)
    lens = torch.from_numpy(mat.context_lens).to(dev)
    B, H_q, H_kv, D = case.B, spec.H_q, spec.H_kv, spec.d
    mcl = case.max_context_len
    out = torch.empty((B, H_q, D), dtype=torch.float32, device=dev)
    ws = pkv.decode_workspace(B, H_q, D, mcl, case.bs, H_kv=H_kv, device=dev)

    s_kv = {"bf16": 2, "e4m3": 1, "f32": 4}[spec.kv_dtype]
    s_q = 4 if spec.q_dtype == "f32" else 2
    s_src = 4 if sd == "f32" else 2
    by = algorithmic_bytes(mat.block_tables, mat.context_lens, case.bs, B, H_q, H_kv, D, s_kv, s_q,
                           len(mat.step_slots), s_src)
    # independent input sets (separate copies of the pools and per-step inputs) so that a
    # workload smaller than 1 GB of KV is not served from the last-level cache on repeat
    n_sets = args.sets if args.sets > 0 else max(1, math.ceil(1e9 / by["kv_logical"]))
    sets = [(k_pool, v_pool, q, tables, lens, step_k, step_v, step_slots)]
    for _ in range(n_sets - 1):
        sets.append(tuple(t.clone() for t in sets[0]))
    torch.cuda.synchronize()
    print(f"# {wkey}: setup {time.time() - t_setup:.1f}s: {spec.name} B={B} NB={case.NB} pool "
          f"{2 * k_pool.numel() * k_pool.element_size() / 1e9:.2f} GB x {n_sets} input set(s)", file=sys.stderr,
          flush=True)

    # one new token per sequence into bf16 pools: the step is one fused call (the append runs
    # inside the decode launch); E4M3 pools take kv_append + decode
    fused = not args.unfused and len(mat.step_slots) == B and case.spec.kv_dtype == "bf16"
    # the host's own count of the batch's tokens (its allocator holds the lengths): a split hint
    # for the decode call, no device sync
    sum_lens = -1 if args.no_length_hint else int(mat.context_lens.astype(np.int64).sum())

    def step(i=0, e0=None, e1=None, e2=None):
        kp, vp, q_, tab, ln, sk, sv, ss = sets[i % n_sets]
        if e0 is not None:
            e0.record()
        if len(mat.step_slots) and not fused:
            pkv.kv_append(sk, sv, ss, kp, vp, k_scale, v_scale)
        if e1 is not None:
            e1.record()
        if fused:
            pkv.decode_step(q_, sk, sv, ss, kp, vp, tab, ln, float(case.scale), k_scale, v_scale, max_context_len=mcl,
                            out=out, workspace=ws, sum_context_lens=sum_lens)
        else:
            pkv.paged_attn_decode(q_, kp, vp, tab, ln, float(case.scale), k_scale, v_scale, max_context_len=mcl,
                                  out=out, workspace=ws, sum_context_lens=sum_lens)
        if e2 is not None:
            e2.record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    K = steps
    # decode alone, eager launches: per-call duration of the dominant kernel(s) on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        step(i, *ev[i])
    torch.cuda.synchronize()
    append_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    decode_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    eager_step_ms = ev[0][0].elapsed_time(ev[-1][2]) / K
    # the timed region: K whole steps (kv_append + decode), replayed from captured HIP graphs
    graphs = multi = None
    R = steps_per_graph(args.graph_steps, n_sets)
    if not args.eager:  # one captured step per input set, replayed in rotation
        graphs = []
        for i in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        if R > 1 and K >= R:
            multi = torch.cuda.CUDAGraph()
            with torch.cuda.graph(multi):
                for i in range(R):
                    step(i)
        for i in range(warmup):
            graphs[i % n_sets].replay()
        if multi is not None:
            multi.replay()
    torch.cuda.synchronize()

    def timed(multi_graph):
        """K steps bracketed by device syncs; returns (ms per step, wall s)."""
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        g0.record()
        if graphs is None:
            for i in range(K):
                step(i)
        else:
            done = 0
            if multi_graph:
                for _ in range(K // R):
                    multi.replay()
                done = K // R * R
            for i in range(done, K):
                graphs[i % n_sets].replay()
        g1.record()
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) / K, time.perf_counter() - t0

    # one graph launch per step first (each launch then pays the gap before its kernel starts), then
    # the timed region proper: R consecutive steps per graph launch, as a decode loop over a model's
    # layers is captured, so the kernels of consecutive steps follow each other without that gap
    single_ms = timed(False)[0] if multi is not None else None
    step_ms, wall = timed(multi is not None)
    print(f"# {wkey}: timed {K} steps in {wall:.3f}s wall ({'eager' if graphs is None else 'graph'}, "
          f"{R if multi is not None else 1} per launch); step {step_ms * 1e3:.1f} us"
          + ("" if single_ms is None else f" (one step per graph launch: {single_ms * 1e3:.1f} us)")
          + f"; eager decode p10/p50/p90 {np.percentile(decode_ms, 10) * 1e3:.1f}/"
          f"{np.median(decode_ms) * 1e3:.1f}/{np.percentile(decode_ms, 90) * 1e3:.1f} us", file=sys.stderr, flush=True)

    call_bytes = by["decode"] + (by["append"] if fused else 0)  # bytes of the timed call
    # the call's average duration: where a step is that one launch, replayed from multi-step graphs,
    # the events around the timed region give it without per-call event overhead (consecutive
    # launches run back to back there); otherwise the events around each eager call
    one_launch = fused or not len(mat.step_slots)
    from_region = one_launch and multi is not None
    dec_avg_s = step_ms / 1e3 if from_region else decode_ms.mean() / 1e3
    dec_gbps = call_bytes / dec_avg_s / 1e9
    step_gbps = (by["decode"] + by["append"]) / (step_ms / 1e3) / 1e9
    traffic = measured_traffic(wkey)
    roofline = {
        "bound": "hbm",
        "kernel": ("decode step call (append fused) = decode_piece_kernel (cut segments merged inside it)"
                   if fused else "paged_attn_decode call = decode_piece_kernel (cut segments merged inside it)"),
        "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_launch": call_bytes,
        "avg_launch_us": round(dec_avg_s * 1e6, 2),
        "launch_timing": ("HIP events around the timed region (one launch per step, back to back)" if from_region
                          else "HIP events around each eager call"),
        "eager_call_us_avg": round(float(decode_ms.mean()) * 1e3, 2),
        "traffic": traffic,
    }
    common = {
        "seqs_per_s": round(B / (step_ms / 1e3), 1),
        "frac_of_hbm_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "decode_us_p50": round(float(np.median(decode_ms)) * 1e3, 2),
        "decode_us_p10_p90": [round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
                              round(float(np.percentile(decode_ms, 90)) * 1e3, 2)],
        "append_us_p50": None if fused or not len(mat.step_slots) else round(float(np.median(append_ms)) * 1e3, 2),
        "step_call": "pkv_decode_step (append fused into the decode launch)" if fused else
                     ("kv_append + paged_attn_decode" if len(mat.step_slots) else "paged_attn_decode") +
                     ("" if sum_lens < 0 else " (with the host's length sum)"),
        "eager_ms_per_step": round(eager_step_ms, 5),
        "step_launch": "eager" if graphs is None else "hip_graph",
        "steps_per_graph": None if graphs is None else (R if multi is not None else 1),
        "ms_per_step_one_graph_per_step": None if single_ms is None else round(single_ms, 5),
        "decode_GBps_unique": round(dec_gbps, 1),
        "decode_GBps_logical": round(by["decode_logical"] / dec_avg_s / 1e9, 1),
        "kv_bytes_unique": by["kv_unique"],
        "kv_bytes_logical": by["kv_logical"],
        "kv_waste": block_waste(mat.block_tables, mat.context_lens, case.bs),
    }
    cfg = {
        "workload": spec.desc, "batch": B, "H_q": H_q, "H_kv": H_kv, "head_dim": D, "block_size": case.bs,
        "kv_dtype": spec.kv_dtype, "max_context": mcl, "mean_context": float(np.mean(mat.context_lens)),
        "pool_blocks": case.NB, "append_tokens_per_step": int(len(mat.step_slots)),
        "tables": "identity" if args.identity_tables else "scattered", "input_sets": n_sets,
    }
    if headline:
        # practical read ceiling: the library's non-temporal 16-byte streaming read over 4 GiB
        buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        sink = pkv.stream_read(buf)
        torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record()
        for _ in range(10):
            pkv.stream_read(buf, sink)
        r1.record()
        torch.cuda.synchronize()
        ceiling = buf.numel() * 10 / (r0.elapsed_time(r1) / 1e3) / 1e9
        del buf
        res = {
            "metric": METRIC, "value": round(step_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
            "warmup": warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": spec.kv_dtype,
            "data": "synthetic (seeded N(0,1) K/V/q rounded to the KV dtype; allocator-scattered block tables)",
            "config": cfg, **common,
            "read_ceiling_GBps": round(ceiling, 1), "frac_of_read_ceiling": round(step_gbps / ceiling, 4),
            "roofline": roofline,
        }
    else:
        res = {"config": cfg, "steps": K, "warmup": warmup, "step_us": round(step_ms * 1e3, 2),
               "value_GBps": round(step_gbps, 1), **common, "roofline": roofline}
    if not args.no_cpu_baseline:
        sample = 1 if wkey == "long128k" else 16  # a 131072-token sequence takes seconds in the oracle
        res["cpu_baseline"] = cpu_baseline(case, mat, out, cpu_seconds, by, B, max_sample=sample)
        if wkey in ("llama70b", "llama8b"):  # the oracle on one host thread as well
            res["cpu_baseline_1thread"] = cpu_baseline(case, mat, out, min(cpu_seconds, 6.0), by, B, threads=1)
    del sets, k_pool, v_pool, out, ws
    torch.cuda.empty_cache()
    return res


def bench_tiny(args, torch, pkv, dev):
    """The tiny fp32 workload (4 sequences, lengths 1/17/33/64): launch-bound, so reported for
    completeness: GPU call time, and the oracle on the host with all its BLAS threads and with one,
    checked against the GPU output."""
    import oracle
    import workloads
    from threadpoolctl import threadpool_limits

    case = workloads.tiny_f32()
    spec = case.spec
    mat = workloads.materialize(case, pkv.Allocator(case.NB, case.bs, case.initial_free_order))
    ks, vs = pkv.pool_shapes(case.NB, spec.H_kv, spec.d, case.bs, pkv.F32)
    kp0 = workloads.initial_pool_fill(case, "k", ks)
    vp0 = workloads.initial_pool_fill(case, "v", vs)
    kp, vp = torch.from_numpy(kp0).to(dev), torch.from_numpy(vp0).to(dev)
    pkv.kv_append(torch.from_numpy(mat.k_src).to(dev), torch.from_numpy(mat.v_src).to(dev),
                  torch.from_numpy(mat.slots).to(dev), kp, vp)
    q, tab, ln = (torch.from_numpy(x).to(dev) for x in (case.q, mat.block_tables, mat.context_lens))
    out = torch.empty((case.B, spec.H_q, spec.d), dtype=torch.float32, device=dev)

    def call():
        pkv.paged_attn_decode(q, kp, vp, tab, ln, float(case.scale), max_context_len=case.max_context_len, out=out)

    for _ in range(20):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(200)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    got = out.cpu().numpy().astype(np.float64)
    kr, vr = oracle.ref_append(kp0, vp0, mat.k_src, mat.v_src, "f32", mat.slots, case.bs, "f32")
    res = {"config": {"workload": spec.desc, "batch": case.B}, "decode_us_p50": round(float(np.median(ms)) * 1e3, 2),
           "seqs_per_s": round(case.B / (np.median(ms) / 1e3), 1),
           "kv_bytes": int(mat.context_lens.sum()) * spec.H_kv * spec.d * 2 * 4}
    for label, threads in (("cpu_baseline", None), ("cpu_baseline_1thread", 1)):
        with threadpool_limits(threads):
            n, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < 1.0:
                ref = oracle.ref_decode(case.q, "f32", kr, vr, "f32", mat.block_tables, mat.context_lens, case.scale,
                                        case.bs)
                n += 1
            dt = time.perf_counter() - t0
        err = float((np.abs(got - ref).max(-1) / np.abs(ref).max(-1)).max())
        res[label] = {"value": round(n * case.B / dt, 1), "unit": "sequences/s", "cores": _blas_threads(),
                      "kind": "oracle", "sample": f"{n} passes over all {case.B} sequences",
                      "seconds": round(dt, 2), "gpu_vs_oracle_max_row_rel_err": err}
        if threads == 1:
            res[label]["cores"] = 1
    print(f"# tiny_f32: decode p50 {res['decode_us_p50']} us", file=sys.stderr, flush=True)
    return res


def bench_mixes(args, torch, pkv, dev):
    """Decode call time on seeded length mixes beyond the five workloads (workloads.length_mix):
    random pools, scattered tables, decode call p50 over 60 eager calls after 10 warm-up calls,
    no length hint.  One JSON line with every batch's p50."""
    import workloads
    cases = [("u4k", s, "bf16") for s in (11, 12, 13, 14)] + [("u8k", 15, "bf16"), ("mix", 16, "bf16")] + \
        [("mix", s, "e4m3") for s in (17, 18, 19)] + [("uni", 20, "e4m3"), ("uni", 21, "bf16")]
    H_q, H_kv, D, bs = 32, 8, 128, 16
    rows = []
    for kind, seed, kv in cases:
        lens = workloads.length_mix(kind, seed)
        B = len(lens)
        nblk = (lens.astype(np.int64) + bs - 1) // bs
        NB = int(nblk.sum()) + 8
        perm = np.random.default_rng(seed).permutation(NB).astype(np.int32)
        tab = np.full((B, int(nblk.max())), -1, np.int32)
        o = 0
        for b in range(B):
            tab[b, :nblk[b]] = perm[o:o + nblk[b]]
            o += nblk[b]
        kvd = pkv.BF16 if kv == "bf16" else pkv.FP8_E4M3
        ks, vs = pkv.pool_shapes(NB, H_kv, D, bs, kvd)
        g = torch.Generator(device=dev).manual_seed(seed)
        if kv == "bf16":
            kp = torch.randn(ks, device=dev, generator=g).to(torch.bfloat16)
            vp = torch.randn(vs, device=dev, generator=g).to(torch.bfloat16)
            ksc = vsc = None
        else:
            kp = torch.randint(0, 120, ks, dtype=torch.uint8, device=dev, generator=g)
            vp = torch.randint(0, 120, vs, dtype=torch.uint8, device=dev, generator=g)
            ksc = torch.full((H_kv,), 0.01, device=dev)
            vsc = torch.full((H_kv,), 0.01, device=dev)
        q = torch.randn((B, H_q, D), device=dev, generator=g).to(torch.bfloat16)
        tabd, lensd = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
        out = torch.empty((B, H_q, D), device=dev)
        mcl = int(lens.max())
        ws = pkv.decode_workspace(B, H_q, D, mcl, bs, H_kv=H_kv, device=dev)

        def call():
            pkv.paged_attn_decode(q, kp, vp, tabd, lensd, 1 / math.sqrt(D), ksc, vsc, max_context_len=mcl, out=out,
                                  workspace=ws)

        for _ in range(10):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(60)]
        for e0, e1 in ev:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        us = float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))
        kv_bytes = int(lens.astype(np.int64).sum()) * H_kv * D * 2 * (2 if kv == "bf16" else 1)
        rows.append({"batch": f"{kind}-{seed}-{kv}", "B": B, "decode_us_p50": round(us, 1),
                     "kv_GBps": round(kv_bytes / us / 1e3, 1)})
        print(f"# mix {rows[-1]}", file=sys.stderr, flush=True)
        del kp, vp, ws
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "decode call p50 on seeded length mixes", "unit": "us", "n_gpus": 1,
                      "config": {"workload": "seeded length mixes (workloads.length_mix)", "H_q": H_q, "H_kv": H_kv,
                                 "head_dim": D, "block_size": bs},
                      "batches": rows}), flush=True)


def bench_paths(args, torch, pkv, dev):
    """Matrix-core against vector decode on one batch: 32 sequences of 4096 tokens, H_kv 8, D 128,
    bs 16, bf16 q, for query heads per KV head G in 1, 2, 4, 8 and bf16 or E4M3 KV.  Random pool,
    scattered tables; the two paths' calls alternate in rounds of 20 (after 10 warm-up calls of
    each) and each reports its p50 over 100 calls.  One JSON line."""
    B, n, H_kv, D, bs = 32, 4096, 8, 128, 16
    nblk = n // bs
    NB = B * nblk + 8
    tab = np.random.default_rng(5).permutation(NB)[:B * nblk].astype(np.int32).reshape(B, nblk)
    lens = np.full(B, n, np.int32)
    tabd, lensd = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
    rows = []
    for kv in ("bf16", "e4m3"):
        kvd = pkv.BF16 if kv == "bf16" else pkv.FP8_E4M3
        ks, vs = pkv.pool_shapes(NB, H_kv, D, bs, kvd)
        g = torch.Generator(device=dev).manual_seed(7)
        if kv == "bf16":
            kp = torch.randn(ks, device=dev, generator=g).to(torch.bfloat16)
            vp = torch.randn(vs, device=dev, generator=g).to(torch.bfloat16)
            ksc = vsc = None
        else:
            kp = torch.randint(0, 120, ks, dtype=torch.uint8, device=dev, generator=g)
            vp = torch.randint(0, 120, vs, dtype=torch.uint8, device=dev, generator=g)
            ksc = torch.full((H_kv,), 0.01, device=dev)
            vsc = torch.full((H_kv,), 0.01, device=dev)
        for G in (1, 2, 4, 8):
            H_q = G * H_kv
            q = torch.randn((B, H_q, D), device=dev, generator=g).to(torch.bfloat16)
            ws = pkv.decode_workspace(B, H_q, D, n, bs, H_kv=H_kv, device=dev)
            outs = {p: torch.empty((B, H_q, D), device=dev) for p in ("matrix", "vector")}
            mode = {"matrix": pkv.DECODE_PATH_AUTO, "vector": pkv.DECODE_PATH_VECTOR}
            times = {p: [] for p in outs}

            def call(p):
                pkv.set_decode_path(mode[p])
                pkv.paged_attn_decode(q, kp, vp, tabd, lensd, 1 / math.sqrt(D), ksc, vsc, max_context_len=n,
                                      out=outs[p], workspace=ws)

            try:
                for p in outs:
                    for _ in range(10):
                        call(p)
                torch.cuda.synchronize()
                for _ in range(5):
                    for p in outs:
                        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                              for _ in range(20)]
                        for e0, e1 in ev:
                            e0.record()
                            call(p)
                            e1.record()
                        torch.cuda.synchronize()
                        times[p] += [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
            finally:
                pkv.set_decode_path(pkv.DECODE_PATH_AUTO)
            om, ov = outs["matrix"].double(), outs["vector"].double()
            rel = float(((om - ov).norm(dim=-1) / om.norm(dim=-1).clamp_min(1e-30)).max())
            kv_bytes = B * n * H_kv * D * 2 * (2 if kv == "bf16" else 1)
            row = {"kv": kv, "G": G, "H_q": H_q}
            for p in outs:
                us = float(np.median(times[p]))
                row[f"{p}_us_p50"] = round(us, 1)
                row[f"{p}_GBps"] = round(kv_bytes / us / 1e3, 1)
            row["vector_over_matrix"] = round(row["vector_us_p50"] / row["matrix_us_p50"], 3)
            row["max_row_rel_diff"] = rel
            rows.append(row)
            print(f"# paths {row}", file=sys.stderr, flush=True)
            del ws, outs, q
        del kp, vp
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "decode call p50, matrix-core vs vector path", "unit": "us", "n_gpus": 1,
                      "config": {"workload": "32 sequences x 4096 tokens, H_kv 8, D 128, bs 16, bf16 q, "
                                             "scattered tables", "B": B, "context": n, "H_kv": H_kv, "head_dim": D,
                                 "block_size": bs},
                      "rows": rows}), flush=True)


def steps_per_graph(graph_steps, n_sets):
    """Steps captured in one multi-step graph: `graph_steps` rounded up to a multiple of the input
    sets, so that the rotation through them carries on across replays; 1 = one graph per step."""
    return n_sets * math.ceil(graph_steps / n_sets) if graph_steps > 1 else 1


def block_waste(tables, lens, bs):
    """Internal waste of the allocator's blocks in use: each distinct block counts once (a shared
    prefix block holds its tokens once), filled to the furthest token any of its holders uses."""
    fill = {}
    for row, n in zip(tables, lens):
        for j in range(-(-int(n) // bs)):
            b = int(row[j])
            fill[b] = max(fill.get(b, 0), min(bs, int(n) - j * bs))
    slots = len(fill) * bs
    used = sum(fill.values())
    return {"blocks_in_use": len(fill), "slots": slots, "tokens": used,
            "internal_frac": round(1 - used / slots, 6) if slots else 0.0}


def bench_copy_blocks(args, torch, pkv, dev):
    """Copy-on-write block copies alone: `pairs` random disjoint (src, dst) block pairs of a pool
    shaped like the 70B layer's (H_kv 8, D 128, bs 16, bf16: 32 KiB per block and pool); GB/s
    counts the bytes read plus the bytes written."""
    H_kv, D, bs = 8, 128, 16
    NB = 2 * args.pairs + 64
    ks, vs = pkv.pool_shapes(NB, H_kv, D, bs, pkv.BF16)
    k_pool = torch.zeros(ks, dtype=torch.bfloat16, device=dev)
    v_pool = torch.zeros(vs, dtype=torch.bfloat16, device=dev)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(NB).astype(np.int32)).to(dev)
    src, dst = perm[:args.pairs].contiguous(), perm[args.pairs:2 * args.pairs].contiguous()
    # a small call takes less GPU time than its Python launch, so calls are timed from a
    # captured graph of R back-to-back copies (per-call time = replay time / R)
    R = 20
    for _ in range(3):
        pkv.copy_blocks(k_pool, v_pool, src, dst)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(R):
            pkv.copy_blocks(k_pool, v_pool, src, dst)
    for _ in range(args.warmup):
        graph.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) / R
    block_bytes = 2 * H_kv * D * bs * 2
    moved = 2 * args.pairs * block_bytes  # read + write
    avg_s = ms.mean() / 1e3
    print(json.dumps({
        "metric": "copy_blocks GB/s (bytes read + written)", "value": round(moved / avg_s / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 5),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic (zero-filled pools, random disjoint pairs)",
        "config": {"workload": f"{args.pairs} block copies, 70B-layer block shape (H_kv 8, D 128, bs 16)",
                   "pairs": args.pairs, "bytes_per_pair_read": block_bytes},
        "us_p50": round(float(np.median(ms)) * 1e3, 2),
        "frac_of_hbm_peak": round(moved / avg_s / 1e9 / HBM_PEAK_GBPS, 4)}), flush=True)


def bench_swap(args, torch, pkv, dev):
    """Swap-out / swap-in of `blocks` scattered blocks of a pool shaped like the 70B layer's
    (H_kv 8, D 128, bs 16, bf16: a 64 KiB K+V record per block), five ways:
      gather_device   gather into a device staging buffer (HBM to HBM)
      gather_pinned   gather straight into pinned host memory (the kernel writes over the link)
      gather_memcpy   gather into device staging, then one DMA copy to pinned host memory
      per_block_dma   the naive swap-out: one DMA copy per K and per V block (2 x blocks copies)
      scatter_pinned  swap-in: scatter straight from pinned host memory into the blocks
    GB/s counts the record bytes moved once (blocks x 64 KiB)."""
    H_kv, D, bs = 8, 128, 16
    n = args.blocks
    NB = 2 * n + 64
    ks, vs = pkv.pool_shapes(NB, H_kv, D, bs, pkv.BF16)
    k_pool = torch.randn(ks, device=dev).to(torch.bfloat16)
    v_pool = torch.randn(vs, device=dev).to(torch.bfloat16)
    perm = np.random.default_rng(9).permutation(NB).astype(np.int32)
    ids = torch.from_numpy(perm[:n].copy()).to(dev)
    rec = pkv.lib.pkv_block_record_bytes(pkv.BF16, bs, H_kv, D)
    st_dev = torch.empty((n, 2, rec // 2), dtype=torch.uint8, device=dev)
    st_host = torch.empty((n, 2, rec // 2), dtype=torch.uint8, pin_memory=True)
    host_k = torch.empty((n,) + tuple(ks[1:]), dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.empty((n,) + tuple(vs[1:]), dtype=torch.bfloat16, pin_memory=True)
    ids_host = perm[:n].tolist()

    def per_block_dma():
        for i, b in enumerate(ids_host):
            host_k[i].copy_(k_pool[b], non_blocking=True)
            host_v[i].copy_(v_pool[b], non_blocking=True)

    ways = {
        "gather_device": lambda: pkv.gather_blocks(k_pool, v_pool, ids, out=st_dev),
        "gather_pinned": lambda: pkv.gather_blocks(k_pool, v_pool, ids, out=st_host),
        "gather_memcpy": lambda: (pkv.gather_blocks(k_pool, v_pool, ids, out=st_dev),
                                  st_host.copy_(st_dev, non_blocking=True)),
        "per_block_dma": per_block_dma,
        "scatter_pinned": lambda: pkv.scatter_blocks(k_pool, v_pool, ids, st_host),
    }
    res = {}
    for name, fn in ways.items():
        reps = 3 if name == "per_block_dma" else max(5, args.steps // 10)
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / reps
        gpu = e0.elapsed_time(e1) / 1e3 / reps
        t = max(wall, gpu)  # the naive path is bound by the host issuing copies
        res[name] = {"ms": round(t * 1e3, 3), "GBps": round(n * rec / t / 1e9, 2)}
    # the pinned gather must hold what the device gather holds
    pkv.gather_blocks(k_pool, v_pool, ids, out=st_dev)
    pkv.gather_blocks(k_pool, v_pool, ids, out=st_host)
    torch.cuda.synchronize()
    same = bool(torch.equal(st_dev.cpu(), st_host))
    print(json.dumps({
        "metric": "swap-out GB/s (scattered blocks gathered into pinned host memory)",
        "value": res["gather_pinned"]["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": 1, "ms_per_step": res["gather_pinned"]["ms"], "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (random pool, random distinct blocks)",
        "config": {"workload": f"{n} scattered blocks, 70B-layer block shape (H_kv 8, D 128, bs 16)",
                   "blocks": n, "record_bytes": rec},
        "ways": res, "pinned_equals_device_gather": same}), flush=True)


def bench_prefill(args, torch, pkv, dev):
    """Causal chunked prefill on the 70B layer shape (H_q 64, H_kv 8, D 128, bf16, bs 16; other query
    head counts and head dims by option): `seqs`
    sequences, each with `prior` earlier tokens and a `chunk` of new ones (appended before the
    timed region).  FLOPs count the two products over the causal range only:
    4 * H_q * D * sum over queries of (position + 1)."""
    H_q, H_kv, D, bs = args.prefill_hq, 8, args.prefill_d, 16
    B, prior, C = args.seqs, args.prior, args.chunk
    n = prior + C
    nb = -(-n // bs)
    NB = B * nb + 16
    rng = np.random.default_rng(17)
    alloc = pkv.Allocator(NB, bs, rng.permutation(NB).astype(np.int32))
    slots = []
    for b in range(B):
        alloc.seq_add(b)
        slots.append(alloc.append_slots(b, n)[1])
    st, tab, lens = alloc.block_tables(list(range(B)), nb)
    fp8 = args.prefill_kv == "e4m3"
    ks, vs = pkv.pool_shapes(NB, H_kv, D, bs, pkv.FP8_E4M3 if fp8 else pkv.BF16)
    pool_dt = torch.uint8 if fp8 else torch.bfloat16
    k_pool = torch.empty(ks, dtype=pool_dt, device=dev)
    v_pool = torch.empty(vs, dtype=pool_dt, device=dev)
    # E4M3: per-head scales that map |x| <= 5 (beyond 5 sigma of N(0,1)) onto the format's 448
    k_scale = torch.full((H_kv,), 5.0 / 448, dtype=torch.float32, device=dev) if fp8 else None
    v_scale = torch.full((H_kv,), 5.0 / 448, dtype=torch.float32, device=dev) if fp8 else None
    kv = torch.randn((B * n, 2, H_kv, D), device=dev).to(torch.bfloat16)
    pkv.kv_append(kv[:, 0].contiguous(), kv[:, 1].contiguous(), torch.from_numpy(np.concatenate(slots)).to(dev),
                  k_pool, v_pool, k_scale, v_scale)
    del kv
    q = torch.randn((B * C, H_q, D), device=dev).to(torch.bfloat16)
    qs = torch.arange(0, B * C + 1, C, dtype=torch.int32, device=dev)
    tab_d, lens_d = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
    out = torch.empty((B * C, H_q, D), dtype=torch.float32, device=dev)
    scale = 1 / np.sqrt(D)

    def call():
        pkv.paged_prefill(q, k_pool, v_pool, tab_d, lens_d, qs, scale, C, k_scale, v_scale, out=out)

    pkv.set_prefill_waves(args.prefill_waves)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    flops = 4.0 * H_q * D * B * sum(p + 1 for p in range(prior, n))
    kv_bytes = B * n * H_kv * D * 2 * (1 if fp8 else 2)
    avg_s = ms.mean() / 1e3
    tf = flops / avg_s / 1e12
    print(f"# prefill: {K} timed calls, average {avg_s * 1e6:.1f} us, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    wkey = f"prefill_{args.prefill_kv}_{B}x{prior}+{C}" + ("" if (H_q, D) == (64, 128) else f"_hq{H_q}_d{D}")
    res = {
        "metric": "paged prefill TFLOP/s (causal, bf16 MFMA)", "value": round(tf, 1), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic (N(0,1) K/V/q, allocator-scattered tables)",
        "config": {"workload": f"{B} sequences x ({prior} earlier + {C} new tokens), "
                               + ("70B layer shape " if (H_q, D) == (64, 128) else "")
                               + f"(H_q {H_q}, H_kv 8, D {D}, bs 16), {args.prefill_kv} KV", "seqs": B, "prior": prior,
                   "chunk": C, "kv": args.prefill_kv, "prefill_waves": args.prefill_waves or "auto"},
        "us_p50": round(float(np.median(ms)) * 1e3, 1), "flops_per_call": flops,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tf, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4), "avg_launch_us": round(avg_s * 1e6, 2),
                     "traffic": measured_traffic(wkey, PREFILL_COUNTERS, PREFILL_SOURCE),
                     "algorithmic_bytes_per_launch": kv_bytes + B * C * H_q * D * (2 + 4) + B * 4 * 2},
        "kv_bytes": kv_bytes, "kv_GBps": round(kv_bytes / avg_s / 1e9, 1)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(torch, k_pool, v_pool, q, out, tab, lens, qs, scale, bs, fp8,
                                                   k_scale, v_scale, prior, C, B, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def prefill_cpu_baseline(torch, k_pool, v_pool, q, out, tab, lens, qs, scale, bs, fp8, k_scale, v_scale, prior, C,
                         B, budget_s):
    """The oracle's causal prefill (numpy fp64) on sampled query rows of the same call, until the
    budget is spent; TFLOP/s counts the sampled rows' causal FLOPs, and the GPU's rows are checked
    against it."""
    import oracle
    kvt = "e4m3" if fp8 else "bf16"

    def host(t):
        return t.cpu().numpy() if fp8 else t.view(torch.int16).cpu().numpy().view(np.uint16)

    kp, vp = host(k_pool), host(v_pool)
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    got = out.cpu().numpy().astype(np.float64)
    ks = None if k_scale is None else k_scale.cpu().numpy()
    vs = None if v_scale is None else v_scale.cpu().numpy()
    qs_h = qs.cpu().numpy()
    H_q, D = q.shape[1], q.shape[2]
    rng = np.random.default_rng(23)
    rows, errs, flops = [], [], 0.0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = int(rng.integers(B))
        r = int(qs_h[b]) + int(rng.integers(C))
        ref = oracle.ref_prefill(qh, "bf16", kp, vp, kvt, tab, lens, qs_h, scale, bs, ks, vs, seqs=[b], rows=[r])
        rows.append(r)
        flops += 4.0 * H_q * D * (prior + (r - int(qs_h[b])) + 1)
        errs.append(float((np.abs(got[r] - ref[r]).max(-1) / np.abs(ref[r]).max(-1)).max()))
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{len(rows)} query rows (all heads) drawn at random from the call, numpy fp64 gather-then-"
                      "attend over each row's causal range",
            "query_rows_per_s": round(len(rows) / dt, 2), "seconds": round(dt, 2), "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "gpu_vs_oracle_max_row_rel_err": float(max(errs))}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the process's CPU affinity
        return len(os.sched_getaffinity(0))


def cpu_baseline(case, mat, out_dev, budget_s, by, B, threads=None, max_sample=16):
    """The oracle (numpy fp64 gather-then-attend) on a bounded sample of the same batch (with
    `threads` BLAS threads, else as many as numpy takes): passes over up to `max_sample`
    sequences spread over the batch until `budget_s` seconds are spent."""
    if threads is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(threads):
            r = cpu_baseline(case, mat, out_dev, budget_s, by, B, max_sample=max_sample)
        r["cores"] = threads
        return r
    import oracle

    spec = case.spec
    sd = "f32" if spec.kv_dtype == "f32" else "bf16"
    sample = list(range(0, B, max(1, B // max_sample)))[:max_sample]
    used = set()
    for b in sample:
        used.update(int(x) for x in mat.block_tables[b, :-(-int(mat.context_lens[b]) // case.bs)])
    used = np.array(sorted(used), np.int64)
    kp, vp = oracle.empty_pools(case.NB, spec.H_kv, spec.d, case.bs, spec.kv_dtype)
    for k, v, s in ((mat.k_src, mat.v_src, mat.slots), (mat.step_k, mat.step_v, mat.step_slots)):
        if len(s):
            keep = np.isin(s // case.bs, used)
            kp, vp = oracle.ref_append(kp, vp, k[keep], v[keep], sd, s[keep], case.bs, spec.kv_dtype,
                                       case.k_scale, case.v_scale)
    got = out_dev.cpu().numpy().astype(np.float64)
    rows, errs = [], []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:  # passes over the sample until the budget is spent
        for b in sample:
            ref = oracle.ref_decode(case.q, spec.q_dtype, kp, vp, spec.kv_dtype, mat.block_tables,
                                    mat.context_lens, case.scale, case.bs, case.k_scale, case.v_scale, rows=[b])
            rows.append(b)
            den = np.abs(ref[b]).max(-1)
            errs.append(float((np.abs(got[b] - ref[b]).max(-1) / den).max()))
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    toks = int(sum(int(mat.context_lens[b]) for b in rows))
    kv = toks * spec.H_kv * spec.d * 2 * {"bf16": 2, "e4m3": 1, "f32": 4}[spec.kv_dtype]
    blas = _blas_threads()
    return {
        "value": round(len(rows) / dt, 3), "unit": "sequences/s", "cores": int(blas), "kind": "oracle",
        "sample": f"{len(rows)} sequence decodes drawn from {len(sample)} of the {B} sequences ({toks} tokens, "
                  f"all heads), numpy fp64 gather-then-attend",
        "kv_GBps": round(kv / dt / 1e9, 3), "seconds": round(dt, 2), "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "gpu_vs_oracle_max_row_rel_err": float(max(errs)),
    }


if __name__ == "__main__":
    main()
