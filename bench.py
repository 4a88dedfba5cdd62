#!/usr/bin/env python3
"""Paged decode-attention benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: copy-on-write block copies
(configuration 4 only), the slot write of the step's new tokens (configurations 1, 3,
4), then decode attention over every sequence (split-KV partitions + merge). Inputs
are synthetic and seeded (workload.py) and resident in HBM before timing starts.

The pool is replicated R times (default 3) and step i uses replica i % R, so that a
step never finds the previous step's KV in the 256 MB Infinity Cache or the L2s.

Output: one JSON line on stdout. `value` is KV-read GB/s over the whole step
(sum_b L_b * 2 * Hkv * d * bytes / step time); `tokens_per_s` is sequences (one new
token each) per second for this one attention layer. `roofline` describes the decode
launch (main + merge kernels): its duration is the mean per launch of the timed steps'
launches replayed from a HIP graph, as a serving loop runs its decode steps (events around
each replay on the stream it runs on; every replay must reproduce the eager output). The
mean of per-launch event pairs in the eager timed region, which adds the stream's kernel
boundary and a marker before and after each call, and its p10/p50/p90 are reported
beside it. It sets its bandwidth against the 8 TB/s peak and
against a read ceiling measured on the same GPU after the timed region (pa_stream_read
over 4 GiB: the library's streaming-read kernel, the best a read-only kernel does here;
a 1 GiB device copy, bytes read plus written, is reported beside it). With the default
workload (3) the Llama-2-7B fp16, prefix-sharing and long-context fp8 workloads (2, 4, 5)
are measured the same way afterwards and reported under `other_workloads`, one
chunked-prefill step (see --path prefill, 20 timed steps) under `prefill`, and the tiny fp32
workload's per-call GPU time from a HIP graph under `tiny_workload_latency`.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the main workload.

With --path prefill the step is one chunked-prefill step instead (workload.chunked_prefill:
16 prompts x 512 new tokens over contexts of up to 8192): the slot write of the chunk's
K/V, then causal multi-token attention (pa_prefill). Its value is attention TFLOP/s
counting only the unmasked work, 4 * d * Hq flops per (query token, attended position),
and its roofline is the bf16 matrix-core peak.

With --path swap the step is a preemption by swapping: 16 384 Llama-3-8B-shaped blocks
(8 kv heads, d=128, bf16: 64 KiB of K and V each, 1 GiB in all) move from the device pool
to a pinned host pool with pa_block_swap and back; value is GB/s per direction against the
host link (PCIe 5.0 x16, 64 GB/s per direction). With --path manager the step is the host
bookkeeping of one decode step of the Llama-3-8B workload (256 sequences, lognormal
lengths): one appended token per sequence (one pa_bm_append_batch call) plus the export of
the block tables (one pa_bm_tables call); value is steps per second, the oracle's Python
manager as baseline.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--config 3]
                       [--path decode|prefill|swap|manager] [--batch B] [--context MIN MAX]
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

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode KV-read GB/s (% HBM peak) & tokens/s, 8B GQA bf16 layer"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published peak
PREFILL_METRIC = "paged-attn chunked-prefill attention TFLOP/s (causal, algorithmic), 8B GQA bf16 layer"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_367_amd", "csrc", f)
                  for f in ("pa_decode.hip", "pa_device.h")]
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_traffic.md")
PREFILL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_367_amd", "csrc", f)
                   for f in ("pa_prefill.hip", "pa_device.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(sources=None) -> str:
    """sha256 (first 16 hex digits) of a kernel's sources (default: the decode's),
    concatenated."""
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(config_name: str, path: str = TRAFFIC_FILE, sources=None):
    """HBM bytes per launch from a committed counter summary, or None when the summary is
    missing or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not h or h.group(1) != kernel_source_hash(sources):
        return None
    m = re.search(rf"traffic_bytes_per_launch\[{re.escape(config_name)}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def copy_ceiling_gbs(mib: int = 1024, reps: int = 5) -> float:
    """Measured HBM ceiling on this GPU: a device-to-device copy of `mib` MiB (torch's
    copy kernel), bytes read plus bytes written per second, best of `reps`."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2 * n / (best * 1e-3) / 1e9


def read_ceiling_gbs(gib: int = 4, reps: int = 5) -> float:
    """Measured read-only HBM ceiling on this GPU: pa_stream_read over `gib` GiB (far
    larger than the caches), bytes read per second, best of `reps`."""
    import torch
    import paged_kv_cache_367_amd as pa
    n = gib << 30
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    pa.pa_stream_read(buf, sink)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pa.pa_stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del buf, sink
    return n / (best * 1e-3) / 1e9


def cpu_baseline(w, gpu_out, k_after, v_after, budget_s: float):
    """Time the oracle on sequences in a seeded order until ~budget_s of CPU work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:  # noqa: BLE001 - reporting only
        threads = None
    order = np.random.default_rng(0).permutation(w.batch)
    done, t0 = [], time.perf_counter()
    refs = []
    for b in order:
        refs.append(oracle.decode_ref(w.q, k_after, v_after, w.block_tables, w.context_lens,
                                      w.scale, q_kind=w.q_dtype, kv_kind=w.kv_dtype,
                                      k_scale=w.k_scale, v_scale=w.v_scale, seqs=[int(b)]))
        done.append(int(b))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    L = w.context_lens[done].astype(np.int64)
    kv = int(L.sum()) * 2 * w.num_kv_heads * w.head_dim * {"f32": 4, "f16": 2, "bf16": 2,
                                                           "fp8_e4m3": 1}[w.kv_dtype]
    err = float(np.max(np.abs(gpu_out[done] - np.concatenate(refs, 0))))
    return {
        "value": kv / dt / 1e9, "unit": "GB/s", "tokens_per_s": len(done) / dt,
        "cores": threads, "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": f"{len(done)} of {w.batch} sequences ({int(L.sum())} tokens), fp64 numpy, "
                  f"{dt:.1f} s",
        "sample_max_abs_err_vs_gpu": err,
    }


def prefill_flops(w) -> float:
    """Unmasked attention work: 4 * d * Hq flops (2 for q.k, 2 for p.v) per query token
    and attended position; token i of a sequence with L cached and n new tokens attends
    over L - n + i + 1 positions."""
    import numpy as np
    L = w.context_lens.astype(np.int64)
    n = w.query_lens
    pairs = n * (L - n) + n * (n + 1) // 2
    return float(4 * w.head_dim * w.num_q_heads * int(pairs.sum()))


def prefill_cpu_baseline(w, gpu_out, budget_s: float):
    """Time the oracle on query rows in a seeded order until ~budget_s of CPU work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:  # noqa: BLE001 - reporting only
        threads = None
    order = np.random.default_rng(0).permutation(w.num_query_tokens)
    seq_of = np.searchsorted(w.query_start, np.arange(w.num_query_tokens), side="right") - 1
    done, flops, err = [], 0.0, 0.0
    t0 = time.perf_counter()
    for r in order:
        ref = oracle.prefill_ref(w.q, w.query_start, w.k_pool, w.v_pool, w.block_tables,
                                 w.context_lens, w.scale, q_kind=w.q_dtype, kv_kind=w.kv_dtype,
                                 k_scale=w.k_scale, v_scale=w.v_scale, rows=[int(r)])
        b = int(seq_of[r])
        pos = int(w.context_lens[b]) - int(w.query_lens[b]) + int(r - w.query_start[b])
        flops += 4.0 * w.head_dim * w.num_q_heads * (pos + 1)
        err = max(err, float(np.max(np.abs(gpu_out[r] - ref[r]))))
        done.append(int(r))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
        "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": f"{len(done)} of {w.num_query_tokens} query rows (all {w.num_q_heads} heads), "
                  f"fp64 numpy, {dt:.1f} s",
        "sample_max_abs_err_vs_gpu": err,
    }


def run_prefill(args) -> int:
    record = prefill_record(args, args.steps, args.warmup, not args.no_cpu_baseline)
    print(json.dumps(record), flush=True)
    return 0


def prefill_record(args, steps, warmup, with_cpu_baseline):
    """One chunked-prefill step (slot write of the chunk's K/V, then pa_prefill) timed over
    `steps` steps after `warmup` untimed ones; returns the JSON record."""
    import numpy as np
    import torch

    import paged_kv_cache_367_amd as pa
    import workload as wl

    log("building the chunked-prefill workload")
    t0 = time.perf_counter()
    w = wl.chunked_prefill()
    B = w.batch
    log(f"workload {w.name}: B={B} query tokens={w.num_query_tokens} "
        f"context tokens={int(w.context_lens.sum())} pool_blocks={w.num_blocks} "
        f"({time.perf_counter() - t0:.1f} s)")
    # the chunk's own K/V rows, written to their slots at the start of every step (the
    # values already there, so every step computes the same thing)
    L = w.context_lens.astype(np.int64)
    tok_seq = np.repeat(np.arange(B), w.query_lens)
    pos = L[tok_seq] - w.query_lens[tok_seq] + (np.arange(w.num_query_tokens) -
                                                w.query_start[tok_seq])
    slots = w.block_tables[tok_seq, pos // 16].astype(np.int64) * 16 + pos % 16
    k_new = w.k_pool.reshape(-1, w.num_kv_heads, w.head_dim)[slots]
    v_new = w.v_pool.reshape(-1, w.num_kv_heads, w.head_dim)[slots]

    def dev(a, kind=None):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if kind == "bf16" \
            else torch.from_numpy(a)
        return t.cuda()

    q = dev(w.q, w.q_dtype)
    tables, lens, qs = dev(w.block_tables), dev(w.context_lens), dev(w.query_start)
    R = max(1, args.replicas)
    ks = [dev(w.k_pool, w.kv_dtype) for _ in range(R)]
    vs = [dev(w.v_pool, w.kv_dtype) for _ in range(R)]
    d_slots = dev(slots)
    d_knew, d_vnew = dev(k_new, w.kv_dtype), dev(v_new, w.kv_dtype)
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log(f"resident: {R} pool replicas")
    flops = prefill_flops(w)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]

    def step(i, timed):
        r = i % R
        pa.pa_cache_write(ks[r], vs[r], d_knew, d_vnew, d_slots)
        if timed:
            ev0[i].record()
        pa.pa_prefill(out, q, ks[r], vs[r], tables, lens, qs, w.max_query_len, w.scale,
                      w.k_scale, w.v_scale)
        if timed:
            ev1[i].record()

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    log(f"warmup done ({warmup} steps)")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i, True)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    lms = [a.elapsed_time(b) for a, b in zip(ev0, ev1)]
    lavg = sum(lms) / len(lms)
    log(f"timed {steps} steps: {ms:.4f} ms/step, prefill launch avg {lavg:.4f} ms "
        f"(min {min(lms):.4f}, max {max(lms):.4f})")
    achieved = flops / (lavg * 1e-3) / 1e12
    record = {
        "metric": PREFILL_METRIC, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded, workload.py)",
        "config": {
            "workload": w.name, "batch": B, "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": 16,
            "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype, "accumulate": "f32",
            "query_tokens": w.num_query_tokens, "context_tokens": int(L.sum()),
            "max_query_len": w.max_query_len, "flops_per_step": flops, "pool_replicas": R,
            "seed": w.seed,
        },
        "query_tokens_per_s": w.num_query_tokens / (ms * 1e-3),
        "roofline": {
            "kernel": "pa_prefill (prefill_kernel)", "bound": "mfma", "achieved": achieved,
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
            "traffic": read_traffic(w.name, PREFILL_TRAFFIC_FILE, PREFILL_SOURCES),
            "launch_ms": lavg,
            "algorithmic_flops_per_launch": flops,
        },
        "cpu_baseline": None,
    }
    if with_cpu_baseline:
        log(f"cpu baseline: timing the oracle (~{args.cpu_budget_s:.0f} s)")
        gpu_out = out.to(torch.float64).cpu().numpy()
        record["cpu_baseline"] = prefill_cpu_baseline(w, gpu_out, args.cpu_budget_s)
        log(f"cpu baseline: {record['cpu_baseline']['sample']}")
    return record


PCIE_PEAK_GBS = 64.0        # PCIe 5.0 x16 host link, per direction


def run_swap(args) -> int:
    import numpy as np
    import torch

    import paged_kv_cache_367_amd as pa

    nblk, Hkv, d = 16384, 8, 128
    Nd = nblk + 1024
    rng = np.random.default_rng(367)
    log(f"swap: {nblk} blocks of {16 * Hkv * d * 2} B per pool (K and V), device pool "
        f"{Nd} blocks, pinned host pool {nblk} blocks")
    kd = torch.randn((Nd, 16, Hkv, d), dtype=torch.bfloat16, device="cuda")
    vd = torch.randn((Nd, 16, Hkv, d), dtype=torch.bfloat16, device="cuda")
    kh = torch.empty((nblk, 16, Hkv, d), dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty((nblk, 16, Hkv, d), dtype=torch.bfloat16, pin_memory=True)
    src = rng.choice(Nd, size=nblk, replace=False)            # scattered device blocks
    out_pairs = torch.from_numpy(np.stack([src, np.arange(nblk)], 1).astype(np.int64)).cuda()
    in_pairs = torch.from_numpy(np.stack([np.arange(nblk), src], 1).astype(np.int64)).cuda()
    moved = 2 * kd[0].numel() * kd.element_size() * nblk      # K and V bytes per direction
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_out, t_in = [], []
    for i in range(args.warmup + args.steps):
        ev[0].record()
        pa.pa_block_swap(kh, vh, kd, vd, out_pairs)
        ev[1].record()
        pa.pa_block_swap(kd, vd, kh, vh, in_pairs)
        ev[2].record()
        torch.cuda.synchronize()
        if i >= args.warmup:
            t_out.append(ev[0].elapsed_time(ev[1]))
            t_in.append(ev[1].elapsed_time(ev[2]))
    ms_out, ms_in = sum(t_out) / len(t_out), sum(t_in) / len(t_in)
    g_out, g_in = moved / ms_out / 1e6, moved / ms_in / 1e6
    log(f"swap-out {ms_out:.3f} ms ({g_out:.1f} GB/s), swap-in {ms_in:.3f} ms ({g_in:.1f} GB/s)")
    # a round trip must leave the device blocks as they were
    ok = bool(torch.equal(kd[torch.from_numpy(src).cuda()].view(torch.int16),
                          kh.cuda().view(torch.int16)))
    record = {
        "metric": "paged KV block swap GB/s per direction (device <-> pinned host), 8B GQA bf16 blocks",
        "value": min(g_out, g_in), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_out + ms_in, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (torch.randn on device, seeded block choice)",
        "config": {"workload": "swap_1gib_llama3_8b_blocks", "blocks": nblk, "kv_heads": Hkv,
                   "head_dim": d, "block_size": 16, "bytes_per_direction": moved},
        "swap_out_gbs": g_out, "swap_in_gbs": g_in, "round_trip_exact": ok,
        "roofline": {"kernel": "pa_block_swap (block_swap_kernel)", "bound": "pcie",
                     "achieved": min(g_out, g_in), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": min(g_out, g_in) / PCIE_PEAK_GBS, "traffic": None,
                     "launch_ms": max(ms_out, ms_in), "algorithmic_bytes_per_launch": moved},
        "cpu_baseline": None,
    }
    print(json.dumps(record), flush=True)
    return 0 if ok else 1


def run_manager(args) -> int:
    import numpy as np

    import paged_kv_cache_367_amd as pa
    import workload as wl

    L = wl.config_lengths(3).astype(np.int64)
    B = L.size
    nblk = int(((L + 15) // 16).sum() * 1.1) + B * ((args.steps + args.warmup) // 16 + 2)
    rng = np.random.default_rng(367)

    def setup(m):
        for b in range(B):
            m.add(b, rng.integers(0, 32000, size=int(L[b])).tolist())

    m = pa.BlockManager(nblk, 16, True)
    setup(m)
    width = int((L.max() + args.steps + args.warmup) // 16 + 2)
    ids = np.arange(B, dtype=np.int64)
    toks = rng.integers(0, 32000, size=(args.warmup + args.steps, B))
    for i in range(args.warmup):
        m.append_batch(ids, toks[i])
        m.tables(ids, width)
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        m.append_batch(ids, toks[i])
        m.tables(ids, width)
    dt = (time.perf_counter() - t0) / args.steps
    log(f"manager: {dt * 1e6:.1f} us per decode step of {B} appends + table export")
    record = {
        "metric": "paged KV block-manager decode-step bookkeeping, steps/s (256 sequences)",
        "value": 1.0 / dt, "unit": "steps/s", "n_gpus": 0, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dt * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic (lengths of the Llama-3-8B workload, random token ids)",
        "config": {"workload": "manager_decode_step_llama3_8b", "batch": B, "blocks": nblk,
                   "block_size": 16, "prefix_cache": True,
                   "calls_per_step": "pa_bm_append_batch + pa_bm_tables"},
        "roofline": None, "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle.block_manager as obm
        r = obm.BlockManager(nblk, 16, True)
        rng = np.random.default_rng(367)
        for b in range(B):
            r.add(b, rng.integers(0, 32000, size=int(L[b])).tolist())
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_budget_s, 10.0) and n < args.steps:
            for b in range(B):
                r.append(b, int(toks[n, b]))
            [r.table(b, width) for b in range(B)]
            n += 1
        rdt = (time.perf_counter() - t0) / max(n, 1)
        record["cpu_baseline"] = {"value": 1.0 / rdt, "unit": "steps/s", "cores": 1,
                                  "kind": "oracle", "sample": f"{n} decode steps of {B} appends"}
    print(json.dumps(record), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = Llama-3-8B GQA bf16)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="tokens per split-KV partition (default: the workload's, else the library's)")
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--batch", type=int, default=None,
                    help="decode: override the workload's sequence count (its shape otherwise)")
    ap.add_argument("--context", type=int, nargs=2, default=None, metavar=("MIN", "MAX"),
                    help="decode: clip the workload's context lengths into [MIN, MAX]")
    ap.add_argument("--path", choices=["decode", "prefill", "swap", "manager"], default="decode",
                    help="decode (the default step), one chunked-prefill step, a block swap "
                         "to pinned host memory and back, or the host block manager")
    ap.add_argument("--extra-configs", default=None,
                    help="decode: other workloads measured after the main one and reported "
                         "under other_workloads (comma list, or 'none'; default 2,4,5 with "
                         "the default --config 3, else none)")
    ap.add_argument("--latency", action="store_true",
                    help="decode: also time pa_decode calls replayed from a HIP graph (GPU time "
                         "per call without host gaps; what small batches should be judged by)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, copy a buffer of this many MiB a few "
                         "times (a reference kernel of known traffic for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported. Each GPU would own a disjoint set of "
              "sequences and pool blocks, so no multi-GPU figure is produced.", file=sys.stderr)
        return 2

    if args.path == "manager":                 # host bookkeeping only: no GPU needed
        return run_manager(args)

    import numpy as np
    import torch

    import paged_kv_cache_367_amd as pa
    import workload as wl

    pa.load_library()          # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 3}), flush=True)
        return 0

    if args.path == "prefill":
        return run_prefill(args)
    if args.path == "swap":
        return run_swap(args)

    log(f"building workload {args.config}")
    t0 = time.perf_counter()
    w = wl.make(args.config, batch=args.batch,
                len_range=tuple(args.context) if args.context else None)
    if args.batch is not None or args.context is not None:      # not the named workload
        w.name = f"{w.name}_b{w.batch}_L{int(w.context_lens.min())}-{int(w.context_lens.max())}"
    log(f"workload {w.name}: B={w.batch} tokens={w.total_tokens} kv_bytes={w.kv_bytes} "
        f"pool_blocks={w.num_blocks} ({time.perf_counter() - t0:.1f} s)")
    part = args.partition_size if args.partition_size is not None else w.partition_size
    m = measure_decode(w, part, args.steps, args.warmup, args.replicas)
    read_gbs = read_ceiling_gbs()
    copy_gbs = copy_ceiling_gbs()
    log(f"ceilings on this GPU: streaming read {read_gbs:.0f} GB/s, device copy "
        f"{copy_gbs:.0f} GB/s (read + write)")
    record = decode_record(w, part, m, args)
    rf = record["roofline"]
    if args.latency:
        us, same = graph_latency(w, part)
        rf["graph_launch_us"] = us
        rf["graph_replays_match_eager"] = same
        log(f"{w.name}: pa_decode from a HIP graph: {us:.1f} us per call (replays equal the "
            f"eager output: {same})")
    rf["read_ceiling_gbs"] = read_gbs
    rf["frac_of_read_ceiling"] = rf["achieved"] / read_gbs
    rf["copy_ceiling_gbs"] = copy_gbs
    extra_arg = args.extra_configs if args.extra_configs is not None else \
        ("2,4,5" if args.config == 3 else "none")
    extra = [] if extra_arg in ("", "none") else \
        [int(x) for x in extra_arg.split(",") if int(x) != args.config]
    if args.batch is not None or args.context is not None:
        extra = []
    if extra:
        record["other_workloads"] = []
        for idx in extra:
            log(f"building workload {idx}")
            wx = wl.make(idx)
            mx = measure_decode(wx, wx.partition_size, min(args.steps, 20), args.warmup,
                                args.replicas)
            rx = decode_record(wx, wx.partition_size, mx, args)
            sub = {k: rx[k] for k in ("value", "unit", "ms_per_step", "tokens_per_s",
                                      "hbm_frac", "dtype", "steps")}
            sub["config"] = rx["config"]
            sub["roofline"] = {k: rx["roofline"][k] for k in (
                "kernel", "bound", "achieved", "peak", "unit", "frac", "traffic", "launch_ms",
                "launch_ms_events_each", "algorithmic_bytes_per_launch")}
            sub["roofline"]["frac_of_read_ceiling"] = rx["roofline"]["achieved"] / read_gbs
            record["other_workloads"].append(sub)
            del mx
            torch.cuda.empty_cache()
    if extra:
        # the multi-token (chunked-prefill) step, fewer steps, no oracle timing
        log("multi-token queries: one chunked-prefill step")
        rp = prefill_record(args, min(args.steps, 20), 5, False)
        record["prefill"] = {k: rp[k] for k in ("metric", "value", "unit", "ms_per_step",
                                                "steps", "dtype")}
        record["prefill"]["config"] = {k: rp["config"][k] for k in (
            "workload", "batch", "query_tokens", "context_tokens", "flops_per_step")}
        record["prefill"]["roofline"] = {k: rp["roofline"][k] for k in (
            "kernel", "bound", "achieved", "peak", "unit", "frac", "traffic", "launch_ms")}
        del rp
        torch.cuda.empty_cache()
        # the tiny fp32 workload is latency-bound: GPU time per call from a HIP graph
        wt = wl.make(1)
        us, same = graph_latency(wt, 0)
        record["tiny_workload_latency"] = {
            "workload": wt.name, "graph_launch_us": us, "graph_replays_match_eager": same,
            "batch": wt.batch, "context_tokens": wt.total_tokens}
        log(f"{wt.name}: pa_decode from a HIP graph: {us:.1f} us per call")
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: applying the step's writes to host pools")
        k_after, v_after = w.k_pool, w.v_pool
        if w.copy_pairs is not None:
            k_after = oracle.block_copy_ref(k_after, w.copy_pairs)
            v_after = oracle.block_copy_ref(v_after, w.copy_pairs)
        if w.slot_mapping is not None:
            k_after = oracle.cache_write_ref(k_after, w.k_new, w.slot_mapping)
            v_after = oracle.cache_write_ref(v_after, w.v_new, w.slot_mapping)
        log(f"cpu baseline: timing the oracle (~{args.cpu_budget_s:.0f} s)")
        record["cpu_baseline"] = cpu_baseline(w, m["out"], k_after, v_after, args.cpu_budget_s)
        log(f"cpu baseline: {record['cpu_baseline']['sample']}")
    print(json.dumps(record), flush=True)
    return 0


def measure_decode(w, part, steps, warmup, replicas):
    """Time `steps` decode steps (copy-on-write copies, slot writes, pa_decode) of workload
    w after `warmup` untimed ones, the pool replicated `replicas` times (step i uses
    replica i % replicas). Returns the step time, the pa_decode launch times (HIP events
    on the stream the kernels run on) and the last output as float64 numpy."""
    import numpy as np
    import torch

    import paged_kv_cache_367_amd as pa

    def dev(a, kind=None):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if kind == "bf16" \
            else torch.from_numpy(a)
        return t.cuda()

    q = dev(w.q, w.q_dtype)
    tables, lens = dev(w.block_tables), dev(w.context_lens)
    R = max(1, replicas)
    ks = [dev(w.k_pool, w.kv_dtype) for _ in range(R)]
    vs = [dev(w.v_pool, w.kv_dtype) for _ in range(R)]
    slots = dev(w.slot_mapping) if w.slot_mapping is not None else None
    k_new = dev(w.k_new, w.kv_dtype) if w.k_new is not None else None
    v_new = dev(w.v_new, w.kv_dtype) if w.v_new is not None else None
    pairs = dev(w.copy_pairs) if w.copy_pairs is not None else None
    out_dtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.out_dtype]
    out = torch.empty(tuple(w.q.shape), dtype=out_dtype, device="cuda")
    desc = pa.binding.make_desc(q, ks[0], tables, out, part)
    ws_bytes = pa.pa_decode_workspace_bytes(desc, w.max_context_len)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    chunks = pa.pa_decode_max_chunks(desc, w.max_context_len)
    torch.cuda.synchronize()
    log(f"{w.name}: resident: {R} pool replicas, workspace {ws_bytes} B, up to {chunks} "
        f"work chunks")
    dec0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    dec1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]

    def step(i, timed):
        r = i % R
        if pairs is not None:
            pa.pa_block_copy(ks[r], vs[r], pairs)
        if slots is not None:
            pa.pa_cache_write(ks[r], vs[r], k_new, v_new, slots)
        if timed:
            dec0[i].record()
        pa.pa_decode(out, q, ks[r], vs[r], tables, lens, w.max_context_len, w.scale, w.k_scale,
                     w.v_scale, workspace=ws, partition_size=part)
        if timed:
            dec1[i].record()

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i, True)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    dec_ms = [a.elapsed_time(b) for a, b in zip(dec0, dec1)]
    dec_avg = sum(dec_ms) / len(dec_ms)
    srt = sorted(dec_ms)
    pct = lambda f: srt[min(len(srt) - 1, int(f * len(srt)))]
    eager = out.clone()
    out_np = out.to(torch.float64).cpu().numpy()
    # the same launches (replicas still rotating) captured in a HIP graph and replayed, as a
    # serving loop runs its decode steps: HIP events around each replay on the stream it
    # runs on, mean per launch; every replay must write the eager output again
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            r = i % R
            pa.pa_decode(out, q, ks[r], vs[r], tables, lens, w.max_context_len, w.scale,
                         w.k_scale, w.v_scale, workspace=ws, partition_size=part)
    torch.cuda.synchronize()
    graph_ms, same = [], True
    for _ in range(3):
        out.zero_()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        graph_ms.append(start.elapsed_time(end) / steps)
        same &= bool(torch.equal(out, eager))
    del g
    if not same:
        raise RuntimeError(f"{w.name}: graph replays did not reproduce the eager output")
    glaunch = sum(graph_ms) / len(graph_ms)
    log(f"{w.name}: timed {steps} steps: {ms:.4f} ms/step, decode launch avg {dec_avg:.4f} ms "
        f"(min {min(dec_ms):.4f}, max {max(dec_ms):.4f}); from a HIP graph {glaunch:.4f} ms "
        f"per launch")
    res = {"ms": ms, "launch_ms": glaunch, "launch_ms_events": dec_avg,
           "pct": [pct(0.1), pct(0.5), pct(0.9)],
           "chunks": chunks, "replicas": R, "steps": steps, "out": out_np}
    del ks, vs, ws
    return res


def graph_latency(w, part, launches=40, reps=5, replicas=3):
    """GPU time of one pa_decode call without host gaps: `launches` calls (cycling over the
    pool replicas) captured in one HIP graph, replayed `reps` times, (replay time) /
    launches, best of the replays. Small batches take less GPU time per call than the host
    takes to submit one, so events around single calls would time the host. Returns
    (microseconds per call, output of the replays equals the eager output)."""
    import numpy as np
    import torch

    import paged_kv_cache_367_amd as pa

    def dev(a, kind=None):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if kind == "bf16" \
            else torch.from_numpy(a)
        return t.cuda()

    q = dev(w.q, w.q_dtype)
    tables, lens = dev(w.block_tables), dev(w.context_lens)
    R = max(1, replicas)
    ks = [dev(w.k_pool, w.kv_dtype) for _ in range(R)]
    vs = [dev(w.v_pool, w.kv_dtype) for _ in range(R)]
    out_dtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.out_dtype]
    out = torch.empty(tuple(w.q.shape), dtype=out_dtype, device="cuda")
    desc = pa.binding.make_desc(q, ks[0], tables, out, part)
    ws = torch.empty(max(pa.pa_decode_workspace_bytes(desc, w.max_context_len), 16),
                     dtype=torch.uint8, device="cuda")

    def call(r):
        pa.pa_decode(out, q, ks[r], vs[r], tables, lens, w.max_context_len, w.scale,
                     w.k_scale, w.v_scale, workspace=ws, partition_size=part)

    call(0)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            call(i % R)
    best, same = float("inf"), True
    for _ in range(reps):
        out.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
        same &= bool(torch.equal(out, eager))
    del g, ks, vs, ws
    return best * 1e3 / launches, same


def decode_record(w, part, m, args):
    """The JSON record of one measured decode workload."""
    gbs = w.kv_bytes / (m["ms"] * 1e-3) / 1e9
    achieved = w.kv_bytes / (m["launch_ms"] * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": m["steps"],
        "warmup": args.warmup, "ms_per_step": m["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3"}[w.kv_dtype],
        "data": "synthetic (seeded, workload.py)",
        "config": {
            "workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
            "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype, "accumulate": "f32",
            "context_tokens": w.total_tokens, "max_context_len": w.max_context_len,
            "kv_bytes_per_step": w.kv_bytes, "partition_size": part,
            "max_work_chunks": m["chunks"], "pool_replicas": m["replicas"], "seed": w.seed,
        },
        "tokens_per_s": w.batch / (m["ms"] * 1e-3),
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "roofline": {
            "kernel": "pa_decode (decode_kernel + merge kernel)", "bound": "hbm",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": read_traffic(w.name),
            "launch_ms": m["launch_ms"], "algorithmic_bytes_per_launch": w.kv_bytes,
            "launch_timing": "the timed steps' pa_decode launches replayed from a HIP graph "
                             "(3 replays, outputs checked against the eager run), HIP events "
                             "around each replay on its stream, mean per launch",
            "launch_ms_events_each": m["launch_ms_events"],
            "launch_ms_events_each_p10_p50_p90": m["pct"],
        },
        "cpu_baseline": None,
    }


if __name__ == "__main__":
    sys.exit(main())
