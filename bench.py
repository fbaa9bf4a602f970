#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one pass of the whole decode hot path over one batch: the cache
append of one new token per sequence, then paged decode attention
(paged_decode_step: the append rides in the work-plan launch, followed by the
partition kernel and the log-sum-exp merge).  A second pass times the phases
one by one (paged_kv_append, paged_decode_attention_plan / _partitions /
_merge).  Host slot allocation is done once before timing (the tables already
list the slot), and the append rewrites the same bytes every step, so the
timed steps are identical.

Default workload: the 70B-shaped GQA decode batch (64 query / 8 KV heads of
128, bf16, B = 16, 256 sequences with log-uniform lengths in [512, 8192],
pool of 1.1x the needed blocks with shuffled ids), drawn on the GPU.

`--workload prefill` times the chunked-prefill path instead: the
multi-token append of 16 whole prompts and causal prefill attention over
them (tokens/s, with the attention kernel priced against the MFMA peak).

Prints one JSON line.  `value` is KV GB/s over the whole step: valid key and
value bytes of every sequence, divided by the step time.  The `roofline`
object prices the partition kernel (the dominant one) against the 8 TB/s HBM
peak, timed with HIP events on the stream it runs on.  `cpu_baseline` is the
float64 CPU oracle on a sample of the same batch, on a pool of worker
processes (one per usable core, at most 16), each with one BLAS thread.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))

WORKLOAD_DESC = {
    1: "tiny fp32: 2 q / 1 kv heads, D 16, B 4, lengths 10/5/13, pool 16 blocks",
    2: "13B-shaped MHA bf16: 40 q = 40 kv heads, D 128, B 16, batch 64, lengths U[64,2048], pool 16384 blocks",
    3: "70B-shaped GQA bf16: 64 q / 8 kv heads, D 128, B 16, batch 256, lengths log-uniform [512,8192], pool 1.1x needed",
    4: "shared-prefix GQA fp16: 32 q / 8 kv heads, D 128, B 16, batch 128, 1024-token shared prefix + U[1,512] private",
    5: "long-context GQA bf16: 64 q / 8 kv heads, D 128, batch 8, lengths U[8192,32768]",
}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", choices=["decode", "prefill", "swap", "cascade"],
                    default="decode",
                    help="decode: the paged decode step on --config (default); prefill: "
                         "multi-token append + causal chunked-prefill attention on a batch of "
                         "16 whole prompts (32 q / 8 kv heads of 128, bf16, B 16); swap: "
                         "preempt a quarter of --config's sequences to pinned host memory "
                         "and back")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--batch", type=int, default=None,
                    help="cascade workload: sequences sharing the prefix (default: config 4's 128)")
    ap.add_argument("--prefix-tokens", type=int, default=1024,
                    help="cascade workload: shared prefix length in tokens (default: config 4's "
                         "1024; a multiple of the block size)")
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="0 = balanced ranges; > 0 = also cap each range at this many tokens")
    ap.add_argument("--kernel", choices=["auto", "valu", "mfma"], default="auto")
    ap.add_argument("--kv-dtype", choices=["native", "fp8"], default="native",
                    help="fp8: E4M3FN pools with per-pool scales (q / out keep the config dtype)")
    ap.add_argument("--cache-kv", choices=["auto", "on", "off"], default="auto",
                    help="PKV_ATTN_CACHE_KV: auto = on when the tables share blocks")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled parity check")
    ap.add_argument("--copy-gib", type=float, default=2.0,
                    help="size of the device-to-device copy that measures practical bandwidth")
    ap.add_argument("--calibrate", action="store_true",
                    help="after timing, run three plain kernels of known size on a 1 GiB fp32 "
                         "buffer written at start-up (read-only sum, fill, elementwise copy) so "
                         "that rocprofv3 FETCH_SIZE / WRITE_SIZE can be scaled to bytes")
    return ap.parse_args(argv)


CSRC = os.path.join(ROOT, "paged_kv_cache_116_amd", "csrc")
# The source file that defines each profiled kernel.
KERNEL_SOURCES = {
    "attn_partition_mfma": "decode_attention.hip",
    "attn_partition_valu": "decode_attention.hip",
    "attn_plan": "decode_attention.hip",
    "attn_merge": "decode_attention.hip",
    "attn_prefill_mfma": "prefill_attention.hip",
    "cascade": "cascade.hip",
    "swap_kernel": "kv_cache_ops.hip",
    "append_kernel": "kv_cache_ops.hip",
}


def _source_closure(path: str, seen: set) -> None:
    """path and every file it includes with #include "...", recursively."""
    path = os.path.normpath(path)
    if path in seen or not os.path.exists(path):
        return
    seen.add(path)
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#include \""):
                _source_closure(os.path.join(os.path.dirname(path), line.split('"')[1]), seen)


def kernel_source_digest(kernel: str = "attn_partition_mfma") -> str:
    """SHA-256 (first 16 hex digits) of the source file that defines `kernel`
    and of every header it includes, so that a profile taken on other code
    shows as stale.  The cascade also runs the decode and prefill kernels."""
    files: set = set()
    roots = ([KERNEL_SOURCES[kernel]] if kernel != "cascade" else
             ["cascade.hip", "decode_attention.hip", "prefill_attention.hip"])
    for name in roots:
        _source_closure(os.path.join(CSRC, name), files)
    h = hashlib.sha256()
    for path in sorted(files):
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per partition launch from committed rocprofv3 counter runs,
    used only while the kernel source is the one that was profiled."""
    path = os.path.join(ROOT, "profiles", "partition_kernel_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(workload, {}).get(kernel)
    if not entry or entry.get("source_digest") != kernel_source_digest("attn_partition_" + kernel):
        return None
    return entry.get("traffic_bytes")


def _oracle_worker(job):
    """One CPU-baseline worker: the float64 oracle (append + gather attention)
    on its share of the sampled sequences, repeated until `seconds` of its
    own time are spent, BLAS limited to one thread.  Runs in a fresh
    interpreter (spawn), which never touches the GPU."""
    import threadpoolctl
    sys.path.insert(0, ROOT)
    from oracle import attention as o_attn
    from oracle import cache_ops as o_cache
    from oracle import fp8 as o_fp8
    c, B, scale, fp8, k_scale, v_scale, seconds = job
    passes, spent = 0, 0.0
    with threadpoolctl.threadpool_limits(1):
        while spent < seconds:
            t = time.perf_counter()
            if fp8:
                kc, vc = o_fp8.append_token_fp8(c["k_pool"], c["v_pool"], c["k_new"], c["v_new"],
                                                c["tables"], c["lens_pre"], B, k_scale, v_scale)
                kp, vp = o_fp8.dequantise(kc, k_scale), o_fp8.dequantise(vc, v_scale)
            else:
                kp, vp = o_cache.append_token(c["k_pool"], c["v_pool"], c["k_new"], c["v_new"],
                                              c["tables"], c["lens_pre"], B)
            o_attn.decode_attention(c["q"], kp, vp, c["tables"], c["lens"], B, scale)
            spent += time.perf_counter() - t
            passes += 1
    return passes, spent


def cpu_oracle_baseline(w, workloads, sample, seconds, fp8):
    """The oracle on a process pool: one worker per usable core (the
    process's CPU affinity, at most 16, the host share of one GPU), each on
    its own slice of the sampled sequences for about `seconds`; returns
    (KV bytes/s, sequences/s, workers)."""
    import concurrent.futures
    import multiprocessing
    n = max(1, min(len(os.sched_getaffinity(0)), 16, len(sample)))
    chunks = [sample[i::n] for i in range(n)]
    jobs = [(workloads.extract_sequences(w, ch, dtype=np.float32), w.block_size, w.scale, fp8,
             w.k_scale, w.v_scale, seconds) for ch in chunks]
    row = w.num_kv_heads * w.head_dim * 2 * w.k_pool.element_size()
    kv = [int(j[0]["lens"].astype(np.int64).sum()) * row for j in jobs]
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    os.environ.update({k: "1" for k in saved})
    try:
        ctx = multiprocessing.get_context("spawn")
        with concurrent.futures.ProcessPoolExecutor(n, mp_context=ctx) as ex:
            res = list(ex.map(_oracle_worker, jobs))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    gbps = sum(p * b / t for (p, t), b in zip(res, kv)) / 1e9
    seqs = sum(p * len(ch) / t for (p, t), ch in zip(res, chunks))
    passes = sum(p for p, _ in res)
    return gbps, seqs, n, passes


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this library has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    sys.path.insert(0, ROOT)
    import paged_kv_cache_116_amd as pkv
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "prefill":
        return run_prefill(args, torch, pkv, workloads, dev)
    if args.workload == "swap":
        return run_swap(args, torch, pkv, workloads, dev)
    if args.workload == "cascade":
        return run_cascade(args, torch, pkv, workloads, dev)

    calib = None
    if args.calibrate:
        # Written now, read after the timed steps: by then gigabytes of KV
        # traffic have evicted it from L2 and the 256 MB MALL.
        calib = torch.ones(2**28, dtype=torch.float32, device=dev)
        calib_out = torch.empty_like(calib)
        torch.cuda.synchronize()

    kw = {}
    if args.block_size:
        kw["block_size"] = args.block_size
    t0 = time.time()
    fp8 = args.kv_dtype == "fp8"
    w = workloads.make_workload(args.config, device=dev, kv_fp8=fp8, **kw)
    torch.cuda.synchronize()
    print(f"# workload {w.name}: {w.num_seqs} seqs, tokens={int(w.lens.sum())}, "
          f"blocks={w.num_blocks}, drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # Host copies for the oracle, taken before any library call touches the pools.
    rng = np.random.default_rng(7)
    check_seqs = sorted(set([int(np.argmax(w.lens))] +
                            rng.choice(w.num_seqs, size=min(4, w.num_seqs), replace=False).tolist()))
    cpu_sample = sorted(rng.choice(w.num_seqs, size=min(64, w.num_seqs), replace=False).tolist())
    check_inputs = None if args.no_check else workloads.extract_sequences(w, check_seqs)

    esize = w.k_pool.element_size()     # 1 for FP8 pools
    qsize = w.q.element_size()
    S, Hq, Hkv, D, B = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    lens64 = w.lens.astype(np.int64)
    kv_bytes = int(lens64.sum()) * Hkv * D * 2 * esize
    table_bytes = int(sum(-(-int(L) // B) for L in lens64)) * 4
    alg_bytes = kv_bytes + 2 * S * Hq * D * qsize + table_bytes + S * 4

    tables = torch.as_tensor(w.tables, device=dev)
    lens = torch.as_tensor(w.lens, device=dev)
    lens_pre = torch.as_tensor(w.lens_pre, device=dev)
    out = torch.empty_like(w.q)
    P = args.partition_tokens
    ws = torch.empty(max(1, pkv.paged_decode_workspace_bytes(S, Hq, D, w.max_blocks * B, P)),
                     dtype=torch.uint8, device=dev)
    kernel = {"auto": pkv.PKV_ATTN_AUTO, "valu": pkv.PKV_ATTN_VALU, "mfma": pkv.PKV_ATTN_MFMA}[args.kernel]
    # A serving system's block manager knows whether any block is referenced by
    # more than one sequence; here the tables say it.
    used = np.concatenate([w.tables[s, : -(-int(w.lens[s]) // B)] for s in range(S)
                           if w.lens[s] > 0] or [np.zeros(0, np.int64)])
    shared = bool(used.size and np.bincount(used).max() > 1)
    cache_kv = shared if args.cache_kv == "auto" else args.cache_kv == "on"
    if cache_kv:
        kernel |= pkv.PKV_ATTN_CACHE_KV
    stream = torch.cuda.current_stream()

    def append():
        if fp8:
            pkv.paged_kv_append_fp8(w.k_pool, w.v_pool, w.k_new, w.v_new, tables, lens_pre,
                                    w.k_scale, w.v_scale, stream=stream)
        else:
            pkv.paged_kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, tables, lens_pre,
                                stream=stream)

    def attention_fp8():
        pkv.paged_decode_attention_fp8(out, w.q, w.k_pool, w.v_pool, tables, lens, w.k_scale,
                                       w.v_scale, kernel=kernel, scale=w.scale,
                                       partition_tokens=P, workspace=ws, stream=stream)

    def plan():
        pkv.paged_decode_attention_plan(kernel, out, w.q, w.k_pool, w.v_pool, tables, lens,
                                        scale=w.scale, partition_tokens=P, workspace=ws,
                                        stream=stream)

    def partitions():
        pkv.paged_decode_attention_partitions(kernel, out, w.q, w.k_pool, w.v_pool, tables, lens,
                                              scale=w.scale, partition_tokens=P, workspace=ws,
                                              stream=stream)

    def merge():
        pkv.paged_decode_attention_merge(kernel, out, w.q, w.k_pool, w.v_pool, tables, lens,
                                         scale=w.scale, partition_tokens=P, workspace=ws,
                                         stream=stream)

    def step():
        # Append + attention; the append rides in the plan launch.
        if fp8:
            pkv.paged_decode_step_fp8(out, w.q, w.k_pool, w.v_pool, w.k_new, w.v_new, tables,
                                      lens, w.k_scale, w.v_scale, kernel=kernel, scale=w.scale,
                                      partition_tokens=P, workspace=ws, stream=stream)
        else:
            pkv.paged_decode_step(out, w.q, w.k_pool, w.v_pool, w.k_new, w.v_new, tables, lens,
                                  kernel=kernel, scale=w.scale, partition_tokens=P,
                                  workspace=ws, stream=stream)

    # FP8 pools have no phase-by-phase entry points: their breakdown times the
    # whole attention call as one phase (so its roofline is conservative).
    phases = [append, attention_fp8] if fp8 else [append, plan, partitions, merge]

    for _ in range(args.warmup):
        for ph in phases:
            ph()
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # The timed region: K whole steps back to back, events only around them.
    start, end = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    # Step-time spread: a second pass with an event between consecutive steps
    # (each interval is one step, launch gap included).
    step_marks = [ev() for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    step_marks[0].record(stream)
    for i in range(args.steps):
        step()
        step_marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t_steps = [step_marks[i].elapsed_time(step_marks[i + 1]) for i in range(args.steps)]

    # Phase breakdown, a separate pass with an event between launches, the
    # append as its own launch (event records add a few microseconds of gap
    # each, so the phases sum to more than ms_step).  The partition kernel's
    # time here is the roofline's.
    marks = [[ev() for _ in range(len(phases) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for m in marks:
        m[0].record(stream)
        for i, ph in enumerate(phases):
            ph()
            m[i + 1].record(stream)
    torch.cuda.synchronize()
    t_app = [m[0].elapsed_time(m[1]) for m in marks]
    if fp8:
        t_part = [m[1].elapsed_time(m[2]) for m in marks]
        t_plan = t_merge = [0.0]
    else:
        t_plan = [m[1].elapsed_time(m[2]) for m in marks]
        t_part = [m[2].elapsed_time(m[3]) for m in marks]
        t_merge = [m[3].elapsed_time(m[4]) for m in marks]
    part_ms = statistics.mean(t_part)
    print(f"# timed {args.steps} steps: {ms_step * 1e3:.1f} us/step, partition {part_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    # Practical ceiling: a large device-to-device copy, outside the timed region.
    copy_gbps = None
    if args.copy_gib > 0:
        n = int(args.copy_gib * 2**30) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(5):
            b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 5 * 2 * n * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del a, b

    if calib is not None:
        # Plain kernels of known size for counter calibration: 1 GiB read
        # (sum), 1 GiB written (fill), 1 GiB read + 1 GiB written (x * 1).
        total = calib.sum()
        calib_out.fill_(2.0)
        torch.mul(calib, 1.0, out=calib_out)
        torch.cuda.synchronize()
        print(f"# calibration kernels ran on 1 GiB buffers (sum={float(total):.0f})",
              file=sys.stderr, flush=True)
        del calib, calib_out

    def oracle_append(c):
        """Oracle append on host copies; FP8 pools are appended as codes and
        decoded (value = code * scale)."""
        from oracle import cache_ops as o_cache
        from oracle import fp8 as o_fp8
        if not fp8:
            return o_cache.append_token(c["k_pool"], c["v_pool"], c["k_new"], c["v_new"],
                                        c["tables"], c["lens_pre"], B)
        kc, vc = o_fp8.append_token_fp8(c["k_pool"], c["v_pool"], c["k_new"], c["v_new"],
                                        c["tables"], c["lens_pre"], B, w.k_scale, w.v_scale)
        return o_fp8.dequantise(kc, w.k_scale), o_fp8.dequantise(vc, w.v_scale)

    parity = None
    if check_inputs is not None:
        from oracle import attention as o_attn
        c = check_inputs
        kp, vp = oracle_append(c)
        ref = o_attn.decode_attention(c["q"], kp, vp, c["tables"], c["lens"], B, w.scale)
        got = out[torch.as_tensor(check_seqs, device=dev)].double().cpu().numpy()
        err = np.abs(got - ref)
        if w.dtype == "f32":
            ok = bool(err.max() <= 1e-5)
        else:
            ok = bool((err <= 2e-2 + 1e-2 * np.abs(ref)).all())
        parity = {"sampled_seqs": check_seqs, "max_abs_err": float(err.max()), "ok": ok}
        print(f"# parity on {check_seqs}: max_abs_err={err.max():.3e} ok={ok}", file=sys.stderr,
              flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        t = time.perf_counter()
        gbps, seqs, n, passes = cpu_oracle_baseline(w, workloads, cpu_sample, args.cpu_seconds,
                                                    fp8)
        wall = time.perf_counter() - t
        cpu = {"value": gbps, "unit": "GB/s", "cores": n, "kind": "oracle",
               "seq_layer_steps_per_s": seqs,
               "sample": f"{len(cpu_sample)} of the {S} sequences (seeded), "
                         f"{int(w.lens[cpu_sample].sum())} tokens, split over {n} worker "
                         f"processes (one BLAS thread each), each repeating its slice for about "
                         f"{args.cpu_seconds:.0f}s ({passes} slice passes in all, {wall:.1f}s "
                         "wall), append + float64 gather attention"}
        print(f"# cpu oracle: {gbps:.4f} GB/s on {n} workers", file=sys.stderr, flush=True)

    kv_gbps_step = kv_bytes / (ms_step * 1e-3) / 1e9
    attn_ms = statistics.mean(t_plan) + statistics.mean(t_part) + statistics.mean(t_merge)
    achieved = alg_bytes / (part_ms * 1e-3) / 1e9
    kname = {"auto": "mfma" if w.dtype != "f32" and D >= 32 else "valu"}.get(args.kernel, args.kernel)
    traffic = (None if fp8 else
               measured_traffic(w.name + (f"_B{B}" if args.config == 5 else ""), kname))
    result = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + seq-layer steps/s",
        "value": round(kv_gbps_step, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[w.dtype],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.config] + (f" (B={B})" if args.config == 5 else ""),
                   "name": w.name, "batch": S, "block_size": B, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "tokens": int(lens64.sum()),
                   "partition_tokens": P, "kernel": kname, "shared_blocks": shared,
                   "cache_kv": cache_kv, "kv_dtype": "fp8_e4m3" if fp8 else w.dtype},
        "pct_of_hbm_peak": round(100 * kv_gbps_step / HBM_PEAK_GBPS, 2),
        "seq_layer_steps_per_s": round(S / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "kv_gbps_attention": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 2),
        "us": {"step": round(ms_step * 1e3, 2),
               "step_median": round(statistics.median(t_steps) * 1e3, 2),
               "step_p10": round(np.percentile(t_steps, 10) * 1e3, 2),
               "step_p90": round(np.percentile(t_steps, 90) * 1e3, 2),
               "append": round(statistics.mean(t_app) * 1e3, 2),
               "plan": round(statistics.mean(t_plan) * 1e3, 2),
               "partitions": round(part_ms * 1e3, 2),
               "partitions_p10": round(np.percentile(t_part, 10) * 1e3, 2),
               "partitions_p90": round(np.percentile(t_part, 90) * 1e3, 2),
               "merge": round(statistics.mean(t_merge) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": ("attention launches (plan + partitions + merge)" if fp8
                                else f"attn_partition_{kname}"),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "copy_gbps": round(copy_gbps, 1) if copy_gbps else None,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0 if (parity is None or parity["ok"]) else 1


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak


def run_prefill(args, torch, pkv, workloads, dev) -> int:
    """A step: paged_kv_append_tokens of every prompt's keys and values, then
    paged_prefill_attention over them (whole prompts, causal).  `value` is
    prompt tokens per second over the step; the roofline prices the
    attention kernel's algorithmic matrix flops, 4 * D per (query head,
    visible key) pair, against the dense bf16 MFMA peak."""
    t0 = time.time()
    w = workloads.make_prefill_workload(device=dev)
    torch.cuda.synchronize()
    S, T = len(w.lens), int(w.cu[-1])
    Hq, Hkv, D, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    print(f"# workload {w.name}: {S} prompts, {T} tokens, blocks={w.num_blocks}, "
          f"drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # FP8 pools: E4M3FN codes drawn field by field (exponents 3..10) for the
    # history, the NaN code in every slot that holds no token yet.
    fp8 = args.kv_dtype == "fp8"
    ks, vs = 0.0625, 0.125
    if fp8:
        g = torch.Generator(device=dev)
        g.manual_seed(2001)
        empty = torch.isnan(w.k_pool.float()).any(dim=-1).any(dim=-1)

        def codes():
            shp = tuple(w.k_pool.shape)
            c = ((torch.randint(0, 2, shp, generator=g, device=dev) << 7) |
                 (torch.randint(3, 11, shp, generator=g, device=dev) << 3) |
                 torch.randint(0, 8, shp, generator=g, device=dev)).to(torch.uint8)
            c[empty] = 0x7F
            return c.view(torch.float8_e4m3fn)
        k_pool, v_pool = codes(), codes()
    else:
        k_pool, v_pool = w.k_pool, w.v_pool

    # Host copies for the oracle, before any library call writes the pools.
    rng = np.random.default_rng(7)
    check = sorted(rng.choice(S, size=2, replace=False).tolist())
    host = {k: getattr(w, k).detach().to("cpu").to(torch.float64).numpy()
            for k in ("k_pool", "v_pool", "k_new", "v_new", "q")} if not args.no_check else None
    if host is not None and fp8:
        host["k_pool"] = k_pool.view(torch.uint8).cpu().numpy()
        host["v_pool"] = v_pool.view(torch.uint8).cpu().numpy()

    pre_len = (w.lens - w.chunks).astype(np.int64)
    visible = sum(int(((pre_len[s] + np.arange(w.chunks[s]) + 1)).sum()) for s in range(S))
    flops = 4.0 * D * Hq * visible
    tables = torch.as_tensor(w.tables, device=dev)
    lens = torch.as_tensor(w.lens, device=dev)
    lens_pre = torch.as_tensor(w.lens_pre, device=dev)
    cu = torch.as_tensor(w.cu, device=dev)
    out = torch.empty_like(w.q)
    max_chunk = int(w.chunks.max())
    stream = torch.cuda.current_stream()

    def append():
        if fp8:
            pkv.paged_kv_append_tokens_fp8(k_pool, v_pool, w.k_new, w.v_new, cu, tables,
                                           lens_pre, ks, vs, stream=stream)
        else:
            pkv.paged_kv_append_tokens(k_pool, v_pool, w.k_new, w.v_new, cu, tables, lens_pre,
                                       stream=stream)

    def attention():
        if fp8:
            pkv.paged_prefill_attention_fp8(out, w.q, k_pool, v_pool, cu, tables, lens, ks, vs,
                                            max_chunk_tokens=max_chunk, scale=w.scale,
                                            stream=stream)
        else:
            pkv.paged_prefill_attention(out, w.q, k_pool, v_pool, cu, tables, lens,
                                        max_chunk_tokens=max_chunk, scale=w.scale, stream=stream)

    def step():
        append()
        attention()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    start, end = ev(), ev()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    marks = [[ev() for _ in range(3)] for _ in range(args.steps)]
    for m in marks:
        m[0].record(stream)
        append()
        m[1].record(stream)
        attention()
        m[2].record(stream)
    torch.cuda.synchronize()
    t_app = statistics.mean(m[0].elapsed_time(m[1]) for m in marks)
    t_attn = [m[1].elapsed_time(m[2]) for m in marks]
    attn_ms = statistics.mean(t_attn)
    print(f"# timed {args.steps} steps: {ms_step * 1e3:.1f} us/step, attention {attn_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    parity = None
    cpu = None
    if host is not None or args.cpu_seconds > 0:
        from oracle import attention as o_attn
        from oracle import cache_ops as o_cache
        from oracle import fp8 as o_fp8

        def oracle_pools(s, sl):
            """Prompt s's tokens appended to host copies of the pools (FP8
            pools: quantised codes, returned decoded)."""
            if not fp8:
                return o_cache.append_tokens(host["k_pool"], host["v_pool"], host["k_new"][sl],
                                             host["v_new"][sl], w.tables[s:s + 1],
                                             w.lens_pre[s:s + 1], [0, int(w.chunks[s])], B)
            kc, vc = o_fp8.append_tokens_fp8(host["k_pool"], host["v_pool"], host["k_new"][sl],
                                             host["v_new"][sl], w.tables[s:s + 1],
                                             w.lens_pre[s:s + 1], [0, int(w.chunks[s])], B, ks,
                                             vs)
            return o_fp8.dequantise(kc, ks), o_fp8.dequantise(vc, vs)

        def oracle_token(s, j):
            """Output of chunk token j of prompt s, as a one-token chunk over
            its p + 1 visible positions."""
            sl = slice(int(w.cu[s]), int(w.cu[s + 1]))
            kp, vp = oracle_pools(s, sl)
            p = int(pre_len[s] + j)
            q1 = host["q"][int(w.cu[s]) + j: int(w.cu[s]) + j + 1]
            return o_attn.prefill_attention(q1, kp, vp, w.tables[s:s + 1], [p + 1], [0, 1], B,
                                            w.scale)

        if host is not None:
            errs, ok = [], True
            for s in check:
                for j in sorted(set([0, int(w.chunks[s]) - 1] +
                                    rng.integers(0, int(w.chunks[s]), 3).tolist())):
                    ref = oracle_token(s, j)
                    got = out[int(w.cu[s]) + j: int(w.cu[s]) + j + 1].double().cpu().numpy()
                    err = np.abs(got - ref)
                    errs.append(float(err.max()))
                    ok &= bool(np.isfinite(got).all() and (err <= 2e-2 + 1e-2 * np.abs(ref)).all())
            parity = {"sampled_prompts": check, "max_abs_err": max(errs), "ok": ok}
        if args.cpu_seconds > 0 and host is not None:
            # The oracle on the shortest prompt, whole (append + attention),
            # repeated for the time budget; single threaded.
            os.environ.setdefault("OMP_NUM_THREADS", "1")
            s = int(np.argmin(w.chunks))
            sl = slice(int(w.cu[s]), int(w.cu[s + 1]))
            spent, passes = 0.0, 0
            while spent < args.cpu_seconds:
                t = time.perf_counter()
                kp, vp = oracle_pools(s, sl)
                o_attn.prefill_attention(host["q"][sl], kp, vp, w.tables[s:s + 1],
                                         w.lens[s:s + 1], [0, int(w.chunks[s])], B, w.scale)
                spent += time.perf_counter() - t
                passes += 1
            cpu = {"value": round(passes * int(w.chunks[s]) / spent, 2), "unit": "tokens/s",
                   "cores": 1, "kind": "oracle",
                   "sample": f"prompt {s} ({int(w.chunks[s])} tokens) of the batch, whole, "
                             f"{passes} pass(es) in {spent:.1f}s, append + float64 causal "
                             "attention"}
            print(f"# cpu oracle: {cpu['value']} tokens/s over {spent:.1f}s", file=sys.stderr,
                  flush=True)

    achieved = flops / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": "paged prefill tokens/s (attention TFLOP/s vs MFMA peak)",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "prefill: 16 whole prompts, log-normal lengths (median 584, p95 "
                               "2155, at most 4096), 32 q / 8 kv heads, D 128, B 16, bf16" +
                               (", FP8 (E4M3FN) pools" if fp8 else ""),
                   "name": w.name, "prompts": S, "tokens": T, "block_size": B,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "kv_dtype": "fp8_e4m3" if fp8 else w.dtype},
        "us": {"step": round(ms_step * 1e3, 2), "append": round(t_app * 1e3, 2),
               "attention": round(attn_ms * 1e3, 2),
               "attention_p10": round(float(np.percentile(t_attn, 10)) * 1e3, 2),
               "attention_p90": round(float(np.percentile(t_attn, 90)) * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_prefill_mfma", "algorithmic_flops_per_launch": flops},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0 if (parity is None or parity["ok"]) else 1


HOST_LINK_PEAK_GBPS = 64.0   # PCIe Gen5 x16, one direction


def run_swap(args, torch, pkv, workloads, dev) -> int:
    """A step: swap every fourth sequence of the decode batch out to pinned
    host memory (paged_kv_swap_out of their blocks, K and V) and back in at
    the same ids (paged_kv_swap_in).  `value` is bytes moved per second over
    the step, both directions; each direction is priced against the host
    link's one-way peak.  The copies are checked bit for bit."""
    w = workloads.make_workload(args.config, device=dev)
    B = w.block_size
    seqs = list(range(0, w.num_seqs, 4))
    ids = np.concatenate([w.tables[s, : -(-int(w.lens[s]) // B)] for s in seqs]).astype(np.int32)
    n = len(ids)
    shape = (n,) + tuple(w.k_pool.shape[1:])
    hk = torch.empty(shape, dtype=w.k_pool.dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=w.k_pool.dtype, pin_memory=True)
    t_ids = torch.as_tensor(ids, device=dev)
    moved = 2 * hk.numel() * hk.element_size()          # K and V, one direction
    print(f"# swap: {len(seqs)} of {w.num_seqs} sequences, {n} blocks, "
          f"{moved / 1e9:.3f} GB per direction", file=sys.stderr, flush=True)
    ref_k = w.k_pool[t_ids.long()].clone()
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for _ in range(min(args.warmup, 3)):
        pkv.paged_kv_swap_out(w.k_pool, w.v_pool, t_ids, hk, hv, stream=stream)
        pkv.paged_kv_swap_in(w.k_pool, w.v_pool, t_ids, hk, hv, stream=stream)
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 10))
    t_out, t_in = [], []
    start, end = ev(), ev()
    start.record(stream)
    for _ in range(steps):
        a, b, c = ev(), ev(), ev()
        a.record(stream)
        pkv.paged_kv_swap_out(w.k_pool, w.v_pool, t_ids, hk, hv, stream=stream)
        b.record(stream)
        pkv.paged_kv_swap_in(w.k_pool, w.v_pool, t_ids, hk, hv, stream=stream)
        c.record(stream)
        t_out.append((a, b))
        t_in.append((b, c))
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    ms_out = statistics.mean(x.elapsed_time(y) for x, y in t_out)
    ms_in = statistics.mean(x.elapsed_time(y) for x, y in t_in)
    ok = bool(torch.equal(hk.view(torch.int16), ref_k.cpu().view(torch.int16)) and
              torch.equal(w.k_pool[t_ids.long()].view(torch.int16), ref_k.view(torch.int16)))
    gbps_out = moved / (ms_out * 1e-3) / 1e9
    gbps_in = moved / (ms_in * 1e-3) / 1e9
    print(f"# out {ms_out * 1e3:.0f} us ({gbps_out:.1f} GB/s), in {ms_in * 1e3:.0f} us "
          f"({gbps_in:.1f} GB/s)", file=sys.stderr, flush=True)
    result = {
        "metric": "paged KV swap GB/s (out + in, pinned host memory)",
        "value": round(2 * moved / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": min(args.warmup, 3),
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"swap every fourth sequence of: {WORKLOAD_DESC[args.config]}",
                   "name": w.name, "sequences": len(seqs), "blocks": n,
                   "bytes_per_direction": moved},
        "us": {"step": round(ms_step * 1e3, 1), "swap_out": round(ms_out * 1e3, 1),
               "swap_in": round(ms_in * 1e3, 1)},
        "roofline": {"bound": "host-link", "achieved": round(min(gbps_out, gbps_in), 2),
                     "achieved_out": round(gbps_out, 2), "achieved_in": round(gbps_in, 2),
                     "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(min(gbps_out, gbps_in) / HOST_LINK_PEAK_GBPS, 4),
                     "traffic": None, "kernel": "swap_kernel"},
        "parity": {"bit_exact": ok, "ok": ok},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0 if ok else 1


def run_cascade(args, torch, pkv, workloads, dev) -> int:
    """The shared-prefix config (config 4: 128 sequences over one 64-block,
    1024-token prefix): a step is the append plus paged_decode_attention_cascade
    with the whole batch as one group, next to the same step through plain
    decode attention (cache-retaining loads).  `value` is logical KV bytes per
    second (every sequence's whole history, as for decode); the roofline
    prices the distinct bytes the cascade has to read (the prefix once, every
    private suffix once, q, out) over the cascade call.  --batch and
    --prefix-tokens draw the same structure at other sizes (suffixes U[1,512])."""
    if args.config != 4:
        print("--workload cascade runs on the shared-prefix config (--config 4)", file=sys.stderr)
        return 2
    t0 = time.time()
    literal = args.batch is None and args.prefix_tokens == 1024
    kw = {} if literal else dict(batch=args.batch or 128, len_range=(1, 512),
                                 prefix_tokens=args.prefix_tokens)
    w = workloads.make_workload(4, device=dev, **kw)
    torch.cuda.synchronize()
    S, Hq, Hkv, D, B = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    npre = len(w.shared_blocks)
    print(f"# workload {w.name}: {S} seqs, prefix {npre} blocks, tokens={int(w.lens.sum())}, "
          f"drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    rng = np.random.default_rng(7)
    check_seqs = sorted(rng.choice(S, size=4, replace=False).tolist())
    check_inputs = None if args.no_check else workloads.extract_sequences(w, check_seqs)

    esize, qsize = w.k_pool.element_size(), w.q.element_size()
    lens64 = w.lens.astype(np.int64)
    row = Hkv * D * 2 * esize                       # K and V bytes of one token
    kv_logical = int(lens64.sum()) * row
    kv_distinct = (npre * B + int((lens64 - npre * B).sum())) * row
    alg_distinct = kv_distinct + 2 * S * Hq * D * qsize

    tables = torch.as_tensor(w.tables, device=dev)
    lens = torch.as_tensor(w.lens, device=dev)
    lens_pre = torch.as_tensor(w.lens_pre, device=dev)
    offsets = torch.as_tensor(np.array([0, S], np.int32), device=dev)
    members = torch.arange(S, dtype=torch.int32, device=dev)
    prefix = torch.as_tensor(np.array([npre], np.int32), device=dev)
    out_c = torch.empty_like(w.q)
    out_d = torch.empty_like(w.q)
    ws_c = torch.empty(max(1, pkv.paged_decode_cascade_workspace_bytes(
        S, Hq, D, w.max_blocks, B)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, pkv.paged_decode_workspace_bytes(S, Hq, D, w.max_blocks * B, 0)),
                       dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def append():
        pkv.paged_kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, tables, lens_pre,
                            stream=stream)

    def cascade():
        pkv.paged_decode_attention_cascade(out_c, w.q, w.k_pool, w.v_pool, tables, lens,
                                           offsets, members, prefix, max_group_size=S,
                                           scale=w.scale, workspace=ws_c, stream=stream)

    def decode():
        pkv.paged_decode_attention_with(pkv.PKV_ATTN_AUTO | pkv.PKV_ATTN_CACHE_KV, out_d, w.q,
                                        w.k_pool, w.v_pool, tables, lens, scale=w.scale,
                                        workspace=ws_d, stream=stream)

    # The append writes the same bytes every time, so repeated steps are
    # idempotent.
    for _ in range(args.warmup):
        append()
        cascade()
        decode()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fns):
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            for f in fns:
                f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_step = timed([append, cascade])
    ms_casc = timed([cascade])
    ms_dec_step = timed([append, decode])
    ms_dec = timed([decode])
    print(f"# cascade step {ms_step * 1e3:.1f} us (attention {ms_casc * 1e3:.1f}); plain decode "
          f"step {ms_dec_step * 1e3:.1f} us (attention {ms_dec * 1e3:.1f})", file=sys.stderr,
          flush=True)

    parity = None
    if check_inputs is not None:
        from oracle import attention as o_attn
        from oracle import cache_ops as o_cache
        c = check_inputs
        kp, vp = o_cache.append_token(c["k_pool"], c["v_pool"], c["k_new"], c["v_new"],
                                      c["tables"], c["lens_pre"], B)
        ref = o_attn.decode_attention(c["q"], kp, vp, c["tables"], c["lens"], B, w.scale)
        idx = torch.as_tensor(check_seqs, device=dev)
        err_c = np.abs(out_c[idx].double().cpu().numpy() - ref)
        err_d = np.abs(out_d[idx].double().cpu().numpy() - ref)
        ok = bool((err_c <= 2e-2 + 1e-2 * np.abs(ref)).all() and
                  (err_d <= 2e-2 + 1e-2 * np.abs(ref)).all())
        parity = {"sampled_seqs": check_seqs, "max_abs_err": float(err_c.max()),
                  "max_abs_err_plain": float(err_d.max()), "ok": ok}
        print(f"# parity on {check_seqs}: cascade {err_c.max():.3e}, plain {err_d.max():.3e}, "
              f"ok={ok}", file=sys.stderr, flush=True)

    achieved = alg_distinct / (ms_casc * 1e-3) / 1e9
    # The library's export policy: a group pays when its prefix holds at least
    # PKV_CASCADE_MIN_PREFIX_TOKENS and members x prefix tokens reach the
    # measured crossover for this head shape; otherwise plain decode.
    min_shared = pkv.pkv_cascade_min_shared_tokens(Hkv, D, esize)
    picks = ("cascade" if npre * B >= pkv.PKV_CASCADE_MIN_PREFIX_TOKENS and
             S * npre * B >= min_shared else "plain")
    result = {
        "metric": "shared-prefix decode attention, logical KV GB/s + seq-layer steps/s",
        "value": round(kv_logical / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "cascade decode over " + (
                       WORKLOAD_DESC[4] if literal else
                       f"shared-prefix GQA fp16: 32 q / 8 kv heads, D 128, B 16, batch {S}, "
                       f"{args.prefix_tokens}-token shared prefix + U[1,512] private"),
                   "name": w.name,
                   "batch": S, "prefix_blocks": npre, "block_size": B, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "tokens": int(lens64.sum())},
        "seq_layer_steps_per_s": round(S / (ms_step * 1e-3), 1),
        "kv_bytes_logical": kv_logical,
        "kv_bytes_distinct": kv_distinct,
        "us": {"step": round(ms_step * 1e3, 2), "cascade": round(ms_casc * 1e3, 2),
               "plain_decode_step": round(ms_dec_step * 1e3, 2),
               "plain_decode_attention": round(ms_dec * 1e3, 2)},
        "speedup_over_plain_decode": round(ms_dec_step / ms_step, 3),
        "policy": {"picks": picks, "min_shared_tokens": min_shared,
                   "step_us": round((ms_step if picks == "cascade" else ms_dec_step) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None,
                     "kernel": "cascade call (prefix + suffix decode + combine launches)",
                     "algorithmic_bytes_per_launch": alg_distinct},
        "parity": parity,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0 if (parity is None or parity["ok"]) else 1


if __name__ == "__main__":
    sys.exit(main())
