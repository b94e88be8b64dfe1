"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dit1k_bf16]

One step = one pass of the whole path over one synthetic batch, inputs resident in HBM:
prefix relayout (replay -> online layout), RoPE on own k (and q) of both CFG branches,
the fused attention launch over [prefix ++ own] for both branches (on the bf16 path it
rotates q as it loads it), CFG combine.
Prints one JSON line. ``value`` is attention TFLOP/s (4*Sq*Skv*Hq*D summed over the
branches, divided by the step time). ``roofline`` is measured on the fused attention
kernel with HIP events recorded on the stream it runs on; ``cpu_baseline`` times the
CPU fp64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and % of MI355X MFMA peak, 4096x(4096+512) GQA bf16"
PEAK = {"bf16": 2516.6, "f32": 157.3, "fp8": 5033.2}   # TFLOP/s, dense MFMA, MI355X published
# the fp8 score GEMM does half the flops on the fp8 unit and half (P.V) on the bf16 unit:
# at both peaks a step would take F/2/fp8 + F/2/bf16, i.e. an effective peak of
PEAK_FP8QK = 2.0 / (1.0 / PEAK["fp8"] + 1.0 / PEAK["bf16"])
HBM_PEAK = 8000.0                               # GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_dit1k_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "bidirectional_transformer_attention_amd", "csrc", "fwd_bf16.hip")


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_record():
    """Per-launch HBM bytes of the fused kernel from the committed rocprofv3 counter runs,
    or None when absent or taken on a different revision of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    return rec


def time_call(fn, stream, reps: int = 20) -> float:
    """Average GPU milliseconds of fn() (which enqueues work on `stream`): HIP events around
    reps calls that were all enqueued behind a spin kernel, so the GPU runs them back to back
    and the host's per-call submission time is not counted."""
    import torch
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(4_000_000)      # about 2 ms of spinning while the calls are enqueued
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def cpu_baseline(wl, rows_per_branch: int, threads: int = 0):
    """Time the CPU fp64 oracle on the first rows of every branch (full keys); threads > 0
    limits the BLAS thread pool to that many threads."""
    import contextlib

    import numpy as np
    import torch

    import oracle
    from bidirectional_transformer_attention_amd import synth

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limit = threadpool_limits(limits=threads) if threads > 0 else contextlib.nullcontext()
        with limit:
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        limit, cores = contextlib.nullcontext(), 1
    with limit:
        return _cpu_baseline(wl, rows_per_branch, cores, np, torch, oracle, synth)


def _cpu_baseline(wl, rows_per_branch, cores, np, torch, oracle, synth):
    inp = synth.make_inputs(wl)
    f64 = lambda t: t.to(torch.float32).numpy().astype(np.float64)  # noqa: E731
    rows = np.arange(wl.seq if rows_per_branch <= 0 else min(rows_per_branch, wl.seq))
    t0 = time.perf_counter()
    flops = 0.0
    for b in range(wl.branches):
        q = oracle.rope(f64(inp.q[b][: len(rows)]), wl.grid, wl.pairs, wl.offsets[b], wl.theta, rows=rows)
        k = oracle.rope(f64(inp.k[b]), wl.grid, wl.pairs, wl.offsets[b], wl.theta)
        p = inp.prefix[b]
        pre = None if p is None else f64(p)
        if pre is not None and wl.prefix_layout == "replay":
            pre = oracle.relayout(pre[None], 0)[0]
        pk = None if pre is None else pre[0]
        if wl.qk_fp8:
            # the fp8 score GEMM's inputs: q (carrying softmax_scale*log2(e)), k and the
            # prefix K through E4M3 and back
            from oracle import fp8 as ofp8
            from bidirectional_transformer_attention_amd.binding import fold_factor
            cf = fold_factor(wl.head_dim)
            q = ofp8.dequantize_fp8(*ofp8.quantize_fp8(q[None] * cf))[0] / cf
            k = ofp8.dequantize_fp8(*ofp8.quantize_fp8(k[None]))[0]
            pk = None if pk is None else ofp8.dequantize_fp8(*ofp8.quantize_fp8(pk[None]))[0]
        oracle.attention(q, k, f64(inp.v[b]), pk, None if pre is None else pre[1])
        flops += 4.0 * len(rows) * (wl.prefix_len[b] + wl.seq) * wl.heads_q * wl.head_dim
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{wl.name}: first {len(rows)} query rows of each of {wl.branches} branches against all "
                      f"keys (RoPE, relayout, fp64 attention), {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit1k_bf16")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="query rows per branch for the CPU oracle timing (0: all, i.e. one whole step)")
    ap.add_argument("--splits", type=int, default=None,
                    help="key ranges per branch in the attention call (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-1thread-rows", type=int, default=-1,
                    help="query rows per branch for the 1-thread CPU oracle timing (-1: seq/16, 0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="after timing, relayout one buffer of this many MB (a plain copy of known size "
                         "used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "nxattn runs on exactly one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is not implemented)"}))
        return 2

    import torch

    import bidirectional_transformer_attention_amd as nx
    from bidirectional_transformer_attention_amd import synth
    from bidirectional_transformer_attention_amd.pipeline import AttentionStep

    nx.load()
    wl = synth.bench_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    step = AttentionStep(wl, synth.make_inputs(wl), "cuda:0", splits=args.splits)
    flops_step = wl.flops()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step.relayout()
        step.rope()
        step.quantize()
        ev[i][0].record(stream)
        step.attention()
        ev[i][1].record(stream)
        step.cfg()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    fwd_ms = sorted(a.elapsed_time(b) for a, b in ev)
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    value = flops_step / (ms_step * 1e-3) / 1e12

    # the headline shape alone: the cond branch, 4096 x (4096 + 512), as a batch-1 launch
    headline = None
    if wl.branches >= 1 and wl.dtype == "bf16" and not wl.qk_fp8:
        q0, k0, v0, o0 = step.q[:1], step.k[:1], step.v[:1], step.o[:1]
        pre0 = step.prefix_online[:1]
        split_kw = dict(num_splits=step.splits, workspace=step.workspace)
        for _ in range(3):
            nx.nxattn_fwd(q0, k0, v0, o0, pre0, **split_kw)
        h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        h0.record(stream)
        for _ in range(reps):
            nx.nxattn_fwd(q0, k0, v0, o0, pre0, **split_kw)
        h1.record(stream)
        torch.cuda.synchronize()
        hms = h0.elapsed_time(h1) / reps
        hfl = wl.flops([0])
        headline = {"shape": f"{wl.seq}x({wl.seq}+{wl.prefix_len[0]}) Hq {wl.heads_q} Hkv {wl.heads_kv} D {wl.head_dim}",
                    "ms": round(hms, 4), "tflops": round(hfl / hms / 1e9, 1),
                    "pct_peak": round(100 * hfl / hms / 1e9 / PEAK[wl.dtype], 2)}

    # with key splits the timed attention phase is the split kernel plus the merge kernel
    # (both on this stream); rocprofv3 separates the two
    achieved = flops_step / (fwd_avg * 1e-3) / 1e12
    peak = PEAK_FP8QK if wl.qk_fp8 else PEAK[wl.dtype]
    rec = traffic_record()

    # the side calls of the step, each timed alone, against the 8 TB/s HBM peak
    es = 2 if wl.dtype == "bf16" else 4
    side = {}
    nbytes = {
        "relayout": sum(2 * 2 * p * wl.heads_kv * wl.head_dim * es for p in wl.prefix_len)
        if wl.prefix_layout == "replay" else 0,
        "rope": 0 if wl.qk_fp8 else 2 * step.k.numel() * es + (0 if step.fuse_q_rope else 2 * step.q.numel() * es),
        "cfg": 3 * step.q[0].numel() * es if step.use_cfg else 0,
        # reads q, k (rotated inside both passes) and the prefix K twice (maximum, then
        # codes), writes one byte per element
        "quantize": (2 * es + 1) * (step.q.numel() + step.k.numel()
                                    + sum(p[0].numel() for p in step.prefix_online if p is not None))
        if wl.qk_fp8 else 0,
    }
    for name, fn in (("relayout", step.relayout), ("rope", step.rope), ("quantize", step.quantize),
                     ("cfg", step.cfg)):
        if nbytes[name] == 0:
            continue
        ms = time_call(fn, stream)
        gbs = nbytes[name] / (ms * 1e-3) / 1e9
        side[name] = {"us": round(1000 * ms, 2), "bytes": nbytes[name], "GB/s": round(gbs, 1),
                      "frac_of_hbm": round(gbs / HBM_PEAK, 4)}
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": (rec["bytes_per_launch"] if rec and rec.get("workload") == wl.name and step.splits <= 1
                        and not wl.qk_fp8 else None),
            "kernel": (f"nx::fp8k::fwd_fp8_kernel<{'true' if step.fold_q else 'false'}>" if wl.qk_fp8 else
                       (f"nx::bf16k::fwd_bf16_kernel<{'true' if step.fuse_q_rope else 'false'}>")
                       if wl.dtype == "bf16" else f"nx::f32k::fwd_f32_kernel<{wl.head_dim}>")
            + (" + nx::mergek::merge_kernel" if step.splits > 1 else ""),
            "kernel_ms_avg": round(fwd_avg, 4), "kernel_ms_min": round(fwd_ms[0], 4)}

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 2
        src = torch.empty((1, 2, 8, n // (2 * 8 * 128), 128), dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty((1, 2, src.shape[3], 8, 128), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        nx.nxattn_kv_relayout(src, dst, 0)
        torch.cuda.synchronize()
        del src, dst

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows)
        r1 = max(32, wl.seq // 16) if args.cpu_1thread_rows < 0 else args.cpu_1thread_rows
        if r1 > 0:
            cpu1 = cpu_baseline(wl, r1, threads=1)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3 QK / bf16 PV" if wl.qk_fp8 else wl.dtype, "data": "synthetic (seeded N(0,1), shapes of the workload)",
        "config": {"workload": wl.name, "branches": wl.branches, "seq_q": wl.seq, "grid": list(wl.grid),
                   "prefix_len": list(wl.prefix_len), "heads_q": wl.heads_q, "heads_kv": wl.heads_kv,
                   "head_dim": wl.head_dim, "rope_offsets": [list(o) for o in wl.offsets],
                   "guidance": wl.guidance, "prefix_layout_in": "replay [2,H,P,D] relaid each step"
                   if wl.prefix_layout == "replay" else "online [2,P,H,D]",
                   "splits": step.splits,
                   "step": ("relayout + rope(k) + fused attention (q rotated on load)" if step.fuse_q_rope
                            else "relayout + fp8 quantize(rope(q), rope(k), prefix k) + fused attention with fp8 QK"
                            if wl.qk_fp8 else "relayout + rope(q,k) + fused attention")
                   + (f" over {step.splits} key ranges + merge" if step.splits > 1 else "") + " + cfg",
                   "pct_of_bf16_peak_step": round(100 * value / PEAK[wl.dtype], 2)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "side_calls": side,
        "headline_cond_branch": headline,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
