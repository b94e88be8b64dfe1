"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dit1k_bf16]

One step = one pass of the whole path over one synthetic batch, inputs resident in HBM:
prefix relayout (replay -> online layout), RoPE on own k (and q) of both CFG branches,
the fused attention launch over [prefix ++ own] for both branches (on the bf16 path it
rotates q as it loads it), CFG combine.
A multi-layer workload (the 27-layer ViT encoder) runs every layer, each on its own seeded
inputs, in one step.
Prints one JSON line. ``value`` is attention TFLOP/s (4*Sq*Skv*Hq*D summed over the
branches, divided by the step time). ``roofline`` is measured on the fused attention
kernel with HIP events recorded on the stream it runs on; ``cpu_baseline`` times the
CPU fp64 oracle on a bounded sample of the same workload. ``gate_16k_tokens`` times the
16K-token 2K DiT step (both CFG branches) beside the headline workload, with its kernel's
fraction of the bf16 MFMA peak. ``fp8_step`` times the same step with the fp8 score GEMM
(q and k as E4M3 codes with one scale per 32-element run) beside it, with its speedup over
the bf16 step of the same run.
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
GATE_WORKLOAD = "dit2k_bf16"   # its prefix is given in the replay layout
FP8_WORKLOAD = "dit1k_fp8blk"  # the headline step with the block-scaled fp8 score GEMM
GATE_WARMUP = 5                # untimed 16K-token steps (about 35 ms) before its timed ones
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


def bf16_kernel_name(step) -> str:
    """The bf16 attention kernel a step launches: q rotated on load, and both CFG branches
    per workgroup (guidance combination in the epilogue)."""
    return (f"nx::bf16k::fwd_bf16_kernel<{'true' if step.fuse_q_rope else 'false'}, "
            f"{'true' if step.fuse_cfg else 'false'}>")


def fp8_kernel_name(step) -> str:
    """The fp8 attention kernel a step launches (softmax fold, block scales, q quantized on
    load, both CFG branches per workgroup)."""
    t = lambda x: "true" if x else "false"  # noqa: E731
    return (f"nx::fp8k::fwd_fp8_kernel<{t(step.fold_q or step.q_on_load)}, {t(step.blocks)}, {t(step.q_on_load)}, "
            f"{t(step.fuse_cfg)}>")


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


def host_cores() -> int:
    """CPU cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        return os.cpu_count() or 1


def fold_constant(head_dim: int) -> float:
    """The softmax fold factor the library documents for q's fp8 codes: fl32(s * fl32(log2 e)),
    s = fl32(1 / fl32(sqrt(head_dim))) (used to build the oracle's fp8 inputs)."""
    import numpy as np
    f32 = np.float32
    return float(f32(f32(1.0) / np.sqrt(f32(head_dim)) * f32(1.4426950408889634)))


def cpu_baseline(wl, rows_per_branch: int, threads: int = 0, layers: int = 1):
    """Time the CPU fp64 oracle on the first rows of every branch (full keys) of the first
    `layers` layers; threads > 0 limits the BLAS thread pool to that many threads."""
    import contextlib

    import numpy as np
    import torch

    import oracle
    from bidirectional_transformer_attention_amd import synth

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limit = threadpool_limits(limits=threads) if threads > 0 else contextlib.nullcontext()
        with limit:
            blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        limit, blas = contextlib.nullcontext(), 1
    with limit:
        return _cpu_baseline(wl, rows_per_branch, blas, layers, np, torch, oracle, synth)


def _cpu_baseline(wl, rows_per_branch, blas, layers, np, torch, oracle, synth):
    f64 = lambda t: t.to(torch.float32).numpy().astype(np.float64)  # noqa: E731
    rows = np.arange(wl.seq if rows_per_branch <= 0 else min(rows_per_branch, wl.seq))
    dt = 0.0
    flops = 0.0
    for layer in range(layers):
        inp = synth.make_inputs(wl, layer=layer)
        t0 = time.perf_counter()
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
                cf = fold_constant(wl.head_dim)
                if wl.fp8_blocks:
                    q = ofp8.dequantize_fp8_blocks(*ofp8.quantize_fp8_blocks(q * cf)) / cf
                    k = ofp8.dequantize_fp8_blocks(*ofp8.quantize_fp8_blocks(k))
                    pk = None if pk is None else ofp8.dequantize_fp8_blocks(*ofp8.quantize_fp8_blocks(pk))
                else:
                    q = ofp8.dequantize_fp8(*ofp8.quantize_fp8(q[None] * cf))[0] / cf
                    k = ofp8.dequantize_fp8(*ofp8.quantize_fp8(k[None]))[0]
                    pk = None if pk is None else ofp8.dequantize_fp8(*ofp8.quantize_fp8(pk[None]))[0]
            oracle.attention(q, k, f64(inp.v[b]), pk, None if pre is None else pre[1])
            flops += 4.0 * len(rows) * (wl.prefix_len[b] + wl.seq) * wl.heads_q * wl.head_dim
        dt += time.perf_counter() - t0
    full = wl.flops() * layers
    part = "all" if len(rows) == wl.seq else f"the first {len(rows)}"
    out = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": host_cores(), "blas_threads": int(blas),
           "kind": "oracle",
           "sample": f"{wl.name}: {part} query rows of each of {wl.branches} branches"
                     + (f" of {layers} layers" if layers > 1 else "")
                     + f" against all keys (RoPE, relayout, fp64 attention), {dt:.1f} s"}
    if len(rows) < wl.seq:
        out["extrapolated_full_step_s"] = round(dt * full / flops, 2)
    return out


def time_graph(graph, steps: int, warmup: int, torch):
    """Time (ms) per replay of a captured step graph, with HIP events on the current stream."""
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_step(step, steps: int, warmup: int, torch):
    """Whole-step and attention-launch times (ms) of an AttentionStep (or of a list of them,
    one per layer, run back to back as one step), with HIP events on the current stream."""
    layers = step if isinstance(step, list) else [step]
    for _ in range(warmup):
        for st in layers:
            st()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
          for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        for st, (e0, e1) in zip(layers, ev[i]):
            st.relayout()
            st.rope()
            st.quantize()
            e0.record(stream)
            st.attention()
            e1.record(stream)
            st.cfg()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    # attention launches of one step (summed over layers)
    fwd = sorted(sum(a.elapsed_time(b) for a, b in row) for row in ev)
    return ms_step, sum(fwd) / len(fwd), fwd[0]


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
    ap.add_argument("--gate-steps", type=int, default=10,
                    help="timed steps of the 16K-token gate workload (2K DiT, both branches); 0: skip")
    ap.add_argument("--order", choices=("gate-first", "headline-first"), default="gate-first",
                    help="whether the 16K-token block is timed before (default) or after the headline step")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as replays of its captured HIP graph instead of eager launches")
    ap.add_argument("--fp8-steps", type=int, default=50,
                    help="timed steps of the headline step with the fp8 score GEMM (dit1k workloads); 0: skip")
    ap.add_argument("--cpu-layers", type=int, default=1,
                    help="layers of a multi-layer workload that the CPU oracle timing covers")
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
    from bidirectional_transformer_attention_amd.pipeline import AttentionStep, capture_steps

    nx.load()
    wl = synth.bench_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    # a step of a multi-layer workload (the 27-layer ViT encoder) runs every layer, each
    # on its own seeded inputs
    layers = wl.layers
    # the production step: with CFG on the bf16 path the attention call writes the guided
    # output itself and the two branch outputs are not stored
    steps_all = [AttentionStep(wl, synth.make_inputs(wl, layer=l), "cuda:0", splits=args.splits,
                               keep_branches=False) for l in range(layers)]
    step = steps_all[0]
    flops_step = wl.flops() * layers
    def fp8_block():
        """The same step with the fp8 score GEMM (block scales), its speedup filled in once
        the bf16 step is timed."""
        if args.fp8_steps <= 0 or wl.name.split("+")[0] != "dit1k_bf16":
            return None
        fwl = synth.bench_workload(FP8_WORKLOAD)
        fstep = AttentionStep(fwl, synth.make_inputs(fwl), "cuda:0", keep_branches=False)
        # its own buffers are fresh: at least 30 untimed steps before timing
        fw = max(args.warmup, 30)
        f_ms, f_fwd, f_min = time_step(fstep, args.fp8_steps, fw, torch)
        if args.graph:
            f_ms = time_graph(capture_steps([fstep]), args.fp8_steps, fw, torch)
        ffl = fwl.flops()
        return {"workload": fwl.name, "steps": args.fp8_steps, "warmup": fw,
                "dtype": "fp8e4m3 QK (E8M0 scale per 32 elements) / bf16 PV",
                "ms_per_step": round(f_ms, 4), "step_tflops": round(ffl / f_ms / 1e9, 1),
                "speedup_vs_bf16_step": None,
                "kernel": fp8_kernel_name(fstep), "kernel_ms_avg": round(f_fwd, 4),
                "kernel_ms_min": round(f_min, 4), "kernel_tflops": round(ffl / f_fwd / 1e9, 1),
                "kernel_frac_of_fp8qk_peak": round(ffl / f_fwd / 1e9 / PEAK_FP8QK, 4)}

    def gate_block():
        """The >= 50 % gate is set on the 16K-token step (2K DiT, both CFG branches, prefix in
        the replay layout): timed beside the headline workload."""
        if args.gate_steps <= 0 or wl.name == GATE_WORKLOAD:
            return None
        gwl = synth.bench_workload(GATE_WORKLOAD)
        gstep = AttentionStep(gwl, synth.make_inputs(gwl), "cuda:0", keep_branches=False)
        g_ms, g_fwd, g_min = time_step(gstep, args.gate_steps, GATE_WARMUP, torch)
        if args.graph:
            g_ms = time_graph(capture_steps([gstep]), args.gate_steps, GATE_WARMUP, torch)
        gfl = gwl.flops()
        return {"workload": gwl.name, "steps": args.gate_steps, "warmup": GATE_WARMUP,
                "gflop_per_step": round(gfl / 1e9, 1),
                "ms_per_step": round(g_ms, 4), "step_tflops": round(gfl / g_ms / 1e9, 1),
                "step_frac": round(gfl / g_ms / 1e9 / PEAK["bf16"], 4),
                "kernel": bf16_kernel_name(gstep), "kernel_ms_avg": round(g_fwd, 4),
                "kernel_ms_min": round(g_min, 4), "kernel_tflops": round(gfl / g_fwd / 1e9, 1),
                "kernel_frac": round(gfl / g_fwd / 1e9 / PEAK["bf16"], 4), "gate_frac": 0.5,
                "gate_ms": round(gfl / (0.5 * PEAK["bf16"]) / 1e9, 4)}

    # On a fresh box the first ~100 ms of work run at a lower clock: with 5 warm-up steps
    # a headline timed first read 9 % lower than one timed after the 16K-token block (same
    # box). So by default that block (about 85 ms of GPU work, reported below) runs first,
    # then the headline, then the fp8 step, which is compared with it.
    fp8 = gate = None
    if args.order == "gate-first":
        gate = gate_block()
    # eager steps with HIP events around each attention launch (the roofline's kernel
    # time); with --graph the step time is taken again from replays of the step captured
    # as one HIP graph (warm, the two measure the same on one box)
    ms_eager, fwd_avg, fwd_min = time_step(steps_all if layers > 1 else step, args.steps, args.warmup, torch)
    ms_step = ms_eager
    if args.graph:
        ms_step = time_graph(capture_steps(steps_all), args.steps, args.warmup, torch)
    value = flops_step / (ms_step * 1e-3) / 1e12
    fp8 = fp8_block()
    if fp8 is not None:
        fp8["speedup_vs_bf16_step"] = round(ms_step / fp8["ms_per_step"], 4)

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
        "cfg": 3 * step.q[0].numel() * es if step.use_cfg and not step.fuse_cfg else 0,
        # per (branch, head): reads q and k twice (rotated inside both passes: maximum, then
        # codes), writes one byte per element; block scales: one read, the codes and one
        # scale byte per 32 elements (the prefix K is quantized once, outside the step)
        "quantize": (((es + 1) * (step.q.numel() + step.k.numel()) + (step.q.numel() + step.k.numel()) // 32)
                     if wl.fp8_blocks else (2 * es + 1) * (step.q.numel() + step.k.numel())) if wl.qk_fp8 else 0,
    }
    if step.fuse_prep:
        # one launch: the rotation of k and the relayouts of the prefixes
        nbytes["rope"] += nbytes["relayout"]
        nbytes["relayout"] = 0
    for name, fn in (("relayout", step.relayout), ("rope", step.rope), ("quantize", step.quantize),
                     ("cfg", step.cfg)):
        if nbytes[name] == 0:
            continue
        ms = time_call(fn, stream)
        gbs = nbytes[name] / (ms * 1e-3) / 1e9
        side[name] = {"us": round(1000 * ms, 2), "bytes": nbytes[name], "GB/s": round(gbs, 1),
                      "frac_of_hbm": round(gbs / HBM_PEAK, 4)}
    if step.fuse_cfg:
        side["cfg"] = "inside the attention call"
    if step.fuse_prep:
        side["relayout"] = "in the launch that rotates k (its bytes are in rope's)"
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": (rec["bytes_per_launch"] if rec and rec.get("workload") == wl.name and step.splits <= 1
                        and not wl.qk_fp8 else None),
            "kernel": (fp8_kernel_name(step) if wl.qk_fp8 else
                       bf16_kernel_name(step) if wl.dtype == "bf16" else f"nx::f32k::fwd_f32_kernel<{wl.head_dim}>")
            + (" + nx::mergek::merge_kernel" if step.splits > 1 else ""),
            "kernel_ms_avg": round(fwd_avg, 4), "kernel_ms_min": round(fwd_min, 4)}
    if layers > 1:
        roof["launches_per_step"] = layers

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 2
        src = torch.empty((1, 2, 8, n // (2 * 8 * 128), 128), dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty((1, 2, src.shape[3], 8, 128), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        nx.nxattn_kv_relayout(src, dst, 0)
        torch.cuda.synchronize()
        del src, dst

    if args.order == "headline-first":
        gate = gate_block()
    if gate is not None and not args.no_cpu_baseline:
        # a row subset of the 16K-token step, with the full-step time extrapolated from it
        gwl = synth.bench_workload(GATE_WORKLOAD)
        gate["cpu_baseline"] = cpu_baseline(gwl, max(32, gwl.seq // 128))

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows, layers=min(layers, args.cpu_layers))
        r1 = max(32, wl.seq // 16) if args.cpu_1thread_rows < 0 else args.cpu_1thread_rows
        if r1 > 0:
            cpu1 = cpu_baseline(wl, r1, threads=1)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "step_launch": "hip graph (one replay per step)" if args.graph else "eager",
        "order": ("16K-token block, then headline, then fp8 step" if args.order == "gate-first"
                  else "headline, then fp8 step, then 16K-token block"),
        "vs_baseline": None,
        "dtype": ("fp8e4m3 QK (E8M0 scale per 32 elements) / bf16 PV" if wl.fp8_blocks else "fp8e4m3 QK / bf16 PV")
        if wl.qk_fp8 else wl.dtype, "data": "synthetic (seeded N(0,1), shapes of the workload)",
        "config": {"workload": wl.name, "branches": wl.branches, "seq_q": wl.seq, "grid": list(wl.grid),
                   "prefix_len": list(wl.prefix_len), "heads_q": wl.heads_q, "heads_kv": wl.heads_kv,
                   "head_dim": wl.head_dim, "rope_offsets": [list(o) for o in wl.offsets],
                   "guidance": wl.guidance, "prefix_layout_in": "replay [2,H,P,D] relaid each step"
                   if wl.prefix_layout == "replay" else "online [2,P,H,D]",
                   "splits": step.splits, "layers_per_step": layers,
                   "step": (("relayout and rope(k) in one launch" if step.fuse_prep else "relayout + rope(k)")
                            + " + fused attention (q rotated on load)" if step.fuse_q_rope
                            else "relayout + fp8 quantize(rope(q), rope(k)) + fused attention with fp8 QK "
                                 "(prefix K codes made once per conditioning cache)"
                            if wl.qk_fp8 else "relayout + rope(q,k) + fused attention")
                   + (f" over {step.splits} key ranges + merge" if step.splits > 1 else "")
                   + ((" with the cfg combine in its epilogue (branch outputs not stored)" if step.fuse_cfg
                       else " + cfg") if step.use_cfg else "") + (f", x {layers} layers" if layers > 1 else ""),
                   "pct_of_bf16_peak_step": round(100 * value / PEAK[wl.dtype], 2)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "side_calls": side,
        "headline_cond_branch": headline,
        "gate_16k_tokens": gate,
        "fp8_step": fp8,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
