"""The benchmark's JSON line on the GPU, in a short form (three timed steps, a row subset of
the CPU oracle, no 16K-token or fp8 blocks): the keys the line carries, their values for
this run, and the arithmetic behind them. `value` is the step's attention flops over the
step time, `roofline.achieved` the same flops over the fused kernel's average launch time,
and `frac` that over the bf16 MFMA peak. Also checked: the kernel time fits in the step,
and the CPU oracle baseline states what it ran on."""
import json
import os
import subprocess
import sys

import pytest

from bidirectional_transformer_attention_amd import synth

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args):
    print(f"[gpu-test] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_bench_line():
    out = run_bench(["--steps", "3", "--warmup", "1", "--gate-steps", "0", "--fp8-steps", "0",
                     "--cpu-rows", "32", "--cpu-1thread-rows", "0"])
    print(f"[gpu-test] value {out['value']} TFLOP/s, kernel frac {out['roofline']['frac']}", flush=True)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["unit"] == "TFLOP/s" and out["higher_is_better"] is True and out["scaling"] == "weak"
    assert out["dtype"] == "bf16" and out["vs_baseline"] is None
    assert out["config"]["workload"] == "dit1k_bf16+replay"
    assert out["gate_16k_tokens"] is None and out["fp8_step"] is None

    flops = synth.bench_workload("dit1k_bf16").flops()
    # both times are printed to 4 decimals of a millisecond: a relative rounding below 1e-3
    assert out["value"] > 0
    assert abs(out["value"] - flops / (out["ms_per_step"] * 1e-3) / 1e12) <= 1e-3 * out["value"]
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2516.6
    assert 0 < roof["kernel_ms_min"] <= roof["kernel_ms_avg"] <= out["ms_per_step"]
    assert abs(roof["achieved"] - flops / (roof["kernel_ms_avg"] * 1e-3) / 1e12) <= 1e-3 * roof["achieved"]
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) <= 1e-4
    assert 0 < roof["frac"] < 1
    assert roof["traffic"] is None or roof["traffic"] > 0

    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOP/s" and cpu["value"] > 0
    assert cpu["cores"] >= 1 and cpu["blas_threads"] >= 1 and "32 query rows" in cpu["sample"]
