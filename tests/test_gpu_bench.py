"""bench.py's output line: one JSON object with the fields its consumers read.

Each case runs bench.py in a child process (few steps) and checks the keys,
their types and the relations between them (frac = achieved / peak, value =
FLOPs / time, the flushed pass no faster than the steady state by more than
noise).
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def run_bench(*args):
    print(f"[bench] {' '.join(args)}", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout
    return json.loads(lines[0])


def check_common(d, steps, warmup):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["warmup_run"]["steps"] >= warmup and d["warmup_run"]["seconds"] >= 0.5
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    assert "workload" in d["config"]
    rl = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rl, k
    assert rl["achieved"] > 0 and rl["peak"] > 0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["traffic"] is None or rl["traffic"] > 0


def test_bench_headline_line():
    d = run_bench("--steps", "5", "--warmup", "2", "--no-cpu-baseline")
    check_common(d, 5, 2)
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16"
    assert d["roofline"]["bound"] == "mfma" and d["roofline"]["unit"] == "TFLOP/s"
    assert d["cpu_baseline"] is None
    gflop = d["config"]["gflop_per_step"]
    assert abs(d["value"] - gflop / d["ms_per_step"]) / d["value"] < 1e-2
    sm, fl = d["step_ms"], d["flushed"]
    assert 0 < sm["min"] <= sm["median"] and 0 < fl["min_ms"] <= fl["median_ms"]
    assert fl["flush_bytes"] == 512 << 20
    assert abs(fl["value_median"] - gflop / fl["median_ms"]) / fl["value_median"] < 1e-2
    # evicting the caches cannot make a step faster (beyond timer noise)
    assert fl["median_ms"] > 0.9 * sm["median"]
    pk = d["peak_device"]
    assert pk is not None and pk["cus"] > 0 and pk["clock_mhz"] > 0
    assert abs(pk["tflops"] - pk["cus"] * pk["clock_mhz"] * 4096 / 1e6) < 0.5
    assert set(d["stages_ms"]) == {"prep", "qkv_proj", "attention", "out_proj", "early_rows"}


def test_bench_cpu_baseline_small_workload():
    d = run_bench("--steps", "3", "--warmup", "1", "--workload", "self_fp32_d512_h8_b2_t128")
    check_common(d, 3, 1)
    assert d["dtype"] == "fp32"
    # the fp32 path is measured against the fp32 matrix peak
    assert d["roofline"]["peak"] == 157.3
    assert abs(d["pct_fp32_peak"] - 100.0 * d["value"] / 157.3) < 0.01
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    small = cb["full_forward_small"]
    assert [r["cores"] for r in small][1] == 1 and all(r["seconds"] > 0 for r in small)


def test_bench_decode_line():
    d = run_bench("--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--workload",
                  "decode_bf16_d1024_h16_b32_t4096")
    check_common(d, 3, 1)
    assert d["unit"] == "GB/s" and d["roofline"]["bound"] == "hbm"
    assert d["roofline"]["unit"] == "GB/s"
    mb = d["config"]["cache_mb_read_per_step"]
    assert abs(d["value"] - mb / d["ms_per_step"]) / d["value"] < 1e-2
