"""Throughput of the multi-head attention forward pass on one MI355X.

One step = one mha_forward call over one batch of seeded synthetic input
(weight preparation, QKV projection, fused attention, output projection and
the fp32 early-row pass), inputs resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--residual] [--y-dtype fp32|bf16]

Beside the headline rate the line carries:
  roofline      the dominant kernel's algorithmic FLOPs per launch divided by
                its average launch time (HIP events on the launch stream
                around that stage, over a second pass of K steps, so the
                event records do not perturb the timed steps), against the MI355X dense
                fp16/bf16 MFMA peak; `traffic` is the HBM bytes per launch from
                the committed rocprofv3 counter summary, or null when that
                summary was taken on a different kernel source.
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample of
                the same workload (whole batch elements, about 10 s of work),
                and one full forward of the smallest workload on all threads
                and on one (full_forward_small).

  python bench.py --oracle-timings [--workload NAME[,NAME...]]

times only the oracle: one full forward of each workload (default all) on
this host's threads, and the two smallest workloads also single-threaded.
  step_ms       median and minimum of single steps (a further pass, one
                event pair per step).
  flushed       the same per-step times with 512 MiB written between steps
                (inputs and weights evicted from L2 and the Infinity Cache).
  peak_device   the dense 16-bit MFMA peak recomputed from the device's CU
                count and peak clock (4096 flop per clock per CU).

Generation-step workloads (--workload decode_*): one step = one mha_decode
call (projection of the new tokens, attention over the KV cache, output
projection); the line reports the cache bytes read per second (value) and
the attention stage against the HBM bandwidth (roofline bound "hbm").
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MHA fwd TFLOP/s + % bf16 MFMA peak, D=1024 h=16 T=4096 causal, 1 GPU"
PEAK_MFMA_16BIT_TFLOPS = 2500.0    # MI355X dense bf16/fp16 MFMA, published
PEAK_MFMA_FP32_TFLOPS = 157.3      # MI355X fp32 matrix, published
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "attention": ["transformer_head_attention_amd/csrc/attn16.hip",
                  "transformer_head_attention_amd/csrc/device_common.h",
                  "transformer_head_attention_amd/csrc/transpose_tile.h"],
    "decode_attention": ["transformer_head_attention_amd/csrc/decode.hip",
                         "transformer_head_attention_amd/csrc/device_common.h"],
    # the QKV projection's GEMM launches (their bytes are summed per step)
    "qkv_proj": ["transformer_head_attention_amd/csrc/gemm16.hip",
                 "transformer_head_attention_amd/csrc/device_common.h"],
}


def source_digest(stage: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stage_flops(w, stage: str) -> float:
    """Algorithmic FLOPs of one launch of a stage (formula counts)."""
    D = w.D
    if stage == "attention":
        f = 4.0 * w.T_q * w.T_k * D * w.B
        return f * 0.5 if w.causal else f
    if stage == "qkv_proj":
        return 2.0 * w.B * (w.T_q * D * D + w.T_k * D * 2 * w.n_g * w.d_k)
    if stage == "out_proj":
        return 2.0 * w.B * w.T_q * D * D
    return 0.0


def read_traffic(stage: str, workload: str):
    """HBM bytes per launch from the committed counter summary of this stage's
    kernel on this workload, if it was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{stage}_hbm_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest(stage):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def step_times(torch, stream, step, n: int, flush_bytes: int = 0):
    """Sorted single-step times (ms): one event pair per step on the launch
    stream. With flush_bytes, a buffer of that size is overwritten before each
    step, outside its events."""
    buf = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0") if flush_bytes else None
    evs = []
    for i in range(n):
        if buf is not None:
            buf.fill_(i & 0xff)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)


def warm_up(torch, step, n: int, min_seconds: float):
    """Untimed warmup: n steps, then further batches of n (at least one step)
    until min_seconds of wall time have passed, so that the clocks have left
    their ramp before the timed steps. Returns (steps run, seconds)."""
    t0 = time.perf_counter()
    if n <= 0 and min_seconds <= 0:
        return 0, 0.0
    batch, done = max(n, 1), 0
    while True:
        for _ in range(batch):
            step()
        done += batch
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= min_seconds:
            return done, time.perf_counter() - t0


def median(v):
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def device_peak():
    """Dense 16-bit MFMA peak from the device's CU count and peak clock, read
    with hipDeviceGetAttribute from the HIP runtime already in the process."""
    import ctypes
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    if path is None:
        return None
    hip = ctypes.CDLL(path)
    clock_khz, cus = ctypes.c_int(0), ctypes.c_int(0)
    # hipDeviceAttributeClockRate = 5, hipDeviceAttributeMultiprocessorCount = 63
    if hip.hipDeviceGetAttribute(ctypes.byref(clock_khz), 5, 0) != 0:
        return None
    if hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, 0) != 0:
        return None
    tflops = cus.value * clock_khz.value * 1e3 * 4096 / 1e12
    return {"cus": cus.value, "clock_mhz": clock_khz.value / 1e3, "tflops": round(tflops, 1)}


def cpu_baseline(w, inp, budget_s: float = 10.0):
    """fp64 oracle on whole batch elements of the workload, one after another
    until about ``budget_s`` seconds of host work, timed on this host."""
    from threadpoolctl import threadpool_info
    from mha_inputs import as_float64_numpy as f
    from oracle import mha_oracle

    mask = inp["key_padding_mask"]
    wq, bq, wo, bo = f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]), f(inp["b_o"])
    done, spent = 0, 0.0
    while done < w.B and spent < budget_s:
        b = slice(done, done + 1)
        t0 = time.perf_counter()
        mha_oracle.mha_forward(
            f(inp["x_q"][b]), wq, bq, wo, bo, w.h,
            x_kv=None if inp["x_kv"] is None else f(inp["x_kv"][b]), causal=w.causal,
            key_padding_mask=None if mask is None else mask[b].numpy(), n_kv_heads=w.n_g,
            gate_w=f(inp["gate_w"]), gate_b=f(inp["gate_b"]))
        spent += time.perf_counter() - t0
        done += 1
    flops = w.flops() / w.B * done
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {w.B} batch elements (all {w.T_q} query rows, all heads), "
                      f"{flops / 1e9:.1f} GFLOP in {spent:.1f} s, fp64 numpy/BLAS"}


def _oracle_threads():
    from threadpoolctl import threadpool_info
    return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))


def oracle_full_forward(w, inp, single_thread: bool = False, repeats: int = 1):
    """One full forward of workload w by the fp64 oracle on this host, every
    batch element and query row (evaluated per batch element and block of
    query rows, in order), timed (the fastest of `repeats`); optionally with
    the BLAS restricted to one thread."""
    from threadpoolctl import threadpool_limits
    from mha_inputs import as_float64_numpy as f
    from oracle import mha_oracle

    mask = inp["key_padding_mask"]
    rows = max(16, (256 << 20) // (w.h * w.T_k * 8))
    last = [time.perf_counter()]

    def progress(b, t0, t1):
        now = time.perf_counter()
        if now - last[0] > 20.0:
            last[0] = now
            print(f"[oracle] {w.name}: batch {b}, rows {t1}/{w.T_q}", file=sys.stderr,
                  flush=True)

    def run():
        t0 = time.perf_counter()
        mha_oracle.mha_forward_blocked(
            f(inp["x_q"]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]), f(inp["b_o"]), w.h,
            x_kv=f(inp["x_kv"]), causal=w.causal,
            key_padding_mask=None if mask is None else mask.numpy(), n_kv_heads=w.n_g,
            gate_w=f(inp["gate_w"]), gate_b=f(inp["gate_b"]), rows_per_block=rows,
            progress=progress)
        return time.perf_counter() - t0

    if single_thread:
        with threadpool_limits(1):
            dt, threads = min(run() for _ in range(repeats)), 1
    else:
        dt, threads = min(run() for _ in range(repeats)), _oracle_threads()
    return {"workload": w.name, "seconds": round(dt, 3),
            "tflops": round(w.flops() / dt / 1e12, 5), "cores": threads}


def oracle_timings(names=None) -> int:
    """One full forward of each named workload (default every one) by the fp64
    oracle on this host's cores, and the two smallest also single-threaded
    (one JSON line)."""
    from mha_inputs import ALL_WORKLOADS, make_inputs
    names = list(ALL_WORKLOADS) if names is None else names
    out = {"kind": "oracle", "host_cpus": len(os.sched_getaffinity(0)), "full_forward": [],
           "single_thread": []}
    for name in names:
        w = ALL_WORKLOADS[name]
        inp = make_inputs(w, seed=0)
        r = oracle_full_forward(w, inp, repeats=3 if w.flops() < 1e10 else 1)
        print(f"[oracle] {name}: {r['seconds']} s on {r['cores']} threads", file=sys.stderr,
              flush=True)
        out["full_forward"].append(r)
    for name in ("self_fp32_d512_h8_b2_t128", "causal_bf16_d512_h8_b16_t1024"):
        if name not in names:
            continue
        w = ALL_WORKLOADS[name]
        r = oracle_full_forward(w, make_inputs(w, seed=0), single_thread=True,
                                repeats=3 if w.flops() < 1e10 else 1)
        print(f"[oracle] {name}: {r['seconds']} s single-threaded", file=sys.stderr, flush=True)
        out["single_thread"].append(r)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_decode(w, inp, budget_s: float = 10.0):
    """fp64 oracle generation step on whole batch elements, one after another
    until about ``budget_s`` seconds of host work."""
    from threadpoolctl import threadpool_info
    from mha_inputs import as_float64_numpy as f
    from oracle import mha_oracle

    done, spent, nbytes = 0, 0.0, 0.0
    while done < w.B and spent < budget_s:
        b = slice(done, done + 1)
        t0 = time.perf_counter()
        mha_oracle.mha_decode(f(inp["x"][b]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                              f(inp["b_o"]), w.h, f(inp["k_cache"][b]), f(inp["v_cache"][b]),
                              inp["cache_len"][b].numpy(), n_kv_heads=w.n_g)
        spent += time.perf_counter() - t0
        nbytes += w.cache_bytes(inp["cache_len"][b].tolist())
        done += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {w.B} sequences (all heads, bf16 cache upcast to fp64), "
                      f"{nbytes / 1e6:.1f} MB of cache in {spent:.1f} s"}


def bench_decode(args, name) -> int:
    import torch
    import transformer_head_attention_amd as mha
    from mha_inputs import DECODE_WORKLOADS, make_decode_inputs

    w = DECODE_WORKLOADS[name]
    inp = make_decode_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    m = mha.MultiHeadAttention(w.D, w.h, "bf16", num_kv_heads=w.n_g)
    y = torch.empty(w.B, w.T_new, w.D, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        # the same cache rows are rewritten every step (cache_len is not advanced)
        m.decode(t["x"], t["w_qkv"], t["w_o"], t["k_cache"], t["v_cache"], t["cache_len"],
                 b_qkv=t["b_qkv"], b_o=t["b_o"], out=y, stream=stream.cuda_stream)

    warm = warm_up(torch, step, args.warmup, args.warmup_seconds)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    mha._check(mha.mha_profile_begin(m.handle, args.steps), "mha_profile_begin")
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    st, stages, _ = mha.mha_profile_end(m.handle)
    mha._check(st, "mha_profile_end")

    lens = inp["cache_len"].tolist()
    cache_bytes = w.cache_bytes(lens)
    att_ms = stages["attention"]
    achieved = cache_bytes / (att_ms * 1e-3) / 1e9 if att_ms > 0 else None
    line = {
        "metric": "MHA decode step: KV-cache bytes read per second, 1 GPU",
        "value": round(cache_bytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"steps": warm[0], "seconds": round(warm[1], 3)},
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "T_new": w.T_new, "T_max": w.T_max,
                   "cached_lengths": list(w.lengths), "D": w.D, "h": w.h, "n_kv_heads": w.n_g,
                   "d_k": w.d_k, "cache_mb_read_per_step": round(cache_bytes / 1e6, 2),
                   "tflops": round(w.flops(lens) / (ms * 1e-3) / 1e12, 3)},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "roofline": {
            "bound": "hbm",
            "achieved": None if achieved is None else round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": None if achieved is None else round(achieved / PEAK_HBM_GBS, 4),
            "traffic": read_traffic("decode_attention", name),
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_decode(w, inp),
    }
    print(json.dumps(line), flush=True)
    return 0


def copy_calibration(torch, steps: int) -> int:
    """A plain copy of known size: each launch reads and writes 1 GiB. Its
    FETCH_SIZE / WRITE_SIZE counters give the scale from counter units to
    HBM bytes."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(max(steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": max(steps, 1)}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="continue the untimed warmup until this much time has passed")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--residual", action="store_true", help="y = x_q + attention output")
    ap.add_argument("--y-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (HBM counter scale)")
    ap.add_argument("--oracle-timings", action="store_true",
                    help="run only the fp64 oracle: one full forward per workload on this host")
    args = ap.parse_args()
    if args.oracle_timings:
        return oracle_timings(args.workload.split(",") if args.workload else None)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        return copy_calibration(torch, args.steps)
    import transformer_head_attention_amd as mha
    from mha_inputs import ALL_WORKLOADS, DECODE_WORKLOADS, HEADLINE, make_inputs

    name = args.workload or HEADLINE
    if name in DECODE_WORKLOADS:
        return bench_decode(args, name)
    w = ALL_WORKLOADS[name]
    inp = make_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    m = mha.MultiHeadAttention(w.D, w.h, w.dtype, num_kv_heads=w.n_g)
    ws = m.workspace(w.B, w.T_q, w.T_k, dev)
    ydt = torch.bfloat16 if args.y_dtype == "bf16" else torch.float32
    y = torch.empty(w.B, w.T_q, w.D, dtype=ydt, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        m.forward(t["x_q"], t["w_qkv"], t["w_o"], b_qkv=t["b_qkv"], b_o=t["b_o"], x_kv=t["x_kv"],
                  causal=w.causal, key_padding_mask=t["key_padding_mask"], out=y, workspace=ws,
                  stream=stream.cuda_stream, residual=args.residual, y_dtype=args.y_dtype,
                  gate_w=t["gate_w"], gate_b=t["gate_b"])

    # Untimed warmup: the first stretch of sustained work runs at a different
    # clock than the steady state that follows.
    warm = warm_up(torch, step, args.warmup, args.warmup_seconds)

    # Timed region: K steps bracketed by events on the launch stream, with no
    # other events inside (an event record between kernels costs ~5 us).
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # Per-stage times: K more steps with the library's stage events (HIP
    # events on the same stream around each stage's kernels).
    mha._check(mha.mha_profile_begin(m.handle, args.steps), "mha_profile_begin")
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    st, stages, ncalls = mha.mha_profile_end(m.handle)
    mha._check(st, "mha_profile_end")

    flops = w.flops()
    single = step_times(torch, stream, step, args.steps)
    flushed = step_times(torch, stream, step, args.steps, flush_bytes=512 << 20)
    tflops = flops / (ms * 1e-3) / 1e12
    dom = max(("qkv_proj", "attention", "out_proj"), key=lambda s: stages[s])
    dom_ms = stages[dom]
    achieved = stage_flops(w, dom) / (dom_ms * 1e-3) / 1e12 if dom_ms > 0 else None
    traffic = read_traffic(dom, name) if dom in KERNEL_SOURCES else None
    # the fp32 path runs on the fp32 matrix cores: its own peak
    peak = PEAK_MFMA_FP32_TFLOPS if w.dtype == "fp32" else PEAK_MFMA_16BIT_TFLOPS
    line = {
        # the headline metric names its workload; other workloads are named in place
        "metric": METRIC if name == HEADLINE else f"MHA fwd TFLOP/s + % bf16 MFMA peak, {name}, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"steps": warm[0], "seconds": round(warm[1], 3)},
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "T_q": w.T_q, "T_k": w.T_k, "D": w.D, "h": w.h,
                   "n_kv_heads": w.n_g, "d_k": w.d_k, "causal": w.causal, "cross": w.cross,
                   "key_padding": w.padding is not None, "gated": w.gate,
                   "gflop_per_step": round(flops / 1e9, 3),
                   "intermediates": ("fp32 Q/K/V/P/O, fp32 accumulate" if w.dtype == "fp32"
                                     else "fp16 Q/K/V/P/O, fp32 accumulate"),
                   "y": args.y_dtype, "residual": args.residual},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_MFMA_16BIT_TFLOPS, 2),
        **({"pct_fp32_peak": round(100.0 * tflops / PEAK_MFMA_FP32_TFLOPS, 2)}
           if w.dtype == "fp32" else {}),
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "step_ms": {"median": round(median(single), 4), "min": round(single[0], 4)},
        "flushed": {"median_ms": round(median(flushed), 4), "min_ms": round(flushed[0], 4),
                    "value_median": round(flops / (median(flushed) * 1e-3) / 1e12, 2),
                    "flush_bytes": 512 << 20},
        "peak_device": device_peak(),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": None if achieved is None else round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": None if achieved is None else round(achieved / peak, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp)
        # the smallest workload in full, on all threads and on one
        from mha_inputs import WORKLOADS as _W
        w1 = _W["self_fp32_d512_h8_b2_t128"]
        inp1 = make_inputs(w1, seed=0)
        line["cpu_baseline"]["full_forward_small"] = [
            oracle_full_forward(w1, inp1, repeats=3),
            oracle_full_forward(w1, inp1, True, repeats=3)]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
