"""Benchmark of the exact attention forward on one MI355X.

One step = one ``fa_fwd`` call over the whole workload (causal Llama-3.1-8B-
shaped prefill, B=1 H=32 T=8192 d=128, bf16 inputs already in HBM).  Prints one
JSON line with the throughput in attention TFLOP/s (4*B*H*T^2*d, halved for
causal), a roofline object for the kernel (measured with HIP events on the
launch stream) and a CPU-baseline object (the fp64 oracle timed on a bounded
row sample on the host cores).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--pass fwd|bwd] [--variant exp2poly]

``--workload c4fp8`` times the FP8 forward (``fa_fwd_fp8``) on the same shape
with E4M3 inputs, against the fp8 MFMA peak.  ``--pass bwd`` times the backward instead (one step = one ``fa_bwd`` call: the
per-row D pass, the dK/dV kernel and the dQ kernel), with O and lse from the
forward computed before the timed region; its FLOP count is the usual 2.5x the
forward's (five T x T x d products instead of two).  ``--variant exp2poly``
times the forward built with part of its exponentials on the FMA path
(``libfa_exp2poly.so``) on any bf16 workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_io_aware_13_amd import build as hip_build  # noqa: E402
from exact_io_aware_13_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 MFMA: 256 CU x 2.4 GHz x 8192 FLOP/clk
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "exact_io_aware_13_amd", "csrc", "fa_fwd.hip")
FP8_SRC = os.path.join(ROOT, "exact_io_aware_13_amd", "csrc", "fa_fwd_fp8.hip")
BWD_SRC = os.path.join(ROOT, "exact_io_aware_13_amd", "csrc", "fa_bwd.hip")


def profile_tag(w: wl.Workload) -> str:
    """The workload's part of a profile file name, e.g. ``causal_b1h32t8192d128``."""
    c = "causal" if w.causal else "noncausal"
    if w.Hkv != w.H or w.Tk != w.T:
        return f"{c}_b{w.B}hq{w.H}hkv{w.Hkv}tq{w.T}tk{w.Tk}d{w.d}"
    return f"{c}_b{w.B}h{w.H}t{w.T}d{w.d}"


def traffic_file(w: wl.Workload, kernel: str = "fa_fwd") -> str:
    """The committed FETCH_SIZE/WRITE_SIZE figure for ``kernel`` on workload ``w``."""
    return os.path.join(ROOT, "profiles", f"{kernel}_traffic_{profile_tag(w)}.json")


def kernel_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(key: str, path: str, src: str = KERNEL_SRC):
    """HBM bytes per launch (per call) from the committed counter runs, if they match this kernel source."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash(src) or t.get("workload") != key:
        return None
    return t.get("bytes_per_launch")


def copy_probe(mib: int, dev) -> None:
    """One device-to-device copy of `mib` MiB, whose counters calibrate FETCH_SIZE and WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_model() -> str:
    """The host CPU's model name (``/proc/cpuinfo``), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: wl.Workload, qb, kb, vb, target_s: float, widened=None):
    """The oracle as it stands, on an evenly spaced row sample sized to ~target_s seconds.
    ``widened``: the float64 operands the oracle reads, when they are not bf16 bits."""
    import oracle
    oracle.build(force=False)
    n_rows_total = w.B * w.H * w.T

    def row_flops(rows):
        i = rows % w.T
        vis = (i + (w.Tk - w.T) + 1) if w.causal else np.full_like(i, w.Tk)
        return float(np.sum(4.0 * w.d * vis))

    def sample(n):
        return np.unique(np.linspace(0, n_rows_total - 1, n).astype(np.int64))

    # widen only what the oracle reads: all heads' rows are needed for K/V
    qd, kd, vd = widened if widened is not None else (oracle.widen_bf16(x) for x in (qb, kb, vb))
    probe = sample(64)
    oracle.attention_rows_f64(qd, kd, vd, w.causal, float(np.float32(w.scale)), probe)   # thread start-up
    t0 = time.perf_counter()
    oracle.attention_rows_f64(qd, kd, vd, w.causal, float(np.float32(w.scale)), probe)
    t_probe = time.perf_counter() - t0
    n = int(min(n_rows_total, max(64, 64 * target_s / max(t_probe, 1e-3))))
    if n >= 0.8 * n_rows_total:
        n = n_rows_total
    rows = sample(n)
    # Repeat the sample until the target is reached (the probe's estimate can
    # be short), so that the figure rests on ~target_s of CPU work.
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention_rows_f64(qd, kd, vd, w.causal, float(np.float32(w.scale)), rows)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 0.7 * target_s or passes >= 8:
            break
    return {
        "value": passes * row_flops(rows) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": ((f"all {n_rows_total} query rows (the whole workload), {passes} pass(es)"
                    if len(rows) == n_rows_total else
                    f"{len(rows)} of {n_rows_total} query rows, evenly spaced over all heads, {passes} pass(es)")
                   + f" ({passes * row_flops(rows) / 1e9:.1f} GFLOP in {dt:.1f} s, fp64, OpenMP)"),
    }


def cpu_baseline_bwd(w: wl.Workload, qb, kb, vb, dob, target_s: float):
    """The backward oracle as it stands, on the first heads of the workload (whole rows).

    The oracle parallelises over key/value heads, so the sample takes as many
    key/value heads as it has threads (all of them if that covers the
    workload), and is repeated until about ``target_s`` seconds have passed."""
    import oracle
    oracle.build(force=False)
    g = w.H // w.Hkv
    n_kv = max(1, min(w.Hkv, oracle.num_threads()))
    sub = lambda x, n: x[:1, :n]
    qs, dos = sub(qb, n_kv * g), sub(dob, n_kv * g)
    ks, vs = sub(kb, n_kv), sub(vb, n_kv)
    per_row_vis = (np.arange(w.T) + (w.Tk - w.T) + 1) if w.causal else np.full(w.T, w.Tk)
    flops = 2.5 * 4.0 * w.d * float(per_row_vis.sum()) * n_kv * g
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.attention_bwd_f64(qs, ks, vs, dos, w.causal, float(np.float32(w.scale)))
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s or passes >= 8:
            break
    whole = n_kv == w.Hkv and w.B == 1
    return {
        "value": passes * flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": ((f"the whole workload ({w.B * w.H} heads)" if whole else
                    f"{n_kv * g} of {w.B * w.H} query heads ({n_kv} key/value heads), every row")
                   + f", {passes} pass(es) ({passes * flops / 1e9:.1f} GFLOP at 2.5x the forward's count "
                     f"in {dt:.1f} s, fp64, OpenMP over key/value heads)"),
    }


def bwd_algorithmic_bytes(w: wl.Workload) -> int:
    """Q, K, V, O, dO and lse read once; dQ, dK, dV written once (the D workspace is not counted)."""
    q = w.B * w.H * w.T * w.d * 2
    kv = w.B * w.Hkv * w.Tk * w.d * 2
    return 4 * q + 4 * kv + w.B * w.H * w.T * 4


def bench_bwd(args, w: wl.Workload, dev) -> int:
    """Time K backward steps; print one JSON line."""
    import torch
    import exact_io_aware_13_amd as fa

    qb, kb, vb = wl.workload_inputs(w)
    dob = wl.workload_grad_output(w)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v, do = up(qb), up(kb), up(vb), up(dob)
    scale = float(np.float32(w.scale))
    o, lse = fa.fwd(q, k, v, w.causal, scale, n_split=1)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    workspace = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.T), dtype=torch.uint8, device=dev)

    def step():
        fa.bwd_out(q, k, v, o, lse, do, dq, dk, dv, w.causal, scale, workspace=workspace)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    kernel_ms = ev0.elapsed_time(ev1) / args.steps   # one fa_bwd call: D pass + dK/dV + dQ kernels
    ms_per_step = wall_ms / args.steps
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all().item(), "non-finite gradient"

    flops = 2.5 * w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    config = {"workload": w.title + " (backward)", "B": w.B, "H": w.H, "T": w.T, "d": w.d, "causal": w.causal}
    if w.Hkv != w.H:
        config["Hkv"] = w.Hkv
    config["pct_of_bf16_peak"] = round(100.0 * value / PEAK_BF16_TFLOPS, 2)
    out = {
        "metric": f"attention bwd TFLOP/s (2.5x forward FLOPs) and % of bf16 MFMA peak, {w.title}",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1), bf16-rounded; dO a separate draw)",
        "config": config,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.key, traffic_file(w, "fa_bwd"), BWD_SRC),
                     "kernel_ms": round(kernel_ms, 4), "algorithmic_bytes": bwd_algorithmic_bytes(w),
                     "kernels": "fa_bwd_prep_kernel + fa_bwd_dkdv_kernel + fa_bwd_dq_kernel (one fa_bwd call)"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_bwd(w, qb, kb, vb, dob, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def bench_fp8(args, w: wl.Workload, dev) -> int:
    """The FP8 forward (``fa_fwd_fp8``) on an FP8 workload; one step = one launch."""
    import torch
    import exact_io_aware_13_amd as fa
    q8, k8, v8, ds = wl.workload_inputs_fp8(w)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (q8, k8, v8))
    o = torch.empty(w.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    scale = float(np.float32(w.scale))
    descales = tuple(float(x) for x in ds)
    n_split = w.n_split if w.n_split is not None else fa.split_count(w.B, w.H, w.Hkv, w.T, w.Tk, w.d, w.causal)
    ws_bytes = fa.split_workspace_bytes(w.B, w.H, w.T, w.Tk, w.d, n_split)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        fa.fwd_fp8_out(q, k, v, o, lse, w.causal, scale, descales, n_split=n_split, workspace=workspace)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall_ms / args.steps
    assert torch.isfinite(lse).all().item(), "non-finite lse"
    flops = w.flops()
    hbm_bound = w.algorithmic_bytes() * PEAK_FP8_TFLOPS * 1e12 > flops * PEAK_HBM_GBS * 1e9
    config = {"workload": w.title, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "causal": w.causal}
    if w.Hkv != w.H or w.Tk != w.T or n_split != 1:
        config.update({"Hkv": w.Hkv, "Tk": w.Tk, "n_split": n_split})
    if hbm_bound:
        gbs = w.algorithmic_bytes() / (kernel_ms * 1e-3) / 1e9
        value, unit = w.algorithmic_bytes() / (ms_per_step * 1e-3) / 1e9, "GB/s"
        metric = f"attention fwd GB/s, {w.title}"
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel_ms": round(kernel_ms, 4),
                "flops": flops}
    else:
        value, unit = flops / (ms_per_step * 1e-3) / 1e12, "TFLOP/s"
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        metric = f"attention fwd TFLOP/s and % of fp8 MFMA peak, {w.title}"
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                "traffic": measured_traffic(w.key, traffic_file(w, "fa_fwd_fp8"), FP8_SRC),
                "kernel_ms": round(kernel_ms, 4), "algorithmic_bytes": w.algorithmic_bytes()}
        config.update({"pct_of_fp8_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
                       "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2)})
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded i.i.d. N(0,1), per-tensor scaled to FP8 E4M3)",
        "config": config,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import fp8 as ofp8
        widened = tuple(ofp8.dequantize(x, d) for x, d in zip((q8, k8, v8), ds))
        out["cpu_baseline"] = cpu_baseline(w, q8, k8, v8, args.cpu_seconds, widened=widened)
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # The clock settles only after a few dozen back-to-back launches (the first
    # ~40 show a power-management transient); 200 warm-up launches (0.1 s at
    # c4) reach the steady state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=wl.BENCH_KEY, choices=sorted(wl.BY_KEY))
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward")
    ap.add_argument("--variant", default=None, choices=sorted(hip_build.VARIANTS),
                    help="time a measurement variant of the forward (libfa_<name>.so) instead of libfa.so")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also launch one device copy of this size (counter calibration runs)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards over heads with no exchange, but no multi-GPU path is built)",
              file=sys.stderr)
        return 2

    import torch
    import exact_io_aware_13_amd as fa

    w = wl.BY_KEY[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = fa.load(fa.variant_path(args.variant)) if args.variant else fa.load()
    if args.variant and (args.pass_ == "bwd" or w.fp8):
        print("--variant applies to the bf16 forward only", file=sys.stderr)
        return 2
    if args.pass_ == "bwd":
        return bench_bwd(args, w, dev)
    if w.fp8:
        return bench_fp8(args, w, dev)

    qb, kb, vb = wl.workload_inputs(w)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(qb), up(kb), up(vb)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    scale = float(np.float32(w.scale))
    n_split = w.n_split if w.n_split is not None else fa.split_count(w.B, w.H, w.Hkv, w.T, w.Tk, w.d, w.causal,
                                                                       lib)
    ws_bytes = fa.split_workspace_bytes(w.B, w.H, w.T, w.Tk, w.d, n_split, lib)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        fa.fwd_out(q, k, v, o, lse, w.causal, scale, n_split=n_split, workspace=workspace, lib=lib)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, dev)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    kernel_ms = ev0.elapsed_time(ev1) / args.steps   # a step is one forward launch (+ the combine when split)
    ms_per_step = wall_ms / args.steps

    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12

    assert torch.isfinite(lse).all().item(), "non-finite lse"

    # the committed counter figure is the product library's; a variant build has none
    traffic = None if args.variant else measured_traffic(w.key, traffic_file(w))
    hbm_bound = w.algorithmic_bytes() * PEAK_BF16_TFLOPS * 1e12 > flops * PEAK_HBM_GBS * 1e9
    if w.key == wl.BENCH_KEY:
        metric = "attention fwd TFLOP/s and % of bf16 MFMA peak, causal B=1 H=32 T=8192 d=128"
    else:
        metric = f"attention fwd {'GB/s' if hbm_bound else 'TFLOP/s'}, {w.title}"
    if hbm_bound:
        gbs = w.algorithmic_bytes() / (kernel_ms * 1e-3) / 1e9
        value_out, unit = w.algorithmic_bytes() / (ms_per_step * 1e-3) / 1e9, "GB/s"
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel_ms": round(kernel_ms, 4), "flops": flops}
    else:
        value_out, unit = value, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic,
                "kernel_ms": round(kernel_ms, 4),
                "algorithmic_bytes": w.algorithmic_bytes()}
    config = {"workload": w.title, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "causal": w.causal}
    if w.Hkv != w.H or w.Tk != w.T or n_split != 1:
        config.update({"Hkv": w.Hkv, "Tk": w.Tk, "n_split": n_split})
    if not hbm_bound:
        config["pct_of_bf16_peak"] = round(100.0 * value / PEAK_BF16_TFLOPS, 2)
    if args.variant:
        config["variant"] = args.variant
    out = {
        "metric": metric,
        "value": round(value_out, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1), bf16-rounded)",
        "config": config,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
