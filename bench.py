"""Benchmark of the fused attention forward (fa_fwd) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one fa_fwd call over the whole workload (every head, every query
tile: Q K^T, mask, online softmax, P V, epilogue).  Inputs are generated on the
host from their seeds and copied to HBM before the timed region.  The timed
region is bracketed by torch.cuda.synchronize() and measured with HIP events
recorded on the stream the kernel is launched on (torch's current stream).
Before the W warmup steps, untimed steps run back to back for --settle seconds:
from idle the GPU needs some tens of milliseconds of load to reach its steady
clocks, and a few warmup steps of a sub-millisecond kernel do not cover that.

Prints ONE JSON line on stdout.  Besides the throughput it carries:
  roofline      the kernel against MI355X's dense bf16/fp16 MFMA peak
                (2516.6 TFLOP/s = 256 CUs x 4096 flop/clk x 2.4 GHz): achieved =
                counted flops per launch / average launch time; traffic = HBM bytes
                per launch from the committed rocprofv3 counter summary in
                profiles/, reported only while the kernel sources still hash to
                the value recorded there (else null);
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded, seeded
                row sample of the same workload (time-budgeted; the sample is
                described in the line).

Counted flops follow the method's definition: 4*B*H*Nq*Nk*d, halved when causal.
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

METRIC = "attention fwd TFLOP/s (bf16, d=128, N=4K/8K/32K) + % of MFMA peak, 1 GPU"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "flashattention_tiling_online_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# the sources each forward kernel family is built from (the HBM-traffic summaries in
# profiles/ that bench.py reads are tied to the family that runs the workload)
KERNEL_SOURCES = {
    "pp": ("fa_common.hpp", "fa_tiles.hpp", "fa_philox.hpp", "fa_fwd_pp.hpp"),        # d = 128
    "mfma16": ("fa_common.hpp", "fa_tiles.hpp", "fa_philox.hpp", "fa_fwd_mfma16.hpp"),  # d = 64
    "f32": ("fa_common.hpp", "fa_fwd_f32.hpp"),                                         # fp32
    "bwd": ("fa_common.hpp", "fa_tiles.hpp", "fa_philox.hpp", "fa_bwd.hpp"),            # backward
    "merge": ("fa_common.hpp", "fa_merge.hpp"),                                         # key-split merge
}


def kernel_family(w) -> str:
    return "f32" if w.dtype == "f32" else ("pp" if w.d == 128 else "mfma16")


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def committed_traffic(w):
    """HBM bytes per launch from profiles/hbm_traffic_<workload>.txt, if still current."""
    path = os.path.join(PROFILES, f"hbm_traffic_{w.name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_sources_sha256_16") != kernel_source_hash(kernel_family(w)):
        log(f"[bench] {path} was taken on other kernel sources: traffic reported as null")
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_sclk_mhz():
    """Current shader clock of GPU 0 in MHz from rocm-smi (None if unavailable)."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    for line in r.stdout.splitlines():
        m = re.search(r"GPU\[0\].*sclk clock level:.*\((\d+)\s*Mhz\)", line)
        if m:
            return float(m.group(1))
    return None


def sclk_under(step_fn, seconds: float = 1.5):
    """Median shader clock (MHz) sampled while step_fn runs back to back."""
    import statistics
    import threading

    import torch
    stop = threading.Event()

    def spin():
        while not stop.is_set():
            for _ in range(16):
                step_fn()
            torch.cuda.synchronize()

    th = threading.Thread(target=spin)
    th.start()
    samples = []
    try:
        time.sleep(0.5)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            v = read_sclk_mhz()
            if v is None:
                break
            samples.append(v)
    finally:
        stop.set()
        th.join()
    return statistics.median(samples) if samples else None


def gemm_ceiling(dev, settle_s: float):
    """hipBLASLt bf16 GEMM (torch.mm, 8192^3) on N(0,1) data: the dense-MFMA rate this
    GPU sustains on random operands, with its clock; context for the roofline."""
    import torch
    n = 8192
    g = torch.Generator(device=dev).manual_seed(1234)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    mm = lambda: torch.mm(a, b, out=c)  # noqa: E731
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        mm()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 50
    e0.record()
    for _ in range(reps):
        mm()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"what": "torch.mm bf16 8192x8192x8192, N(0,1) operands (hipBLASLt)",
            "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "sclk_mhz": sclk_under(mm, 1.0)}


def to_device(a, dtype, dev):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def cpu_baseline(w, q, k, v, budget_s: float):
    """The oracle (part 1, fp64, all host threads) on a seeded row sample, for about
    budget_s seconds of wall time; returns the dict for the JSON line."""
    import numpy as np

    import oracle
    from flashattention_tiling_online_amd import inputs

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    bh, rows = inputs.sample_rows(w, w.B * w.H, w.Nq)  # every row, in a seeded order
    perm = np.random.Generator(np.random.PCG64(inputs.SAMPLE_SEED)).permutation(bh.size)
    bh, rows = bh[perm], rows[perm]
    chunk = max(cores * 64, 256)
    done = 0
    flops = 0.0
    t0 = time.perf_counter()
    while done < bh.size and time.perf_counter() - t0 < budget_s:
        sel = slice(done, min(done + chunk, bh.size))
        order = np.lexsort((rows[sel], bh[sel]))  # rows of one head adjacent
        b_, r_ = bh[sel][order], rows[sel][order]
        oracle.ref_rows_f64(q, k, v, w.causal, w.scale, w.dtype, b_, r_, threads=cores)
        vis = np.minimum(r_ + 1, w.Nk) if w.causal else np.full(r_.size, w.Nk)
        flops += float((4.0 * w.d * vis).sum())
        done = sel.stop
    dt = time.perf_counter() - t0
    rate = flops / dt
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            # the whole workload at the sample's rate: an extrapolation, flop-scaled
            "extrapolated_full_workload_seconds": round(w.flops / rate, 1),
            "sample_fraction_of_flops": round(flops / w.flops, 4),
            "threads_used": cores, "os_cpu_count": os.cpu_count(),
            "affinity_cores": (len(os.sched_getaffinity(0))
                               if hasattr(os, "sched_getaffinity") else None),
            "sample": (f"{done} of the {bh.size} rows of {w.name} (all heads), taken in a "
                       f"seeded random order until the {budget_s:g} s budget ran out; fp64 "
                       f"three-step oracle on {cores} threads; rate = 4*d*visible_keys per "
                       f"row summed over those rows / wall time")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=1.0, metavar="SECONDS",
                    help="before the warmup steps, untimed steps for at least this long so "
                         "the GPU clocks reach their steady state")
    ap.add_argument("--workload", default="self_8k_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=None, metavar="N",
                    help="time fa_fwd_split with N key ranges (0: fa_split_hint's count) "
                         "instead of fa_fwd; a step is then both kernels (ranges + merge)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="oracle seconds (wall)")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (fa_bwd: D, dK/dV and dQ kernels) after one "
                         "forward that supplies O and L; counted flops 2.5x the forward's")
    ap.add_argument("--dropout", type=float, default=None, metavar="P",
                    help="time fa_fwd_dropout (with --bwd: fa_bwd_dropout) with drop "
                         "probability P and a fixed seed instead of fa_fwd / fa_bwd")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the sclk readings and the GEMM ceiling run")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 3 plain device copies of MIB MiB "
                         "(reference dispatches for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import flashattention_tiling_online_amd as fa
    from flashattention_tiling_online_amd import inputs

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 3}), flush=True)
        return 0

    w = inputs.WORKLOADS[args.workload]
    log(f"[bench] {w.describe()}: generating inputs")
    q, k, v = inputs.make_qkv(w)
    tq, tk, tv = (to_device(a, w.dtype, dev) for a in (q, k, v))
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    splits = None
    p_drop = args.dropout
    seed = 0x5EEDF00D
    if p_drop is not None and (args.splits is not None or w.dtype == "f32"):
        print("bench.py --dropout: bf16/fp16 workloads without --splits only", file=sys.stderr)
        return 2
    if args.bwd:
        if w.dtype == "f32":
            print("bench.py --bwd: the backward pass takes bf16/fp16 inputs", file=sys.stderr)
            return 2
        if p_drop is None:
            fa.fa_fwd(tq, tk, tv, causal=w.causal, scale=w.scale, o=o, lse=lse, stream=stream)
        else:
            fa.fa_fwd_dropout(tq, tk, tv, p_drop, seed, causal=w.causal, scale=w.scale, o=o,
                              lse=lse, stream=stream)
        tdo = to_device(inputs.make_do(w), w.dtype, dev)
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        bws = torch.empty(max(16, fa.fa_bwd_workspace(w.B, w.H, w.Nq, w.d)), dtype=torch.uint8,
                          device=dev)
        log("[bench] timing fa_bwd (gradients of sum(dO o O)); counted flops = 2.5 x forward")

        def step():
            if p_drop is None:
                fa.fa_bwd(tq, tk, tv, o, lse, tdo, causal=w.causal, scale=w.scale, dq=dq,
                          dk=dk, dv=dv, workspace=bws, stream=stream)
            else:
                fa.fa_bwd_dropout(tq, tk, tv, o, lse, tdo, p_drop, seed, causal=w.causal,
                                  scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=bws,
                                  stream=stream)
    elif args.splits is not None:
        code = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16, "f32": fa.FA_DTYPE_F32}[w.dtype]
        splits = args.splits or max(1, fa.fa_split_hint(w.B, w.H, w.Nq, w.Nk, w.d, w.causal, code))
        ws = torch.empty(max(16, fa.fa_fwd_split_workspace(w.B, w.H, w.Nq, w.d, splits)),
                         dtype=torch.uint8, device=dev)
        log(f"[bench] fa_fwd_split with {splits} key ranges requested")

        def step():
            fa.fa_fwd_split(tq, tk, tv, causal=w.causal, scale=w.scale, n_splits=splits, o=o,
                            lse=lse, workspace=ws, stream=stream)
    elif p_drop is not None:
        log(f"[bench] timing fa_fwd_dropout, p = {p_drop}")

        def step():
            fa.fa_fwd_dropout(tq, tk, tv, p_drop, seed, causal=w.causal, scale=w.scale, o=o,
                              lse=lse, stream=stream)
    else:
        def step():
            fa.fa_fwd(tq, tk, tv, causal=w.causal, scale=w.scale, o=o, lse=lse, stream=stream)

    settled = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(8):
            step()
        settled += 8
        torch.cuda.synchronize()
    log(f"[bench] settle {settled} steps, warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps
    flops = w.flops * (2.5 if args.bwd else 1.0)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.4f} ms/step ({t_wall / args.steps * 1e3:.4f} ms wall), {tflops:.1f} TFLOP/s")

    peak = PEAK_TFLOPS[w.dtype]
    traffic = (None if (args.bwd or splits is not None or p_drop is not None)
               else committed_traffic(w))
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic}
    if not args.no_clocks:
        # the same rate against 256 CUs x 4096 flop/clk at the clock measured while
        # this kernel runs, and the GEMM rate this GPU reaches on random data
        sclk = sclk_under(step)
        if sclk:
            at = 256 * 4096 * sclk * 1e6 / 1e12 if w.dtype != "f32" else None
            roofline["sclk_mhz"] = sclk
            if at:
                roofline["peak_at_sclk"] = round(at, 1)
                roofline["frac_at_sclk"] = round(tflops / at, 4)
        if w.dtype != "f32":
            ceil = gemm_ceiling(dev, args.settle)
            roofline["gemm_reference"] = ceil
            log(f"[bench] sclk {sclk} MHz under fa_fwd; {ceil['what']}: {ceil['tflops']} TFLOP/s "
                f"at {ceil['sclk_mhz']} MHz")

    cpu = None
    if not args.no_cpu_baseline and not args.bwd and p_drop is None:
        log(f"[bench] cpu baseline (~{args.cpu_budget:.0f} s)")
        cpu = cpu_baseline(w, q, k, v, args.cpu_budget)
        log(f"[bench] cpu baseline: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} cores")

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settled,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "scale": "1/sqrt(d)",
                   "entry": (("fa_bwd" if args.bwd else "fa_fwd" if splits is None
                              else f"fa_fwd_split(n_splits={splits})")
                             + ("" if p_drop is None else "_dropout")),
                   **({} if p_drop is None else {"p_drop": p_drop}),
                   "inputs": f"N(0,{w.sigma_q:g}^2) Q, N(0,{w.sigma_k:g}^2) K, "
                             f"N(0,{w.sigma_v:g}^2) V, seeded"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fwd_kernel_sources_sha256_16": kernel_source_hash(kernel_family(w)),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
