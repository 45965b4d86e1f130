"""Benchmark: one step = attention forward + the full recomputation backward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3]

Prints ONE JSON line on stdout.  The default workload is the causal d=128
training shape (B=8, H=16, N=2048, d=128, 16K tokens) on one GPU; inputs are
seeded synthetic bf16 N(0,1) tensors already resident in HBM when timing starts.

Timing: HIP events on the stream the kernels run on (torch's current stream,
which is the stream handed to libfa), one event between every kernel launch,
so each kernel's duration is measured live in every timed step; the line reports
medians over the timed steps (means alongside).  After timing, one more step is
compared bit for bit with the last timed one (deterministic_rerun), and the GPU
clock is sampled over one second of further steps.

FLOP accounting (algorithmic, not what the kernels execute):
  forward   4 * B * H * N^2 * d, halved for causal, times the active-block
            fraction for a block mask;
  backward  2.5 x forward;  a step is forward + backward = 3.5 x forward.
Per kernel (for the roofline of the dominant kernel): forward kernel = 1 x
forward (two products), dK/dV kernel = 2 x forward (four products), dQ kernel =
1.5 x forward (three products; it also forms D_i = rowsum(dO * O), which is
not counted).
Peak: MI355X dense bf16 matrix throughput 2516.6 TFLOP/s (256 CU x 2.4 GHz x
4096 flop/clk), HBM 8 TB/s.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed, so that a
    change of comments or layout alone keeps the hash (string literals in these
    sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the code (not the comments) of every kernel and host source file."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "exact_io_aware_62_amd", "csrc", "*"))):
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def mask_fraction(cfg) -> float:
    if cfg.causal:
        return 0.5
    bm = cfg.blockmask()
    if bm is not None:
        return float(bm.mean())
    return 1.0


def measured_traffic(workload: str, kernel: str, launches_per_step: int = 1):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when absent or taken on different kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as f:
        data = json.load(f)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = data.get("workloads", {}).get(workload, {}).get(kernel)
    if not entry:
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def sample_clock(run, seconds: float, torch, dev):
    """Median, min and max of the GPU's current graphics clock (MHz) while `run` keeps the
    GPU busy: batches of steps are queued and the clock is read from this same thread
    while the queued work runs (a sampler thread would hold up the launches and let the
    GPU idle).  None when the clock cannot be read on this system."""
    try:
        torch.cuda.clock_rate(dev)
    except Exception:
        return None
    samples = []
    for _ in range(20):           # queue work ahead before the first reading
        run()
    t_end = time.perf_counter() + seconds
    batches = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            run()
        try:
            samples.append(float(torch.cuda.clock_rate(dev)))
        except Exception:
            break
        batches += 1
        if batches % 8 == 0:      # bound the queue depth
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # a reading of 0 means the query failed at that moment, not a stopped clock
    zeros = sum(1 for x in samples if x <= 0.0)
    samples = [x for x in samples if x > 0.0]
    if not samples:
        return None
    return {"median": float(np.median(samples)), "min": min(samples), "max": max(samples),
            "samples": len(samples), "failed_reads": zeros,
            "source": (f"torch.cuda.clock_rate (current graphics clock) read between queued "
                       f"steps over {seconds:.1f} s of back-to-back steps")}


def gemm_reference(torch, dev, n: int = 8192, reps: int = 10):
    """TFLOP/s of a plain dense bf16 product (n x n x n, torch.matmul -> hipBLASLt) on the
    same GPU, median of `reps` timed calls: what a matrix-core-bound library kernel
    reaches on this GPU at the clock it runs at, as context for the attention kernels'
    own rates (the roofline's peak stays the published one)."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del a, b, c
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS, "ms": ms,
            "what": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), median of {reps}"}


def cpu_baseline(cfg, bits, budget_s: float, gpu_out=None):
    """Time the fp64 oracle head by head on host cores until the budget is spent:
    the forward alone and forward + backward, per head.  Also returns the parity of
    the GPU result on those heads."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max((p.get("num_threads", 1) for p in blas), default=1)
    except Exception:  # threadpoolctl missing: report the affinity set
        cores = len(os.sched_getaffinity(0))
    N = cfg.N
    allowed = oracle.allowed_mask(N, N, cfg.causal, cfg.blockmask(), cfg.mask_block)
    heads = []
    worst = {}
    t_total = 0.0
    t_fwd = 0.0
    for bh in range(cfg.B * cfg.H):
        b, h = divmod(bh, cfg.H)
        q, k, v, do = (synth.bf16_bits_to_f64(bits[x][b, h]) for x in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        o, lse, _ = oracle.head_forward(q, k, v, cfg.scale, allowed)
        t1 = time.perf_counter()
        dq, dk, dv = oracle.head_backward(q, k, v, do, cfg.scale, allowed)
        t_total += time.perf_counter() - t0
        t_fwd += t1 - t0
        heads.append(bh)
        if gpu_out is not None:
            for name, ref in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
                got = gpu_out[name](b, h)
                e = float(np.abs(got - ref).max() / np.abs(ref).max())
                worst[name] = max(worst.get(name, 0.0), e)
            e = float(np.abs(gpu_out["lse"](b, h) - lse).max())
            worst["lse_abs"] = max(worst.get("lse_abs", 0.0), e)
        if t_total >= budget_s:
            break
    flops_head = 3.5 * 4.0 * N * N * cfg.d * mask_fraction(cfg)
    tflops = flops_head * len(heads) / t_total / 1e12
    n_all = cfg.B * cfg.H
    cpu = {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{len(heads)} of {n_all} heads of the same workload, forward + "
                   f"backward, fp64 numpy (S and P materialised), {t_total:.1f} s"),
        "cpu_model": cpu_model(),
        "fwd_s": t_fwd,
        "fwd_bwd_s": t_total,
        "heads_timed": len(heads),
        "fwd_tflops": 4.0 * N * N * cfg.d * mask_fraction(cfg) * len(heads) / t_fwd / 1e12,
        # whole workload: measured when every head was timed, else scaled by heads
        "fwd_s_whole_workload": t_fwd * n_all / len(heads),
        "fwd_bwd_s_whole_workload": t_total * n_all / len(heads),
    }
    return cpu, worst


def decode_bench(args, torch, fa, dev):
    """One decoding step (B=8, H=16, Nq=1, Nk=args.decode, d=128, causal): the split-KV
    forward against the unsplit one.  Decoding is bound by reading K and V once, so the
    figure is K+V bytes per second against the 8 TB/s HBM peak."""
    B, H, Nq, Nk, d = 8, 16, 1, args.decode, 128
    bits = synth.draw_inputs_nqk(B, H, Nq, Nk, d, 4242)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = (up(bits[x]) for x in ("q", "k", "v"))
    scale = d ** -0.5
    splits = fa.splitkv_num_splits(B, H, Nq, Nk, d)
    o, lse = torch.empty_like(q), torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    timings = {}
    for name, fn in (("splitkv", lambda: fa.forward_splitkv(q, k, v, scale, True, out=o, lse=lse)),
                     ("unsplit", lambda: fa.forward(q, k, v, scale, True, out=o, lse=lse))):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        timings[name] = e0.elapsed_time(e1) / args.steps
    kv_bytes = 2.0 * B * H * Nk * d * 2
    gbs = {n: kv_bytes / (t * 1e-3) / 1e9 for n, t in timings.items()}
    log(f"[bench] decode B{B} H{H} Nq{Nq} Nk{Nk} d{d}: split-KV ({splits} splits) "
        f"{timings['splitkv'] * 1e3:.1f} us = {gbs['splitkv']:.0f} GB/s; unsplit "
        f"{timings['unsplit'] * 1e3:.1f} us = {gbs['unsplit']:.0f} GB/s")
    line = {
        "metric": "decode attention: K+V bytes read per second (one query row per head)",
        "value": gbs["splitkv"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": timings["splitkv"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode: B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal, split-KV",
                   "splits": splits, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": gbs["splitkv"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs["splitkv"] / PEAK_HBM_GBS, "traffic": None},
        "unsplit_GBps": gbs["unsplit"],
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


def fp8_bench(args, torch, fa, dev, cfg):
    """Forward only, FP8 (E4M3) Q, K, V with per-tensor descales (fa_fwd_fp8), on the
    workload's shape and mask, next to the bf16 forward on the same shape.  FLOPs as
    for the bf16 forward; peak = the dense 8-bit matrix rate, twice the bf16 one."""
    B, H, N, d = cfg.shape()
    inp = synth.draw_inputs_fp8(B, H, N, d, cfg.seed)
    q8, k8, v8 = (torch.from_numpy(inp[x]).to(dev) for x in ("q", "k", "v"))
    bits = synth.draw_inputs(B, H, N, d, cfg.seed, with_do=False)
    q, k, v = (torch.from_numpy(bits[x].view(np.int16)).to(dev).view(torch.bfloat16)
               for x in ("q", "k", "v"))
    bm = cfg.blockmask()
    bmg = None if bm is None else torch.from_numpy(bm).to(dev)
    s, causal, mb = cfg.scale, cfg.causal, cfg.mask_block
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    runs = {
        "fp8": lambda: fa.forward_fp8(q8, k8, v8, inp["q_descale"], inp["k_descale"],
                                      inp["v_descale"], s, causal, bmg, mb, out=o, lse=lse),
        "bf16": lambda: fa.forward(q, k, v, s, causal, bmg, mb, out=o, lse=lse),
    }
    ms = {}
    for name, fn in runs.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / args.steps
    flops = 4.0 * B * H * N * N * d * mask_fraction(cfg)
    tf = {n: flops / (t * 1e-3) / 1e12 for n, t in ms.items()}
    peak8 = 2 * PEAK_BF16_TFLOPS
    log(f"[bench] FP8 forward {cfg.name}: {ms['fp8'] * 1e3:.1f} us = {tf['fp8']:.0f} TFLOP/s; "
        f"bf16 forward {ms['bf16'] * 1e3:.1f} us = {tf['bf16']:.0f} TFLOP/s")
    line = {
        "metric": "attention fwd TFLOP/s, FP8 E4M3 Q/K/V with per-tensor descales",
        "value": tf["fp8"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms["fp8"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} H={H} N={N} d={d} {cfg.mask}, forward only, "
                               "FP8 inputs (descale = max|x| / 448)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": tf["fp8"], "peak": peak8, "unit": "TFLOP/s",
                     "frac": tf["fp8"] / peak8, "traffic": None},
        "bf16_forward_TFLOPs": tf["bf16"],
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C3", choices=sorted(synth.CONFIGS))
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability on P (0 = none, the default workload); with "
                         "p > 0 the step is fa_fwd_dropout + fa_bwd_dropout, timed as two parts")
    ap.add_argument("--decode", type=int, default=0, metavar="NK",
                    help="instead of the training step, time one decoding step: B=8 H=16, one "
                         "query row per head against an NK-key cache (d=128, causal), "
                         "split-KV forward and the unsplit forward, as HBM GB/s of K and V")
    ap.add_argument("--fp8", action="store_true",
                    help="instead of the training step, time the FP8 forward (fa_fwd_fp8) on "
                         "the workload's shape, next to the bf16 forward")
    ap.add_argument("--no-clock", dest="clock", action="store_false",
                    help="skip sampling the GPU clock over 1 s of extra steps")
    ap.add_argument("--no-gemm-ref", dest="gemm_ref", action="store_false",
                    help="skip timing the dense bf16 GEMM reference")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the oracle timed on host cores (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (a "
                         "known-size reference for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 copies of 1 GiB done")
        return
    if args.gpus != 1:
        log(f"bench.py times one GPU; --gpus {args.gpus} is not supported (the heads "
            "would shard across GPUs with no exchange between them).")
        sys.exit(2)

    import torch
    import exact_io_aware_62_amd as fa

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        sys.exit(1)
    fa.load_library()
    dev = torch.device("cuda:0")
    if args.decode > 0:
        return decode_bench(args, torch, fa, dev)
    cfg = synth.CONFIGS[args.workload]
    if args.fp8:
        return fp8_bench(args, torch, fa, dev, cfg)
    B, H, N, d = cfg.shape()
    bits = synth.config_inputs(cfg)

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v, do = (up(bits[x]) for x in ("q", "k", "v", "do"))
    bm = cfg.blockmask()
    bmg = None if bm is None else torch.from_numpy(bm).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dsum = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    s, causal, mb = cfg.scale, cfg.causal, cfg.mask_block

    # the launches of forward + fa_bwd (dQ with D, then dK/dV), one stage call each
    kernels = ["fwd", "dq", "dkdv"]
    pdrop = float(args.dropout)
    dseed, doff = 20261202, 0
    if pdrop > 0:
        kernels = ["fwd", "bwd"]

    def step_dropout(ev=None):
        if ev is not None:
            ev[0].record()
        fa.forward(q, k, v, s, causal, bmg, mb, out=o, lse=lse, dropout_p=pdrop, seed=dseed,
                   offset=doff)
        if ev is not None:
            ev[1].record()
        fa.backward(q, k, v, o, do, lse, s, causal, bmg, mb, workspace=ws, dq=dq, dk=dk, dv=dv,
                    dropout_p=pdrop, seed=dseed, offset=doff)
        if ev is not None:
            ev[2].record()

    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if pdrop > 0:
            return step_dropout(ev)
        if ev is not None:
            ev[0].record()
        fa.forward(q, k, v, s, causal, bmg, mb, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        fa.bwd_dq_dsum(q, k, v, o, do, lse, s, causal, bmg, mb, dsum=dsum, dq=dq)
        if ev is not None:
            ev[2].record()
        fa.bwd_dkdv(q, k, v, do, lse, dsum, s, causal, bmg, mb, dk=dk, dv=dv)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_mean = ms_total / args.steps
    # medians over the timed steps: per step (first to last event of the step) and per
    # kernel (the events on either side of its launch)
    step_ms = [e[0].elapsed_time(e[-1]) for e in evs]
    ms_per_step = float(np.median(step_ms))
    kern_ms = {name: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs]))
               for j, name in enumerate(kernels)}
    kern_ms_mean = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
                    for j, name in enumerate(kernels)}

    # determinism: one more step into fresh outputs must give the same bits
    torch.cuda.synchronize()
    saved = [t.clone() for t in (o, lse, dq, dk, dv)]
    step()
    torch.cuda.synchronize()
    deterministic = all(torch.equal(a, b) for a, b in zip(saved, (o, lse, dq, dk, dv)))
    del saved
    clock = sample_clock(step, 1.0, torch, dev) if args.clock else None
    gemm = gemm_reference(torch, dev) if args.gemm_ref else None

    frac = mask_fraction(cfg)
    fwd_flops = 4.0 * B * H * N * N * d * frac
    step_flops = 3.5 * fwd_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    kflops = {"fwd": fwd_flops, "dkdv": 2.0 * fwd_flops, "dq": 1.5 * fwd_flops,
              "bwd": 2.5 * fwd_flops}
    per_kernel = {}
    for name in kernels:
        t = kern_ms[name] * 1e-3
        tf = kflops[name] / t / 1e12
        per_kernel[name] = {"ms": kern_ms[name], "TFLOP/s": tf,
                            "frac_mfma": tf / PEAK_BF16_TFLOPS}
    # the dominant single kernel (with dropout the backward's two launches are timed
    # together, so the forward is the one single-kernel figure)
    dominant = "fwd" if pdrop > 0 else max(("fwd", "dkdv", "dq"), key=lambda n: kern_ms[n])
    achieved = per_kernel[dominant]["TFLOP/s"]
    roofline = {
        "bound": "mfma",
        "kernel": dominant,
        "achieved": achieved,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / PEAK_BF16_TFLOPS,
        "traffic": measured_traffic(cfg.name, dominant),
    }
    fwd_tflops = fwd_flops / (kern_ms["fwd"] * 1e-3) / 1e12
    bwd_ms = kern_ms["bwd"] if pdrop > 0 else kern_ms["dq"] + kern_ms["dkdv"]
    bwd_tflops = 2.5 * fwd_flops / (bwd_ms * 1e-3) / 1e12
    log(f"[bench] {cfg.name} B{B} H{H} N{N} d{d} causal={causal}: {ms_per_step:.3f} ms/step "
        f"median (mean {ms_mean:.3f}, wall {wall / args.steps * 1e3:.3f}), fwd+bwd "
        f"{value:.1f} TFLOP/s, fwd {fwd_tflops:.1f}, bwd {bwd_tflops:.1f}; kernel medians "
        f"{json.dumps(kern_ms)}; deterministic re-run: {deterministic}; clock {clock}")

    # keep the last step's outputs for the spot parity check
    torch.cuda.synchronize()

    def host(t):
        return lambda b, h: synth.bf16_bits_to_f64(
            t[b, h].view(torch.int16).cpu().numpy().view(np.uint16))

    gpu_out = {"o": host(o), "dq": host(dq), "dk": host(dk), "dv": host(dv),
               "lse": lambda b, h: lse[b, h].cpu().numpy().astype(np.float64)}
    cpu = None
    parity = None
    if args.cpu_seconds > 0 and pdrop == 0:
        cpu, parity = cpu_baseline(cfg, bits, args.cpu_seconds, gpu_out)
        log(f"[bench] oracle on host: {cpu}")
        log(f"[bench] parity on the oracle's heads: {parity}")

    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": "attention fwd / fwd+bwd TFLOP/s (bf16, causal, d=128) and % of MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_mean": ms_mean,
        "timing": "median over the timed steps (HIP events on the launch stream)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: attention forward+backward, B={B} H={H} N={N} d={d}, "
                         f"{'causal' if causal else ('butterfly block-sparse' if bm is not None else 'dense')}"
                         + (f", dropout p={pdrop}" if pdrop > 0 else "")),
            "global_batch": B, "heads": H, "seq_len": N, "head_dim": d, "causal": causal,
            "dropout": pdrop, "parallelism": "single GPU",
        },
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_tflops,
        "fwd_frac_of_peak": fwd_tflops / PEAK_BF16_TFLOPS,
        "bwd_tflops": bwd_tflops,
        "kernels": per_kernel,
        "kernel_ms_mean": kern_ms_mean,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "deterministic_rerun": deterministic,
        "clock_mhz": clock,
        "gemm_reference": gemm,
        "frac_of_gemm_reference": ({n: v["TFLOP/s"] / gemm["tflops"] for n, v in per_kernel.items()}
                                   if gemm else None),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
