"""Throughput of the fused attention hot path on one MI355X.

One step = one pass of the whole path over one batch of the varlen THD workload (the
largest of the pages' problem statements that fits one GPU; "Add support for cuDNN
FusedAttention + THD + CP", TransformerEngine issue 885): 8 causal sequences with lengths
uniform on [256, 4096], packed with int32 cu_seqlens, 16 q heads over 4 kv heads, head_dim
128, bf16, scale 1/sqrt(128); sdpa_fwd (O and LSE) then sdpa_bwd (Delta pre-pass, dK/dV and
dQ), inputs resident in HBM.  value = algorithmic TFLOP/s of the median step (forward
4 D per visible pair, backward 10 D).

Timing follows the pages' benchmark table (RETURNN PR 1798: warm-up steps discarded, then
min / median / mean / stddev / rounds): W warm-up steps, a timed region of exactly K steps
bracketed by device synchronisations, then a statistics pass with one hipEvent pair per
step over at least 100 steps and 200 ms, during which the shader clock is sampled.  The
same JSON line carries the dominant kernel's roofline (per-launch hipEvents recorded by the
library on its launch stream), the fp64 oracle timed on the host on a bounded sample of
the step, and extra measurements: the long-sequence causal forward sweep, the pages' bf16
C2 case, fp32, the packed MQA fp16 case, block-sparse masks, FP8, the merge kernels and
short sequences.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                       [--no-extra]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s on 1 MI355X and % of gfx950 MFMA peak per dtype"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "fp8": 5033.2}  # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {  # which source files build each kernel (for the traffic-staleness check)
    "attn_fwd": "fwd.hip", "bwd_dkdv": "bwd.hip", "bwd_dq": ("bwd.hip", "bwd_dq128.hip"), "bwd_pre": "bwd.hip",
    "bwd_main": "bwd.hip",
    "merge_fwd": "merge.hip", "merge_bwd": "merge.hip", "attn_fwd_short": "fwd.hip",
    "bwd_short": "bwd.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# headers every kernel source includes (device helpers, parameter blocks, tile sizes)
KERNEL_HEADERS = ("device.h", "params.h", "tiles.h", "launch.h", "profile.h")


def source_hash(kernel: str) -> str:
    files = KERNEL_SOURCES[kernel]
    h = hashlib.sha256()
    for name in ((files,) if isinstance(files, str) else files) + KERNEL_HEADERS:
        with open(os.path.join(ROOT, "scaled_dot_product_05_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    rec = tab.get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """hipEvent timing on the current stream around a block of launches."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()

    def ms(self):
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def step_stats(torch, fn, rounds):
    """Per-call hipEvent pairs on the current stream (the stream the library launches on)
    around ``rounds`` back-to-back calls: min / median / mean / stddev / rounds in ms."""
    import statistics
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(rounds)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    return {"min_ms": round(min(t), 5), "median_ms": round(statistics.median(t), 5),
            "mean_ms": round(statistics.fmean(t), 5),
            "stddev_ms": round(statistics.pstdev(t), 5), "rounds": rounds}


def stat_rounds(ms_est, lo=100, min_ms=200.0, hi=5000):
    """At least ``lo`` calls and at least ``min_ms`` of GPU time."""
    return int(min(hi, max(lo, math.ceil(min_ms / max(ms_est, 1e-4)))))


class ClockSampler:
    """Samples the GPU shader clock while a timed region runs: the current sclk level of
    the device's DPM table in sysfs (the value rocm-smi reports), every 25 ms."""

    def __init__(self):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self.stop = threading.Event()
        self.th = threading.Thread(target=self._run, daemon=True)

    def read(self):
        for p in self.paths:
            try:
                with open(p) as f:
                    for line in f:
                        if "*" in line:
                            return float(line.split(":")[1].strip().split("M")[0].strip("( "))
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self.stop.is_set():
            v = self.read()
            if v is not None:
                self.samples.append(v)
            self.stop.wait(0.025)

    def __enter__(self):
        self.th.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.th.join()

    def summary(self):
        import statistics
        if not self.samples:
            return {"source": "sysfs pp_dpm_sclk", "samples": 0, "median_mhz": None}
        return {"source": "sysfs pp_dpm_sclk (current level), sampled every 25 ms during the "
                          "statistics pass", "samples": len(self.samples),
                "median_mhz": statistics.median(self.samples), "min_mhz": min(self.samples),
                "max_mhz": max(self.samples)}


class Step:
    """One pass of the hot path over one batch of a workload, inputs resident in HBM:
    sdpa_fwd then (unless forward-only) sdpa_bwd, through the C ABI on the current stream,
    into preallocated outputs and workspaces."""

    def __init__(self, torch, S, w, dev, fwd_only=False):
        import numpy as np
        self.w = w
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        g = torch.empty_like(q) if fwd_only else w.dout.to(dev)
        if w.is_thd:
            self.cu = torch.from_numpy(w.cu_seqlens_q).to(dev)
            lens = np.diff(w.cu_seqlens_q).astype(np.int64)
            pr = S.Problem(q, k, "thd", w.scale, w.window, cu_seqlens_q=self.cu,
                           max_seqlen_q=int(lens.max()))
            self.nvis = w.heads_q * sum(S.n_visible(int(L), int(L), w.window) for L in lens)
        else:
            pr = S.Problem(q, k, w.layout, w.scale, w.window)
            self.nvis = w.batch * w.heads_q * S.n_visible(w.seqlen_q, w.seqlen_k, w.window)
        self.pr = pr
        o = torch.empty_like(q)
        lse = torch.empty(pr.lse_shape, dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nf, nb = S.sdpa_fwd_workspace_size(pr.desc), S.sdpa_bwd_workspace_size(pr.desc)
        self.wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device=dev)
        self.wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        self.keep = (q, k, v, g, o, lse, dq, dk, dv)
        self.h = [S.tensor(t) for t in (q, k, v, o, g, dq, dk, dv)]
        self.hl, self.hnull = S.rowstat(lse), S.rowstat(None)
        self.wf = (ctypes.c_void_p(self.wsf.data_ptr()) if nf else None, nf)
        self.wb = (ctypes.c_void_p(self.wsb.data_ptr()) if nb else None, nb)
        self.stream = torch.cuda.current_stream().cuda_stream
        self.lib, self.S, self.fwd_only = S.lib(), S, fwd_only
        d = w.head_dim
        self.flops = 4 * d * self.nvis + (0 if fwd_only else 10 * d * self.nvis)
        # algorithmic flops per launch: forward 4 D per visible pair; backward 10 D, of which
        # dK/dV (S, dP, dV, dK products) 8 D and dQ 2 D when they run as separate launches
        self.alg_flops = {"attn_fwd": 4 * d * self.nvis, "bwd_main": 10 * d * self.nvis,
                          "bwd_dkdv": 8 * d * self.nvis, "bwd_dq": 2 * d * self.nvis}

    def __call__(self):
        hq, hk, hv, ho, hg, hdq, hdk, hdv = self.h
        desc = ctypes.byref(self.pr.desc)
        r1 = self.lib.sdpa_fwd(desc, hq, hk, hv, ho, self.hl, self.wf[0], self.wf[1], self.stream)
        r2 = 0 if self.fwd_only else self.lib.sdpa_bwd(
            desc, hq, hk, hv, ho, self.hl, hg, self.hnull, hdq, hdk, hdv, 0, self.wb[0],
            self.wb[1], self.stream)
        if r1 or r2:
            raise self.S.SdpaError(r1 or r2, self.lib.sdpa_last_error().decode())


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra measurements")
    ap.add_argument("--workload", choices=tuple(MFMA_WORKLOADS) + tuple(HBM_WORKLOADS), default="c4",
                    help="c4 (default): varlen THD causal bf16 fwd+bwd, 8 sequences of "
                         "U[256,4096] tokens, Hq16/Hk4 D128; c2: causal bf16 fwd+bwd B4 S1024 H8 "
                         "D64; target / target_d128: causal bf16 forward B8 S4096 H8 D64 / H16 "
                         "D128; target_step: fwd+bwd B8 S4096 H8 D64; f32_step: causal fp32 "
                         "fwd+bwd B4 S4096 H8 D64 (these for profiling); short / merge: the "
                         "HBM-bound short-sequence and merge kernels (the line reports GB/s)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scales HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode; run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import scaled_dot_product_05_amd as S
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    S.lib()
    if args.workload in HBM_WORKLOADS:
        return hbm_main(args, torch, S, synth, dev)

    wl = args.workload
    fwd_only = wl in ("target", "target_d128")
    w = {"c4": lambda: synth.c4(), "c4_seed3": lambda: synth.c4(3), "c2": lambda: synth.c2(),
         "target": lambda: synth.target(),
         "target_d128": lambda: synth.target(h=16, d=128),
         "target_step": lambda: synth.target(with_grad=True),
         "f32_step": lambda: synth.target(b=4, s=4096, with_grad=True, dtype="f32")}[wl]()
    step = Step(torch, S, w, dev, fwd_only)
    dtype = w.dtype
    peak = PEAK_TFLOPS[dtype]

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps back to back, bracketed by a device synchronisation and
    # by events on the launch stream; no per-launch events inside it.
    t0 = time.perf_counter()
    with Timer(torch) as tm:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    region_ms = max((t1 - t0) * 1e3 / args.steps, tm.ms() / args.steps)
    # Statistics pass: one event pair per step around at least 100 steps and 200 ms,
    # while the shader clock is sampled; the median step is the headline.
    rounds = stat_rounds(region_ms)
    with ClockSampler() as clk:
        st = step_stats(torch, step, rounds)
    ms_step = st["median_ms"]
    value = step.flops / (ms_step * 1e-3) / 1e12
    log(f"timed region {args.steps} steps: {region_ms:.4f} ms/step; statistics over {rounds} "
        f"steps: median {ms_step:.4f} min {st['min_ms']:.4f} mean {st['mean_ms']:.4f} "
        f"sd {st['stddev_ms']:.4f} ms -> {value:.2f} TFLOP/s; sclk {clk.summary()}")
    # Per-kernel durations: the library records a hipEvent pair around each kernel launch on
    # the stream it launches on, over the same number of steps again.
    S.sdpa_profile_enable(True)
    for _ in range(rounds):
        step()
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    kern = S.sdpa_profile_read()
    kernels = {name: {"launches": n, "avg_ms": round(tot / n, 6)} for name, (n, tot) in kern.items()}
    dom = max(kern, key=lambda n: kern[n][1])
    dom_ms = kern[dom][1] / kern[dom][0]
    ach = step.alg_flops[dom] / (dom_ms * 1e-3) / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3), "peak": peak,
            "unit": "TFLOP/s", "frac": round(ach / peak, 5), "traffic": traffic_for(dom, wl),
            "avg_launch_ms": round(dom_ms, 6),
            "algorithmic_flops_per_launch": step.alg_flops[dom]}
    log(f"kernels: {kernels}; roofline {dom}: {ach:.1f} TFLOP/s = {ach / peak:.4f} of {peak}")

    cfg = {"workload": MFMA_WORKLOADS[wl], "dtype": dtype, "heads_q": w.heads_q,
           "heads_kv": w.heads_kv, "head_dim": w.head_dim, "mask": "causal",
           "softmax_scale": w.scale, "visible_pairs": step.nvis, "flops_per_step": step.flops}
    if w.is_thd:
        import numpy as np
        cfg.update({"layout": "thd", "sequences": w.batch,
                    "lengths": np.diff(w.cu_seqlens_q).astype(int).tolist(),
                    "total_tokens": int(w.cu_seqlens_q[-1])})
    else:
        cfg.update({"layout": w.layout, "batch": w.batch, "seq_len": w.seqlen_q})
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "config": cfg,
        "frac_of_peak": round(value / peak, 5),
        "step_stats": st,
        "timed_region": {"steps": args.steps, "ms_per_step": round(region_ms, 5),
                         "TFLOP/s": round(step.flops / (region_ms * 1e-3) / 1e12, 3)},
        "sclk": clk.summary(),
        "roofline": roof,
        "kernels": kernels,
        "kernel_timing": ("per-launch hipEvent pairs recorded by the library on the launch "
                          f"stream, over {rounds} further steps"),
    }

    if not args.no_extra:
        out["extra"] = extra(torch, S, synth, dev)

    if not args.no_cpu and wl in ("c4", "c2"):
        out["cpu_baseline"] = cpu_baseline(w, step)

    print(json.dumps(out), flush=True)
    return 0


MFMA_WORKLOADS = {
    "c4": ("varlen THD causal self-attention fwd+bwd, bf16: 8 sequences with lengths uniform on "
           "[256,4096] (seed 0), int32 cu_seqlens, 16 q heads, 4 kv heads (GQA), head_dim 128, "
           "scale 1/sqrt(128), N(0,1) q, k, v, dO"),
    "c4_seed3": ("the same varlen THD GQA D128 fwd+bwd with the lengths of seed 3 (290, 3706, 2500, "
                 "2006, 1179, 706, 2958, 651): one dominant sequence, whose first key tiles the "
                 "backward splits in halves"),
    "c2": ("causal self-attention fwd+bwd, bf16, B4 S1024 H8 D64, BSHD contiguous, scale 1/8, "
           "N(0,1) inputs"),
    "target": ("causal self-attention forward, bf16, B8 S4096 H8 D64, BSHD contiguous, scale 1/8, "
               "N(0,1) inputs"),
    "target_d128": ("causal self-attention forward, bf16, B8 S4096 H16 D128, BSHD contiguous, "
                    "scale 1/sqrt(128), N(0,1) inputs"),
    "target_step": ("causal self-attention fwd+bwd, bf16, B8 S4096 H8 D64, BSHD contiguous, "
                    "scale 1/8, N(0,1) inputs"),
    "f32_step": ("causal self-attention fwd+bwd, fp32, B4 S4096 H8 D64, BSHD contiguous, "
                 "scale 1/8, N(0,1) inputs"),
}

HBM_WORKLOADS = {
    "short": ("short-sequence forward + backward, bf16, B4096 S32 H16 D64, no mask, BSHD "
              "contiguous, scale 1/8, N(0,1) inputs"),
    "merge": ("LSE merge forward + backward, fp32, x [4,8192,16,128] BSHD, lse [4,16,8192], "
              "N(0,1) inputs"),
}


def hbm_main(args, torch, S, synth, dev) -> int:
    """The HBM-bound kernels on their own: one step is a short-sequence forward plus its
    backward, or a merge forward plus its backward.  Algorithmic bytes per launch: every
    input read once and every output written once."""
    if args.workload == "short":
        b, s, h, d = 4096, 32, 16, 64
        w = synth.dense(0, 6, "bf16", "bshd", b, s, s, h, h, d, 0.125, with_grad=True,
                        name="short")
        q, k, v, g = (t.to(dev) for t in (w.q, w.k, w.v, w.dout))
        o = torch.empty_like(q)
        lse = torch.empty(b, h, s, dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def step():
            S.forward(q, k, v, "bshd", 0.125, (-1, -1), out=o, lse=lse)
            S.backward(q, k, v, o, lse, g, "bshd", 0.125, (-1, -1), dq=dq, dk=dk, dv=dv)
        tb = q.numel() * 2
        alg = {"attn_fwd_short": 4 * tb + lse.numel() * 4,  # q, k, v in; o, lse out
               "bwd_short": 8 * tb + lse.numel() * 4}      # q, k, v, o, dO, lse in; dq, dk, dv out
        cfg = {"batch": b, "seq_len": s, "heads": h, "head_dim": d, "mask": "none"}
    else:
        b, s, h, d = 4, 8192, 16, 128
        g = torch.Generator().manual_seed(7)
        xa, xb, gx = (torch.randn(b, s, h, d, generator=g).to(dev) for _ in range(3))
        la, lb, gl = (torch.randn(b, h, s, generator=g).to(dev) for _ in range(3))
        x, l = torch.empty_like(xa), torch.empty_like(la)
        rows = b * s * h

        def step():
            S.merge(xa, la, xb, lb, "bshd", out=x, lse=l)
            S.merge_backward(xa, la, xb, lb, gx, gl, "bshd")
        alg = {"merge_fwd": rows * (3 * d * 4 + 3 * 4), "merge_bwd": rows * (5 * d * 4 + 5 * 4)}
        cfg = {"batch": b, "seq_len": s, "heads": h, "head_dim": d}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with Timer(torch) as tm:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_step = max(wall_ms, tm.ms() / args.steps)
    S.sdpa_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    kern = S.sdpa_profile_read()
    kernels = {}
    for name, (n, tot) in kern.items():
        avg = tot / n
        rec = {"launches": n, "avg_ms": avg}
        if name in alg:
            ach = alg[name] / (avg * 1e-3) / 1e9
            rec.update({"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes_per_launch": alg[name],
                        "traffic": traffic_for(name, args.workload)})
        kernels[name] = rec
        log(f"{name}: {avg * 1e3:.2f} us/launch", rec.get("achieved", ""), "GB/s")
    dom = max((n for n in kern if n in alg), key=lambda n: kern[n][1])
    roof = {k: kernels[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof.update({"kernel": dom, "avg_launch_ms": round(kernels[dom]["avg_ms"], 6)})
    total = sum(alg.values())
    print(json.dumps({
        "metric": "HBM GB/s of the " + ("short-sequence forward and backward"
                                        if args.workload == "short" else "LSE merge kernels"),
        "value": round(total / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if args.workload == "short" else "f32", "data": "synthetic",
        "config": {"workload": HBM_WORKLOADS[args.workload], **cfg},
        "roofline": roof, "kernels": kernels}), flush=True)
    return 0


def copy_calibration() -> int:
    """A plain 1 GiB device-to-device copy, 5 times: its HBM counters read 1 GiB per
    dispatch in each direction, which gives the scale of FETCH_SIZE / WRITE_SIZE."""
    import torch
    x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 1 << 30, "dispatches": 5}))
    return 0


def time_calls(torch, fn, warm=3):
    """Median of per-call hipEvent times over at least 20 calls and 50 ms (warm-up calls
    discarded first)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    with Timer(torch) as tm:
        fn()
    est = tm.ms()
    return step_stats(torch, fn, stat_rounds(est, lo=20, min_ms=50.0, hi=1000))["median_ms"]


def extra(torch, S, synth, dev):
    """Forward sweep at long S (the >= 50% of bf16 peak target), and the other kernels."""
    res = {}
    sweep = []
    for (b, s, h, hk, d) in [(8, 4096, 8, 8, 64), (4, 8192, 8, 8, 64), (2, 16384, 8, 8, 64),
                             (8, 4096, 16, 16, 128), (8, 4096, 16, 4, 128)]:
        w = synth.target(b=b, s=s, h=h, hk=hk, d=d)
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        o = torch.empty_like(q)
        lse = torch.empty(b, h, s, dtype=torch.float32, device=dev)
        ms = time_calls(torch, lambda: S.forward(q, k, v, "bshd", w.scale, (-1, 0), out=o, lse=lse))
        nvis = b * h * s * (s + 1) // 2
        tf = 4 * d * nvis / (ms * 1e-3) / 1e12
        sweep.append({"B": b, "S": s, "Hq": h, "Hk": hk, "D": d, "fwd_ms": round(ms, 4),
                      "TFLOP/s": round(tf, 2), "frac": round(tf / PEAK_TFLOPS["bf16"], 4)})
        log(f"target fwd B{b} S{s} H{h}/{hk} D{d}: {ms:.3f} ms {tf:.1f} TFLOP/s")
        del q, k, v, o, lse
    res["causal_fwd_sweep_bf16"] = sweep

    # packed MQA fp16 views (TransformerEngine issue 1195 shape)
    w = synth.c3(scale=0.1)
    buf = w.extra["packed"].to(dev)
    q, k, v = buf.split([16, 1, 1], dim=2)
    ms = time_calls(torch, lambda: S.forward(q, k, v, "sbhd", 0.1, (-1, 0)))
    nvis = 16 * 2048 * 2049 // 2
    res["c3_fwd_f16_packed"] = {"ms": round(ms, 4),
                                "TFLOP/s": round(4 * 64 * nvis / (ms * 1e-3) / 1e12, 2)}

    # the pages' bf16 causal case (B4 S1024 H8 D64): latency-bound, reported for context
    res["c2_causal_fwd_bwd_bf16"] = fwd_bwd_split(torch, S, synth.c2(), dev)
    # fp32 (true fp32: scores in fp64, no reduced-precision products) against the fp32 peak
    res["f32_causal_fwd_bwd"] = fwd_bwd_split(torch, S, synth.target(b=4, s=4096, with_grad=True,
                                                                      dtype="f32"), dev)

    # context-parallel ring emulated on one GPU (TE 885): 2 cp load-balanced chunks, per-hop
    # forward/backward over (q chunk, kv chunk) pairs folded with the LSE merge, against the
    # plain call on the same inputs
    res["cp_ring_emulated_bf16"] = cp_ring(torch, S, synth, dev)
    res["block_sparse_bf16"] = block_sparse(torch, S, synth, dev)
    res["fp8_e4m3_fwd"] = fp8_forward(torch, S, synth, dev)

    # merge kernels, HBM bound: x [4,16,8192,128] fp32, lse [4,16,8192]
    mg = {}
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        xa, xb = (torch.randn(4, 8192, 16, 128, device=dev).to(tdt) for _ in range(2))
        la, lb = (torch.randn(4, 16, 8192, device=dev) for _ in range(2))
        gx, gl = torch.randn(4, 8192, 16, 128, device=dev).to(tdt), torch.randn(4, 16, 8192, device=dev)
        es = xa.element_size()
        nrow = 4 * 16 * 8192
        msf = time_calls(torch, lambda: S.merge(xa, la, xb, lb, "bshd"))
        msb = time_calls(torch, lambda: S.merge_backward(xa, la, xb, lb, gx, gl, "bshd"))
        fb = nrow * (3 * 128 * es + 3 * 4)
        bb = nrow * (5 * 128 * es + 5 * 4)
        mg[dt] = {"fwd_GB/s": round(fb / (msf * 1e-3) / 1e9, 1),
                  "bwd_GB/s": round(bb / (msb * 1e-3) / 1e9, 1)}
        del xa, xb, gx
    res["merge_hbm"] = mg

    # short sequences (HBM bound): non-causal bf16 D64, B*H*S = 2^21
    ss = []
    for s in (16, 32, 64, 128, 512):
        b = (1 << 21) // (16 * s)
        q, k, v = (torch.randn(b, s, 16, 64, device=dev, dtype=torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty(b, 16, s, device=dev)
        ms = time_calls(torch, lambda: S.forward(q, k, v, "bshd", 0.125, out=o, lse=lse))
        nbytes = 4 * q.numel() * 2 + lse.numel() * 4
        g = torch.randn_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        msb = time_calls(torch, lambda: S.backward(q, k, v, o, lse, g, "bshd", 0.125, dq=dq,
                                                   dk=dk, dv=dv))
        bbytes = 8 * q.numel() * 2 + lse.numel() * 4
        ss.append({"S": s, "B": b, "H": 16, "ms": round(ms, 4),
                   "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bwd_ms": round(msb, 4),
                   "bwd_GB/s": round(bbytes / (msb * 1e-3) / 1e9, 1)})
        del q, k, v, o, lse, g, dq, dk, dv
    res["short_seq_fwd_bf16"] = ss
    return res


def cp_ring(torch, S, synth, dev):
    """Causal B2 S16384 H8 D64 bf16 fwd+bwd: plain calls, and the ring emulated at cp 2 and 4
    (the same algorithmic flops, 14 D per visible pair)."""
    w = synth.target(b=2, s=16384, with_grad=True)
    q, k, v, g = (t.to(dev) for t in (w.q, w.k, w.v, w.dout))
    flops = 14 * 64 * (2 * 8 * 16384 * 16385 // 2)

    def plain():
        o, lse = S.forward(q, k, v, "bshd", w.scale, (-1, 0))
        S.backward(q, k, v, o, lse, g, "bshd", w.scale, (-1, 0))

    ms = time_calls(torch, plain)
    out = {"B": 2, "S": 16384, "H": 8, "D": 64, "plain_ms": round(ms, 4),
           "plain_TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2)}
    for cp in (2, 4):
        def ring():
            o, lse = S.cp_forward(q, k, v, "bshd", w.scale, (-1, 0), cp)
            S.cp_backward(q, k, v, o, lse, g, "bshd", w.scale, (-1, 0), cp)

        ms = time_calls(torch, ring)
        out[f"cp{cp}_ms"] = round(ms, 4)
        out[f"cp{cp}_TFLOP/s"] = round(flops / (ms * 1e-3) / 1e12, 2)
        log(f"cp ring cp={cp}: {ms:.3f} ms (plain {out['plain_ms']:.3f} ms)")
    del q, k, v, g
    return out


def fwd_bwd_split(torch, S, w, dev):
    """Forward and backward of one workload timed separately (median per call), with
    TFLOP/s and the fraction of the dtype's dense MFMA peak."""
    fwd = Step(torch, S, w, dev, fwd_only=True)
    both = Step(torch, S, w, dev)
    msf = time_calls(torch, fwd)
    msb = time_calls(torch, both) - msf
    peak = PEAK_TFLOPS[w.dtype]
    tf = lambda fl, ms: fl / (ms * 1e-3) / 1e12
    d, n = w.head_dim, fwd.nvis
    r = {"dtype": w.dtype, "B": w.batch, "S": w.seqlen_q, "Hq": w.heads_q, "Hk": w.heads_kv,
         "D": d, "fwd_ms": round(msf, 4), "bwd_ms": round(msb, 4),
         "fwd_TFLOP/s": round(tf(4 * d * n, msf), 2), "bwd_TFLOP/s": round(tf(10 * d * n, msb), 2),
         "fwd_frac": round(tf(4 * d * n, msf) / peak, 4), "bwd_frac": round(tf(10 * d * n, msb) / peak, 4),
         "peak_TFLOP/s": peak, "bwd_ms_is": "fwd+bwd step median minus fwd median"}
    log(f"{w.name} {w.dtype} B{w.batch} S{w.seqlen_q} D{d}: fwd {msf:.3f} ms ({r['fwd_TFLOP/s']} TF), "
        f"bwd {msb:.3f} ms ({r['bwd_TFLOP/s']} TF)")
    del fwd, both
    return r


def block_sparse(torch, S, synth, dev):
    """Block-sparse masks (FlexAttention's BlockMask model) at B8 S4096 H8 D64 bf16, forward
    and backward, next to the native path that computes the same attention: a causal
    sliding window (band 512) against the window descriptor, and five causal documents per
    row against THD varlen over the same documents.  FLOPs count the mask's visible pairs."""
    import numpy as np
    b, s, h, d = 8, 4096, 8, 64
    w = synth.target(b=b, s=s, h=h, d=d, with_grad=True)
    q, k, v, g = (t.to(dev) for t in (w.q, w.k, w.v, w.dout))
    docs = [700, 1500, 396, 1000, 500]
    out = {}
    for name, m, native in (
            ("sliding_window_causal_512", synth.flex_mask("sliding_window_causal", s, s, band=512),
             "window"),
            ("document_5_causal", synth.flex_mask("document", s, s, doc_lengths=docs), "thd")):
        bits = torch.from_numpy(np.ascontiguousarray(synth.pack_mask(m[None, None])).view(np.int64)).to(dev)
        ms_build = time_calls(torch, lambda: S.BlockMask(bits, s, s))
        bm = S.BlockMask(bits, s, s)
        nvis = b * h * int(m.sum())
        o, lse = S.forward(q, k, v, "bshd", w.scale, block_mask=bm)
        msf = time_calls(torch, lambda: S.forward(q, k, v, "bshd", w.scale, block_mask=bm, out=o, lse=lse))
        msb = time_calls(torch, lambda: S.backward(q, k, v, o, lse, g, "bshd", w.scale, block_mask=bm))
        if native == "window":
            nf = lambda: S.forward(q, k, v, "bshd", w.scale, (512, 0), out=o, lse=lse)
            S.forward(q, k, v, "bshd", w.scale, (512, 0), out=o, lse=lse)
            nb = lambda: S.backward(q, k, v, o, lse, g, "bshd", w.scale, (512, 0))
        else:
            cu = torch.tensor(np.concatenate([[0], np.cumsum(docs * b)]), dtype=torch.int32, device=dev)
            qt, kt, vt, gt = (t.reshape(b * s, h, d) for t in (q, k, v, g))
            ot = o.reshape(b * s, h, d)
            lt = torch.empty(h, b * s, dtype=torch.float32, device=dev)
            kw = dict(cu_seqlens_q=cu, max_seqlen_q=max(docs))
            nf = lambda: S.forward(qt, kt, vt, "thd", w.scale, (-1, 0), out=ot, lse=lt, **kw)
            nf()
            nb = lambda: S.backward(qt, kt, vt, ot, lt, gt, "thd", w.scale, (-1, 0), **kw)
        msnf = time_calls(torch, nf)
        msnb = time_calls(torch, nb)
        tf = lambda flops, ms: round(flops / (ms * 1e-3) / 1e12, 2)
        out[name] = {"visible_pairs": nvis, "mask_build_ms": round(ms_build, 4),
                     "fwd_ms": round(msf, 4), "bwd_ms": round(msb, 4),
                     "fwd_TFLOP/s": tf(4 * d * nvis, msf), "bwd_TFLOP/s": tf(10 * d * nvis, msb),
                     f"{native}_fwd_ms": round(msnf, 4), f"{native}_bwd_ms": round(msnb, 4),
                     f"{native}_fwd_TFLOP/s": tf(4 * d * nvis, msnf),
                     f"{native}_bwd_TFLOP/s": tf(10 * d * nvis, msnb)}
        log(f"block mask {name}: build {ms_build:.3f} ms fwd {msf:.3f} ms bwd {msb:.3f} ms; "
            f"{native} fwd {msnf:.3f} ms bwd {msnb:.3f} ms")
    return out


def fp8_forward(torch, S, synth, dev):
    """FP8 (E4M3) forward: causal at long S (TFLOP/s against the FP8 and the bf16 MFMA
    peaks) and non-causal short sequences (bytes: q, k, v codes read once, bf16 O and fp32
    LSE written once)."""
    out = {"causal": [], "short_seq": []}
    for (b, s, h, d) in [(8, 4096, 8, 64), (2, 16384, 8, 64), (8, 4096, 16, 128)]:
        w = synth.target(b=b, s=s, h=h, d=d)
        codes = [synth.e4m3_codes(synth.f64(t)) for t in (w.q, w.k, w.v)]
        q, k, v = (c.to(dev) for c, _ in codes)
        ds = [torch.tensor([x], dtype=torch.float32, device=dev) for _, x in codes]
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(b, h, s, dtype=torch.float32, device=dev)
        ms = time_calls(torch, lambda: S.forward_fp8(q, k, v, "bshd", w.scale, *ds, window=(-1, 0),
                                                     out=o, lse=lse))
        tf = 4 * d * (b * h * s * (s + 1) // 2) / (ms * 1e-3) / 1e12
        out["causal"].append({"B": b, "S": s, "H": h, "D": d, "fwd_ms": round(ms, 4),
                              "TFLOP/s": round(tf, 2),
                              "frac_fp8_peak": round(tf / PEAK_TFLOPS["fp8"], 4),
                              "frac_bf16_peak": round(tf / PEAK_TFLOPS["bf16"], 4)})
        log(f"fp8 fwd B{b} S{s} H{h} D{d}: {ms:.3f} ms {tf:.1f} TFLOP/s")
        del q, k, v, o, lse
    for s in (128, 512):
        b = (1 << 21) // (16 * s)
        q, k, v = (torch.randn(b, s, 16, 64, device=dev).to(torch.float8_e4m3fn) for _ in range(3))
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(b, 16, s, device=dev)
        ms = time_calls(torch, lambda: S.forward_fp8(q, k, v, "bshd", 0.125, out=o, lse=lse))
        nbytes = 3 * q.numel() + 2 * o.numel() + 4 * lse.numel()
        out["short_seq"].append({"S": s, "B": b, "H": 16, "D": 64, "ms": round(ms, 4),
                                 "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        del q, k, v, o, lse
    return out


def host_cores():
    """Logical cores of the host, the cores this process may run on, the BLAS pool and the
    CPU model."""
    info = {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}
    try:
        info["nproc"] = int(subprocess.run(["nproc"], capture_output=True, text=True,
                                           timeout=10).stdout.strip())
    except Exception:  # pragma: no cover
        info["nproc"] = None
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        info["blas_threads"] = None
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((l.split(":", 1)[1].strip() for l in f
                                      if l.startswith("model name")), None)
    except OSError:  # pragma: no cover
        info["cpu_model"] = None
    return info


def cpu_baseline(w, step, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same step: forward then
    backward of whole sequences (THD) or whole batch entries, every head, taken in a fixed
    order until about ``budget_s`` seconds of CPU time have passed.  The rate is the sample's
    algorithmic flops over its time; the full step's time is extrapolated by visible pairs."""
    import numpy as np
    import oracle
    import scaled_dot_product_05_amd as S
    import synth
    cores = host_cores()
    d, done_pairs, units = w.head_dim, 0, []
    t0 = time.perf_counter()
    if w.is_thd:
        # units: (sequence, kv head with its group of q heads), in the workload's order
        cu = w.cu_seqlens_q
        grp = w.heads_q // w.heads_kv
        for s_ in range(w.batch):
            a, b = int(cu[s_]), int(cu[s_ + 1])
            for kh in range(w.heads_kv):
                hs = slice(kh * grp, (kh + 1) * grp)
                sl = lambda t, h: synth.f64(t[a:b, h]).transpose(1, 0, 2)[None]
                q, g = sl(w.q, hs), sl(w.dout, hs)
                k, v = sl(w.k, slice(kh, kh + 1)), sl(w.v, slice(kh, kh + 1))
                oracle.windowed_forward(q, k, v, w.scale, w.window)
                oracle.windowed_backward(q, k, v, g, w.scale, w.window)
                done_pairs += grp * S.n_visible(b - a, b - a, w.window)
                units.append((s_, b - a, kh))
                if time.perf_counter() - t0 >= budget_s:
                    break
            if time.perf_counter() - t0 >= budget_s:
                break
    else:
        f = lambda t: synth.f64(synth.to_bhsd(t, w.layout))
        for bi in range(w.batch):
            q, k, v, g = (f(t[bi:bi + 1]) for t in (w.q, w.k, w.v, w.dout))
            oracle.windowed_forward(q, k, v, w.scale, w.window)
            oracle.windowed_backward(q, k, v, g, w.scale, w.window)
            done_pairs += w.heads_q * S.n_visible(w.seqlen_q, w.seqlen_k, w.window)
            units.append((bi, w.seqlen_q, None))
            if time.perf_counter() - t0 >= budget_s:
                break
    el = time.perf_counter() - t0
    per = {}
    for u, L, kh in units:
        per.setdefault((u, L), []).append(kh)
    what = "; ".join((f"sequence {u} ({L} tokens), kv heads {hs[0]}-{hs[-1]} of {w.heads_kv}"
                      if hs[0] is not None else f"batch entry {u}") for (u, L), hs in per.items())
    fl = 14 * d * done_pairs
    full_s = el * step.nvis / done_pairs
    log(f"oracle: {len(units)} units, {el:.2f} s, {fl / el / 1e12:.6f} TFLOP/s; full step "
        f"~{full_s:.1f} s; cores {cores}")
    return {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores["blas_threads"] or cores["affinity"], "kind": "oracle",
            "sample": (f"fp64 oracle forward then backward of {what} "
                       f"of the same workload: {done_pairs} of its {step.nvis} visible pairs, "
                       f"one run, {el:.2f} s; value = those pairs' algorithmic flops "
                       f"(14 D per pair) / time"),
            "seconds": round(el, 3), "extrapolated_seconds_per_step": round(full_s, 2),
            "host": cores}


if __name__ == "__main__":
    sys.exit(main())
