"""Throughput of the fused attention hot path on one MI355X.

One step = one pass of the whole path over the causal self-attention workload of the
pages' bf16 case (B4 S1024 H8 D64, BSHD, scale 1/8): sdpa_fwd (O and LSE) then sdpa_bwd
(Delta pre-pass, dK/dV, dQ), inputs resident in HBM.  value = algorithmic TFLOP/s of the
step (forward 4 D per visible pair, backward 10 D).  The same JSON line carries the
dominant kernel's roofline (live hipEvent timing on its stream), the fp64 oracle timed on
the host, and extra measurements: the long-sequence causal forward sweep, the packed MQA
fp16 case, the varlen THD GQA case, the merge kernels and the short-sequence forward.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
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
KERNEL_SOURCES = {  # which source file holds each kernel (for the traffic-staleness check)
    "attn_fwd": "fwd.hip", "bwd_dkdv": "bwd.hip", "bwd_dq": "bwd.hip", "bwd_pre": "bwd.hip",
    "bwd_main": "bwd.hip",
    "merge_fwd": "merge.hip", "merge_bwd": "merge.hip", "attn_fwd_short": "fwd.hip",
    "bwd_short": "bwd.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    path = os.path.join(ROOT, "scaled_dot_product_05_amd", "csrc", KERNEL_SOURCES[kernel])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra measurements")
    ap.add_argument("--workload", choices=tuple(MFMA_WORKLOADS) + tuple(HBM_WORKLOADS), default="c2",
                    help="c2: causal bf16 fwd+bwd B4 S1024 H8 D64 (default); target: causal bf16 "
                         "forward only, B8 S4096 H8 D64; target_d128: the same forward at H16 "
                         "D128; target_step: fwd+bwd at B8 S4096 H8 D64 (the last three for "
                         "profiling the long-sequence kernels); short / merge: the HBM-bound "
                         "short-sequence forward and merge kernels (for profiling them; the "
                         "line reports GB/s)")
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

    # ---------------- the step: causal bf16 fwd + bwd, B4 S1024 H8 D64 ----------------
    fwd_only = args.workload in ("target", "target_d128")
    w = {"c2": lambda: synth.c2(), "target": lambda: synth.target(),
         "target_d128": lambda: synth.target(h=16, d=128),
         "target_step": lambda: synth.target(with_grad=True)}[args.workload]()
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    g = torch.empty_like(q) if fwd_only else w.dout.to(dev)
    pr = S.Problem(q, k, "bshd", w.scale, w.window)
    o = torch.empty_like(q)
    lse = torch.empty(pr.lse_shape, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(S.sdpa_bwd_workspace_size(pr.desc), dtype=torch.uint8, device=dev)
    lib = S.lib()
    hq, hk, hv, ho, hg = (S.tensor(t) for t in (q, k, v, o, g))
    hdq, hdk, hdv = (S.tensor(t) for t in (dq, dk, dv))
    hl, hnull = S.rowstat(lse), S.rowstat(None)
    desc = pr.desc
    stream = torch.cuda.current_stream().cuda_stream
    wsp, wsn = ctypes.c_void_p(ws.data_ptr()), ws.numel()

    def step():
        r1 = lib.sdpa_fwd(ctypes.byref(desc), hq, hk, hv, ho, hl, None, 0, stream)
        r2 = 0 if fwd_only else lib.sdpa_bwd(ctypes.byref(desc), hq, hk, hv, ho, hl, hg, hnull,
                                             hdq, hdk, hdv, 0, wsp, wsn, stream)
        if r1 or r2:
            raise S.SdpaError(r1 or r2, lib.sdpa_last_error().decode())

    nvis = w.batch * w.heads_q * S.n_visible(w.seqlen_q, w.seqlen_k, w.window)
    d = w.head_dim
    flops_step = S.flops(nvis, d) + (0 if fwd_only else S.flops(nvis, d, backward=True))
    # algorithmic flops per launch: forward 4 D per visible pair; backward 10 D, of which
    # dK/dV (S, dP, dV, dK products) 8 D and dQ 2 D when they run as separate launches
    alg_flops = {"attn_fwd": 4 * d * nvis, "bwd_main": 10 * d * nvis, "bwd_dkdv": 8 * d * nvis,
                 "bwd_dq": 2 * d * nvis}

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: K steps back to back, bracketed by events on the launch stream and by
    # the host clock.  No per-launch events inside it (they add a few microseconds each).
    t0 = time.perf_counter()
    with Timer(torch) as tm:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    gpu_ms = tm.ms() / args.steps
    ms_step = max(wall_ms, gpu_ms)
    value = flops_step / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step:.4f} ms (wall {wall_ms:.4f}, events {gpu_ms:.4f}) -> {value:.2f} TFLOP/s")
    # Per-kernel durations: the same K steps again with a hipEvent pair around every launch
    # (recorded by the library on the stream the kernel runs on).
    S.sdpa_profile_enable(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    S.sdpa_profile_enable(False)
    kern = S.sdpa_profile_read()
    prof_ms = (t3 - t2) * 1e3 / args.steps
    log(f"per-kernel pass: {prof_ms:.4f} ms/step with per-launch events")
    kernels = {name: {"launches": n, "avg_ms": tot / n} for name, (n, tot) in kern.items()}
    dom = max(kern, key=lambda n: kern[n][1])
    dom_ms = kern[dom][1] / kern[dom][0]
    if dom in alg_flops:
        ach = alg_flops[dom] / (dom_ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3),
                "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": round(ach / PEAK_TFLOPS["bf16"], 5),
                "traffic": traffic_for(dom, args.workload), "avg_launch_ms": round(dom_ms, 6),
                "algorithmic_flops_per_launch": alg_flops[dom]}
    else:
        nbytes = 2 * w.batch * w.seqlen_q * w.heads_q * d * 2 + w.batch * w.heads_q * w.seqlen_q * 4
        ach = nbytes / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 5),
                "traffic": traffic_for(dom, args.workload), "avg_launch_ms": round(dom_ms, 6)}

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": MFMA_WORKLOADS[args.workload],
                   "batch": w.batch, "seq_len": w.seqlen_q, "heads": w.heads_q,
                   "head_dim": w.head_dim, "mask": "causal", "flops_per_step": flops_step},
        "frac_of_peak": round(value / PEAK_TFLOPS["bf16"], 5),
        "roofline": roof,
        "kernels": kernels,
        "kernel_timing": ("per-launch hipEvent pairs on the launch stream, in a second pass of "
                          f"the same {args.steps} steps ({prof_ms:.4f} ms/step with the events)"),
    }

    if not args.no_extra:
        out["extra"] = extra(torch, S, synth, dev)

    if not args.no_cpu and args.workload == "c2":
        out["cpu_baseline"] = cpu_baseline(w, flops_step)

    print(json.dumps(out), flush=True)
    return 0


MFMA_WORKLOADS = {
    "c2": ("causal self-attention fwd+bwd, bf16, B4 S1024 H8 D64, BSHD contiguous, scale 1/8, "
           "N(0,1) inputs"),
    "target": ("causal self-attention forward, bf16, B8 S4096 H8 D64, BSHD contiguous, scale 1/8, "
               "N(0,1) inputs"),
    "target_d128": ("causal self-attention forward, bf16, B8 S4096 H16 D128, BSHD contiguous, "
                    "scale 1/sqrt(128), N(0,1) inputs"),
    "target_step": ("causal self-attention fwd+bwd, bf16, B8 S4096 H8 D64, BSHD contiguous, "
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


def time_calls(torch, fn, iters=10, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    with Timer(torch) as tm:
        for _ in range(iters):
            fn()
    return tm.ms() / iters


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

    # varlen THD GQA bf16 fwd + bwd
    w = synth.c4()
    q, k, v, g = (t.to(dev) for t in (w.q, w.k, w.v, w.dout))
    cu = torch.from_numpy(w.cu_seqlens_q).to(dev)
    lens = [int(x) for x in (w.cu_seqlens_q[1:] - w.cu_seqlens_q[:-1])]
    nvis = 16 * sum(L * (L + 1) // 2 for L in lens)
    o, lse = S.forward(q, k, v, "thd", w.scale, (-1, 0), cu_seqlens_q=cu, max_seqlen_q=max(lens))
    msf = time_calls(torch, lambda: S.forward(q, k, v, "thd", w.scale, (-1, 0), cu_seqlens_q=cu,
                                              max_seqlen_q=max(lens), out=o, lse=lse))
    msb = time_calls(torch, lambda: S.backward(q, k, v, o, lse, g, "thd", w.scale, (-1, 0),
                                               cu_seqlens_q=cu, max_seqlen_q=max(lens)))
    res["c4_thd_gqa_bf16"] = {"lengths": lens, "fwd_ms": round(msf, 4), "bwd_ms": round(msb, 4),
                              "fwd_TFLOP/s": round(4 * 128 * nvis / (msf * 1e-3) / 1e12, 2),
                              "bwd_TFLOP/s": round(10 * 128 * nvis / (msb * 1e-3) / 1e12, 2)}

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
    try:
        clk = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                             timeout=20).stdout
        res["sclk"] = [l.strip() for l in clk.splitlines() if "sclk" in l.lower()][:2]
    except Exception:  # pragma: no cover
        pass
    return res


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


def cpu_baseline(w, flops_step):
    """The fp64 oracle (as it stands) on the full step: forward then backward, every head."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    f = lambda t: synth.f64(synth.to_bhsd(t, w.layout))
    q, k, v, g = (f(t) for t in (w.q, w.k, w.v, w.dout))
    times = []
    reps = 0
    t_start = time.perf_counter()
    while reps < 5 and (time.perf_counter() - t_start) < 20.0:
        t0 = time.perf_counter()
        oracle.windowed_forward(q, k, v, w.scale, w.window)
        oracle.windowed_backward(q, k, v, g, w.scale, w.window)
        times.append(time.perf_counter() - t0)
        reps += 1
    med = float(np.median(times))
    log(f"oracle step {med:.3f} s over {reps} runs, {threads} threads")
    return {"value": round(flops_step / med / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds_per_step": round(med, 4),
            "sample": f"the full step (fp64 forward then backward of all 4x8 heads, "
                      f"B4 S1024 D64 causal), median of {reps} runs"}


if __name__ == "__main__":
    sys.exit(main())
