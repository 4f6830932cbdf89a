#!/usr/bin/env python3
"""Benchmark: one FP8 nn.Linear step on one MI355X through libfgfp8.

A step is one pass of the whole hot path over one batch (tokens=8192,
in=7168, out=4096, bf16 randn inputs, 1x128 / 128x128 fp32 scales):

  forward  cast x per token; cast W per 128x128 block (+ its transpose);
           y  = GEMM(xq, Wq)                  [8192, 4096] bf16
  dgrad    cast dY per token;  dX = GEMM(dYq, WqT)   [8192, 7168] bf16
  wgrad    cast dY^T and x^T per token (groups along tokens);
           dW += GEMM(dYTq, xTq)             [4096, 7168] fp32

`value` is the step's GEMM work (3 x 2*8192*4096*7168 flop) over the whole
step time, casts included.  Per-kernel times come from HIP events recorded
on the launch stream inside the timed region.  Extra kernel measurements
(the 16384x4096 cast, the 4096x7168x7168 GEMM) run after the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOPS (% FP8 MFMA peak); cast GB/s (% HBM peak)"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    return ap.parse_args()


class Linear:
    """Preallocated device buffers of one FP8 linear step."""

    def __init__(self, fg, torch, si, tokens, d_in, d_out):
        dev = "cuda"
        self.fg, self.torch = fg, torch
        self.T, self.I, self.O = tokens, d_in, d_out
        self.x = si.randn((tokens, d_in), si.SEED_A).to(dev)
        self.W = si.randn((d_out, d_in), si.SEED_B).to(dev)
        self.dY = si.randn((tokens, d_out), si.SEED_DY).to(dev)
        u8, f32 = torch.uint8, torch.float32
        mk = lambda r, c: torch.empty((r, c), dtype=u8, device=dev)
        self.xq, self.sx = mk(tokens, d_in), fg.mn_major_scales(tokens, d_in // 128)
        self.Wq, self.sW = mk(d_out, d_in), torch.empty((d_out // 128, d_in // 128), dtype=f32, device=dev)
        self.WqT, self.sWT = mk(d_in, d_out), torch.empty((d_in // 128, d_out // 128), dtype=f32, device=dev)
        self.dYq, self.sdY = mk(tokens, d_out), fg.mn_major_scales(tokens, d_out // 128)
        self.dYTq, self.sdYT = mk(d_out, tokens), fg.mn_major_scales(d_out, tokens // 128)
        self.xTq, self.sxT = mk(d_in, tokens), fg.mn_major_scales(d_in, tokens // 128)
        self.y = torch.empty((tokens, d_out), dtype=torch.bfloat16, device=dev)
        self.dX = torch.empty((tokens, d_in), dtype=torch.bfloat16, device=dev)
        self.dW = torch.zeros((d_out, d_in), dtype=f32, device=dev)

    def ops(self):
        fg = self.fg
        return [
            ("cast_x", lambda: fg.cast_per_token(self.x, self.xq, self.sx, 128, fg.SF_FP32)),
            ("cast_W", lambda: fg.cast_per_block(self.W, self.Wq, self.sW, self.WqT, self.sWT, fg.SF_FP32)),
            ("gemm_fwd", lambda: fg.gemm_fp8_nt_bf16(self.xq, self.sx, self.Wq, self.sW, self.y)),
            ("cast_dY", lambda: fg.cast_per_token(self.dY, self.dYq, self.sdY, 128, fg.SF_FP32)),
            ("gemm_dgrad", lambda: fg.gemm_fp8_nt_bf16(self.dYq, self.sdY, self.WqT, self.sWT, self.dX)),
            ("cast_dYT", lambda: fg.cast_per_token(self.dY.t(), self.dYTq, self.sdYT, 128, fg.SF_FP32)),
            ("cast_xT", lambda: fg.cast_per_token(self.x.t(), self.xTq, self.sxT, 128, fg.SF_FP32)),
            ("gemm_wgrad", lambda: fg.wgrad_gemm_fp8_nt_fp32(self.dYTq, self.sdYT, self.xTq, self.sxT, self.dW)),
        ]

    def work(self):
        """Algorithmic flops (GEMMs) and HBM bytes (casts: read input once, write q + scales once)."""
        T, I, O = self.T, self.I, self.O
        f = 2.0 * T * I * O
        tok = lambda r, c: r * c * 2 + r * c + r * (c // 128) * 4
        blk = O * I * 2 + 2 * O * I + 2 * (O // 128) * (I // 128) * 4
        # GEMM bytes: A + B + scales + output (wgrad reads and writes fp32 D)
        return {
            "cast_x": ("GB/s", tok(T, I)), "cast_W": ("GB/s", blk),
            "cast_dY": ("GB/s", tok(T, O)), "cast_dYT": ("GB/s", tok(O, T)), "cast_xT": ("GB/s", tok(I, T)),
            "gemm_fwd": ("TFLOPS", f), "gemm_dgrad": ("TFLOPS", f), "gemm_wgrad": ("TFLOPS", f),
        }


def timed_ops(torch, ops, steps, warmup):
    for _ in range(warmup):
        for _, fn in ops:
            fn()
    torch.cuda.synchronize()
    ev = {name: [] for name, _ in ops}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        for name, fn in ops:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[name].append((a, b))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per = {name: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) for name, pairs in ev.items()}
    return total_ms, per


def rate(unit, amount, ms):
    if unit == "TFLOPS":
        v = amount / (ms * 1e-3) / 1e12
        return {"ms": ms, "tflops": v, "frac_fp8_peak": v / PEAK_FP8_TFLOPS}
    v = amount / (ms * 1e-3) / 1e9
    return {"ms": ms, "gbs": v, "frac_hbm_peak": v / PEAK_HBM_GBS}


def extra_kernels(fg, torch, si):
    """Single-kernel measurements outside the timed step (fresh buffers, median of 20)."""
    out = {}

    def med(fn, reps=20):
        ts = []
        for _ in range(3):
            fn()
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        v = sorted(a.elapsed_time(b) for a, b in ts)
        return v[len(v) // 2]

    # 16384 x 4096 per-token casts (group 128 fp32 scales; group 32 packed UE8M0)
    rows, cols = 16384, 4096
    xs = [si.randn((rows, cols), s).cuda() for s in range(3)]          # rotate > L2 + MALL
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    for gran, fmt, name in ((128, fg.SF_FP32, "cast_16384x4096_g128_fp32"),
                            (32, fg.SF_PACKED_UE8M0, "cast_16384x4096_g32_packed")):
        G = cols // gran
        sf = fg.mn_major_scales(rows, -(-G // 4) if fmt == fg.SF_PACKED_UE8M0 else G,
                                torch.int32 if fmt == fg.SF_PACKED_UE8M0 else torch.float32)
        it = iter(range(1 << 30))
        ms = med(lambda: fg.cast_per_token(xs[next(it) % 3], q, sf, gran, fmt))
        units = sf.shape[1]
        nbytes = rows * cols * 3 + rows * units * 4
        out[name] = rate("GB/s", nbytes, ms)
    del xs
    # prefill GEMM 4096 x 7168 x 7168
    for (m, n, k) in ((4096, 7168, 7168), (4096, 4096, 7168)):
        A = torch.randint(0, 0x70, (m, k), dtype=torch.uint8, device="cuda")
        B = torch.randint(0, 0x70, (n, k), dtype=torch.uint8, device="cuda")
        sa = fg.mn_major_scales(m, k // 128)
        sa.fill_(0.01)
        sb = torch.full((n // 128, k // 128), 0.01, dtype=torch.float32, device="cuda")
        D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ms = med(lambda: fg.gemm_fp8_nt_bf16(A, sa, B, sb, D))
        out[f"gemm_{m}x{n}x{k}"] = rate("TFLOPS", 2.0 * m * n * k, ms)
    return out


def cpu_baseline(si):
    """The oracle, as it stands, on a bounded sample of the same step: the forward
    GEMM for 128 tokens x 1024 output features (k = 7168) plus the per-token cast of
    those 128 tokens.  Reported in the step metric's unit (GEMM TFLOPS)."""
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    T, I, Osub = 128, 7168, 1024
    x = si.randn((T, I), si.SEED_A)
    W = si.randn((Osub, I), si.SEED_B)
    t0 = time.perf_counter()
    qa, sa = oracle.cast_per_token(si.host_array(x), 128, oracle.SF_FP32)
    qb, sb = oracle.cast_per_block(si.host_array(W), oracle.SF_FP32)
    ref, _ = oracle.gemm_nt(qa, sa, qb, sb)
    dt = time.perf_counter() - t0
    flops = 2.0 * T * I * Osub
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"forward GEMM {T}x{Osub}x{I} (fp64 exact block sums) + casts of its operands; "
                      f"{dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path runs "
              f"on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    import fine_grained_block_token_amd as fg
    import synth_inputs as si
    fg.load()
    torch.cuda.set_device(0)
    cfg = si.LINEAR
    lin = Linear(fg, torch, si, cfg["tokens"], cfg["d_in"], cfg["d_out"])
    ops = lin.ops()
    total_ms, per = timed_ops(torch, ops, args.steps, args.warmup)
    ms_step = total_ms / args.steps
    work = lin.work()
    flops_step = sum(a for (u, a) in work.values() if u == "TFLOPS")
    kernels = {name: rate(*work[name], per[name]) for name in per}
    dom = max((n for n in per if n.startswith("gemm")), key=lambda n: per[n])
    dom_tflops = work[dom][1] / (per[dom] * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": flops_step / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "fp8_linear_step tokens=8192 in=7168 out=4096 "
                               "(casts + fwd + dgrad + wgrad GEMMs)",
                   "tokens": cfg["tokens"], "d_in": cfg["d_in"], "d_out": cfg["d_out"],
                   "gran_k": 128, "scales": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": dom_tflops, "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": dom_tflops / PEAK_FP8_TFLOPS, "traffic": None},
        "kernels": kernels,
    }
    if not args.no_extra:
        result["extra"] = extra_kernels(fg, torch, si)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(si)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
