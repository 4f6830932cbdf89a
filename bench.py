#!/usr/bin/env python3
"""Benchmark: one FP8 nn.Linear step on one MI355X through libfgfp8.

A step is one pass of the whole hot path over one batch (tokens=8192,
in=7168, out=4096, bf16 randn inputs, 1x128 / 128x128 fp32 scales):

  forward  cast x per token, row-wise and transposed (groups along tokens)
           in one read; cast W per 128x128 block (+ its transpose);
           y  = GEMM(xq, Wq)                  [8192, 4096] bf16
  dgrad    cast dY per token, both orientations; dX = GEMM(dYq, WqT)  [8192, 7168] bf16
  wgrad    dW += GEMM(dYTq, xTq)             [4096, 7168] fp32

`value` is the step's GEMM work (3 x 2*8192*4096*7168 flop) over the whole
step time, casts included.  Per-kernel times come from HIP events recorded
on the launch stream inside the timed region.  Extra kernel measurements
(16384x4096 casts, the other per-token cast shapes, the 1..16384-token cast
sweep, the 128x256x512, prefill and decode GEMMs)
run after the timed region; `cpu_baseline` times the oracle on a bounded
sample of the same step.
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
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (the weight gradient's instruction)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def mfma_peak(op):
    """Dense peak of the MFMA an op runs on: the weight gradients take their block sums on
    the bf16 MFMA (FP8 operands widened exactly in registers), the other GEMMs on FP8."""
    return ("bf16", PEAK_BF16_TFLOPS) if "wgrad" in op else ("fp8", PEAK_FP8_TFLOPS)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the GPU's clocks settle over the first ~12 steps (the weight gradient runs 630 us in the
    # first step and 480-500 us from about the twelfth on), so the default warm-up covers them
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (a kernel of known HBM traffic "
                         "for scaling hardware byte counters)")
    return ap.parse_args()


class Linear:
    """The FP8 linear step on synthetic inputs: fine_grained_block_token_amd.linear.Fp8Linear
    for each recipe, with the bench's op names."""

    def __init__(self, fg, torch, si, tokens, d_in, d_out):
        from fine_grained_block_token_amd.linear import Fp8Linear
        dev = "cuda"
        self.fg, self.torch, self._cls = fg, torch, Fp8Linear
        self.T, self.I, self.O = tokens, d_in, d_out
        self.x = si.randn((tokens, d_in), si.SEED_A).to(dev)
        self.W = si.randn((d_out, d_in), si.SEED_B).to(dev)
        self.dY = si.randn((tokens, d_out), si.SEED_DY).to(dev)
        self.step = Fp8Linear(tokens, d_in, d_out, "fp32", dev)
        self._ue8m0 = self._g32 = None

    def __getattr__(self, name):
        # the fp32-scale step's buffers (xq, sx, Wq, sW, y, ...) read as attributes
        step = self.__dict__.get("step")
        if step is None:
            raise AttributeError(name)
        return getattr(step, name)

    @staticmethod
    def _named(ops, names):
        return [(n, fn) for n, (_, fn) in zip(names, ops)]

    def ops(self):
        """The step: x and dY are each read once by the dual-orientation cast, which emits
        both the row-wise operand (forward / dgrad) and the transposed one (wgrad)."""
        return self._named(self.step.ops(self.x, self.W, self.dY),
                           ["cast_x_dual", "cast_W", "gemm_fwd", "cast_dY_dual", "gemm_dgrad", "gemm_wgrad"])

    def separate_cast_ops(self):
        """The same four per-token casts as separate single-orientation launches (for reference)."""
        fg, L = self.fg, self.step
        return [
            ("cast_x", lambda: fg.cast_per_token(self.x, L.xq, L.sx, 128, fg.SF_FP32)),
            ("cast_xT", lambda: fg.cast_per_token(self.x.t(), L.xTq, L.sxT, 128, fg.SF_FP32)),
            ("cast_dY", lambda: fg.cast_per_token(self.dY, L.dYq, L.sdY, 128, fg.SF_FP32)),
            ("cast_dYT", lambda: fg.cast_per_token(self.dY.t(), L.dYTq, L.sdYT, 128, fg.SF_FP32)),
        ]

    def ue8m0_ops(self):
        """The same step with the casts' UE8M0 option (every scale a power of two, stored as
        fp32): all three GEMMs apply the exponents on the scaled MFMA, without promotion."""
        if self._ue8m0 is None:
            self._ue8m0 = self._cls(self.T, self.I, self.O, "ue8m0")
        return self._named(self._ue8m0.ops(self.x, self.W, self.dY),
                           ["cast_x_dual_ue8m0", "cast_W_ue8m0", "gemm_fwd_ue8m0", "cast_dY_dual_ue8m0",
                            "gemm_dgrad_ue8m0", "gemm_wgrad_ue8m0"])

    def g32_ops(self):
        """The same step in the UE8M0 group-32 recipe: x, W and dY each cast once in both
        orientations with 32-wide groups and packed UE8M0 scales, and the three GEMMs on the
        scaled MFMA."""
        if self._g32 is None:
            self._g32 = self._cls(self.T, self.I, self.O, "ue8m0_g32")
        return self._named(self._g32.ops(self.x, self.W, self.dY),
                           ["cast_x_dual_g32", "cast_W_dual_g32", "gemm_fwd_g32", "cast_dY_dual_g32",
                            "gemm_dgrad_g32", "gemm_wgrad_g32"])

    def work(self):
        """Algorithmic flops (GEMMs) and HBM bytes (casts: read input once, write q + scales once)."""
        T, I, O = self.T, self.I, self.O
        f = 2.0 * T * I * O
        tok = lambda r, c: r * c * 2 + r * c + r * (c // 128) * 4
        dual = lambda r, c: r * c * 2 + 2 * r * c + (r * (c // 128) + c * (r // 128)) * 4
        blk = O * I * 2 + 2 * O * I + 2 * (O // 128) * (I // 128) * 4
        return {
            "cast_x_dual": ("GB/s", dual(T, I)), "cast_W": ("GB/s", blk), "cast_dY_dual": ("GB/s", dual(T, O)),
            "cast_x": ("GB/s", tok(T, I)), "cast_xT": ("GB/s", tok(I, T)),
            "cast_dY": ("GB/s", tok(T, O)), "cast_dYT": ("GB/s", tok(O, T)),
            "gemm_fwd": ("TFLOPS", f), "gemm_dgrad": ("TFLOPS", f), "gemm_wgrad": ("TFLOPS", f),
            "cast_x_dual_ue8m0": ("GB/s", dual(T, I)), "cast_W_ue8m0": ("GB/s", blk),
            "cast_dY_dual_ue8m0": ("GB/s", dual(T, O)),
            "gemm_fwd_ue8m0": ("TFLOPS", f), "gemm_dgrad_ue8m0": ("TFLOPS", f), "gemm_wgrad_ue8m0": ("TFLOPS", f),
            "cast_x_dual_g32": ("GB/s", dual(T, I)), "cast_W_dual_g32": ("GB/s", dual(O, I)),
            "cast_dY_dual_g32": ("GB/s", dual(T, O)),
            "gemm_fwd_g32": ("TFLOPS", f), "gemm_dgrad_g32": ("TFLOPS", f), "gemm_wgrad_g32": ("TFLOPS", f),
        }


def timed_ops(torch, ops, steps, warmup):
    """Warm-up steps, then `steps` eager steps with one HIP event between consecutive kernels
    (each kernel's time is the interval between the events around it, so the intervals add
    up to the timed region); returns the total and the mean time of each op."""
    for _ in range(warmup):
        for _, fn in ops:
            fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps * len(ops) + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    j = 0
    for _ in range(steps):
        for _, fn in ops:
            fn()
            j += 1
            evs[j].record()
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    per = {name: 0.0 for name, _ in ops}
    for j in range(steps * len(ops)):
        per[ops[j % len(ops)][0]] += evs[j].elapsed_time(evs[j + 1])
    per = {name: v / steps for name, v in per.items()}
    return total_ms, per


def rate(unit, amount, ms, op=""):
    if unit == "TFLOPS":
        v = amount / (ms * 1e-3) / 1e12
        r = {"ms": ms, "tflops": v, "frac_fp8_peak": v / PEAK_FP8_TFLOPS}
        kind, peak = mfma_peak(op)
        if kind != "fp8":
            r["mfma"] = kind
            r[f"frac_{kind}_peak"] = v / peak
        return r
    v = amount / (ms * 1e-3) / 1e9
    return {"ms": ms, "gbs": v, "frac_hbm_peak": v / PEAK_HBM_GBS}


def _quantiles(ts):
    v = sorted(ts)
    q = lambda f: v[min(len(v) - 1, int(f * len(v)))]
    return q(0.5), q(0.1), q(0.9)


def _time(torch, fn, reps=20, warm=3):
    """Median / p10 / p90 of `reps` event-timed launches on the current stream."""
    for _ in range(warm):
        fn()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return _quantiles([a.elapsed_time(b) for a, b in ts])


def _time_graph(torch, fn, reps=20):
    """Per-launch time of `reps` launches captured in one HIP graph (one replay)."""
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                fn()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _measure(torch, unit, amount, fn, reps=20, op=""):
    """Rate from the per-launch time of `reps` graph-captured launches (no host gaps:
    a small kernel's eager time is mostly launch overhead), plus the eager median,
    p10 and p90 of `reps` event-timed launches."""
    q = _time(torch, fn, reps)
    g = _time_graph(torch, fn, reps)
    r = rate(unit, amount, g, op)
    r["eager_ms"], r["eager_p10_ms"], r["eager_p90_ms"] = q
    return r


def _gemm_operands(fg, torch, si, m, n, k):
    """randn*0.1 operands cast on the GPU: A per token (1x128 fp32, MN-major), B per 128x128 block."""
    a = si.randn((m, k), si.SEED_A, 0.1).cuda()
    b = si.randn((n, k), si.SEED_B, 0.1).cuda()
    A = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa = fg.mn_major_scales(m, k // 128)
    fg.cast_per_token(a, A, sa, 128, fg.SF_FP32)
    B = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    sb = torch.empty((-(-n // 128), k // 128), dtype=torch.float32, device="cuda")
    fg.cast_per_block(b, B, sb, sf_fmt=fg.SF_FP32)
    D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    return A, sa, B, sb, D


def extra_kernels(fg, torch, si):
    """Single-kernel measurements outside the timed step: median (p10, p90) of 20 event-timed
    launches; inputs that must come from HBM rotate over buffers larger than L2 + MALL."""
    out = {}
    # 16384 x 4096 per-token casts (group 128 fp32 scales; group 32 packed UE8M0), 3 inputs rotated
    rows, cols = 16384, 4096
    xs = [si.randn((rows, cols), s).cuda() for s in range(3)]
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    for gran, fmt, name in ((128, fg.SF_FP32, "cast_16384x4096_g128_fp32"),
                            (32, fg.SF_FP32, "cast_16384x4096_g32_fp32"),
                            (32, fg.SF_PACKED_UE8M0, "cast_16384x4096_g32_packed")):
        G = cols // gran
        units = -(-G // 4) if fmt == fg.SF_PACKED_UE8M0 else G
        sf = fg.mn_major_scales(rows, units, torch.int32 if fmt == fg.SF_PACKED_UE8M0 else torch.float32)
        it = iter(range(1 << 30))
        out[name] = _measure(torch, "GB/s", rows * cols * 3 + rows * units * 4,
                             lambda: fg.cast_per_token(xs[next(it) % 3], q, sf, gran, fmt))
    del xs
    # token sweep of the fused-cast table (hidden 4096, g32, packed UE8M0): eager and graph-captured
    sweep = {}
    for t in (1, 64, 512, 4096, 16384):
        x = si.randn((t, 4096), si.SEED_A).cuda()
        qt = torch.empty((t, 4096), dtype=torch.uint8, device="cuda")
        sf = fg.mn_major_scales(t, 32, torch.int32)
        qs = _time(torch, lambda: fg.cast_per_token(x, qt, sf, 32, fg.SF_PACKED_UE8M0))
        gms = _time_graph(torch, lambda: fg.cast_per_token(x, qt, sf, 32, fg.SF_PACKED_UE8M0))
        nbytes = t * 4096 * 3 + t * 32 * 4
        sweep[str(t)] = {"eager_us": qs[0] * 1e3, "graph_us": gms * 1e3,
                         "graph_gbs": nbytes / (gms * 1e-3) / 1e9}
        del x, qt, sf
    out["cast_token_sweep_4096_g32_packed"] = sweep
    # the other per-token cast shapes (with the all-zero and x1e4 groups): every group size and
    # scale format, MN-major scales, graph-timed (these are launch-scale or L2-resident)
    shapes = {}
    for rows, cols in si.CAST_SHAPES[:-1]:
        x = si.cast_workload(rows, cols).cuda()
        qs = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
        per = {}
        for gran in (128, 32):
            for fmt, fname in ((fg.SF_FP32, "fp32"), (fg.SF_UE8M0, "ue8m0"), (fg.SF_PACKED_UE8M0, "packed")):
                G = -(-cols // gran)
                units = -(-G // 4) if fmt == fg.SF_PACKED_UE8M0 else G
                sf = fg.mn_major_scales(rows, units, torch.int32 if fmt == fg.SF_PACKED_UE8M0 else torch.float32)
                gms = _time_graph(torch, lambda: fg.cast_per_token(x, qs, sf, gran, fmt))
                nbytes = rows * cols * 3 + rows * units * 4
                per[f"g{gran}_{fname}"] = {"graph_us": round(gms * 1e3, 2),
                                           "graph_gbs": round(nbytes / (gms * 1e-3) / 1e9, 1)}
        shapes[f"{rows}x{cols}"] = per
        del x, qs
    out["cast_per_token_shapes"] = shapes
    # the small GEMM (m=128, n=256, k=512): launch-scale, reported in microseconds
    m, n, k = si.GEMM_SMALL
    A, sa, B, sb, D = _gemm_operands(fg, torch, si, m, n, k)
    q = _time(torch, lambda: fg.gemm_fp8_nt_bf16(A, sa, B, sb, D))
    gms = _time_graph(torch, lambda: fg.gemm_fp8_nt_bf16(A, sa, B, sb, D))
    out[f"gemm_{m}x{n}x{k}"] = {"graph_us": gms * 1e3, "eager_us": q[0] * 1e3, "eager_p10_us": q[1] * 1e3,
                                "eager_p90_us": q[2] * 1e3}
    del A, sa, B, sb, D
    # prefill and decode GEMMs on randn*0.1 operands; a decode GEMM reads B once, so
    # 12 copies of B (> 256 MiB) rotate to keep it coming from HBM
    for (m, n, k) in list(si.GEMM_PREFILL) + list(si.GEMM_DECODE):
        A, sa, B, sb, D = _gemm_operands(fg, torch, si, m, n, k)
        Bs = [B] if m > 512 else [B] + [B.clone() for _ in range(11)]
        it = iter(range(1 << 30))
        r = _measure(torch, "TFLOPS", 2.0 * m * n * k,
                     lambda: fg.gemm_fp8_nt_bf16(A, sa, Bs[next(it) % len(Bs)], sb, D))
        nbytes = m * k + n * k + m * (k // 128) * 4 + sb.numel() * 4 + m * n * 2
        r["gbs"] = nbytes / (r["ms"] * 1e-3) / 1e9
        r["frac_hbm_peak"] = r["gbs"] / PEAK_HBM_GBS
        out[f"gemm_{m}x{n}x{k}"] = r
        if fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k) > 0:
            # the split-K GEMM on the same operands (m <= 64: stream-K shares evenly over
            # the CUs; m = 512: each 128x128 tile's K in 2 or 4 slices)
            ws = torch.empty((fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k) // 4,), dtype=torch.float32,
                             device="cuda")
            r = _measure(torch, "TFLOPS", 2.0 * m * n * k,
                         lambda: fg.gemm_fp8_nt_bf16_splitk(A, sa, Bs[next(it) % len(Bs)], sb, D, ws))
            r["gbs"] = nbytes / (r["ms"] * 1e-3) / 1e9
            r["frac_hbm_peak"] = r["gbs"] / PEAK_HBM_GBS
            r["workspace_bytes"] = ws.numel() * 4
            out[f"gemm_splitk_{m}x{n}x{k}"] = r
            del ws
        del A, sa, B, sb, D, Bs
    # UE8M0 group-32 recipe (both operands scaled per row and 32-wide K group, applied by the
    # scaled MFMA: no promotion) at the prefill and linear-forward shapes
    for (m, n, k) in ((4096, 7168, 7168), (8192, 4096, 7168)):
        a = si.randn((m, k), si.SEED_A, 0.1).cuda()
        b = si.randn((n, k), si.SEED_B, 0.1).cuda()
        A = torch.empty((m, k), dtype=torch.uint8, device="cuda")
        B = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        wa = fg.mn_major_scales(m, k // 128, torch.int32)
        wb = fg.mn_major_scales(n, k // 128, torch.int32)
        fg.cast_per_token(a, A, wa, 32, fg.SF_PACKED_UE8M0)
        fg.cast_per_token(b, B, wb, 32, fg.SF_PACKED_UE8M0)
        D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        out[f"gemm_ue8m0_g32_{m}x{n}x{k}"] = _measure(torch, "TFLOPS", 2.0 * m * n * k,
                                                      lambda: fg.gemm_fp8_nt_bf16_ue8m0_g32(A, wa, B, wb, D))
        del a, b, A, B, wa, wb, D
    # the casts' UE8M0 option (power-of-two 1x128 and 128x128 scales) at the same shapes: one or
    # two rounds of 256x256 tiles, so the wide kernel runs
    for (m, n, k) in ((4096, 7168, 7168), (8192, 4096, 7168)):
        a = si.randn((m, k), si.SEED_A, 0.1).cuda()
        b = si.randn((n, k), si.SEED_B, 0.1).cuda()
        A = torch.empty((m, k), dtype=torch.uint8, device="cuda")
        B = torch.empty((n, k), dtype=torch.uint8, device="cuda")
        sa = fg.mn_major_scales(m, k // 128)
        sb = torch.empty((-(-n // 128), k // 128), dtype=torch.float32, device="cuda")
        fg.cast_per_token(a, A, sa, 128, fg.SF_UE8M0)
        fg.cast_per_block(b, B, sb, sf_fmt=fg.SF_UE8M0)
        D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        out[f"gemm_ue8m0_{m}x{n}x{k}"] = _measure(torch, "TFLOPS", 2.0 * m * n * k,
                                                  lambda: fg.gemm_fp8_nt_bf16_ue8m0(A, sa, B, sb, D, fg.SF_UE8M0))
        del a, b, A, B, sa, sb, D
    # its weight gradient at the linear step's shape: dW [4096, 7168] += dY^T x over 8192 tokens,
    # operands cast along tokens from the transposed views
    T, I, O = si.LINEAR["tokens"], si.LINEAR["d_in"], si.LINEAR["d_out"]
    dy = si.randn((T, O), si.SEED_DY).cuda()
    x = si.randn((T, I), si.SEED_A).cuda()
    A = torch.empty((O, T), dtype=torch.uint8, device="cuda")
    B = torch.empty((I, T), dtype=torch.uint8, device="cuda")
    wa = fg.mn_major_scales(O, T // 128, torch.int32)
    wb = fg.mn_major_scales(I, T // 128, torch.int32)
    fg.cast_per_token(dy.t(), A, wa, 32, fg.SF_PACKED_UE8M0)
    fg.cast_per_token(x.t(), B, wb, 32, fg.SF_PACKED_UE8M0)
    D = torch.zeros((O, I), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    out[f"wgrad_ue8m0_g32_{O}x{I}x{T}"] = _measure(torch, "TFLOPS", 2.0 * O * I * T,
                                                   lambda: fg.wgrad_gemm_fp8_nt_fp32_ue8m0_g32(A, wa, B, wb, D),
                                                   op="wgrad")
    del dy, x, A, B, wa, wb, D
    # m-grouped contiguous GEMM: the 8-expert token mix of the grouped-GEMM exercise
    # (hidden 2048), as given and with 32x the tokens per expert
    for scale in (1, 32):
        tokens = [t * scale for t in si.MOE_TOKENS_8]
        out[f"m_grouped_8experts_tokens{sum(tokens)}_hidden2048"] = grouped_gemm_rate(fg, torch, si, tokens, 2048, 2048)
        out[f"m_grouped_ue8m0_g32_8experts_tokens{sum(tokens)}_hidden2048"] = grouped_gemm_g32_rate(
            fg, torch, si, tokens, 2048, 2048)
    return out


def fused_output_cast(fg, torch, lin):
    """The forward GEMM whose epilogue also emits the per-token FP8 cast of y (the next
    layer's operand), against the forward GEMM followed by a separate cast of y."""
    T, O = lin.T, lin.O
    yq = torch.empty((T, O), dtype=torch.uint8, device="cuda")
    ysf = fg.mn_major_scales(T, O // 128)
    f = 2.0 * T * lin.I * O
    fused = _measure(torch, "TFLOPS", f, lambda: fg.gemm_fp8_nt_bf16_cast(lin.xq, lin.sx, lin.Wq, lin.sW, lin.y,
                                                                        yq, ysf))

    def separate():
        fg.gemm_fp8_nt_bf16(lin.xq, lin.sx, lin.Wq, lin.sW, lin.y)
        fg.cast_per_token(lin.y, yq, ysf, 128, fg.SF_FP32)
    return {"fused_ms": fused["ms"], "fused_tflops": fused["tflops"],
            "gemm_then_cast_ms": _measure(torch, "TFLOPS", f, separate)["ms"]}


def grouped_gemm_rate(fg, torch, si, tokens, n, k):
    """Per-launch time of the m-grouped GEMM on randn*0.1 operands; TFLOPS over the routed
    (non-padding) rows, which is the useful work."""
    import numpy as np
    m_idx = torch.from_numpy(si.grouped_layout(tokens)).cuda()
    m, E = m_idx.numel(), len(tokens)
    a = si.randn((m, k), si.SEED_A, 0.1).cuda()
    A = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa = fg.mn_major_scales(m, k // 128)
    fg.cast_per_token(a, A, sa, 128, fg.SF_FP32)
    B = torch.empty((E, n, k), dtype=torch.uint8, device="cuda")
    sb = torch.empty((E, -(-n // 128), k // 128), dtype=torch.float32, device="cuda")
    for e in range(E):
        fg.cast_per_block(si.randn((n, k), si.SEED_B + e, 0.1).cuda(), B[e], sb[e], sf_fmt=fg.SF_FP32)
    D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    r = _measure(torch, "TFLOPS", 2.0 * sum(tokens) * n * k,
                 lambda: fg.m_grouped_gemm_fp8_nt_bf16_contiguous(A, sa, B, sb, m_idx, D))
    r["rows_with_padding"] = m
    return r


def grouped_gemm_g32_rate(fg, torch, si, tokens, n, k):
    """As grouped_gemm_rate, in the UE8M0 group-32 recipe (A and every expert's B cast per
    row with 32-wide groups and packed scales)."""
    m_idx = torch.from_numpy(si.grouped_layout(tokens)).cuda()
    m, E = m_idx.numel(), len(tokens)
    a = si.randn((m, k), si.SEED_A, 0.1).cuda()
    A = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa = fg.mn_major_scales(m, k // 128, torch.int32)
    fg.cast_per_token(a, A, sa, 32, fg.SF_PACKED_UE8M0)
    B = torch.empty((E, n, k), dtype=torch.uint8, device="cuda")
    ld = -(-n // 4) * 4
    sb = torch.empty((E, k // 128, ld), dtype=torch.int32, device="cuda").permute(0, 2, 1)[:, :n]
    for e in range(E):
        fg.cast_per_token(si.randn((n, k), si.SEED_B + e, 0.1).cuda(), B[e], sb[e], 32, fg.SF_PACKED_UE8M0)
    D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    r = _measure(torch, "TFLOPS", 2.0 * sum(tokens) * n * k,
                 lambda: fg.m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(A, sa, B, sb, m_idx, D))
    r["rows_with_padding"] = m
    return r


def cpu_baseline(si, target_s=20.0):
    """The oracle, as it stands, on a bounded sample of the same step: one complete
    linear step (casts, forward, dgrad, wgrad) at in=7168, out=4096 and T tokens, T a
    multiple of 128 sized from a 128-token calibration run so that the sample takes
    about `target_s` seconds.  Reported in the step metric's unit (GEMM TFLOPS)."""
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    I, O = si.LINEAR["d_in"], si.LINEAR["d_out"]

    def step(T):
        x = si.host_array(si.randn((T, I), si.SEED_A))
        W = si.host_array(si.randn((O, I), si.SEED_B))
        dy = si.host_array(si.randn((T, O), si.SEED_DY))
        t0 = time.perf_counter()
        qx, sx = oracle.cast_per_token(x, 128, oracle.SF_FP32)
        qw, sw = oracle.cast_per_block(W, oracle.SF_FP32)
        oracle.gemm_nt(qx, sx, qw, sw)
        qd, sd = oracle.cast_per_token(dy, 128, oracle.SF_FP32)
        oracle.gemm_nt(qd, sd, np.ascontiguousarray(qw.T), np.ascontiguousarray(sw.T))
        qdT, sdT = oracle.cast_per_token(dy, 128, oracle.SF_FP32, transpose=True)
        qxT, sxT = oracle.cast_per_token(x, 128, oracle.SF_FP32, transpose=True)
        oracle.wgrad_nt(qdT, sdT, qxT, sxT, np.zeros((O, I), np.float32))
        return time.perf_counter() - t0

    cal = step(128)
    T = int(min(si.LINEAR["tokens"], max(128, 128 * round(target_s / cal))))
    dt = step(T)
    flops = 3 * 2.0 * T * I * O
    # the casts alone, one thread and all threads: x [1024, 7168] per token (g128 fp32 scales)
    x = si.host_array(si.randn((1024, I), si.SEED_A))
    cast_bytes = x.size * 3 + x.shape[0] * (I // 128) * 4
    cast_rate = {}
    for n in (1, threads):
        oracle.set_threads(n)
        t0 = time.perf_counter()
        oracle.cast_per_token(x, 128, oracle.SF_FP32)
        cast_rate[f"{n}_threads_gbs"] = cast_bytes / (time.perf_counter() - t0) / 1e9
    oracle.set_threads(threads)
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"one full linear step (per-token and block casts, forward, dgrad, wgrad; fp64 exact "
                      f"block sums) at {T} of the 8192 tokens, in=7168, out=4096: {dt:.1f} s",
            "cast_per_token_1024x7168_g128": cast_rate}


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family and model numbers (a
    virtualised host may report only a generic name)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                      # the first processor's block is enough
                key, _, val = line.partition(":")
                info.setdefault(key.strip(), val.strip())
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    if "cpu family" in info and "model" in info:
        name += f" (family {info['cpu family']}, model {info['model']})"
    return name


def _source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "fine_grained_block_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(op):
    """HBM bytes per launch of `op` from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy of known size), or None when the summary is missing or
    the kernel's sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_fp8_linear_step.md")
    try:
        text = open(path).read()
        data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        entry = data["ops"][op]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    files = (["gemm.hip", "tile_common.h"] if op.startswith("gemm") else ["cast.hip"]) + ["device_common.h", "launch.h"]
    return entry["traffic_bytes"] if entry["source"] == _source_digest(files) else None


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
    if args.calibration_copy:
        src = torch.ones(args.calibration_copy << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = si.LINEAR
    lin = Linear(fg, torch, si, cfg["tokens"], cfg["d_in"], cfg["d_out"])
    ops = lin.ops()
    # per-kernel times: an eager pass with HIP events around every launch (after the warm-up)
    total_ms, per = timed_ops(torch, ops, args.steps, args.warmup)
    eager_ms_step = total_ms / args.steps

    # the step time: exactly `steps` steps captured in one HIP graph, replayed once after a
    # warm replay and timed between two synchronisations (no host launches, no events
    # between the kernels)
    def whole_step():
        for _, fn in ops:
            fn()
    ms_step = _time_graph(torch, whole_step, args.steps)
    work = lin.work()
    flops_step = sum(work[name][1] for name, _ in ops if work[name][0] == "TFLOPS")
    kernels = {name: rate(*work[name], per[name], name) for name in per}
    dom = max((n for n in per if n.startswith("gemm")), key=lambda n: per[n])
    dom_tflops = work[dom][1] / (per[dom] * 1e-3) / 1e12
    dom_kind, dom_peak = mfma_peak(dom)
    result = {
        "metric": METRIC,
        "value": flops_step / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "eager_ms_per_step": eager_ms_step,
        "step_timing": "steps captured in one HIP graph, one timed replay; per-kernel times from an eager pass "
                       "with HIP events around each launch",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 operands; fp8 MFMA (forward, dgrad), bf16 MFMA (wgrad); fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "fp8_linear_step tokens=8192 in=7168 out=4096 "
                               "(dual-orientation casts of x and dY, block cast of W, fwd + dgrad + wgrad GEMMs)",
                   "tokens": cfg["tokens"], "d_in": cfg["d_in"], "d_out": cfg["d_out"],
                   "gran_k": 128, "scales": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": dom, "mfma": dom_kind, "achieved": dom_tflops, "peak": dom_peak,
                     "unit": "TFLOP/s", "frac": dom_tflops / dom_peak, "frac_fp8_peak": dom_tflops / PEAK_FP8_TFLOPS,
                     "traffic": measured_traffic(dom),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_flop_per_launch": work[dom][1]},
        "kernels": kernels,
    }
    if not args.no_extra:
        result["extra"] = extra_kernels(fg, torch, si)
        result["extra"]["linear_step_separate_casts"] = {
            name: _measure(torch, *work[name], fn) for name, fn in lin.separate_cast_ops()}
        result["extra"]["forward_with_output_cast"] = fused_output_cast(fg, torch, lin)
        ue = lin.ue8m0_ops()
        u_ms, u_per = timed_ops(torch, ue, 10, 2)
        u_ms /= 10
        result["extra"]["linear_step_ue8m0_scales"] = {
            "ms_per_step": u_ms, "tflops": flops_step / (u_ms * 1e-3) / 1e12,
            "kernels": {name: rate(*work[name], u_per[name], name) for name in u_per}}
        g32 = lin.g32_ops()
        g_ms, g_per = timed_ops(torch, g32, 10, 2)
        g_ms /= 10
        result["extra"]["linear_step_ue8m0_g32"] = {
            "ms_per_step": g_ms, "tflops": flops_step / (g_ms * 1e-3) / 1e12,
            "kernels": {name: rate(*work[name], g_per[name], name) for name in g_per}}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(si)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
