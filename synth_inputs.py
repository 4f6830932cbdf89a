"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it only draws random
tensors of the workloads' shapes and value distributions on the CPU.  The
same host tensors feed both the oracle and (after a copy to the device) the
HIP library.

Recipe: ``torch.Generator().manual_seed(seed)`` -> ``torch.randn(shape,
float32) * scale`` -> ``.to(bfloat16)`` (or kept as float32).  Seeds: 0 for
the first operand (A / x), 1 for the second (B / W), 2 for the output
gradient dY.  The cast workloads also carry two special groups: an all-zero
group (row ``rows // 2``, columns ``[0, 128)``) and a group scaled by 1e4 (the
last 128-column group of the last row, which is also the partial group when
``cols % 128 != 0``).
"""
from __future__ import annotations

import numpy as np
import torch

SEED_A, SEED_B, SEED_DY = 0, 1, 2


def randn(shape, seed: int, scale: float = 1.0, dtype=torch.bfloat16) -> torch.Tensor:
    """CPU randn(seed) * scale, rounded to ``dtype`` (bf16 or fp32)."""
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def cast_workload(rows: int, cols: int, seed: int = SEED_A, dtype=torch.bfloat16,
                  special: bool = True) -> torch.Tensor:
    """Per-token cast input with an all-zero group and a x1e4 group."""
    x = randn((rows, cols), seed, 1.0, dtype)
    if special:
        zr = rows // 2
        x[zr, : min(128, cols)] = 0
        c0 = 128 * ((cols - 1) // 128)
        x[rows - 1, c0:] = (x[rows - 1, c0:].float() * 1e4).to(dtype)
    return x


def bf16_bits(x: torch.Tensor):
    """bf16 CPU tensor -> numpy uint16 bit patterns (no copy of values' meaning)."""
    assert x.dtype == torch.bfloat16
    return x.contiguous().view(torch.int16).numpy().view("uint16")


def host_array(x: torch.Tensor):
    """CPU tensor -> numpy array the oracle accepts (bf16 bits or float32)."""
    if x.dtype == torch.bfloat16:
        return bf16_bits(x)
    assert x.dtype == torch.float32
    return x.contiguous().numpy()


# Workload shapes.
CAST_SHAPES = [(1, 512), (7, 4096), (129, 7168), (64, 1000), (3000, 4096), (16384, 4096)]
CAST_TOKEN_SWEEP = [1, 64, 512, 4096, 16384]          # x 4096, group 32, packed UE8M0
GEMM_SMALL = (128, 256, 512)                           # m, n, k
GEMM_PREFILL = [(4096, 7168, 7168), (4096, 4096, 7168)]
GEMM_DECODE = [(m, n, k) for m in (1, 64, 512) for (n, k) in ((7168, 4096), (4096, 7168))]
LINEAR = dict(tokens=8192, d_in=7168, d_out=4096)


def grouped_layout(tokens_per_expert, align: int = 128):
    """m_indices of the contiguous grouped layout: expert e's tokens follow one another,
    each expert's segment is padded to a multiple of ``align`` rows, padding rows are -1."""
    parts = []
    for e, t in enumerate(tokens_per_expert):
        padded = -(-t // align) * align
        parts.append(np.full(t, e, dtype=np.int32))
        parts.append(np.full(padded - t, -1, dtype=np.int32))
    return np.concatenate(parts) if parts else np.zeros(0, np.int32)


# expert token counts of the grouped-GEMM walkthrough (4 experts) and of its
# 8-expert exercise
MOE_TOKENS_4 = [128, 96, 112, 144]
MOE_TOKENS_8 = [64, 128, 96, 112, 88, 144, 72, 104]
