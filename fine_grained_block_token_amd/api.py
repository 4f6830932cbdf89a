"""The library's calls in the form the pages write them: ``(fp8, scales)`` tuples and an
output tensor, plus the layout helpers they use.

"DeepGEMM Essentials: High-Performance FP8 Matrix Multiplication" calls the NT GEMM as
``gemm_fp8_fp8_bf16_nt((lhs_fp8, lhs_scales), (rhs_fp8, rhs_scales), out)`` (Parts 5-6),
the weight gradient as ``wgrad_gemm_fp8_fp8_fp32_nt`` (Parts 12-13) and the MoE GEMM as
``m_grouped_gemm_fp8_fp8_bf16_nt_contiguous`` (Parts 8-11), with the LHS scales passed
through ``get_col_major_tma_aligned_tensor`` (Part 5).  "deep-gemm: fused per-token FP8
cast in Triton" gives the cast's signature (``x, use_ue8m0, gran_k, use_packed_ue8m0,
out, out_sf``).  Every function here only allocates outputs when none are passed and
forwards to the entry points of the same package; the work runs in the library's
kernels.  There is no tensor-memory accelerator on MI355X: "TMA-aligned" here is the
GEMM's LHS scale layout, MN-major with a leading dimension rounded up to 4 rows.
"""
from __future__ import annotations

import torch

from . import (SF_FP32, SF_PACKED_UE8M0, SF_UE8M0, Fgfp8Error, cast_per_block, cast_per_token,
               gemm_fp8_nt_bf16, gemm_fp8_nt_bf16_ue8m0_g32, m_grouped_gemm_fp8_nt_bf16_contiguous,
               m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous, mn_major_scales, num_groups,
               wgrad_gemm_fp8_nt_fp32, wgrad_gemm_fp8_nt_fp32_ue8m0, wgrad_gemm_fp8_nt_fp32_ue8m0_g32)

_M_ALIGNMENT = 128


def get_m_alignment_for_contiguous_layout() -> int:
    """Rows per expert segment of the m-grouped contiguous layout (each segment is padded to
    a multiple of this, padding rows marked -1 in ``m_indices``)."""
    return _M_ALIGNMENT


def get_col_major_tma_aligned_tensor(sf: torch.Tensor) -> torch.Tensor:
    """Copy of 2-D scales ``sf`` [rows, groups] in the GEMM's LHS layout: MN-major (element
    (r, g) at g*ld + r), ld = rows rounded up to 4.  Returned as is when already laid out so."""
    if sf.dim() != 2:
        raise Fgfp8Error("scales must be a 2-D [rows, groups] tensor")
    rows, groups = sf.shape
    ld = -(-rows // 4) * 4
    if (rows == 1 or sf.stride(0) == 1) and sf.stride(1) == ld:
        return sf
    out = mn_major_scales(rows, groups, sf.dtype, sf.device)
    out.copy_(sf)
    return out


def _sf_fmt(use_ue8m0: bool, use_packed_ue8m0: bool) -> int:
    if use_packed_ue8m0:
        if not use_ue8m0:
            raise Fgfp8Error("use_packed_ue8m0 needs use_ue8m0")
        return SF_PACKED_UE8M0
    return SF_UE8M0 if use_ue8m0 else SF_FP32


def per_token_cast_to_fp8(x: torch.Tensor, use_ue8m0: bool = False, gran_k: int = 128,
                          use_packed_ue8m0: bool = False, out: torch.Tensor | None = None,
                          out_sf: torch.Tensor | None = None):
    """Per-token FP8 cast of bf16 or fp32 ``x`` [rows, cols] (any 2-D view) in 1 x ``gran_k``
    groups.  Returns ``(q, sf)``: q float8_e4m3fn [rows, cols]; sf [rows, G] float32 (fp32 or
    UE8M0 2^e scales, row-major) or, with ``use_packed_ue8m0``, int32 [rows, ceil(G/4)] in the
    MN-major layout.  ``out`` / ``out_sf`` may be views of larger buffers; they are written in
    place and returned."""
    if x.dim() != 2:
        raise Fgfp8Error("x must be 2-D")
    rows, cols = x.shape
    fmt = _sf_fmt(use_ue8m0, use_packed_ue8m0)
    g = num_groups(cols, gran_k)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float8_e4m3fn, device=x.device)
    if out_sf is None:
        if fmt == SF_PACKED_UE8M0:
            out_sf = mn_major_scales(rows, -(-g // 4), torch.int32, x.device)
        else:
            out_sf = torch.empty((rows, g), dtype=torch.float32, device=x.device)
    cast_per_token(x, out, out_sf, gran_k, fmt)
    return out, out_sf


fused_per_token_cast_to_fp8 = per_token_cast_to_fp8


def per_block_cast_to_fp8(x: torch.Tensor, use_ue8m0: bool = False):
    """128 x 128 block FP8 cast of row-major ``x`` [rows, cols].  Returns ``(q, sf)``: q
    float8_e4m3fn [rows, cols], sf float32 [ceil(rows/128), ceil(cols/128)] row-major."""
    if x.dim() != 2:
        raise Fgfp8Error("x must be 2-D")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.float8_e4m3fn, device=x.device)
    sf = torch.empty((-(-rows // 128), -(-cols // 128)), dtype=torch.float32, device=x.device)
    cast_per_block(x, q, sf, sf_fmt=SF_UE8M0 if use_ue8m0 else SF_FP32)
    return q, sf


def _lhs(lhs, what):
    a, sa = lhs
    if sa.shape[0] > 1 and sa.stride(0) != 1:
        raise Fgfp8Error(f"{what}: LHS scales must be MN-major; pass them through get_col_major_tma_aligned_tensor")
    return a, sa, (SF_PACKED_UE8M0 if sa.dtype == torch.int32 else SF_FP32)


def gemm_fp8_fp8_bf16_nt(lhs, rhs, out: torch.Tensor) -> None:
    """out [m, n] (bf16) = lhs @ rhs^T with lhs = (A [m, k] E4M3, per-token scales
    [m, k/128] float32 or [m, ceil(k/512)] int32 packed UE8M0, MN-major) and rhs = (B [n, k]
    E4M3, block scales [ceil(n/128), k/128] float32).  With int32 scales on the RHS too, both
    operands are taken as cast per 1 x 32 group with packed UE8M0 words ([m, k/128] and
    [n, k/128], MN-major) and the group-32 kernel runs."""
    a, sa, fmt = _lhs(lhs, "gemm_fp8_fp8_bf16_nt")
    b, sb = rhs
    if sb.dtype == torch.int32:
        if sa.dtype != torch.int32:
            raise Fgfp8Error("gemm_fp8_fp8_bf16_nt: packed RHS scales need packed LHS scales")
        gemm_fp8_nt_bf16_ue8m0_g32(a, sa, b, sb, out)
    else:
        gemm_fp8_nt_bf16(a, sa, b, sb, out, fmt)


def wgrad_gemm_fp8_fp8_fp32_nt(lhs, rhs, out: torch.Tensor, gran_k: int | None = None) -> None:
    """out [m, n] (fp32) += lhs @ rhs^T with both operands cast per token along K (the
    tokens): lhs = (A [m, k], scales), rhs = (B [n, k], scales), scales MN-major.

    float32 scales [m, k/128] / [n, k/128]: the fp32-scale weight gradient.  int32 packed
    UE8M0 words on both operands: 1 x 128 groups ([rows, ceil(k/512)] words, one exponent byte
    per 128-token block) or 1 x 32 groups ([rows, k/128] words, four bytes per block), told
    apart by their shape; with k = 128 the two shapes coincide and ``gran_k`` (128 or 32) must
    name the cast."""
    what = "wgrad_gemm_fp8_fp8_fp32_nt"
    a, sa, fmt = _lhs(lhs, what)
    b, sb = rhs
    if sb.shape[0] > 1 and sb.stride(0) != 1:
        raise Fgfp8Error(f"{what}: RHS scales must be MN-major; pass them through get_col_major_tma_aligned_tensor")
    if sa.dtype != sb.dtype or sa.dtype not in (torch.float32, torch.int32):
        raise Fgfp8Error(f"{what}: both operands take float32 scales, or both int32 packed UE8M0 words")
    if sa.dtype == torch.float32:
        wgrad_gemm_fp8_nt_fp32(a, sa, b, sb, out)
        return
    kb = a.shape[-1] // 128
    units = sa.shape[1] if sa.dim() == 2 else -1
    if gran_k is None:
        if kb == -(-kb // 4):
            raise Fgfp8Error(f"{what}: with k = 128 packed words of 1 x 128 and 1 x 32 groups look alike; "
                             "pass gran_k=128 or gran_k=32")
        gran_k = 32 if units == kb else 128
    if gran_k == 32:
        wgrad_gemm_fp8_nt_fp32_ue8m0_g32(a, sa, b, sb, out)
    elif gran_k == 128:
        wgrad_gemm_fp8_nt_fp32_ue8m0(a, sa, b, sb, out, SF_PACKED_UE8M0)
    else:
        raise Fgfp8Error(f"{what}: gran_k must be 128 or 32")


def m_grouped_gemm_fp8_fp8_bf16_nt_contiguous(lhs, rhs, out: torch.Tensor, m_indices: torch.Tensor) -> None:
    """MoE forward over token-contiguous expert segments: out[i] = lhs[i] @ rhs[e]^T with
    e = m_indices[i] (int32; -1 marks a padding row, which is left unwritten).  lhs as in
    gemm_fp8_fp8_bf16_nt; rhs = (B [E, n, k] E4M3, scales [E, ceil(n/128), k/128] float32).
    As in gemm_fp8_fp8_bf16_nt, int32 RHS scales select the group-32 recipe: packed words
    [E, n, k/128] with each expert's words MN-major (stride(1) == 1, e.g. a [E, k/128, n]
    buffer permuted), and packed group-32 LHS scales."""
    a, sa, fmt = _lhs(lhs, "m_grouped_gemm_fp8_fp8_bf16_nt_contiguous")
    b, sb = rhs
    if sb.dtype == torch.int32:
        if sa.dtype != torch.int32:
            raise Fgfp8Error("m_grouped_gemm_fp8_fp8_bf16_nt_contiguous: packed RHS scales need packed LHS scales")
        m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(a, sa, b, sb, m_indices, out)
    else:
        m_grouped_gemm_fp8_nt_bf16_contiguous(a, sa, b, sb, m_indices, out, fmt)
