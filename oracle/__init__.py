"""CPU oracle for the fine-grained block-scaled FP8 path (test infrastructure).

This package is NOT part of the product.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It wraps ``fgfp8_oracle.c`` (plain C, fp64 GEMM) with ctypes and numpy and
shares no code with the HIP library in ``fine_grained_block_token_amd``.

Every function follows a passage of the pages it cites:

* per-token cast -- "DeepGEMM Essentials: High-Performance FP8 Matrix
  Multiplication", Part 3, with the format and group options of
  "deep-gemm: fused per-token FP8 cast in Triton";
* per-block cast -- "DeepGEMM Essentials", Part 4;
* NT GEMM -- "DeepGEMM Essentials", Parts 1 and 6, and the scale-row reply in
  "[Help] Starter script for nn.Linear for fwd,bwd";
* wgrad -- "DeepGEMM Essentials", Parts 12-13 (accumulates into fp32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fgfp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfgfp8_oracle.so")

IN_BF16, IN_FP32 = 0, 1
SF_FP32, SF_UE8M0, SF_PACKED_UE8M0 = 0, 1, 2

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.orc_cast_per_token.argtypes = [p, i32, i64, i64, i64, i64, i32, i32, p, i64, p, i64, i64]
    lib.orc_cast_per_token.restype = i32
    lib.orc_cast_per_block.argtypes = [p, i32, i64, i64, i64, i32, p, i64, p, i64]
    lib.orc_cast_per_block.restype = i32
    lib.orc_gemm_nt.argtypes = [p, i64, p, i64, i64, p, i64, p, i64, i64, i32, i64, i64, i64,
                                p, p, i64, p, p]
    lib.orc_gemm_nt.restype = i32
    lib.orc_e4m3_round_array.argtypes = [p, i64, p]
    lib.orc_e4m3_value_array.argtypes = [p, i64, p]
    lib.orc_round_bf16_array.argtypes = [p, i64, p]
    lib.orc_set_threads.argtypes = [i32]
    lib.orc_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    return int(_load().orc_max_threads())


# --------------------------------------------------------------------------
# element-wise helpers
# --------------------------------------------------------------------------

def e4m3_round(v) -> np.ndarray:
    """fp32 values -> E4M3 codes (nearest, ties to even, NaN above 448)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().orc_e4m3_round_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_value(codes) -> np.ndarray:
    """E4M3 codes -> exact fp64 values."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_value_array(_ptr(c), c.size, _ptr(out))
    return out


def round_bf16(v) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), rounded once, ties to even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_round_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_bits_to_f32(h) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact widening)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# casts
# --------------------------------------------------------------------------

def _x_dtype(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return IN_BF16
    if x.dtype == np.float32:
        return IN_FP32
    raise TypeError("x must hold bf16 bits (uint16) or float32")


def cast_per_token(x: np.ndarray, gran: int = 128, sf_fmt: int = SF_FP32,
                   transpose: bool = False):
    """Per-token cast of a 2-D array (bf16 bits as uint16, or float32).

    With ``transpose=True`` the cast runs over ``x.T`` (groups along the
    original rows), reading ``x`` through strides, as the wgrad operands are.
    Returns ``(q, sf)``: q uint8 [rows, cols]; sf float32 [rows, G] for fp32 /
    UE8M0 scales, or uint32 [rows, ceil(G/4)] packed words.
    """
    x = np.ascontiguousarray(x)
    dt = _x_dtype(x)
    if transpose:
        rows, cols = x.shape[1], x.shape[0]
        xs_row, xs_col = 1, x.shape[1]
    else:
        rows, cols = x.shape
        xs_row, xs_col = x.shape[1], 1
    groups = -(-cols // gran)
    q = np.empty((rows, cols), dtype=np.uint8)
    if sf_fmt == SF_PACKED_UE8M0:
        sf = np.empty((rows, -(-groups // 4)), dtype=np.uint32)
    else:
        sf = np.empty((rows, groups), dtype=np.float32)
    rc = _load().orc_cast_per_token(_ptr(x), dt, rows, cols, xs_row, xs_col, gran, sf_fmt,
                                    _ptr(q), cols, _ptr(sf), sf.shape[1], 1)
    if rc != 0:
        raise ValueError("oracle cast_per_token rejected its arguments")
    return q, sf


def cast_per_block(x: np.ndarray, sf_fmt: int = SF_FP32):
    """128 x 128 block cast of a row-major 2-D array.  Returns (q, sf [ceil(r/128), ceil(c/128)])."""
    x = np.ascontiguousarray(x)
    dt = _x_dtype(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    sf = np.empty((-(-rows // 128), -(-cols // 128)), dtype=np.float32)
    rc = _load().orc_cast_per_block(_ptr(x), dt, rows, cols, cols, sf_fmt, _ptr(q), cols,
                                    _ptr(sf), sf.shape[1])
    if rc != 0:
        raise ValueError("oracle cast_per_block rejected its arguments")
    return q, sf


def unpack_ue8m0(words: np.ndarray, groups: int) -> np.ndarray:
    """Packed UE8M0 words [rows, ceil(G/4)] -> fp32 scales 2^(byte-127) [rows, G]."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    b = w.view(np.uint8).reshape(w.shape[0], -1)[:, :groups]     # little-endian bytes
    return np.ldexp(np.float32(1.0), b.astype(np.int32) - 127).astype(np.float32)


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

def gemm_nt(A: np.ndarray, sa: np.ndarray, B: np.ndarray, sb: np.ndarray,
            sb_block: bool = True, idx=None):
    """fp64 reference of the block-scaled NT GEMM.

    A uint8 E4M3 [m, k]; sa float32 [m, k/128] (one scale per row and K block);
    B uint8 E4M3 [n, k]; sb float32 [ceil(n/128), k/128] when ``sb_block`` (one
    scale per 128x128 block) else [n, k/128] (one per row and K block).
    ``idx`` = (i_array, j_array) computes only those outputs.
    Returns (ref, absum): fp64 arrays [m, n] (or [len(idx)]).
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    m, k = A.shape
    n = B.shape[0]
    if B.shape[1] != k or k % 128:
        raise ValueError("bad GEMM shapes")
    kb = k // 128
    if sa.shape != (m, kb):
        raise ValueError("sa must be [m, k/128]")
    if sb_block and sb.shape != (-(-n // 128), kb):
        raise ValueError("sb must be [ceil(n/128), k/128]")
    if not sb_block and sb.shape != (n, kb):
        raise ValueError("sb must be [n, k/128]")
    if idx is None:
        ii = jj = None
        count = m * n
        shape = (m, n)
    else:
        ii = np.ascontiguousarray(idx[0], dtype=np.int64)
        jj = np.ascontiguousarray(idx[1], dtype=np.int64)
        count = ii.size
        shape = (count,)
    ref = np.empty(shape, dtype=np.float64)
    absum = np.empty(shape, dtype=np.float64)
    rc = _load().orc_gemm_nt(_ptr(A), k, _ptr(sa), kb, 1, _ptr(B), k, _ptr(sb), kb, 1,
                             128 if sb_block else 1, m, n, k, _ptr(ii), _ptr(jj), count,
                             _ptr(ref), _ptr(absum))
    if rc != 0:
        raise ValueError("oracle gemm rejected its arguments")
    return ref, absum


def wgrad_nt(A, sa, B, sb, d_in, idx=None):
    """wgrad reference: D_in + A.B^T with per-row 1x128 scales on both operands."""
    ref, absum = gemm_nt(A, sa, B, sb, sb_block=False, idx=idx)
    d = np.asarray(d_in, dtype=np.float64)
    if idx is not None:
        d = d[idx[0], idx[1]]
    return d + ref, absum + np.abs(d)


def m_grouped_gemm_nt(A, sa, B, sb, m_indices, idx=None):
    """fp64 reference of the m-grouped contiguous GEMM ("DeepGEMM Essentials",
    Parts 8-11): row i of A uses expert e = m_indices[i] and gives
    D[i] = (A[i] * sa[i]) (B[e] * sb[e])^T; rows with m_indices[i] == -1 are
    padding and have no reference (NaN).

    A uint8 [m, k]; sa float32 [m, k/128]; B uint8 [E, n, k]; sb float32
    [E, ceil(n/128), k/128]; m_indices int [m].  ``idx`` = (i_array, j_array)
    computes only those outputs.  Returns (ref, absum) like gemm_nt.
    """
    A = np.asarray(A)
    B = np.asarray(B)
    sb = np.asarray(sb)
    e_of = np.asarray(m_indices, dtype=np.int64)
    m, n = A.shape[0], B.shape[1]
    if idx is None:
        ref = np.full((m, n), np.nan)
        absum = np.full((m, n), np.nan)
        for e in range(B.shape[0]):
            rows = np.nonzero(e_of == e)[0]
            if rows.size:
                r, s = gemm_nt(A[rows], sa[rows], B[e], sb[e])
                ref[rows], absum[rows] = r, s
        return ref, absum
    ii = np.asarray(idx[0], dtype=np.int64)
    jj = np.asarray(idx[1], dtype=np.int64)
    ref = np.full(ii.size, np.nan)
    absum = np.full(ii.size, np.nan)
    for e in range(B.shape[0]):
        sel = np.nonzero(e_of[ii] == e)[0]
        if sel.size:
            r, s = gemm_nt(A, sa, B[e], sb[e], idx=(ii[sel], jj[sel]))
            ref[sel], absum[sel] = r, s
    return ref, absum


def gemm_nt_g32(A, sa, B, sb, idx=None):
    """fp64 reference of the NT GEMM with one scale per row and 32-wide K group on both
    operands (the UE8M0 group-32 recipe named in "deep-gemm: fused per-token FP8 cast
    in Triton"): D[i, j] = sum_g sa[i, g] sb[j, g] sum_{t in g} A[i, t] B[j, t].

    A uint8 E4M3 [m, k]; sa float32 [m, k/32]; B uint8 E4M3 [n, k]; sb float32
    [n, k/32] (the scales as values, e.g. unpack_ue8m0 of the packed words).  The
    dequantised operands are exact in fp64 (E4M3 values times powers of two); the sum
    uses a library fp64 matrix product.  ``idx`` = (i_array, j_array) computes only
    those outputs.  Returns (ref, absum) like gemm_nt.
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    m, k = A.shape
    n = B.shape[0]
    if B.shape[1] != k or k % 32 or np.shape(sa) != (m, k // 32) or np.shape(sb) != (n, k // 32):
        raise ValueError("bad group-32 GEMM shapes")
    a = e4m3_value(A).astype(np.float64) * np.repeat(np.asarray(sa, np.float64), 32, axis=1)
    b = e4m3_value(B).astype(np.float64) * np.repeat(np.asarray(sb, np.float64), 32, axis=1)
    if idx is None:
        return a @ b.T, np.abs(a) @ np.abs(b).T
    ii = np.asarray(idx[0], dtype=np.int64)
    jj = np.asarray(idx[1], dtype=np.int64)
    return np.einsum("ij,ij->i", a[ii], b[jj]), np.einsum("ij,ij->i", np.abs(a[ii]), np.abs(b[jj]))


def m_grouped_gemm_nt_g32(A, sa, B, sb, m_indices, idx=None):
    """fp64 reference of the m-grouped contiguous GEMM ("DeepGEMM Essentials",
    Parts 8-11) in the group-32 recipe: row i uses expert e = m_indices[i] and
    gives D[i] = gemm_nt_g32 of (A[i], sa[i]) with (B[e], sb[e]); padding rows
    (m_indices[i] == -1) have no reference (NaN).

    A uint8 [m, k]; sa float32 [m, k/32]; B uint8 [E, n, k]; sb float32
    [E, n, k/32]; m_indices int [m].  Returns (ref, absum) like gemm_nt.
    """
    B = np.asarray(B)
    sb = np.asarray(sb)
    e_of = np.asarray(m_indices, dtype=np.int64)
    m, n = np.shape(A)[0], B.shape[1]
    if idx is None:
        ref = np.full((m, n), np.nan)
        absum = np.full((m, n), np.nan)
        for e in range(B.shape[0]):
            rows = np.nonzero(e_of == e)[0]
            if rows.size:
                ref[rows], absum[rows] = gemm_nt_g32(np.asarray(A)[rows], np.asarray(sa)[rows], B[e], sb[e])
        return ref, absum
    ii = np.asarray(idx[0], dtype=np.int64)
    jj = np.asarray(idx[1], dtype=np.int64)
    ref = np.full(ii.size, np.nan)
    absum = np.full(ii.size, np.nan)
    for e in range(B.shape[0]):
        sel = np.nonzero(e_of[ii] == e)[0]
        if sel.size:
            ref[sel], absum[sel] = gemm_nt_g32(A, sa, B[e], sb[e], idx=(ii[sel], jj[sel]))
    return ref, absum


def wgrad_nt_g32(A, sa, B, sb, d_in, idx=None):
    """Weight-gradient form of gemm_nt_g32 ("DeepGEMM Essentials", Parts 12-13: K
    runs over tokens and the fp32 output is accumulated): D_in + gemm_nt_g32.
    Returns (ref, absum) with |D_in| included in absum."""
    ref, absum = gemm_nt_g32(A, sa, B, sb, idx=idx)
    d = np.asarray(d_in, dtype=np.float64)
    if idx is not None:
        d = d[idx[0], idx[1]]
    return d + ref, absum + np.abs(d)
