"""Python binding of libfgfp8.so: fine-grained block-scaled FP8 cast and NT GEMM on MI355X.

Argument marshalling only.  Each function takes PyTorch tensors that already
live on the GPU, passes their pointers, sizes and strides to the C entry point
of the same name (``include/fgfp8.h``) on the current stream, and raises on a
non-zero return code.  Every step of the computation runs in the library's
HIP kernels; there is no fallback: if the library is missing, ``load()``
raises.

Scale layouts follow the C ABI: a scale tensor of logical shape
``[rows, groups]`` may be row-major or MN-major (``stride(0) == 1``), as
``mn_major_scales`` allocates it for the GEMM's LHS.
"""
from __future__ import annotations

import ctypes
import os

import torch

IN_BF16, IN_FP32 = 0, 1
SF_FP32, SF_UE8M0, SF_PACKED_UE8M0 = 0, 1, 2

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfgfp8.so")
_lib = None


class Fgfp8Error(RuntimeError):
    pass


def load():
    """Load libfgfp8.so (built in-tree by ``_build.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Fgfp8Error(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.cast_per_token.argtypes = [p, i32, i64, i64, i64, i64, i32, i32, p, i64, p, i64, i64, p]
    lib.cast_per_block.argtypes = [p, i32, i64, i64, i64, i32, p, i64, p, i64, p, i64, p, i64, p]
    lib.cast_per_token_dual.argtypes = [p, i32, i64, i64, i64, i32, i32, p, i64, p, i64, i64, p, i64, p, i64, i64, p]
    lib.gemm_fp8_nt_bf16.argtypes = [p, i64, p, i32, i64, p, i64, p, i64, p, i64, i64, i64, i64, p]
    lib.wgrad_gemm_fp8_nt_fp32.argtypes = [p, i64, p, i64, p, i64, p, i64, p, i64, i64, i64, i64, p]
    lib.gemm_fp8_nt_bf16_cast.argtypes = [p, i64, p, i32, i64, p, i64, p, i64, p, i64, i32, p, i64, p, i64, i64,
                                          i64, i64, i64, p]
    lib.gemm_fp8_nt_bf16_ue8m0_g32.argtypes = [p, i64, p, i64, p, i64, p, i64, p, i64, i64, i64, i64, p]
    lib.wgrad_gemm_fp8_nt_fp32_ue8m0_g32.argtypes = [p, i64, p, i64, p, i64, p, i64, p, i64, i64, i64, i64, p]
    lib.wgrad_gemm_fp8_nt_fp32_ue8m0.argtypes = [p, i64, p, i32, i64, p, i64, p, i64, p, i64, i64, i64, i64, p]
    lib.gemm_fp8_nt_bf16_ue8m0.argtypes = [p, i64, p, i32, i64, p, i64, p, i64, p, i64, i64, i64, i64, p]
    lib.m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous.argtypes = [p, i64, p, i64, p, i64, i64, p, i64, i64, p, i64,
                                                                    p, i64, i64, i64, i64, p]
    lib.m_grouped_gemm_fp8_nt_bf16_contiguous.argtypes = [p, i64, p, i32, i64, p, i64, i64, p, i64, i64, p, i64,
                                                          p, i64, i64, i64, i64, p]
    lib.gemm_fp8_nt_bf16_splitk.argtypes = [p, i64, p, i32, i64, p, i64, p, i64, p, i64, i64, i64, i64, p, i64, p]
    lib.gemm_fp8_nt_bf16_splitk_noalloc.argtypes = [p, i64, p, i32, i64, p, i64, p, i64, p, i64, i64, i64, i64, p]
    lib.gemm_fp8_nt_bf16_splitk_workspace.argtypes = [i64, i64, i64]
    lib.gemm_fp8_nt_bf16_splitk_workspace.restype = i64
    for f in ("cast_per_token", "cast_per_block", "cast_per_token_dual", "gemm_fp8_nt_bf16",
              "wgrad_gemm_fp8_nt_fp32", "m_grouped_gemm_fp8_nt_bf16_contiguous", "gemm_fp8_nt_bf16_cast",
              "gemm_fp8_nt_bf16_ue8m0_g32", "wgrad_gemm_fp8_nt_fp32_ue8m0_g32",
              "m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous", "wgrad_gemm_fp8_nt_fp32_ue8m0",
              "gemm_fp8_nt_bf16_ue8m0", "gemm_fp8_nt_bf16_splitk", "gemm_fp8_nt_bf16_splitk_noalloc"):
        getattr(lib, f).restype = i32
    lib.fgfp8_status_string.argtypes = [i32]
    lib.fgfp8_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


EXPORTED = ("cast_per_token", "cast_per_block", "cast_per_token_dual", "gemm_fp8_nt_bf16",
            "wgrad_gemm_fp8_nt_fp32", "m_grouped_gemm_fp8_nt_bf16_contiguous", "gemm_fp8_nt_bf16_cast",
            "gemm_fp8_nt_bf16_ue8m0_g32", "wgrad_gemm_fp8_nt_fp32_ue8m0_g32",
            "m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous", "wgrad_gemm_fp8_nt_fp32_ue8m0",
            "gemm_fp8_nt_bf16_ue8m0", "gemm_fp8_nt_bf16_splitk", "gemm_fp8_nt_bf16_splitk_workspace",
            "gemm_fp8_nt_bf16_splitk_noalloc", "fgfp8_status_string")


def _check(rc: int, what: str):
    if rc != 0:
        msg = load().fgfp8_status_string(rc).decode()
        raise Fgfp8Error(f"{what}: {msg} (status {rc})")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return IN_BF16
    if x.dtype == torch.float32:
        return IN_FP32
    raise TypeError("input must be bfloat16 or float32")


def _u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


# ---------------------------------------------------------------------------
# allocation helpers (device memory only; no computation)
# ---------------------------------------------------------------------------

def mn_major_scales(rows: int, groups: int, dtype=torch.float32, device="cuda", align: int = 4):
    """[rows, groups] tensor in MN-major layout: element (r, g) at g*ld + r, ld = align(rows, 4)."""
    ld = -(-rows // align) * align
    return torch.empty(groups, ld, dtype=dtype, device=device).t()[:rows]


def num_groups(cols: int, gran_k: int) -> int:
    return -(-cols // gran_k)


# ---------------------------------------------------------------------------
# marshalling checks
# ---------------------------------------------------------------------------
# The C ABI sees pointers, sizes and strides only, so it cannot tell a scale tensor of
# the wrong shape from a right one.  Each wrapper first checks that every tensor is a
# CUDA tensor of exactly the logical shape and dtype the entry point addresses, so no
# kernel reads or writes outside the tensors it is given.  Layouts (row-major or
# MN-major strides) are checked by the entry points themselves.

_FP8 = (torch.uint8, torch.float8_e4m3fn)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _req(t, name: str, shape, dtypes, row_major: bool = False, mn_major: bool = False) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA tensor")
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(int(d) for d in shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if row_major and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    if mn_major and t.shape[0] > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be MN-major (stride(0) == 1)")


def _sf_spec(fmt: int, groups: int):
    """(units, dtypes) of a per-token scale tensor with `groups` groups per row."""
    if fmt == SF_PACKED_UE8M0:
        return -(-groups // 4), _I32
    return groups, _F32


def _gemm_operands(A, B, what: str, b_dims: int = 2):
    """A [m, k] and B [n, k] (or [E, n, k]) E4M3, row-major; returns (A, B, m, n, k)."""
    A, B = _u8(A), _u8(B)
    if A.dim() != 2 or B.dim() != b_dims:
        raise ValueError(f"{what}: A must be 2-D and B {b_dims}-D")
    m, k = A.shape
    n = B.shape[-2]
    _req(A, f"{what}: A", (m, k), _FP8, row_major=True)
    _req(B, f"{what}: B", tuple(B.shape[:-1]) + (k,), _FP8, row_major=True)
    return A, B, m, n, k


def _kb(k: int, what: str) -> int:
    if k <= 0 or k % 128 != 0:
        raise ValueError(f"{what}: k = {k} must be a positive multiple of 128")
    return k // 128


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def cast_per_token(x: torch.Tensor, q: torch.Tensor, sf: torch.Tensor, gran_k: int = 128,
                   sf_fmt: int = SF_FP32) -> None:
    """Per-token FP8 cast of a 2-D view ``x`` [rows, cols] (row-major or transposed) into
    ``q`` (uint8 or float8_e4m3fn view [rows, cols]) and ``sf`` ([rows, G] float32, or
    [rows, ceil(G/4)] int32 for packed UE8M0; row-major or MN-major view)."""
    q = _u8(q)
    rows, cols = x.shape
    _req(x, "cast_per_token: x", (rows, cols), (torch.bfloat16, torch.float32))
    _req(q, "cast_per_token: q", (rows, cols), _FP8, row_major=True)
    if gran_k in (32, 128) and sf_fmt in (SF_FP32, SF_UE8M0, SF_PACKED_UE8M0):
        units, sdt = _sf_spec(sf_fmt, num_groups(cols, gran_k))
        _req(sf, "cast_per_token: sf", (rows, units), sdt)
    _check(load().cast_per_token(_ptr(x), _x_dtype(x), rows, cols, x.stride(0), x.stride(1), gran_k, sf_fmt,
                                 _ptr(q), q.stride(0), _ptr(sf), sf.stride(0), sf.stride(1), _stream(x)),
           "cast_per_token")


def cast_per_block(x: torch.Tensor, q: torch.Tensor, sf: torch.Tensor, qT: torch.Tensor | None = None,
                   sfT: torch.Tensor | None = None, sf_fmt: int = SF_FP32) -> None:
    """128x128 block FP8 cast of row-major ``x`` [rows, cols] into ``q`` and ``sf``
    [ceil(rows/128), ceil(cols/128)]; optionally also ``qT`` = q^T and ``sfT`` = sf^T."""
    q = _u8(q)
    qT = None if qT is None else _u8(qT)
    rows, cols = x.shape
    rb, cb = -(-rows // 128), -(-cols // 128)
    _req(x, "cast_per_block: x", (rows, cols), (torch.bfloat16, torch.float32), row_major=True)
    _req(q, "cast_per_block: q", (rows, cols), _FP8, row_major=True)
    _req(sf, "cast_per_block: sf", (rb, cb), _F32, row_major=True)
    if (qT is None) != (sfT is None):
        raise ValueError("cast_per_block: qT and sfT go together")
    if qT is not None:
        _req(qT, "cast_per_block: qT", (cols, rows), _FP8, row_major=True)
        _req(sfT, "cast_per_block: sfT", (cb, rb), _F32, row_major=True)
    _check(load().cast_per_block(_ptr(x), _x_dtype(x), rows, cols, x.stride(0), sf_fmt, _ptr(q), q.stride(0),
                                 _ptr(sf), sf.stride(0), _ptr(qT), 0 if qT is None else qT.stride(0),
                                 _ptr(sfT), 0 if sfT is None else sfT.stride(0), _stream(x)),
           "cast_per_block")


def cast_per_token_dual(x: torch.Tensor, q: torch.Tensor, sf: torch.Tensor, qT: torch.Tensor,
                        sfT: torch.Tensor, sf_fmt: int = SF_FP32, gran_k: int = 128) -> None:
    """Both 1 x gran_k per-token casts of row-major bf16 or fp32 ``x`` [rows, cols] from one read:
    ``q``/``sf`` as cast_per_token(x, gran_k, sf_fmt) and ``qT`` [cols, rows] / ``sfT`` as
    cast_per_token(x.t(), gran_k, sf_fmt) (float scales, or int32 packed-UE8M0 words)."""
    q, qT = _u8(q), _u8(qT)
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must be row-major")
    _req(x, "cast_per_token_dual: x", (rows, cols), (torch.bfloat16, torch.float32))
    _req(q, "cast_per_token_dual: q", (rows, cols), _FP8, row_major=True)
    _req(qT, "cast_per_token_dual: qT", (cols, rows), _FP8, row_major=True)
    if gran_k in (32, 128) and sf_fmt in (SF_FP32, SF_UE8M0, SF_PACKED_UE8M0):
        units, sdt = _sf_spec(sf_fmt, num_groups(cols, gran_k))
        unitsT, _ = _sf_spec(sf_fmt, num_groups(rows, gran_k))
        _req(sf, "cast_per_token_dual: sf", (rows, units), sdt)
        _req(sfT, "cast_per_token_dual: sfT", (cols, unitsT), sdt)
    _check(load().cast_per_token_dual(_ptr(x), _x_dtype(x), rows, cols, x.stride(0), gran_k, sf_fmt, _ptr(q),
                                      q.stride(0),
                                      _ptr(sf), sf.stride(0), sf.stride(1), _ptr(qT), qT.stride(0),
                                      _ptr(sfT), sfT.stride(0), sfT.stride(1), _stream(x)),
           "cast_per_token_dual")


def _bf16_gemm_checks(what: str, A, sa, B, sb, D, sa_fmt: int):
    """Operands of the fp32/UE8M0-scale bf16 GEMMs: sa [m, k/128] float32 or [m, ceil(k/512)]
    int32 (packed), MN-major; sb [ceil(n/128), k/128] float32 block scales; D [m, n] bf16."""
    A, B, m, n, k = _gemm_operands(A, B, what)
    kb = _kb(k, what)
    if sa_fmt in (SF_FP32, SF_UE8M0, SF_PACKED_UE8M0):
        units, sdt = _sf_spec(sa_fmt, kb)
        _req(sa, f"{what}: sa", (m, units), sdt, mn_major=True)
    _req(sb, f"{what}: sb", (-(-n // 128), kb), _F32, row_major=True)
    if D is not None:
        _req(D, f"{what}: D", (m, n), (torch.bfloat16,), row_major=True)
    return A, B, m, n, k


def gemm_fp8_nt_bf16(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor,
                     sa_fmt: int = SF_FP32) -> None:
    """D[m, n] (bf16) = (A*sa)(B*sb)^T.  sa: MN-major view [m, k/128] (float32) or
    [m, ceil(k/512)] (int32, packed UE8M0); sb: [ceil(n/128), k/128] float32."""
    A, B, m, n, k = _bf16_gemm_checks("gemm_fp8_nt_bf16", A, sa, B, sb, D, sa_fmt)
    _check(load().gemm_fp8_nt_bf16(_ptr(A), A.stride(0), _ptr(sa), sa_fmt, sa.stride(1), _ptr(B), B.stride(0),
                                   _ptr(sb), sb.stride(0), _ptr(D), D.stride(0), m, n, k, _stream(A)),
           "gemm_fp8_nt_bf16")


def gemm_fp8_nt_bf16_splitk_workspace(m: int, n: int, k: int) -> int:
    """Bytes of workspace gemm_fp8_nt_bf16_splitk needs for an [m, k] x [n, k]^T product (0: none)."""
    r = load().gemm_fp8_nt_bf16_splitk_workspace(m, n, k)
    if r < 0:
        raise Fgfp8Error(f"gemm_fp8_nt_bf16_splitk_workspace: {load().fgfp8_status_string(int(r)).decode()}")
    return int(r)


def gemm_fp8_nt_bf16_splitk(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor,
                            workspace: torch.Tensor, sa_fmt: int = SF_FP32) -> None:
    """gemm_fp8_nt_bf16 with K split over workgroups (stream-K shares for m <= 64, K slices of
    128x128 tiles above); ``workspace`` is a contiguous device tensor of at least
    gemm_fp8_nt_bf16_splitk_workspace(m, n, k) bytes (any dtype, contents ignored)."""
    A, B, m, n, k = _bf16_gemm_checks("gemm_fp8_nt_bf16_splitk", A, sa, B, sb, D, sa_fmt)
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("gemm_fp8_nt_bf16_splitk: workspace must be a contiguous CUDA tensor")
    _check(load().gemm_fp8_nt_bf16_splitk(_ptr(A), A.stride(0), _ptr(sa), sa_fmt, sa.stride(1), _ptr(B), B.stride(0),
                                          _ptr(sb), sb.stride(0), _ptr(D), D.stride(0), m, n, k, _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(A)),
           "gemm_fp8_nt_bf16_splitk")


def gemm_fp8_nt_bf16_splitk_noalloc(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor,
                                    D: torch.Tensor, sa_fmt: int = SF_FP32) -> None:
    """gemm_fp8_nt_bf16_splitk with the library's static 32 MiB device scratch in place of a workspace
    (allocates nothing; calls that overlap on one GPU race)."""
    A, B, m, n, k = _bf16_gemm_checks("gemm_fp8_nt_bf16_splitk_noalloc", A, sa, B, sb, D, sa_fmt)
    _check(load().gemm_fp8_nt_bf16_splitk_noalloc(_ptr(A), A.stride(0), _ptr(sa), sa_fmt, sa.stride(1), _ptr(B),
                                                  B.stride(0), _ptr(sb), sb.stride(0), _ptr(D), D.stride(0), m, n, k,
                                                  _stream(A)),
           "gemm_fp8_nt_bf16_splitk_noalloc")


def gemm_fp8_nt_bf16_cast(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor,
                          D: torch.Tensor | None, q: torch.Tensor, q_sf: torch.Tensor, sa_fmt: int = SF_FP32,
                          q_sf_fmt: int = SF_FP32) -> None:
    """gemm_fp8_nt_bf16 whose epilogue also emits the 1x128 per-token FP8 cast of the bf16 output:
    ``q`` [m, n] E4M3 and ``q_sf`` [m, ceil(n/128)] float32 (row-major or MN-major view).  ``D`` may
    be None to store only the FP8 output."""
    A, B, m, n, k = _bf16_gemm_checks("gemm_fp8_nt_bf16_cast", A, sa, B, sb, D, sa_fmt)
    q = _u8(q)
    _req(q, "gemm_fp8_nt_bf16_cast: q", (m, n), _FP8, row_major=True)
    _req(q_sf, "gemm_fp8_nt_bf16_cast: q_sf", (m, -(-n // 128)), _F32)
    _check(load().gemm_fp8_nt_bf16_cast(_ptr(A), A.stride(0), _ptr(sa), sa_fmt, sa.stride(1), _ptr(B), B.stride(0),
                                        _ptr(sb), sb.stride(0), _ptr(D), 0 if D is None else D.stride(0), q_sf_fmt,
                                        _ptr(q), q.stride(0), _ptr(q_sf), q_sf.stride(0), q_sf.stride(1), m, n, k,
                                        _stream(A)),
           "gemm_fp8_nt_bf16_cast")


def gemm_fp8_nt_bf16_ue8m0_g32(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor,
                               D: torch.Tensor) -> None:
    """D[m, n] (bf16) = (A*sa)(B*sb)^T with one power-of-two scale per row and 32-wide K group on both
    operands: sa [m, k/128] and sb [n, k/128] int32 packed-UE8M0 words in MN-major views (what
    cast_per_token(gran_k=32, SF_PACKED_UE8M0) writes into mn_major_scales(..., torch.int32))."""
    what = "gemm_fp8_nt_bf16_ue8m0_g32"
    A, B, m, n, k = _gemm_operands(A, B, what)
    kb = _kb(k, what)
    _req(sa, f"{what}: sa", (m, kb), _I32, mn_major=True)
    _req(sb, f"{what}: sb", (n, kb), _I32, mn_major=True)
    _req(D, f"{what}: D", (m, n), (torch.bfloat16,), row_major=True)
    _check(load().gemm_fp8_nt_bf16_ue8m0_g32(_ptr(A), A.stride(0), _ptr(sa), sa.stride(1), _ptr(B), B.stride(0),
                                             _ptr(sb), sb.stride(1), _ptr(D), D.stride(0), m, n, k, _stream(A)),
           what)


def gemm_fp8_nt_bf16_ue8m0(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor, D: torch.Tensor,
                           sa_fmt: int = SF_UE8M0) -> None:
    """gemm_fp8_nt_bf16 with power-of-two scales throughout, applied by the scaled MFMA (no
    promotion): sa [m, k/128] float32 2^e (SF_UE8M0) or [m, ceil(k/512)] int32 packed words,
    MN-major; sb [ceil(n/128), k/128] float32 2^e block scales."""
    A, B, m, n, k = _bf16_gemm_checks("gemm_fp8_nt_bf16_ue8m0", A, sa, B, sb, D, sa_fmt)
    _check(load().gemm_fp8_nt_bf16_ue8m0(_ptr(A), A.stride(0), _ptr(sa), sa_fmt, sa.stride(1), _ptr(B), B.stride(0),
                                         _ptr(sb), sb.stride(0), _ptr(D), D.stride(0), m, n, k, _stream(A)),
           "gemm_fp8_nt_bf16_ue8m0")


def _wgrad_checks(what: str, A, sa, B, sb, D, units: int, sdt):
    A, B, m, n, k = _gemm_operands(A, B, what)
    _kb(k, what)
    _req(sa, f"{what}: sa", (m, units), sdt, mn_major=True)
    _req(sb, f"{what}: sb", (n, units), sdt, mn_major=True)
    _req(D, f"{what}: D", (m, n), _F32, row_major=True)
    return A, B, m, n, k


def wgrad_gemm_fp8_nt_fp32_ue8m0(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor,
                                 D: torch.Tensor, sf_fmt: int = SF_UE8M0) -> None:
    """wgrad_gemm_fp8_nt_fp32 for power-of-two 1x128 scales on both operands, applied by the
    scaled MFMA (no promotion): sa [m, k/128] / sb [n, k/128] float32 2^e values (SF_UE8M0) or
    [m, ceil(k/512)] / [n, ceil(k/512)] int32 packed words (SF_PACKED_UE8M0), MN-major views."""
    what = "wgrad_gemm_fp8_nt_fp32_ue8m0"
    k = _u8(A).shape[-1]
    units, sdt = _sf_spec(sf_fmt, _kb(k, what))
    A, B, m, n, k = _wgrad_checks(what, A, sa, B, sb, D, units, sdt)
    _check(load().wgrad_gemm_fp8_nt_fp32_ue8m0(_ptr(A), A.stride(0), _ptr(sa), sf_fmt, sa.stride(1), _ptr(B),
                                               B.stride(0), _ptr(sb), sb.stride(1), _ptr(D), D.stride(0), m, n, k,
                                               _stream(A)),
           what)


def wgrad_gemm_fp8_nt_fp32_ue8m0_g32(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor,
                                     D: torch.Tensor) -> None:
    """D[m, n] (fp32) += (A*sa)(B*sb)^T, K over tokens, with the UE8M0 group-32 scales of
    gemm_fp8_nt_bf16_ue8m0_g32 on both operands (packed words in MN-major views)."""
    what = "wgrad_gemm_fp8_nt_fp32_ue8m0_g32"
    k = _u8(A).shape[-1]
    A, B, m, n, k = _wgrad_checks(what, A, sa, B, sb, D, _kb(k, what), _I32)
    _check(load().wgrad_gemm_fp8_nt_fp32_ue8m0_g32(_ptr(A), A.stride(0), _ptr(sa), sa.stride(1), _ptr(B),
                                                   B.stride(0), _ptr(sb), sb.stride(1), _ptr(D), D.stride(0), m, n, k,
                                                   _stream(A)),
           what)


def _m_indices(m_indices, m: int, what: str):
    if not isinstance(m_indices, torch.Tensor) or m_indices.dtype != torch.int32 or m_indices.numel() != m \
            or m_indices.device.type != "cuda" or not m_indices.is_contiguous():
        raise ValueError(f"{what}: m_indices must be a contiguous int32 CUDA tensor of {m} elements")


def m_grouped_gemm_fp8_nt_bf16_contiguous(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor,
                                          m_indices: torch.Tensor, D: torch.Tensor, sa_fmt: int = SF_FP32) -> None:
    """MoE forward over a token-contiguous LHS: row i of D (bf16 [m, n]) = (A[i]*sa[i]) (B[e]*sb[e])^T with
    e = m_indices[i] (int32, -1 = padding row, not written).  B: [E, n, k] E4M3; sb: [E, ceil(n/128), k/128]
    float32; A, sa as gemm_fp8_nt_bf16."""
    what = "m_grouped_gemm_fp8_nt_bf16_contiguous"
    A, B, m, n, k = _gemm_operands(A, B, what, b_dims=3)
    kb = _kb(k, what)
    E = B.shape[0]
    if sa_fmt in (SF_FP32, SF_UE8M0, SF_PACKED_UE8M0):
        units, sdt = _sf_spec(sa_fmt, kb)
        _req(sa, f"{what}: sa", (m, units), sdt, mn_major=True)
    _req(sb, f"{what}: sb", (E, -(-n // 128), kb), _F32, row_major=True)
    _req(D, f"{what}: D", (m, n), (torch.bfloat16,), row_major=True)
    _m_indices(m_indices, m, what)
    _check(load().m_grouped_gemm_fp8_nt_bf16_contiguous(
        _ptr(A), A.stride(0), _ptr(sa), sa_fmt, sa.stride(1), _ptr(B), B.stride(1), B.stride(0), _ptr(sb),
        sb.stride(1), sb.stride(0), _ptr(m_indices), E, _ptr(D), D.stride(0), m, n, k, _stream(A)),
        what)


def m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor,
                                                    sb: torch.Tensor, m_indices: torch.Tensor,
                                                    D: torch.Tensor) -> None:
    """m-grouped contiguous GEMM in the UE8M0 group-32 recipe: row i of D (bf16 [m, n]) =
    (A[i]*sa[i]) (B[e]*sb[e])^T, e = m_indices[i] (int32, -1 = padding row, not written).
    A, sa as gemm_fp8_nt_bf16_ue8m0_g32; B [E, n, k] E4M3; sb [E, n, k/128] int32 packed words with
    stride(1) == 1: expert e's word (j, kb) at sb[e] offset kb*stride(2) + j."""
    what = "m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous"
    A, B, m, n, k = _gemm_operands(A, B, what, b_dims=3)
    kb = _kb(k, what)
    E = B.shape[0]
    _req(sa, f"{what}: sa", (m, kb), _I32, mn_major=True)
    _req(sb, f"{what}: sb", (E, n, kb), _I32)
    if sb.shape[1] > 1 and sb.stride(1) != 1:
        raise ValueError("sb must be [E, n, k/128] with each expert's words MN-major (stride(1) == 1)")
    _req(D, f"{what}: D", (m, n), (torch.bfloat16,), row_major=True)
    _m_indices(m_indices, m, what)
    _check(load().m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(
        _ptr(A), A.stride(0), _ptr(sa), sa.stride(1), _ptr(B), B.stride(1), B.stride(0), _ptr(sb), sb.stride(2),
        sb.stride(0), _ptr(m_indices), E, _ptr(D), D.stride(0), m, n, k, _stream(A)),
        what)


def wgrad_gemm_fp8_nt_fp32(A: torch.Tensor, sa: torch.Tensor, B: torch.Tensor, sb: torch.Tensor,
                           D: torch.Tensor) -> None:
    """D[m, n] (float32) += (A*sa)(B*sb)^T with MN-major views sa [m, k/128], sb [n, k/128]."""
    what = "wgrad_gemm_fp8_nt_fp32"
    k = _u8(A).shape[-1]
    A, B, m, n, k = _wgrad_checks(what, A, sa, B, sb, D, _kb(k, what), _F32)
    _check(load().wgrad_gemm_fp8_nt_fp32(_ptr(A), A.stride(0), _ptr(sa), sa.stride(1), _ptr(B), B.stride(0),
                                         _ptr(sb), sb.stride(1), _ptr(D), D.stride(0), m, n, k, _stream(A)),
           what)
