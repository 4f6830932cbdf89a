"""The allocation-free split-K decode GEMM (gemm_fp8_nt_bf16_splitk_noalloc),
called through the C ABI, against the workspace entry point
gemm_fp8_nt_bf16_splitk on the same operands: the same kernels in the same
order, so the bf16 outputs must be bit-identical.  Two problems in a row, the
second smaller, so the second call runs on the static scratch as the first left
it; each result is also checked against the oracle's fp64 product ("DeepGEMM
Essentials", Parts 1 and 6) with the bf16 GEMM tolerances.  A problem whose
partial sums would not fit the 32 MiB scratch is refused with FGFP8_ESCRATCH
and writes nothing.
"""
import ctypes

import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, mfma_truncation_bound, sample_idx, say

pytestmark = pytest.mark.gpu

FGFP8_ESCRATCH = -4
SCRATCH_BYTES = 32 << 20


def _operands(m, n, k):
    a = si.randn((m, k), si.SEED_A, 0.1)
    b = si.randn((n, k), si.SEED_B, 0.1)
    qa, sa = oracle.cast_per_token(si.host_array(a), 128, oracle.SF_FP32)
    qb, sb = oracle.cast_per_block(si.host_array(b), oracle.SF_FP32)
    return qa, sa, qb, sb


def _device(qa, sa, qb, sb):
    m, u = sa.shape
    ld = -(-m // 4) * 4
    buf = torch.zeros((u, ld), dtype=torch.float32)
    buf[:, :m] = torch.from_numpy(np.ascontiguousarray(sa.T))
    return (torch.from_numpy(qa).cuda(), buf.cuda().t()[:m], torch.from_numpy(qb).cuda(),
            torch.from_numpy(sb).cuda())


def _out(m, n):
    ldd = -(-n // 8) * 8
    return torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")


def _bits(D, n):
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, n:] == 0x7FC0).all(), "padding columns of D were written"
    return Dh[:, :n]


def test_noalloc_matches_workspace_entry_point(gpu):
    # (64, 7168, 7168) needs 25.7 MB of the 32 MiB: 392 shares of 8 units, every tile
    # shared 7 ways; then a smaller problem with ragged n and 18 one-unit shares
    for m, n, k in [(64, 7168, 7168), (5, 1000, 1152)]:
        assert fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k) <= SCRATCH_BYTES
        qa, sa, qb, sb = _operands(m, n, k)
        A, sa_d, B, sb_d = _device(qa, sa, qb, sb)
        ws = torch.full((fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k) // 4,), float("nan"),
                        dtype=torch.float32, device="cuda")
        D_ws, D_na = _out(m, n), _out(m, n)
        say("gemm_fp8_nt_bf16_splitk", (m, n, k))
        fg.gemm_fp8_nt_bf16_splitk(A, sa_d, B, sb_d, D_ws[:, :n].view(torch.bfloat16), ws)
        torch.cuda.synchronize()
        say("gemm_fp8_nt_bf16_splitk_noalloc", (m, n, k))
        fg.gemm_fp8_nt_bf16_splitk_noalloc(A, sa_d, B, sb_d, D_na[:, :n].view(torch.bfloat16))
        torch.cuda.synchronize()
        got_ws, got_na = _bits(D_ws, n), _bits(D_na, n)
        assert np.array_equal(got_na, got_ws), f"noalloc differs from the workspace entry point at {(m, n, k)}"
        ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
        check_bf16_gemm(got_na, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128,
                        f"splitk noalloc {(m, n, k)}")


def test_noalloc_kslices_matches_workspace_entry_point(gpu):
    # m > 64 takes K slices of 128x128 tiles: 512 x 4096 x 7168 fills all 32 MiB (128
    # tiles x 4 slices of 64 KB), then a smaller ragged problem (6 tiles x 2 slices)
    for m, n, k in [(512, 4096, 7168), (130, 300, 2176)]:
        wsb = fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k)
        assert 0 < wsb <= SCRATCH_BYTES
        qa, sa, qb, sb = _operands(m, n, k)
        A, sa_d, B, sb_d = _device(qa, sa, qb, sb)
        ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device="cuda")
        D_ws, D_na = _out(m, n), _out(m, n)
        say("gemm_fp8_nt_bf16_splitk", (m, n, k))
        fg.gemm_fp8_nt_bf16_splitk(A, sa_d, B, sb_d, D_ws[:, :n].view(torch.bfloat16), ws)
        torch.cuda.synchronize()
        say("gemm_fp8_nt_bf16_splitk_noalloc", (m, n, k))
        fg.gemm_fp8_nt_bf16_splitk_noalloc(A, sa_d, B, sb_d, D_na[:, :n].view(torch.bfloat16))
        torch.cuda.synchronize()
        got_ws, got_na = _bits(D_ws, n), _bits(D_na, n)
        assert np.array_equal(got_na, got_ws), f"noalloc differs from the workspace entry point at {(m, n, k)}"
        ii, jj = sample_idx(m, n, 20000, 5)
        ref, absum = oracle.gemm_nt(qa, sa, qb, sb, idx=(ii, jj))
        check_bf16_gemm(got_na[ii, jj], ref, absum, mfma_truncation_bound(qa, sa, qb, sb, idx=(ii, jj)), k // 128,
                        f"splitk noalloc kslices {(m, n, k)}")


def test_noalloc_refuses_problems_beyond_the_scratch(gpu):
    # k = 16384 at m = 64, n = 7168: 7168 units in 896 shares need 58.7 MB of partial sums
    m, n, k = 64, 7168, 16384
    assert fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k) > SCRATCH_BYTES
    A = torch.zeros((m, k), dtype=torch.uint8, device="cuda")
    B = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    sa = torch.ones((k // 128, m), dtype=torch.float32, device="cuda").t()
    sb = torch.ones((n // 128, k // 128), dtype=torch.float32, device="cuda")
    D = _out(m, n)
    lib = fg.load()
    say("gemm_fp8_nt_bf16_splitk_noalloc oversize", (m, n, k))
    rc = lib.gemm_fp8_nt_bf16_splitk_noalloc(ctypes.c_void_p(A.data_ptr()), k, ctypes.c_void_p(sa.data_ptr()),
                                             fg.SF_FP32, m, ctypes.c_void_p(B.data_ptr()), k,
                                             ctypes.c_void_p(sb.data_ptr()), k // 128,
                                             ctypes.c_void_p(D.data_ptr()), D.stride(0), m, n, k, None)
    torch.cuda.synchronize()
    assert rc == FGFP8_ESCRATCH
    assert (D.cpu().numpy().view(np.uint16) == 0x7FC0).all(), "a refused call wrote D"
