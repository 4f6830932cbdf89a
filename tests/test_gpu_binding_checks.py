"""The Python binding's marshalling checks: each call whose tensors do not have exactly the
shapes, dtypes and device the entry point addresses raises ValueError before anything is
launched, and leaves its outputs untouched.  (The C ABI sees only pointers and strides,
so these checks are what keeps a kernel inside the tensors it is given.)"""
import pytest
import torch

import fine_grained_block_token_amd as fg

pytestmark = pytest.mark.gpu

M, N, K = 130, 256, 512
KB = K // 128


def _gemm_args():
    A = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    B = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    sa = fg.mn_major_scales(M, KB)
    sb = torch.ones((N // 128, KB), dtype=torch.float32, device="cuda")
    D = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    return A, sa, B, sb, D


def _untouched(D, v=3.0):
    torch.cuda.synchronize()
    assert (D.float() == v).all()


@pytest.mark.parametrize("bad", ["sb_short", "sb_dtype", "sa_rows", "sa_dtype", "D_shape", "D_dtype",
                                 "B_k", "A_transposed", "sa_row_major", "cpu_sb"])
def test_gemm_rejects_bad_tensors(gpu, bad):
    A, sa, B, sb, D = _gemm_args()
    if bad == "sb_short":
        sb = sb[:1]
    elif bad == "sb_dtype":
        sb = sb.to(torch.int32)
    elif bad == "sa_rows":
        sa = fg.mn_major_scales(M - 1, KB)
    elif bad == "sa_dtype":
        sa = fg.mn_major_scales(M, KB, torch.int32)
    elif bad == "D_shape":
        D = D[:, :N - 8]
    elif bad == "D_dtype":
        D = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    elif bad == "B_k":
        B = B[:, :K - 128]
    elif bad == "A_transposed":
        A = torch.zeros((K, M), dtype=torch.uint8, device="cuda").t()
    elif bad == "sa_row_major":
        sa = torch.ones((M, KB), dtype=torch.float32, device="cuda")
    elif bad == "cpu_sb":
        sb = sb.cpu()
    with pytest.raises(ValueError):
        fg.gemm_fp8_nt_bf16(A, sa, B, sb, D)
    _untouched(D)


def test_gemm_accepts_the_same_tensors(gpu):
    A, sa, B, sb, D = _gemm_args()
    sa.fill_(1.0)
    fg.gemm_fp8_nt_bf16(A, sa, B, sb, D)
    _untouched(D, 0.0)   # zero operands: zero output


def test_wgrad_rejects_bad_tensors(gpu):
    A = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    B = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    sa, sb = fg.mn_major_scales(M, KB), fg.mn_major_scales(N, KB)
    D = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fg.wgrad_gemm_fp8_nt_fp32(A, sa, B, fg.mn_major_scales(N, KB - 1), D)
    with pytest.raises(ValueError):
        fg.wgrad_gemm_fp8_nt_fp32(A, sa, B, sb, D.to(torch.bfloat16))
    with pytest.raises(ValueError):
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0(A, sa, B, sb, D, fg.SF_PACKED_UE8M0)   # float32 given for packed words
    with pytest.raises(ValueError):
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0_g32(A, sa, B, sb, D)                   # float32 given for int32 words
    _untouched(D)


def test_casts_reject_bad_tensors(gpu):
    x = torch.ones((M, K), dtype=torch.bfloat16, device="cuda")
    q = torch.full((M, K), 0xA5, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fg.cast_per_token(x, q, torch.empty((M, KB - 1), device="cuda"))
    with pytest.raises(ValueError):
        fg.cast_per_token(x, q, torch.empty((M, KB), dtype=torch.int32, device="cuda"))   # fp32 format
    with pytest.raises(ValueError):
        fg.cast_per_token(x, q, torch.empty((M, KB), device="cuda"), 128, fg.SF_PACKED_UE8M0)
    with pytest.raises(ValueError):
        fg.cast_per_block(x, q, torch.empty((1, KB), device="cuda"))
    with pytest.raises(ValueError):
        fg.cast_per_block(x.t().contiguous().t(), q, torch.empty((2, KB), device="cuda"))   # column-major x
    with pytest.raises(ValueError):
        fg.cast_per_token_dual(x, q, torch.empty((M, KB), device="cuda"),
                               torch.empty((K, M), dtype=torch.uint8, device="cuda"), torch.empty((K, 1), device="cuda"))
    torch.cuda.synchronize()
    assert (q == 0xA5).all()


def test_grouped_rejects_bad_tensors(gpu):
    E = 2
    A = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    B = torch.zeros((E, N, K), dtype=torch.uint8, device="cuda")
    sa = fg.mn_major_scales(M, KB)
    sb = torch.ones((E, N // 128, KB), dtype=torch.float32, device="cuda")
    idx = torch.zeros((M,), dtype=torch.int32, device="cuda")
    D = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fg.m_grouped_gemm_fp8_nt_bf16_contiguous(A, sa, B, sb[:1], idx, D)
    with pytest.raises(ValueError):
        fg.m_grouped_gemm_fp8_nt_bf16_contiguous(A, sa, B, sb, idx[:-1], D)
    with pytest.raises(ValueError):
        fg.m_grouped_gemm_fp8_nt_bf16_contiguous(A, sa, B, sb, idx.to(torch.int64), D)
    _untouched(D)
