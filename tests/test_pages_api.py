"""Host-side checks of fine_grained_block_token_amd.api, the calls in the form the pages
write them ("DeepGEMM Essentials", Parts 5-13; "deep-gemm: fused per-token FP8 cast in
Triton"): the scale-layout helper and the argument checks that run before any launch."""
import pytest
import torch

from fine_grained_block_token_amd import Fgfp8Error, api


def test_m_alignment():
    # expert segments of the contiguous grouped layout are padded to whole 128-row blocks
    assert api.get_m_alignment_for_contiguous_layout() == 128


@pytest.mark.parametrize("rows,groups", [(1, 1), (1, 7), (3, 1), (4, 2), (130, 5), (8192, 56)])
def test_col_major_tma_aligned(rows, groups):
    sf = torch.arange(rows * groups, dtype=torch.float32).reshape(rows, groups) + 0.5
    out = api.get_col_major_tma_aligned_tensor(sf)
    ld = -(-rows // 4) * 4
    assert out.shape == (rows, groups) and out.dtype == sf.dtype
    assert out.stride(1) == ld and (rows == 1 or out.stride(0) == 1)
    assert torch.equal(out, sf)
    # (r, g) sits at g * ld + r in the underlying storage
    flat = torch.as_strided(out, (groups * ld,), (1,))
    r, g = rows - 1, groups - 1
    assert flat[g * ld + r] == sf[r, g]
    # already laid out: returned as is
    assert api.get_col_major_tma_aligned_tensor(out) is out


def test_col_major_tma_aligned_int32_words():
    words = torch.randint(0, 2 ** 31 - 1, (77, 3), dtype=torch.int32)
    out = api.get_col_major_tma_aligned_tensor(words)
    assert out.dtype == torch.int32 and torch.equal(out, words) and out.stride() == (1, 80)


def test_col_major_tma_aligned_refuses_non_2d():
    with pytest.raises(Fgfp8Error):
        api.get_col_major_tma_aligned_tensor(torch.zeros(4))


def test_cast_argument_checks():
    with pytest.raises(Fgfp8Error):
        api.per_token_cast_to_fp8(torch.zeros(2, 3, 128, dtype=torch.bfloat16))
    with pytest.raises(Fgfp8Error):
        api.per_token_cast_to_fp8(torch.zeros(4, 128, dtype=torch.bfloat16), use_ue8m0=False, use_packed_ue8m0=True)
    with pytest.raises(Fgfp8Error):
        api.per_block_cast_to_fp8(torch.zeros(128, dtype=torch.bfloat16))
    assert api.fused_per_token_cast_to_fp8 is api.per_token_cast_to_fp8


def test_gemm_refuses_row_major_lhs_scales():
    a = torch.zeros(8, 256, dtype=torch.uint8)
    sa = torch.ones(8, 2)                  # row-major: stride(0) == 2
    b = torch.zeros(128, 256, dtype=torch.uint8)
    sb = torch.ones(1, 2)
    out = torch.empty(8, 128, dtype=torch.bfloat16)
    with pytest.raises(Fgfp8Error, match="get_col_major_tma_aligned_tensor"):
        api.gemm_fp8_fp8_bf16_nt((a, sa), (b, sb), out)
    with pytest.raises(Fgfp8Error, match="get_col_major_tma_aligned_tensor"):
        api.m_grouped_gemm_fp8_fp8_bf16_nt_contiguous((a, sa), (b[None], sb[None]), out,
                                                       torch.zeros(8, dtype=torch.int32))
    with pytest.raises(Fgfp8Error, match="packed LHS"):
        api.gemm_fp8_fp8_bf16_nt((a, api.get_col_major_tma_aligned_tensor(sa)),
                                 (b, torch.zeros(128, 2, dtype=torch.int32)), out)


def test_wgrad_refuses_bad_scales():
    a = torch.zeros(8, 256, dtype=torch.uint8)
    b = torch.zeros(16, 256, dtype=torch.uint8)
    out = torch.zeros(8, 16)
    sa = api.get_col_major_tma_aligned_tensor(torch.ones(8, 2))
    with pytest.raises(Fgfp8Error, match="RHS scales"):
        api.wgrad_gemm_fp8_fp8_fp32_nt((a, sa), (b, torch.ones(16, 2)), out)
    sb = api.get_col_major_tma_aligned_tensor(torch.ones(16, 2))
    with pytest.raises(Fgfp8Error, match="both operands"):
        api.wgrad_gemm_fp8_fp8_fp32_nt((a, sa.to(torch.int32)), (b, sb), out)
    with pytest.raises(Fgfp8Error, match="both operands"):
        api.wgrad_gemm_fp8_fp8_fp32_nt((a, sa.to(torch.float64)), (b, sb.to(torch.float64)), out)


def test_wgrad_packed_words_need_gran_k_when_k_is_128():
    # with k = 128 a 1 x 128 packed word and a group-32 word are both one word per row
    a = torch.zeros(8, 128, dtype=torch.uint8)
    b = torch.zeros(16, 128, dtype=torch.uint8)
    out = torch.zeros(8, 16)
    sa = api.get_col_major_tma_aligned_tensor(torch.zeros(8, 1, dtype=torch.int32))
    sb = api.get_col_major_tma_aligned_tensor(torch.zeros(16, 1, dtype=torch.int32))
    with pytest.raises(Fgfp8Error, match="gran_k"):
        api.wgrad_gemm_fp8_fp8_fp32_nt((a, sa), (b, sb), out)
    with pytest.raises(Fgfp8Error, match="gran_k must be"):
        api.wgrad_gemm_fp8_fp8_fp32_nt((a, sa), (b, sb), out, gran_k=64)
