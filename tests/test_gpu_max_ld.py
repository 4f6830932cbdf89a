"""Calls at the C ABI's size limits, against the oracle.

GEMMs at the largest leading dimension the ABI accepts (lda, ldb = 2^24 - 16 bytes,
the limit of the kernels' 32-bit in-tile copy offsets).

The operands sit in the first k columns of [rows, 2^24 - 16] buffers (about 2.2 GB each), so
the copy offsets of the last tile rows come within 1% of 2^31.  Covered: the 128x128 kernel
(one K chain, and two for 8 K blocks on a 4-tile grid), the skinny decode kernel, the
weight gradient, and the group-32 kernel.  Tolerances as in test_gpu_gemm and test_gpu_g32.
Definitions: "DeepGEMM Essentials", Parts 1, 6, 12-13.

The per-token cast of a transposed view with the most column tiles the ABI accepts
(65535 tiles of 128 tokens along the launch grid's y), bit for bit ("DeepGEMM
Essentials", Part 3)."""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, check_wgrad, gpu_cast_per_token, mfma_truncation_bound, oracle_sf_bits, say

pytestmark = pytest.mark.gpu

LD = (1 << 24) - 16


def _wide(q: np.ndarray) -> torch.Tensor:
    """[rows, k] bytes placed in the first k columns of a [rows, LD] device buffer."""
    rows, k = q.shape
    buf = torch.empty((rows, LD), dtype=torch.uint8, device="cuda")
    buf[:, :k] = torch.from_numpy(q).cuda()
    return buf[:, :k]


def _mn(sa: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    m, u = sa.shape
    ld = -(-m // 4) * 4
    buf = torch.zeros((u, ld), dtype=dtype)
    buf[:, :m] = torch.from_numpy(np.ascontiguousarray(sa.T).view(np.int32 if dtype == torch.int32 else np.float32))
    return buf.cuda().t()[:m]


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mnk", [(130, 136, 256), (130, 136, 1024), (40, 136, 512)])
def test_gemm_max_leading_dimension(gpu, mnk):
    m, n, k = mnk
    qa, sa = oracle.cast_per_token(si.host_array(si.randn((m, k), si.SEED_A)))
    qb, sb = oracle.cast_per_block(si.host_array(si.randn((n, k), si.SEED_B)))
    A, B = _wide(qa), _wide(qb)
    assert A.stride(0) == LD and B.stride(0) == LD
    D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    say("gemm_fp8_nt_bf16 lda=ldb=2^24-16", mnk)
    fg.gemm_fp8_nt_bf16(A, _mn(sa), B, torch.from_numpy(sb).cuda(), D)
    torch.cuda.synchronize()
    got = D.view(torch.int16).cpu().numpy().view(np.uint16)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128, f"gemm max ld {mnk}")


def test_wgrad_max_leading_dimension(gpu):
    tokens, d_out, d_in = 256, 130, 136
    qa, sa = oracle.cast_per_token(si.host_array(si.randn((tokens, d_out), si.SEED_DY)), transpose=True)
    qb, sb = oracle.cast_per_token(si.host_array(si.randn((tokens, d_in), si.SEED_A)), transpose=True)
    d0 = si.randn((d_out, d_in), 5, 0.1, torch.float32).numpy()
    A, B = _wide(qa), _wide(qb)
    D = torch.from_numpy(d0.copy()).cuda()
    say("wgrad_gemm_fp8_nt_fp32 lda=ldb=2^24-16", (d_out, d_in, tokens))
    fg.wgrad_gemm_fp8_nt_fp32(A, _mn(sa), B, _mn(sb), D)
    torch.cuda.synchronize()
    ref, absum = oracle.wgrad_nt(qa, sa, qb, sb, d0)
    check_wgrad(D.cpu().numpy(), ref, absum, tokens // 128, "wgrad max ld")


def test_g32_max_leading_dimension(gpu):
    m, n, k = 130, 136, 512
    qa, wa = oracle.cast_per_token(si.host_array(si.randn((m, k), si.SEED_A)), 32, oracle.SF_PACKED_UE8M0)
    qb, wb = oracle.cast_per_token(si.host_array(si.randn((n, k), si.SEED_B)), 32, oracle.SF_PACKED_UE8M0)
    A, B = _wide(qa), _wide(qb)
    D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    say("gemm_fp8_nt_bf16_ue8m0_g32 lda=ldb=2^24-16", (m, n, k))
    fg.gemm_fp8_nt_bf16_ue8m0_g32(A, _mn(wa, torch.int32), B, _mn(wb, torch.int32), D)
    torch.cuda.synchronize()
    got = D.view(torch.int16).cpu().numpy().view(np.uint16)
    sa, sb = oracle.unpack_ue8m0(wa, k // 32), oracle.unpack_ue8m0(wb, k // 32)
    ref, absum = oracle.gemm_nt_g32(qa, sa, qb, sb)
    tb = mfma_truncation_bound(qa, sa, qb, sb, sb_block=False, group=32)
    check_bf16_gemm(got, ref, absum, tb, k // 8, "g32 max ld")


def test_transposed_cast_most_column_tiles(gpu):
    # x [tokens, 16 features]; its transposed view [16, tokens] is cast with 1x128 groups along
    # the tokens, 65535 column tiles of 128: the largest grid the ABI accepts for this path
    tokens = 65535 * 128
    x = si.cast_workload(tokens, 16, seed=si.SEED_A)
    q, sf, _, _, _ = gpu_cast_per_token(x, 128, oracle.SF_FP32, mn_major=True, transpose=True)
    oq, osf = oracle.cast_per_token(si.host_array(x), 128, oracle.SF_FP32, transpose=True)
    assert q.shape == (16, tokens)
    assert np.array_equal(q, oq), "E4M3 bytes differ"
    assert np.array_equal(sf, oracle_sf_bits(osf)), "scale bits differ"
