"""GPU parity of the m-grouped contiguous GEMM ("DeepGEMM Essentials",
Parts 8-11) against the oracle: row i uses expert m_indices[i]; padding rows
(-1) and rows outside a block's expert are not written.  Tolerance as for the
plain GEMM (see test_gpu_gemm)."""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, mfma_truncation_bound, say

pytestmark = pytest.mark.gpu


def _operands(m_idx, E, n, k, seed=0, a_fmt=oracle.SF_FP32):
    m = m_idx.size
    qa, sa = oracle.cast_per_token(si.host_array(si.randn((m, k), seed, 0.1)), 128, a_fmt)
    qb = np.empty((E, n, k), np.uint8)
    sb = np.empty((E, -(-n // 128), k // 128), np.float32)
    for e in range(E):
        qb[e], sb[e] = oracle.cast_per_block(si.host_array(si.randn((n, k), seed + 1 + e, 0.1)), oracle.SF_FP32)
    return qa, sa, qb, sb


def _dev_mn(sa, dtype=torch.float32):
    m, u = sa.shape
    ld = -(-m // 4) * 4
    buf = torch.zeros((u, ld), dtype=dtype)
    buf[:, :m] = torch.from_numpy(np.ascontiguousarray(sa.T).view(np.int32 if dtype == torch.int32 else np.float32))
    return buf.cuda().t()[:m]


def _run(qa, sa, qb, sb, m_idx, sa_fmt=fg.SF_FP32):
    m, k = qa.shape
    E, n = qb.shape[0], qb.shape[1]
    ldd = -(-n // 8) * 8
    D = torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")
    say("m_grouped_gemm", (m, n, k), "experts", E, "sa_fmt", sa_fmt)
    fg.m_grouped_gemm_fp8_nt_bf16_contiguous(
        torch.from_numpy(qa).cuda(), _dev_mn(sa, torch.int32 if sa_fmt == fg.SF_PACKED_UE8M0 else torch.float32),
        torch.from_numpy(qb).cuda(), torch.from_numpy(sb).cuda(), torch.from_numpy(m_idx).cuda(),
        D[:, :n].view(torch.bfloat16), sa_fmt)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, n:] == 0x7FC0).all()
    return Dh[:, :n]


def _trunc_bound(qa, sa, qb, sb, m_idx):
    t = np.zeros((qa.shape[0], qb.shape[1]))
    for e in range(qb.shape[0]):
        rows = np.nonzero(m_idx == e)[0]
        if rows.size:
            t[rows] = mfma_truncation_bound(qa[rows], sa[rows], qb[e], sb[e])
    return t


def _check(tokens, n, k, seed=0):
    m_idx = si.grouped_layout(tokens)
    qa, sa, qb, sb = _operands(m_idx, len(tokens), n, k, seed)
    got = _run(qa, sa, qb, sb, m_idx)
    ref, absum = oracle.m_grouped_gemm_nt(qa, sa, qb, sb, m_idx)
    pad = m_idx < 0
    assert (got[pad] == 0x7FC0).all(), "padding rows were written"
    valid = ~pad
    check_bf16_gemm(got[valid], ref[valid], absum[valid], _trunc_bound(qa, sa, qb, sb, m_idx)[valid], k // 128,
                    f"m_grouped {tokens} n={n} k={k}")


def test_walkthrough_four_experts(gpu):
    _check(si.MOE_TOKENS_4, 256, 512)


def test_exercise_eight_experts_hidden_2048(gpu):
    _check(si.MOE_TOKENS_8, 2048, 2048, seed=3)


@pytest.mark.parametrize("tokens", [[1], [300], [0, 5, 0, 129], [128, 128, 128]])
def test_segment_edges(gpu, tokens):
    _check(tokens, 200, 384, seed=5)


def test_each_row_uses_its_expert(gpu):
    # all-ones operands, expert e's blocks scaled by 2^e: D = k * 2^e exactly
    tokens = [3, 128, 40, 1]
    m_idx = si.grouped_layout(tokens)
    k, n = 256, 136
    qa = np.full((m_idx.size, k), 0x38, np.uint8)
    sa = np.ones((m_idx.size, k // 128), np.float32)
    qb = np.full((len(tokens), n, k), 0x38, np.uint8)
    sb = np.stack([np.full((2, k // 128), 2.0 ** e, np.float32) for e in range(len(tokens))])
    got = oracle.bf16_bits_to_f32(_run(qa, sa, qb, sb, m_idx)).astype(np.float64)
    for i, e in enumerate(m_idx):
        if e >= 0:
            assert (got[i] == k * 2.0 ** e).all(), f"row {i}"


def test_packed_ue8m0_lhs(gpu):
    m_idx = si.grouped_layout([100, 200])
    qa, words, qb, sb = _operands(m_idx, 2, 256, 1024, seed=7, a_fmt=oracle.SF_PACKED_UE8M0)
    sa = oracle.unpack_ue8m0(words, 1024 // 128)
    got = _run(qa, words, qb, sb, m_idx, sa_fmt=fg.SF_PACKED_UE8M0)
    ref, absum = oracle.m_grouped_gemm_nt(qa, sa, qb, sb, m_idx)
    v = m_idx >= 0
    check_bf16_gemm(got[v], ref[v], absum[v], _trunc_bound(qa, sa, qb, sb, m_idx)[v], 8, "m_grouped packed sa")


def test_invalid_ids_and_mixed_blocks_leave_rows_unwritten(gpu):
    # block 0: expert 1; block 1: id 7 >= E (skipped); block 2: experts 0 and 1 mixed
    m_idx = np.full(384, -1, np.int32)
    m_idx[:100] = 1
    m_idx[128:200] = 7
    m_idx[256:300] = 0
    m_idx[300:310] = 1
    qa, sa, qb, sb = _operands(m_idx, 2, 128, 256, seed=9)
    got = _run(qa, sa, qb, sb, m_idx)
    assert (got[128:256] == 0x7FC0).all()           # invalid id: nothing written
    assert (got[256:300] == 0x7FC0).all()           # expert 0 rows in a block computed for expert 1
    assert (got[310:] == 0x7FC0).all() and (got[100:128] == 0x7FC0).all()
    rows = np.r_[0:100, 300:310]
    ref, absum = oracle.m_grouped_gemm_nt(qa[rows], sa[rows], qb, sb, m_idx[rows])
    check_bf16_gemm(got[rows], ref, absum, _trunc_bound(qa[rows], sa[rows], qb, sb, m_idx[rows]), 2, "mixed")


def test_all_padding_writes_nothing(gpu):
    # every row padding (-1): the launch runs and no output row is written
    m_idx = np.full(256, -1, np.int32)
    qa, sa, qb, sb = _operands(m_idx, 3, 256, 384, seed=12)
    got = _run(qa, sa, qb, sb, m_idx)
    assert (got == 0x7FC0).all()
