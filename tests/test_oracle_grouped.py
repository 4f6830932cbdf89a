"""Pins for the oracle's m-grouped contiguous GEMM (CPU only): row i uses the
expert m_indices[i] ("DeepGEMM Essentials", Parts 8-11: tokens of one expert
are contiguous, each expert's segment padded to a multiple of 128 rows, -1
marks padding).  Independent pins: fp64 brute force per row over operands
dequantised with PyTorch's float8 decoder, and a closed form in which every
expert's weights give a distinct power of two."""
import numpy as np
import torch

import oracle
import synth_inputs as si


def _dequant(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _grouped_operands(tokens, n, k, seed=0):
    m_idx = si.grouped_layout(tokens)
    m, E = m_idx.size, len(tokens)
    a = si.randn((m, k), seed)
    qa, sa = oracle.cast_per_token(si.host_array(a), 128, oracle.SF_FP32)
    qb = np.empty((E, n, k), np.uint8)
    sb = np.empty((E, -(-n // 128), k // 128), np.float32)
    for e in range(E):
        qb[e], sb[e] = oracle.cast_per_block(si.host_array(si.randn((n, k), seed + 1 + e)), oracle.SF_FP32)
    return qa, sa, qb, sb, m_idx


def test_layout_of_the_walkthrough():
    m_idx = si.grouped_layout(si.MOE_TOKENS_4)
    assert m_idx.size == 128 + 128 + 128 + 256
    assert (m_idx[:128] == 0).all()
    assert (m_idx[128:224] == 1).all() and (m_idx[224:256] == -1).all()
    assert (m_idx[256:368] == 2).all() and (m_idx[368:384] == -1).all()
    assert (m_idx[384:528] == 3).all() and (m_idx[528:] == -1).all()


def test_grouped_matches_brute_force():
    qa, sa, qb, sb, m_idx = _grouped_operands([5, 130, 128], 200, 256)
    ref, absum = oracle.m_grouped_gemm_nt(qa, sa, qb, sb, m_idx)
    a = _dequant(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    for i in range(m_idx.size):
        e = m_idx[i]
        if e < 0:
            assert np.isnan(ref[i]).all()
            continue
        sbe = np.repeat(np.repeat(sb[e].astype(np.float64), 128, axis=0)[:200], 128, axis=1)
        b = _dequant(qb[e]) * sbe
        want = b @ a[i]
        assert np.all(np.abs(ref[i] - want) <= 1e-12 * (np.abs(b) @ np.abs(a[i])) + 1e-300)
        assert np.allclose(absum[i], np.abs(b) @ np.abs(a[i]), rtol=1e-12, atol=0)


def test_each_row_uses_its_expert():
    # all-ones operands; expert e's weights carry the scale 2^e in every block
    tokens = [3, 128, 40, 1]
    m_idx = si.grouped_layout(tokens)
    k, n = 256, 130
    qa = np.full((m_idx.size, k), 0x38, np.uint8)
    sa = np.ones((m_idx.size, k // 128), np.float32)
    qb = np.full((len(tokens), n, k), 0x38, np.uint8)
    sb = np.stack([np.full((2, k // 128), 2.0 ** e, np.float32) for e in range(len(tokens))])
    ref, _ = oracle.m_grouped_gemm_nt(qa, sa, qb, sb, m_idx)
    for i, e in enumerate(m_idx):
        if e >= 0:
            assert (ref[i] == k * 2.0 ** e).all()


def test_sampled_outputs_equal_full():
    qa, sa, qb, sb, m_idx = _grouped_operands(si.MOE_TOKENS_4, 256, 512)
    ref, absum = oracle.m_grouped_gemm_nt(qa, sa, qb, sb, m_idx)
    rng = np.random.default_rng(1)
    ii = rng.integers(0, m_idx.size, 300)
    jj = rng.integers(0, 256, 300)
    r2, a2 = oracle.m_grouped_gemm_nt(qa, sa, qb, sb, m_idx, idx=(ii, jj))
    same = np.isnan(r2) == np.isnan(ref[ii, jj])
    assert same.all()
    ok = ~np.isnan(r2)
    assert np.array_equal(r2[ok], ref[ii, jj][ok]) and np.array_equal(a2[ok], absum[ii, jj][ok])
