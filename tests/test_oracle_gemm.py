"""Pins for the oracle's block-scaled NT GEMM and wgrad (CPU only).

The GEMM is D = (A * sa)(B * sb)^T with A [m, k] E4M3 and one fp32 scale per
row and 128-wide K block, B [n, k] E4M3 and one fp32 scale per 128 x 128
block ("DeepGEMM Essentials: High-Performance FP8 Matrix Multiplication",
Parts 1, 3-6; the scale-row reply in "[Help] Starter script for nn.Linear for
fwd,bwd").  wgrad adds A.B^T to an fp32 tensor with one scale per row and K
block on both operands ("DeepGEMM Essentials", Parts 12-13).

Independent pins: fp64 brute force over operands dequantised with PyTorch's
float8 decoder; closed forms (all-ones operands with power-of-two scales;
one-hot K positions that expose the scale indexing); accumulate semantics;
bf16 rounding against PyTorch's fp32->bf16 conversion.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si


def _dequant(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _operands(m, n, k, seed=0, scale=1.0):
    a = si.randn((m, k), seed, scale)
    b = si.randn((n, k), seed + 1, scale)
    qa, sa = oracle.cast_per_token(si.host_array(a), 128, oracle.SF_FP32)
    qb, sb = oracle.cast_per_block(si.host_array(b), oracle.SF_FP32)
    return qa, sa, qb, sb


def _brute(qa, sa, qb, sb, sb_block=True):
    m, k = qa.shape
    n = qb.shape[0]
    a = _dequant(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    if sb_block:
        sbe = np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:n], 128, axis=1)
    else:
        sbe = np.repeat(sb.astype(np.float64), 128, axis=1)
    b = _dequant(qb) * sbe
    return a @ b.T, np.abs(a) @ np.abs(b).T


@pytest.mark.parametrize("mnk", [(1, 128, 128), (3, 256, 384), (129, 200, 256), (128, 256, 512)])
def test_blockwise_matches_brute_force(mnk):
    qa, sa, qb, sb = _operands(*mnk)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    bf, bfabs = _brute(qa, sa, qb, sb)
    assert np.all(np.abs(ref - bf) <= 1e-12 * bfabs + 1e-300)
    assert np.allclose(absum, bfabs, rtol=1e-12, atol=0)


def test_sampled_outputs_equal_full():
    qa, sa, qb, sb = _operands(129, 200, 256)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    rng = np.random.default_rng(0)
    ii = rng.integers(0, 129, 50)
    jj = rng.integers(0, 200, 50)
    r2, a2 = oracle.gemm_nt(qa, sa, qb, sb, idx=(ii, jj))
    assert np.array_equal(r2, ref[ii, jj]) and np.array_equal(a2, absum[ii, jj])


def test_all_ones_power_of_two_scales():
    m, n, k = 5, 300, 384
    kb = k // 128
    qa = np.full((m, k), 0x38, np.uint8)         # E4M3 1.0
    qb = np.full((n, k), 0x38, np.uint8)
    pa = np.array([[(i % 3) - kb_ for kb_ in range(kb)] for i in range(m)])
    pb = np.array([[jb + (kb_ % 2) for kb_ in range(kb)] for jb in range(3)])
    sa = np.ldexp(np.float32(1), pa).astype(np.float32)
    sb = np.ldexp(np.float32(1), pb).astype(np.float32)
    ref, _ = oracle.gemm_nt(qa, sa, qb, sb)
    for i in range(m):
        for j in range(n):
            want = sum(128 * 2.0 ** (pa[i, t] + pb[j // 128, t]) for t in range(kb))
            assert ref[i, j] == want


def test_one_hot_pins_scale_indexing():
    """A(i0,t0) = B(j0,t0) = 1: D(i0,j0) = sa(i0, t0/128) * sb(j0/128, t0/128), rest 0."""
    m, n, k = 7, 300, 384
    rng = np.random.default_rng(1)
    sa = rng.uniform(0.5, 2, (m, k // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (3, k // 128)).astype(np.float32)
    for i0, j0, t0 in [(0, 0, 0), (6, 299, 383), (3, 130, 200), (5, 257, 129)]:
        qa = np.zeros((m, k), np.uint8)
        qb = np.zeros((n, k), np.uint8)
        qa[i0, t0] = 0x38
        qb[j0, t0] = 0x38
        ref, _ = oracle.gemm_nt(qa, sa, qb, sb)
        want = np.zeros((m, n))
        want[i0, j0] = float(sa[i0, t0 // 128]) * float(sb[j0 // 128, t0 // 128])
        assert np.array_equal(ref, want)


def test_signs_and_negative_codes():
    m, n, k = 2, 2, 128
    qa = np.zeros((m, k), np.uint8)
    qb = np.zeros((n, k), np.uint8)
    qa[0, :2] = [0x38, 0xB8]          # +1, -1
    qb[0, :2] = [0x40, 0x40]          # +2, +2
    qb[1, :2] = [0x40, 0xC0]          # +2, -2
    sa = np.ones((m, 1), np.float32)
    sb = np.ones((1, 1), np.float32)
    ref, _ = oracle.gemm_nt(qa, sa, qb, sb)
    assert ref[0, 0] == 0.0 and ref[0, 1] == 4.0 and ref[1, 0] == 0.0


def test_wgrad_row_scales_and_accumulate():
    m, n, k = 33, 130, 256          # k plays the role of tokens
    a = si.randn((k, m), 0)         # dY [tokens, out]
    b = si.randn((k, n), 1)         # x  [tokens, in]
    qa, sa = oracle.cast_per_token(si.host_array(a), 128, oracle.SF_FP32, transpose=True)
    qb, sb = oracle.cast_per_token(si.host_array(b), 128, oracle.SF_FP32, transpose=True)
    d_in = si.randn((m, n), 2, 0.1, torch.float32).numpy()
    ref, absum = oracle.wgrad_nt(qa, sa, qb, sb, d_in)
    bf, bfabs = _brute(qa, sa, qb, sb, sb_block=False)
    assert np.all(np.abs(ref - (d_in + bf)) <= 1e-12 * (bfabs + np.abs(d_in)))
    zero, _ = oracle.wgrad_nt(qa, sa, qb, sb, np.zeros((m, n), np.float32))
    twice, _ = oracle.wgrad_nt(qa, sa, qb, sb, zero)
    assert np.allclose(twice, 2 * zero, rtol=1e-15, atol=0)


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.38e38)]
    ties = (np.arange(0x3F800000, 0x3F800000 + 0x10000 * 64, 0x8000, dtype=np.uint32)).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.float32([0.0, -0.0, 1e-40, -3e-39])])
    ours = oracle.round_bf16(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_round_bf16_uses_all_fp64_bits():
    # just above / below an exact bf16 tie: fp64 resolves what fp32 could not
    tie = 1.0 + 2.0 ** -8                    # halfway between 1.0 and 1.0078125
    got = oracle.round_bf16(np.array([tie, tie + 2.0 ** -40, tie - 2.0 ** -40]))
    assert list(got) == [0x3F80, 0x3F81, 0x3F80]
