"""Pins for the oracle's group-32 GEMM (both operands scaled per row and 32-wide
K group; the UE8M0 group-32 recipe of "deep-gemm: fused per-token FP8 cast in
Triton").  Independent pins: a per-element loop over PyTorch's float8 decoder
on a tiny shape; equality with the 128-block oracle (the C implementation)
when the four 32-groups of every 128-block share one scale; an all-ones closed
form; the packed-UE8M0 cast round trip."""
import numpy as np
import torch

import oracle
import synth_inputs as si


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _g32_operands(m, n, k, seed):
    qa, wa = oracle.cast_per_token(si.host_array(si.randn((m, k), seed)), 32, oracle.SF_PACKED_UE8M0)
    qb, wb = oracle.cast_per_token(si.host_array(si.randn((n, k), seed + 1)), 32, oracle.SF_PACKED_UE8M0)
    return qa, oracle.unpack_ue8m0(wa, k // 32), qb, oracle.unpack_ue8m0(wb, k // 32)


def test_loop_brute_force():
    qa, sa, qb, sb = _g32_operands(3, 5, 128, seed=4)
    ref, absum = oracle.gemm_nt_g32(qa, sa, qb, sb)
    a, b = _dec(qa), _dec(qb)
    for i in range(3):
        for j in range(5):
            want = sum(float(sa[i, t // 32]) * float(sb[j, t // 32]) * a[i, t] * b[j, t] for t in range(128))
            assert ref[i, j] == want or abs(ref[i, j] - want) <= 1e-15 * absum[i, j]


def test_equals_block_oracle_when_groups_share_a_scale():
    m, n, k = 40, 70, 512
    qa, sa, qb, sb = _g32_operands(m, n, k, seed=8)
    sa128 = sa[:, ::4].copy()
    sb128 = sb[:, ::4].copy()
    ref, _ = oracle.gemm_nt_g32(qa, np.repeat(sa128, 4, axis=1), qb, np.repeat(sb128, 4, axis=1))
    want, _ = oracle.gemm_nt(qa, sa128, qb, sb128, sb_block=False)
    assert np.allclose(ref, want, rtol=1e-14, atol=0)


def test_all_ones_closed_form():
    m, n, k = 4, 6, 256
    rng = np.random.default_rng(0)
    ea = rng.integers(-3, 4, (m, k // 32))
    eb = rng.integers(-3, 4, (n, k // 32))
    ref, _ = oracle.gemm_nt_g32(np.full((m, k), 0x38, np.uint8), np.ldexp(1.0, ea).astype(np.float32),
                                np.full((n, k), 0x38, np.uint8), np.ldexp(1.0, eb).astype(np.float32))
    want = np.array([[sum(32 * 2.0 ** (ea[i, g] + eb[j, g]) for g in range(k // 32)) for j in range(n)]
                     for i in range(m)])
    assert np.array_equal(ref, want)


def test_sampled_equals_full():
    qa, sa, qb, sb = _g32_operands(33, 65, 256, seed=12)
    ref, absum = oracle.gemm_nt_g32(qa, sa, qb, sb)
    ii, jj = np.array([0, 32, 5, 17]), np.array([64, 0, 33, 1])
    r, a = oracle.gemm_nt_g32(qa, sa, qb, sb, idx=(ii, jj))
    assert np.allclose(r, ref[ii, jj], rtol=1e-15, atol=1e-300) and np.allclose(a, absum[ii, jj], rtol=1e-15)


def test_wgrad_g32_loop_brute_force():
    # D_in + the per-element sum over tokens, element by element
    qa, sa, qb, sb = _g32_operands(3, 4, 256, seed=30)
    d_in = np.array([[0.5 * (i - j) for j in range(4)] for i in range(3)], np.float32)
    ref, absum = oracle.wgrad_nt_g32(qa, sa, qb, sb, d_in)
    a, b = _dec(qa), _dec(qb)
    for i in range(3):
        for j in range(4):
            want = float(d_in[i, j]) + sum(float(sa[i, t // 32]) * float(sb[j, t // 32]) * a[i, t] * b[j, t]
                                           for t in range(256))
            assert abs(ref[i, j] - want) <= 1e-15 * absum[i, j]


def test_wgrad_g32_all_ones_closed_form_with_d_in():
    m, n, k = 5, 3, 384
    rng = np.random.default_rng(31)
    ea = rng.integers(-2, 3, (m, k // 32))
    eb = rng.integers(-2, 3, (n, k // 32))
    d_in = rng.integers(-8, 9, (m, n)).astype(np.float32)
    ref, _ = oracle.wgrad_nt_g32(np.full((m, k), 0x38, np.uint8), np.ldexp(1.0, ea).astype(np.float32),
                                 np.full((n, k), 0x38, np.uint8), np.ldexp(1.0, eb).astype(np.float32), d_in)
    want = d_in.astype(np.float64) + np.array(
        [[sum(32 * 2.0 ** (ea[i, g] + eb[j, g]) for g in range(k // 32)) for j in range(n)] for i in range(m)])
    assert np.array_equal(ref, want)


def test_grouped_g32_one_expert_is_the_plain_gemm():
    qa, sa, qb, sb = _g32_operands(40, 70, 256, seed=40)
    ref, absum = oracle.m_grouped_gemm_nt_g32(qa, sa, qb[None], sb[None], np.zeros(40, np.int32))
    want, wabs = oracle.gemm_nt_g32(qa, sa, qb, sb)
    assert np.array_equal(ref, want) and np.array_equal(absum, wabs)


def test_grouped_g32_matches_block_oracle_when_groups_share_a_scale():
    # every expert's rows of B share one scale per 128x128 block and K block, and A's four
    # 32-groups of a 128-block share one scale: the C implementation of the 128-block
    # grouped oracle must then agree
    m_idx = si.grouped_layout([50, 130, 7])
    m, n, k, E = m_idx.size, 200, 512, 3
    qa, sa, _, _ = _g32_operands(m, 8, k, seed=41)
    sa128 = sa[:, ::4].copy()
    rng = np.random.default_rng(42)
    qb = rng.integers(0, 0x7F, (E, n, k)).astype(np.uint8) | (rng.integers(0, 2, (E, n, k)) << 7).astype(np.uint8)
    sb_blk = np.ldexp(1.0, rng.integers(-3, 4, (E, -(-n // 128), k // 128))).astype(np.float32)
    sb32 = np.repeat(np.repeat(sb_blk, 128, axis=1)[:, :n], 4, axis=2)
    ref, _ = oracle.m_grouped_gemm_nt_g32(qa, np.repeat(sa128, 4, axis=1), qb, sb32, m_idx)
    want, _ = oracle.m_grouped_gemm_nt(qa, sa128, qb, sb_blk, m_idx)
    pad = m_idx < 0
    assert np.isnan(ref[pad]).all() and np.isnan(want[pad]).all()
    assert np.allclose(ref[~pad], want[~pad], rtol=1e-13, atol=0)
