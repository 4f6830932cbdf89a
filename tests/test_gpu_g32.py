"""GPU parity of the UE8M0 group-32 GEMM (both operands scaled per row and
32-wide K group by powers of two, applied by the gfx950 scaled FP8 MFMA)
against the oracle's fp64 definition.  Tolerance: 2 bf16 ulps + the fp32
accumulation bound with one rounding per run of 8 K products (the MFMA
accumulates all of K in fp32) + the MFMA's run-truncation bound with the
group-32 scales; normalised Frobenius error <= 1e-3."""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, check_wgrad, mfma_truncation_bound, sample_idx, say

pytestmark = pytest.mark.gpu


def _operands(m, n, k, scale=1.0, seeds=(si.SEED_A, si.SEED_B)):
    qa, wa = oracle.cast_per_token(si.host_array(si.randn((m, k), seeds[0], scale)), 32, oracle.SF_PACKED_UE8M0)
    qb, wb = oracle.cast_per_token(si.host_array(si.randn((n, k), seeds[1], scale)), 32, oracle.SF_PACKED_UE8M0)
    return qa, wa, qb, wb


def _dev_words(w):
    r, u = w.shape
    ld = -(-r // 4) * 4
    buf = torch.zeros((u, ld), dtype=torch.int32)
    buf[:, :r] = torch.from_numpy(np.ascontiguousarray(w.T).view(np.int32))
    return buf.cuda().t()[:r]


def _run(qa, wa, qb, wb):
    m, k = qa.shape
    n = qb.shape[0]
    ldd = -(-n // 8) * 8
    D = torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")
    say("gemm_fp8_nt_bf16_ue8m0_g32", (m, n, k))
    fg.gemm_fp8_nt_bf16_ue8m0_g32(torch.from_numpy(qa).cuda(), _dev_words(wa), torch.from_numpy(qb).cuda(),
                                  _dev_words(wb), D[:, :n].view(torch.bfloat16))
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, n:] == 0x7FC0).all()
    return Dh[:, :n]


@pytest.mark.parametrize("mnk", [(128, 256, 512), (1, 128, 128), (129, 200, 256), (257, 130, 640),
                                 (64, 1000, 1024), (256, 384, 7168), (128 * 600, 100, 128)])
def test_g32_full_compare(gpu, mnk):
    # the last shape: 600 tiles in one column, more than one round, so the first
    # round reads B (100 one-chunk rows) ahead of its K loop
    qa, wa, qb, wb = _operands(*mnk)
    k = mnk[2]
    sa, sb = oracle.unpack_ue8m0(wa, k // 32), oracle.unpack_ue8m0(wb, k // 32)
    got = _run(qa, wa, qb, wb)
    ref, absum = oracle.gemm_nt_g32(qa, sa, qb, sb)
    tb = mfma_truncation_bound(qa, sa, qb, sb, sb_block=False, group=32)
    check_bf16_gemm(got, ref, absum, tb, k // 8, f"g32 {mnk}")


def test_g32_closed_form_pins_group_scales(gpu):
    # all-ones operands; every (row, 32-group) and (column, 32-group) has its own power of two
    m, n, k = 130, 260, 512
    rng = np.random.default_rng(21)
    ea = rng.integers(-4, 5, (m, k // 32))
    eb = rng.integers(-4, 5, (n, k // 32))
    pack = lambda e: (e + 127).astype(np.uint32).reshape(e.shape[0], -1, 4) @ (1 << (8 * np.arange(4, dtype=np.uint32)))
    wa, wb = pack(ea).astype(np.uint32), pack(eb).astype(np.uint32)
    qa = np.full((m, k), 0x38, np.uint8)
    qb = np.full((n, k), 0x38, np.uint8)
    got = oracle.bf16_bits_to_f32(_run(qa, wa, qb, wb)).astype(np.float64)
    want = (np.ldexp(1.0, ea)[:, None, :] * np.ldexp(1.0, eb)[None, :, :]).sum(axis=2) * 32
    assert np.array_equal(got, oracle.bf16_bits_to_f32(oracle.round_bf16(want)).astype(np.float64))


# One or two full rounds of 256x256 tiles (256 to 512) and 8 K blocks: the wide kernel,
# whose lane (r, h) of the block's MFMA s carries 16-byte K chunks 4s + h and 4s + 2 + h
# under the exponent of group 2s + h.  Ragged: 4100 rows, 4000 and 3900 columns.
@pytest.mark.parametrize("mnk", [(4100, 4000, 1024), (4100, 3900, 1152), (4096, 4096, 1024), (4097, 3902, 1024)])
def test_g32_wide_sampled(gpu, mnk):
    m, n, k = mnk
    qa, wa, qb, wb = _operands(m, n, k, scale=0.1)
    sa, sb = oracle.unpack_ue8m0(wa, k // 32), oracle.unpack_ue8m0(wb, k // 32)
    got = _run(qa, wa, qb, wb)
    ii, jj = sample_idx(m, n, 20000, 14)
    ref, absum = oracle.gemm_nt_g32(qa, sa, qb, sb, idx=(ii, jj))
    tb = mfma_truncation_bound(qa, sa, qb, sb, sb_block=False, idx=(ii, jj), group=32)
    check_bf16_gemm(got[ii, jj], ref, absum, tb, k // 8, f"g32 wide {mnk}")


def test_g32_wide_closed_form(gpu):
    # all-ones operands, a distinct power of two per (row, 32-K group) and (column, group):
    # every output is 32 * sum_g 2^(ea + eb), exact in fp32, so the lane-to-group
    # exponent mapping of the wide kernel is pinned exactly
    m, n, k = 4100, 3900, 1024
    rng = np.random.default_rng(27)
    ea = rng.integers(-4, 5, (m, k // 32))
    eb = rng.integers(-4, 5, (n, k // 32))
    pack = lambda e: (e + 127).astype(np.uint32).reshape(e.shape[0], -1, 4) @ (1 << (8 * np.arange(4, dtype=np.uint32)))
    wa, wb = pack(ea).astype(np.uint32), pack(eb).astype(np.uint32)
    got = oracle.bf16_bits_to_f32(_run(np.full((m, k), 0x38, np.uint8), wa, np.full((n, k), 0x38, np.uint8), wb))
    want = 32 * (np.ldexp(1.0, ea) @ np.ldexp(1.0, eb).T)
    assert np.array_equal(got.astype(np.float64), oracle.bf16_bits_to_f32(oracle.round_bf16(want)).astype(np.float64))


def test_g32_wide_matches_128_tiles(gpu):
    # the m-grouped group-32 GEMM with one expert computes the same product on the
    # 128x128 kernel; the wide kernel must give the same bits
    m, n, k = 4100, 3900, 1024
    qa, wa, qb, wb = _operands(m, n, k, scale=0.1)
    wide = _run(qa, wa, qb, wb)
    sbw = torch.zeros((1, k // 128, -(-n // 4) * 4), dtype=torch.int32)
    sbw[0, :, :n] = torch.from_numpy(np.ascontiguousarray(wb.T).view(np.int32))
    sb3 = sbw.cuda().transpose(1, 2)[:, :n]          # [1, n, k/128], stride(1) == 1
    D = torch.full((m, -(-n // 8) * 8), 0x7FC0, dtype=torch.int16, device="cuda")
    say("m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous one expert", (m, n, k))
    fg.m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(torch.from_numpy(qa).cuda(), _dev_words(wa),
                                                        torch.from_numpy(qb).cuda()[None], sb3,
                                                        torch.zeros(m, dtype=torch.int32, device="cuda"),
                                                        D[:, :n].view(torch.bfloat16))
    torch.cuda.synchronize()
    tiles128 = D.cpu().numpy().view(np.uint16)[:, :n]
    assert np.array_equal(wide, tiles128)


def test_g32_prefill_sampled(gpu):
    m, n, k = 4096, 7168, 7168
    qa, wa, qb, wb = _operands(m, n, k, scale=0.1)
    sa, sb = oracle.unpack_ue8m0(wa, k // 32), oracle.unpack_ue8m0(wb, k // 32)
    got = _run(qa, wa, qb, wb)
    rng = np.random.default_rng(4)
    ii = np.concatenate([rng.integers(0, m, 20000), [0, m - 1, 127, 128]])
    jj = np.concatenate([rng.integers(0, n, 20000), [0, n - 1, 128, 127]])
    ref, absum = oracle.gemm_nt_g32(qa, sa, qb, sb, idx=(ii, jj))
    tb = mfma_truncation_bound(qa, sa, qb, sb, sb_block=False, idx=(ii, jj), group=32)
    check_bf16_gemm(got[ii, jj], ref, absum, tb, k // 8, f"g32 prefill {(m, n, k)}")


# weight gradient in the group-32 recipe: D += (A*sa)(B*sb)^T in fp32, K over tokens.
# Tolerance per element: (K/8 + 20) 2^-24 (sum|terms| + |D_in|) + the MFMA's
# run-truncation bound with the group-32 scales (same derivation as the fp32-scale
# wgrad, with one fp32 rounding per run of 8 tokens).

def _wgrad_operands(tokens, d_out, d_in):
    dy = si.host_array(si.randn((tokens, d_out), si.SEED_DY))
    x = si.host_array(si.randn((tokens, d_in), si.SEED_A))
    qa, wa = oracle.cast_per_token(dy, 32, oracle.SF_PACKED_UE8M0, transpose=True)   # [d_out, tokens]
    qb, wb = oracle.cast_per_token(x, 32, oracle.SF_PACKED_UE8M0, transpose=True)    # [d_in, tokens]
    return qa, wa, qb, wb


def _run_wgrad(qa, wa, qb, wb, d_in_np, times=1):
    m, k = qa.shape
    n = qb.shape[0]
    ldd = -(-n // 4) * 4 + 4
    D = torch.full((m, ldd), -1.0, dtype=torch.float32)
    D[:, :n] = torch.from_numpy(d_in_np)
    Dd = D.cuda()
    A, B, sa, sb = torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda(), _dev_words(wa), _dev_words(wb)
    for _ in range(times):
        say("wgrad_gemm_fp8_nt_fp32_ue8m0_g32", (m, n, k))
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0_g32(A, sa, B, sb, Dd[:, :n])
    torch.cuda.synchronize()
    out = Dd.cpu().numpy()
    assert (out[:, n:] == -1.0).all()
    return out[:, :n]


@pytest.mark.parametrize("shape", [(256, 512, 1024), (384, 130, 200), (1024, 256, 128), (384, 250, 38360),
                                   (128, 128 * 600, 100)])
def test_wgrad_g32_full_compare(gpu, shape):
    tokens, d_out, d_in = shape
    qa, wa, qb, wb = _wgrad_operands(tokens, d_out, d_in)
    sa, sb = oracle.unpack_ue8m0(wa, tokens // 32), oracle.unpack_ue8m0(wb, tokens // 32)
    d_in_np = si.randn((d_out, d_in), 7, 0.1, torch.float32).numpy()
    got = _run_wgrad(qa, wa, qb, wb, d_in_np)
    ref, absum = oracle.wgrad_nt_g32(qa, sa, qb, sb, d_in_np)
    check_wgrad(got, ref, absum, tokens // 32, f"wgrad g32 {shape}")


def test_wgrad_g32_closed_form_accumulates(gpu):
    # all-ones operands with a power of two per (row, 32-group) and (column, 32-group):
    # every partial sum is exact, so two calls give D_in + 2 * closed form exactly
    m, n, k = 130, 260, 512
    rng = np.random.default_rng(23)
    ea = rng.integers(-4, 5, (m, k // 32))
    eb = rng.integers(-4, 5, (n, k // 32))
    pack = lambda e: (e + 127).astype(np.uint32).reshape(e.shape[0], -1, 4) @ (1 << (8 * np.arange(4, dtype=np.uint32)))
    wa, wb = pack(ea).astype(np.uint32), pack(eb).astype(np.uint32)
    d_in = rng.integers(-64, 65, (m, n)).astype(np.float32)
    got = _run_wgrad(np.full((m, k), 0x38, np.uint8), wa, np.full((n, k), 0x38, np.uint8), wb, d_in, times=2)
    want = d_in.astype(np.float64) + 2 * 32 * (np.ldexp(1.0, ea)[:, None, :] * np.ldexp(1.0, eb)[None, :, :]).sum(axis=2)
    assert np.array_equal(got.astype(np.float64), want)


def test_wgrad_g32_linear_size_sampled(gpu):
    tokens, d_out, d_in = si.LINEAR["tokens"], si.LINEAR["d_out"], si.LINEAR["d_in"]
    qa, wa, qb, wb = _wgrad_operands(tokens, d_out, d_in)
    sa, sb = oracle.unpack_ue8m0(wa, tokens // 32), oracle.unpack_ue8m0(wb, tokens // 32)
    zero = np.zeros((d_out, d_in), np.float32)
    got = _run_wgrad(qa, wa, qb, wb, zero)
    rng = np.random.default_rng(9)
    ii = np.concatenate([rng.integers(0, d_out, 20000), [0, d_out - 1, 127, 128]])
    jj = np.concatenate([rng.integers(0, d_in, 20000), [0, d_in - 1, 128, 127]])
    ref, absum = oracle.wgrad_nt_g32(qa, sa, qb, sb, zero, idx=(ii, jj))
    check_wgrad(got[ii, jj], ref, absum, tokens // 32, "wgrad g32 4096x7168x8192")


# m-grouped contiguous GEMM in the group-32 recipe: rows of expert e use B[e] and its
# per-row group-32 scales; padding rows (-1) must stay untouched.

def _grouped_operands(m_idx, E, n, k, seed):
    m = m_idx.size
    qa, wa = oracle.cast_per_token(si.host_array(si.randn((m, k), seed, 0.1)), 32, oracle.SF_PACKED_UE8M0)
    qb = np.empty((E, n, k), np.uint8)
    wb = np.empty((E, n, k // 128), np.uint32)
    for e in range(E):
        qb[e], wb[e] = oracle.cast_per_token(si.host_array(si.randn((n, k), seed + 1 + e, 0.1)), 32,
                                             oracle.SF_PACKED_UE8M0)
    return qa, wa, qb, wb


def _run_grouped(qa, wa, qb, wb, m_idx):
    m, k = qa.shape
    E, n = qb.shape[0], qb.shape[1]
    ld = -(-n // 4) * 4 + 4
    sb = torch.zeros((E, k // 128, ld), dtype=torch.int32)
    sb[:, :, :n] = torch.from_numpy(np.ascontiguousarray(wb.transpose(0, 2, 1)).view(np.int32))
    sb = sb.cuda().permute(0, 2, 1)[:, :n]
    ldd = -(-n // 8) * 8
    D = torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")
    say("m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous", (m, n, k), "experts", E)
    fg.m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(
        torch.from_numpy(qa).cuda(), _dev_words(wa), torch.from_numpy(qb).cuda(), sb,
        torch.from_numpy(m_idx).cuda(), D[:, :n].view(torch.bfloat16))
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, n:] == 0x7FC0).all()
    return Dh[:, :n]


@pytest.mark.parametrize("tokens,n,k", [(si.MOE_TOKENS_4, 256, 512), (si.MOE_TOKENS_8, 200, 384),
                                        ([1, 300, 0, 129], 130, 256)])
def test_grouped_g32_full_compare(gpu, tokens, n, k):
    m_idx = si.grouped_layout(tokens)
    E = len(tokens)
    qa, wa, qb, wb = _grouped_operands(m_idx, E, n, k, seed=50)
    got = _run_grouped(qa, wa, qb, wb, m_idx)
    sa = oracle.unpack_ue8m0(wa, k // 32)
    sb = np.stack([oracle.unpack_ue8m0(wb[e], k // 32) for e in range(E)])
    ref, absum = oracle.m_grouped_gemm_nt_g32(qa, sa, qb, sb, m_idx)
    pad = m_idx < 0
    assert (got[pad] == 0x7FC0).all(), "padding rows were written"
    valid = np.nonzero(~pad)[0]
    tb = np.zeros((valid.size, n))
    for e in range(E):
        rows = np.nonzero(m_idx[valid] == e)[0]
        if rows.size:
            tb[rows] = mfma_truncation_bound(qa[valid[rows]], sa[valid[rows]], qb[e], sb[e], sb_block=False, group=32)
    check_bf16_gemm(got[valid], ref[valid], absum[valid], tb, k // 8, f"grouped g32 {tokens}")


def test_grouped_g32_all_padding_writes_nothing(gpu):
    m_idx = np.full(256, -1, np.int32)
    qa, wa, qb, wb = _grouped_operands(m_idx, 3, 256, 384, seed=13)
    got = _run_grouped(qa, wa, qb, wb, m_idx)
    assert (got == 0x7FC0).all()
