"""GPU parity of the block-scaled NT GEMM and the wgrad GEMM against the
oracle's fp64 reference ("DeepGEMM Essentials", Parts 1, 6, 12-13; the
scale-row reply in "[Help] Starter script for nn.Linear for fwd,bwd").

Tolerances, derived from the arithmetic of the path.  The gfx950 FP8 MFMA
sums each run of 8 consecutive K products after aligning them to the run's
largest exponent sum with 13 fraction bits (truncating toward zero) and adds
the run sums in fp32 (measured on the hardware; see mfma_truncation_bound).
* bf16 output, per element: |g - ref| <= 2 ulp_bf16(ref)
  + (KB + 20) 2^-24 sum|terms| + the MFMA truncation bound;
  ||g - bf16(ref)|| / ||bf16(ref)|| <= 1e-3; and at most 2 + 0.25% of the
  outputs beyond 2 ulps of ref itself (check_bf16_gemm).
* wgrad fp32 (block sums on the f16 / bf16 MFMA, exact to fp32 rounding), per
  element: |g - ref| <= (roundings + 20) 2^-24 (sum|terms| + |D_in|); and the
  relative Frobenius error ||g - ref|| / ||ref|| <= 1e-5 (check_wgrad).
"""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, check_wgrad, mfma_truncation_bound, sample_idx, say

pytestmark = pytest.mark.gpu


def _cast_operands(m, n, k, scale=1.0, a_fmt=oracle.SF_FP32, seeds=(si.SEED_A, si.SEED_B)):
    a = si.randn((m, k), seeds[0], scale)
    b = si.randn((n, k), seeds[1], scale)
    qa, sa = oracle.cast_per_token(si.host_array(a), 128, a_fmt)
    qb, sb = oracle.cast_per_block(si.host_array(b), oracle.SF_FP32)
    return qa, sa, qb, sb


def _to_dev_mn(sa: np.ndarray, dtype=torch.float32):
    """Host [m, units] scales -> device MN-major view (ld = align(m, 4))."""
    m, u = sa.shape
    ld = -(-m // 4) * 4
    buf = torch.zeros((u, ld), dtype=dtype)
    buf[:, :m] = torch.from_numpy(np.ascontiguousarray(sa.T).view(np.int32 if dtype == torch.int32 else np.float32))
    return buf.cuda().t()[:m]


def _run_gemm(qa, sa, qb, sb, sa_fmt=fg.SF_FP32):
    m, k = qa.shape
    n = qb.shape[0]
    A = torch.from_numpy(qa).cuda()
    B = torch.from_numpy(qb).cuda()
    sa_d = _to_dev_mn(sa, torch.int32 if sa_fmt == fg.SF_PACKED_UE8M0 else torch.float32)
    sb_d = torch.from_numpy(sb).cuda()
    ldd = -(-n // 8) * 8
    D = torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")
    say("gemm_fp8_nt_bf16", (m, n, k), "sa_fmt", sa_fmt)
    fg.gemm_fp8_nt_bf16(A, sa_d, B, sb_d, D[:, :n].view(torch.bfloat16), sa_fmt)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, n:] == 0x7FC0).all()
    return Dh[:, :n]


@pytest.mark.parametrize("mnk", [(128, 256, 512), (1, 128, 128), (129, 200, 256), (3, 300, 384),
                                 (257, 130, 640), (64, 1000, 1024), (256, 384, 7168)])
def test_gemm_full_compare(gpu, mnk):
    qa, sa, qb, sb = _cast_operands(*mnk)
    got = _run_gemm(qa, sa, qb, sb)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), mnk[2] // 128, f"gemm {mnk}")


def test_gemm_packed_ue8m0_lhs(gpu):
    m, n, k = 200, 256, 1024
    qa, words, qb, sb = _cast_operands(m, n, k, a_fmt=oracle.SF_PACKED_UE8M0)
    sa = oracle.unpack_ue8m0(words, k // 128)
    got = _run_gemm(qa, words, qb, sb, sa_fmt=fg.SF_PACKED_UE8M0)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128, "gemm packed sa")
    got2 = _run_gemm(qa, sa, qb, sb, sa_fmt=fg.SF_UE8M0)
    assert np.array_equal(got, got2)


def test_gemm_closed_form_all_ones(gpu):
    m, n, k = 130, 260, 384
    kb = k // 128
    qa = np.full((m, k), 0x38, np.uint8)
    qb = np.full((n, k), 0x38, np.uint8)
    pa = np.array([[(i % 5) - t for t in range(kb)] for i in range(m)])
    pb = np.array([[jb - (t % 2) for t in range(kb)] for jb in range(3)])
    sa = np.ldexp(np.float32(1), pa).astype(np.float32)
    sb = np.ldexp(np.float32(1), pb).astype(np.float32)
    got = oracle.bf16_bits_to_f32(_run_gemm(qa, sa, qb, sb)).astype(np.float64)
    want = np.array([[sum(128 * 2.0 ** (pa[i, t] + pb[j // 128, t]) for t in range(kb)) for j in range(n)]
                     for i in range(m)])
    assert np.array_equal(got, want)          # every value is exact in bf16


def test_gemm_one_hot_scale_indexing(gpu):
    m, n, k = 140, 300, 512
    rng = np.random.default_rng(3)
    sa = rng.uniform(0.5, 2, (m, k // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (3, k // 128)).astype(np.float32)
    qa = np.zeros((m, k), np.uint8)
    qb = np.zeros((n, k), np.uint8)
    hits = [(0, 0, 0), (139, 299, 511), (70, 130, 200), (5, 257, 129), (128, 128, 300)]
    for i0, j0, t0 in hits:
        qa[i0, t0] = 0x38
        qb[j0, t0] = 0x38
    got = oracle.bf16_bits_to_f32(_run_gemm(qa, sa, qb, sb)).astype(np.float64)
    ref, _ = oracle.gemm_nt(qa, sa, qb, sb)
    want = oracle.bf16_bits_to_f32(oracle.round_bf16(ref)).astype(np.float64)
    assert np.array_equal(got, want)



@pytest.mark.parametrize("mnk", [(1, 1, 128), (5, 1, 128), (64, 3, 1152), (130, 7, 256), (300, 17, 384),
                                 (256, 9, 1152)])
def test_gemm_tiny_n(gpu, mnk):
    # fewer columns than one 16-wide MFMA tile: the decode kernel (m <= 64), the 128x128
    # kernel and the two-K-chain kernel (2 tiles, 9 K blocks) with every B row past n clamped
    qa, sa, qb, sb = _cast_operands(*mnk)
    got = _run_gemm(qa, sa, qb, sb)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), mnk[2] // 128, f"gemm tiny n {mnk}")

@pytest.mark.parametrize("mnk", [(4096, 7168, 7168), (4096, 4096, 7168)])
def test_gemm_prefill_sampled(gpu, mnk):
    m, n, k = mnk
    qa, sa, qb, sb = _cast_operands(m, n, k, scale=0.1)
    got = _run_gemm(qa, sa, qb, sb)
    ii, jj = sample_idx(m, n, 20000, 1)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb, idx=(ii, jj))
    tb = mfma_truncation_bound(qa, sa, qb, sb, idx=(ii, jj))
    check_bf16_gemm(got[ii, jj], ref, absum, tb, k // 128, f"prefill {mnk}")
    assert np.isfinite(oracle.bf16_bits_to_f32(got)).all()


@pytest.mark.parametrize("m", [1, 64, 512])
@pytest.mark.parametrize("nk", [(7168, 4096), (4096, 7168)])
def test_gemm_decode(gpu, m, nk):
    n, k = nk
    qa, sa, qb, sb = _cast_operands(m, n, k, scale=0.1)
    got = _run_gemm(qa, sa, qb, sb)
    if m <= 64:
        ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
        check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128, f"decode {(m, n, k)}")
    else:
        ii, jj = sample_idx(m, n, 20000, 2)
        ref, absum = oracle.gemm_nt(qa, sa, qb, sb, idx=(ii, jj))
        tb = mfma_truncation_bound(qa, sa, qb, sb, idx=(ii, jj))
        check_bf16_gemm(got[ii, jj], ref, absum, tb, k // 128, f"decode {(m, n, k)}")


@pytest.mark.parametrize("mnk", [(512, 7168, 1024), (300, 700, 1152), (129, 130, 2176), (384, 1000, 4096)])
@pytest.mark.parametrize("fmt", [oracle.SF_FP32, oracle.SF_PACKED_UE8M0], ids=["fp32", "packed"])
def test_gemm_two_k_chains(gpu, mnk, fmt):
    # fewer 128x128 tiles than CUs and at least 8 K blocks: two groups of waves take the
    # even and the odd K blocks of each tile and add their sums at the end; 9 and 17 K
    # blocks leave the second group one step without a block
    m, n, k = mnk
    qa, sa, qb, sb = _cast_operands(m, n, k, scale=0.1, a_fmt=fmt)
    sa_f = oracle.unpack_ue8m0(sa, k // 128) if fmt == oracle.SF_PACKED_UE8M0 else sa
    got = _run_gemm(qa, sa, qb, sb, sa_fmt=fg.SF_PACKED_UE8M0 if fmt == oracle.SF_PACKED_UE8M0 else fg.SF_FP32)
    ref, absum = oracle.gemm_nt(qa, sa_f, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa_f, qb, sb), k // 128, f"two K chains {mnk} fmt {fmt}")


def test_gemm_two_k_chains_one_hot(gpu):
    # one nonzero K position per row, in an odd or an even K block: each output is one
    # product a*b*sa*sb (exact in bf16), so a block summed by the wrong group, twice or
    # not at all, or a wrong scale, shows as a wrong value
    m, n, k = 200, 300, 1152
    KB = k // 128
    rng = np.random.default_rng(11)
    qa = np.zeros((m, k), np.uint8)
    pos = rng.integers(0, k, m)
    qa[np.arange(m), pos] = 0x38  # 1.0
    qb = np.full((n, k), 0x40, np.uint8)  # 2.0
    sa = np.ldexp(1.0, rng.integers(-4, 5, (m, KB))).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-4, 5, (-(-n // 128), KB))).astype(np.float32)
    got = _run_gemm(qa, sa, qb, sb)
    want = 2.0 * sa[np.arange(m), pos // 128][:, None] * sb[np.arange(n) // 128][:, pos // 128].T
    want_bits = (want.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(got, want_bits)


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 63, 64, 65])
@pytest.mark.parametrize("nk", [(1000, 128), (200, 1152), (4096, 2176), (9000, 256), (7168, 1408)])
def test_gemm_skinny_edges(gpu, m, nk):
    # decode-sized m: every row count around the 16 / 32 / 64-row configurations,
    # ragged n, fewer K blocks than the waves that split them (k = 128) and an
    # uneven split (9 and 17 blocks over 8 or 16 waves).  n = 1000 and 200 take the
    # 16-wave 16-row configuration, n = 4096 with m > 32 the 16-wave 32-row one,
    # n = 7168 with m > 16 the 8-wave ones (or 16-wave 32-row for m <= 32), and
    # n = 9000 (282 column workgroups) the 8-wave ones for every m > 16.
    n, k = nk
    qa, sa, qb, sb = _cast_operands(m, n, k, scale=0.1)
    got = _run_gemm(qa, sa, qb, sb)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128, f"skinny {(m, n, k)}")


@pytest.mark.parametrize("m", [3, 40])
def test_gemm_skinny_packed_ue8m0(gpu, m):
    n, k = 384, 1024
    qa, words, qb, sb = _cast_operands(m, n, k, scale=0.1, a_fmt=oracle.SF_PACKED_UE8M0)
    sa = oracle.unpack_ue8m0(words, k // 128)
    got = _run_gemm(qa, words, qb, sb, sa_fmt=fg.SF_PACKED_UE8M0)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128, f"skinny packed m={m}")
    assert np.array_equal(got, _run_gemm(qa, sa, qb, sb, sa_fmt=fg.SF_UE8M0))


def test_gemm_skinny_one_hot(gpu):
    # one-hot K positions pin the skinny path's scale indexing (row, K block, 128-column block)
    m, n, k = 20, 300, 1280
    rng = np.random.default_rng(5)
    sa = rng.uniform(0.5, 2, (m, k // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (3, k // 128)).astype(np.float32)
    qa = np.zeros((m, k), np.uint8)
    qb = np.zeros((n, k), np.uint8)
    for i0, j0, t0 in [(0, 0, 0), (19, 299, 1279), (7, 130, 700), (16, 257, 129), (3, 128, 1151)]:
        qa[i0, t0] = 0x38
        qb[j0, t0] = 0x38
    got = oracle.bf16_bits_to_f32(_run_gemm(qa, sa, qb, sb)).astype(np.float64)
    ref, _ = oracle.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(got, oracle.bf16_bits_to_f32(oracle.round_bf16(ref)).astype(np.float64))


# ---------------------------------------------------------------------------
# More tiles than run at once (2 per CU): 250 x 38360 has 2 x 300 = 600 ragged
# tiles over 3 K blocks, so the XCD tile ranges, bands and both edges are exercised.
_MANY_MNK = (250, 38360, 384)


def test_gemm_many_ragged_tiles(gpu):
    qa, sa, qb, sb = _cast_operands(*_MANY_MNK)
    got = _run_gemm(qa, sa, qb, sb)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), _MANY_MNK[2] // 128,
                    f"gemm many ragged tiles {_MANY_MNK}")


def test_gemm_tall_thin_many_tiles(gpu):
    # 600 tiles in one column of tiles: more than one round, so the first round
    # reads B ahead of its K loop, and B (100 rows of one 1 KB chunk) is smaller
    # than the 512 shares of that read (most workgroups repeat its last chunk)
    m, n, k = 128 * 600, 100, 128
    qa, sa, qb, sb = _cast_operands(m, n, k)
    got = _run_gemm(qa, sa, qb, sb)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128, f"gemm tall thin {(m, n, k)}")


def test_gemm_many_ragged_tiles_packed_ue8m0(gpu):
    qa, words, qb, sb = _cast_operands(*_MANY_MNK, a_fmt=oracle.SF_PACKED_UE8M0)
    sa = oracle.unpack_ue8m0(words, _MANY_MNK[2] // 128)
    got = _run_gemm(qa, words, qb, sb, sa_fmt=fg.SF_PACKED_UE8M0)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), _MANY_MNK[2] // 128,
                    f"gemm many ragged tiles packed {_MANY_MNK}")


# wgrad
# ---------------------------------------------------------------------------

def _wgrad_operands(tokens, d_out, d_in):
    dy = si.randn((tokens, d_out), si.SEED_DY)
    x = si.randn((tokens, d_in), si.SEED_A)
    qa, sa = oracle.cast_per_token(si.host_array(dy), 128, oracle.SF_FP32, transpose=True)   # [d_out, tokens]
    qb, sb = oracle.cast_per_token(si.host_array(x), 128, oracle.SF_FP32, transpose=True)    # [d_in, tokens]
    return qa, sa, qb, sb


def _run_wgrad(qa, sa, qb, sb, d_in_np):
    m, k = qa.shape
    n = qb.shape[0]
    ldd = -(-n // 4) * 4 + 4
    D = torch.full((m, ldd), -1.0, dtype=torch.float32)
    D[:, :n] = torch.from_numpy(d_in_np)
    Dd = D.cuda()
    say("wgrad_gemm_fp8_nt_fp32", (m, n, k))
    fg.wgrad_gemm_fp8_nt_fp32(torch.from_numpy(qa).cuda(), _to_dev_mn(sa), torch.from_numpy(qb).cuda(),
                              _to_dev_mn(sb), Dd[:, :n])
    torch.cuda.synchronize()
    out = Dd.cpu().numpy()
    assert (out[:, n:] == -1.0).all()
    return out[:, :n]


@pytest.mark.parametrize("shape", [(256, 512, 1024), (384, 130, 200), (1024, 256, 128)])
def test_wgrad_full_compare(gpu, shape):
    tokens, d_out, d_in = shape
    qa, sa, qb, sb = _wgrad_operands(tokens, d_out, d_in)
    d_in_np = si.randn((d_out, d_in), 5, 0.1, torch.float32).numpy()
    got = _run_wgrad(qa, sa, qb, sb, d_in_np)
    ref, absum = oracle.wgrad_nt(qa, sa, qb, sb, d_in_np)
    check_wgrad(got, ref, absum, -(-tokens // 128), f"wgrad {shape}")



@pytest.mark.parametrize("shape", [(128, 1, 1), (256, 3, 130), (384, 130, 5)])
def test_wgrad_tiny(gpu, shape):
    # one output, a 3-row gradient over 130 columns, and 5 columns over 130 rows:
    # partial 4-column groups and rows past m or n clamped in the copies
    tokens, d_out, d_in = shape
    qa, sa, qb, sb = _wgrad_operands(tokens, d_out, d_in)
    d_in_np = si.randn((d_out, d_in), 7, 0.1, torch.float32).numpy()
    got = _run_wgrad(qa, sa, qb, sb, d_in_np)
    ref, absum = oracle.wgrad_nt(qa, sa, qb, sb, d_in_np)
    check_wgrad(got, ref, absum, -(-tokens // 128), f"wgrad tiny {shape}")

def test_wgrad_many_ragged_tiles(gpu):
    # d_out x d_in = 250 x 38360: 600 ragged tiles, 3 K blocks
    tokens, d_out, d_in = 384, 250, 38360
    qa, sa, qb, sb = _wgrad_operands(tokens, d_out, d_in)
    d_in_np = si.randn((d_out, d_in), 6, 0.1, torch.float32).numpy()
    got = _run_wgrad(qa, sa, qb, sb, d_in_np)
    ref, absum = oracle.wgrad_nt(qa, sa, qb, sb, d_in_np)
    check_wgrad(got, ref, absum, tokens // 128, "wgrad many ragged tiles (384, 250, 38360)")


def test_wgrad_linear_size_sampled(gpu):
    tokens, d_out, d_in = si.LINEAR["tokens"], si.LINEAR["d_out"], si.LINEAR["d_in"]
    qa, sa, qb, sb = _wgrad_operands(tokens, d_out, d_in)
    zero = np.zeros((d_out, d_in), np.float32)
    got = _run_wgrad(qa, sa, qb, sb, zero)
    ii, jj = sample_idx(d_out, d_in, 20000, 4)
    ref, absum = oracle.wgrad_nt(qa, sa, qb, sb, zero, idx=(ii, jj))
    check_wgrad(got[ii, jj], ref, absum, tokens // 128, "wgrad 4096x7168x8192")


# wgrad with UE8M0 1x128 scales on both operands (the cast's UE8M0 option): the powers of
# two are folded into the bf16 conversion and the bf16 MFMA accumulates all of K in
# fp32, so the fp32 accumulation term counts one rounding per MFMA of 32 tokens.

def _wgrad_operands_ue8m0(tokens, d_out, d_in, fmt):
    dy = si.randn((tokens, d_out), si.SEED_DY)
    x = si.randn((tokens, d_in), si.SEED_A)
    qa, sa = oracle.cast_per_token(si.host_array(dy), 128, fmt, transpose=True)
    qb, sb = oracle.cast_per_token(si.host_array(x), 128, fmt, transpose=True)
    return qa, sa, qb, sb


def _run_wgrad_ue8m0(qa, sa, qb, sb, d_in_np, fmt, times=1):
    m, k = qa.shape
    n = qb.shape[0]
    ldd = -(-n // 4) * 4 + 4
    D = torch.full((m, ldd), -1.0, dtype=torch.float32)
    D[:, :n] = torch.from_numpy(d_in_np)
    Dd = D.cuda()
    dt = torch.int32 if fmt == fg.SF_PACKED_UE8M0 else torch.float32
    A, B, sa_d, sb_d = torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda(), _to_dev_mn(sa, dt), _to_dev_mn(sb, dt)
    for _ in range(times):
        say("wgrad_gemm_fp8_nt_fp32_ue8m0", (m, n, k), "fmt", fmt)
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0(A, sa_d, B, sb_d, Dd[:, :n], fmt)
    torch.cuda.synchronize()
    out = Dd.cpu().numpy()
    assert (out[:, n:] == -1.0).all()
    return out[:, :n]


@pytest.mark.parametrize("shape", [(256, 512, 1024), (384, 130, 200), (1024, 256, 128), (640, 250, 38360)])
@pytest.mark.parametrize("fmt", [fg.SF_UE8M0, fg.SF_PACKED_UE8M0], ids=["ue8m0", "packed"])
def test_wgrad_ue8m0_full_compare(gpu, shape, fmt):
    tokens, d_out, d_in = shape
    qa, sa, qb, sb = _wgrad_operands_ue8m0(tokens, d_out, d_in, fmt)
    if fmt == fg.SF_PACKED_UE8M0:
        sa_v, sb_v = oracle.unpack_ue8m0(sa, tokens // 128), oracle.unpack_ue8m0(sb, tokens // 128)
    else:
        sa_v, sb_v = sa, sb
    d_in_np = si.randn((d_out, d_in), 8, 0.1, torch.float32).numpy()
    got = _run_wgrad_ue8m0(qa, sa, qb, sb, d_in_np, fmt)
    ref, absum = oracle.wgrad_nt(qa, sa_v, qb, sb_v, d_in_np)
    check_wgrad(got, ref, absum, tokens // 32, f"wgrad ue8m0 {shape} fmt {fmt}")


def test_wgrad_ue8m0_closed_form_accumulates(gpu):
    # all-ones operands with a power of two per (row, K block), |ea|, |eb| <= 3: every
    # partial sum the MFMAs form (a multiple of 32 * 2^-6 below 2^17) is exact in fp32,
    # so two calls give D_in + 2 * sum_kb 128 * 2^(ea + eb) exactly
    m, n, k = 130, 260, 640
    rng = np.random.default_rng(24)
    ea = rng.integers(-3, 4, (m, k // 128))
    eb = rng.integers(-3, 4, (n, k // 128))
    sa, sb = np.ldexp(1.0, ea).astype(np.float32), np.ldexp(1.0, eb).astype(np.float32)
    d_in = rng.integers(-64, 65, (m, n)).astype(np.float32)
    got = _run_wgrad_ue8m0(np.full((m, k), 0x38, np.uint8), sa, np.full((n, k), 0x38, np.uint8), sb, d_in,
                           fg.SF_UE8M0, times=2)
    want = d_in.astype(np.float64) + 2 * 128 * (np.ldexp(1.0, ea)[:, None, :] * np.ldexp(1.0, eb)[None, :, :]).sum(axis=2)
    assert np.array_equal(got.astype(np.float64), want)


def test_wgrad_ue8m0_linear_size_sampled(gpu):
    tokens, d_out, d_in = si.LINEAR["tokens"], si.LINEAR["d_out"], si.LINEAR["d_in"]
    qa, sa, qb, sb = _wgrad_operands_ue8m0(tokens, d_out, d_in, fg.SF_PACKED_UE8M0)
    sa_v, sb_v = oracle.unpack_ue8m0(sa, tokens // 128), oracle.unpack_ue8m0(sb, tokens // 128)
    zero = np.zeros((d_out, d_in), np.float32)
    got = _run_wgrad_ue8m0(qa, sa, qb, sb, zero, fg.SF_PACKED_UE8M0)
    ii, jj = sample_idx(d_out, d_in, 20000, 11)
    ref, absum = oracle.wgrad_nt(qa, sa_v, qb, sb_v, zero, idx=(ii, jj))
    check_wgrad(got[ii, jj], ref, absum, tokens // 32, "wgrad ue8m0 4096x7168x8192")


# forward GEMM with every scale a power of two (UE8M0 per-token A scales, UE8M0 128x128 B
# block scales), applied by the scaled MFMA: tolerance as the plain GEMM with one fp32
# rounding per run of 8 K products (K/8 + 20 in the accumulation term).

def _cast_operands_ue8m0(m, n, k, a_fmt, scale=1.0):
    a = si.randn((m, k), si.SEED_A, scale)
    b = si.randn((n, k), si.SEED_B, scale)
    qa, sa = oracle.cast_per_token(si.host_array(a), 128, a_fmt)
    qb, sb = oracle.cast_per_block(si.host_array(b), oracle.SF_UE8M0)
    return qa, sa, qb, sb


def _run_gemm_ue8m0(qa, sa, qb, sb, sa_fmt):
    m, k = qa.shape
    n = qb.shape[0]
    sa_d = _to_dev_mn(sa, torch.int32 if sa_fmt == fg.SF_PACKED_UE8M0 else torch.float32)
    ldd = -(-n // 8) * 8
    D = torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")
    say("gemm_fp8_nt_bf16_ue8m0", (m, n, k), "sa_fmt", sa_fmt)
    fg.gemm_fp8_nt_bf16_ue8m0(torch.from_numpy(qa).cuda(), sa_d, torch.from_numpy(qb).cuda(),
                              torch.from_numpy(sb).cuda(), D[:, :n].view(torch.bfloat16), sa_fmt)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    assert (Dh[:, n:] == 0x7FC0).all()
    return Dh[:, :n]


@pytest.mark.parametrize("mnk", [(128, 256, 512), (1, 128, 128), (129, 200, 256), (3, 300, 384), (257, 130, 640),
                                 (256, 384, 7168), (250, 38360, 384)])
@pytest.mark.parametrize("fmt", [fg.SF_UE8M0, fg.SF_PACKED_UE8M0], ids=["ue8m0", "packed"])
def test_gemm_ue8m0_full_compare(gpu, mnk, fmt):
    m, n, k = mnk
    qa, sa, qb, sb = _cast_operands_ue8m0(m, n, k, fmt)
    sa_v = oracle.unpack_ue8m0(sa, k // 128) if fmt == fg.SF_PACKED_UE8M0 else sa
    got = _run_gemm_ue8m0(qa, sa, qb, sb, fmt)
    ref, absum = oracle.gemm_nt(qa, sa_v, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa_v, qb, sb), k // 8, f"gemm ue8m0 {mnk}")


def test_gemm_ue8m0_closed_form_pins_scale_indexing(gpu):
    # all-ones operands; per-(row, K block) and per-(128-column block, K block) exponents
    m, n, k = 130, 300, 640
    rng = np.random.default_rng(25)
    ea = rng.integers(-5, 6, (m, k // 128))
    eb = rng.integers(-5, 6, (-(-n // 128), k // 128))
    sa, sb = np.ldexp(1.0, ea).astype(np.float32), np.ldexp(1.0, eb).astype(np.float32)
    got = oracle.bf16_bits_to_f32(_run_gemm_ue8m0(np.full((m, k), 0x38, np.uint8), sa, np.full((n, k), 0x38, np.uint8),
                                                  sb, fg.SF_UE8M0)).astype(np.float64)
    ebj = np.repeat(eb, 128, axis=0)[:n]
    want = 128 * (np.ldexp(1.0, ea)[:, None, :] * np.ldexp(1.0, ebj)[None, :, :]).sum(axis=2)
    assert np.array_equal(got, oracle.bf16_bits_to_f32(oracle.round_bf16(want)).astype(np.float64))


# One or two full rounds of 256x256 tiles (256 to 512) and 8 K blocks: the wide kernel
# (4 waves of 128x128 on the 32x32x64 scaled MFMA).  Ragged shapes: 4100 rows leave 4
# in the last tile row; 4000 columns leave 160 in the last tile column, across two
# B blocks; 3900 leave 60, so the tile's second B block lies past the matrix; 3902
# ends in a 2-column store (4097 rows: one row in the last tile row).
@pytest.mark.parametrize("mnk", [(4100, 4000, 1024), (4100, 3900, 1152), (4096, 4096, 1024), (4097, 3902, 1024)])
@pytest.mark.parametrize("fmt", [fg.SF_UE8M0, fg.SF_PACKED_UE8M0], ids=["ue8m0", "packed"])
def test_gemm_ue8m0_wide_sampled(gpu, mnk, fmt):
    m, n, k = mnk
    qa, sa, qb, sb = _cast_operands_ue8m0(m, n, k, fmt, scale=0.1)
    sa_v = oracle.unpack_ue8m0(sa, k // 128) if fmt == fg.SF_PACKED_UE8M0 else sa
    got = _run_gemm_ue8m0(qa, sa, qb, sb, fmt)
    ii, jj = sample_idx(m, n, 20000, 13)
    ref, absum = oracle.gemm_nt(qa, sa_v, qb, sb, idx=(ii, jj))
    tb = mfma_truncation_bound(qa, sa_v, qb, sb, idx=(ii, jj))
    check_bf16_gemm(got[ii, jj], ref, absum, tb, k // 8, f"gemm ue8m0 wide {mnk}")


@pytest.mark.parametrize("fmt", [fg.SF_UE8M0, fg.SF_PACKED_UE8M0], ids=["ue8m0", "packed"])
def test_gemm_ue8m0_wide_closed_form(gpu, fmt):
    # all-ones operands with per-(row, K block) and per-(128-column block, K block)
    # exponents: every output is 128 * sum_kb 2^(ea + eb), exact in fp32, so the wide
    # kernel's rows, columns, K halves and both B blocks of a tile are pinned exactly
    m, n, k = 4100, 3900, 1024
    KB = k // 128
    rng = np.random.default_rng(26)
    ea = rng.integers(-5, 6, (m, KB))
    eb = rng.integers(-5, 6, (-(-n // 128), KB))
    if fmt == fg.SF_PACKED_UE8M0:
        bytes_ = (ea + 127).astype(np.uint32)
        sa = (bytes_.reshape(m, -1, 4) << (8 * np.arange(4, dtype=np.uint32))).sum(axis=2).astype(np.uint32)
    else:
        sa = np.ldexp(1.0, ea).astype(np.float32)
    sb = np.ldexp(1.0, eb).astype(np.float32)
    got = oracle.bf16_bits_to_f32(_run_gemm_ue8m0(np.full((m, k), 0x38, np.uint8), sa, np.full((n, k), 0x38, np.uint8),
                                                  sb, fmt)).astype(np.float64)
    want = 128 * (np.ldexp(1.0, ea) @ np.ldexp(1.0, eb).T)    # [m, n blocks], exact in fp64
    want = np.repeat(want, 128, axis=1)[:, :n]
    assert np.array_equal(got, oracle.bf16_bits_to_f32(oracle.round_bf16(want)).astype(np.float64))


def test_gemm_ue8m0_prefill_sampled(gpu):
    m, n, k = 4096, 7168, 7168
    qa, sa, qb, sb = _cast_operands_ue8m0(m, n, k, fg.SF_PACKED_UE8M0, scale=0.1)
    sa_v = oracle.unpack_ue8m0(sa, k // 128)
    got = _run_gemm_ue8m0(qa, sa, qb, sb, fg.SF_PACKED_UE8M0)
    ii, jj = sample_idx(m, n, 20000, 12)
    ref, absum = oracle.gemm_nt(qa, sa_v, qb, sb, idx=(ii, jj))
    tb = mfma_truncation_bound(qa, sa_v, qb, sb, idx=(ii, jj))
    check_bf16_gemm(got[ii, jj], ref, absum, tb, k // 8, "gemm ue8m0 prefill")
