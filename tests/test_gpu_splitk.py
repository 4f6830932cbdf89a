"""GPU parity of the split-K GEMM (gemm_fp8_nt_bf16_splitk) against the oracle's
fp64 reference: the product of "DeepGEMM Essentials", Parts 1 and 6 (per-token
1x128 LHS scales, 128x128 RHS block scales, fp32 promotion per K block).  For
m <= 64 the K blocks of all 128-column tiles are dealt out to the workgroups in
equal shares and a shared tile's partial sums are added in share order by a
second kernel; for m > 64 each 128x128 tile's K blocks are cut into 2-4
slices, one workgroup each, whose partial sums a second kernel adds in slice
order.

Tolerances are those of gemm_fp8_nt_bf16 (check_bf16_gemm): the split changes
only how the per-block fp32 additions are grouped, which the (KB + 20) 2^-24
sum|terms| term already covers.  The shapes walk the plan: 1 to 8 units a
share, shares inside one tile, across a tile boundary and over whole tiles,
a short last share, ragged n and every row count around the 16 / 32 / 64-row
kernels.  The workspace starts filled with NaN (its contents must not matter),
and a second call on it must give the same bits.
"""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, mfma_truncation_bound, sample_idx, say

pytestmark = pytest.mark.gpu


def _cast_operands(m, n, k, a_fmt=oracle.SF_FP32, scale=0.1):
    a = si.randn((m, k), si.SEED_A, scale)
    b = si.randn((n, k), si.SEED_B, scale)
    qa, sa = oracle.cast_per_token(si.host_array(a), 128, a_fmt)
    qb, sb = oracle.cast_per_block(si.host_array(b), oracle.SF_FP32)
    return qa, sa, qb, sb


def _to_dev_mn(sa: np.ndarray, dtype=torch.float32):
    m, u = sa.shape
    ld = -(-m // 4) * 4
    buf = torch.zeros((u, ld), dtype=dtype)
    buf[:, :m] = torch.from_numpy(np.ascontiguousarray(sa.T).view(np.int32 if dtype == torch.int32 else np.float32))
    return buf.cuda().t()[:m]


def _run_splitk(qa, sa, qb, sb, sa_fmt=fg.SF_FP32, calls=1):
    m, k = qa.shape
    n = qb.shape[0]
    A = torch.from_numpy(qa).cuda()
    B = torch.from_numpy(qb).cuda()
    sa_d = _to_dev_mn(sa, torch.int32 if sa_fmt == fg.SF_PACKED_UE8M0 else torch.float32)
    sb_d = torch.from_numpy(sb).cuda()
    ldd = -(-n // 8) * 8
    wsb = fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k)
    # the workspace's contents on entry must not matter: NaN
    ws = torch.full((max(wsb // 4, 1),), float("nan"), dtype=torch.float32, device="cuda")
    outs = []
    for c in range(calls):
        D = torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")
        say("gemm_fp8_nt_bf16_splitk", (m, n, k), "sa_fmt", sa_fmt, "workspace", wsb, "call", c)
        fg.gemm_fp8_nt_bf16_splitk(A, sa_d, B, sb_d, D[:, :n].view(torch.bfloat16), ws, sa_fmt)
        torch.cuda.synchronize()
        Dh = D.cpu().numpy().view(np.uint16)
        assert (Dh[:, n:] == 0x7FC0).all(), "padding columns of D were written"
        outs.append(Dh[:, :n])
    return outs


def _check(qa, sa, qb, sb, got, what):
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), qa.shape[1] // 128, what)


@pytest.mark.parametrize("m", [1, 64])
@pytest.mark.parametrize("nk", [(7168, 4096), (4096, 7168), (7168, 7168)])
def test_splitk_decode(gpu, m, nk):
    # the decode shapes: 1792 units in 256 shares of 7 (each tile shared by 5 or 6
    # workgroups), and 3136 units in 392 shares of 8; two calls give the same bits
    n, k = nk
    qa, sa, qb, sb = _cast_operands(m, n, k)
    got = _run_splitk(qa, sa, qb, sb, calls=2)
    assert np.array_equal(got[0], got[1]), "result differs between calls"
    _check(qa, sa, qb, sb, got[0], f"splitk decode {(m, n, k)}")


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 63, 64])
@pytest.mark.parametrize("nk", [(1000, 128), (200, 1152), (4096, 2176), (9000, 256), (7168, 1408), (7168, 6656),
                                (4096, 4224), (130, 384), (38400, 256), (40000, 128)])
def test_splitk_edges(gpu, m, nk):
    # (1000, 128): 8 one-unit shares, each a whole tile; (200, 1152): 18 shares of one
    # unit, tiles shared 9 ways; (4096, 2176): 544 units, shares of 3 crossing tiles;
    # (9000, 256): 142 one-unit shares; (7168, 1408): 616 units in shares of 3;
    # (7168, 6656): 2912 units in 364 shares of 8; (4096, 4224): 1056 units
    # in shares of 5, the last short; (130, 384): a 2-column last tile; (38400, 256):
    # shares of 3 over 2-block tiles, a whole tile stored before a shared one;
    # (40000, 128): shares of 2 whole one-block tiles, the last tile 64 columns wide
    n, k = nk
    qa, sa, qb, sb = _cast_operands(m, n, k)
    got = _run_splitk(qa, sa, qb, sb)[0]
    _check(qa, sa, qb, sb, got, f"splitk {(m, n, k)}")


@pytest.mark.parametrize("m", [3, 40])
def test_splitk_ue8m0_scales(gpu, m):
    # power-of-two LHS scales, unpacked floats and packed words, give the same bits
    n, k = 384, 2048
    qa, words, qb, sb = _cast_operands(m, n, k, a_fmt=oracle.SF_PACKED_UE8M0)
    sa = oracle.unpack_ue8m0(words, k // 128)
    got = _run_splitk(qa, words, qb, sb, sa_fmt=fg.SF_PACKED_UE8M0)[0]
    _check(qa, sa, qb, sb, got, f"splitk packed ue8m0 m={m}")
    assert np.array_equal(got, _run_splitk(qa, sa, qb, sb, sa_fmt=fg.SF_UE8M0)[0])


@pytest.mark.parametrize("mnk", [(37, 520, 2560), (200, 520, 4096), (130, 260, 2176)])
def test_splitk_one_hot(gpu, mnk):
    # one nonzero K position per row: each output is a single product a*b*sa*sb, exact in
    # bf16 here, so a wrong row, K block, split or 128-column scale block shows as a
    # wrong value (scales distinct per row, K block and column block).  m = 200 and 130
    # take the K slices (4 slices of 8 blocks; 2 slices of 8 and 9 blocks).
    m, n, k = mnk
    KB = k // 128
    rng = np.random.default_rng(7)
    qa = np.zeros((m, k), np.uint8)
    pos = rng.integers(0, k, m)
    qa[np.arange(m), pos] = 0x38  # 1.0
    qb = np.full((n, k), 0x40, np.uint8)  # 2.0
    sa = np.ldexp(1.0, rng.integers(-4, 5, (m, KB))).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-4, 5, (-(-n // 128), KB))).astype(np.float32)
    got = _run_splitk(qa, sa, qb, sb)[0]
    want = 2.0 * sa[np.arange(m), pos // 128][:, None] * sb[np.arange(n) // 128][:, pos // 128].T
    want_bits = (want.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(got, want_bits)


# m > 64: K slices of 128x128 tiles.  (130, 300, 2176): 17 K blocks in slices of 8 and
# 9, ragged m and n; (65, 130, 3200): 25 K blocks in 3 slices, a 2-column last tile;
# (300, 520, 4096): 15 tiles in 4 slices; (200, 1000, 2048): 16 tiles in 2 slices;
# (512, 256, 2048): whole tiles only.  Two calls give the same bits.
@pytest.mark.parametrize("mnk", [(130, 300, 2176), (65, 130, 3200), (300, 520, 4096), (200, 1000, 2048),
                                 (512, 256, 2048)])
def test_splitk_kslices(gpu, mnk):
    qa, sa, qb, sb = _cast_operands(*mnk)
    assert fg.gemm_fp8_nt_bf16_splitk_workspace(*mnk) > 0
    got = _run_splitk(qa, sa, qb, sb, calls=2)
    assert np.array_equal(got[0], got[1]), "result differs between calls"
    _check(qa, sa, qb, sb, got[0], f"splitk kslices {mnk}")


@pytest.mark.parametrize("nk", [(4096, 7168), (2048, 7168)])
def test_splitk_kslices_m512(gpu, nk):
    # m = 512: 128 tiles in 4 slices (the whole 32 MiB of slots), 64 tiles in 4;
    # 20,000 sampled outputs plus tile corners
    m, (n, k) = 512, nk
    qa, sa, qb, sb = _cast_operands(m, n, k)
    got = _run_splitk(qa, sa, qb, sb)[0]
    ii, jj = sample_idx(m, n, 20000, 3)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb, idx=(ii, jj))
    check_bf16_gemm(got[ii, jj], ref, absum, mfma_truncation_bound(qa, sa, qb, sb, idx=(ii, jj)), k // 128,
                    f"splitk kslices {(m, n, k)}")


def test_splitk_kslices_ue8m0_scales(gpu):
    # packed words and unpacked powers of two give the same bits through the K slices
    m, n, k = 257, 384, 4096
    qa, words, qb, sb = _cast_operands(m, n, k, a_fmt=oracle.SF_PACKED_UE8M0)
    sa = oracle.unpack_ue8m0(words, k // 128)
    got = _run_splitk(qa, words, qb, sb, sa_fmt=fg.SF_PACKED_UE8M0)[0]
    _check(qa, sa, qb, sb, got, f"splitk kslices packed ue8m0 {(m, n, k)}")
    assert np.array_equal(got, _run_splitk(qa, sa, qb, sb, sa_fmt=fg.SF_UE8M0)[0])


@pytest.mark.parametrize("mnk", [(1024, 512, 1024), (65, 256, 256), (512, 7168, 4096)])
def test_splitk_plain_when_no_slices(gpu, mnk):
    # too few K blocks for two slices of 8, or more than 128 tiles: no workspace,
    # gemm_fp8_nt_bf16's kernels and bits
    m, n, k = mnk
    assert fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k) == 0
    qa, sa, qb, sb = _cast_operands(m, n, k)
    got = _run_splitk(qa, sa, qb, sb)[0]
    D = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    say("gemm_fp8_nt_bf16", (m, n, k))
    fg.gemm_fp8_nt_bf16(torch.from_numpy(qa).cuda(), _to_dev_mn(sa), torch.from_numpy(qb).cuda(),
                        torch.from_numpy(sb).cuda(), D)
    torch.cuda.synchronize()
    assert np.array_equal(got, D.view(torch.int16).cpu().numpy().view(np.uint16))
