"""GPU parity of the GEMM with the per-token cast of its output fused into the
epilogue (gemm_fp8_nt_bf16_cast).

Exact-arithmetic inputs: E4M3 codes for +-0.5, +-1, +-2 and 0, and scales in
{0.5, 1, 2}.  Every product, MFMA run sum, promotion and accumulation is then
exact in fp32, so the GPU's bf16 output equals the oracle's bf16-rounded fp64
GEMM bit for bit, and the fused FP8 output must equal the oracle's 1x128
per-token cast of it ("DeepGEMM Essentials", Part 3) bit for bit.  On randn
data the bf16 output is checked to the GEMM tolerance, and the FP8 output must
equal the oracle's per-token cast of that bf16 output, bit for bit (the fused
cast is defined as the cast of the stored output, whatever its rounding)."""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, mfma_truncation_bound, say

pytestmark = pytest.mark.gpu

CODES = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)   # 0, +-0.5, +-1, +-2


def _exact_operands(m, n, k, seed):
    rng = np.random.default_rng(seed)
    qa = CODES[rng.integers(0, CODES.size, (m, k))]
    qb = CODES[rng.integers(0, CODES.size, (n, k))]
    qa[m // 3] = 0                                   # an all-zero output row: clamped groups
    sa = np.float32(2.0) ** rng.integers(-1, 2, (m, k // 128)).astype(np.float32)
    sb = np.float32(2.0) ** rng.integers(-1, 2, (-(-n // 128), k // 128)).astype(np.float32)
    return qa, sa.astype(np.float32), qb, sb.astype(np.float32)


def _dev_mn(sa):
    m, u = sa.shape
    ld = -(-m // 4) * 4
    buf = torch.zeros((u, ld), dtype=torch.float32)
    buf[:, :m] = torch.from_numpy(np.ascontiguousarray(sa.T))
    return buf.cuda().t()[:m]


def _run(qa, sa, qb, sb, fmt, with_d=True, mn_major=True):
    m, k = qa.shape
    n = qb.shape[0]
    G = -(-n // 128)
    ldd = -(-n // 8) * 8
    q_ld = -(-(n + 4) // 4) * 4
    D = torch.full((m, ldd), 0x7FC0, dtype=torch.int16, device="cuda")
    qbuf = torch.full((m, q_ld), 0xA5, dtype=torch.uint8, device="cuda")
    if mn_major:
        sbuf = torch.full((G, -(-(m + 4) // 4) * 4), -7, dtype=torch.int32, device="cuda")
        qsf = sbuf.view(torch.float32).t()[:m]
    else:
        sbuf = torch.full((m, G + 2), -7, dtype=torch.int32, device="cuda")
        qsf = sbuf.view(torch.float32)[:, :G]
    say("gemm_fp8_nt_bf16_cast", (m, n, k), "fmt", fmt, "D", with_d, "mn", mn_major)
    fg.gemm_fp8_nt_bf16_cast(torch.from_numpy(qa).cuda(), _dev_mn(sa), torch.from_numpy(qb).cuda(),
                             torch.from_numpy(sb).cuda(), D[:, :n].view(torch.bfloat16) if with_d else None,
                             qbuf[:, :n], qsf, q_sf_fmt=fmt)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy().view(np.uint16)
    qb_h = qbuf.cpu().numpy()
    assert (qb_h[:, n:] == 0xA5).all(), "q written outside its view"
    sb_h = sbuf.cpu().numpy()
    assert ((sb_h[:, m:] if mn_major else sb_h[:, G:]) == -7).all(), "scales written outside their view"
    if with_d:
        assert (Dh[:, n:] == 0x7FC0).all()
    else:
        assert (Dh == 0x7FC0).all(), "D written although not requested"
    return Dh[:, :n], qb_h[:, :n], qsf.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("mnk", [(128, 128, 256), (300, 520, 1024), (129, 200, 384), (1, 256, 128), (64, 130, 512)])
@pytest.mark.parametrize("fmt", [oracle.SF_FP32, oracle.SF_UE8M0], ids=["fp32", "ue8m0"])
def test_fused_cast_exact_inputs(gpu, mnk, fmt):
    qa, sa, qb, sb = _exact_operands(*mnk, seed=sum(mnk))
    d, q, sf = _run(qa, sa, qb, sb, fmt)
    ref, _ = oracle.gemm_nt(qa, sa, qb, sb)
    y = oracle.round_bf16(ref)                       # bf16 bits of the exact GEMM
    assert np.array_equal(d, y), "bf16 output differs from the exact GEMM"
    oq, osf = oracle.cast_per_token(y, 128, fmt)
    assert np.array_equal(q, oq), "fused E4M3 bytes differ from the per-token cast of the output"
    assert np.array_equal(sf, osf.view(np.uint32)), "fused scales differ"


def test_fused_cast_without_bf16_output_and_row_major_scales(gpu):
    qa, sa, qb, sb = _exact_operands(256, 384, 512, seed=11)
    _, q, sf = _run(qa, sa, qb, sb, oracle.SF_FP32, with_d=False, mn_major=False)
    y = oracle.round_bf16(oracle.gemm_nt(qa, sa, qb, sb)[0])
    oq, osf = oracle.cast_per_token(y, 128, oracle.SF_FP32)
    assert np.array_equal(q, oq) and np.array_equal(sf, osf.view(np.uint32))


@pytest.mark.parametrize("fmt", [oracle.SF_FP32, oracle.SF_UE8M0], ids=["fp32", "ue8m0"])
def test_fused_cast_randn(gpu, fmt):
    # the bf16 output is checked against the oracle's GEMM to the GEMM tolerance; the
    # fused FP8 output is by definition the per-token cast of that stored output, so
    # it must equal the oracle's cast of the GPU's own D, byte for byte and bit for bit
    m, n, k = 512, 1000, 2048
    qa, sa = oracle.cast_per_token(si.host_array(si.randn((m, k), si.SEED_A, 0.1)), 128, oracle.SF_FP32)
    qb, sb = oracle.cast_per_block(si.host_array(si.randn((n, k), si.SEED_B, 0.1)), oracle.SF_FP32)
    d, q, sf = _run(qa, sa, qb, sb, fmt)
    ref, absum = oracle.gemm_nt(qa, sa, qb, sb)
    check_bf16_gemm(d, ref, absum, mfma_truncation_bound(qa, sa, qb, sb), k // 128, f"fused-cast gemm fmt {fmt}")
    oq, osf = oracle.cast_per_token(np.ascontiguousarray(d), 128, fmt)
    assert np.array_equal(q, oq), "fused E4M3 bytes differ from the per-token cast of the stored output"
    assert np.array_equal(sf, osf.view(np.uint32)), "fused scales differ from the per-token cast of the stored output"
