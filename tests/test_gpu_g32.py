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
from gpu_util import check_bf16_gemm, mfma_truncation_bound, say

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
                                 (64, 1000, 1024), (256, 384, 7168)])
def test_g32_full_compare(gpu, mnk):
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
