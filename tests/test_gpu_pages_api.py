"""GPU parity of fine_grained_block_token_amd.api, the calls in the form the pages write
them: cast the operands, pass the LHS scales through get_col_major_tma_aligned_tensor,
call the GEMM on (fp8, scales) tuples ("DeepGEMM Essentials", Parts 5-13;
"deep-gemm: fused per-token FP8 cast in Triton" for the cast's options).

Each flow runs from bf16 inputs on the GPU and is checked against the oracle: the
casts bit for bit, the GEMM outputs with the tolerances of the direct entry points'
tests (see test_gpu_gemm and test_gpu_g32).  Each GEMM result must also equal, bit
for bit, the same entry point called directly on the same operands."""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
from fine_grained_block_token_amd import api
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, check_wgrad, mfma_truncation_bound, oracle_sf_bits, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _sf_bits(t):
    return np.ascontiguousarray(t.contiguous().view(torch.int32).cpu().numpy()).view(np.uint32)


@pytest.mark.parametrize("mnk", [(200, 384, 1024), (1, 128, 128), (129, 296, 640)])
def test_forward_flow(gpu, mnk):
    m, n, k = mnk
    x = si.randn((m, k), si.SEED_A)
    W = si.randn((n, k), si.SEED_B)
    say("api forward", mnk)
    q, s = api.per_token_cast_to_fp8(x.cuda())
    wq, ws = api.per_block_cast_to_fp8(W.cuda())
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    sa = api.get_col_major_tma_aligned_tensor(s)
    api.gemm_fp8_fp8_bf16_nt((q, sa), (wq, ws), out)
    direct = torch.empty_like(out)
    fg.gemm_fp8_nt_bf16(q, sa, wq, ws, direct)
    torch.cuda.synchronize()
    qa, sa_o = oracle.cast_per_token(si.host_array(x))
    qb, sb_o = oracle.cast_per_block(si.host_array(W))
    assert q.dtype == torch.float8_e4m3fn and s.shape == (m, k // 128)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), qa)
    assert np.array_equal(_sf_bits(s), oracle_sf_bits(sa_o))
    assert np.array_equal(wq.view(torch.uint8).cpu().numpy(), qb)
    assert np.array_equal(_sf_bits(ws), oracle_sf_bits(sb_o))
    got = _bits(out)
    assert np.array_equal(got, _bits(direct))
    ref, absum = oracle.gemm_nt(qa, sa_o, qb, sb_o)
    check_bf16_gemm(got, ref, absum, mfma_truncation_bound(qa, sa_o, qb, sb_o), k // 128, f"api forward {mnk}")


@pytest.mark.parametrize("shape", [(256, 200, 384), (128, 8, 136)])
def test_wgrad_flow(gpu, shape):
    # the pages' wgrad: both operands cast per token along the tokens (the transposed
    # views of dY and x), dW += dY^T x in fp32
    tokens, d_out, d_in = shape
    dY = si.randn((tokens, d_out), si.SEED_DY)
    x = si.randn((tokens, d_in), si.SEED_A)
    d0 = si.randn((d_out, d_in), 5, 0.1, torch.float32)
    say("api wgrad", shape)
    gq, gs = api.per_token_cast_to_fp8(dY.cuda().t())
    xq, xs = api.per_token_cast_to_fp8(x.cuda().t())
    grad = d0.cuda()
    api.wgrad_gemm_fp8_fp8_fp32_nt((gq, api.get_col_major_tma_aligned_tensor(gs)),
                                   (xq, api.get_col_major_tma_aligned_tensor(xs)), grad)
    direct = d0.cuda()
    fg.wgrad_gemm_fp8_nt_fp32(gq, api.get_col_major_tma_aligned_tensor(gs), xq,
                              api.get_col_major_tma_aligned_tensor(xs), direct)
    torch.cuda.synchronize()
    qa, sa = oracle.cast_per_token(si.host_array(dY), transpose=True)
    qb, sb = oracle.cast_per_token(si.host_array(x), transpose=True)
    assert np.array_equal(gq.view(torch.uint8).cpu().numpy(), qa)
    assert np.array_equal(_sf_bits(gs), oracle_sf_bits(sa))
    assert np.array_equal(xq.view(torch.uint8).cpu().numpy(), qb)
    assert np.array_equal(_sf_bits(xs), oracle_sf_bits(sb))
    got = grad.cpu().numpy()
    assert np.array_equal(got, direct.cpu().numpy())
    ref, absum = oracle.wgrad_nt(qa, sa, qb, sb, d0.numpy())
    check_wgrad(got, ref, absum, tokens // 128, f"api wgrad {shape}")


def test_grouped_flow(gpu):
    # four experts with ragged token counts, each segment padded to the m alignment
    E, n, k = 4, 256, 512
    m_idx = si.grouped_layout([100, 0, 257, 31], api.get_m_alignment_for_contiguous_layout())
    m = m_idx.size
    x = si.randn((m, k), si.SEED_A, 0.1)
    Ws = [si.randn((n, k), 10 + e, 0.1) for e in range(E)]
    say("api m-grouped", (m, n, k), "experts", E)
    q, s = api.per_token_cast_to_fp8(x.cuda())
    rq = torch.empty((E, n, k), dtype=torch.float8_e4m3fn, device="cuda")
    rs = torch.empty((E, n // 128, k // 128), dtype=torch.float32, device="cuda")
    for e in range(E):
        rq[e], rs[e] = api.per_block_cast_to_fp8(Ws[e].cuda())
    idx = torch.from_numpy(m_idx).cuda()
    out = torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda")
    sa = api.get_col_major_tma_aligned_tensor(s)
    api.m_grouped_gemm_fp8_fp8_bf16_nt_contiguous((q, sa), (rq, rs), out, idx)
    direct = torch.full_like(out, 7.0)
    fg.m_grouped_gemm_fp8_nt_bf16_contiguous(q, sa, rq, rs, idx, direct)
    torch.cuda.synchronize()
    got = _bits(out)
    assert np.array_equal(got, _bits(direct))
    pad = m_idx < 0
    assert (oracle.bf16_bits_to_f32(got[pad]) == 7.0).all()
    qa, sa_o = oracle.cast_per_token(si.host_array(x))
    qb = np.stack([oracle.cast_per_block(si.host_array(w))[0] for w in Ws])
    sb = np.stack([oracle.cast_per_block(si.host_array(w))[1] for w in Ws])
    ref, absum = oracle.m_grouped_gemm_nt(qa, sa_o, qb, sb, m_idx)
    rows = ~pad
    tb = np.zeros((m, n))
    for e in range(E):
        r = np.nonzero(m_idx == e)[0]
        if r.size:
            tb[r] = mfma_truncation_bound(qa[r], sa_o[r], qb[e], sb[e])
    check_bf16_gemm(got[rows], ref[rows], absum[rows], tb[rows], k // 128, "api m-grouped")


@pytest.mark.parametrize("use_packed", [False, True])
def test_cast_options_and_out_views(gpu, use_packed):
    # UE8M0 scales, as fp32 powers of two or packed words (1 x 32 groups), written into
    # caller-owned views of larger buffers
    rows, cols = 130, 1000
    x = si.cast_workload(rows, cols)
    gran = 32 if use_packed else 128
    fmt = oracle.SF_PACKED_UE8M0 if use_packed else oracle.SF_UE8M0
    qbuf = torch.full((rows, 1024), 0xA5, dtype=torch.uint8, device="cuda")
    q = qbuf[:, :cols].view(torch.float8_e4m3fn)
    G = -(-cols // gran)
    if use_packed:
        sbuf = torch.full((-(-G // 4), 136), -7, dtype=torch.int32, device="cuda")
        sf = sbuf.t()[:rows]
    else:
        sbuf = torch.full((rows, G + 3), -7.0, dtype=torch.float32, device="cuda")
        sf = sbuf[:, :G]
    say("api cast options", (rows, cols), "gran", gran, "packed", use_packed)
    rq, rsf = api.fused_per_token_cast_to_fp8(x.cuda(), use_ue8m0=True, gran_k=gran,
                                              use_packed_ue8m0=use_packed, out=q, out_sf=sf)
    torch.cuda.synchronize()
    assert rq is q and rsf is sf
    qa, sa = oracle.cast_per_token(si.host_array(x), gran, fmt)
    assert np.array_equal(qbuf[:, :cols].cpu().numpy(), qa)
    assert (qbuf[:, cols:].cpu() == 0xA5).all()
    assert np.array_equal(_sf_bits(sf), oracle_sf_bits(sa))
    if use_packed:
        assert (sbuf[:, rows:].cpu() == -7).all()
    else:
        assert (sbuf[:, G:].cpu() == -7.0).all()


def test_g32_flow(gpu):
    # packed UE8M0 words on both operands select the group-32 kernel
    m, n, k = 129, 256, 512
    x = si.randn((m, k), si.SEED_A)
    W = si.randn((n, k), si.SEED_B)
    say("api g32", (m, n, k))
    q, s = api.per_token_cast_to_fp8(x.cuda(), use_ue8m0=True, gran_k=32, use_packed_ue8m0=True)
    wq, ws = api.per_token_cast_to_fp8(W.cuda(), use_ue8m0=True, gran_k=32, use_packed_ue8m0=True)
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    api.gemm_fp8_fp8_bf16_nt((q, s), (wq, ws), out)
    direct = torch.empty_like(out)
    fg.gemm_fp8_nt_bf16_ue8m0_g32(q, s, wq, ws, direct)
    torch.cuda.synchronize()
    got = _bits(out)
    assert np.array_equal(got, _bits(direct))
    qa, wa = oracle.cast_per_token(si.host_array(x), 32, oracle.SF_PACKED_UE8M0)
    qb, wb = oracle.cast_per_token(si.host_array(W), 32, oracle.SF_PACKED_UE8M0)
    assert np.array_equal(_sf_bits(s), oracle_sf_bits(wa)) and np.array_equal(_sf_bits(ws), oracle_sf_bits(wb))
    sa, sb = oracle.unpack_ue8m0(wa, k // 32), oracle.unpack_ue8m0(wb, k // 32)
    ref, absum = oracle.gemm_nt_g32(qa, sa, qb, sb)
    tb = mfma_truncation_bound(qa, sa, qb, sb, sb_block=False, group=32)
    check_bf16_gemm(got, ref, absum, tb, k // 8, "api g32")


def test_grouped_g32_flow(gpu):
    # int32 RHS scales select the group-32 m-grouped kernel: the LHS cast per 1 x 32 group with
    # packed words, each expert's weight cast the same way into an MN-major slice of an
    # [E, k/128, n] word buffer
    E, n, k = 4, 256, 512
    m_idx = si.grouped_layout([100, 0, 257, 31], api.get_m_alignment_for_contiguous_layout())
    m = m_idx.size
    x = si.randn((m, k), si.SEED_A, 0.1)
    Ws = [si.randn((n, k), 20 + e, 0.1) for e in range(E)]
    say("api m-grouped g32", (m, n, k), "experts", E)
    q, s = api.per_token_cast_to_fp8(x.cuda(), use_ue8m0=True, gran_k=32, use_packed_ue8m0=True)
    rq = torch.empty((E, n, k), dtype=torch.float8_e4m3fn, device="cuda")
    rs = torch.empty((E, k // 128, n), dtype=torch.int32, device="cuda").permute(0, 2, 1)
    for e in range(E):
        api.fused_per_token_cast_to_fp8(Ws[e].cuda(), use_ue8m0=True, gran_k=32, use_packed_ue8m0=True,
                                        out=rq[e], out_sf=rs[e])
    idx = torch.from_numpy(m_idx).cuda()
    out = torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda")
    api.m_grouped_gemm_fp8_fp8_bf16_nt_contiguous((q, s), (rq, rs), out, idx)
    direct = torch.full_like(out, 7.0)
    fg.m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(q, s, rq, rs, idx, direct)
    torch.cuda.synchronize()
    got = _bits(out)
    assert np.array_equal(got, _bits(direct))
    pad = m_idx < 0
    assert (oracle.bf16_bits_to_f32(got[pad]) == 7.0).all()
    qa, wa = oracle.cast_per_token(si.host_array(x), 32, oracle.SF_PACKED_UE8M0)
    casts = [oracle.cast_per_token(si.host_array(w), 32, oracle.SF_PACKED_UE8M0) for w in Ws]
    qb = np.stack([c[0] for c in casts])
    assert np.array_equal(rq.view(torch.uint8).cpu().numpy(), qb)
    sa = oracle.unpack_ue8m0(wa, k // 32)
    sb = np.stack([oracle.unpack_ue8m0(c[1], k // 32) for c in casts])
    ref, absum = oracle.m_grouped_gemm_nt_g32(qa, sa, qb, sb, m_idx)
    rows = ~pad
    tb = np.zeros((m, n))
    for e in range(E):
        r = np.nonzero(m_idx == e)[0]
        if r.size:
            tb[r] = mfma_truncation_bound(qa[r], sa[r], qb[e], sb[e], sb_block=False, group=32)
    check_bf16_gemm(got[rows], ref[rows], absum[rows], tb[rows], k // 8, "api m-grouped g32")


@pytest.mark.parametrize("tokens,gran,pass_gran", [(256, 128, False), (256, 32, False), (128, 128, True),
                                                   (128, 32, True)])
def test_wgrad_packed_words_flow(gpu, tokens, gran, pass_gran):
    # both operands cast along the tokens with packed UE8M0 words: 1 x 128 groups run the
    # UE8M0 1x128 weight gradient, 1 x 32 groups the group-32 one; the word shapes tell them
    # apart, except at 128 tokens, where gran_k names the cast (feature counts whose bf16 rows
    # are whole 16-byte units, as the transposed views need)
    d_out, d_in = 136, 200
    dY = si.randn((tokens, d_out), si.SEED_DY)
    x = si.randn((tokens, d_in), si.SEED_A)
    d0 = si.randn((d_out, d_in), 5, 0.1, torch.float32)
    say("api wgrad packed", (tokens, d_out, d_in), "gran", gran)
    gq, gs = api.per_token_cast_to_fp8(dY.cuda().t(), use_ue8m0=True, gran_k=gran, use_packed_ue8m0=True)
    xq, xs = api.per_token_cast_to_fp8(x.cuda().t(), use_ue8m0=True, gran_k=gran, use_packed_ue8m0=True)
    grad = d0.cuda()
    api.wgrad_gemm_fp8_fp8_fp32_nt((gq, gs), (xq, xs), grad, gran_k=gran if pass_gran else None)
    direct = d0.cuda()
    if gran == 32:
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0_g32(gq, gs, xq, xs, direct)
    else:
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0(gq, gs, xq, xs, direct, fg.SF_PACKED_UE8M0)
    torch.cuda.synchronize()
    got = grad.cpu().numpy()
    assert np.array_equal(got, direct.cpu().numpy())
    qa, wa = oracle.cast_per_token(si.host_array(dY), gran, oracle.SF_PACKED_UE8M0, transpose=True)
    qb, wb = oracle.cast_per_token(si.host_array(x), gran, oracle.SF_PACKED_UE8M0, transpose=True)
    assert np.array_equal(gq.view(torch.uint8).cpu().numpy(), qa)
    assert np.array_equal(_sf_bits(gs), oracle_sf_bits(wa)) and np.array_equal(_sf_bits(xs), oracle_sf_bits(wb))
    sa, sb = oracle.unpack_ue8m0(wa, tokens // gran), oracle.unpack_ue8m0(wb, tokens // gran)
    wgrad = oracle.wgrad_nt_g32 if gran == 32 else oracle.wgrad_nt
    ref, absum = wgrad(qa, sa, qb, sb, d0.numpy())
    check_wgrad(got, ref, absum, tokens // 32, f"api wgrad packed {tokens} gran {gran}")
