"""The entry points inside a captured HIP graph: every replay must reproduce the
eager result bit for bit (the library allocates nothing, never synchronises and
records no memset, so its launches are capturable).  The graph is replayed
several times with the program's own eager work and synchronisations in between.
"""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import synth_inputs as si
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu):
    T, I, O = 384, 1024, 640
    x = si.randn((T, I), si.SEED_A).cuda()
    W = si.randn((O, I), si.SEED_B).cuda()
    u8, f32 = torch.uint8, torch.float32
    xq = torch.empty((T, I), dtype=u8, device="cuda")
    sx = fg.mn_major_scales(T, I // 128)
    xq1 = torch.empty((1, I), dtype=u8, device="cuda")
    sx1 = fg.mn_major_scales(1, I // 128)
    Wq = torch.empty((O, I), dtype=u8, device="cuda")
    sW = torch.empty((O // 128, I // 128), dtype=f32, device="cuda")
    xTq = torch.empty((I, T), dtype=u8, device="cuda")
    sxT = fg.mn_major_scales(I, T // 128)
    wp = torch.empty((T, I), dtype=u8, device="cuda")
    swp = fg.mn_major_scales(T, I // 32 // 4, torch.int32)
    y = torch.empty((T, O), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty((1, O), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((I, I), dtype=f32, device="cuda")
    # dual cast, fused output cast, group-32 GEMM and wgrad, m-grouped GEMM
    dq, dsx = torch.empty((T, I), dtype=u8, device="cuda"), fg.mn_major_scales(T, I // 128)
    dqT, dsxT = torch.empty((I, T), dtype=u8, device="cuda"), fg.mn_major_scales(I, T // 128)
    yq, ysf = torch.empty((T, O), dtype=u8, device="cuda"), fg.mn_major_scales(T, O // 128)
    y2 = torch.empty((T, O), dtype=torch.bfloat16, device="cuda")
    W32, sW32 = torch.empty((O, I), dtype=u8, device="cuda"), fg.mn_major_scales(O, I // 128, torch.int32)
    y32 = torch.empty((T, O), dtype=torch.bfloat16, device="cuda")
    xT32, sxT32 = torch.empty((I, T), dtype=u8, device="cuda"), fg.mn_major_scales(I, T // 128, torch.int32)
    dW32 = torch.empty((I, I), dtype=f32, device="cuda")
    m_idx = torch.from_numpy(si.grouped_layout([100, 200])).cuda()   # 384 rows, 2 experts
    E = 2
    Wg = torch.stack([W, W.flip(0)])
    Wgq = torch.empty((E, O, I), dtype=u8, device="cuda")
    sWg = torch.empty((E, O // 128, I // 128), dtype=f32, device="cuda")
    yg = torch.empty((m_idx.numel(), O), dtype=torch.bfloat16, device="cuda")
    Wg32 = torch.empty((E, O, I), dtype=u8, device="cuda")
    sWg32 = torch.empty((E, I // 128, O), dtype=torch.int32, device="cuda").permute(0, 2, 1)
    yg32 = torch.empty((m_idx.numel(), O), dtype=torch.bfloat16, device="cuda")
    xu, sxu = torch.empty((T, I), dtype=u8, device="cuda"), fg.mn_major_scales(T, I // 128)
    Wu, sWu = torch.empty((O, I), dtype=u8, device="cuda"), torch.empty((O // 128, I // 128), dtype=f32, device="cuda")
    yu = torch.empty((T, O), dtype=torch.bfloat16, device="cuda")
    xTu, sxTu = torch.empty((I, T), dtype=u8, device="cuda"), fg.mn_major_scales(I, T // 128)
    dWu = torch.empty((I, I), dtype=f32, device="cuda")

    def step():
        fg.cast_per_token(x, xq, sx, 128, fg.SF_FP32)
        fg.cast_per_token(x[:1], xq1, sx1, 128, fg.SF_FP32)
        fg.cast_per_token(x, wp, swp, 32, fg.SF_PACKED_UE8M0)
        fg.cast_per_token(x.t(), xTq, sxT, 128, fg.SF_FP32)
        fg.cast_per_block(W, Wq, sW, sf_fmt=fg.SF_FP32)
        fg.gemm_fp8_nt_bf16(xq, sx, Wq, sW, y)
        fg.gemm_fp8_nt_bf16(xq1, sx1, Wq, sW, y1)          # decode-sized path
        fg.wgrad_gemm_fp8_nt_fp32(xTq, sxT, xTq, sxT, dW)  # dW += xT xT^T
        fg.cast_per_token_dual(x, dq, dsx, dqT, dsxT)
        fg.gemm_fp8_nt_bf16_cast(xq, sx, Wq, sW, y2, yq, ysf)
        fg.cast_per_token(W, W32, sW32, 32, fg.SF_PACKED_UE8M0)
        fg.gemm_fp8_nt_bf16_ue8m0_g32(wp, swp, W32, sW32, y32)
        fg.cast_per_token(x.t(), xT32, sxT32, 32, fg.SF_PACKED_UE8M0)
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0_g32(xT32, sxT32, xT32, sxT32, dW32)
        for e in range(E):
            fg.cast_per_block(Wg[e], Wgq[e], sWg[e], sf_fmt=fg.SF_FP32)
        fg.m_grouped_gemm_fp8_nt_bf16_contiguous(xq[:m_idx.numel()], sx[:m_idx.numel()], Wgq, sWg, m_idx, yg)
        for e in range(E):
            fg.cast_per_token(Wg[e], Wg32[e], sWg32[e], 32, fg.SF_PACKED_UE8M0)
        fg.m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(wp, swp, Wg32, sWg32, m_idx, yg32)
        fg.cast_per_token(x, xu, sxu, 128, fg.SF_UE8M0)
        fg.cast_per_block(W, Wu, sWu, sf_fmt=fg.SF_UE8M0)
        fg.gemm_fp8_nt_bf16_ue8m0(xu, sxu, Wu, sWu, yu)
        fg.cast_per_token(x.t(), xTu, sxTu, 128, fg.SF_UE8M0)
        fg.wgrad_gemm_fp8_nt_fp32_ue8m0(xTu, sxTu, xTu, sxTu, dWu)

    outs = [xq, sx, xq1, sx1, wp, swp, xTq, sxT, Wq, sW, y, y1, dq, dsx, dqT, dsxT, yq, ysf, y2, W32, sW32, y32,
            xT32, sxT32, dW32, Wgq, sWg, yg, Wg32, yg32, xu, sxu, Wu, sWu, yu, xTu, sxTu, dWu]

    def snap():
        return [o.cpu().clone() for o in outs], dW.cpu().clone()

    def clear():
        for o in outs + [dW]:
            o.zero_()

    say("graph: eager reference")
    clear()
    step()
    torch.cuda.synchronize()
    ref, ref_dw = snap()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for r in range(3):
        say("graph: replay", r)
        clear()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got, got_dw = snap()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {r} differs from the eager result"
        # wgrad accumulates into dW: zeroed, then one pass, on both sides
        assert torch.equal(got_dw, ref_dw), f"replay {r}: wgrad differs"
        del junk


def test_graph_replays_match_eager_splitk_and_wide(gpu):
    # split-K (stream-K shares at m = 1 and 64, K slices at m = 384), its allocation-free form,
    # and the 256x256 kernel of the power-of-two recipes (4096 x 4096 outputs, 8 K blocks)
    u8, f32 = torch.uint8, torch.float32
    n, k = 1024, 2048
    W = si.randn((n, k), si.SEED_B).cuda()
    Wq, sW = torch.empty((n, k), dtype=u8, device="cuda"), torch.empty((n // 128, k // 128), dtype=f32, device="cuda")
    fg.cast_per_block(W, Wq, sW, sf_fmt=fg.SF_FP32)
    cases = []
    for m in (1, 64, 384):
        x = si.randn((m, k), si.SEED_A + m).cuda()
        xq, sx = torch.empty((m, k), dtype=u8, device="cuda"), fg.mn_major_scales(m, k // 128)
        fg.cast_per_token(x, xq, sx, 128, fg.SF_FP32)
        wsb = fg.gemm_fp8_nt_bf16_splitk_workspace(m, n, k)
        assert wsb > 0, (m, n, k)
        ws = torch.empty((wsb // 4,), dtype=f32, device="cuda")
        cases.append((xq, sx, ws, torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                      torch.empty((m, n), dtype=torch.bfloat16, device="cuda")))
    M = N = 4096
    K = 1024
    a = si.randn((M, K), si.SEED_A, 0.1).cuda()
    b = si.randn((N, K), si.SEED_B, 0.1).cuda()
    A, B = torch.empty((M, K), dtype=u8, device="cuda"), torch.empty((N, K), dtype=u8, device="cuda")
    sa, sb = fg.mn_major_scales(M, K // 128), torch.empty((N // 128, K // 128), dtype=f32, device="cuda")
    fg.cast_per_token(a, A, sa, 128, fg.SF_UE8M0)
    fg.cast_per_block(b, B, sb, sf_fmt=fg.SF_UE8M0)
    A32, B32 = torch.empty((M, K), dtype=u8, device="cuda"), torch.empty((N, K), dtype=u8, device="cuda")
    wa, wb = fg.mn_major_scales(M, K // 128, torch.int32), fg.mn_major_scales(N, K // 128, torch.int32)
    fg.cast_per_token(a, A32, wa, 32, fg.SF_PACKED_UE8M0)
    fg.cast_per_token(b, B32, wb, 32, fg.SF_PACKED_UE8M0)
    yw = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yw32 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    def step():
        for xq, sx, ws, y, y_na in cases:
            fg.gemm_fp8_nt_bf16_splitk(xq, sx, Wq, sW, y, ws)
            fg.gemm_fp8_nt_bf16_splitk_noalloc(xq, sx, Wq, sW, y_na)
        fg.gemm_fp8_nt_bf16_ue8m0(A, sa, B, sb, yw)
        fg.gemm_fp8_nt_bf16_ue8m0_g32(A32, wa, B32, wb, yw32)

    outs = [c[3] for c in cases] + [c[4] for c in cases] + [yw, yw32]

    def clear():
        for o in outs:
            o.zero_()

    say("graph (split-K, wide): eager reference")
    clear()
    step()
    torch.cuda.synchronize()
    ref = [o.cpu().clone() for o in outs]
    for c in cases:                       # the allocation-free form gives the same bits
        assert torch.equal(c[3], c[4])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        say("graph (split-K, wide): replay", r)
        clear()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outs, ref):
            assert torch.equal(o.cpu(), want), f"replay {r} differs from the eager result"
        del junk
