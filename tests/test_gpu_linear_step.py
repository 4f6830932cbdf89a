"""End-to-end GPU parity of one FP8 nn.Linear step (tokens 8192, in 7168, out
4096), run by fine_grained_block_token_amd.linear.Fp8Linear as the benchmark runs
it ("[Help] Starter script for nn.Linear for fwd,bwd": forward x.W^T, dgrad dY.W,
wgrad dY^T.x with the operands cast per token / per block; "DeepGEMM Essentials",
Part 18):

  cast_per_token_dual(x)  -> xq, sx (1x128 along in) and xTq, sxT (along tokens)
  cast_per_block(W)       -> Wq, sW and the exact transpose WqT, sWT
  gemm_fp8_nt_bf16        y  = (xq, sx) . (Wq, sW)^T            [8192, 4096]
  cast_per_token_dual(dY) -> dYq, sdY and dYTq, sdYT
  gemm_fp8_nt_bf16        dX = (dYq, sdY) . (WqT, sWT)^T        [8192, 7168]
  wgrad_gemm_fp8_nt_fp32  dW += (dYTq, sdYT) . (xTq, sxT)^T     [4096, 7168]

Every cast output (E4M3 bytes and scale bits, both orientations) must equal the
oracle's cast of the same host input.  y and dX are checked on 20,000 sampled
outputs plus tile corners against the oracle's fp64 GEMM of the oracle's own
casts (2 bf16 ulps + the fp32 accumulation and FP8 MFMA terms, the 1e-3
Frobenius gate and the literal 2-ulp ceiling); dW against the oracle's wgrad with
the fp32 accumulation bound and the relative Frobenius gate of 1e-5.  The step
also runs in the UE8M0 scale option and the UE8M0 group-32 recipe, each against
its own oracle.
"""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
from fine_grained_block_token_amd.linear import Fp8Linear
import oracle
import synth_inputs as si
from gpu_util import check_bf16_gemm, check_wgrad, mfma_truncation_bound, sample_idx, say

pytestmark = pytest.mark.gpu

T, I, O = si.LINEAR["tokens"], si.LINEAR["d_in"], si.LINEAR["d_out"]


@pytest.fixture(scope="module")
def host_inputs():
    x = si.randn((T, I), si.SEED_A)
    W = si.randn((O, I), si.SEED_B)
    dY = si.randn((T, O), si.SEED_DY)
    return si.host_array(x), si.host_array(W), si.host_array(dY)


def _run(recipe):
    x = si.randn((T, I), si.SEED_A).cuda()
    W = si.randn((O, I), si.SEED_B).cuda()
    dY = si.randn((T, O), si.SEED_DY).cuda()
    L = Fp8Linear(T, I, O, recipe)
    for name, fn in L.ops(x, W, dY):
        say("linear step", recipe, name)
        fn()
    torch.cuda.synchronize()
    return L


def _u8(t):
    return t.cpu().numpy()


def _bits(t):
    """Device scales (any strides) -> host [rows, units] uint32 bit patterns."""
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def _same(got_q, got_sf, want_q, want_sf, what):
    assert np.array_equal(_u8(got_q), want_q), f"{what}: E4M3 bytes differ"
    assert np.array_equal(_bits(got_sf), np.ascontiguousarray(want_sf).view(np.uint32)), f"{what}: scale bits differ"


def _bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_linear_step_fp32_scales(gpu, host_inputs):
    xh, Wh, dYh = host_inputs
    L = _run("fp32")

    # casts: bit-exact, both orientations
    qx, sx = oracle.cast_per_token(xh, 128, oracle.SF_FP32)
    qxT, sxT = oracle.cast_per_token(xh, 128, oracle.SF_FP32, transpose=True)
    qdY, sdY = oracle.cast_per_token(dYh, 128, oracle.SF_FP32)
    qdYT, sdYT = oracle.cast_per_token(dYh, 128, oracle.SF_FP32, transpose=True)
    qW, sW = oracle.cast_per_block(Wh, oracle.SF_FP32)
    qWT, sWT = oracle.cast_per_block(np.ascontiguousarray(Wh.T), oracle.SF_FP32)
    _same(L.xq, L.sx, qx, sx, "x")
    _same(L.xTq, L.sxT, qxT, sxT, "x^T")
    _same(L.dYq, L.sdY, qdY, sdY, "dY")
    _same(L.dYTq, L.sdYT, qdYT, sdYT, "dY^T")
    _same(L.Wq, L.sW, qW, sW, "W")
    _same(L.WqT, L.sWT, qWT, sWT, "W^T")

    # forward y = x W^T
    ii, jj = sample_idx(T, O, 20000, 31)
    ref, absum = oracle.gemm_nt(qx, sx, qW, sW, idx=(ii, jj))
    tb = mfma_truncation_bound(qx, sx, qW, sW, idx=(ii, jj))
    check_bf16_gemm(_bf16_bits(L.y)[ii, jj], ref, absum, tb, I // 128, "linear step forward 8192x4096x7168")

    # dgrad dX = dY W
    ii, jj = sample_idx(T, I, 20000, 32)
    ref, absum = oracle.gemm_nt(qdY, sdY, qWT, sWT, idx=(ii, jj))
    tb = mfma_truncation_bound(qdY, sdY, qWT, sWT, idx=(ii, jj))
    check_bf16_gemm(_bf16_bits(L.dX)[ii, jj], ref, absum, tb, O // 128, "linear step dgrad 8192x7168x4096")

    # wgrad dW = dY^T x (dW starts at zero)
    ii, jj = sample_idx(O, I, 20000, 33)
    ref, absum = oracle.wgrad_nt(qdYT, sdYT, qxT, sxT, np.zeros((O, I), np.float32), idx=(ii, jj))
    check_wgrad(L.dW.cpu().numpy()[ii, jj], ref, absum, T // 128, "linear step wgrad 4096x7168x8192")


def test_linear_step_ue8m0_scales(gpu, host_inputs):
    # the same step with the casts' UE8M0 option: every scale a power of two, applied
    # by the scaled MFMA in all three GEMMs
    xh, Wh, dYh = host_inputs
    L = _run("ue8m0")
    U = oracle.SF_UE8M0
    qx, sx = oracle.cast_per_token(xh, 128, U)
    qxT, sxT = oracle.cast_per_token(xh, 128, U, transpose=True)
    qdY, sdY = oracle.cast_per_token(dYh, 128, U)
    qdYT, sdYT = oracle.cast_per_token(dYh, 128, U, transpose=True)
    qW, sW = oracle.cast_per_block(Wh, U)
    qWT, sWT = oracle.cast_per_block(np.ascontiguousarray(Wh.T), U)
    for got, want, what in [((L.xq, L.sx), (qx, sx), "x"), ((L.xTq, L.sxT), (qxT, sxT), "x^T"),
                            ((L.dYq, L.sdY), (qdY, sdY), "dY"), ((L.dYTq, L.sdYT), (qdYT, sdYT), "dY^T"),
                            ((L.Wq, L.sW), (qW, sW), "W"), ((L.WqT, L.sWT), (qWT, sWT), "W^T")]:
        _same(*got, *want, f"ue8m0 {what}")
    ii, jj = sample_idx(T, O, 20000, 34)
    ref, absum = oracle.gemm_nt(qx, sx, qW, sW, idx=(ii, jj))
    tb = mfma_truncation_bound(qx, sx, qW, sW, idx=(ii, jj))
    check_bf16_gemm(_bf16_bits(L.y)[ii, jj], ref, absum, tb, I // 8, "linear step ue8m0 forward")
    ii, jj = sample_idx(T, I, 20000, 35)
    ref, absum = oracle.gemm_nt(qdY, sdY, qWT, sWT, idx=(ii, jj))
    tb = mfma_truncation_bound(qdY, sdY, qWT, sWT, idx=(ii, jj))
    check_bf16_gemm(_bf16_bits(L.dX)[ii, jj], ref, absum, tb, O // 8, "linear step ue8m0 dgrad")
    ii, jj = sample_idx(O, I, 20000, 36)
    ref, absum = oracle.wgrad_nt(qdYT, sdYT, qxT, sxT, np.zeros((O, I), np.float32), idx=(ii, jj))
    check_wgrad(L.dW.cpu().numpy()[ii, jj], ref, absum, T // 32, "linear step ue8m0 wgrad")


def test_linear_step_g32_recipe(gpu, host_inputs):
    # the UE8M0 group-32 recipe: x, W and dY each cast once in both orientations with
    # 1x32 groups and packed scales; the three GEMMs on the scaled MFMA
    xh, Wh, dYh = host_inputs
    L = _run("ue8m0_g32")
    P = oracle.SF_PACKED_UE8M0
    casts = {}
    for name, h, gq, gs, gqT, gsT in [("x", xh, L.xq, L.sx, L.xTq, L.sxT), ("W", Wh, L.Wq, L.sW, L.WqT, L.sWT),
                                       ("dY", dYh, L.dYq, L.sdY, L.dYTq, L.sdYT)]:
        q, w = oracle.cast_per_token(h, 32, P)
        qT, wT = oracle.cast_per_token(h, 32, P, transpose=True)
        _same(gq, gs, q, w, f"g32 {name}")
        _same(gqT, gsT, qT, wT, f"g32 {name}^T")
        casts[name] = (q, oracle.unpack_ue8m0(w, -(-q.shape[1] // 32)),
                       qT, oracle.unpack_ue8m0(wT, -(-qT.shape[1] // 32)))
    qx, sx, qxT, sxT = casts["x"]
    qW, sW, qWT, sWT = casts["W"]
    qdY, sdY, qdYT, sdYT = casts["dY"]
    ii, jj = sample_idx(T, O, 20000, 37)
    ref, absum = oracle.gemm_nt_g32(qx, sx, qW, sW, idx=(ii, jj))
    tb = mfma_truncation_bound(qx, sx, qW, sW, sb_block=False, idx=(ii, jj), group=32)
    check_bf16_gemm(_bf16_bits(L.y)[ii, jj], ref, absum, tb, I // 8, "linear step g32 forward")
    ii, jj = sample_idx(T, I, 20000, 38)
    ref, absum = oracle.gemm_nt_g32(qdY, sdY, qWT, sWT, idx=(ii, jj))
    tb = mfma_truncation_bound(qdY, sdY, qWT, sWT, sb_block=False, idx=(ii, jj), group=32)
    check_bf16_gemm(_bf16_bits(L.dX)[ii, jj], ref, absum, tb, O // 8, "linear step g32 dgrad")
    ii, jj = sample_idx(O, I, 20000, 39)
    ref, absum = oracle.wgrad_nt_g32(qdYT, sdYT, qxT, sxT, np.zeros((O, I), np.float32), idx=(ii, jj))
    check_wgrad(L.dW.cpu().numpy()[ii, jj], ref, absum, T // 32, "linear step g32 wgrad")


@pytest.mark.parametrize("recipe", ["fp32", "ue8m0", "ue8m0_g32"])
def test_linear_step_graph_replay(gpu, recipe):
    # the whole step captured in one HIP graph (as the benchmark times it): every replay
    # gives the eager step's y and dX bit for bit, and dW accumulates exactly as the same
    # number of eager steps does
    t, i, o = 512, 384, 256
    x = si.randn((t, i), si.SEED_A).cuda()
    W = si.randn((o, i), si.SEED_B).cuda()
    dY = si.randn((t, o), si.SEED_DY).cuda()
    eager, graphed = Fp8Linear(t, i, o, recipe), Fp8Linear(t, i, o, recipe)
    say("linear step graph", recipe, (t, i, o))
    graphed.step(x, W, dY)                      # warm (and the first accumulation into dW)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            graphed.step(x, W, dY)
    torch.cuda.current_stream().wait_stream(s)
    eager.step(x, W, dY)
    for r in range(3):
        g.replay()
        eager.step(x, W, dY)
        torch.cuda.synchronize()
        assert torch.equal(graphed.y.view(torch.int16), eager.y.view(torch.int16)), f"y differs on replay {r}"
        assert torch.equal(graphed.dX.view(torch.int16), eager.dX.view(torch.int16)), f"dX differs on replay {r}"
        assert torch.equal(graphed.dW, eager.dW), f"dW differs after replay {r}"
