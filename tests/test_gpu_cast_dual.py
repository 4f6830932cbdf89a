"""GPU parity of the dual-orientation per-token cast: one read of bf16 or fp32 x gives
q/sf bit-identical to the oracle's per-token cast of x and qT/sfT bit-identical
to its per-token cast of x^T (1x128 or 1x32 groups, fp32 / UE8M0 / packed UE8M0
scales; "DeepGEMM Essentials", Part 3, the wgrad operands of "[Help] Starter
script for nn.Linear for fwd,bwd", and the group-32 formats of "deep-gemm:
fused per-token FP8 cast in Triton").  Writes must stay inside the given views."""
import numpy as np
import pytest
import torch

import fine_grained_block_token_amd as fg
import oracle
import synth_inputs as si
from gpu_util import oracle_sf_bits, say, sentinel_u8

pytestmark = pytest.mark.gpu


def _scale_view(rows, groups, mn_major, pad, packed=False):
    """Scale view [rows, groups] (float32, or int32 words when packed) over a sentinel-filled
    buffer; returns (view, buffer)."""
    dt = torch.int32 if packed else torch.float32
    if mn_major:
        ld = -(-(rows + pad) // 4) * 4
        buf = torch.full((groups, ld), -7, dtype=torch.int32, device="cuda")
        return buf.view(dt).t()[:rows], buf
    buf = torch.full((rows, groups + pad), -7, dtype=torch.int32, device="cuda")
    return buf.view(dt)[:, :groups], buf


def _run_dual(x_cpu, fmt, mn_major=True, gran=128):
    rows, cols = x_cpu.shape
    x_ld = -(-cols // 8) * 8          # the kernel reads 16-byte chunks of each row
    xbuf = torch.zeros((rows, x_ld), dtype=x_cpu.dtype, device="cuda")
    xbuf[:, :cols] = x_cpu.cuda()
    x = xbuf[:, :cols]
    q_ld = -(-(cols + 8) // 8) * 8
    qT_ld = -(-(rows + 16) // 16) * 16
    qbuf, qTbuf = sentinel_u8((rows, q_ld)), sentinel_u8((cols, qT_ld))
    q, qT = qbuf[:, :cols], qTbuf[:, :rows]
    packed = fmt == oracle.SF_PACKED_UE8M0
    G, GT = fg.num_groups(cols, gran), fg.num_groups(rows, gran)
    if packed:
        G, GT = -(-G // 4), -(-GT // 4)   # words of four groups
    sf, sbuf = _scale_view(rows, G, mn_major, 4, packed)
    sfT, sTbuf = _scale_view(cols, GT, mn_major, 4, packed)
    say("cast_per_token_dual", (rows, cols), x_cpu.dtype, "gran", gran, "fmt", fmt, "mn", mn_major)
    fg.cast_per_token_dual(x, q, sf, qT, sfT, fmt, gran)
    torch.cuda.synchronize()
    got = (q.cpu().numpy(), sf.contiguous().view(torch.int32).cpu().numpy().view(np.uint32),
           qT.cpu().numpy(), sfT.contiguous().view(torch.int32).cpu().numpy().view(np.uint32))
    # nothing outside the views changed
    assert (qbuf.cpu().numpy()[:, cols:] == 0xA5).all()
    assert (qTbuf.cpu().numpy()[:, rows:] == 0xA5).all()
    for buf, n, g in ((sbuf, rows, G), (sTbuf, cols, GT)):
        b = buf.cpu().numpy()
        assert ((b[:, n:] if mn_major else b[:, g:]) == -7).all()
    return got


def _check(x_cpu, fmt, mn_major=True, gran=128):
    q, sf, qT, sfT = _run_dual(x_cpu, fmt, mn_major, gran)
    oq, osf = oracle.cast_per_token(si.host_array(x_cpu), gran, fmt)
    oqT, osfT = oracle.cast_per_token(si.host_array(x_cpu), gran, fmt, transpose=True)
    assert np.array_equal(q, oq), "row-wise E4M3 bytes differ"
    assert np.array_equal(sf, oracle_sf_bits(osf)), "row-wise scale bits differ"
    assert np.array_equal(qT, oqT), "transposed E4M3 bytes differ"
    assert np.array_equal(sfT, oracle_sf_bits(osfT)), "transposed scale bits differ"


@pytest.mark.parametrize("shape", [(1, 512), (7, 4096), (129, 7168), (64, 1000), (128, 128), (129, 257),
                                   (200, 300), (3000, 4096), (5, 3)])
@pytest.mark.parametrize("fmt", [oracle.SF_FP32, oracle.SF_UE8M0], ids=["fp32", "ue8m0"])
def test_dual_matches_both_casts(gpu, shape, fmt):
    # the cast workloads carry an all-zero group and a group scaled by 1e4
    _check(si.cast_workload(*shape, seed=si.SEED_A), fmt, mn_major=True)


@pytest.mark.parametrize("shape", [(1, 512), (7, 4096), (129, 7168), (64, 1000), (128, 128), (129, 257),
                                   (200, 300), (5, 3), (640, 96), (300, 1000)])
@pytest.mark.parametrize("fmt", [oracle.SF_FP32, oracle.SF_UE8M0, oracle.SF_PACKED_UE8M0],
                         ids=["fp32", "ue8m0", "packed"])
def test_dual_group32(gpu, shape, fmt):
    _check(si.cast_workload(*shape, seed=si.SEED_A), fmt, mn_major=True, gran=32)


@pytest.mark.parametrize("shape", [(1, 512), (129, 7168), (64, 1000), (200, 300), (5, 3), (640, 96), (700, 1300)])
def test_dual_group128_packed(gpu, shape):
    # one packed word spans four 128-column tiles: each tile stores its own byte
    _check(si.cast_workload(*shape, seed=si.SEED_B), oracle.SF_PACKED_UE8M0, mn_major=True, gran=128)


# fp32 input ("deep-gemm: fused per-token FP8 cast in Triton" tests bf16 and fp32
# inputs): every group size and scale format, ragged and single-row shapes, the
# fp32 extremes of the cast workloads (an all-zero group and a x1e4 group)
@pytest.mark.parametrize("shape", [(1, 512), (7, 4096), (129, 7168), (64, 1000), (129, 257), (5, 3), (300, 1000),
                                   (3000, 4096)])
@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("fmt", [oracle.SF_FP32, oracle.SF_UE8M0, oracle.SF_PACKED_UE8M0],
                         ids=["fp32", "ue8m0", "packed"])
def test_dual_fp32_input(gpu, shape, gran, fmt):
    _check(si.cast_workload(*shape, seed=si.SEED_A, dtype=torch.float32), fmt, mn_major=True, gran=gran)


def test_dual_fp32_input_extremes_row_major(gpu):
    # fp32 values beyond the bf16 grid: huge, tiny and subnormal magnitudes, row-major scales
    x = si.randn((256, 384), 5, 1.0, torch.float32)
    x[0, :128] *= 1e36
    x[1, 128:256] *= 1e-36
    x[:, 300] = 1e-42
    x[200:, 7] = -3.4e38
    for gran in (32, 128):
        for fmt in (oracle.SF_FP32, oracle.SF_UE8M0, oracle.SF_PACKED_UE8M0):
            _check(x, fmt, mn_major=False, gran=gran)


@pytest.mark.parametrize("shape", [(300, 200), (1000, 64)])
@pytest.mark.parametrize("gran_fmt", [(128, oracle.SF_FP32), (32, oracle.SF_FP32), (32, oracle.SF_PACKED_UE8M0),
                                      (128, oracle.SF_PACKED_UE8M0)], ids=["g128", "g32", "g32packed", "g128packed"])
def test_dual_row_major_scales(gpu, shape, gran_fmt):
    gran, fmt = gran_fmt
    _check(si.cast_workload(*shape, seed=si.SEED_B), fmt, mn_major=False, gran=gran)


@pytest.mark.parametrize("shape", [(8192, 7168), (8192, 4096)], ids=["x", "dY"])
def test_dual_linear_operands(gpu, shape):
    # the linear step's x [tokens, in] and dY [tokens, out] at full size
    _check(si.randn(shape, si.SEED_A if shape[1] == 7168 else si.SEED_DY), oracle.SF_FP32, mn_major=True)


@pytest.mark.parametrize("shape", [(8192, 7168), (4096, 7168)], ids=["x", "W"])
def test_dual_group32_packed_linear_operands(gpu, shape):
    # the group-32 recipe's x (and x^T), and W (and W^T), at full size
    _check(si.randn(shape, si.SEED_A if shape[0] == 8192 else si.SEED_B), oracle.SF_PACKED_UE8M0, mn_major=True,
           gran=32)


def test_dual_zero_size_is_noop(gpu):
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((0, 256), dtype=torch.uint8, device="cuda")
    qT = torch.empty((256, 16), dtype=torch.uint8, device="cuda")[:, :0]
    sf = fg.mn_major_scales(0, 2)
    sfT = fg.mn_major_scales(256, 0)
    fg.cast_per_token_dual(x, q, sf, qT, sfT)
    torch.cuda.synchronize()
