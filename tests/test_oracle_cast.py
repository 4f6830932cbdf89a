"""Pins for the oracle's per-token and per-block casts (CPU only).

What the casts compute is fixed by "DeepGEMM Essentials: High-Performance
FP8 Matrix Multiplication", Part 3 (per token, 1 x 128 groups) and Part 4
(128 x 128 blocks), with the group-32, UE8M0 and packed-UE8M0 options and the
bf16/fp32 inputs of "deep-gemm: fused per-token FP8 cast in Triton".

Independent pins:
* hand-worked groups (tests/golden/cast_hand_groups.txt);
* a second implementation built from PyTorch tensor ops (reshape, amax,
  clamp, PyTorch's own ``448.0 / amax``, ``frexp`` and its float8 converter)
  over the page-3 test matrix: {bf16, fp32} x {g32, g128} x {fp32, UE8M0,
  packed UE8M0} x five shapes, plus the zero and x1e4 groups;
* invariants: the amax element of an unclamped fp32-scale group becomes
  +-448; UE8M0 scales are the least power of two >= amax/448; the partial
  last group equals zero padding; a strided (transposed) read equals a
  contiguous copy; the block cast commutes with transposition.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from golden_io import cast_hand_groups

FMT = {"fp32": oracle.SF_FP32, "ue8m0": oracle.SF_UE8M0, "packed": oracle.SF_PACKED_UE8M0}


# ---------------------------------------------------------------------------
# a second implementation from PyTorch tensor ops
# ---------------------------------------------------------------------------

def _pow2(e: torch.Tensor) -> torch.Tensor:
    return ((e.to(torch.int32) + 127) << 23).view(torch.float32)


def torch_cast_per_token(x: torch.Tensor, gran: int, fmt: int):
    rows, cols = x.shape
    groups = -(-cols // gran)
    padded = torch.zeros(rows, groups * gran, dtype=x.dtype)
    padded[:, :cols] = x
    g = padded.view(rows, groups, gran).float()
    amax = g.abs().amax(dim=2).clamp(min=1e-4)
    if fmt == oracle.SF_FP32:
        sf = amax / 448.0
        mult = 448.0 / amax                   # PyTorch: reciprocal, then times 448
    else:
        mant, ex = torch.frexp(amax / 448.0)  # s = mant * 2^ex, mant in [0.5, 1)
        e = torch.where(mant == 0.5, ex - 1, ex)
        sf, mult = _pow2(e), _pow2(-e)
    q = (g * mult.unsqueeze(2)).to(torch.float8_e4m3fn).view(torch.uint8)
    q = q.reshape(rows, groups * gran)[:, :cols].contiguous().numpy()
    if fmt == oracle.SF_PACKED_UE8M0:
        words = -(-groups // 4)
        b = torch.zeros(rows, 4 * words, dtype=torch.uint8)
        b[:, :groups] = (e + 127).to(torch.uint8)
        return q, b.view(torch.int32).numpy().view(np.uint32)
    return q, sf.numpy()


def torch_cast_per_block(x: torch.Tensor, fmt: int):
    rows, cols = x.shape
    br, bc = -(-rows // 128), -(-cols // 128)
    padded = torch.zeros(br * 128, bc * 128, dtype=x.dtype)
    padded[:rows, :cols] = x
    blocks = padded.view(br, 128, bc, 128).float()
    amax = blocks.abs().amax(dim=(1, 3)).clamp(min=1e-4)
    if fmt == oracle.SF_FP32:
        sf, mult = amax / 448.0, 448.0 / amax
    else:
        mant, ex = torch.frexp(amax / 448.0)
        e = torch.where(mant == 0.5, ex - 1, ex)
        sf, mult = _pow2(e), _pow2(-e)
    q = (blocks * mult[:, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(br * 128, bc * 128)[:rows, :cols].contiguous().numpy(), sf.numpy()


# ---------------------------------------------------------------------------
# hand-worked groups
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", sorted(cast_hand_groups()))
def test_hand_groups(name):
    case = cast_hand_groups()[name]
    vals = case["values"]
    row = np.zeros(128, dtype=np.float32)
    row[: len(vals)] = vals
    x = torch.from_numpy(row[None, :]).to(torch.bfloat16)
    assert torch.equal(x.float()[0, : len(vals)], torch.tensor(vals))  # values are exact in bf16
    fmts = ["fp32"] if case["fmt"] == "fp32" else ["ue8m0", "packed"]
    for f in fmts:
        q, sf = oracle.cast_per_token(si.bf16_bits(x), 128, FMT[f])
        codes = case["codes"]
        if len(codes) == 1:          # one code for the whole group
            assert (q[0] == codes[0]).all()
        else:
            assert list(q[0, : len(codes)]) == codes
            assert (q[0, len(codes):] == 0).all()
        if f == "packed":
            assert int(sf[0, 0]) == case["packed_byte"]      # group 0 in byte 0, pad bytes 0
        else:
            assert int(sf.view(np.uint32)[0, 0]) == case["scale_bits"]


# ---------------------------------------------------------------------------
# the page-3 test matrix against the PyTorch-op implementation
# ---------------------------------------------------------------------------

SHAPES = [(1, 512), (7, 4096), (129, 7168), (64, 1000), (3000, 4096)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_matches_torch_definition(shape, dtype):
    x = si.cast_workload(*shape, seed=si.SEED_A, dtype=dtype)
    xa = si.host_array(x)
    for gran in (32, 128):
        for f in ("fp32", "ue8m0", "packed"):
            q, sf = oracle.cast_per_token(xa, gran, FMT[f])
            tq, tsf = torch_cast_per_token(x, gran, FMT[f])
            assert np.array_equal(q, tq), (shape, dtype, gran, f)
            assert np.array_equal(sf.view(np.uint32), tsf.view(np.uint32)), (shape, dtype, gran, f)


def test_fp32_input_extremes():
    """fp32 input reaches scales bf16 cannot: huge and tiny groups."""
    x = si.randn((4, 512), 5, 1.0, torch.float32)
    x[0, :128] *= 1e36          # amax/448 near 2^113
    x[1, 128:256] *= 1e-30      # clamped group
    x[2, :] = 0
    x[3, 0] = 3.4e38            # 1/amax is an fp32 subnormal
    for gran in (32, 128):
        for f in ("fp32", "ue8m0", "packed"):
            q, sf = oracle.cast_per_token(x.numpy(), gran, FMT[f])
            tq, tsf = torch_cast_per_token(x, gran, FMT[f])
            assert np.array_equal(q, tq) and np.array_equal(sf.view(np.uint32), tsf.view(np.uint32))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_fp32_groups_reach_448():
    x = si.cast_workload(129, 7168)
    q, sf = oracle.cast_per_token(si.host_array(x), 128, oracle.SF_FP32)
    mag = (q & 0x7F).reshape(129, 56, 128).max(axis=2)
    clamped = x.float().abs().reshape(129, 56, 128).amax(dim=2).numpy() < np.float32(1e-4)
    assert (mag[~clamped] == 0x7E).all()
    assert clamped.sum() == 1 and (mag[clamped] == 0).all()          # the all-zero group


@pytest.mark.parametrize("gran", [32, 128])
def test_ue8m0_bounds(gran):
    x = si.cast_workload(64, 1000)
    q, sf = oracle.cast_per_token(si.host_array(x), gran, oracle.SF_UE8M0)
    G = sf.shape[1]
    bits = sf.view(np.uint32)
    assert ((bits & 0x7FFFFF) == 0).all()                              # powers of two
    xs = np.zeros((64, G * gran), np.float32)
    xs[:, :1000] = x.float().numpy()
    amax = np.maximum(np.abs(xs).reshape(64, G, gran).max(axis=2), np.float32(1e-4))
    s = amax / np.float32(448.0)
    assert (sf >= s).all() and (sf / 2 < s).all()
    vals = np.abs(oracle.e4m3_value(q))
    qpad = np.zeros((64, G * gran))
    qpad[:, :1000] = vals
    gmax = qpad.reshape(64, G, gran).max(axis=2)
    live = amax > np.float32(1e-4)
    # amax * 2^-e lies in (224, 448]; rounding is monotone and 224 is a code
    assert (gmax[live] >= 224).all() and (gmax[live] <= 448).all()


def test_packed_matches_unpacked():
    x = si.cast_workload(129, 7168)
    for gran in (32, 128):
        _, sfu = oracle.cast_per_token(si.host_array(x), gran, oracle.SF_UE8M0)
        _, sfp = oracle.cast_per_token(si.host_array(x), gran, oracle.SF_PACKED_UE8M0)
        assert np.array_equal(oracle.unpack_ue8m0(sfp, sfu.shape[1]), sfu)
        G = sfu.shape[1]
        pad = sfp.view(np.uint8).reshape(129, -1)[:, G:]
        assert (pad == 0).all()


@pytest.mark.parametrize("gran", [32, 128])
def test_partial_group_equals_zero_padding(gran):
    x = si.cast_workload(64, 1000)
    padded = torch.zeros(64, 1024, dtype=torch.bfloat16)
    padded[:, :1000] = x
    for f in ("fp32", "ue8m0"):
        q, sf = oracle.cast_per_token(si.host_array(x), gran, FMT[f])
        qp, sfp = oracle.cast_per_token(si.host_array(padded), gran, FMT[f])
        assert np.array_equal(q, qp[:, :1000])
        assert np.array_equal(sf.view(np.uint32), sfp.view(np.uint32)[:, : sf.shape[1]])
    assert oracle.cast_per_token(si.host_array(x), 128)[1].shape == (64, 8)
    assert oracle.cast_per_token(si.host_array(x), 32)[1].shape == (64, 32)


@pytest.mark.parametrize("shape", [(256, 384), (300, 500), (7, 1000)])
def test_transposed_read_equals_contiguous(shape):
    x = si.randn(shape, 3)
    for gran in (32, 128):
        for f in ("fp32", "packed"):
            q, sf = oracle.cast_per_token(si.host_array(x), gran, FMT[f], transpose=True)
            qc, sfc = oracle.cast_per_token(si.host_array(x.t().contiguous()), gran, FMT[f])
            assert np.array_equal(q, qc) and np.array_equal(sf.view(np.uint32), sfc.view(np.uint32))


# ---------------------------------------------------------------------------
# per-block cast
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(256, 512), (300, 500), (128, 1000), (7, 7)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_block_cast_matches_torch_definition(shape, dtype):
    x = si.randn(shape, si.SEED_B, 1.0, dtype)
    x[: min(128, shape[0]), : min(128, shape[1])] *= 1e4 if shape[0] > 128 else 1
    for f in ("fp32", "ue8m0"):
        q, sf = oracle.cast_per_block(si.host_array(x), FMT[f])
        tq, tsf = torch_cast_per_block(x, FMT[f])
        assert np.array_equal(q, tq) and np.array_equal(sf.view(np.uint32), tsf.view(np.uint32))


@pytest.mark.parametrize("shape", [(300, 500), (256, 384), (129, 7)])
def test_block_cast_commutes_with_transpose(shape):
    x = si.randn(shape, 4)
    for f in ("fp32", "ue8m0"):
        q, sf = oracle.cast_per_block(si.host_array(x), FMT[f])
        qt, sft = oracle.cast_per_block(si.host_array(x.t().contiguous()), FMT[f])
        assert np.array_equal(q.T, qt) and np.array_equal(sf.T, sft)


def test_block_cast_zero_block():
    x = torch.zeros(256, 256, dtype=torch.bfloat16)
    x[128:, 128:] = si.randn((128, 128), 1)
    q, sf = oracle.cast_per_block(si.host_array(x), oracle.SF_FP32)
    assert sf.view(np.uint32)[0, 0] == 0x346FACAD and (q[:128, :128] == 0).all()
