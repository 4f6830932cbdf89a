"""GPU parity of the casts against the oracle: bit-exact E4M3 bytes and scale
bits ("DeepGEMM Essentials", Parts 3-4; options of "deep-gemm: fused
per-token FP8 cast in Triton"), plus writes confined to the given views."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import gpu_cast_per_token, oracle_sf_bits, say, sentinel_u8

pytestmark = pytest.mark.gpu

FMTS = [oracle.SF_FP32, oracle.SF_UE8M0, oracle.SF_PACKED_UE8M0]
_cache = {}


def _oracle_tok(x_cpu, gran, fmt, transpose=False):
    key = (id(x_cpu), gran, fmt, transpose)
    if key not in _cache:
        _cache[key] = oracle.cast_per_token(si.host_array(x_cpu), gran, fmt, transpose=transpose)
    return _cache[key]


_inputs = {}


def _cast_input(shape, dtype):
    key = (shape, dtype)
    if key not in _inputs:
        _inputs.clear()
        _cache.clear()
        _inputs[key] = si.cast_workload(*shape, seed=si.SEED_A, dtype=dtype)
    return _inputs[key]


def _check_tok(x_cpu, gran, fmt, mn_major=False, transpose=False, sf_pad=4, sf_align=4):
    q, sf, qbuf, sbuf, (q_ld, units) = gpu_cast_per_token(x_cpu, gran, fmt, mn_major, transpose, q_pad=16,
                                                          sf_pad=sf_pad, sf_align=sf_align)
    oq, osf = _oracle_tok(x_cpu, gran, fmt, transpose)
    assert np.array_equal(q, oq), "E4M3 bytes differ"
    assert np.array_equal(sf, oracle_sf_bits(osf)), "scale bits differ"
    # nothing outside the views changed
    rows, cols = oq.shape
    qb = qbuf.cpu().numpy()
    assert (qb[:, cols:] == 0xA5).all()
    sb = sbuf.view(torch.int32).cpu().numpy()
    if mn_major:
        assert (sb[:, rows:] == -7).all()
    else:
        assert (sb[:, units:] == -7).all()


CAST_SHAPES = [(1, 512), (7, 4096), (129, 7168), (64, 1000), (3000, 4096)]


@pytest.mark.parametrize("shape", CAST_SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("fmt", FMTS, ids=["fp32", "ue8m0", "packed"])
def test_per_token_matrix(gpu, shape, dtype, gran, fmt):
    x = _cast_input(shape, dtype)
    _check_tok(x, gran, fmt, mn_major=False)
    _check_tok(x, gran, fmt, mn_major=True)


@pytest.mark.parametrize("cols", [1, 7, 33, 129])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("fmt", FMTS, ids=["fp32", "ue8m0", "packed"])
def test_per_token_single_row_tiny(gpu, cols, dtype, gran, fmt):
    # one token of 1..129 features: a lone partial group, or (129) an all-zero full group and a
    # partial one scaled by 1e4
    x = si.cast_workload(1, cols, seed=si.SEED_A + cols, dtype=dtype, special=cols > 128)
    _check_tok(x, gran, fmt, mn_major=False)
    _check_tok(x, gran, fmt, mn_major=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("fmt", FMTS, ids=["fp32", "ue8m0", "packed"])
def test_per_token_16384x4096(gpu, dtype, gran, fmt):
    x = _cast_input((16384, 4096), dtype)
    _check_tok(x, gran, fmt, mn_major=True)
    _check_tok(x, gran, fmt, mn_major=False)


@pytest.mark.parametrize("rows", [2049, 16383])
@pytest.mark.parametrize("gran,fmt", [(128, 0), (32, 0), (32, 2), (128, 2), (32, 1)])
def test_per_token_row_quads_partial(gpu, rows, gran, fmt):
    """MN-major scales with aligned columns and at least 8192 tasks take the row-quad
    order; rows % 4 != 0 leaves a last quad of 1 or 3 rows, whose scale store is
    element-wise."""
    x = _cast_input((rows, 4096), torch.bfloat16)
    _check_tok(x, gran, fmt, mn_major=True)


@pytest.mark.parametrize("tokens", [1, 64, 512, 4096])
def test_token_sweep_g32_packed(gpu, tokens):
    x = si.randn((tokens, 4096), si.SEED_A)
    _check_tok(x, 32, oracle.SF_PACKED_UE8M0, mn_major=True)


@pytest.mark.parametrize("shape", [(7, 4096), (129, 7168), (64, 1000)])
@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("fmt", FMTS, ids=["fp32", "ue8m0", "packed"])
def test_per_token_mn_major_odd_ld(gpu, shape, gran, fmt):
    """MN-major scales whose columns are not 16-byte aligned (ld = rows + 1): the
    row-major task order stores each scale on its own; an aligned ld takes the
    row-quad order with 16-byte stores of four rows (the other tests)."""
    x = _cast_input(shape, torch.bfloat16)
    _check_tok(x, gran, fmt, mn_major=True, sf_pad=1, sf_align=1)


def test_ragged_columns_strided_rows(gpu):
    """cols % 8 != 0 through a row-strided view of a wider buffer."""
    base = si.randn((100, 1008), 7)
    xv = base[:, :1003]
    x = base.cuda()[:, :1003]
    for gran in (32, 128):
        for fmt in FMTS:
            G = -(-1003 // gran)
            units = -(-G // 4) if fmt == 2 else G
            q = sentinel_u8((100, 1008))
            sf = torch.zeros((100, units), dtype=torch.int32 if fmt == 2 else torch.float32, device="cuda")
            say("ragged", gran, fmt)
            import fine_grained_block_token_amd as fg
            fg.cast_per_token(x, q[:, :1003], sf, gran, fmt)
            oq, osf = oracle.cast_per_token(si.host_array(xv.contiguous()), gran, fmt)
            qh = q.cpu().numpy()
            assert np.array_equal(qh[:, :1003], oq) and (qh[:, 1003:] == 0xA5).all()
            assert np.array_equal(sf.view(torch.int32).cpu().numpy().view(np.uint32), oracle_sf_bits(osf))


def test_empty_is_noop(gpu):
    import fine_grained_block_token_amd as fg
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((0, 512), dtype=torch.uint8, device="cuda")
    sf = torch.zeros((0, 4), dtype=torch.float32, device="cuda")
    fg.cast_per_token(x, q, sf, 128, 0)


def test_fp32_extremes(gpu):
    x = si.randn((8, 512), 5, 1.0, torch.float32)
    x[0, :128] *= 1e36
    x[1, 128:256] *= 1e-30
    x[2, :] = 0
    x[3, 0] = 3.4e38
    x[4, 5] = -0.0
    x[5, :] = -x[5, :].abs()
    for gran in (32, 128):
        for fmt in FMTS:
            _check_tok(x, gran, fmt)


def test_e4m3_rounding_sweep(gpu):
    """Every group holds 448, so its multiplier is exactly 1 and each other element is
    rounded as itself: a sweep of fp32 values in [-448, 448] against the oracle."""
    limit = int(np.float32(448.0).view(np.uint32))
    bits = np.arange(0, limit + 1, 61, dtype=np.uint64).astype(np.uint32)
    mids = []
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = oracle.e4m3_value(codes)
    for a, b in zip(vals[:-1], vals[1:]):
        m = np.float32((a + b) / 2)
        mids += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    v = np.concatenate([bits.view(np.float32), np.array(mids, np.float32)])
    v = np.concatenate([v, -v])
    per_row = 127
    rows = -(-v.size // per_row)
    buf = np.zeros(rows * per_row, np.float32)
    buf[: v.size] = v
    x = np.concatenate([np.full((rows, 1), 448.0, np.float32), buf.reshape(rows, per_row)], axis=1)
    xt = torch.from_numpy(x)
    q, sf, *_ = gpu_cast_per_token(xt, 128, oracle.SF_FP32)
    assert (sf == 0x3F800000).all()
    want = oracle.e4m3_round(x)
    assert np.array_equal(q, want)


# ---------------------------------------------------------------------------
# transposed views (the wgrad operands)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(8192, 4096), (8192, 7168)])
def test_transposed_linear_operands(gpu, shape):
    x = si.randn(shape, si.SEED_DY if shape[1] == 4096 else si.SEED_A)
    _check_tok(x, 128, oracle.SF_FP32, mn_major=True, transpose=True)


@pytest.mark.parametrize("shape", [(300, 200), (256, 64), (129, 8), (1000, 136)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_transposed_ragged(gpu, shape, dtype):
    x = si.randn(shape, 11, 1.0, dtype)
    x[: min(128, shape[0]), 0] = 0          # an all-zero group in feature 0
    for gran in (32, 128):
        for fmt in FMTS:
            _check_tok(x, gran, fmt, mn_major=True, transpose=True)
            _check_tok(x, gran, fmt, mn_major=False, transpose=True)


# ---------------------------------------------------------------------------
# per-block cast
# ---------------------------------------------------------------------------

def _gpu_block(x_cpu, fmt, trans, pad=16, x_dev=None):
    import fine_grained_block_token_amd as fg
    rows, cols = x_cpu.shape
    x = x_cpu.cuda() if x_dev is None else x_dev
    br, bc = -(-rows // 128), -(-cols // 128)
    qbuf = sentinel_u8((rows, -(-(cols + pad) // 16) * 16))
    sf = torch.full((br, bc + 1), -7, dtype=torch.int32, device="cuda").view(torch.float32)
    qT = sfT = qTbuf = None
    if trans:
        qTbuf = sentinel_u8((cols, -(-(rows + pad) // 16) * 16))
        qT = qTbuf[:, :rows]
        sfT = torch.full((bc, br + 1), -7, dtype=torch.int32, device="cuda").view(torch.float32)
    say("cast_per_block", (rows, cols), x_cpu.dtype, fmt, trans)
    fg.cast_per_block(x, qbuf[:, :cols], sf[:, :bc], qT, None if sfT is None else sfT[:, :br], fmt)
    torch.cuda.synchronize()
    return qbuf.cpu().numpy(), sf.view(torch.int32).cpu().numpy(), \
        (None if qTbuf is None else qTbuf.cpu().numpy()), (None if sfT is None else sfT.view(torch.int32).cpu().numpy())


@pytest.mark.parametrize("shape", [(4096, 7168), (7168, 4096), (300, 512), (128, 128), (1, 256)])
@pytest.mark.parametrize("fmt", [0, 1], ids=["fp32", "ue8m0"])
def test_per_block(gpu, shape, fmt):
    x = si.randn(shape, si.SEED_B)
    x[:1, :1] = 3000.0                       # one block with a large amax
    qb, sfb, qTb, sfTb = _gpu_block(x, fmt, trans=True)
    oq, osf = oracle.cast_per_block(si.host_array(x), fmt)
    rows, cols = shape
    br, bc = osf.shape
    assert np.array_equal(qb[:, :cols], oq) and (qb[:, cols:] == 0xA5).all()
    assert np.array_equal(sfb[:, :bc].view(np.uint32), oracle_sf_bits(osf)) and (sfb[:, bc:] == -7).all()
    assert np.array_equal(qTb[:, :rows], oq.T) and (qTb[:, rows:] == 0xA5).all()
    assert np.array_equal(sfTb[:, :br].view(np.uint32), oracle_sf_bits(osf).T) and (sfTb[:, br:] == -7).all()


@pytest.mark.parametrize("shape", [(300, 500), (129, 7)])
def test_per_block_ragged_fp32(gpu, shape):
    base = si.randn((shape[0], 512), 3, 1.0, torch.float32)
    xv = base[:, : shape[1]].contiguous()
    qb, sfb, _, _ = _gpu_block(xv, 0, trans=False, x_dev=base.cuda()[:, : shape[1]])
    oq, osf = oracle.cast_per_block(si.host_array(xv), 0)
    assert np.array_equal(qb[:, : shape[1]], oq)
    assert np.array_equal(sfb[:, : osf.shape[1]].view(np.uint32), oracle_sf_bits(osf))
