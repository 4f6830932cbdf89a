"""The C ABI on the CPU: the library loads, exports every entry point that
include/fgfp8.h declares, and rejects invalid arguments on the host before
touching the GPU (status -1, nothing launched).  No compute call is made."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fgfp8.h")


@pytest.fixture(scope="module")
def lib():
    import fine_grained_block_token_amd as fg
    return fg.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("cast_per_token", "cast_per_block", "cast_per_token_dual", "gemm_fp8_nt_bf16",
              "wgrad_gemm_fp8_nt_fp32", "m_grouped_gemm_fp8_nt_bf16_contiguous", "gemm_fp8_nt_bf16_cast",
              "gemm_fp8_nt_bf16_ue8m0_g32", "wgrad_gemm_fp8_nt_fp32_ue8m0_g32",
              "m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous", "wgrad_gemm_fp8_nt_fp32_ue8m0",
              "gemm_fp8_nt_bf16_ue8m0", "gemm_fp8_nt_bf16_splitk", "gemm_fp8_nt_bf16_splitk_workspace",
              "gemm_fp8_nt_bf16_splitk_noalloc", "fgfp8_status_string"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for rc in (0, -1, -2, -3, -4):
        assert lib.fgfp8_status_string(rc)
    assert b"invalid" in lib.fgfp8_status_string(-1)
    assert b"scratch" in lib.fgfp8_status_string(-4)


# fake but 16-byte aligned addresses: validation rejects before any access
P = ctypes.c_void_p(0x10000)
Q = ctypes.c_void_p(0x20000)
S = ctypes.c_void_p(0x30000)


def tok(lib, **kw):
    a = dict(x=P, dt=0, rows=4, cols=256, srow=256, scol=1, gran=128, fmt=0, q=Q, qld=256, sf=S,
             sfr=2, sfg=1, st=None)
    a.update(kw)
    return lib.cast_per_token(a["x"], a["dt"], a["rows"], a["cols"], a["srow"], a["scol"], a["gran"],
                              a["fmt"], a["q"], a["qld"], a["sf"], a["sfr"], a["sfg"], a["st"])


@pytest.mark.parametrize("kw", [
    dict(gran=64), dict(fmt=3), dict(dt=2), dict(rows=-1),
    dict(x=None), dict(q=None), dict(sf=None),
    dict(srow=255), dict(scol=2), dict(srow=7, scol=3),
    dict(x=ctypes.c_void_p(0x10008)), dict(q=ctypes.c_void_p(0x20004)), dict(qld=200), dict(qld=260),
    dict(sfr=1, sfg=1), dict(sfr=1, sfg=3), dict(sf=ctypes.c_void_p(0x30002)),
])
def test_cast_per_token_rejects(lib, kw):
    assert tok(lib, **kw) == -1


def test_cast_per_token_zero_size_is_ok(lib):
    assert tok(lib, rows=0) == 0 and tok(lib, cols=0) == 0


def blk(lib, **kw):
    a = dict(x=P, dt=0, rows=256, cols=256, xld=256, fmt=0, q=Q, qld=256, sf=S, sfld=2, qT=None,
             qTld=0, sfT=None, sfTld=0, st=None)
    a.update(kw)
    return lib.cast_per_block(a["x"], a["dt"], a["rows"], a["cols"], a["xld"], a["fmt"], a["q"], a["qld"],
                              a["sf"], a["sfld"], a["qT"], a["qTld"], a["sfT"], a["sfTld"], a["st"])


@pytest.mark.parametrize("kw", [
    dict(fmt=2), dict(xld=100), dict(qld=252), dict(sfld=1), dict(qT=Q, qTld=256),
    dict(sfT=S, sfTld=2), dict(qT=Q, qTld=255, sfT=S, sfTld=2), dict(x=None),
])
def test_cast_per_block_rejects(lib, kw):
    assert blk(lib, **kw) == -1


def dual(lib, **kw):
    a = dict(x=P, dt=0, rows=256, cols=384, xld=384, gran=128, fmt=0, q=Q, qld=384, sf=S, sfr=1, sfg=256,
             qT=Q, qTld=256, sfT=S, sfTr=1, sfTg=384, st=None)
    a.update(kw)
    return lib.cast_per_token_dual(a["x"], a["dt"], a["rows"], a["cols"], a["xld"], a["gran"], a["fmt"], a["q"],
                                   a["qld"], a["sf"], a["sfr"], a["sfg"], a["qT"], a["qTld"], a["sfT"], a["sfTr"],
                                   a["sfTg"], a["st"])


@pytest.mark.parametrize("kw", [
    dict(dt=2), dict(dt=-1), dict(dt=1, xld=386), dict(fmt=3), dict(gran=64), dict(gran=0),
    dict(fmt=2, gran=32, sfr=2, sfg=1),
    dict(fmt=2, gran=32, sfTr=1, sfTg=1), dict(gran=32, sfr=11, sfg=1), dict(rows=-1), dict(x=None), dict(q=None), dict(sf=None), dict(qT=None),
    dict(sfT=None), dict(xld=380), dict(xld=388), dict(x=ctypes.c_void_p(0x10008)), dict(qld=380),
    dict(q=ctypes.c_void_p(0x20004)), dict(qTld=255), dict(qTld=264), dict(qT=ctypes.c_void_p(0x20008)),
    dict(sfg=255), dict(sfr=2, sfg=1), dict(sfTg=383), dict(sfTr=1, sfTg=1), dict(sf=ctypes.c_void_p(0x30002)),
])
def test_cast_per_token_dual_rejects(lib, kw):
    assert dual(lib, **kw) == -1


def test_cast_per_token_dual_zero_size_is_ok(lib):
    assert dual(lib, rows=0) == 0 and dual(lib, cols=0) == 0 and dual(lib, rows=0, gran=32, fmt=2) == 0


def gemm(lib, **kw):
    a = dict(A=P, lda=256, sa=S, fmt=0, sald=128, B=Q, ldb=256, sb=S, sbld=2, D=P, ldd=256, m=128,
             n=256, k=256, st=None)
    a.update(kw)
    return lib.gemm_fp8_nt_bf16(a["A"], a["lda"], a["sa"], a["fmt"], a["sald"], a["B"], a["ldb"], a["sb"],
                                a["sbld"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [
    dict(k=200), dict(k=0), dict(lda=200), dict(ldb=250), dict(sald=100), dict(sbld=1), dict(ldd=100),
    dict(ldd=252), dict(fmt=5), dict(A=None), dict(D=ctypes.c_void_p(0x10004)), dict(m=-1),
    dict(lda=1 << 24), dict(ldb=1 << 24),
])
def test_gemm_rejects(lib, kw):
    assert gemm(lib, **kw) == -1


def test_gemm_zero_size_is_ok(lib):
    assert gemm(lib, m=0) == 0 and gemm(lib, n=0) == 0


def wgrad(lib, **kw):
    a = dict(A=P, lda=256, sa=S, sald=128, B=Q, ldb=256, sb=S, sbld=256, D=P, ldd=256, m=128, n=256,
             k=256, st=None)
    a.update(kw)
    return lib.wgrad_gemm_fp8_nt_fp32(a["A"], a["lda"], a["sa"], a["sald"], a["B"], a["ldb"], a["sb"],
                                      a["sbld"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [dict(sbld=100), dict(k=100), dict(ldd=254), dict(sb=None), dict(lda=1 << 24)])
def test_wgrad_rejects(lib, kw):
    assert wgrad(lib, **kw) == -1


def grouped(lib, **kw):
    a = dict(A=P, lda=256, sa=S, fmt=0, sald=256, B=Q, ldb=256, bes=256 * 256, sb=S, sbld=2, sbes=4,
             mi=S, E=4, D=P, ldd=256, m=256, n=256, k=256, st=None)
    a.update(kw)
    return lib.m_grouped_gemm_fp8_nt_bf16_contiguous(
        a["A"], a["lda"], a["sa"], a["fmt"], a["sald"], a["B"], a["ldb"], a["bes"], a["sb"], a["sbld"], a["sbes"],
        a["mi"], a["E"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [
    dict(mi=None), dict(mi=ctypes.c_void_p(0x30002)), dict(E=0), dict(E=-1), dict(bes=255 * 256 + 200),
    dict(bes=256 * 256 + 8), dict(sbes=3), dict(k=200), dict(sald=100), dict(fmt=7), dict(ldd=100),
    dict(lda=1 << 24),
])
def test_m_grouped_rejects(lib, kw):
    assert grouped(lib, **kw) == -1


def test_m_grouped_zero_size_is_ok(lib):
    assert grouped(lib, m=0) == 0 and grouped(lib, n=0) == 0


def gcast(lib, **kw):
    a = dict(A=P, lda=256, sa=S, fmt=0, sald=128, B=Q, ldb=256, sb=S, sbld=2, D=P, ldd=256, qfmt=0, q=Q, qld=256,
             qsf=S, qsr=1, qsg=128, m=128, n=256, k=256, st=None)
    a.update(kw)
    return lib.gemm_fp8_nt_bf16_cast(a["A"], a["lda"], a["sa"], a["fmt"], a["sald"], a["B"], a["ldb"], a["sb"],
                                     a["sbld"], a["D"], a["ldd"], a["qfmt"], a["q"], a["qld"], a["qsf"], a["qsr"],
                                     a["qsg"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [
    dict(qfmt=2), dict(q=None), dict(qsf=None), dict(qld=250), dict(qld=258), dict(q=ctypes.c_void_p(0x20002)),
    dict(qsr=1, qsg=100), dict(qsr=1, qsg=1), dict(ldd=100), dict(D=ctypes.c_void_p(0x10004)), dict(k=200),
])
def test_gemm_cast_rejects(lib, kw):
    assert gcast(lib, **kw) == -1


def test_gemm_cast_zero_size_is_ok(lib):
    assert gcast(lib, m=0) == 0 and gcast(lib, n=0) == 0


def g32(lib, **kw):
    a = dict(A=P, lda=256, sa=S, sald=128, B=Q, ldb=256, sb=S, sbld=256, D=P, ldd=256, m=128, n=256, k=256, st=None)
    a.update(kw)
    return lib.gemm_fp8_nt_bf16_ue8m0_g32(a["A"], a["lda"], a["sa"], a["sald"], a["B"], a["ldb"], a["sb"], a["sbld"],
                                          a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [dict(sbld=255), dict(sald=127), dict(k=96), dict(sa=None), dict(sb=None),
                                dict(ldd=252), dict(A=ctypes.c_void_p(0x10008))])
def test_g32_rejects(lib, kw):
    assert g32(lib, **kw) == -1


def test_g32_zero_size_is_ok(lib):
    assert g32(lib, m=0) == 0 and g32(lib, n=0) == 0


def wg32(lib, **kw):
    a = dict(A=P, lda=256, sa=S, sald=128, B=Q, ldb=256, sb=S, sbld=256, D=P, ldd=256, m=128, n=256, k=256, st=None)
    a.update(kw)
    return lib.wgrad_gemm_fp8_nt_fp32_ue8m0_g32(a["A"], a["lda"], a["sa"], a["sald"], a["B"], a["ldb"], a["sb"],
                                                a["sbld"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [dict(sbld=255), dict(sald=127), dict(k=96), dict(sa=None), dict(sb=None), dict(D=None),
                                dict(ldd=254), dict(ldd=255), dict(D=ctypes.c_void_p(0x10008)),
                                dict(A=ctypes.c_void_p(0x10008)), dict(lda=1 << 24)])
def test_wgrad_g32_rejects(lib, kw):
    assert wg32(lib, **kw) == -1


def test_wgrad_g32_zero_size_is_ok(lib):
    assert wg32(lib, m=0) == 0 and wg32(lib, n=0) == 0


MI = ctypes.c_void_p(0x40000)


def gg32(lib, **kw):
    a = dict(A=P, lda=256, sa=S, sald=384, B=Q, ldb=256, bes=256 * 256, sb=S, sbld=256, sbes=512, mi=MI, ne=4,
             D=P, ldd=256, m=384, n=256, k=256, st=None)
    a.update(kw)
    return lib.m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(
        a["A"], a["lda"], a["sa"], a["sald"], a["B"], a["ldb"], a["bes"], a["sb"], a["sbld"], a["sbes"], a["mi"],
        a["ne"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [dict(sbld=255), dict(sald=383), dict(k=96), dict(sb=None), dict(mi=None),
                                dict(mi=ctypes.c_void_p(0x40002)), dict(ne=0), dict(bes=256 * 256 - 1),
                                dict(bes=256 * 255 + 256 + 8), dict(sbes=511), dict(ldd=252),
                                dict(D=ctypes.c_void_p(0x10008))])
def test_grouped_g32_rejects(lib, kw):
    assert gg32(lib, **kw) == -1


def test_grouped_g32_zero_size_is_ok(lib):
    assert gg32(lib, m=0) == 0 and gg32(lib, n=0) == 0


def wue(lib, **kw):
    a = dict(A=P, lda=256, sa=S, fmt=1, sald=128, B=Q, ldb=256, sb=S, sbld=256, D=P, ldd=256, m=128, n=256, k=256,
             st=None)
    a.update(kw)
    return lib.wgrad_gemm_fp8_nt_fp32_ue8m0(a["A"], a["lda"], a["sa"], a["fmt"], a["sald"], a["B"], a["ldb"], a["sb"],
                                            a["sbld"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [dict(fmt=0), dict(fmt=3), dict(sbld=255), dict(sald=127), dict(k=96), dict(sa=None),
                                dict(sb=None), dict(D=None), dict(ldd=254), dict(D=ctypes.c_void_p(0x10008))])
def test_wgrad_ue8m0_rejects(lib, kw):
    assert wue(lib, **kw) == -1


def test_wgrad_ue8m0_zero_size_is_ok(lib):
    assert wue(lib, m=0) == 0 and wue(lib, n=0, fmt=2) == 0


def gue(lib, **kw):
    a = dict(A=P, lda=256, sa=S, fmt=1, sald=128, B=Q, ldb=256, sb=S, sbld=2, D=P, ldd=256, m=128, n=256, k=256,
             st=None)
    a.update(kw)
    return lib.gemm_fp8_nt_bf16_ue8m0(a["A"], a["lda"], a["sa"], a["fmt"], a["sald"], a["B"], a["ldb"], a["sb"],
                                      a["sbld"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [dict(fmt=0), dict(fmt=3), dict(sbld=1), dict(sald=127), dict(k=96), dict(sa=None),
                                dict(sb=None), dict(D=None), dict(ldd=252), dict(D=ctypes.c_void_p(0x10008))])
def test_gemm_ue8m0_rejects(lib, kw):
    assert gue(lib, **kw) == -1


def test_gemm_ue8m0_zero_size_is_ok(lib):
    assert gue(lib, m=0) == 0 and gue(lib, n=0, fmt=2) == 0


def splitk(lib, **kw):
    a = dict(A=P, lda=256, sa=S, fmt=0, sald=64, B=Q, ldb=256, sb=S, sbld=2, D=P, ldd=256, m=64, n=256, k=256,
             ws=ctypes.c_void_p(0x40000), wsb=1 << 20, st=None)
    a.update(kw)
    return lib.gemm_fp8_nt_bf16_splitk(a["A"], a["lda"], a["sa"], a["fmt"], a["sald"], a["B"], a["ldb"], a["sb"],
                                       a["sbld"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["ws"], a["wsb"],
                                       a["st"])


# m = 512, n = 256, k = 2048: 8 tiles of 128x128 in 2 K slices, a 1 MiB workspace
KSLICE = dict(m=512, sald=512, k=2048, lda=2048, ldb=2048, sbld=16)


@pytest.mark.parametrize("kw", [
    dict(k=200), dict(k=0), dict(lda=200), dict(sbld=1), dict(ldd=252), dict(fmt=5),
    dict(A=None), dict(ws=None), dict(ws=ctypes.c_void_p(0x40008)), dict(wsb=2 * 4 * 64 * 512 - 4),
    dict(D=ctypes.c_void_p(0x10004)), dict(m=-1), dict(KSLICE, ws=None), dict(KSLICE, wsb=(1 << 20) - 4),
    dict(KSLICE, sald=511), dict(KSLICE, ws=ctypes.c_void_p(0x40004)),
])
def test_splitk_rejects(lib, kw):
    assert splitk(lib, **kw) == -1


def test_splitk_zero_size_is_ok(lib):
    assert splitk(lib, m=0, ws=None, wsb=0) == 0 and splitk(lib, n=0, ws=None, wsb=0) == 0


def test_splitk_workspace_size(lib):
    ws = lib.gemm_fp8_nt_bf16_splitk_workspace
    assert ws(0, 4096, 7168) == 0 and ws(64, 0, 7168) == 0
    for bad in [(-1, 4096, 7168), (64, -1, 7168), (64, 4096, 0), (64, 4096, 100),
                (64, 1 << 40, 128 * 1024), (512, 4096, 100)]:
        assert ws(*bad) == -1
    # m > 64: one 128x128 fp32 slot per tile and K slice; with at most 128 tiles, S =
    # min(4, K blocks / 8) when that is 2 or more, else 0 (the plain kernel)
    slot = 128 * 128 * 4
    assert ws(512, 4096, 7168) == 128 * 4 * slot          # 32 MiB: the static scratch's size
    assert ws(200, 1000, 2048) == 16 * 2 * slot          # 16 K blocks: two slices of 8
    assert ws(65, 130, 3200) == 2 * 3 * slot             # 25 K blocks: three slices
    assert ws(128, 7168, 4096) == 56 * 4 * slot
    # beyond 256 workgroups a slice needs 12 K blocks: 96 and 112 tiles of 32 blocks take 2
    assert ws(384, 4096, 4096) == 96 * 2 * slot and ws(256, 7168, 4096) == 112 * 2 * slot
    for zero in [(65, 256, 256), (512, 4096, 1024), (4096, 4096, 7168), (512, 7168, 4096), (1024, 2176, 7168)]:
        assert ws(*zero) == 0                              # too few K blocks, or more than 128 tiles
    assert ws(1024, 2048, 7168) == 128 * 4 * slot          # 128 tiles: the most that take slices
    # two partial-sum slots per workgroup of 16*ceil(m/16) x 128 fp32 (16, 32 or 64 rows); the
    # workgroup count depends on n and k only, at least one per 8 units (128-column tile x K
    # block) and at most one per unit
    for n, k in [(7168, 4096), (4096, 7168), (1000, 128), (130, 384), (9000, 256), (38400, 256)]:
        units = -(-n // 128) * (k // 128)
        for m, rows in ((1, 16), (16, 16), (17, 32), (32, 32), (33, 64), (64, 64)):
            b = ws(m, n, k)
            assert b % (2 * rows * 512) == 0
            g = b // (2 * rows * 512)
            assert -(-units // 8) <= g <= units
            assert g == ws(1, n, k) // (2 * 16 * 512)
    # the decode shapes: 1792 units in 256 shares of 7
    assert ws(64, 7168, 4096) == 2 * 256 * 64 * 512
    assert ws(64, 4096, 7168) == 2 * 256 * 64 * 512


def noalloc(lib, **kw):
    a = dict(A=P, lda=7168, sa=S, fmt=0, sald=64, B=Q, ldb=7168, sb=S, sbld=56, D=P, ldd=7168, m=64, n=7168,
             k=7168, st=None)
    a.update(kw)
    return lib.gemm_fp8_nt_bf16_splitk_noalloc(a["A"], a["lda"], a["sa"], a["fmt"], a["sald"], a["B"], a["ldb"],
                                               a["sb"], a["sbld"], a["D"], a["ldd"], a["m"], a["n"], a["k"], a["st"])


@pytest.mark.parametrize("kw", [dict(m=512, sald=511), dict(k=200), dict(lda=200), dict(sbld=1), dict(ldd=7164),
                                dict(fmt=5), dict(A=None), dict(D=ctypes.c_void_p(0x10004)), dict(m=-1)])
def test_splitk_noalloc_rejects(lib, kw):
    assert noalloc(lib, **kw) == -1


def test_splitk_noalloc_scratch_limit(lib):
    # 64 x 7168 x 16384 needs 58.7 MB of partial sums, beyond the 32 MiB static scratch: refused on
    # the host (FGFP8_ESCRATCH) before any device call; zero sizes are accepted
    assert lib.gemm_fp8_nt_bf16_splitk_workspace(64, 7168, 16384) > 32 << 20
    assert noalloc(lib, k=16384, lda=16384, ldb=16384, sbld=128) == -4
    assert lib.gemm_fp8_nt_bf16_splitk_workspace(64, 7168, 7168) <= 32 << 20
    assert noalloc(lib, m=0) == 0 and noalloc(lib, n=0) == 0


def test_splitk_rejects_grids_beyond_32_bits(lib):
    # n = 2^36 columns: 2^29 tiles of 128, whose fix-up grid (up to 4 workgroups a tile) would not fit 32 bits
    n = 1 << 36
    assert lib.gemm_fp8_nt_bf16_splitk_workspace(1, n, 128) == -1
    assert splitk(lib, m=1, sald=4, n=n, k=128, lda=128, ldb=128, sbld=1, ldd=n) == -1
    assert noalloc(lib, m=1, sald=4, n=n, k=128, lda=128, ldb=128, sbld=1, ldd=n) == -1


def test_size_limits_are_rejected_on_the_host(lib):
    # beyond the header's size limits every call returns FGFP8_EINVAL before any device
    # call (tile counts stay in 32-bit ints; no launch exceeds 2^32 work-items)
    tiles, max_n = 1 << 22, 1 << 24
    m = 2 ** 21 + 128                       # 16385 row tiles x 256 column tiles > 2^22
    assert gemm(lib, m=m, sald=m, n=1 << 15, ldd=1 << 15) == -1
    assert gemm(lib, m=tiles * 128 + 1, sald=tiles * 128 + 1, n=8, ldd=8) == -1
    assert gemm(lib, m=1, n=max_n + 8, ldd=max_n + 8) == -1
    assert wgrad(lib, m=m, sald=m, n=1 << 15, sbld=1 << 15, ldd=1 << 15) == -1
    assert lib.gemm_fp8_nt_bf16_splitk_workspace(1, max_n + 128, 128) == -1
    assert lib.gemm_fp8_nt_bf16_splitk_workspace(m, 1 << 15, 1024) == -1
    # dual cast: 65536 x 257 tiles of 128 x 128 > 2^24
    r, c = 1 << 23, 32769
    assert dual(lib, rows=r, cols=c, xld=32776, qld=32776, qTld=r, sfr=1, sfg=r, sfTr=1, sfTg=c) == -1
    # per-token cast of a transposed view: 65536 column tiles of 128 along the grid's y
    c = 1 << 23
    assert tok(lib, rows=4, cols=c, srow=1, scol=64, qld=c, sfr=1, sfg=4) == -1
