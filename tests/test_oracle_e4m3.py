"""Pins for the oracle's E4M3 rounding and decoding (CPU only).

The cast of "DeepGEMM Essentials: High-Performance FP8 Matrix
Multiplication", Part 3, converts the scaled fp32 group to float8_e4m3fn; the
oracle writes that rounding from the OCP FP8 definition.  These tests pin it
to hand-worked codes, to the structure of the code grid (every code maps to
itself, every midpoint to its even neighbour) and to PyTorch's own CPU
converter, an implementation independent of the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from golden_io import e4m3_hand_values

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_decode_closed_forms():
    v = oracle.e4m3_value(np.array([0x00, 0x80, 0x01, 0x08, 0x38, 0x30, 0x7E, 0xFE, 0x07, 0x0F], np.uint8))
    assert v[0] == 0.0 and math.copysign(1, v[1]) == -1
    assert v[2] == 2.0 ** -9            # smallest subnormal
    assert v[3] == 2.0 ** -6            # smallest normal
    assert v[4] == 1.0 and v[5] == 0.5
    assert v[6] == 448.0 and v[7] == -448.0
    assert v[8] == 7 * 2.0 ** -9        # largest subnormal
    assert v[9] == 1.875 * 2.0 ** -6
    assert np.isnan(oracle.e4m3_value(np.array([0x7F, 0xFF], np.uint8))).all()


def test_decode_matches_torch():
    codes = np.array(FINITE, dtype=np.uint8)
    ours = oracle.e4m3_value(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, theirs)


def test_hand_values():
    cases = e4m3_hand_values()
    vals = np.array([v for v, _ in cases], dtype=np.float32)
    got = oracle.e4m3_round(vals)
    for (v, code), g in zip(cases, got):
        assert g == code, f"{v!r}: got {g:#04x}, want {code:#04x}"


def test_every_code_maps_to_itself():
    codes = np.array(FINITE, dtype=np.uint8)
    vals = oracle.e4m3_value(codes).astype(np.float32)
    got = oracle.e4m3_round(vals)
    # +0 and -0 keep their sign; every other code round-trips
    assert np.array_equal(got, codes)


def _neighbours():
    """Consecutive positive finite codes (c, c+1) and their midpoint."""
    out = []
    for c in range(0, 0x7E):
        lo = float(oracle.e4m3_value(np.array([c], np.uint8))[0])
        hi = float(oracle.e4m3_value(np.array([c + 1], np.uint8))[0])
        out.append((c, c + 1, (lo + hi) / 2))
    return out


def test_midpoints_round_to_even_and_neighbours_round_away_from_tie():
    for lo, hi, mid in _neighbours():
        even = lo if lo % 2 == 0 else hi
        m32 = np.float32(mid)
        assert float(m32) == mid               # every midpoint is exact in fp32
        below = np.nextafter(m32, np.float32(0))
        above = np.nextafter(m32, np.float32(1e9))
        got = oracle.e4m3_round(np.array([m32, below, above, -m32, -below, -above], np.float32))
        assert got[0] == even, (lo, hi, mid)
        assert got[1] == lo and got[2] == hi
        assert got[3] == even | 0x80 and got[4] == lo | 0x80 and got[5] == hi | 0x80


def test_overflow_is_nan_not_saturated():
    v = np.array([464.0, np.nextafter(np.float32(464), np.float32(1e9)), 1e6, -1e6, np.inf, np.nan],
                 dtype=np.float32)
    got = oracle.e4m3_round(v)
    assert got[0] == 0x7E
    assert list(got[1:4]) == [0x7F, 0x7F, 0xFF]
    assert got[4] == 0x7F and (got[5] & 0x7F) == 0x7F


@pytest.mark.parametrize("stride", [7919, 104729])
def test_sweep_matches_torch_converter(stride):
    """Strided sweep over fp32 bit patterns with |v| <= 464 (both signs)."""
    limit = np.float32(464.0).view(np.uint32)
    bits = np.arange(0, int(limit) + 1, stride, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    ours = oracle.e4m3_round(v)
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)
