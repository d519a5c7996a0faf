"""Pins of the oracle's number formats (E2M1, E4M3, bf16) against what the pages and the format definitions fix."""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden


def test_e2m1_grid_matches_pages(orc, e2m1_grid):
    # the printed non-negative grid, code order 0..7 (QeRL technical review §3.1)
    assert [orc.e2m1_value(c) for c in range(8)] == e2m1_grid
    # codes 8..15 are the negatives (sign bit 3); code 8 is -0
    for c in range(8):
        assert orc.e2m1_value(c | 8) == -e2m1_grid[c]
    assert math.copysign(1.0, orc.e2m1_value(8)) == -1.0
    # "not a uniformly spaced grid": the gaps are 0.5, 0.5, 0.5, 0.5, 1, 1, 2
    assert np.diff(e2m1_grid).tolist() == [0.5, 0.5, 0.5, 0.5, 1, 1, 2]


# Known E4M3 (OCP "FN") encodings: exponent bias 7, 3 mantissa bits, max 448, S.1111.111 = NaN.
E4M3_KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x39: 1.125,
              0x3C: 1.5, 0x40: 2.0, 0x48: 4.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0}


def test_e4m3_known_values(orc):
    for b, v in E4M3_KNOWN.items():
        assert orc.e4m3_value(b) == v, hex(b)
        assert orc.e4m3_value(b | 0x80) == -v
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))


def test_e4m3_exhaustive_structure(orc):
    vals = [orc.e4m3_value(b) for b in range(0x7F)]  # 127 non-negative finite codes
    assert len(set(vals)) == 127
    assert all(a < b for a, b in zip(vals, vals[1:]))  # monotone in the code
    assert max(vals) == 448.0 and min(v for v in vals if v > 0) == 2.0 ** -9
    # within every normal binade there are 8 equally spaced values with spacing 2^(e-3)
    for e in range(-6, 9):
        binade = [v for v in vals if 2.0 ** e <= v < 2.0 ** (e + 1)]
        assert binade == [2.0 ** e * (1 + m / 8) for m in range(8)] or (e == 8 and len(binade) == 7)
    # every finite code round-trips through the encoder (sign dropped: scales are non-negative)
    for b in range(0x7F):
        assert orc.e4m3_encode(orc.e4m3_value(b)) == b


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38),        # midpoint 1 | 1.125 -> even mantissa (1.0)
    (1.1875, 0x3A),        # midpoint 1.125 | 1.25 -> 1.25
    (1.0625 + 1e-9, 0x39),  # just above the midpoint
    (464.0, 0x7E),         # beyond 448: saturate (no infinities)
    (1e30, 0x7E),
    (2.0 ** -10, 0x00),    # midpoint 0 | 2^-9 -> 0
    (1.5 * 2.0 ** -9, 0x02),  # midpoint 1 | 2 (x 2^-9) -> 2
    (1.25 * 2.0 ** -9, 0x01),
    (0.0, 0x00),
])
def test_e4m3_encode_rounding(orc, value, code):
    assert orc.e4m3_encode(value) == code


def test_bf16_rounding_matches_torch(orc, syn):
    # f32 values -> bf16 is a single RNE rounding; torch's float32 -> bfloat16 conversion is the library routine
    x = syn.normal_f32(7, 20000, std=3.0)
    x[:5] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 3.0e38, 1e-40]
    ours = orc.bf16_round_array(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert orc.bf16_value(ours[0]) == 1.0 and orc.bf16_value(ours[1]) == 1.0 + 2.0 ** -6


def test_bf16_value_exhaustive(orc):
    # every bf16 pattern widens to the float32 with the same upper half
    for b in range(0, 65536, 97):
        v = orc.bf16_value(b)
        f = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        assert (math.isnan(v) and math.isnan(f)) or v == float(f)


def test_storage_formula_matches_pages(orc):
    n, k, nv, bf, ratio = read_golden("nvfp4_storage.txt")[0].split()
    n, k = int(n), int(k)
    assert orc.nvfp4_bytes(n, k) == int(nv) == 9 * n * k // 16
    assert 2 * n * k == int(bf)
    assert round(int(bf) / int(nv), 2) == float(ratio)
    assert int(bf) / int(nv) == pytest.approx(32 / 9)
