"""Pins of the oracle's NVFP4 quantizer: brute-force argmin in binary128, scale-rule invariants, fixed points,
exhaustive dequantization against exact rational products."""
import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def brute():
    src = os.path.join(HERE, "brute", "argmin_q128.c")
    so = os.path.join(HERE, "brute", "libargmin_q128.so")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        tmp = so + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", src, "-o", tmp])
        os.replace(tmp, so)
    lib = ctypes.CDLL(so)
    lib.brute_codes.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]
    lib.brute_codes.restype = None
    return lib


def unpack(codes):
    """canonical packed [n, k/2] -> one code per element [n, k] (low nibble = even element)."""
    n, k2 = codes.shape
    out = np.empty((n, 2 * k2), dtype=np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def brute_codes(brute, w, S_blocks, grid):
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n, k = w.shape
    S = np.ascontiguousarray(S_blocks, dtype=np.float64)
    g = np.ascontiguousarray(grid, dtype=np.float64)
    out = np.empty((n, k), dtype=np.uint8)
    brute.brute_codes(w.ctypes.data, n, k, S.ctypes.data, g.ctypes.data, out.ctypes.data)
    return out


def block_S(orc, s_b, s_g):
    e4 = np.array([orc.e4m3_value(b) for b in range(256)])
    return float(s_g) * e4[s_b]  # exact: 24-bit x 4-bit significands


def test_exhaustive_bf16_against_brute_force(orc, brute, e2m1_grid):
    """All 65,536 bf16 patterns x all 126 positive finite E4M3 scales (s_g = 1), fixed-scale mode.

    binary128 distances are exact whenever |w| < 2^100 (S*g has its lowest bit at or above 2^-10); far below the
    first candidate the rounding cannot reorder distances. For |w| >= 2^100 every candidate lies below |w|, so the
    largest grid value (code 7, with the sign of w) is nearest: that closed form replaces the brute force there."""
    w = np.tile(np.arange(65536, dtype=np.uint16), (126, 1))
    s_b = np.repeat(np.arange(1, 127, dtype=np.uint8)[:, None], 65536 // 16, axis=1)
    codes, _, _, flags = orc.nvfp4_quantize(w, scale_mode=1, s_b=s_b, s_g=1.0)
    assert flags == 1  # the NaN/inf patterns were seen
    ref = brute_codes(brute, w, block_S(orc, s_b, 1.0), e2m1_grid)
    got = unpack(codes)
    expo = (w >> 7) & 0xFF
    finite = expo != 0xFF
    huge = finite & (expo >= 127 + 100)
    exact = finite & ~huge
    assert np.array_equal(got[exact], ref[exact])
    assert np.all(got[huge] == (7 | ((w[huge] >> 15) << 3)))
    assert np.all(got[~finite] == 0)  # non-finite weights encode as code 0


@pytest.mark.parametrize("sb", [0x01, 0x07, 0x08, 0x38, 0x6F, 0x7E])
def test_exhaustive_bf16_exact_integer_brute_force(orc, e2m1_grid, sb):
    """Exact integer arithmetic (Python ints, every value scaled by 2^200) over all finite bf16 patterns."""
    w = np.arange(65536, dtype=np.uint16)
    finite = ((w >> 7) & 0xFF) != 0xFF
    wv = w[finite]
    S = Fraction(orc.e4m3_value(sb))
    codes, _, _, _ = orc.nvfp4_quantize(wv[None, :], scale_mode=1, s_b=np.full((1, wv.size // 16), sb, np.uint8),
                                        s_g=1.0)
    got = unpack(codes)[0]
    SCALE = 2 ** 200
    cand = [int(S * Fraction(g) * SCALE) for g in e2m1_grid]
    f32 = (wv.astype(np.uint32) << 16).view(np.float32)
    for i in range(wv.size):
        W = int(Fraction(float(f32[i])) * SCALE)
        a = abs(W)
        d = [abs(a - c) for c in cand]
        dmin = min(d)
        best = [j for j in range(8) if d[j] == dmin]
        mag = best[0] if len(best) == 1 else [j for j in best if j % 2 == 0][0]
        expect = mag | (8 if (wv[i] >> 15) else 0)
        assert got[i] == expect, (hex(int(wv[i])), sb)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_blocks_with_tensor_scale_against_brute_force(orc, brute, syn, e2m1_grid, seed):
    rng = np.random.default_rng(seed)
    n, k = 64, 256
    w = syn.normal_bf16(100 + seed, (n, k), std=0.05)
    s_g = float(np.float32(rng.uniform(1e-5, 1e-3)))
    s_b = rng.integers(0, 127, size=(n, k // 16)).astype(np.uint8)
    codes, _, _, _ = orc.nvfp4_quantize(w, scale_mode=1, s_b=s_b, s_g=s_g)
    assert np.array_equal(unpack(codes), brute_codes(brute, w, block_S(orc, s_b, s_g), e2m1_grid))


def test_exact_midpoints_tie_to_even_code(orc, brute, e2m1_grid):
    """Weights placed exactly on every midpoint between neighbouring grid values, for every scale."""
    mids = [(a + b) / 2 for a, b in zip(e2m1_grid, e2m1_grid[1:])]  # 0.25, 0.75, ..., 5
    expect = [0, 2, 2, 4, 4, 6, 6]  # even-code neighbour of each midpoint
    for sb in range(1, 127):
        S = orc.e4m3_value(sb)
        for mid, e in zip(mids, expect):
            v = np.float32(mid * S)
            b = int(np.array([v], dtype=np.float32).view(np.uint32)[0])
            if b & 0xFFFF:
                continue  # midpoint not representable in bf16 at this scale
            wb = b >> 16
            assert orc.nvfp4_code(wb, S) == e
            assert orc.nvfp4_code(wb | 0x8000, S) == e | 8


def test_scale_rule_invariants(orc, syn):
    w = syn.normal_bf16(11, (96, 512), std=0.02)
    codes, s_b, s_g, flags = orc.nvfp4_quantize(w)
    assert flags == 0
    wf = syn.bf16_to_f32(w).astype(np.float64)
    amax = np.abs(wf).max()
    assert s_g == pytest.approx(amax / 2688, rel=2 ** -23)
    blocks = np.abs(wf).reshape(96, 32, 16)
    bmax = blocks.max(axis=2)
    # the block holding the tensor's largest magnitude gets the largest E4M3 scale, 448
    assert s_b.reshape(-1)[np.argmax(bmax)] == 0x7E
    # every block scale is within E4M3 rounding (2^-4 relative for normals) of amax_b / (6 s_g)
    e4 = np.array([orc.e4m3_value(b) for b in range(256)])
    target = bmax / (6 * s_g)
    normal = (s_b & 0x78) != 0
    assert np.all(np.abs(e4[s_b][normal] / target[normal] - 1) <= 2 ** -4 + 1e-6)
    # for normal scales, the block maximum maps onto the top code 6 (amax_b / S_b in [5.65, 6.4])
    q = unpack(codes).reshape(96, 32, 16)
    arg = blocks.argmax(axis=2)
    top = np.take_along_axis(q, arg[..., None], axis=2)[..., 0] & 7
    assert np.all(top[normal] == 7)


def test_on_grid_weights_are_fixed_points(orc, syn):
    rng = np.random.default_rng(5)
    n, k = 32, 128
    q = rng.integers(0, 16, size=(n, k))
    s_b = rng.integers(1, 127, size=(n, k // 16)).astype(np.uint8)
    e4 = np.array([orc.e4m3_value(b) for b in range(256)])
    e2 = np.array([orc.e2m1_value(c) for c in range(16)])
    vals = e4[s_b].repeat(16, axis=1) * e2[q]  # s_g = 1: s_b * q has <= 6 significant bits -> exact in bf16
    w = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(syn.bf16_to_f32(w).astype(np.float64), vals)
    codes, _, _, _ = orc.nvfp4_quantize(w, scale_mode=1, s_b=s_b, s_g=1.0)
    assert np.array_equal(unpack(codes), q)


def test_dequant_exhaustive_codes_scales(orc):
    """16 codes x 127 scales (incl. 0) x several tensor scales vs exact rational products."""
    s_gs = [1.0, float(np.float32(3.0517578125e-05)), float(np.float32(0.1234567)), float(np.float32(7.77e-3))]
    k = 16 * 16
    q = np.tile(np.arange(16, dtype=np.uint8), 16)  # each block of 16 holds all 16 codes
    codes = np.zeros((127, k // 2), dtype=np.uint8)
    codes[:, :] = (q[0::2] | (q[1::2] << 4))[None, :]
    s_b = np.repeat(np.arange(127, dtype=np.uint8)[:, None], k // 16, axis=1)
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]
    for s_g in s_gs:
        we, wf = orc.nvfp4_dequantize(codes, s_b, s_g)
        for sb in range(127):
            S = Fraction(s_g) * Fraction(orc.e4m3_value(sb))
            for j in range(16):
                c = int(q[j])
                exact = S * grid[c & 7] * (-1 if c & 8 else 1)
                assert Fraction(we[sb, j]) == exact
                assert wf[sb, j] == np.float32(float(exact))  # exact fits in a double: one rounding to f32


def test_zero_and_tiny_blocks(orc):
    w = np.zeros((2, 32), dtype=np.uint16)
    w[1, 16] = 0x3F80  # 1.0 in the second block of row 1
    w[0, 3] = 0x8000   # -0.0
    codes, s_b, s_g, _ = orc.nvfp4_quantize(w)
    assert s_g == np.float32(1.0) / np.float32(2688.0)
    assert s_b[0, 0] == 0 and s_b[1, 1] == 0x7E
    q = unpack(codes)
    assert q[1, 16] == 7 and q[0, 3] == 8 and q[0, 0] == 0


def test_all_zero_tensor(orc):
    codes, s_b, s_g, flags = orc.nvfp4_quantize(np.zeros((4, 64), dtype=np.uint16))
    assert s_g == 1.0 and np.all(s_b == 0) and np.all(codes == 0) and flags == 0


@pytest.mark.parametrize("seed", [1, 2])
def test_quantize_rows_equals_rows_of_whole_quantization(orc, syn, seed):
    """The row-subset quantizer (used for sampled full-size parity) gives exactly the selected rows of the whole
    tensor's amax-rule quantization, with the same tensor scale; heavy-tailed blocks put the largest magnitude in
    rows that are not selected, so s_g must come from the whole tensor."""
    n, k = 96, 256
    w = syn.student_t4_bf16(syn.seed_for(9, seed, "w_q"), (n, k), 0.02, 16, syn.seed_for(9, seed, "block_exp"), -14)
    codes, sb, sg, flags = orc.nvfp4_quantize(w)
    rows = np.array([0, 5, 17, 17, 40, n - 1], dtype=np.int64)
    c2, sb2, sg2, f2 = orc.nvfp4_quantize_rows(w, rows)
    assert sg2 == sg and f2 == flags
    assert np.array_equal(c2, codes[rows]) and np.array_equal(sb2, sb[rows])
    # all rows in order: the whole quantization
    c3, sb3, sg3, _ = orc.nvfp4_quantize_rows(w, np.arange(n))
    assert sg3 == sg and np.array_equal(c3, codes) and np.array_equal(sb3, sb)
    # the tensor scale is not the subset's own: quantizing the subset as a tensor gives a different s_g
    amax_rows = np.abs(syn.bf16_to_f32(w[rows])).max()
    amax_all = np.abs(syn.bf16_to_f32(w)).max()
    if amax_rows < amax_all:
        assert orc.nvfp4_quantize(w[rows])[2] != sg
