"""Pins of the oracle's MXFP4 variant (the OCP Microscaling FP4 format the papers calibrate beside NVFP4, "QeRL 阅读笔记"
§3.1; the pages give no more detail, so the reading is OCP MX v1.0: one E8M0 scale X = 2^(E - 127) per 32 weights
along k, E = floor(log2(block amax)) - 2, elements the nearest E2M1 value to w / X, ties to even, saturating at 6).

Pinned against: the exponent rule at the edges where floor(log2) changes (amax = 2^e, 6 * 2^e, just below and at
8 * 2^e); a brute-force nearest-grid search written here from the E2M1 table of the pages (every code and scale of
random blocks spanning many binades); the exact midpoints going to the even code; zero, negative-zero and
non-finite blocks; and the MXFP4 linear against the independent dense-bf16 linear of the same dequantized weights.
"""
import numpy as np
import pytest


def f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16(v):
    """fp64 values that are exactly representable in bf16 -> bit patterns (asserted exact)."""
    f = np.asarray(v, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(f64(bits), np.asarray(v, dtype=np.float64)), "value not exact in bf16"
    return bits


def block_row(vals, k=32):
    row = np.zeros(k, dtype=np.float64)
    row[:len(vals)] = vals
    return bf16(row)[None, :]


def brute(w_bits, grid):
    """Independent MX quantization: E from numpy's log2, codes by exhaustive search over the 8 magnitudes."""
    n, k = w_bits.shape
    w = f64(w_bits)
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 32), dtype=np.uint8)
    mags = np.array(grid)
    for i in range(n):
        for b in range(k // 32):
            blk = w[i, 32 * b:32 * b + 32]
            fin = np.isfinite(blk)
            amax = np.max(np.abs(blk[fin])) if fin.any() else 0.0
            E = 0 if amax == 0 else int(np.clip(np.floor(np.log2(amax)) - 2 + 127, 0, 254))
            scales[i, b] = E
            X = 2.0 ** (E - 127)
            for j in range(32):
                v = blk[j]
                if not np.isfinite(v):
                    continue
                d = np.abs(np.abs(v) - mags * X)
                best = np.flatnonzero(d == d.min())
                c = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                codes[i, 32 * b + j] = c | (8 if np.signbit(v) else 0)
    return codes, scales


def unpack(codes):
    out = np.zeros((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


@pytest.mark.parametrize("e", [-20, -8, -1, 0, 3, 10])
def test_exponent_rule_at_its_edges(orc, e):
    s = 2.0 ** e
    cases = [(s, e - 2, 6),            # amax 2^e: X = 2^(e-2), amax / X = 4 -> code 6
             (6 * s, e, 7),            # amax 6 * 2^e: X = 2^e, exactly 6 -> code 7
             (7.5 * s, e, 7),          # below 8 * 2^e: X = 2^e, 7.5 saturates to 6
             (8 * s, e + 1, 6)]        # 8 * 2^e: X = 2^(e+1), amax / X = 4
    for amax, ex, code in cases:
        codes, sc, flags = orc.mxfp4_quantize(block_row([0.5 * s, -amax]))
        assert flags == 0
        assert sc[0, 0] == ex + 127, (amax, sc[0, 0])
        assert unpack(codes)[0, 1] == (code | 8)


def test_matches_brute_force(orc, syn, e2m1_grid):
    rng = np.random.default_rng(3)
    n, k = 6, 256
    w = rng.normal(0.0, 1.0, (n, k)) * 2.0 ** rng.integers(-30, 20, (n, k // 32)).repeat(32, axis=1)
    bits = (w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits[0, 5] = 0x8000   # -0
    bits[2, 64:96] = 0    # an all-zero block (block 2 of row 2)
    codes, sc, flags = orc.mxfp4_quantize(bits)
    bc, bs = brute(bits, e2m1_grid)
    assert flags == 0
    assert np.array_equal(sc, bs)
    assert np.array_equal(unpack(codes), bc)
    assert sc[2, 2] == 0 and np.all(unpack(codes)[2, 64:96] == 0)
    assert unpack(codes)[0, 5] == 8


def test_midpoints_go_to_the_even_code(orc):
    # X = 1 (amax 4 -> E = 127): midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 between the grid values
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0, 2, 2, 4, 4, 6, 6]  # the even neighbour of each midpoint
    codes, sc, _ = orc.mxfp4_quantize(block_row([4.0] + mids + [-m for m in mids]))
    assert sc[0, 0] == 127
    q = unpack(codes)[0]
    assert list(q[1:8]) == expect
    assert list(q[8:15]) == [c | 8 for c in expect]


def test_non_finite_weights_are_flagged_and_left_out(orc):
    row = block_row([1.0, 3.0])
    row[0, 4] = 0x7F80  # +inf
    row[0, 7] = 0x7FC0  # NaN
    codes, sc, flags = orc.mxfp4_quantize(row)
    assert flags & 1
    assert sc[0, 0] == 127 - 1  # amax 3 (the infinity left out): floor(log2 3) - 2 = -1
    q = unpack(codes)[0]
    assert q[4] == 0 and q[7] == 0 and q[1] == 7  # 3 / 0.5 = 6


def test_dequantize_and_linear_against_dense_bf16(orc, syn):
    """The MX linear equals the independent dense-bf16 linear of the dequantized weights (exact in bf16: E2M1 values
    carry at most two significant bits) plus the LoRA term in fp64 numpy."""
    s = lambda t: syn.seed_for(31, 0, t)
    m, n, k, r = 3, 40, 96, 8
    w = syn.normal_bf16(s("w_q"), (n, k), std=0.02)
    h = syn.normal_bf16(s("x"), (m, k))
    A = syn.normal_bf16(s("a_q"), (r, k), std=0.05)
    B = syn.normal_bf16(s("b_q"), (n, r), std=0.05)
    codes, sc, _ = orc.mxfp4_quantize(w)
    we, wf = orc.mxfp4_dequantize(codes, sc)
    assert np.array_equal(we, wf.astype(np.float64))  # exact in f32 as well
    wb = bf16(we)
    y = orc.mxfp4_lora_linear(h, codes, sc, A, B, 2.0)
    ref = orc.dense_linear(h, wb) + 2.0 * (f64(h) @ f64(A).T) @ f64(B).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)
    # each weight's error is at most half the grid spacing at its magnitude times the block scale (spacing 0.5 up to
    # 2, 1 up to 4, 2 up to 6), and at most 2 X where the block's largest values (below 8 X) saturate to 6 X
    X = 2.0 ** (sc.astype(np.int64) - 127).repeat(32, axis=1)
    a, err = np.abs(f64(w)), np.abs(f64(w) - we)
    half = np.where(a <= 2 * X, 0.25, np.where(a <= 4 * X, 0.5, np.where(a <= 6 * X, 1.0, 2.0))) * X
    assert np.all(err <= half)
