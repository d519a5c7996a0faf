"""Pins of the oracle's seeded AQN noise: the Philox4x64-10 block against numpy's independent Philox bit generator,
the counter and word layout of a draw, the Box-Muller output's distribution, and the draw scope."""
import math

import numpy as np
import pytest
from scipy import stats

M64 = (1 << 64) - 1


def numpy_block(counter, key):
    """numpy's Philox4x64-10 block at this counter: numpy adds one to the 256-bit counter before each block, so it
    is started one below."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    start = np.array([(c >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=start)
    return g.random_raw(4)


def test_philox_block_matches_numpy(orc):
    rng = np.random.default_rng(5)
    cases = [([1, 0, 0, 0], [1, 2]), ([0, 0, 0, 0], [0, 0]), ([M64, M64, M64, M64], [M64, M64]),
             ([0, 7, 0, 0], [123456789, 0])]
    for _ in range(40):
        cases.append(([int(v) for v in rng.integers(0, 1 << 63, 4, dtype=np.uint64)],
                      [int(v) for v in rng.integers(0, 1 << 63, 2, dtype=np.uint64)]))
    for ctr, key in cases:
        assert np.array_equal(orc.philox4x64_10(ctr, key), numpy_block(ctr, key)), (ctr, key)


def u_of(w):
    return ((int(w) >> 9) + 0.5) / 2.0 ** 23


def test_noise_layout_from_numpy_blocks(orc):
    """Column 8c + 2p (+1) of draw r comes from words 2p, 2p+1 of the block at counter (c, r, 0, 0), key (seed,
    stream): checked against numpy's blocks on sampled elements (d not a multiple of 8: the ragged last block)."""
    seed, stream, row_offset, m, d = 0x1234ABCD5678, 9, 40, 6, 100
    eps = orc.aqn_noise(seed, stream, row_offset, 1, m, d)
    for i in range(m):
        for c in range((d + 7) // 8):
            blk = numpy_block([c, row_offset + i, 0, 0], [seed, stream])
            for p in range(4):
                wa, wb = int(blk[p]) & 0xFFFFFFFF, int(blk[p]) >> 32
                rho = math.sqrt(-2.0 * math.log(u_of(wa)))
                th = 2.0 * math.pi * u_of(wb)
                for j, v in ((8 * c + 2 * p, rho * math.cos(th)), (8 * c + 2 * p + 1, rho * math.sin(th))):
                    if j < d:
                        assert eps[i, j] == np.float32(v), (i, j)


def test_noise_is_standard_normal(orc):
    """2^20 draws: Kolmogorov-Smirnov against N(0, 1); pairs' squared radius against chi-square(2) (exponential,
    mean 2); pairs uncorrelated. A wrong angle (pi instead of 2 pi), a wrong log base or a dropped factor fails."""
    eps = orc.aqn_noise(2024, 1, 0, 1, 256, 4096).astype(np.float64)
    flat = eps.ravel()
    assert stats.kstest(flat, "norm").pvalue > 1e-3
    assert abs(flat.mean()) < 5 * (1 / math.sqrt(flat.size))
    assert abs(flat.var() - 1.0) < 5 * math.sqrt(2.0 / flat.size)
    r2 = flat[0::2] ** 2 + flat[1::2] ** 2
    assert stats.kstest(r2, "expon", args=(0, 2.0)).pvalue > 1e-3
    assert abs(np.corrcoef(flat[0::2], flat[1::2])[0, 1]) < 5 / math.sqrt(flat.size / 2)
    # the angle of each pair is uniform on the circle
    ang = np.arctan2(flat[1::2], flat[0::2])
    assert stats.kstest(ang, "uniform", args=(-math.pi, 2 * math.pi)).pvalue > 1e-3


def test_noise_scope_and_keys(orc):
    m, d = 8, 64
    shared = orc.aqn_noise(11, 0, 5, 0, m, d)
    assert all(np.array_equal(shared[i], shared[0]) for i in range(m))
    assert np.array_equal(shared[0], orc.aqn_noise(11, 0, 5, 1, 1, d)[0])   # draw row_offset for every row
    per4 = orc.aqn_noise(11, 0, 5, 4, m, d)
    assert np.array_equal(per4[0], per4[3]) and np.array_equal(per4[4], per4[7])
    assert not np.array_equal(per4[0], per4[4])
    assert np.array_equal(per4[4], orc.aqn_noise(11, 0, 6, 1, 1, d)[0])       # rows 4..7 take draw 5 + 1
    per_row = orc.aqn_noise(11, 0, 5, 1, m, d)
    assert len({per_row[i].tobytes() for i in range(m)}) == m
    assert not np.array_equal(per_row, orc.aqn_noise(12, 0, 5, 1, m, d))
    assert not np.array_equal(per_row, orc.aqn_noise(11, 1, 5, 1, m, d))
    assert np.array_equal(per_row, orc.aqn_noise(11, 0, 5, 1, m, d))         # reproducible
    assert np.all(np.isfinite(per_row))


@pytest.mark.parametrize("w", [0, 1, 511, 512, 0xFFFFFFFF, 0x80000000])
def test_word_uniform_bounds(orc, w):
    """The uniform never reaches 0 or 1, so the logarithm is finite: the extreme words give the largest radius
    sqrt(-2 ln 2^-24) ~ 5.77 and a tiny one."""
    u = u_of(w)
    assert 0.0 < u < 1.0
    assert np.float32(u) == u  # exact in f32 as well
