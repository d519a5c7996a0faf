"""GPU parity of the seeded AQN noise: the standalone generator against the oracle's draw, and the noise drawn inside
the norm and the linear prologue against the same values read from a buffer."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, LINEAR_TOL, dev_bf16, dev_f32, host_bf16, rel_err

pytestmark = pytest.mark.gpu

# The device draws in f32: the uniforms are exact, the logarithm, square root and sin/cos are the f32 library
# functions (about 1-2 ulp each), against the oracle's fp64 values rounded to f32. rho <= sqrt(-2 ln 2^-24) = 5.8,
# so |error| <= rho * (2 ulp of 1 in sin/cos) + |eps| * (4 ulp for log, sqrt and the product): bounded by
# NOISE_ABS + NOISE_REL * |eps|.
NOISE_ABS = 1.5e-6
NOISE_REL = 5e-7


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


@pytest.mark.parametrize("seed,subseed,row_offset,draw_rows,m,d", [
    (1, 0, 0, 1, 16, 3584),            # decode: one draw per response
    (0xDEADBEEF12345678, 7, 1000, 1, 3, 100),   # ragged d (last block partly used), large seed and offset
    (42, 1, 5, 0, 9, 4096),            # one draw for every row
    (42, 1, 5, 4, 33, 5120),           # 4 rows per draw (tokens of one response)
    (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 2, 1, 2, 24),  # counter and key words at their maximum
])
def test_noise_matches_oracle(qn, seed, subseed, row_offset, draw_rows, m, d):
    draw = qn.NoiseDraw(seed, subseed, row_offset, draw_rows)
    eps = qn.aqn_noise(draw, m, d, DEV)
    torch.cuda.synchronize()
    got = eps.cpu().numpy().astype(np.float64)
    ref = oracle.aqn_noise(seed, subseed, row_offset, draw_rows, m, d).astype(np.float64)
    err = np.abs(got - ref)
    bound = NOISE_ABS + NOISE_REL * np.abs(ref)
    assert np.all(err <= bound), (err.max(), np.unravel_index(np.argmax(err - bound), err.shape))
    assert np.mean(err == 0) > 0.5   # most values are the correctly rounded ones


def test_noise_strided_output_and_errors(qn):
    draw = qn.NoiseDraw(3, 0, 0, 1)
    buf = torch.full((4, 40), float("nan"), dtype=torch.float32, device=DEV)
    qn.aqn_noise(draw, 4, 36, DEV, out=buf[:, :36])
    torch.cuda.synchronize()
    assert torch.isnan(buf[:, 36:]).all()   # nothing written past d
    ref = oracle.aqn_noise(3, 0, 0, 1, 4, 36)
    assert np.abs(buf[:, :36].cpu().numpy() - ref).max() <= NOISE_ABS + NOISE_REL * np.abs(ref).max()
    with pytest.raises(qn.QnError):
        qn.aqn_noise(qn.NoiseDraw(3, 0, 0, -1), 4, 36, DEV)
    g = dev_bf16(synth.normal_bf16(5, (64,)))
    with pytest.raises(ValueError):
        qn.make_aqn(g, dev_f32(np.zeros(64)), 0.01, draw=draw)


@pytest.mark.parametrize("m,d,draw_rows", [(16, 3584, 1), (7, 100, 0), (40, 4096, 4), (3, 40960, 1)])
def test_norm_with_drawn_noise(qn, m, d, draw_rows):
    """Drawn inside the norm == read from the generator's buffer (bit for bit); and within one bf16 ulp of the oracle
    norm on the oracle's draw, differing only where the noise's last bits move a rounding."""
    x = synth.normal_bf16(synth.seed_for(7, m, "x"), (m, d))
    gamma = synth.normal_bf16(synth.seed_for(7, m, "gamma"), (d,))
    sigma = float(np.float32(1e-2))
    draw = qn.NoiseDraw(99, 3, 17, draw_rows)
    xd, gd = dev_bf16(x), dev_bf16(gamma)
    h_draw = qn.aqn_rmsnorm(xd, gd, None, sigma, 1e-6, draw=draw)
    eps = qn.aqn_noise(qn.NoiseDraw(99, 3, 17, draw_rows), m, d, DEV)
    if draw_rows == 0:
        eps = eps[:1].contiguous()
        h_buf = qn.aqn_rmsnorm(xd, gd, eps[0], sigma, 1e-6)
    else:
        h_buf = qn.aqn_rmsnorm(xd, gd, eps, sigma, 1e-6, noise_per_row=True)
    torch.cuda.synchronize()
    assert torch.equal(h_draw.view(torch.int16), h_buf.view(torch.int16))
    ref_eps = oracle.aqn_noise(99, 3, 17, draw_rows, m, d)
    _, ref = oracle.aqn_rmsnorm(x, gamma, ref_eps, sigma, 1e-6, noise_per_row=True)
    got = host_bf16(h_draw)
    diff = np.abs(got.astype(np.int64) - ref.astype(np.int64))
    same_sign = (got >> 15) == (ref >> 15)
    assert np.all((diff <= 1) & (same_sign | (diff == 0))), diff.max()
    assert np.mean(diff != 0) <= 1e-3


@pytest.mark.parametrize("m,k,draw_rows", [(16, 3584, 1), (5, 272, 0), (300, 1024, 4), (17, 512, 1)])
def test_linear_with_drawn_noise(qn, m, k, draw_rows):
    """The linear call drawing its noise in the prologue (and in the row statistics kernel from 256 tokens on) gives
    the bits of the same call reading the generator's buffer, and the oracle's result on the oracle's draw."""
    n, r, lam = 96, 32, 2.0
    x = synth.normal_bf16(synth.seed_for(8, m, "x"), (m, k))
    gamma = synth.normal_bf16(synth.seed_for(8, m, "gamma"), (k,))
    w = synth.normal_bf16(synth.seed_for(8, m, "w_q"), (n, k), std=0.02)
    A = synth.normal_bf16(synth.seed_for(8, m, "a_q"), (r, k), std=0.02)
    B = synth.normal_bf16(synth.seed_for(8, m, "b_q"), (n, r), std=0.02)
    sigma = float(np.float32(1e-2))
    wq = qn.quantize(dev_bf16(w), qn.LAYOUT_TILED)
    xd, gd, Ad, Bd = dev_bf16(x), dev_bf16(gamma), dev_bf16(A), dev_bf16(B)
    draw = qn.NoiseDraw(1234, 5, 6, draw_rows)
    y1 = torch.empty(m, n, dtype=torch.float32, device=DEV)
    qn.lora_linear(xd, [qn.Projection(wq, y1, Ad, Bd, lam)], qn.make_aqn(gd, None, sigma, 1e-6, draw=draw))
    eps = qn.aqn_noise(draw, m, k, DEV)
    y2 = torch.empty(m, n, dtype=torch.float32, device=DEV)
    if draw_rows == 0:
        aqn = qn.make_aqn(gd, eps[0].contiguous(), sigma, 1e-6)
    else:
        aqn = qn.make_aqn(gd, eps, sigma, 1e-6, noise_per_row=True)
    qn.lora_linear(xd, [qn.Projection(wq, y2, Ad, Bd, lam)], aqn)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    _, h = oracle.aqn_rmsnorm(x, gamma, oracle.aqn_noise(1234, 5, 6, draw_rows, m, k), sigma, 1e-6,
                              noise_per_row=True)
    cc, sb, sg, _ = oracle.nvfp4_quantize(w)
    assert rel_err(y1.cpu().numpy(), oracle.lora_linear(h, cc, sb, sg, A, B, lam)) <= LINEAR_TOL
