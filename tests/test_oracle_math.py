"""Pins of the oracle's linear, AQN-RMSNorm, sigma schedule and group advantage."""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden


def bf16_of(vals):
    v = np.asarray(vals, dtype=np.float32)
    b = v.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


def pack(q):
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def test_lora_param_count_matches_pages():
    d_o, d_i, r, P, lora, pct = read_golden("lora_params.txt")[0].split()
    d_o, d_i, r = int(d_o), int(d_i), int(r)
    assert d_o * d_i == int(P)
    assert r * (d_i + d_o) == int(lora)
    A = np.zeros((r, d_i)); B = np.zeros((d_o, r))
    assert A.size + B.size == int(lora)
    assert 100 * int(lora) / int(P) == float(pct)


def test_linear_one_hot_columns(orc, syn):
    """A one-hot activation selects one column of W_hat: catches transposed operands and nibble/index errors."""
    n, k = 48, 64
    w = syn.normal_bf16(21, (n, k), std=0.02)
    codes, s_b, s_g, _ = orc.nvfp4_quantize(w)
    w_exact, _ = orc.nvfp4_dequantize(codes, s_b, s_g)
    for c in (0, 1, 15, 16, 17, 63):
        h = np.zeros((1, k), dtype=np.uint16)
        h[0, c] = bf16_of([1.0])[0]
        y = orc.lora_linear(h, codes, s_b, s_g, None, None, 0.0)
        assert np.array_equal(y[0], w_exact[:, c])


def test_linear_integer_exact_case(orc, e2m1_grid):
    """s_g = 1, s_b = 1, small-integer activations: every product and sum is exact, so the result is the integer
    matrix product over the printed E2M1 grid (twice the grid is an integer), computed here with int64."""
    rng = np.random.default_rng(3)
    m, n, k, r = 3, 40, 96, 4
    q = rng.integers(0, 16, size=(n, k))
    s_b = np.full((n, k // 16), 0x38, dtype=np.uint8)  # 1.0
    hv = rng.integers(-4, 5, size=(m, k))
    Av = rng.integers(-2, 3, size=(r, k))
    Bv = rng.integers(-2, 3, size=(n, r))
    lam = 2.0
    grid2 = np.array([int(2 * g) for g in e2m1_grid], dtype=np.int64)
    w2 = grid2[q & 7] * np.where(q & 8, -1, 1)  # 2 * W_hat, integers
    ref2 = hv @ w2.T + 2 * int(lam) * ((hv @ Av.T) @ Bv.T)  # 2 * y
    y = orc.lora_linear(bf16_of(hv), pack(q), s_b, 1.0, bf16_of(Av), bf16_of(Bv), lam)
    assert np.array_equal(2 * y, ref2.astype(np.float64))


def test_linear_lora_branch_reduces(orc, syn):
    m, n, k, r = 2, 32, 64, 8
    h = syn.normal_bf16(31, (m, k))
    w = syn.normal_bf16(32, (n, k), std=0.02)
    A = syn.normal_bf16(33, (r, k), std=0.02)
    B = syn.normal_bf16(34, (n, r), std=0.02)
    codes, s_b, s_g, _ = orc.nvfp4_quantize(w)
    base = orc.lora_linear(h, codes, s_b, s_g, None, None, 0.0)
    assert np.array_equal(orc.lora_linear(h, codes, s_b, s_g, A, B, 0.0), base)       # lambda = 0
    zeroB = np.zeros_like(B)
    assert np.array_equal(orc.lora_linear(h, codes, s_b, s_g, A, zeroB, 2.0), base)   # B = 0
    # lambda scales the branch linearly: y(2) - y(0) = 2 (y(1) - y(0))
    y1 = orc.lora_linear(h, codes, s_b, s_g, A, B, 1.0)
    y2 = orc.lora_linear(h, codes, s_b, s_g, A, B, 2.0)
    assert np.allclose(y2 - base, 2 * (y1 - base), rtol=1e-12, atol=1e-15)
    # quantized vs the dense bf16 product: NVFP4 error stays at the format's relative level, not a wrong operand
    dense = orc.dense_linear(h, w)
    assert np.abs(base - dense).max() < 0.15 * np.abs(dense).max()


def test_rmsnorm_sigma_zero_is_textbook(orc, syn):
    """sigma = 0 reduces AQN-RMSNorm to plain RMSNorm; compare with torch's rms_norm in float64."""
    m, d = 4, 384
    x = syn.normal_bf16(41, (m, d))
    gamma = syn.normal_bf16(42, (d,), std=1.0)
    noise = syn.normal_f32(43, (d,))
    he, hb = orc.aqn_rmsnorm(x, gamma, noise, 0.0, eps=1e-6)
    xt = torch.from_numpy(syn.bf16_to_f32(x).astype(np.float64))
    gt = torch.from_numpy(syn.bf16_to_f32(gamma).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (d,), weight=gt, eps=float(np.float32(1e-6))).numpy()
    assert np.allclose(he, ref, rtol=1e-13, atol=1e-15)
    assert np.array_equal(hb, orc.bf16_round_array(he))


def test_aqn_is_row_modulation_50_cases(orc, syn):
    """h_z W = h diag(1 + z/w) W on 50 seeded float64 cases (QeRL technical review §5.1 identity; §9.3 reports a
    maximum absolute discrepancy of about 3.6e-15)."""
    cases, printed = read_golden("rmsnorm_identity.txt")[0].split()
    worst = 0.0
    for c in range(int(cases)):
        m, d, n = 3, 64, 24
        x = syn.normal_bf16(1000 + c, (m, d))
        gamma = syn.normal_bf16(2000 + c, (d,), std=1.0)
        z = syn.normal_f32(3000 + c, (d,))
        sigma = 0.05
        W = syn.normal_f64(4000 + c, (d, n))
        hz, _ = orc.aqn_rmsnorm(x, gamma, z, sigma)
        h, _ = orc.aqn_rmsnorm(x, gamma, None, 0.0)
        w = syn.bf16_to_f32(gamma).astype(np.float64)
        zz = np.float64(np.float32(sigma)) * z.astype(np.float64)
        lhs = hz @ W
        rhs = h @ (np.diag(1 + zz / w) @ W)
        worst = max(worst, np.abs(lhs - rhs).max())
    assert worst < 100 * float(printed)


def test_sigma_schedule_matches_pages(orc):
    start, end, stages = read_golden("aqn_schedule.txt")[0].split()
    start, end, stages = float(start), float(end), int(stages)
    s = [orc.aqn_sigma(k, start, end) for k in range(stages)]
    assert s[0] == 0.0
    assert s[1] == start
    assert s[9] == pytest.approx(end, rel=1e-15)
    ratios = [s[k + 1] / s[k] for k in range(1, 9)]
    assert np.allclose(ratios, (end / start) ** (1 / 8), rtol=1e-14)
    assert all(a > b for a, b in zip(s[1:], s[2:]))  # monotone decay


def test_group_advantage_matches_pages(orc):
    lines = read_golden("advantage_example.txt")
    env = {"sqrt": math.sqrt}
    for ln in lines:
        rew, adv = ln.split("|")
        R = np.array([[float(v) for v in rew.split()]], dtype=np.float32)
        expect = [eval(e, env) for e in adv.split()]
        got = orc.group_advantage(R, eps=0.0 if R.std() > 0 else 1e-6)[0]
        assert np.allclose(got, expect, rtol=1e-15, atol=0)
    # with the 1e-6 epsilon of the workload: sqrt(3)/4 + 1e-6 in the denominator
    got = orc.group_advantage(np.array([[1, 0, 0, 0]], dtype=np.float32), eps=1e-6)[0]
    assert got[0] == pytest.approx(0.75 / (math.sqrt(3) / 4 + 1e-6), rel=1e-15)


def test_silu_mul_closed_form(orc):
    g = np.array([0.0, 1.0, -1.0, 20.0, -20.0])
    u = np.array([3.0, 2.0, 2.0, 1.0, 1.0])
    out = orc.silu_mul(g, u)
    assert out[0] == 0.0
    assert out[1] == pytest.approx(2 / (1 + math.e ** -1), rel=1e-15)
    assert out[2] == pytest.approx(-2 / (1 + math.e), rel=1e-15)
    assert out[3] == pytest.approx(20.0, rel=1e-8) and abs(out[4]) < 1e-7
