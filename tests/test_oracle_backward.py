"""Pins of the oracle's backward through the frozen NVFP4 weight ("QeRL: When Quantized Weights Help Reinforcement
Learning, and Where the Evidence Stops", §2.1: the backbone is frozen, gradients update A and B and may pass through
the frozen projection to reach an earlier adapter).

The forward oracle (lora_linear, pinned on its own) fixes the backward: with L = <g, y> and y linear in each of h, A
and B separately, every gradient is the exact derivative of a linear function, so
  - Euler / adjoint identities: <g, y(h)> = <h, dh>, the LoRA part <g, lambda B A h> = <A, dA> = <B, dB>;
  - a perturbation of a single entry by delta changes L by exactly delta times that gradient entry (this catches a
    transposed or shifted index, which the sums alone might not);
  - lambda = 0 or B = 0 leaves dA = dB = 0 and dh = the base's transposed product.
All in fp64; inputs are bf16 and every perturbed value is chosen exactly representable.
"""
import numpy as np
import pytest


def setup(orc, syn, m=5, n=40, k=64, r=8, seed=0, lam=2.0):
    s = lambda t: syn.seed_for(12, seed, t)
    w = syn.normal_bf16(s("w_q"), (n, k), std=0.02)
    codes, sb, sg, _ = orc.nvfp4_quantize(w)
    h = syn.normal_bf16(s("x"), (m, k))
    g = syn.normal_bf16(s("eps_norm1"), (m, n))
    A = syn.normal_bf16(s("a_q"), (r, k), std=0.05)
    B = syn.normal_bf16(s("b_q"), (n, r), std=0.05)
    return dict(w=w, codes=codes, sb=sb, sg=sg, h=h, g=g, A=A, B=B, lam=lam)


def f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def loss(orc, c, h=None, A=None, B=None, lora_only=False):
    """L = <g, y> from the forward oracle (or of the LoRA term alone)."""
    h = c["h"] if h is None else h
    A = c["A"] if A is None else A
    B = c["B"] if B is None else B
    y = orc.lora_linear(h, c["codes"], c["sb"], c["sg"], A, B, c["lam"])
    if lora_only:
        y = y - orc.lora_linear(h, c["codes"], c["sb"], c["sg"], None, None, 0.0)
    return float((f64(c["g"]) * y).sum())


@pytest.mark.parametrize("seed,shape", [(0, (5, 40, 64, 8)), (1, (3, 33, 48, 12)), (2, (17, 16, 160, 32))])
def test_adjoint_identities(orc, syn, seed, shape):
    m, n, k, r = shape
    c = setup(orc, syn, m, n, k, r, seed)
    d = orc.lora_linear_backward(c["g"], c["h"], c["codes"], c["sb"], c["sg"], c["A"], c["B"], c["lam"])
    L = loss(orc, c)
    assert abs(L - float((f64(c["h"]) * d["dh"]).sum())) <= 1e-12 * max(1.0, abs(L))
    Ll = loss(orc, c, lora_only=True)
    assert abs(Ll - float((f64(c["A"]) * d["dA"]).sum())) <= 1e-12 * max(1.0, abs(Ll))
    assert abs(Ll - float((f64(c["B"]) * d["dB"]).sum())) <= 1e-12 * max(1.0, abs(Ll))


def bump(a, idx, rng):
    """Copy of bf16 array `a` with entry idx replaced by another bf16 value; returns (copy, exact delta)."""
    b = a.copy()
    old = f64(a[idx])
    new_bits = np.uint16(np.float32(old + rng.choice([-1, 1]) * (abs(old) + 0.125)).view(np.uint32) >> 16)
    b[idx] = new_bits
    return b, float(f64(new_bits) - old)


def test_single_entry_perturbations(orc, syn):
    c = setup(orc, syn, 4, 36, 48, 12, seed=5)
    d = orc.lora_linear_backward(c["g"], c["h"], c["codes"], c["sb"], c["sg"], c["A"], c["B"], c["lam"])
    L0 = loss(orc, c)
    rng = np.random.default_rng(0)
    for _ in range(12):
        i, kk = rng.integers(0, 4), rng.integers(0, 48)
        h2, dl = bump(c["h"], (i, kk), rng)
        assert abs(loss(orc, c, h=h2) - L0 - dl * d["dh"][i, kk]) <= 1e-11 * max(1.0, abs(L0))
        j, kk = rng.integers(0, 12), rng.integers(0, 48)
        A2, dl = bump(c["A"], (j, kk), rng)
        assert abs(loss(orc, c, A=A2) - L0 - dl * d["dA"][j, kk]) <= 1e-11 * max(1.0, abs(L0))
        o, j = rng.integers(0, 36), rng.integers(0, 12)
        B2, dl = bump(c["B"], (o, j), rng)
        assert abs(loss(orc, c, B=B2) - L0 - dl * d["dB"][o, j]) <= 1e-11 * max(1.0, abs(L0))


def test_no_adapter_is_the_transposed_base(orc, syn):
    c = setup(orc, syn, 6, 32, 64, 8, seed=7)
    d0 = orc.lora_linear_backward(c["g"], c["h"], c["codes"], c["sb"], c["sg"], c["A"], c["B"], 0.0)
    assert np.all(d0["dA"] == 0.0) and np.all(d0["dB"] == 0.0)
    dn = orc.lora_linear_backward(c["g"], c["h"], c["codes"], c["sb"], c["sg"], None, None, 2.0)
    we, _ = orc.nvfp4_dequantize(c["codes"], c["sb"], c["sg"])
    assert np.allclose(dn["dh"], f64(c["g"]) @ we, rtol=1e-13, atol=1e-15)
    assert np.allclose(d0["dh"], dn["dh"], rtol=1e-13, atol=1e-15)
    zB = np.zeros_like(c["B"])
    dz = orc.lora_linear_backward(c["g"], c["h"], c["codes"], c["sb"], c["sg"], c["A"], zB, 2.0)
    assert np.all(dz["dA"] == 0.0) and np.allclose(dz["dh"], dn["dh"], rtol=1e-13, atol=1e-15)
