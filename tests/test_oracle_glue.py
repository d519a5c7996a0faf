"""Pins of the oracle's layer glue against independent fp64 implementations in PyTorch (CPU).

The decode layer the pages describe puts one norm before q/k/v and one before the gated feed-forward block, the gating
product and its nonlinearity before Down ("QeRL: When Quantized Weights Help Reinforcement Learning, and Where the
Evidence Stops", §5.1), with the attention scores left out of the workload. With the scores left out, attention is
taken over a single key position: softmax of one score is exactly 1, so each query head returns the value vector of
the key/value head its group shares. These tests hold the oracle to:
- torch's scaled_dot_product_attention with grouped key/value heads (enable_gqa), over one key position, in fp64:
  fixes which query heads read which value head;
- torch's SiLU in fp64: fixes the sign and form of the gating nonlinearity;
- a layer composed from torch fp64 primitives (rms_norm, matmul on the dequantized weight, the LoRA term, the same
  attention call, SiLU, residuals, bf16 casts at the storage points): fixes the order and wiring of the whole layer.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def sdpa_one_key(q, k, v, heads_q, heads_kv, head_dim):
    """Attention over a single key position with grouped kv heads: [m, Hq*hd], [m, Hkv*hd], [m, Hkv*hd] -> [m, Hq*hd]."""
    m = v.shape[0]
    qt = torch.as_tensor(q, dtype=torch.float64).reshape(m, heads_q, 1, head_dim)
    kt = torch.as_tensor(k, dtype=torch.float64).reshape(m, heads_kv, 1, head_dim)
    vt = torch.as_tensor(v, dtype=torch.float64).reshape(m, heads_kv, 1, head_dim)
    return F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True).reshape(m, heads_q * head_dim).numpy()


@pytest.mark.parametrize("group,heads_kv,head_dim", [(7, 4, 128), (5, 8, 128), (4, 2, 32), (1, 3, 16)])
def test_gqa_broadcast_is_attention_over_one_key(orc, group, heads_kv, head_dim):
    rng = np.random.default_rng(group * 100 + heads_kv)
    m = 3
    v = rng.standard_normal((m, heads_kv * head_dim))
    q = rng.standard_normal((m, heads_kv * group * head_dim))
    k = rng.standard_normal((m, heads_kv * head_dim))
    ref = sdpa_one_key(q, k, v, heads_kv * group, heads_kv, head_dim)
    got = orc.gqa_broadcast(v, group, head_dim)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_gqa_broadcast_detects_a_swapped_mapping(orc):
    """The pin separates the grouped mapping (query head j reads kv head j // group) from the tiled one (j % heads)."""
    rng = np.random.default_rng(1)
    m, hkv, g, hd = 2, 4, 7, 8
    v = rng.standard_normal((m, hkv * hd))
    ref = sdpa_one_key(rng.standard_normal((m, hkv * g * hd)), rng.standard_normal((m, hkv * hd)), v, hkv * g, hkv, hd)
    tiled = np.tile(v.reshape(m, hkv, hd), (1, g, 1)).reshape(m, -1)
    assert not np.array_equal(tiled, ref)
    assert np.array_equal(orc.gqa_broadcast(v, g, hd), ref)


def test_silu_mul_is_torch_silu(orc):
    rng = np.random.default_rng(2)
    g = np.concatenate([rng.standard_normal(5000) * 4, [0.0, -0.0, 1e-300, -700.0, 700.0, 30.0, -30.0]])
    u = rng.standard_normal(g.size)
    ref = (F.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    got = orc.silu_mul(g, u)
    assert np.all(np.abs(got - ref) <= 4e-16 * np.abs(ref) + 1e-300)
    # a sign-flipped nonlinearity (x / (1 + e^x)) is far from it
    flipped = g / (1.0 + np.exp(np.clip(g, -700, 700))) * u
    assert np.abs(flipped - ref).max() > 1.0


def bf16_t(a64: torch.Tensor) -> torch.Tensor:
    """fp64 -> bf16 (torch's round-to-nearest-even cast) -> fp64."""
    return a64.to(torch.bfloat16).to(torch.float64)


def bits_to_t(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def torch_decoder_layer(x, qw, lora, gamma1, gamma2, noise1, noise2, sigma, lam, group, head_dim, eps=1e-6):
    """The decode layer from torch fp64 primitives: rms_norm with weight gamma + sigma*noise, x W^T on the exactly
    dequantized weight, lambda (x A^T) B^T, attention over one key position with grouped kv heads, SiLU(gate)*up,
    pre-norm residuals; bf16 casts where the device stores bf16 tensors."""
    def lin(h, nm):
        W = torch.from_numpy(qw[nm])
        A, B = (bits_to_t(t) for t in lora[nm])
        return h @ W.T + lam * ((h @ A.T) @ B.T)

    xt = bits_to_t(x)
    d = xt.shape[1]
    w1 = bits_to_t(gamma1) + sigma * torch.from_numpy(noise1.astype(np.float64))
    h1 = bf16_t(F.rms_norm(xt, (d,), weight=w1, eps=eps))
    q, k, v = bf16_t(lin(h1, "q")), bf16_t(lin(h1, "k")), bf16_t(lin(h1, "v"))
    hq, hkv = q.shape[1] // head_dim, v.shape[1] // head_dim
    attn = torch.from_numpy(sdpa_one_key(q.numpy(), k.numpy(), v.numpy(), hq, hkv, head_dim))
    x2 = bf16_t(lin(attn, "o") + xt)
    w2 = bits_to_t(gamma2) + sigma * torch.from_numpy(noise2.astype(np.float64))
    h2 = bf16_t(F.rms_norm(x2, (d,), weight=w2, eps=eps))
    a = bf16_t(F.silu(lin(h2, "gate")) * lin(h2, "up"))
    out = bf16_t(lin(a, "down") + x2)
    return {"q": q, "k": k, "attn": attn, "x2": x2, "a": a, "out": out}


@pytest.mark.parametrize("m,hidden,kv,inter,head_dim", [(4, 256, 64, 512, 32), (3, 384, 128, 640, 64)])
def test_decoder_layer_matches_torch_composition(orc, syn, m, hidden, kv, inter, head_dim):
    group = hidden // kv
    s = lambda t: syn.seed_for(11, m, t)
    shapes = {"q": (hidden, hidden), "k": (kv, hidden), "v": (kv, hidden), "o": (hidden, hidden),
              "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)}
    w = {nm: syn.normal_bf16(s("w_" + nm), nk, std=0.02) for nm, nk in shapes.items()}
    lora = {nm: (syn.normal_bf16(s("a_" + nm), (8, nk[1]), std=0.02), syn.normal_bf16(s("b_" + nm), (nk[0], 8), std=0.02))
            for nm, nk in shapes.items()}
    x = syn.normal_bf16(s("x"), (m, hidden))
    g1, g2 = syn.normal_bf16(s("gamma"), (hidden,), std=1.0), syn.bf16_const(1.0, (hidden,))
    n1, n2 = syn.normal_f32(s("eps_norm1"), (hidden,)), syn.normal_f32(s("eps_norm2"), (hidden,))
    sigma = float(np.float32(orc.aqn_sigma(3)))
    qref = {nm: orc.nvfp4_quantize(v)[:3] for nm, v in w.items()}
    qw = {nm: orc.nvfp4_dequantize(*qref[nm])[0] for nm in w}
    got = orc.decoder_layer(x, qref, lora, g1, g2, n1, n2, sigma, 2.0, group, head_dim)
    ref = torch_decoder_layer(x, qw, lora, g1, g2, n1, n2, sigma, 2.0, group, head_dim)
    for name in ("q", "k", "attn", "x2", "a", "out"):
        g = bits_to_t(got[name]).numpy()
        r = ref[name].numpy()
        # both sides round the same fp64 sums to bf16; sums taken in another order may cross a rounding boundary
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
        assert np.all(np.abs(g - r) <= ulp), name
        assert np.mean(g == r) > 0.99, name
