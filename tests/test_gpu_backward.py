"""GPU parity of the backward through the frozen NVFP4 weight (nvfp4_lora_linear_backward) against the fp64 oracle.

dh = s_g W_hat^T g + lambda A^T (B^T g), dA = lambda (B^T g)^T h, dB = lambda g^T (A h), checked with the bar of the
forward (max |y - r| / max |r| <= 2e-3 on f32 outputs) on ragged shapes (output rows not a multiple of 32, input
channels not a multiple of 128, token counts not a multiple of 16), ranks 8..64 and none, lambda = 0, bf16 dh, the 7B
gate and down shapes with every output, and the 8192-token batch (dA, dB in full, dh on sampled tokens).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, LINEAR_TOL, dev_bf16, host_bf16, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


class Bwd:
    def __init__(self, m, n, k, r, seed, lam=2.0, g_std=1.0):
        s = lambda t: synth.seed_for(13, seed, t)
        self.m, self.n, self.k, self.r, self.lam = m, n, k, r, lam
        self.w = synth.normal_bf16(s("w_q"), (n, k), std=0.02)
        self.h = synth.normal_bf16(s("x"), (m, k))
        self.g = synth.normal_bf16(s("eps_norm1"), (m, n), std=g_std)
        self.A = synth.normal_bf16(s("a_q"), (r, k), std=0.02) if r else None
        self.B = synth.normal_bf16(s("b_q"), (n, r), std=0.02) if r else None

    def gpu(self, qn, dh_dtype=torch.float32, want=("dh", "dA", "dB")):
        wq = qn.quantize(dev_bf16(self.w), qn.LAYOUT_TILED)
        A = dev_bf16(self.A) if self.r else None
        B = dev_bf16(self.B) if self.r else None
        out = qn.lora_linear_backward(dev_bf16(self.g), dev_bf16(self.h), wq, A, B, self.lam, dh_dtype, want)
        torch.cuda.synchronize()
        return out

    def ref(self, rows=None, want=("dh", "dA", "dB")):
        c, sb, sg, _ = oracle.nvfp4_quantize(self.w)
        g, h = (self.g, self.h) if rows is None else (self.g[rows], self.h[rows])
        return oracle.lora_linear_backward(g, h, c, sb, sg, self.A, self.B, self.lam, want)


@pytest.mark.parametrize("m,n,k,r", [(5, 40, 64, 8), (17, 33, 160, 12), (130, 100, 256, 32), (64, 48, 128, 64),
                                     (1, 16, 128, 32), (257, 520, 1040, 32), (40, 1000, 640, 16)])
def test_backward_ragged(qn, m, n, k, r):
    c = Bwd(m, n, k, r, seed=m * 7 + n)
    got, ref = c.gpu(qn), c.ref()
    for key in ("dh", "dA", "dB"):
        assert rel_err(got[key].cpu().numpy(), ref[key]) <= LINEAR_TOL, key


def test_backward_no_adapter_and_zero_lambda(qn):
    c = Bwd(24, 72, 384, 0, seed=3)
    got = c.gpu(qn, want=("dh",))
    assert rel_err(got["dh"].cpu().numpy(), c.ref(want=("dh",))["dh"]) <= LINEAR_TOL
    c = Bwd(24, 72, 384, 16, seed=4, lam=0.0)
    got, ref = c.gpu(qn), c.ref()
    assert rel_err(got["dh"].cpu().numpy(), ref["dh"]) <= LINEAR_TOL
    assert torch.count_nonzero(got["dA"]) == 0 and torch.count_nonzero(got["dB"]) == 0


def test_backward_bf16_dh_is_rounded_f32(qn):
    c = Bwd(33, 200, 512, 32, seed=5)
    d32 = c.gpu(qn, torch.float32, ("dh",))["dh"]
    d16 = c.gpu(qn, torch.bfloat16, ("dh",))["dh"]
    assert torch.equal(d16, d32.to(torch.bfloat16))


def test_backward_deterministic(qn):
    c = Bwd(100, 300, 640, 32, seed=6)
    a, b = c.gpu(qn), c.gpu(qn)
    for key in ("dh", "dA", "dB"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("m,n,k", [(128, 18944, 3584), (64, 3584, 18944)])
def test_backward_7b_shapes_full(qn, m, n, k):
    """The 7B gate (18944 x 3584) and down (3584 x 18944) shapes, rank 32, every output."""
    c = Bwd(m, n, k, 32, seed=n % 101)
    print(f"[backward] {m} x {n} x {k}: oracle", flush=True)
    got, ref = c.gpu(qn), c.ref()
    for key in ("dh", "dA", "dB"):
        assert rel_err(got[key].cpu().numpy(), ref[key]) <= LINEAR_TOL, key


def test_backward_prefill_batch(qn):
    """8192 tokens through the 7B gate shape: dA and dB (sums over every token) in full, dh on 16 sampled tokens."""
    m, n, k = 8192, 18944, 3584
    c = Bwd(m, n, k, 32, seed=8192)
    got = c.gpu(qn)
    print("[backward] 8192 tokens: oracle dA, dB", flush=True)
    ref = c.ref(want=("dA", "dB"))
    assert rel_err(got["dA"].cpu().numpy(), ref["dA"]) <= LINEAR_TOL
    assert rel_err(got["dB"].cpu().numpy(), ref["dB"]) <= LINEAR_TOL
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(0).integers(0, m, 14)]))
    refh = c.ref(rows=rows, want=("dh",))["dh"]
    assert rel_err(got["dh"].cpu().numpy()[rows], refh) <= LINEAR_TOL
