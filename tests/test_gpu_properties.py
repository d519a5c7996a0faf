"""Properties of the linear that hold exactly or up to f32 summation order, checked GPU against GPU (no oracle):

- negation symmetry: y(-x) = -y(x) without a residual or SiLU, with and without the norm, up to the matrix cores'
  own rounding. Every step the kernels take is odd in x: the norm's rstd and the activations' power-of-two
  exponents depend on |x| only, and the f16 and E4M3 conversions and the bf16 hi/lo split of t round to nearest
  even. The MFMA's internal sums are not rounded symmetrically, though: a few outputs of a call differ by about an
  ulp (measured up to 2.3e-7 of max |y|), so the bar is 1e-6 of max |y|; a sign or index mistake would be O(1).
- split-k invariance: the decode kernels' k-chunk counts change only the order of the f32 partial sums.
- row independence: each row of a batch equals the call on that row alone, up to f32 summation order (different
  batch sizes may take different kernels and cuts; on the cases here the rows came out bit-identical).
- special cases, bit for bit: sigma = 0 is the plain RMSNorm whatever the noise; B = 0 is lambda = 0.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, dev_bf16, dev_f32
from test_gpu_linear import Case

pytestmark = pytest.mark.gpu

SUM_ORDER_TOL = 1e-4  # max |a - b| / max |b| between two summation orders of the same exact products
NEGATION_TOL = 1e-6   # max |y(-x) + y(x)| / max |y(x)|: the matrix cores' asymmetric internal rounding


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


def negated(c):
    n = Case.__new__(Case)
    n.__dict__.update(c.__dict__)
    n.x = c.x ^ np.uint16(0x8000)
    return n


@pytest.mark.parametrize("m,n,k,aqn,kernel", [(16, 512, 2048, False, "AUTO"), (16, 512, 2048, True, "DECODE"),
                                              (8, 96, 256, True, "GENERAL"), (40, 256, 1024, False, "WIDE"),
                                              (4, 64, 256, True, "FUSED"), (300, 256, 512, True, "MANY")])
def test_negation_symmetry(qn, m, n, k, aqn, kernel):
    c = Case(m, [n], k, seed=21, aqn=aqn)
    opts = qn.LinearOpts(kernel=getattr(qn, "KERNEL_" + kernel))
    y = c.gpu(qn, opts=opts)[0].clone()
    yn = negated(c).gpu(qn, opts=opts)[0]
    assert torch.isfinite(y).all()
    err = float((yn + y).abs().max() / y.abs().max())
    assert err <= NEGATION_TOL, err


def test_negation_symmetry_mxfp4_native(qn):
    """The same on the scaled-MFMA MXFP4 kernel: the E4M3 hi/lo parts and their block exponents are odd in x too."""
    m, n, k = 200, 256, 640
    c = Case(m, [n], k, seed=22, aqn=True)
    wq = qn.mxfp4_quantize(dev_bf16(c.w[0]), qn.LAYOUT_ROWMAJOR)
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
    out = []
    for xb in (c.x, c.x ^ np.uint16(0x8000)):
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
        qn.mxfp4_lora_linear(dev_bf16(xb), [qn.Projection(wq, y, dev_bf16(c.A[0]), dev_bf16(c.B[0]), c.lam)], aqn)
        out.append(y)
    torch.cuda.synchronize()
    assert torch.isfinite(out[0]).all()
    err = float((out[1] + out[0]).abs().max() / out[0].abs().max())
    assert err <= NEGATION_TOL, err


@pytest.mark.parametrize("m,n,k,kernel,chunks", [(16, 256, 2048, "DECODE", [1, 2, 4, 8]),
                                                 (40, 256, 1024, "WIDE", [1, 2, 4])])
def test_split_k_invariance(qn, m, n, k, kernel, chunks):
    c = Case(m, [n], k, seed=23, aqn=True)
    ys = [c.gpu(qn, opts=qn.LinearOpts(kernel=getattr(qn, "KERNEL_" + kernel), decode_kchunks=nk))[0].clone()
          for nk in chunks]
    ref = ys[0]
    for nk, y in zip(chunks[1:], ys[1:]):
        err = float((y - ref).abs().max() / ref.abs().max())
        assert err <= SUM_ORDER_TOL, (nk, err)


@pytest.mark.parametrize("m,n,k", [(16, 384, 1024), (40, 200, 640)])
def test_rows_match_single_token_calls(qn, m, n, k):
    c = Case(m, [n], k, seed=24, aqn=True)
    ys = c.gpu(qn)[0].clone()
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
    A, B = dev_bf16(c.A[0]), dev_bf16(c.B[0])
    for r in range(m):
        y1 = torch.full((1, n), float("nan"), dtype=torch.float32, device=DEV)
        qn.lora_linear(c.xd[r:r + 1], [qn.Projection(c.wq[0], y1, A, B, c.lam)], aqn)
        torch.cuda.synchronize()
        err = float((y1[0] - ys[r]).abs().max() / ys[r].abs().max())
        assert err <= SUM_ORDER_TOL, (r, err)


def test_zero_sigma_ignores_the_noise(qn):
    """sigma = 0 is the plain RMSNorm whatever noise is given: the standalone norm and the fused prologue give the
    bits they give without noise."""
    c = Case(16, [256], 1024, seed=25, aqn=True, sigma=0.0)
    x, g, z = dev_bf16(c.x), dev_bf16(c.gamma), dev_f32(c.noise)
    assert torch.equal(qn.aqn_rmsnorm(x, g, z, 0.0, 1e-6).view(torch.int16),
                       qn.aqn_rmsnorm(x, g, None, 0.0, 1e-6).view(torch.int16))
    y = c.gpu(qn)[0].clone()
    c.noise = np.zeros_like(c.noise)
    assert torch.equal(c.gpu(qn)[0], y)


@pytest.mark.parametrize("m", [16, 300])
def test_zero_adapter_is_the_base(qn, m):
    """B = 0 gives the bits of lambda = 0: the LoRA term adds exactly zero."""
    c = Case(m, [256], 512, seed=26, aqn=True)
    c.B = [np.zeros_like(b) for b in c.B]
    y = c.gpu(qn)[0].clone()
    c.lam = 0.0
    assert torch.equal(c.gpu(qn)[0], y)
