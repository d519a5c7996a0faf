"""GPU parity of the MXFP4 variant (OCP MX: E2M1 elements with one E8M0 scale per 32 weights) against the oracle.

- the quantizer's canonical layout bit for bit (codes and E8M0 scales), on normal weights, heavy-tailed weights whose
  block exponents span many binades, crafted blocks at the exponent rule's edges and midpoints, zero and non-finite
  blocks, and the full 7B gate weight;
- the canonical dequantization bit for bit (X * q rounded once to f32);
- the tiled form (the same weight re-expressed with power-of-two NVFP4 block and tensor scales): its reconstruction
  through nvfp4_dequantize equals the MXFP4 reconstruction bit for bit, and a block too far below the tensor's largest
  is reported;
- the linear through every kernel (decode, general, many-token) and the backward with MXFP4 weights, against the
  oracle's MXFP4 linear at the linear bar (max |y - r| / max |r| <= 2e-3);
- mxfp4_lora_linear on the scaled FP4 x FP8 MFMA kernel (canonical weights, activations as E4M3 hi and lo parts with
  block scales) against the same oracle: ragged shapes and token counts, wide-range activations, the SiLU epilogue,
  a residual, and the 7B gate|up weights at 512 tokens on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, LINEAR_TOL, bf16_bits_to_f64, dev_bf16, dev_f32, host_u8, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


def gpu_mx(qn, w_np, flags=None):
    n, k = w_np.shape
    wq = qn.mxfp4_quantize(dev_bf16(w_np), qn.LAYOUT_ROWMAJOR, flags)
    torch.cuda.synchronize()
    return host_u8(wq.codes)[: n * k // 2].reshape(n, k // 2), host_u8(wq.scales)[: n * k // 32].reshape(n, k // 32), wq


def heavy(seed, n, k, emin=-30, emax=20):
    """Normal weights times 2^e per 32-block, e uniform on emin..emax (block exponents over many binades)."""
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, 1.0, (n, k)) * 2.0 ** rng.integers(emin, emax + 1, (n, k // 32)).repeat(32, axis=1)
    return (w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("n,k,kind", [(64, 256, "normal"), (40, 96, "normal"), (17, 32, "normal"),
                                      (96, 3584, "heavy"), (33, 4096, "heavy")])
def test_quantize_bitexact(qn, n, k, kind):
    w = synth.normal_bf16(n + k, (n, k), std=0.02) if kind == "normal" else heavy(n + k, n, k)
    c, s, _ = gpu_mx(qn, w)
    oc, os_, _ = oracle.mxfp4_quantize(w)
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc)


def test_quantize_edges_and_special_blocks(qn):
    """Blocks whose largest magnitude sits at the exponent rule's edges (2^e, 6 * 2^e, just under 8 * 2^e, 8 * 2^e),
    exact midpoints, a zero block with negative zeros, non-finite weights, and the smallest and largest bf16."""
    rows = []
    for e in (-126, -20, 0, 20, 100):
        for top in (1.0, 6.0, 7.5, 8.0):
            r = np.zeros(32)
            r[0] = top * 2.0 ** e
            r[1:8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 2.0 ** (e - 2 if top < 6 else e)
            r[8:15] = -r[1:8]
            rows.append(r)
    w = np.array(rows, dtype=np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    extra = np.zeros((3, 32), dtype=np.uint16)
    extra[0, :] = 0x8000               # all negative zeros
    extra[1, :4] = [0x7F80, 0xFF80, 0x7FC0, 0x3F80]  # +inf, -inf, NaN, 1.0
    extra[2, :3] = [0x0001, 0x7F7F, 0x8001]          # smallest subnormal, largest finite, -smallest
    bits = np.concatenate([bits, extra])
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    c, s, _ = gpu_mx(qn, bits, flags)
    oc, os_, ofl = oracle.mxfp4_quantize(bits)
    assert np.array_equal(s, os_) and np.array_equal(c, oc)
    assert int(flags.item()) == ofl == 1


def test_quantize_7b_gate_full_size(qn):
    """The 7B gate weight (18,944 x 3,584) with the benchmark's weight distribution, every code and scale."""
    w = synth.normal_bf16(synth.seed_for(2, 0, "w_gate"), (18944, 3584), std=0.02)
    c, s, _ = gpu_mx(qn, w)
    oc, os_, _ = oracle.mxfp4_quantize(w)
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc)


def test_dequantize_bitexact(qn):
    w = heavy(7, 48, 512)
    _, _, wq = gpu_mx(qn, w)
    got = qn.mxfp4_dequantize(wq).cpu().numpy()
    oc, os_, _ = oracle.mxfp4_quantize(w)
    _, ref = oracle.mxfp4_dequantize(oc, os_)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n,k,kind", [(64, 256, "normal"), (40, 320, "normal"), (96, 3584, "heavy15")])
def test_tiled_form_reconstructs_the_mx_weight(qn, n, k, kind):
    """nvfp4_dequantize of the tiled form == the MXFP4 reconstruction, bit for bit; ragged n and k % 128 != 0 pad."""
    w = synth.normal_bf16(n * 3 + k, (n, k), std=0.02) if kind == "normal" else heavy(11, n, k, emin=-14, emax=0)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    wt = qn.mxfp4_quantize(dev_bf16(w), qn.LAYOUT_TILED, flags)
    got = qn.dequantize(wt).cpu().numpy()
    oc, os_, _ = oracle.mxfp4_quantize(w)
    _, ref = oracle.mxfp4_dequantize(oc, os_)
    assert int(flags.item()) == 0
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_tiled_form_reports_blocks_out_of_its_range(qn):
    w = synth.normal_bf16(5, (16, 128), std=0.02).copy()
    tiny = (np.float32(2.0 ** -40) * np.ones(32, np.float32)).view(np.uint32) >> 16
    w[3, 32:64] = tiny.astype(np.uint16)  # a block 2^-30 below the others: past the 17 binades the form holds
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    qn.mxfp4_quantize(dev_bf16(w), qn.LAYOUT_TILED, flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 2


class MxCase:
    def __init__(self, m, ns, k, r=32, seed=0, lam=2.0, aqn=True):
        s = lambda t, p=0: synth.seed_for(140 + seed, p, t)
        self.m, self.ns, self.k, self.r, self.lam, self.aqn = m, ns, k, r, lam, aqn
        self.x = synth.normal_bf16(s("x"), (m, k))
        self.w = [synth.normal_bf16(s("w_q", p), (n, k), std=0.02) for p, n in enumerate(ns)]
        self.A = [synth.normal_bf16(s("a_q", p), (r, k), std=0.02) if r else None for p in range(len(ns))]
        self.B = [synth.normal_bf16(s("b_q", p), (n, r), std=0.02) if r else None for p, n in enumerate(ns)]
        self.gamma = synth.normal_bf16(s("gamma"), (k,), std=1.0)
        self.noise = synth.normal_f32(s("eps_norm1"), (k,))
        self.sigma = float(np.float32(1e-2))

    def h(self):
        return oracle.aqn_rmsnorm(self.x, self.gamma, self.noise, self.sigma, 1e-6)[1] if self.aqn else self.x

    def ref(self, p):
        c, sc, _ = oracle.mxfp4_quantize(self.w[p])
        return oracle.mxfp4_lora_linear(self.h(), c, sc, self.A[p], self.B[p], self.lam)

    def gpu(self, qn, epilogue=0, opts=None):
        ys, projs = [], []
        for p, n in enumerate(self.ns):
            wt = qn.mxfp4_quantize(dev_bf16(self.w[p]), qn.LAYOUT_TILED)
            y = torch.full((self.m, n), float("nan"), dtype=torch.float32, device=DEV)
            ys.append(y)
            A = dev_bf16(self.A[p]) if self.r else None
            B = dev_bf16(self.B[p]) if self.r else None
            projs.append(qn.Projection(wt, None if (epilogue and p == 1) else y, A, B, self.lam))
        aqn = qn.make_aqn(dev_bf16(self.gamma), dev_f32(self.noise), self.sigma, 1e-6) if self.aqn else None
        qn.lora_linear(dev_bf16(self.x), projs, aqn, epilogue, opts=opts)
        torch.cuda.synchronize()
        return ys


@pytest.mark.parametrize("m,ns,k,path", [(1, [200], 1024, "auto"), (16, [520, 64], 1024, "decode"),
                                         (16, [384], 3584, "general"), (40, [272], 640, "auto"),
                                         (300, [256], 512, "auto"), (130, [96, 64], 1024, "many")])
def test_linear_with_mxfp4_weights(qn, m, ns, k, path):
    opts = {"auto": None, "decode": qn.LinearOpts(kernel=qn.KERNEL_DECODE),
            "general": qn.LinearOpts(kernel=qn.KERNEL_GENERAL), "many": qn.LinearOpts(kernel=qn.KERNEL_MANY)}[path]
    c = MxCase(m, ns, k, seed=m + k)
    ys = c.gpu(qn, opts=opts)
    for p in range(len(ns)):
        assert rel_err(ys[p].cpu().numpy(), c.ref(p)) <= LINEAR_TOL, (path, p)


def native(qn, c, epilogue=0, residual=None):
    """The case through mxfp4_lora_linear: canonical MX weights on the scaled FP4 x FP8 MFMA kernel."""
    ys, projs = [], []
    for p, n in enumerate(c.ns):
        wq = qn.mxfp4_quantize(dev_bf16(c.w[p]), qn.LAYOUT_ROWMAJOR)
        y = torch.full((c.m, n), float("nan"), dtype=torch.float32, device=DEV)
        ys.append(y)
        A = dev_bf16(c.A[p]) if c.r else None
        B = dev_bf16(c.B[p]) if c.r else None
        projs.append(qn.Projection(wq, None if (epilogue and p == 1) else y, A, B, c.lam, residual=residual))
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6) if c.aqn else None
    qn.mxfp4_lora_linear(dev_bf16(c.x), projs, aqn, epilogue)
    torch.cuda.synchronize()
    return ys


@pytest.mark.parametrize("m,ns,k,r,aqn", [(5, [96], 256, 32, True), (130, [200, 72], 1056, 16, True),
                                          (300, [1000], 512, 0, False), (256, [512], 4096, 64, True),
                                          (1, [48], 32, 32, False), (129, [16, 40, 24], 384, 32, True)])
def test_native_mxfp4_linear(qn, m, ns, k, r, aqn):
    """mxfp4_lora_linear on the scaled-MFMA kernel against the oracle's MXFP4 linear: one to three projections,
    ragged n (1000, 40) and token counts (1, 5, 129, 130, 300), a k whose last 128-wide k-tile is a single 32-block
    (1056) and k = 32, ranks 0 to 64, with and without the norm."""
    c = MxCase(m, ns, k, r=r, seed=7 * m + k, aqn=aqn)
    ys = native(qn, c)
    for p in range(len(ns)):
        assert rel_err(ys[p].cpu().numpy(), c.ref(p)) <= LINEAR_TOL, p


def test_native_mxfp4_wide_range_activations(qn):
    """Activations spanning 2^-20..2^0 within every 32-block (normal values times 2^e, e uniform on -20..0), so many
    values lie below the hi part's range and live in the lo part, or below both."""
    c = MxCase(140, [256], 1024, seed=11, aqn=False)
    rng = np.random.default_rng(11)
    x = rng.normal(0.0, 1.0, c.x.shape) * 2.0 ** rng.integers(-20, 1, c.x.shape)
    c.x = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = native(qn, c)[0]
    assert rel_err(y.cpu().numpy(), c.ref(0)) <= LINEAR_TOL


def test_native_mxfp4_silu_epilogue_and_residual(qn):
    """SiLU(gate) * up from a gate|up pair, and a single projection with a residual added, on the scaled-MFMA
    kernel."""
    c = MxCase(200, [384, 384], 640, seed=12)
    y = native(qn, c, epilogue=qn.EPI_SILU_MUL)[0]
    assert rel_err(y.cpu().numpy(), oracle.silu_mul(c.ref(0), c.ref(1))) <= LINEAR_TOL
    c2 = MxCase(150, [256], 512, seed=13)
    res = synth.normal_bf16(synth.seed_for(153, 0, "x"), (150, 256))
    y2 = native(qn, c2, residual=dev_bf16(res))[0]
    assert rel_err(y2.cpu().numpy(), c2.ref(0) + bf16_bits_to_f64(res)) <= LINEAR_TOL


def test_native_mxfp4_7b_gate_up_sampled(qn):
    """The 7B gate|up weights (18,944 x 3,584 each, canonical MXFP4) at 512 tokens with the norm and SiLU(gate) * up,
    every output of 48 sampled rows against the oracle on those rows."""
    m, n, k = 512, 18944, 3584
    s = lambda t: synth.seed_for(154, 0, t)
    c = MxCase(m, [n, n], k, seed=14)
    y = native(qn, c, epilogue=qn.EPI_SILU_MUL)[0].cpu().numpy()
    rows = np.random.default_rng(14).choice(n, 48, replace=False)
    h = c.h()
    outs = []
    for p in range(2):
        cc, sc, _ = oracle.mxfp4_quantize(c.w[p][rows])
        outs.append(oracle.mxfp4_lora_linear(h, cc, sc, c.A[p], c.B[p][rows], c.lam))
    assert rel_err(y[:, rows], oracle.silu_mul(outs[0], outs[1])) <= LINEAR_TOL


def test_linear_silu_epilogue_with_mxfp4_weights(qn):
    c = MxCase(8, [384, 384], 1024, seed=3)
    y = c.gpu(qn, epilogue=qn.EPI_SILU_MUL)[0]
    ref = oracle.silu_mul(c.ref(0), c.ref(1))
    assert rel_err(y.cpu().numpy(), ref) <= LINEAR_TOL


def test_backward_with_mxfp4_weights(qn):
    """dh = W_hat^T g + lambda A^T (B^T g) with an MXFP4 W_hat (tiled form); the reference is fp64 numpy on the
    oracle's exact MXFP4 reconstruction."""
    m, n, k, r, lam = 33, 200, 512, 32, 2.0
    s = lambda t: synth.seed_for(151, 0, t)
    w = synth.normal_bf16(s("w_q"), (n, k), std=0.02)
    h = synth.normal_bf16(s("x"), (m, k))
    g = synth.normal_bf16(s("eps_norm1"), (m, n))
    A = synth.normal_bf16(s("a_q"), (r, k), std=0.02)
    B = synth.normal_bf16(s("b_q"), (n, r), std=0.02)
    wt = qn.mxfp4_quantize(dev_bf16(w), qn.LAYOUT_TILED)
    got = qn.lora_linear_backward(dev_bf16(g), dev_bf16(h), wt, dev_bf16(A), dev_bf16(B), lam, torch.float32,
                                  ("dh",))["dh"].cpu().numpy()
    oc, os_, _ = oracle.mxfp4_quantize(w)
    we, _ = oracle.mxfp4_dequantize(oc, os_)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = f(g) @ we + lam * (f(g) @ f(B)) @ f(A)
    assert rel_err(got, ref) <= LINEAR_TOL
