"""GPU parity of AQN-RMSNorm, the NVFP4 + LoRA linear and the decode layer against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, LINEAR_TOL, bf16_bits_to_f64, dev_bf16, dev_f32, host_bf16, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


class Case:
    """Seeded inputs of one projection group: x [m, k]; weights [n_p, k]; LoRA; norm parameters."""

    def __init__(self, m, ns, k, r=32, seed=0, aqn=True, sigma=1e-2, wdist="normal", lam=2.0):
        self.m, self.ns, self.k, self.r, self.lam = m, ns, k, r, lam
        s = lambda t, p=0: synth.seed_for(100 + seed, p, t)
        self.x = synth.normal_bf16(s("x"), (m, k))
        self.w, self.A, self.B = [], [], []
        for p, n in enumerate(ns):
            if wdist == "normal":
                self.w.append(synth.normal_bf16(s("w_q", p), (n, k), std=0.02))
            else:
                self.w.append(synth.student_t4_bf16(s("w_q", p), (n, k), 0.02, 16, s("block_exp", p), -14))
            self.A.append(synth.normal_bf16(s("a_q", p), (r, k), std=0.02) if r else None)
            self.B.append(synth.normal_bf16(s("b_q", p), (n, r), std=0.02) if r else None)
        self.aqn = aqn
        self.gamma = synth.normal_bf16(s("gamma"), (k,), std=1.0) if aqn else None
        self.noise = synth.normal_f32(s("eps_norm1"), (k,)) if aqn else None
        self.sigma = float(np.float32(sigma))

    def oracle_h(self):
        if not self.aqn:
            return self.x
        return oracle.aqn_rmsnorm(self.x, self.gamma, self.noise, self.sigma, 1e-6)[1]

    def oracle_y(self, p, rows=None):
        B = self.B[p]
        if rows is None:
            c, sb, sg, _ = oracle.nvfp4_quantize(self.w[p])
        else:  # s_g from the whole tensor, codes of the sampled rows only
            c, sb, sg, _ = oracle.nvfp4_quantize_rows(self.w[p], rows)
            B = None if B is None else B[rows]
        return oracle.lora_linear(self.oracle_h(), c, sb, sg, self.A[p], B, self.lam)

    def gpu(self, qn, y_dtype=torch.float32, epilogue=0, residual=None, opts=None):
        self.wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in self.w]
        ys, projs = [], []
        for p, n in enumerate(self.ns):
            y = torch.full((self.m, n), float("nan"), dtype=y_dtype, device=DEV)
            ys.append(y)
            A = dev_bf16(self.A[p]) if self.r else None
            B = dev_bf16(self.B[p]) if self.r else None
            projs.append(qn.Projection(self.wq[p], y, A, B, self.lam, residual=residual))
        aqn = qn.make_aqn(dev_bf16(self.gamma), dev_f32(self.noise), self.sigma, 1e-6) if self.aqn else None
        self.xd = dev_bf16(self.x)
        qn.lora_linear(self.xd, projs, aqn, epilogue, opts=opts)
        torch.cuda.synchronize()
        return ys


@pytest.mark.parametrize("m", [1, 2, 5, 16, 17, 40, 64, 65, 128, 130])
def test_linear_batch_sizes(qn, m):
    c = Case(m, [200], 1024, seed=m)
    y = c.gpu(qn)[0].cpu().numpy()
    assert rel_err(y, c.oracle_y(0)) <= LINEAR_TOL


@pytest.mark.parametrize("n,k", [(16, 128), (40, 272), (1000, 144), (33, 3584), (512, 1040)])
def test_linear_ragged_shapes(qn, n, k):
    for m in (1, 16):
        c = Case(m, [n], k, seed=n + k)
        y = c.gpu(qn)[0].cpu().numpy()
        assert rel_err(y, c.oracle_y(0)) <= LINEAR_TOL, (m, n, k)


def test_linear_three_projections_share_norm(qn):
    """q | k | v in one call, one AQN-RMSNorm feeding all three."""
    c = Case(8, [256, 64, 64], 512, seed=3)
    ys = c.gpu(qn)
    for p in range(3):
        assert rel_err(ys[p].cpu().numpy(), c.oracle_y(p)) <= LINEAR_TOL, p


@pytest.mark.parametrize("r", [0, 4, 8, 12, 32, 64])
def test_linear_lora_ranks(qn, r):
    c = Case(4, [128], 256, r=r, seed=r)
    y = c.gpu(qn)[0].cpu().numpy()
    assert rel_err(y, c.oracle_y(0)) <= LINEAR_TOL


def test_linear_no_norm_heavy_tail(qn):
    c = Case(16, [256], 5120, aqn=False, wdist="student", seed=9)
    y = c.gpu(qn)[0].cpu().numpy()
    assert rel_err(y, c.oracle_y(0)) <= LINEAR_TOL


def test_linear_lambda_zero_is_base(qn):
    c = Case(3, [64], 256, lam=0.0, seed=4)
    y = c.gpu(qn)[0].cpu().numpy()
    h = c.oracle_h()
    cc, sb, sg, _ = oracle.nvfp4_quantize(c.w[0])
    assert rel_err(y, oracle.lora_linear(h, cc, sb, sg, None, None, 0.0)) <= LINEAR_TOL


def test_linear_silu_mul_epilogue(qn):
    c = Case(16, [384, 384], 512, seed=5)
    ys = c.gpu(qn, epilogue=qn.EPI_SILU_MUL)
    ref = oracle.silu_mul(c.oracle_y(0), c.oracle_y(1))
    assert rel_err(ys[0].cpu().numpy(), ref) <= LINEAR_TOL


def test_linear_residual(qn):
    m, n, k = 8, 256, 256
    res = synth.normal_bf16(55, (m, n))
    c = Case(m, [n], k, seed=6)
    y = c.gpu(qn, residual=dev_bf16(res))[0].cpu().numpy()
    assert rel_err(y, c.oracle_y(0) + bf16_bits_to_f64(res)) <= LINEAR_TOL


def test_linear_bf16_output_is_rounded_f32(qn):
    """The bf16 output is the RNE rounding of the same kernel's f32 result (the kernel is deterministic)."""
    c = Case(16, [256], 1024, seed=7)
    y32 = c.gpu(qn, torch.float32)[0]
    y16 = c.gpu(qn, torch.bfloat16)[0]
    assert torch.equal(y16, y32.to(torch.bfloat16))


def test_linear_gqa_broadcast(qn):
    m, kv, hd, group, k = 4, 256, 128, 3, 384
    c = Case(m, [kv], k, seed=8)
    wq = qn.quantize(dev_bf16(c.w[0]), qn.LAYOUT_TILED)
    y = torch.full((m, kv * group), float("nan"), dtype=torch.float32, device=DEV)
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
    qn.lora_linear(dev_bf16(c.x), [qn.Projection(wq, y, dev_bf16(c.A[0]), dev_bf16(c.B[0]), c.lam, y_repeat=group,
                                                 head_dim=hd)], aqn)
    ref = oracle.gqa_broadcast(c.oracle_y(0), group, hd)
    assert rel_err(y.cpu().numpy(), ref) <= LINEAR_TOL


def test_linear_per_row_noise(qn):
    m, n, k = 5, 128, 256
    c = Case(m, [n], k, seed=10)
    noise = synth.normal_f32(77, (m, k))
    wq = qn.quantize(dev_bf16(c.w[0]), qn.LAYOUT_TILED)
    y = torch.empty(m, n, dtype=torch.float32, device=DEV)
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(noise), c.sigma, 1e-6, noise_per_row=True)
    qn.lora_linear(dev_bf16(c.x), [qn.Projection(wq, y, dev_bf16(c.A[0]), dev_bf16(c.B[0]), c.lam)], aqn)
    _, h = oracle.aqn_rmsnorm(c.x, c.gamma, noise, c.sigma, 1e-6, noise_per_row=True)
    cc, sb, sg, _ = oracle.nvfp4_quantize(c.w[0])
    assert rel_err(y.cpu().numpy(), oracle.lora_linear(h, cc, sb, sg, c.A[0], c.B[0], c.lam)) <= LINEAR_TOL


@pytest.mark.parametrize("m,k,per_row", [(16, 3584, False), (5, 272, True), (16, 2048, True), (1, 3968, False),
                                         (300, 1024, False), (17, 40960, True), (128, 9216, True),
                                         (128, 18944, False)])
def test_fused_norm_matches_standalone_norm(qn, m, k, per_row):
    """The norm inside the linear call gives the bits of the standalone norm: y(fused) == y(norm, then plain linear),
    both calls on the same kernel and cut (without the norm the library may split k, which changes the summation
    order of the product, not h).

    Covers the one-wave statistics in both thread counts (k > 32768 uses 1024), the fused decode kernel's statistics
    from registers in one and two rounds of 256 chunks, per-row noise, a ragged k, the separate statistics kernel
    taken from 256 tokens on, and a token tile's statistics split over four, two (128 x 9216: 72 workgroups per
    split) and one workgroup (128 x 18944: 152)."""
    c = Case(m, [96], k, seed=m + k)
    noise = synth.normal_f32(78, (m, k) if per_row else (k,))
    wq = qn.quantize(dev_bf16(c.w[0]), qn.LAYOUT_TILED)
    A, B = dev_bf16(c.A[0]), dev_bf16(c.B[0])
    g, z, x = dev_bf16(c.gamma), dev_f32(noise), dev_bf16(c.x)
    opts = qn.LinearOpts(kernel=qn.KERNEL_FUSED, decode_kchunks=1) if m <= 16 and k <= 3968 else None
    y1 = torch.empty(m, 96, dtype=torch.float32, device=DEV)
    qn.lora_linear(x, [qn.Projection(wq, y1, A, B, c.lam)], qn.make_aqn(g, z, c.sigma, 1e-6, noise_per_row=per_row),
                   opts=opts)
    h = qn.aqn_rmsnorm(x, g, z, c.sigma, 1e-6, noise_per_row=per_row)
    y2 = torch.empty(m, 96, dtype=torch.float32, device=DEV)
    qn.lora_linear(h, [qn.Projection(wq, y2, A, B, c.lam)], opts=opts)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# The two streaming kernels and the split-k form of the decode kernel, each named through the call's options, on the
# same cases: default choice, the general kernel, the decode kernel without and with a split k, and the decode kernel
# with two weight tiles in flight.
def kernel_paths(qn):
    return {"default": None, "general": qn.LinearOpts(kernel=qn.KERNEL_GENERAL),
            "decode": qn.LinearOpts(kernel=qn.KERNEL_DECODE, decode_kchunks=1),
            "decode-splitk": qn.LinearOpts(kernel=qn.KERNEL_DECODE, decode_kchunks=3),
            "decode-depth2": qn.LinearOpts(kernel=qn.KERNEL_DECODE, decode_depth=2),
            "fused": qn.LinearOpts(kernel=qn.KERNEL_FUSED),
            "fused-splitk": qn.LinearOpts(kernel=qn.KERNEL_FUSED, decode_kchunks=3)}


KERNEL_PATHS = ["default", "general", "decode", "decode-splitk", "decode-depth2", "fused", "fused-splitk"]


def decode_fits(m, nu, k, nchunks, nr):
    """Whether the decode kernel can take a call with a cut of `nchunks` k-chunks (0: any cut): the rule the library
    documents for QN_KERNEL_DECODE, restated from its limits (144 KiB of activations and LoRA slots in LDS, at most 8
    row units per workgroup, about 256 workgroups)."""
    if m > 32:
        return False
    tmt, KT = -(-m // 16), -(-k // 128)
    cap = (147456 - 8 * nr * tmt * 64 * 16) // (tmt * (4 * 64 * 16 + 64))
    for nk in ([nchunks] if nchunks else range(1, min(KT, 64) + 1)):
        tmax = -(-KT // nk)
        nbr = min(256 // nk, nu)
        if tmax <= cap and tmax * tmt <= 40 and nbr >= 1 and -(-nu // nbr) <= 8:
            return True
    return False


def fused_fits(m, nu, k, nchunks, nr, npairs, norm=True):
    """Whether the fused decode kernel can take a call: up to 16 tokens, a cut whose chunk fits in LDS under the LoRA
    slots or the 16 KiB LoRA-down reduction (whichever is larger), with the norm a single k-chunk, at most 8 row units
    per workgroup, and LoRA-down items (one per 4 k-tiles without a split, one per chunk with one) no more than the
    workgroups. For a cut the caller names (nchunks > 0) this is exact; with the library's own cut the test cases are
    ones where every feasible cut also has room for the items."""
    if m > 16 or (norm and nchunks > 1):
        return False
    KT = -(-k // 128)
    cap = (147456 - max(8 * nr * 64 * 16, 16384)) // (4 * 64 * 16 + 64)
    for nk in ([1] if norm else [nchunks] if nchunks else range(1, min(KT, 64) + 1)):
        tmax = -(-KT // nk)
        nbr = min(256 // nk, nu)
        if not (tmax <= cap and tmax <= 40 and nbr >= 1 and -(-nu // nbr) <= 8):
            continue
        if nk > 1 and npairs > nbr:
            continue
        return True
    return False


@pytest.mark.parametrize("path", KERNEL_PATHS)
@pytest.mark.parametrize("m,ns,k,silu,residual,r,gqa", [
    (1, [200], 1024, False, False, 32, 1),
    (16, [520, 64, 64], 1040, False, False, 64, 1),
    (17, [96], 3584, False, True, 12, 1),
    (32, [256], 512, False, True, 32, 1),
    (16, [384, 384], 512, True, False, 32, 1),
    (5, [1040, 1040], 384, True, False, 8, 1),
    (32, [128, 128], 1024, True, False, 0, 1),
    (9, [512, 128, 128], 640, False, False, 32, 4),
])
def test_linear_kernel_paths(qn, path, m, ns, k, silu, residual, r, gqa):
    opts = kernel_paths(qn)[path]
    c = Case(m, ns, k, r=r, seed=m * 7 + k)
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    res = synth.normal_bf16(56, (m, ns[0])) if residual else None
    ys, projs = [], []
    for p, n in enumerate(ns):
        rep = gqa if p == len(ns) - 1 and gqa > 1 else 1
        y = torch.full((m, n * rep), float("nan"), dtype=torch.float32, device=DEV)
        ys.append(y)
        A = dev_bf16(c.A[p]) if r else None
        B = dev_bf16(c.B[p]) if r else None
        projs.append(qn.Projection(wq[p], None if (silu and p == 1) else y, A, B, c.lam,
                                   residual=dev_bf16(res) if (residual and p == 0) else None,
                                   y_repeat=rep, head_dim=64))
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
    nu = -(-ns[0] // 16) if silu else sum(-(-n // 16) for n in ns)
    npairs = len(ns) * (-(-r // 32))
    if (path.startswith("decode") and not decode_fits(m, nu, k, opts.decode_kchunks, 2 if silu else 1)) or \
            (path.startswith("fused") and not fused_fits(m, nu, k, opts.decode_kchunks, 2 if silu else 1, npairs)):
        with pytest.raises(qn.QnError) as e:  # refused on the host, nothing launched
            qn.lora_linear(dev_bf16(c.x), projs, aqn, qn.EPI_SILU_MUL if silu else qn.EPI_NONE, opts=opts)
        assert e.value.status == qn.QN_ERR_UNSUPPORTED
        return
    qn.lora_linear(dev_bf16(c.x), projs, aqn, qn.EPI_SILU_MUL if silu else qn.EPI_NONE, opts=opts)
    torch.cuda.synchronize()
    if silu:
        ref = oracle.silu_mul(c.oracle_y(0), c.oracle_y(1))
        assert rel_err(ys[0].cpu().numpy(), ref) <= LINEAR_TOL
        return
    for p in range(len(ns)):
        ref = c.oracle_y(p)
        if residual and p == 0:
            ref = ref + bf16_bits_to_f64(res)
        rep = gqa if p == len(ns) - 1 and gqa > 1 else 1
        if rep > 1:
            ref = oracle.gqa_broadcast(ref, rep, 64)
        assert rel_err(ys[p].cpu().numpy(), ref) <= LINEAR_TOL, (path, p)


def wide_fits(m, nu, k, nchunks):
    """Whether the decode kernel for 17-64 tokens can take a call: the rule the library documents for
    QN_KERNEL_WIDE, restated from its limits (at most 5 row units per workgroup; with a split k at most 256 row
    blocks; a named cut of at most as many k-chunks as k-tiles)."""
    KT = -(-k // 128)
    if not 17 <= m <= 64 or nchunks > min(KT, 64):
        return False
    return -(-nu // 5) <= (256 if nchunks > 1 else 16384)


# The decode kernel for 17 to 64 tokens, named through the options, against the oracle on every output: one and
# several projections (with a GQA broadcast), SiLU * up, residuals, ranks none to 64 (odd ones too), ragged rows and
# k, long rows, split-k cuts named and the library's own, token counts at and between the tile boundaries.
@pytest.mark.parametrize("m,ns,k,silu,residual,r,gqa,nchunks", [
    (17, [96], 3584, False, True, 12, 1, 0),
    (24, [520, 64, 64], 1040, False, False, 64, 1, 0),
    (32, [256], 512, False, True, 32, 1, 2),
    (33, [384, 384], 512, True, False, 32, 1, 0),
    (48, [1040, 1040], 384, True, False, 8, 1, 0),
    (64, [128, 128], 1024, True, False, 0, 1, 0),
    (64, [512, 128, 128], 640, False, False, 32, 4, 0),
    (50, [200], 2048, False, True, 33, 1, 3),
    (64, [2048], 4736, False, True, 32, 1, 0),
    (64, [1024], 1040, False, False, 64, 1, 7),
    (40, [200, 200], 2176, True, True, 12, 1, 4),
    (20, [48], 128, False, False, 32, 1, 1),
    (64, [6000], 256, False, False, 32, 1, 2),
    (40, [21000], 256, False, True, 32, 1, 0),   # more than 256 row blocks: several rounds, no split
    (20, [21000], 256, False, False, 32, 1, 2),  # refused: a split needs a counter per block
])
def test_linear_wide_kernel(qn, m, ns, k, silu, residual, r, gqa, nchunks):
    opts = qn.LinearOpts(kernel=qn.KERNEL_WIDE, decode_kchunks=nchunks)
    c = Case(m, ns, k, r=r, seed=m * 11 + k)
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    res = synth.normal_bf16(57, (m, ns[0])) if residual else None
    ys, projs = [], []
    for p, n in enumerate(ns):
        rep = gqa if p == len(ns) - 1 and gqa > 1 else 1
        y = torch.full((m, n * rep), float("nan"), dtype=torch.float32, device=DEV)
        ys.append(y)
        A = dev_bf16(c.A[p]) if r else None
        B = dev_bf16(c.B[p]) if r else None
        projs.append(qn.Projection(wq[p], None if (silu and p == 1) else y, A, B, c.lam,
                                   residual=dev_bf16(res) if (residual and p == 0) else None,
                                   y_repeat=rep, head_dim=64))
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
    nu = -(-ns[0] // 16) if silu else sum(-(-n // 16) for n in ns)
    if not wide_fits(m, nu, k, nchunks):
        with pytest.raises(qn.QnError) as e:  # refused on the host, nothing launched
            qn.lora_linear(dev_bf16(c.x), projs, aqn, qn.EPI_SILU_MUL if silu else qn.EPI_NONE, opts=opts)
        assert e.value.status == qn.QN_ERR_UNSUPPORTED
        return
    qn.lora_linear(dev_bf16(c.x), projs, aqn, qn.EPI_SILU_MUL if silu else qn.EPI_NONE, opts=opts)
    torch.cuda.synchronize()
    if silu:
        ref = oracle.silu_mul(c.oracle_y(0), c.oracle_y(1))
        if residual:
            ref = ref + bf16_bits_to_f64(res)
        got = ys[0].cpu().numpy()
        assert np.all(np.isfinite(got))
        assert rel_err(got, ref) <= LINEAR_TOL
        return
    for p in range(len(ns)):
        ref = c.oracle_y(p)
        if residual and p == 0:
            ref = ref + bf16_bits_to_f64(res)
        rep = gqa if p == len(ns) - 1 and gqa > 1 else 1
        if rep > 1:
            ref = oracle.gqa_broadcast(ref, rep, 64)
        got = ys[p].cpu().numpy()
        assert np.all(np.isfinite(got)), p
        assert rel_err(got, ref) <= LINEAR_TOL, p


def test_linear_wide_kernel_refusals(qn):
    """Calls the kernel for 17-64 tokens cannot take are refused on the host: 16 or 65 tokens, a cut of more
    k-chunks than k-tiles, depth 2."""
    c = Case(16, [64], 256, seed=1)
    wq = qn.quantize(dev_bf16(c.w[0]), qn.LAYOUT_TILED)
    for m, opts in ((16, qn.LinearOpts(kernel=qn.KERNEL_WIDE)), (65, qn.LinearOpts(kernel=qn.KERNEL_WIDE)),
                    (32, qn.LinearOpts(kernel=qn.KERNEL_WIDE, decode_kchunks=3)),
                    (32, qn.LinearOpts(kernel=qn.KERNEL_WIDE, decode_depth=2))):
        x = torch.zeros(m, 256, dtype=torch.bfloat16, device=DEV)
        y = torch.empty(m, 64, dtype=torch.float32, device=DEV)
        with pytest.raises(qn.QnError) as e:
            qn.lora_linear(x, [qn.Projection(wq, y)], opts=opts)
        assert e.value.status == qn.QN_ERR_UNSUPPORTED, (m, opts)


def test_shared_workspace_calls_of_other_shapes(qn):
    """One workspace shared by calls of different shapes, in turn: the kernel for 17-64 tokens (SiLU pair, and long
    rows with a split k), the fused decode kernel and the decode kernel. Each call's data regions lie at offsets of
    their own, so the words that must stay zero between calls (arrival counters, the fused kernel's ready flags) have
    to sit where no call writes data. Regression: with those words placed after the data, a long-row call's
    activations landed on another call's LoRA-down arrival counters, and its next call read a t never summed (NaN)."""
    ws = qn.Workspace(DEV)
    cases = [(Case(40, [512, 512], 512, seed=5), qn.EPI_SILU_MUL, qn.LinearOpts(kernel=qn.KERNEL_WIDE)),
             (Case(40, [256], 6144, seed=6), qn.EPI_NONE, qn.LinearOpts(kernel=qn.KERNEL_WIDE, decode_kchunks=4)),
             (Case(8, [256], 512, seed=7), qn.EPI_NONE, qn.LinearOpts(kernel=qn.KERNEL_FUSED)),
             (Case(16, [384], 3072, seed=8), qn.EPI_NONE, qn.LinearOpts(kernel=qn.KERNEL_DECODE, decode_kchunks=3))]
    calls = []
    for c, epi, opts in cases:
        wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
        ys = [torch.full((c.m, n), float("nan"), dtype=torch.float32, device=DEV) for n in c.ns]
        projs = [qn.Projection(wq[p], None if (epi == qn.EPI_SILU_MUL and p == 1) else ys[p], dev_bf16(c.A[p]),
                               dev_bf16(c.B[p]), c.lam) for p in range(len(c.ns))]
        aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
        ref = oracle.silu_mul(c.oracle_y(0), c.oracle_y(1)) if epi == qn.EPI_SILU_MUL else c.oracle_y(0)
        calls.append((qn.LinearCall(dev_bf16(c.x), projs, aqn, epi, ws, opts), ys[0], ref))
    for rep in range(3):
        for i, (call, y, ref) in enumerate(calls):
            y.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            assert np.all(np.isfinite(got)), (rep, i)
            assert rel_err(got, ref) <= LINEAR_TOL, (rep, i)


# The fused decode kernel without the norm (the o and down projections of a layer): its split-k form, which the calls
# with the norm never take, on rows too long for one chunk and on cuts named through the options, with residuals,
# several projections, mixed and odd ranks; every output checked against the oracle.
@pytest.mark.parametrize("m,ns,k,r,nchunks,residual", [
    (16, [520], 4992, 32, 0, True),      # 39 k-tiles: more than one chunk holds
    (1, [3584], 18944, 32, 0, True),     # the 7B down projection's row length
    (7, [200, 72], 2048, 12, 3, False),
    (16, [1040, 64, 64], 1040, 64, 2, False),
    (3, [96], 640, 0, 4, True),
    (16, [384], 3584, 33, 5, False),
])
def test_fused_split_k_without_norm(qn, m, ns, k, r, nchunks, residual):
    c = Case(m, ns, k, r=r, seed=k + m, aqn=False)
    res = synth.normal_bf16(57, (m, ns[0])) if residual else None
    opts = qn.LinearOpts(kernel=qn.KERNEL_FUSED, decode_kchunks=nchunks)
    nu = sum(-(-n // 16) for n in ns)
    npairs = len(ns) * (-(-r // 32))
    if not fused_fits(m, nu, k, nchunks, 1, npairs, norm=False):
        pytest.skip("cut outside the fused kernel's limits")
    ys = c.gpu(qn, residual=dev_bf16(res) if residual else None, opts=opts)
    for p in range(len(ns)):
        ref = c.oracle_y(p)
        if residual:
            ref = ref + bf16_bits_to_f64(res)
        assert rel_err(ys[p].cpu().numpy(), ref) <= LINEAR_TOL, p


# Many tokens (more than 128): the MFMA kernel with one activation exponent per token, and the general kernel in
# 128-token launches (named through the options), on shapes that leave ragged token blocks, ragged row blocks and
# mixed ranks.
def many_paths(qn):
    return {"mfma": None, "mfma-elem-store": qn.LinearOpts(kernel=qn.KERNEL_MANY, elem_store=1),
            "general": qn.LinearOpts(kernel=qn.KERNEL_GENERAL)}


@pytest.mark.parametrize("path", ["mfma", "mfma-elem-store", "general"])
@pytest.mark.parametrize("m,ns,k,silu,residual,r,gqa,aqn", [
    (129, [200], 1024, False, False, 32, 1, True),
    (300, [384, 384], 512, True, False, 8, 1, True),
    (257, [520, 64, 64], 1040, False, False, 64, 4, True),
    (200, [96], 3584, False, True, 12, 1, False),
    (513, [272, 272], 640, True, False, 0, 1, True),
    (1000, [48], 256, False, False, 33, 1, True),
    (150, [256, 256, 72], 256, False, True, 16, 1, True),
    (160, [200, 72, 40], 512, False, False, 16, 1, False),
])
def test_linear_many_tokens(qn, path, m, ns, k, silu, residual, r, gqa, aqn):
    opts = many_paths(qn)[path]
    c = Case(m, ns, k, r=r, seed=m * 5 + k, aqn=aqn)
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    res = synth.normal_bf16(57, (m, ns[0])) if residual else None
    ys, projs = [], []
    for p, n in enumerate(ns):
        rep = gqa if p == len(ns) - 1 and gqa > 1 else 1
        y = torch.full((m, n * rep), float("nan"), dtype=torch.float32, device=DEV)
        ys.append(y)
        A = dev_bf16(c.A[p]) if r else None
        B = dev_bf16(c.B[p]) if r else None
        projs.append(qn.Projection(wq[p], None if (silu and p == 1) else y, A, B, c.lam,
                                   residual=dev_bf16(res) if (residual and p == 0) else None,
                                   y_repeat=rep, head_dim=16))
    norm = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6) if aqn else None
    qn.lora_linear(dev_bf16(c.x), projs, norm, qn.EPI_SILU_MUL if silu else qn.EPI_NONE, opts=opts)
    torch.cuda.synchronize()
    if silu:
        ref = oracle.silu_mul(c.oracle_y(0), c.oracle_y(1))
        assert rel_err(ys[0].cpu().numpy(), ref) <= LINEAR_TOL
        return
    for p in range(len(ns)):
        ref = c.oracle_y(p)
        if residual and p == 0:
            ref = ref + bf16_bits_to_f64(res)
        rep = gqa if p == len(ns) - 1 and gqa > 1 else 1
        if rep > 1:
            ref = oracle.gqa_broadcast(ref, rep, 16)
        assert rel_err(ys[p].cpu().numpy(), ref) <= LINEAR_TOL, (path, p)


@pytest.mark.parametrize("m,ns,k,silu,residual", [
    (300, [512, 512], 640, True, False),
    (200, [520], 1024, False, True),
    (129, [256, 256], 384, False, True),
])
def test_linear_many_tokens_bf16_store_paths(qn, m, ns, k, silu, residual):
    """Many tokens with bf16 outputs: the 16-byte stores through the LDS tile and the per-element stores give the
    same bits (same f32 values, residual added before the one rounding), and both meet the bar against the oracle
    with one bf16 rounding on top (ragged row blocks and token blocks included)."""
    c = Case(m, ns, k, r=16, seed=m + 3 * k, aqn=True)
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    res = synth.normal_bf16(91, (m, ns[0])) if residual else None
    outs = {}
    for store in ("fast", "elem"):
        opts = qn.LinearOpts(elem_store=1) if store == "elem" else None
        ys, projs = [], []
        for p, n in enumerate(ns):
            y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
            ys.append(y)
            projs.append(qn.Projection(wq[p], None if (silu and p == 1) else y, dev_bf16(c.A[p]), dev_bf16(c.B[p]),
                                       c.lam, residual=dev_bf16(res) if (residual and p == 0) else None))
        qn.lora_linear(dev_bf16(c.x), projs, qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6),
                       qn.EPI_SILU_MUL if silu else qn.EPI_NONE, opts=opts)
        torch.cuda.synchronize()
        outs[store] = [host_bf16(y) for y in (ys[:1] if silu else ys)]
    for a, b in zip(outs["fast"], outs["elem"]):
        assert np.array_equal(a, b)
    refs = [oracle.silu_mul(c.oracle_y(0), c.oracle_y(1))] if silu else [c.oracle_y(p) for p in range(len(ns))]
    if residual:
        refs[0] = refs[0] + bf16_bits_to_f64(res)
    for got, ref in zip(outs["fast"], refs):
        g = bf16_bits_to_f64(got)
        assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + LINEAR_TOL * np.abs(ref).max())


@pytest.mark.parametrize("m,n,k", [(200, 520, 640), (129, 256, 384)])
def test_linear_many_tokens_residual_aliases_output(qn, m, n, k):
    """Many tokens, bf16 output with the residual read from the output buffer itself (the one aliasing the API
    allows): the same bits as with a separate residual buffer, on both store paths."""
    c = Case(m, [n], k, r=16, seed=m + k, aqn=True)
    wq = qn.quantize(dev_bf16(c.w[0]), qn.LAYOUT_TILED)
    res = synth.normal_bf16(93, (m, n))
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
    for store in ("fast", "elem"):
        opts = qn.LinearOpts(elem_store=1) if store == "elem" else None
        y_sep = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
        qn.lora_linear(dev_bf16(c.x), [qn.Projection(wq, y_sep, dev_bf16(c.A[0]), dev_bf16(c.B[0]), c.lam,
                                                     residual=dev_bf16(res))], aqn, opts=opts)
        y_alias = dev_bf16(res)
        qn.lora_linear(dev_bf16(c.x), [qn.Projection(wq, y_alias, dev_bf16(c.A[0]), dev_bf16(c.B[0]), c.lam,
                                                     residual=y_alias)], aqn, opts=opts)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16(y_sep), host_bf16(y_alias)), store


def test_linear_many_tokens_row_scales(qn):
    """One exponent per token: rows whose magnitudes differ by 2^40 across the batch, and a row of zeros, keep their
    own relative accuracy (each token is checked against its own scale)."""
    m, n, k = 200, 128, 512
    c = Case(m, [n], k, r=16, seed=5, aqn=False)
    scale = 2.0 ** np.linspace(-20, 20, m)
    xs = (c.x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * scale[:, None]
    xs[17] = 0.0
    c.x = oracle.bf16_round_array(xs)  # power-of-two scaling of bf16 values: exact
    y = c.gpu(qn)[0].cpu().numpy()
    ref = c.oracle_y(0)
    for t in range(m):
        if t == 17:
            assert np.all(y[t] == ref[t])
            continue
        assert np.abs(y[t] - ref[t]).max() <= LINEAR_TOL * np.abs(ref[t]).max(), t


@pytest.mark.parametrize("m,n,k,kernel", [(16, 512, 2048, "AUTO"), (8, 128, 256, "FUSED"), (16, 96, 256, "GENERAL"),
                                          (40, 256, 1024, "WIDE"), (300, 256, 512, "AUTO")])
def test_linear_main_kernel_events(qn, m, n, k, kernel):
    """A call whose main kernel records the caller's event pair (qn_linear_opts main_begin / main_end, a launch
    through hipExtLaunchKernel, for timing) gives the same bits as the same call without it, on the decode, fused,
    general, 17-64-token and many-token kernels, and the pair spans a positive time."""
    c = Case(m, [n], k, seed=13)
    kid = getattr(qn, "KERNEL_" + kernel)
    ref = c.gpu(qn, opts=qn.LinearOpts(kernel=kid))[0].clone()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()  # each event exists before the launch records it
    got = c.gpu(qn, opts=qn.LinearOpts(kernel=kid, main_events=ev))[0]
    assert torch.equal(ref, got)
    assert ev[0].elapsed_time(ev[1]) > 0.0


def test_linear_deterministic(qn):
    c = Case(16, [512], 2048, seed=11)
    a = c.gpu(qn)[0].clone()
    b = c.gpu(qn)[0]
    assert torch.equal(a, b)


def test_aqn_rmsnorm_parity(qn):
    m, d = 16, 3584
    x = synth.normal_bf16(61, (m, d))
    gamma = synth.normal_bf16(62, (d,), std=1.0)
    noise = synth.normal_f32(63, (d,))
    sigma = float(np.float32(oracle.aqn_sigma(3)))
    h = host_bf16(qn.aqn_rmsnorm(dev_bf16(x), dev_bf16(gamma), dev_f32(noise), sigma, 1e-6))
    he, hb = oracle.aqn_rmsnorm(x, gamma, noise, sigma, 1e-6)
    hv = bf16_bits_to_f64(h)
    # f32 arithmetic then one bf16 rounding: within one bf16 ulp (2^-7 relative) of the exact value, and equal to
    # the oracle's rounding except where the exact value sits within f32 error of a rounding boundary
    assert np.all(np.abs(hv - he) <= 2.0 ** -7 * np.abs(he) + 1e-30)
    assert np.mean(h == hb) > 0.999
    # sigma = 0 is plain RMSNorm
    h0 = host_bf16(qn.aqn_rmsnorm(dev_bf16(x), dev_bf16(gamma), None, 0.0, 1e-6))
    he0, _ = oracle.aqn_rmsnorm(x, gamma, None, 0.0, 1e-6)
    assert np.all(np.abs(bf16_bits_to_f64(h0) - he0) <= 2.0 ** -7 * np.abs(he0) + 1e-30)


def test_empty_batch(qn):
    c = Case(1, [64], 128, seed=12)
    wq = qn.quantize(dev_bf16(c.w[0]), qn.LAYOUT_TILED)
    y = torch.empty(0, 64, dtype=torch.float32, device=DEV)
    x = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    qn.lora_linear(x, [qn.Projection(wq, y)])
    torch.cuda.synchronize()


# ---- full-size shapes, sampled outputs ------------------------------------------------------------------------------
def sampled_rows(n, count=96, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, count)]))
    return rows


@pytest.mark.parametrize("m,n,k,aqn", [
    (1, 4096, 4096, True),       # single 4096 x 4096 projection, one token
    (16, 18944, 3584, True),     # 7B gate shape at decode batch 16
    (8, 3584, 18944, False),     # 7B down shape
    (32, 5120, 5120, True),      # 32B q/o shape at batch 32
    (128, 1024, 5120, True),     # 32B k/v shape at batch 128
])
def test_linear_full_size_sampled(qn, m, n, k, aqn):
    c = Case(m, [n], k, seed=n % 97, aqn=aqn)
    y = c.gpu(qn)[0].cpu().numpy()
    rows = sampled_rows(n)
    ref = c.oracle_y(0, rows)
    assert rel_err(y[:, rows], ref) <= LINEAR_TOL


# 32B-shaped projections (config 4) at decode batch 32 (decode kernel) and 128 (general kernel), heavy-tailed
# weights whose 16-blocks carry exponents 2^e, e in -14..0: sampled output rows against the oracle.
@pytest.mark.parametrize("m", [32, 128])
def test_32b_gate_up_full_size_sampled(qn, m):
    n, k = 27648, 5120
    c = Case(m, [n, n], k, seed=32, r=32, wdist="t4")
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    projs = [qn.Projection(wq[0], y, dev_bf16(c.A[0]), dev_bf16(c.B[0]), c.lam),
             qn.Projection(wq[1], None, dev_bf16(c.A[1]), dev_bf16(c.B[1]), c.lam)]
    qn.lora_linear(dev_bf16(c.x), projs, qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6),
                   qn.EPI_SILU_MUL)
    torch.cuda.synchronize()
    rows = sampled_rows(n, 48)
    ref = oracle.silu_mul(c.oracle_y(0, rows), c.oracle_y(1, rows))
    assert rel_err(y.cpu().numpy()[:, rows], ref) <= LINEAR_TOL


@pytest.mark.parametrize("m", [32, 128])
def test_32b_down_full_size_sampled(qn, m):
    n, k = 5120, 27648
    c = Case(m, [n], k, seed=33, r=32, wdist="t4", aqn=False)
    res = synth.normal_bf16(34, (m, n))
    y = c.gpu(qn, residual=dev_bf16(res))[0].cpu().numpy()
    rows = sampled_rows(n, 48)
    ref = c.oracle_y(0, rows) + bf16_bits_to_f64(res)[:, rows]
    assert rel_err(y[:, rows], ref) <= LINEAR_TOL


def test_32b_qkv_gqa_full_size_sampled(qn):
    """32B q|k|v (5,120 + 1,024 + 1,024 rows) sharing one AQN-RMSNorm at batch 128, v broadcast to its 5 query
    heads per kv head (head_dim 128)."""
    m, k = 128, 5120
    ns = [5120, 1024, 1024]
    c = Case(m, ns, k, seed=35, r=32, wdist="t4")
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    ys = [torch.full((m, n * (5 if p == 2 else 1)), float("nan"), dtype=torch.float32, device=DEV)
          for p, n in enumerate(ns)]
    projs = [qn.Projection(wq[p], ys[p], dev_bf16(c.A[p]), dev_bf16(c.B[p]), c.lam,
                           y_repeat=5 if p == 2 else 1, head_dim=128) for p in range(3)]
    qn.lora_linear(dev_bf16(c.x), projs, qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6))
    torch.cuda.synchronize()
    for p, n in enumerate(ns):
        rows = sampled_rows(n, 32)
        ref = c.oracle_y(p, rows)
        got = ys[p].cpu().numpy()
        if p == 2:  # every copy of a sampled v row: head h's copies sit at (h*5 + g)*128 + row % 128
            for g in range(5):
                cols = (rows // 128 * 5 + g) * 128 + rows % 128
                assert rel_err(got[:, cols], ref) <= LINEAR_TOL, g
        else:
            assert rel_err(got[:, rows], ref) <= LINEAR_TOL, p


def test_prefill_gate_up_full_size_sampled(qn):
    """7B gate/up at 8192 prefill tokens through the MFMA kernel with the SiLU product, rank-32 LoRA: sampled rows."""
    m, n, k = 8192, 18944, 3584
    c = Case(m, [n, n], k, seed=8192, r=32)
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    projs = [qn.Projection(wq[0], y, dev_bf16(c.A[0]), dev_bf16(c.B[0]), c.lam),
             qn.Projection(wq[1], None, dev_bf16(c.A[1]), dev_bf16(c.B[1]), c.lam)]
    qn.lora_linear(dev_bf16(c.x), projs, qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6),
                   qn.EPI_SILU_MUL)
    torch.cuda.synchronize()
    rows = sampled_rows(n, 48)
    got = bf16_bits_to_f64(host_bf16(y))[:, rows]
    ref = oracle.silu_mul(c.oracle_y(0, rows), c.oracle_y(1, rows))
    # bf16 output: one rounding (2^-8 relative) on top of the linear bar
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + LINEAR_TOL * np.abs(ref).max())


# ---- decoder layer ---------------------------------------------------------------------------------------------------
def make_layer_inputs(shape, m, seed, sigma):
    s = lambda t: synth.seed_for(2, seed, t)
    w = {nm: synth.normal_bf16(s("w_" + nm), nk, std=0.02) for nm, nk in shape.projections().items()}
    lora = {nm: (synth.normal_bf16(s("a_" + nm), (shape.rank, nk[1]), std=0.02),
                 synth.normal_bf16(s("b_" + nm), (nk[0], shape.rank), std=0.02)) for nm, nk in shape.projections().items()}
    x = synth.normal_bf16(s("x"), (m, shape.hidden))
    g1 = synth.bf16_const(1.0, (shape.hidden,))
    g2 = synth.bf16_const(1.0, (shape.hidden,))
    e1 = synth.normal_f32(s("eps_norm1"), (shape.hidden,))
    e2 = synth.normal_f32(s("eps_norm2"), (shape.hidden,))
    return w, lora, x, g1, g2, e1, e2, float(np.float32(sigma))


def bf16_chain_ok(got, ref):
    """A bf16 result of a chain with bf16 storage between ops: within two bf16 ulps (a rounding decision may flip
    at each of the two last storage points) plus the linear bar, and tight (within the linear bar) almost
    everywhere."""
    g = bf16_bits_to_f64(got)
    r = bf16_bits_to_f64(ref)
    scale = np.abs(r).max()
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    err = np.abs(g - r)
    return bool(np.all(err <= 2 * ulp + LINEAR_TOL * scale)) and float(np.mean(err <= LINEAR_TOL * scale)) > 0.99


@pytest.mark.parametrize("m", [1, 8, 16])
def test_decoder_layer_small(qn, m):
    from nvfp4_weight_only_amd.layer import DecoderLayer, LayerShape
    shape = LayerShape(hidden=512, q_dim=512, kv_dim=128, inter=1024, head_dim=128, rank=32)
    w, lora, x, g1, g2, e1, e2, sigma = make_layer_inputs(shape, m, 1, 1e-2)
    layer = DecoderLayer.from_bf16(shape, {k: dev_bf16(v) for k, v in w.items()},
                                   {k: (dev_bf16(a), dev_bf16(b)) for k, (a, b) in lora.items()},
                                   dev_bf16(g1), dev_bf16(g2), dev_f32(e1), dev_f32(e2), sigma, 2.0)
    bound = layer.bind(dev_bf16(x))
    bound()
    torch.cuda.synchronize()
    qref = {k: oracle.nvfp4_quantize(v)[:3] for k, v in w.items()}
    ref = oracle.decoder_layer(x, qref, lora, g1, g2, e1, e2, sigma, 2.0, shape.group, shape.head_dim)
    for name in ("q", "k", "attn", "x2", "a", "out"):
        got = host_bf16(getattr(bound, name))
        assert bf16_chain_ok(got, ref[name]), name


def test_decoder_chain_28_layers_m64(qn):
    """28 Qwen2.5-7B-shaped layers chained at M = 64 with sigma_3 = 0.01 * 0.05^(1/4) in all 56 norms, a fresh noise
    vector per norm, two weight sets alternating (layer l uses set l % 2). The chain runs on the GPU end to end; the
    last layer is then checked op by op, each op fed the bf16 tensors the GPU consumed (teacher forcing), on sampled
    output columns: q, k, v (all seven broadcast copies), o + residual, SiLU(gate) * up, down + residual."""
    from nvfp4_weight_only_amd.layer import QWEN25_7B, DecoderLayer
    shape, m, nl = QWEN25_7B, 64, 28
    sigma = float(np.float32(oracle.aqn_sigma(3)))
    assert abs(sigma - 4.728708e-3) < 1e-9
    sets = []
    for ws in range(2):
        w, lora, _, g1, g2, _, _, _ = make_layer_inputs(shape, 1, 40 + ws, sigma)
        layer = DecoderLayer.from_bf16(shape, {k: dev_bf16(v) for k, v in w.items()},
                                       {k: (dev_bf16(a), dev_bf16(b)) for k, (a, b) in lora.items()},
                                       dev_bf16(g1), dev_bf16(g2), None, None, sigma, 2.0)
        sets.append((w if ws == (nl - 1) % 2 else None, lora, layer))
    noise = [[synth.normal_f32(synth.seed_for(3, l, t), (shape.hidden,)) for t in ("eps_norm1", "eps_norm2")]
             for l in range(nl)]
    x0 = synth.normal_bf16(synth.seed_for(3, 0, "x"), (m, shape.hidden))
    ws_buf = qn.Workspace(DEV)
    bound, x = [], dev_bf16(x0)
    for l in range(nl):
        base = sets[l % 2][2]
        layer = DecoderLayer(shape, base.w, base.lora, base.gamma1, base.gamma2, dev_f32(noise[l][0]),
                             dev_f32(noise[l][1]), sigma, 2.0)
        b = layer.bind(x, ws_buf)
        bound.append(b)
        x = b.out
    for b in bound:
        b()
    torch.cuda.synchronize()
    last = bound[-1]
    w, lora, base = sets[(nl - 1) % 2]
    g = {name: host_bf16(getattr(last, name)) for name in ("x", "attn", "x2", "a", "out", "q", "k")}
    assert np.all(np.isfinite(bf16_bits_to_f64(g["out"])))
    gamma1, gamma2 = host_bf16(base.gamma1), host_bf16(base.gamma2)

    def lin(h, name, rows):
        c, sb, sg, _ = oracle.nvfp4_quantize_rows(w[name], rows)
        A, B = lora[name]
        return oracle.lora_linear(h, c, sb, sg, A, B[rows], 2.0)

    def check(got, ref):  # bf16 outputs: one rounding on top of the linear bar
        gf = bf16_bits_to_f64(got)
        assert np.all(np.abs(gf - ref) <= 2.0 ** -8 * np.abs(ref) + LINEAR_TOL * np.abs(ref).max())

    h1 = oracle.aqn_rmsnorm(g["x"], gamma1, noise[nl - 1][0], sigma, 1e-6)[1]
    for name, key in (("q", "q"), ("k", "k")):
        rows = sampled_rows(w[name].shape[0], 32)
        check(g[key][:, rows], lin(h1, name, rows))
    rows = sampled_rows(shape.kv_dim, 32)
    vref = lin(h1, "v", rows)
    for gi in range(shape.group):
        check(g["attn"][:, (rows // 128 * shape.group + gi) * 128 + rows % 128], vref)
    rows = sampled_rows(shape.hidden, 32)
    check(g["x2"][:, rows], lin(g["attn"], "o", rows) + bf16_bits_to_f64(g["x"])[:, rows])
    h2 = oracle.aqn_rmsnorm(g["x2"], gamma2, noise[nl - 1][1], sigma, 1e-6)[1]
    rows = sampled_rows(shape.inter, 32)
    check(g["a"][:, rows], oracle.silu_mul(lin(h2, "gate", rows), lin(h2, "up", rows)))
    rows = sampled_rows(shape.hidden, 32)
    check(g["out"][:, rows], lin(g["a"], "down", rows) + bf16_bits_to_f64(g["x2"])[:, rows])
