"""GPU parity of the NVFP4 quantizer / packer and reconstruction: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, dev_bf16, host_u8

pytestmark = pytest.mark.gpu


def gpu_quantize_rowmajor(qn, w_np, scale_mode=0, s_b=None, s_g=None, flags=None):
    n, k = w_np.shape
    out = qn.alloc_weight(n, k, qn.LAYOUT_ROWMAJOR, DEV)
    if scale_mode == 1:
        out.scales.copy_(torch.from_numpy(np.ascontiguousarray(s_b).reshape(-1)).to(DEV))
        out.tensor_scale.fill_(float(s_g))
    qn.quantize(dev_bf16(w_np), qn.LAYOUT_ROWMAJOR, scale_mode, out, flags)
    torch.cuda.synchronize()
    return (host_u8(out.codes)[: n * k // 2].reshape(n, k // 2), host_u8(out.scales)[: n * k // 16].reshape(n, k // 16),
            float(out.tensor_scale.item()))


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


@pytest.mark.parametrize("n,k,seed", [(64, 256, 1), (40, 272, 2), (17, 16, 3), (96, 3584, 4), (512, 4096, 5)])
def test_quantize_bitexact(qn, n, k, seed):
    w = synth.normal_bf16(seed, (n, k), std=0.02)
    c, s, g = gpu_quantize_rowmajor(qn, w)
    oc, os_, og, _ = oracle.nvfp4_quantize(w)
    assert g == og
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc)


def test_quantize_heavy_tail_block_exponents(qn):
    """Student-t(4) weights with per-block 2^e scaling (e in -16..0): block scales in every E4M3 binade, normal and
    subnormal, and blocks that underflow to scale 0."""
    n, k = 128, 5120
    w = synth.student_t4_bf16(41, (n, k), 0.02, block=16, exp_seed=42, emin=-16)
    c, s, g = gpu_quantize_rowmajor(qn, w)
    oc, os_, og, _ = oracle.nvfp4_quantize(w)
    assert g == og and np.array_equal(s, os_) and np.array_equal(c, oc)
    assert (os_ == 0).any() and ((os_ & 0x78) == 0).any() and (os_ == 0x7E).any()


def test_quantize_exhaustive_fixed_scales(qn):
    """All 65,536 bf16 patterns x all 126 positive finite E4M3 scales, s_g = 1 (scale_mode 1)."""
    w = np.tile(np.arange(65536, dtype=np.uint16), (126, 1))
    s_b = np.repeat(np.arange(1, 127, dtype=np.uint8)[:, None], 65536 // 16, axis=1)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    c, _, _ = gpu_quantize_rowmajor(qn, w, 1, s_b, 1.0, flags)
    oc, _, _, ofl = oracle.nvfp4_quantize(w, 1, s_b, 1.0)
    assert np.array_equal(c, oc)
    assert int(flags.item()) == ofl == 1


@pytest.mark.parametrize("s_g", [1.0, float(np.float32(7.77e-3)), float(np.float32(1.3e-36)), float(np.float32(1.5e30))])
def test_quantize_fixed_tensor_scale(qn, s_g):
    n, k = 64, 512
    w = synth.normal_bf16(77, (n, k), std=0.3)
    rng = np.random.default_rng(3)
    s_b = rng.integers(0, 127, size=(n, k // 16)).astype(np.uint8)
    c, _, _ = gpu_quantize_rowmajor(qn, w, 1, s_b, s_g)
    oc, _, _, _ = oracle.nvfp4_quantize(w, 1, s_b, s_g)
    assert np.array_equal(c, oc)


def test_nonfinite_and_zero(qn):
    n, k = 32, 64
    w = synth.normal_bf16(5, (n, k), std=0.02)
    w[3, 5] = 0x7F80   # +inf
    w[7, 9] = 0xFFC1   # NaN
    w[1, :16] = 0      # an all-zero block
    w[2, 0] = 0x8000   # -0
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    c, s, g = gpu_quantize_rowmajor(qn, w, flags=flags)
    oc, os_, og, ofl = oracle.nvfp4_quantize(w)
    assert int(flags.item()) == ofl == 1
    assert g == og and np.array_equal(s, os_) and np.array_equal(c, oc)
    z, _, zg = gpu_quantize_rowmajor(qn, np.zeros((16, 32), np.uint16))
    assert zg == 1.0 and not z.any()


@pytest.mark.parametrize("n,k", [(64, 256), (40, 272), (33, 3584), (16, 128)])
def test_tiled_dequant_matches_oracle(qn, n, k):
    w = synth.normal_bf16(n * 7 + k, (n, k), std=0.02)
    wq = qn.quantize(dev_bf16(w), qn.LAYOUT_TILED)
    got = qn.dequantize(wq).cpu().numpy()
    oc, os_, og, _ = oracle.nvfp4_quantize(w)
    _, wf = oracle.nvfp4_dequantize(oc, os_, og)
    assert np.array_equal(got.view(np.uint32), wf.view(np.uint32))
    assert float(wq.tensor_scale.item()) == og
    cb, sb = qn.tiled_bytes(n, k)
    assert wq.codes.numel() == cb and wq.scales.numel() == sb


def test_dequant_exhaustive_codes_scales(qn):
    """16 codes x 127 scales (0 included) x several tensor scales, row-major and tiled, bit-exact."""
    k = 256
    q = np.tile(np.arange(16, dtype=np.uint8), k // 16)
    codes = np.repeat((q[0::2] | (q[1::2] << 4))[None, :], 127, axis=0)
    s_b = np.repeat(np.arange(127, dtype=np.uint8)[:, None], k // 16, axis=1)
    for s_g in [1.0, float(np.float32(3.0517578125e-05)), float(np.float32(0.1234567)), float(np.float32(1e-38))]:
        wq = qn.NVFP4Weight(torch.from_numpy(codes.reshape(-1)).to(DEV), torch.from_numpy(s_b.reshape(-1)).to(DEV),
                            torch.tensor([s_g], dtype=torch.float32, device=DEV), 127, k, qn.LAYOUT_ROWMAJOR)
        got = qn.dequantize(wq).cpu().numpy()
        _, wf = oracle.nvfp4_dequantize(codes, s_b, s_g)
        assert np.array_equal(got.view(np.uint32), wf.view(np.uint32)), s_g


def test_quantize_is_deterministic(qn):
    w = dev_bf16(synth.normal_bf16(9, (256, 1024), std=0.02))
    a = qn.quantize(w)
    b = qn.quantize(w)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert torch.equal(a.tensor_scale, b.tensor_scale)


def test_group_advantage(qn):
    R = synth.bernoulli_f32(synth.seed_for(5, 0, "rewards"), (8, 8), 0.3)
    R[0] = [1, 0, 0, 0, 0, 0, 0, 0]
    R[1] = 0.0
    got = qn.group_advantage(torch.from_numpy(R).to(DEV), 1e-6).cpu().numpy()
    ref = oracle.group_advantage(R, 1e-6)
    assert np.allclose(got, ref, rtol=2 ** -23, atol=1e-7)
    assert np.all(got[1] == 0)
