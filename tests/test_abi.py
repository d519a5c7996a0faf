"""The C-ABI library loads, exports every entry point the header declares, and validates arguments on the host
(these calls return before anything touches a GPU)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qerl_nvfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("nvfp4_quantize", "nvfp4_lora_linear", "aqn_rmsnorm"):
        assert f in names


def test_library_exports_every_declared_symbol(qn):
    lib = ctypes.CDLL(qn.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(qn.EXPORTS) == declared_functions()


def test_validation_errors(qn):
    L = qn.lib
    P = ctypes.c_void_p
    fake = P(256)  # never dereferenced: validation fails first
    # quantize: k % 16 != 0, negative n, bad enum, NULL, misaligned codes
    assert L.nvfp4_quantize(fake, 16, 24, 24, 0, 1, fake, fake, fake, None, None) == qn.QN_ERR_SHAPE
    assert L.nvfp4_quantize(fake, -1, 32, 32, 0, 1, fake, fake, fake, None, None) == qn.QN_ERR_SHAPE
    assert L.nvfp4_quantize(fake, 16, 32, 32, 2, 1, fake, fake, fake, None, None) == qn.QN_ERR_VALUE
    assert L.nvfp4_quantize(fake, 16, 32, 32, 0, 7, fake, fake, fake, None, None) == qn.QN_ERR_VALUE
    assert L.nvfp4_quantize(None, 16, 32, 32, 0, 1, fake, fake, fake, None, None) == qn.QN_ERR_NULL
    assert L.nvfp4_quantize(fake, 16, 32, 16, 0, 1, fake, fake, fake, None, None) == qn.QN_ERR_SHAPE
    assert L.nvfp4_quantize(fake, 16, 32, 32, 0, 1, P(258), fake, fake, None, None) == qn.QN_ERR_ALIGN
    assert L.nvfp4_quantize(fake, 0, 32, 32, 0, 1, None, None, None, None, None) == qn.QN_OK  # empty
    # dequantize
    assert L.nvfp4_dequantize(fake, fake, fake, 16, 20, 1, fake, 20, None) == qn.QN_ERR_SHAPE
    assert L.nvfp4_dequantize(fake, fake, None, 16, 32, 1, fake, 32, None) == qn.QN_ERR_NULL
    # MXFP4 quantize / dequantize: k % 32 != 0, bad layout, NULL tensor scale for the tiled form, misaligned codes
    assert L.mxfp4_quantize(fake, 16, 48, 48, 0, fake, fake, None, None, None) == qn.QN_ERR_SHAPE
    assert L.mxfp4_quantize(fake, 16, 64, 32, 0, fake, fake, None, None, None) == qn.QN_ERR_SHAPE
    assert L.mxfp4_quantize(fake, 16, 64, 64, 3, fake, fake, None, None, None) == qn.QN_ERR_VALUE
    assert L.mxfp4_quantize(fake, 16, 64, 64, 1, fake, fake, None, None, None) == qn.QN_ERR_NULL
    assert L.mxfp4_quantize(fake, 16, 64, 64, 0, P(264), fake, None, None, None) == qn.QN_ERR_ALIGN
    assert L.mxfp4_quantize(fake, 0, 64, 64, 1, None, None, None, None, None) == qn.QN_OK  # empty
    assert L.mxfp4_dequantize(fake, fake, 16, 48, fake, 48, None) == qn.QN_ERR_SHAPE
    assert L.mxfp4_dequantize(fake, None, 16, 64, fake, 64, None) == qn.QN_ERR_NULL
    assert L.mxfp4_scales_bytes(16, 64) == 32 and L.mxfp4_scales_bytes(16, 48) == 0
    # norm: negative sigma, NaN eps, NULL aqn
    a = qn.QnAqn(gamma=256, noise=None, noise_ld=0, sigma=-1.0, eps=1e-6)
    assert L.aqn_rmsnorm(fake, 2, 32, 32, ctypes.byref(a), fake, 32, None) == qn.QN_ERR_VALUE
    a.sigma, a.eps = 0.01, float("nan")
    assert L.aqn_rmsnorm(fake, 2, 32, 32, ctypes.byref(a), fake, 32, None) == qn.QN_ERR_VALUE
    assert L.aqn_rmsnorm(fake, 2, 32, 32, None, fake, 32, None) == qn.QN_ERR_NULL
    # linear
    p = qn.QnProj(codes=256, block_scales=256, tensor_scale=256, n=64, lora_a=256, lora_b=256, r=32, lambda_=2.0,
                  y=256, y_dtype=0, ldy=64)
    arr = (qn.QnProj * 1)(p)
    need = L.nvfp4_lora_linear_workspace(4, 128, arr, 1)
    assert need > 0
    ok_args = lambda **kw: dict(dict(x=fake, m=4, k=128, ldx=128, aqn=None, projs=arr, nproj=1, epi=0, ws=P(1 << 20),
                                     wsb=need, stream=None), **kw)

    def call(**kw):
        a_ = ok_args(**kw)
        return L.nvfp4_lora_linear(a_["x"], a_["m"], a_["k"], a_["ldx"], a_["aqn"], a_["projs"], a_["nproj"],
                                   a_["epi"], a_["ws"], a_["wsb"], a_["stream"])

    assert call(k=120) == qn.QN_ERR_SHAPE
    assert call(ldx=64) == qn.QN_ERR_SHAPE
    assert call(nproj=0) == qn.QN_ERR_SHAPE
    assert call(nproj=5) == qn.QN_ERR_UNSUPPORTED
    assert call(epi=3) == qn.QN_ERR_VALUE
    assert call(epi=1) == qn.QN_ERR_SHAPE  # SiLU epilogue needs two projections
    assert call(wsb=need - 1) == qn.QN_ERR_WORKSPACE
    assert call(ws=None) == qn.QN_ERR_WORKSPACE
    assert call(x=None) == qn.QN_ERR_NULL
    assert call(m=0) == qn.QN_OK  # empty batch: nothing to do
    p.r = 65
    arr[0] = p
    assert call() == qn.QN_ERR_UNSUPPORTED
    p.r = 32
    p.codes = 264  # not 16-byte aligned
    arr[0] = p
    assert call() == qn.QN_ERR_ALIGN
    p.codes = 256
    p.lambda_ = float("inf")
    arr[0] = p
    assert call() == qn.QN_ERR_VALUE
    p.lambda_ = 2.0
    arr[0] = p
    # noise drawn on the device: not together with a noise buffer, draws per row >= 0 (norm and linear)
    a = qn.QnAqn(gamma=256, noise=256, noise_ld=0, sigma=0.01, eps=1e-6, draw=1, seed=1, subseed=0, row_offset=0,
                 draw_rows=1)
    assert L.aqn_rmsnorm(fake, 2, 32, 32, ctypes.byref(a), fake, 32, None) == qn.QN_ERR_VALUE
    assert call(aqn=ctypes.byref(a)) == qn.QN_ERR_VALUE
    a.noise, a.draw_rows = None, -1
    assert L.aqn_rmsnorm(fake, 2, 32, 32, ctypes.byref(a), fake, 32, None) == qn.QN_ERR_SHAPE
    assert call(aqn=ctypes.byref(a)) == qn.QN_ERR_SHAPE
    # standalone noise: shapes, row stride, draws per row, NULL output; empty is a no-op
    assert L.aqn_noise(1, 0, 0, 1, -1, 32, fake, 32, None) == qn.QN_ERR_SHAPE
    assert L.aqn_noise(1, 0, 0, 1, 2, 32, fake, 16, None) == qn.QN_ERR_SHAPE
    assert L.aqn_noise(1, 0, 0, -1, 2, 32, fake, 32, None) == qn.QN_ERR_SHAPE
    assert L.aqn_noise(1, 0, 0, 1, 2, 32, None, 32, None) == qn.QN_ERR_NULL
    assert L.aqn_noise(1, 0, 0, 1, 2, 32, P(258), 32, None) == qn.QN_ERR_ALIGN
    assert L.aqn_noise(1, 0, 0, 1, 0, 32, None, 32, None) == qn.QN_OK
    # GRPO surrogate: shapes, widths, aggregation, NULL statistics
    gs = L.grpo_clipped_surrogate
    assert gs(fake, fake, 8, fake, fake, -1, 8, 0.2, 0.2, 0, None, None, fake, None) == qn.QN_ERR_SHAPE
    assert gs(fake, fake, 4, fake, fake, 2, 8, 0.2, 0.2, 0, None, None, fake, None) == qn.QN_ERR_SHAPE
    assert gs(fake, fake, 8, fake, fake, 2, 8, 1.0, 0.2, 0, None, None, fake, None) == qn.QN_ERR_VALUE
    assert gs(fake, fake, 8, fake, fake, 2, 8, 0.2, -0.1, 0, None, None, fake, None) == qn.QN_ERR_VALUE
    assert gs(fake, fake, 8, fake, fake, 2, 8, 0.2, float("nan"), 0, None, None, fake, None) == qn.QN_ERR_VALUE
    assert gs(fake, fake, 8, fake, fake, 2, 8, 0.2, 0.2, 2, None, None, fake, None) == qn.QN_ERR_VALUE
    assert gs(fake, fake, 8, fake, fake, 2, 8, 0.2, 0.2, 0, None, None, None, None) == qn.QN_ERR_NULL
    assert gs(None, fake, 8, fake, fake, 2, 8, 0.2, 0.2, 0, None, None, fake, None) == qn.QN_ERR_NULL
    # backward: shapes, rank, dtype, NULLs, workspace
    order = ("g", "m", "n", "ldg", "h", "k", "ldh", "c", "s", "sg", "a", "b", "r", "lam", "dh", "dt", "lddh", "da", "db",
             "ws", "wsb", "st")

    def bw(**kw):
        args = dict(g=fake, m=4, n=64, ldg=64, h=fake, k=128, ldh=128, c=fake, s=fake, sg=fake, a=fake, b=fake, r=32,
                    lam=2.0, dh=fake, dt=1, lddh=128, da=fake, db=fake, ws=P(1 << 20), wsb=1 << 30, st=None)
        args.update(kw)
        return L.nvfp4_lora_linear_backward(*[args[key] for key in order])

    assert bw(k=120) == qn.QN_ERR_SHAPE
    assert bw(ldg=32) == qn.QN_ERR_SHAPE
    assert bw(r=65) == qn.QN_ERR_UNSUPPORTED
    assert bw(dt=5) == qn.QN_ERR_VALUE
    assert bw(lam=float("inf")) == qn.QN_ERR_VALUE
    assert bw(g=None) == qn.QN_ERR_NULL
    assert bw(h=None) == qn.QN_ERR_NULL
    assert bw(wsb=16) == qn.QN_ERR_WORKSPACE
    assert bw(g=P(257)) == qn.QN_ERR_ALIGN
    assert bw(m=0) == qn.QN_OK
    # advantage
    assert L.grpo_group_advantage(fake, 8, 8, -1.0, fake, None) == qn.QN_ERR_VALUE
    assert L.grpo_group_advantage(None, 8, 8, 1e-6, fake, None) == qn.QN_ERR_NULL


def test_host_helpers(qn):
    assert qn.aqn_sigma(0) == 0.0 and qn.aqn_sigma(1) == 0.01
    assert abs(qn.aqn_sigma(9) - 5e-4) < 1e-18
    cb, sb = qn.tiled_bytes(4096, 4096)
    assert cb == 4096 * 4096 // 2 and sb == 4096 * 4096 // 16  # no padding when n % 16 == 0 and k % 128 == 0
    cb, sb = qn.tiled_bytes(17, 144)
    assert cb == 2 * 2 * 1024 and sb == 2 * 2 * 128
    for s in range(8):
        assert qn.status_string(s)


def test_library_reads_no_environment():
    """Which kernel a call runs depends on its arguments and its explicit options only: no source of the library
    reads an environment variable."""
    csrc = os.path.join(ROOT, "nvfp4_weight_only_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, name)).read()
        assert "getenv" not in text and "environ" not in text, name


def test_linear_options_validation(qn):
    """Options out of range are QN_ERR_VALUE; a kernel that cannot serve the call is QN_ERR_UNSUPPORTED; both are
    decided on the host before any launch (every call here returns without touching a GPU)."""
    L = qn.lib
    P = ctypes.c_void_p
    fake = P(256)
    p = qn.QnProj(codes=256, block_scales=256, tensor_scale=256, n=64, lora_a=256, lora_b=256, r=32, lambda_=2.0,
                  y=256, y_dtype=0, ldy=64)
    arr = (qn.QnProj * 1)(p)

    def call(m, o, k=128, ws_bytes=None, aqn=None):
        oc = o.to_c()
        need = L.nvfp4_lora_linear_workspace_opts(m, k, arr, 1, ctypes.byref(oc))
        return L.nvfp4_lora_linear_opts(fake, m, k, k, ctypes.byref(aqn) if aqn else None, arr, 1, 0, ctypes.byref(oc),
                                        P(1 << 20), need if ws_bytes is None else ws_bytes, None)

    bad = [qn.LinearOpts(kernel=6), qn.LinearOpts(kernel=-1), qn.LinearOpts(decode_kchunks=65),
           qn.LinearOpts(decode_depth=4), qn.LinearOpts(general_rows=2), qn.LinearOpts(general_waves=8),
           qn.LinearOpts(elem_store=2)]
    for o in bad:
        assert call(4, o) == qn.QN_ERR_VALUE, o
        oc = o.to_c()
        assert L.nvfp4_lora_linear_workspace_opts(4, 128, arr, 1, ctypes.byref(oc)) == 0, o
    # the main kernel's event pair: both or neither (nothing is recorded before the options are checked), and it
    # does not change the workspace
    for begin, end in ((256, None), (None, 256)):
        oc = qn.LinearOpts().to_c()
        oc.main_begin, oc.main_end = begin, end
        assert L.nvfp4_lora_linear_workspace_opts(4, 128, arr, 1, ctypes.byref(oc)) == 0
        assert L.nvfp4_lora_linear_opts(fake, 4, 128, 128, None, arr, 1, 0, ctypes.byref(oc), P(1 << 20), 1 << 20,
                                        None) == qn.QN_ERR_VALUE
    oc = qn.LinearOpts().to_c()
    oc.main_begin, oc.main_end = 256, 512
    assert L.nvfp4_lora_linear_workspace_opts(4, 128, arr, 1, ctypes.byref(oc)) == L.nvfp4_lora_linear_workspace(
        4, 128, arr, 1)
    assert call(64, qn.LinearOpts(kernel=qn.KERNEL_DECODE)) == qn.QN_ERR_UNSUPPORTED  # decode kernel: m <= 32
    assert call(100, qn.LinearOpts(kernel=qn.KERNEL_MANY)) == qn.QN_ERR_UNSUPPORTED  # MFMA kernel: m > 128
    assert call(16, qn.LinearOpts(kernel=qn.KERNEL_WIDE)) == qn.QN_ERR_UNSUPPORTED  # 17 <= m <= 64
    assert call(65, qn.LinearOpts(kernel=qn.KERNEL_WIDE)) == qn.QN_ERR_UNSUPPORTED
    assert call(40, qn.LinearOpts(kernel=qn.KERNEL_WIDE, decode_depth=2)) == qn.QN_ERR_UNSUPPORTED
    # fused decode kernel: m <= 16, depth 0 or 3, not split into phases, with the norm the whole row in one k-chunk
    norm = qn.QnAqn(gamma=256, noise=None, noise_ld=0, sigma=0.01, eps=1e-6)
    assert call(17, qn.LinearOpts(kernel=qn.KERNEL_FUSED)) == qn.QN_ERR_UNSUPPORTED
    assert call(4, qn.LinearOpts(kernel=qn.KERNEL_FUSED), k=32 * 128, aqn=norm) == qn.QN_ERR_UNSUPPORTED
    assert call(4, qn.LinearOpts(kernel=qn.KERNEL_FUSED, decode_kchunks=2), aqn=norm) == qn.QN_ERR_UNSUPPORTED
    assert call(4, qn.LinearOpts(kernel=qn.KERNEL_FUSED, decode_depth=2)) == qn.QN_ERR_UNSUPPORTED
    oc = qn.LinearOpts(kernel=qn.KERNEL_FUSED).to_c()
    need = L.nvfp4_lora_linear_workspace_opts(4, 128, arr, 1, ctypes.byref(oc))
    for phase in (qn.RUN_PROLOGUE_ONLY, qn.RUN_MAIN_ONLY):
        assert L.nvfp4_lora_linear_opts(fake, 4, 128, 128, None, arr, 1, phase, ctypes.byref(oc), P(1 << 20), need,
                                        None) == qn.QN_ERR_UNSUPPORTED
    assert call(4, qn.LinearOpts(kernel=qn.KERNEL_GENERAL, general_rows=3, general_waves=5)) == qn.QN_ERR_UNSUPPORTED
    # a decode cut whose k-chunk does not fit the kernel's LDS: 32 tokens over a 40960-long row in one chunk
    assert call(32, qn.LinearOpts(kernel=qn.KERNEL_DECODE, decode_kchunks=1), k=40960) == qn.QN_ERR_UNSUPPORTED
    # the workspace check still applies with options
    assert call(4, qn.LinearOpts(kernel=qn.KERNEL_GENERAL), ws_bytes=16) == qn.QN_ERR_WORKSPACE
    # the plain entry point is the options entry point with the library's defaults
    assert L.nvfp4_lora_linear_workspace(4, 128, arr, 1) == L.nvfp4_lora_linear_workspace_opts(4, 128, arr, 1, None)


def test_workspace_covers_the_sub_calls_of_a_split_call(qn):
    """At 65 to 128 tokens a call on the big feed-forward projections runs as sub-calls of at most 64 tokens that
    share its workspace: its size covers each sub-call's (7B gate|up with SiLU, 7B down, 32B gate|up), and grows
    with m. Host-pure queries: nothing is launched."""
    L = qn.lib

    def ws(m, n, k, nproj):
        p = qn.QnProj(codes=256, block_scales=256, tensor_scale=256, n=n, lora_a=256, lora_b=256, r=32, lambda_=2.0,
                      y=256, y_dtype=0, ldy=n)
        arr = (qn.QnProj * nproj)(*([p] * nproj))
        return L.nvfp4_lora_linear_workspace(m, k, arr, nproj)

    for n, k, nproj in [(18944, 3584, 2), (3584, 18944, 1), (27648, 5120, 2)]:
        prev = 0
        for m in range(1, 129):
            w = ws(m, n, k, nproj)
            assert w >= prev, (n, k, m)
            prev = w
            if m > 64:
                assert w >= ws(64, n, k, nproj) and w >= ws(m - 64, n, k, nproj), (n, k, m)


def test_sigma_schedule_matches_oracle(qn, orc):
    """The library's sigma_k for every stage of the ten-stage schedule (0.01 -> 5e-4) equals the oracle's; stage 3 is
    the value the 28-layer configuration uses."""
    for k in range(10):
        assert qn.aqn_sigma(k) == orc.aqn_sigma(k), k
    assert abs(qn.aqn_sigma(3) - 4.728708e-3) < 5e-10
    # another start/end pair, and stages past 9 continuing the decay
    for k in range(12):
        assert qn.aqn_sigma(k, 0.05, 5e-4) == orc.aqn_sigma(k, 0.05, 5e-4), k
