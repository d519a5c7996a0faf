"""nvfp4_lora_linear_noalloc (the entry point that allocates nothing) against nvfp4_lora_linear on the same inputs.

Both run the same kernels; the only difference is where the scratch space lives (the library's own device array
instead of a caller's workspace), so the outputs must be bit-identical, and both within the bar of the fp64 oracle.
Two calls in a row, the second smaller than the first, so the second runs on an array that still holds the first
call's contents (partial sums, arrival counters, activation fragments).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, LINEAR_TOL, bf16_bits_to_f64, dev_bf16, dev_f32, rel_err
from test_gpu_linear import Case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


def run_both(qn, c, epilogue=0, residual=None, aqn=True):
    """The call through nvfp4_lora_linear and through nvfp4_lora_linear_noalloc: (outputs, outputs)."""
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    norm = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6) if aqn else None
    outs = []
    for entry in ("workspace", "noalloc"):
        ys, projs = [], []
        for p, n in enumerate(c.ns):
            y = torch.full((c.m, n), float("nan"), dtype=torch.float32, device=DEV)
            ys.append(y)
            projs.append(qn.Projection(wq[p], None if (epilogue and p == 1) else y, dev_bf16(c.A[p]), dev_bf16(c.B[p]),
                                       c.lam, residual=residual))
        x = dev_bf16(c.x)
        if entry == "workspace":
            qn.lora_linear(x, projs, norm, epilogue)
        else:
            qn.lora_linear_noalloc(x, projs, norm, epilogue)
        torch.cuda.synchronize()
        outs.append(ys[:1] if epilogue else ys)
    return outs


def test_noalloc_two_calls_match_workspace_entry(qn):
    # 1. the 7B down projection at 16 tokens with its residual: the decode kernel with an 8-way split k (part sums and
    #    arrival counters in the scratch array)
    c1 = Case(16, [3584], 18944, seed=501, aqn=False)
    res = dev_bf16(np.asarray(c1.x[:, :3584]))
    a, b = run_both(qn, c1, residual=res, aqn=False)
    assert torch.equal(a[0], b[0])
    ref = c1.oracle_y(0) + bf16_bits_to_f64(np.asarray(c1.x[:, :3584]))
    assert rel_err(b[0].cpu().numpy(), ref) <= LINEAR_TOL
    # 2. smaller: q | k | v sharing an AQN-RMSNorm at 4 tokens (the general kernel), on the array the first call left
    c2 = Case(4, [512, 128, 128], 1024, seed=502)
    a, b = run_both(qn, c2)
    for p in range(3):
        assert torch.equal(a[p], b[p]), p
        assert rel_err(b[p].cpu().numpy(), c2.oracle_y(p)) <= LINEAR_TOL, p
    # 3. gate | up with SiLU(gate) * up at 8 tokens (the decode kernel with the pair epilogue)
    c3 = Case(8, [1024, 1024], 512, seed=503)
    a, b = run_both(qn, c3, epilogue=qn.EPI_SILU_MUL)
    assert torch.equal(a[0], b[0])
    assert rel_err(b[0].cpu().numpy(), oracle.silu_mul(c3.oracle_y(0), c3.oracle_y(1))) <= LINEAR_TOL
    # 4. the 7B gate | up at 40 tokens (the kernel for 17-64 tokens; the prologue sums t with arrival counters that
    #    must be left zero in the array for the next call)
    c4 = Case(40, [18944, 18944], 3584, seed=505)
    for _ in range(2):
        a, b = run_both(qn, c4, epilogue=qn.EPI_SILU_MUL)
        assert torch.equal(a[0], b[0])
    assert rel_err(b[0].cpu().numpy(), oracle.silu_mul(c4.oracle_y(0), c4.oracle_y(1))) <= LINEAR_TOL
    # 5. the 7B down at 80 tokens with its residual: run as two sub-calls (64 tokens on the kernel for 17-64 tokens
    #    with a split k, then 16 on the decode kernel with its own), one after the other on the same array
    c5 = Case(80, [3584], 18944, seed=506, aqn=False)
    res5 = dev_bf16(np.asarray(c5.x[:, :3584]))
    a, b = run_both(qn, c5, residual=res5, aqn=False)
    assert torch.equal(a[0], b[0])
    ref5 = c5.oracle_y(0) + bf16_bits_to_f64(np.asarray(c5.x[:, :3584]))
    assert rel_err(b[0].cpu().numpy(), ref5) <= LINEAR_TOL


def test_noalloc_rejects_calls_beyond_its_array(qn):
    """A call whose scratch would exceed the array (8192 tokens of the 7B gate|up) is refused on the host."""
    assert qn.lib.nvfp4_lora_linear_noalloc_max_bytes() == 32 << 20
    c = Case(1, [256, 256], 3584, seed=504)
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    x = torch.zeros(8192, 3584, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(8192, 256, dtype=torch.bfloat16, device=DEV)
    projs = [qn.Projection(wq[0], y, dev_bf16(c.A[0]), dev_bf16(c.B[0]), 2.0),
             qn.Projection(wq[1], None, dev_bf16(c.A[1]), dev_bf16(c.B[1]), 2.0)]
    assert qn.linear_workspace_bytes(8192, 3584, projs) > qn.lib.nvfp4_lora_linear_noalloc_max_bytes()
    with pytest.raises(qn.QnError) as e:
        qn.lora_linear_noalloc(x, projs, None, qn.EPI_SILU_MUL)
    assert e.value.status == qn.QN_ERR_WORKSPACE
