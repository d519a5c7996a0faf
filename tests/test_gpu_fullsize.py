"""GPU parity at the configurations' full sizes, every output checked against the fp64 oracle.

- The quantizer on every configuration's weights (4096 x 4096; the 7B gate/up and down shapes; the 32B gate/up shape
  with heavy-tailed blocks whose 16-blocks carry exponents 2^e, e in -14..0): codes, block scales and tensor scale
  bit-exact in the row-major layout, and the tiled layout's dequantized f32 weights bit-exact.
- One Qwen2.5-7B-shaped decoder layer at M = 1, 8 and 16 tokens, op by op: each of the layer's four calls, with the
  same projection groups and the same kernels as the layer (q|k|v with v broadcast to its query heads, o with the
  residual, gate|up with SiLU(gate)*up, down with the residual), is fed the oracle's own bf16 input of that op, and
  all of its outputs are checked on the f32 result; then the layer itself runs end to end with bf16 storage and every
  element of its bf16 tensors is checked against the oracle's chain.
- The feed-forward calls at 80 and 128 tokens, which the library runs as sub-calls of at most 64 tokens, with the
  norm's noise drawn in draws that straddle the sub-calls' boundary.
- A ragged q|k|v whose projection boundaries fall inside two-row-group workgroups of the general kernel.
- The LoRA branch alone (zero base weight), against its own scale.
- A call on a side stream whose workspace is released while its kernels may still run.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, LINEAR_TOL, bf16_bits_to_f64, dev_bf16, dev_f32, host_bf16, host_u8, rel_err
from test_gpu_linear import bf16_chain_ok, make_layer_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import nvfp4_weight_only_amd as qn
    return qn


# ---- quantizer at full size ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n,k,dist", [
    (4096, 4096, "normal"),     # the single 4096 x 4096 projection
    (18944, 3584, "normal"),    # 7B gate / up
    (3584, 18944, "normal"),    # 7B down
    (27648, 5120, "t4"),        # 32B gate / up, Student-t (nu = 4) x 0.02 x 2^e per 16-block
])
def test_quantize_full_size_bitexact(qn, n, k, dist):
    s = lambda t: synth.seed_for(4, 0, t)
    if dist == "normal":
        w = synth.normal_bf16(s("w_gate") + n, (n, k), std=0.02)
    else:
        w = synth.student_t4_bf16(s("w_gate"), (n, k), 0.02, 16, s("block_exp"), -14)
    print(f"[quantize full size] {n} x {k} {dist}", flush=True)
    wd = dev_bf16(w)
    rm = qn.quantize(wd, qn.LAYOUT_ROWMAJOR)
    tl = qn.quantize(wd, qn.LAYOUT_TILED)
    deq = qn.dequantize(tl)
    torch.cuda.synchronize()
    codes, sb, sg, flags = oracle.nvfp4_quantize(w)
    assert flags == 0
    assert np.float32(rm.tensor_scale.item()) == np.float32(sg)
    assert np.array_equal(host_u8(rm.codes).reshape(n, k // 2), codes)
    assert np.array_equal(host_u8(rm.scales).reshape(n, k // 16), sb)
    assert np.float32(tl.tensor_scale.item()) == np.float32(sg)
    _, wf = oracle.nvfp4_dequantize(codes, sb, sg)
    del codes
    got = deq.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), wf.view(np.uint32))  # bit-exact, signs of zero included
    if dist == "t4":  # the heavy-tailed blocks reach every E4M3 binade, normal and subnormal, and zero
        used = np.unique(sb)
        assert used.min() == 0 and used.max() == 0x7e and np.any((used > 0) & (used < 8))


# ---- the 7B decoder layer, op by op and end to end ------------------------------------------------------------------
@pytest.fixture(scope="module")
def layer7b():
    from nvfp4_weight_only_amd.layer import QWEN25_7B
    shape = QWEN25_7B
    w, lora, _, g1, g2, e1, e2, sigma = make_layer_inputs(shape, 1, 7, 1e-2)
    print("[7B layer] quantizing the seven projections in the oracle", flush=True)
    qref = {nm: oracle.nvfp4_quantize(v)[:3] for nm, v in w.items()}
    return shape, w, lora, g1, g2, e1, e2, sigma, qref


@pytest.fixture(scope="module")
def layer7b_dev(qn, layer7b):
    from nvfp4_weight_only_amd.layer import DecoderLayer
    shape, w, lora, g1, g2, e1, e2, sigma, _ = layer7b
    return DecoderLayer.from_bf16(shape, {k: dev_bf16(v) for k, v in w.items()},
                                  {k: (dev_bf16(a), dev_bf16(b)) for k, (a, b) in lora.items()},
                                  dev_bf16(g1), dev_bf16(g2), dev_f32(e1), dev_f32(e2), sigma, 2.0)


def oracle_chain(layer7b, x):
    """The oracle's layer step, keeping each op's fp64 result and the bf16 tensor the next op consumes."""
    shape, _, lora, g1, g2, e1, e2, sigma, qref = layer7b

    def lin(h, nm):
        c, sb, sg = qref[nm]
        A, B = lora[nm]
        return oracle.lora_linear(h, c, sb, sg, A, B, 2.0)

    r = {}
    _, r["h1"] = oracle.aqn_rmsnorm(x, g1, e1, sigma, 1e-6)
    r["q64"], r["k64"], r["v64"] = lin(r["h1"], "q"), lin(r["h1"], "k"), lin(r["h1"], "v")
    r["q"], r["k"] = oracle.bf16_round_array(r["q64"]), oracle.bf16_round_array(r["k64"])
    r["attn"] = oracle.gqa_broadcast(oracle.bf16_round_array(r["v64"]), shape.group, shape.head_dim)
    r["x2_64"] = lin(r["attn"], "o") + bf16_bits_to_f64(x)
    r["x2"] = oracle.bf16_round_array(r["x2_64"])
    _, r["h2"] = oracle.aqn_rmsnorm(r["x2"], g2, e2, sigma, 1e-6)
    r["a64"] = oracle.silu_mul(lin(r["h2"], "gate"), lin(r["h2"], "up"))
    r["a"] = oracle.bf16_round_array(r["a64"])
    r["out64"] = lin(r["a"], "down") + bf16_bits_to_f64(r["x2"])
    r["out"] = oracle.bf16_round_array(r["out64"])
    return r


@pytest.mark.parametrize("m", [1, 8, 16])
def test_decoder_layer_7b_full(qn, layer7b, layer7b_dev, m):
    """Config-2 layer at M tokens. Every op at the layer's shapes and kernels, fed the oracle's input, all outputs
    within the bar on f32 results; then the layer end to end in bf16, every element against the oracle's chain."""
    shape, w, lora, g1, g2, e1, e2, sigma, qref = layer7b
    L = layer7b_dev
    x = synth.normal_bf16(synth.seed_for(2, 7, "x") + m, (m, shape.hidden))
    print(f"[7B layer] M={m}: oracle chain", flush=True)
    r = oracle_chain(layer7b, x)
    f32 = dict(dtype=torch.float32, device=DEV)

    def proj(nm, y, **kw):
        A, B = L.lora[nm]
        return qn.Projection(L.w[nm], y, A, B, 2.0, **kw)

    aqn1 = qn.make_aqn(L.gamma1, L.noise1, sigma, 1e-6)
    aqn2 = qn.make_aqn(L.gamma2, L.noise2, sigma, 1e-6)
    # 1. norm -> q | k | v (v broadcast to its 7 query heads)
    yq, yk, yv = torch.empty(m, shape.q_dim, **f32), torch.empty(m, shape.kv_dim, **f32), torch.empty(m, shape.q_dim, **f32)
    qn.lora_linear(dev_bf16(x), [proj("q", yq), proj("k", yk), proj("v", yv, y_repeat=shape.group,
                                                                   head_dim=shape.head_dim)], aqn1)
    # 2. o + residual, fed the oracle's attention output
    x_dev = dev_bf16(x)
    yo = torch.empty(m, shape.hidden, **f32)
    qn.lora_linear(dev_bf16(r["attn"]), [proj("o", yo, residual=x_dev)])
    # 3. norm -> gate | up, SiLU(gate) * up, fed the oracle's x2
    ya = torch.empty(m, shape.inter, **f32)
    qn.lora_linear(dev_bf16(r["x2"]), [proj("gate", ya), proj("up", None)], aqn2, qn.EPI_SILU_MUL)
    # 4. down + residual, fed the oracle's SiLU(gate) * up
    yd = torch.empty(m, shape.hidden, **f32)
    qn.lora_linear(dev_bf16(r["a"]), [proj("down", yd, residual=dev_bf16(r["x2"]))])
    torch.cuda.synchronize()
    assert rel_err(yq.cpu().numpy(), r["q64"]) <= LINEAR_TOL
    assert rel_err(yk.cpu().numpy(), r["k64"]) <= LINEAR_TOL
    assert rel_err(yv.cpu().numpy(), oracle.gqa_broadcast(r["v64"], shape.group, shape.head_dim)) <= LINEAR_TOL
    assert rel_err(yo.cpu().numpy(), r["x2_64"]) <= LINEAR_TOL
    assert rel_err(ya.cpu().numpy(), r["a64"]) <= LINEAR_TOL
    assert rel_err(yd.cpu().numpy(), r["out64"]) <= LINEAR_TOL

    # the layer itself, bf16 storage between ops, exactly as the benchmark runs it
    bound = L.bind(dev_bf16(x))
    bound()
    torch.cuda.synchronize()
    for name in ("q", "k", "attn", "x2", "a", "out"):
        assert bf16_chain_ok(host_bf16(getattr(bound, name)), r[name]), name


@pytest.mark.parametrize("m,draw_rows", [(80, 0), (128, 24)])
def test_feed_forward_split_into_sub_calls(qn, layer7b, layer7b_dev, m, draw_rows):
    """At 65 to 128 tokens the library runs the 7B feed-forward calls as sub-calls of at most 64 tokens (80 = 64 + 16,
    the second on the 16-token decode kernel; 128 = 64 + 64). gate|up with the norm and SiLU(gate) * up, and down with
    the residual: every output against the oracle. The norm's noise is drawn on the device in draws of draw_rows rows
    (24: a draw straddles the boundary at row 64), so every row must keep the draw of the whole call; the drawn call
    also gives the bits of the same call reading the generator's buffer."""
    shape, w, lora, g1, g2, e1, e2, sigma, qref = layer7b
    L = layer7b_dev
    x2 = synth.normal_bf16(synth.seed_for(2, 9, "x") + m, (m, shape.hidden))
    a = synth.normal_bf16(synth.seed_for(2, 10, "x") + m, (m, shape.inter))
    f32 = dict(dtype=torch.float32, device=DEV)

    def proj(nm, y, **kw):
        A, B = L.lora[nm]
        return qn.Projection(L.w[nm], y, A, B, 2.0, **kw)

    print(f"[split calls] M={m}, draws of {draw_rows} rows", flush=True)
    draw = qn.NoiseDraw(77, 2, 5, draw_rows)
    x2d = dev_bf16(x2)
    ya = torch.empty(m, shape.inter, **f32)
    qn.lora_linear(x2d, [proj("gate", ya), proj("up", None)], qn.make_aqn(L.gamma2, None, sigma, 1e-6, draw=draw),
                   qn.EPI_SILU_MUL)
    eps = qn.aqn_noise(draw, m, shape.hidden, DEV)
    read = qn.make_aqn(L.gamma2, eps, sigma, 1e-6, noise_per_row=True) if draw_rows else \
        qn.make_aqn(L.gamma2, eps[0].contiguous(), sigma, 1e-6)
    ya2 = torch.empty(m, shape.inter, **f32)
    qn.lora_linear(x2d, [proj("gate", ya2), proj("up", None)], read, qn.EPI_SILU_MUL)
    yd = torch.empty(m, shape.hidden, **f32)
    qn.lora_linear(dev_bf16(a), [proj("down", yd, residual=x2d)])
    torch.cuda.synchronize()
    assert torch.equal(ya, ya2)

    def lin(h, nm):
        c, sb, sg = qref[nm]
        A, B = lora[nm]
        return oracle.lora_linear(h, c, sb, sg, A, B, 2.0)

    _, h2 = oracle.aqn_rmsnorm(x2, g2, oracle.aqn_noise(77, 2, 5, draw_rows, m, shape.hidden), sigma, 1e-6,
                               noise_per_row=True)
    assert rel_err(ya.cpu().numpy(), oracle.silu_mul(lin(h2, "gate"), lin(h2, "up"))) <= LINEAR_TOL
    assert rel_err(yd.cpu().numpy(), lin(a, "down") + bf16_bits_to_f64(x2)) <= LINEAR_TOL


@pytest.mark.parametrize("m", [1, 8, 16])
def test_qkv_ragged_boundaries_inside_workgroups(qn, m):
    """q | k | v with 257 + 34 + 33 row groups (more than 256, so the general kernel takes two row groups per
    workgroup): the q/k and k/v boundaries both fall inside one workgroup, and q and v end in half-filled row groups.
    Every output row against the oracle, with the library's choice and with the two-group shape named explicitly."""
    ns, k = [4104, 536, 520], 3584
    from test_gpu_linear import Case
    c = Case(m, ns, k, seed=4104 + m)
    wq = [qn.quantize(dev_bf16(w), qn.LAYOUT_TILED) for w in c.w]
    refs = [c.oracle_y(p) for p in range(3)]
    for opts in (None, qn.LinearOpts(kernel=qn.KERNEL_GENERAL, general_rows=2, general_waves=8)):
        ys = [torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV) for n in ns]
        projs = [qn.Projection(wq[p], ys[p], dev_bf16(c.A[p]), dev_bf16(c.B[p]), c.lam) for p in range(3)]
        qn.lora_linear(dev_bf16(c.x), projs, qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6),
                       opts=opts)
        torch.cuda.synchronize()
        for p in range(3):
            got = ys[p].cpu().numpy()
            assert np.all(np.isfinite(got)), p
            assert rel_err(got, refs[p]) <= LINEAR_TOL, (opts, p)


# ---- the LoRA branch alone -------------------------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,k,r,kern", [(1, 4096, 4096, 32, None), (16, 18944, 3584, 32, None),
                                           (8, 3584, 18944, 32, None), (16, 520, 1040, 12, "general"),
                                           (300, 512, 640, 64, None), (64, 18944, 3584, 32, None),
                                           (40, 3584, 18944, 32, None), (24, 1040, 1024, 64, "wide")])
def test_lora_term_alone(qn, m, n, k, r, kern):
    """With a zero base weight the output is lambda * B (A h) alone: checked against the oracle's LoRA term at the bar,
    relative to that term's own magnitude (the branch is about a fifth of a full output, so the bar on the full
    output would hide errors of a few per cent in it)."""
    s = lambda t: synth.seed_for(6, m, t)
    h = synth.normal_bf16(s("x"), (m, k))
    A = synth.normal_bf16(s("a_q"), (r, k), std=0.02)
    B = synth.normal_bf16(s("b_q"), (n, r), std=0.02)
    w0 = np.zeros((n, k), dtype=np.uint16)
    wq = qn.quantize(dev_bf16(w0), qn.LAYOUT_TILED)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    opts = {"general": qn.LinearOpts(kernel=qn.KERNEL_GENERAL), "wide": qn.LinearOpts(kernel=qn.KERNEL_WIDE),
            None: None}[kern]
    qn.lora_linear(dev_bf16(h), [qn.Projection(wq, y, dev_bf16(A), dev_bf16(B), 2.0)], opts=opts)
    torch.cuda.synchronize()
    codes, sb, sg, _ = oracle.nvfp4_quantize(w0)
    ref = oracle.lora_linear(h, codes, sb, sg, A, B, 2.0)
    assert np.abs(ref).max() > 0
    assert rel_err(y.cpu().numpy(), ref) <= LINEAR_TOL


# ---- streams and concurrent work -------------------------------------------------------------------------------------
@pytest.mark.parametrize("where", ["side-stream", "beside-other-kernels"])
def test_calls_correct_with_concurrent_work(qn, where):
    """Calls whose kernels run while other kernels occupy the GPU: on a side stream whose workspace the binding drops
    at once (its memory must not be handed to the current stream's fills while the side stream uses it), or on the
    current stream while a side stream fills memory. Every output of 24 calls of the 7B gate shape at 16 tokens
    (decode kernel, LoRA term in its LoRA wave) is checked. Regression: the LoRA wave once stored its MFMA result one
    instruction after the MFMA on a taken branch, and a 4-row x 16-token block came out wrong in a few per cent of
    calls, in up to a third with other kernels running beside it."""
    from test_gpu_linear import Case
    c = Case(16, [18944], 3584, seed=77)
    wq = qn.quantize(dev_bf16(c.w[0]), qn.LAYOUT_TILED)
    A, B, x = dev_bf16(c.A[0]), dev_bf16(c.B[0]), dev_bf16(c.x)
    aqn = qn.make_aqn(dev_bf16(c.gamma), dev_f32(c.noise), c.sigma, 1e-6)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()

    def fills():  # allocations of every size class, filled at once
        return [torch.full((1 << e,), 7, dtype=torch.uint8, device=DEV) for e in range(12, 23) for _ in range(2)]

    outs = []
    for _ in range(24):
        y = torch.empty(16, 18944, dtype=torch.float32, device=DEV)
        if where == "side-stream":
            y.record_stream(side)
            side.wait_stream(torch.cuda.current_stream())  # the caller's part: y may reuse memory of pending work
            qn.lora_linear(x, [qn.Projection(wq, y, A, B, c.lam)], aqn, stream=side)  # workspace dropped on return
            junk = fills()
        else:
            with torch.cuda.stream(side):
                junk = fills()
            qn.lora_linear(x, [qn.Projection(wq, y, A, B, c.lam)], aqn)
        outs.append(y)
        del junk
    torch.cuda.synchronize()
    ref = c.oracle_y(0)
    for i, y in enumerate(outs):
        yv = y.cpu().numpy()
        err = np.abs(yv - ref) / np.abs(ref).max()
        bad = np.where(err.max(axis=0) > LINEAR_TOL)[0]
        assert rel_err(yv, ref) <= LINEAR_TOL, (i, len(bad), np.unique(bad // 16)[:16].tolist())
