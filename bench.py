#!/usr/bin/env python3
"""Benchmark of the QeRL rollout-decode linear layer (NVFP4 weights, rank-32 bf16 LoRA, AQN-RMSNorm) on one GPU.

Headline (the one JSON line's `value`): one Qwen2.5-7B-shaped decoder layer at decode, M = 16 tokens (hidden 3584;
q/o 3584x3584; k/v 512x3584; gate/up 18944x3584; down 3584x18944). A step is one decode pass of the whole layer:
AQN-RMSNorm -> q|k|v (v broadcast to its query heads; attention scores excluded) -> o + residual -> AQN-RMSNorm ->
gate|up + SiLU*up -> down + residual. Steps rotate over several copies of the layer's weights so the working set is
well beyond the 256 MB Infinity Cache (cold HBM). `value` = M / (28 x layer step time): 28-layer-equivalent decode
tokens/s. All inputs are seeded synthetic tensors (synth/): W ~ N(0, 0.02) quantized on the GPU, x ~ N(0, 1),
sigma = 1e-2 (stage 1 of the ten-stage schedule).

The same line carries, under `configs`, every other workload of the layer's configuration list, each timed on its
own (wall clock over timed steps, bracketed by device synchronisation; cold weights wherever the workload fits the
cache):
  c1_proj4096_m1      one 4096x4096 projection with AQN-RMSNorm and rank-32 LoRA, 1 token (52 weight copies rotated)
  c2_layer7b_m1/_m8   the headline layer at M = 1 and 8
  c3_stack28_7b_m64   28 chained 7B-shaped layers at M = 64, sigma_3 = 0.01 * 0.05^(1/4) in all 56 norms
  c4_layer32b_m32/_m128  one Qwen2.5-32B-shaped layer (hidden 5120; q/o 5120^2; k/v 1024x5120; gate/up 27648x5120;
                      down 5120x27648), heavy-tailed weights (Student-t nu = 4 x 0.02 x 2^e per 16-block)
  c5_prefill_m8192    8192 tokens through the 7B gate|up with LoRA and SiLU*up on the MFMA kernel, then the group
                      advantages of 8 groups of 8 Bernoulli(0.3) rewards
  f3_mxfp4_layer7b_m16    the headline layer with MXFP4 weights (the exact tiled form through the same kernels)
  f3_mxfp4_prefill_m8192  the prefill gate|up with MXFP4 weights on the scaled FP4 x FP8 MFMA kernel
                      (mxfp4_lora_linear), and through the tiled form on the f16 MFMA kernel for comparison
  f2_backward_gate_m8192  backward of the 7B gate projection at 8192 tokens: dh through the frozen NVFP4 weight, dA, dB
  f4_grpo_surrogate_8192  GRPO token ratios and clipped surrogate over the same 64 responses x 128 tokens
plus `hbm_stream_read` (a plain streaming-read kernel over 4 GiB: the achievable read rate, the second roofline
denominator) and `cpu_baseline` (the fp64 oracle on the host, all threads and one thread).

`--workload prefill` prints the prefill line alone (value = TFLOP/s of the step).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16 / bf16 matrix peak, published
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix peak, published
PROFILE = os.path.join(ROOT, "profiles", "decode_layer_7b_m16.md")
PREFILL_PROFILE = os.path.join(ROOT, "profiles", "prefill_gateup_7b_m8192.md")
KERNEL_SOURCE = os.path.join(ROOT, "nvfp4_weight_only_amd", "csrc", "linear.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def profile_value(profile, key, tag):
    """A figure a committed rocprofv3 summary records for the current kernel source (`key[tag] = V (linear.hip
    sha256 H)`), or None when the summary is missing or was taken on another version of the kernels."""
    try:
        text = open(profile).read()
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    m = re.search(re.escape(key) + r"\[" + re.escape(tag) + r"\] = ([0-9.]+) \(linear\.hip sha256 ([0-9a-f]{64})\)", text)
    if not m or m.group(2) != sha:
        return None
    return float(m.group(1))


# ---- byte and flop accounting (algorithmic: what the method must move / compute) -----------------------------------
def proj_bytes(n, k, m, r):
    """NVFP4 9NK/16 + 4 (codes, E4M3 scales, f32 tensor scale), LoRA 2r(N+K), activations in/out 2M(N+K)."""
    return 9 * n * k // 16 + 4 + 2 * r * (n + k) + 2 * m * (n + k)


def layer_bytes(shape, m):
    """Per layer step: every projection, plus gamma (bf16) and noise (f32) of the two norms, 6d each."""
    return sum(proj_bytes(n, k, m, shape.rank) for n, k in shape.projections().values()) + 2 * 6 * shape.hidden


def layer_flops(shape, m):
    return sum(2 * m * n * k + 2 * m * shape.rank * (n + k) for n, k in shape.projections().values())


def gateup_main_bytes(shape, m):
    """Algorithmic bytes of the gate|up main kernel: both NVFP4 weights, both LoRA-B, the activation in, a out."""
    n, k = shape.inter, shape.hidden
    return 2 * (9 * n * k // 16 + 4) + 2 * 2 * shape.rank * n + 2 * m * k + 2 * m * n


def prefill_flops(shape, m):
    """gate and up: 2 M N K each, plus the rank-r LoRA of each (down 2 M r K, up 2 M r N)."""
    n, k, r = shape.inter, shape.hidden, shape.rank
    return 2 * (2 * m * n * k + 2 * m * r * (n + k))


def hbm_entry(t_s, nbytes, stream_gbs=None, extra=None):
    gbs = nbytes / t_s / 1e9
    d = {"us_per_step": t_s * 1e6, "algorithmic_bytes": nbytes, "GBps": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}
    if stream_gbs:
        d["frac_of_stream_read"] = gbs / stream_gbs
    if extra:
        d.update(extra)
    return d


# ---- device set-up -------------------------------------------------------------------------------------------------
def bf16_dev(a, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def build_layer(shape, workload, dev, sigma, wdist="normal"):
    """One layer's packed weights and adapters from the seeded generators (quantized on the device)."""
    import torch

    import synth
    from nvfp4_weight_only_amd.layer import DecoderLayer

    s = lambda t: synth.seed_for(workload, 0, t)
    w = {}
    for nm, nk in shape.projections().items():
        if wdist == "normal":
            w[nm] = bf16_dev(synth.normal_bf16(s("w_" + nm), nk, std=0.02), dev)
        else:  # heavy tail: Student-t (nu = 4) x 0.02 x 2^e per 16-block, e uniform on -14..0
            w[nm] = bf16_dev(synth.student_t4_bf16(s("w_" + nm), nk, 0.02, 16, s("block_exp") + len(nm), -14), dev)
    lora = {nm: (bf16_dev(synth.normal_bf16(s("a_" + nm), (shape.rank, nk[1]), std=0.02), dev),
                 bf16_dev(synth.normal_bf16(s("b_" + nm), (nk[0], shape.rank), std=0.02), dev))
            for nm, nk in shape.projections().items()}
    g = bf16_dev(synth.bf16_const(1.0, (shape.hidden,)), dev)
    e1 = torch.from_numpy(synth.normal_f32(s("eps_norm1"), (shape.hidden,))).to(dev)
    e2 = torch.from_numpy(synth.normal_f32(s("eps_norm2"), (shape.hidden,))).to(dev)
    layer = DecoderLayer.from_bf16(shape, w, lora, g, g, e1, e2, sigma, 2.0)
    del w
    torch.cuda.synchronize()
    return layer


def copies_of(layer, count, noises=None):
    """`count` layers with distinct copies of the packed weights and adapters (same values, new addresses)."""
    from nvfp4_weight_only_amd.layer import DecoderLayer
    out = []
    for i in range(count):
        if i == 0:
            wq, lo = layer.w, layer.lora
        else:
            wq = {nm: type(q)(q.codes.clone(), q.scales.clone(), q.tensor_scale.clone(), q.n, q.k, q.layout)
                  for nm, q in layer.w.items()}
            lo = {nm: (a.clone(), b.clone()) for nm, (a, b) in layer.lora.items()}
        n1, n2 = noises[i] if noises else (layer.noise1, layer.noise2)
        out.append(DecoderLayer(layer.shape, wq, lo, layer.gamma1, layer.gamma2, n1, n2, layer.sigma, layer.lam,
                                draws=layer.draws))
    return out


def time_steps(step, steps, warmup):
    """Wall-clock seconds per step over `steps` timed steps after `warmup` untimed ones, bracketed by device
    synchronisation."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


# ---- the configurations --------------------------------------------------------------------------------------------
def run_stream_read(dev, steps):
    import torch
    import nvfp4_weight_only_amd as qn
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    t = time_steps(lambda i: qn.stream_read(buf, sink), max(steps, 10), 3)
    gbs = buf.numel() / t / 1e9
    del buf
    return {"GBps": gbs, "bytes": 4 << 30, "us_per_read": t * 1e6, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
            "kernel": "qn_stream_read: 16-byte non-temporal loads, 2048 workgroups x 256 threads, grid-stride"}


def run_c1(dev, sigma, steps, warmup, stream_gbs):
    """One 4096 x 4096 projection with AQN-RMSNorm, rank-32 LoRA, lambda 2, 1 token; 52 copies rotated (> 512 MB)."""
    import torch
    import nvfp4_weight_only_amd as qn
    import synth
    n = k = 4096
    s = lambda t: synth.seed_for(1, 0, t)
    wq = qn.quantize(bf16_dev(synth.normal_bf16(s("w_q"), (n, k), std=0.02), dev), qn.LAYOUT_TILED)
    A = bf16_dev(synth.normal_bf16(s("a_q"), (32, k), std=0.02), dev)
    B = bf16_dev(synth.normal_bf16(s("b_q"), (n, 32), std=0.02), dev)
    x = bf16_dev(synth.normal_bf16(s("x"), (1, k)), dev)
    g = bf16_dev(synth.bf16_const(1.0, (k,)), dev)
    z = torch.from_numpy(synth.normal_f32(s("eps_norm1"), (k,))).to(dev)
    aqn = qn.make_aqn(g, z, sigma, 1e-6)
    y = torch.empty(1, n, dtype=torch.bfloat16, device=dev)
    ws = qn.Workspace(dev)
    calls = []
    for i in range(52):
        w_i = wq if i == 0 else type(wq)(wq.codes.clone(), wq.scales.clone(), wq.tensor_scale.clone(), n, k, wq.layout)
        calls.append(qn.LinearCall(x, [qn.Projection(w_i, y, A.clone(), B.clone(), 2.0)], aqn, qn.EPI_NONE, ws))
    t = time_steps(lambda i: calls[i % len(calls)](), max(steps, 52), warmup)
    nbytes = proj_bytes(n, k, 1, 32) + 6 * k
    return hbm_entry(t, nbytes, stream_gbs, {"tokens_per_s": 1.0 / t, "copies_rotated": 52,
                                            "kernels": "prologue (norm, fragments, LoRA-down) + main (weight stream)"})


def run_layer(layers, shape, m, dev, steps, warmup, stream_gbs, layers_equiv, x_seed):
    import nvfp4_weight_only_amd as qn
    import synth
    x = bf16_dev(synth.normal_bf16(x_seed, (m, shape.hidden)), dev)
    ws = qn.Workspace(dev)
    bound = [L.bind(x, ws) for L in layers]
    t = time_steps(lambda i: bound[i % len(bound)](), steps, warmup)
    fl = layer_flops(shape, m)
    return hbm_entry(t, layer_bytes(shape, m), stream_gbs,
                     {"tokens_per_s": m / (layers_equiv * t), "tokens_per_s_basis": f"M / ({layers_equiv} x layer step)",
                      "TFLOPs": fl / t / 1e12, "frac_of_mfma_peak": fl / t / 1e12 / MFMA_PEAK_TFLOPS,
                      "copies_rotated": len(layers)})


def run_f3(base, shape, dev, steps, warmup, stream_gbs):
    """The 7B layer at M = 16 with MXFP4 weights (E8M0 scale per 32; the same seeded bf16 weights quantized by the MX
    rule and written in the tiled form the kernels read), 5 copies rotated. The tiled form stores the MX scale once
    per 16 weights, so the bytes read are NVFP4's."""
    import torch
    import nvfp4_weight_only_amd as qn
    import synth
    from nvfp4_weight_only_amd.layer import DecoderLayer
    s = lambda t: synth.seed_for(2, 0, t)
    w = {nm: qn.mxfp4_quantize(bf16_dev(synth.normal_bf16(s("w_" + nm), nk, std=0.02), dev), qn.LAYOUT_TILED)
         for nm, nk in shape.projections().items()}
    mx = DecoderLayer(shape, w, base.lora, base.gamma1, base.gamma2, base.noise1, base.noise2, base.sigma, base.lam)
    torch.cuda.synchronize()
    layers = copies_of(mx, 5)
    out = run_layer(layers, shape, 16, dev, steps, warmup, stream_gbs, 28, synth.seed_for(2, 0, "x") + 16)
    out["weights"] = "MXFP4 (OCP MX rule), tiled form with power-of-two NVFP4 block and tensor scales"
    return out


def run_c3(base, shape, dev, steps, warmup, stream_gbs):
    """28 chained layers (distinct weight copies), M = 64, sigma_3 in all 56 norms, a fresh noise vector per norm."""
    import torch
    import nvfp4_weight_only_amd as qn
    import synth
    m, nl = 64, 28
    sigma3 = float(qn.aqn_sigma(3))
    noises = [tuple(torch.from_numpy(synth.normal_f32(synth.seed_for(3, l, t), (shape.hidden,))).to(dev)
                    for t in ("eps_norm1", "eps_norm2")) for l in range(nl)]
    layers = copies_of(base, nl, noises)
    for L in layers:
        L.sigma = sigma3
    ws = qn.Workspace(dev)
    x = bf16_dev(synth.normal_bf16(synth.seed_for(3, 0, "x"), (m, shape.hidden)), dev)
    bound, h = [], x
    for L in layers:
        b = L.bind(h, ws)
        bound.append(b)
        h = b.out

    def step(i):
        for b in bound:
            b()

    t = time_steps(step, max(3, steps // 4), max(1, warmup // 2))
    nbytes = nl * layer_bytes(shape, m)
    fl = nl * layer_flops(shape, m)
    r = hbm_entry(t, nbytes, stream_gbs, {"tokens_per_s": m / t, "layers": nl, "sigma": sigma3,
                                           "TFLOPs": fl / t / 1e12, "frac_of_mfma_peak": fl / t / 1e12 / MFMA_PEAK_TFLOPS})
    del bound, layers
    return r


class LaunchEvent:
    """A HIP event for a main kernel's own launch interval (qn_linear_opts main_begin / main_end), created with
    hipEventDisableSystemFence: without it the end event adds a system-scope release to the kernel (on the 7B
    gate|up ≈ 1.3 µs of the measured interval and ≈ 3 µs of the step)."""
    _hip = None

    def __init__(self):
        import ctypes
        if LaunchEvent._hip is None:
            LaunchEvent._hip = ctypes.CDLL("libamdhip64.so")  # the HIP runtime torch runs on
        self._h = ctypes.c_void_p()
        if LaunchEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._h), ctypes.c_uint(0x20000000)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = self._h.value

    def record(self, stream):
        import ctypes
        if LaunchEvent._hip.hipEventRecord(self._h, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        if LaunchEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self._h, end._h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if LaunchEvent._hip is not None and self._h:
            LaunchEvent._hip.hipEventDestroy(self._h)


def launch_event_pairs(keys, stream):
    """A (begin, end) LaunchEvent pair per key, each event recorded once so it exists before a launch records it."""
    out = {}
    for key in keys:
        out[key] = (LaunchEvent(), LaunchEvent())
        for e in out[key]:
            e.record(stream)
    return out


def run_c5(base, shape, dev, steps, warmup):
    """8192 tokens through the 7B gate|up (the headline layer's weights) + LoRA + SiLU*up, then group advantages."""
    import torch
    import nvfp4_weight_only_amd as qn
    import synth
    m, n, k = 8192, shape.inter, shape.hidden
    s = lambda t: synth.seed_for(5, 0, t)
    x = bf16_dev(synth.normal_bf16(s("x"), (m, k)), dev)
    y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    rewards = torch.from_numpy(synth.bernoulli_f32(s("rewards"), (8, 8), 0.3)).to(dev)
    (Ag, Bg), (Au, Bu) = base.lora["gate"], base.lora["up"]
    call = qn.LinearCall(x, [qn.Projection(base.w["gate"], y, Ag, Bg, 2.0),
                             qn.Projection(base.w["up"], None, Au, Bu, 2.0)], None, qn.EPI_SILU_MUL)
    stream = torch.cuda.current_stream()
    nsteps = max(5, steps // 2)
    ev = launch_event_pairs(range(nsteps), stream)
    timed = {"on": False}

    def step(i):
        # timed steps: the many-token kernel records its own begin and end in the step's event pair
        call(main_events=ev[i] if timed["on"] else None)
        qn.group_advantage(rewards)

    for i in range(max(2, warmup // 2)):
        step(i)
    timed["on"] = True
    t = time_steps(step, nsteps, 0)
    main_s = sum(a.elapsed_time(b) for a, b in ev.values()) / nsteps * 1e-3
    fl = prefill_flops(shape, m)
    prof_us = profile_value(PREFILL_PROFILE, "avg_duration_us", "k_gemm gate|up")
    r = {"us_per_step": t * 1e6, "prefill_tokens_per_s": m / t, "step_TFLOPs": fl / t / 1e12,
         "flops_per_step": fl, "kernel": "k_gemm<SILU> (many-token MFMA kernel)", "kernel_us_events": main_s * 1e6,
         "kernel_TFLOPs_events": fl / main_s / 1e12, "frac_of_mfma_peak_events": fl / main_s / 1e12 / MFMA_PEAK_TFLOPS}
    if prof_us:
        r.update({"kernel_us_profile": prof_us, "frac_of_mfma_peak_profile": fl / (prof_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS})
    del x, y
    return r


def run_f3_prefill(base, shape, dev, steps, warmup):
    """MXFP4 weights at prefill: 8192 tokens through the 7B gate|up (the headline layer's seeded weights, quantized to
    OCP MXFP4) with LoRA and SiLU*up, on the scaled FP4 x FP8 MFMA kernel (mxfp4_lora_linear, canonical weights) and,
    for comparison, on the f16 MFMA kernel through the exact tiled form (nvfp4_lora_linear)."""
    import torch
    import nvfp4_weight_only_amd as qn
    import synth
    m, n, k = 8192, shape.inter, shape.hidden
    s = lambda t: synth.seed_for(2, 0, t)
    wb = {nm: bf16_dev(synth.normal_bf16(s("w_" + nm), (n, k), std=0.02), dev) for nm in ("gate", "up")}
    canon = {nm: qn.mxfp4_quantize(w, qn.LAYOUT_ROWMAJOR) for nm, w in wb.items()}
    tiled = {nm: qn.mxfp4_quantize(w, qn.LAYOUT_TILED) for nm, w in wb.items()}
    del wb
    x = bf16_dev(synth.normal_bf16(synth.seed_for(5, 0, "x"), (m, k)), dev)
    y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    (Ag, Bg), (Au, Bu) = base.lora["gate"], base.lora["up"]
    ws = qn.Workspace(dev)

    def projs(w):
        return [qn.Projection(w["gate"], y, Ag, Bg, 2.0), qn.Projection(w["up"], None, Au, Bu, 2.0)]

    native_call = lambda i: qn.mxfp4_lora_linear(x, projs(canon), None, qn.EPI_SILU_MUL, ws)
    tiled_call = qn.LinearCall(x, projs(tiled), None, qn.EPI_SILU_MUL, ws)
    nsteps = max(5, steps // 2)
    t_native = time_steps(native_call, nsteps, max(2, warmup // 2))
    t_tiled = time_steps(lambda i: tiled_call(), nsteps, max(2, warmup // 2))
    fl = prefill_flops(shape, m)
    # the scaled instruction does the product twice (hi and lo parts of the activations) at the FP8 rate
    mfma_work = 2 * (2 * m * n * k * 2)
    r = {"us_per_call": t_native * 1e6, "TFLOPs": fl / t_native / 1e12, "flops_per_call": fl,
         "frac_of_fp8_mfma_peak": mfma_work / t_native / 1e12 / FP8_PEAK_TFLOPS,
         "kernel": "k_gemm<SILU, MX>: v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 weights x E4M3 hi/lo activations",
         "tiled_form_us_per_call": t_tiled * 1e6, "tiled_form_TFLOPs": fl / t_tiled / 1e12}
    del x, y, canon, tiled
    return r


def run_f4(dev, steps, warmup):
    """GRPO token ratios and clipped surrogate over 8 prompts x 8 responses x 128 tokens (the prefill batch): seeded
    log-probabilities (log pi_b = -Exponential(2) per token, log pi_theta = log pi_b + N(0, 0.3)), advantages of
    Bernoulli(0.3) rewards from the device's group advantage."""
    import numpy as np
    import torch
    import nvfp4_weight_only_amd as qn
    import synth
    n_seq, t = 64, 128
    rng = np.random.default_rng(20251013)
    lp_old = torch.from_numpy((-rng.exponential(2.0, (n_seq, t))).astype(np.float32)).to(dev)
    lp = lp_old + torch.from_numpy(rng.normal(0.0, 0.3, (n_seq, t)).astype(np.float32)).to(dev)
    lengths = torch.from_numpy(rng.integers(1, t + 1, n_seq).astype(np.int32)).to(dev)
    rewards = torch.from_numpy(synth.bernoulli_f32(synth.seed_for(5, 0, "rewards"), (8, 8), 0.3)).to(dev)
    adv = qn.group_advantage(rewards).reshape(-1)
    out = {}

    def step(i):
        out["r"] = qn.grpo_surrogate(lp, lp_old, lengths, adv)

    tm = time_steps(step, max(steps, 20), warmup)
    nbytes = n_seq * t * 4 * 4 + n_seq * 8  # logp, logp_old in; surrogate, grad out; lengths, advantages
    st = qn.grpo_stats(out["r"][2])
    return {"us_per_call": tm * 1e6, "tokens": int(st["tokens"]), "algorithmic_bytes": nbytes,
            "GBps": nbytes / tm / 1e9, "bound": "latency (one workgroup; 128 KB moved)",
            "loss": st["loss"], "clipped_tokens": int(st["clipped"])}


def run_f2(base, shape, dev, steps, warmup):
    """Backward of the 7B gate projection (18944 x 3584, rank-32 LoRA) at the 8192-token prefill batch: dh through
    the frozen NVFP4 weight, dA and dB. The upstream gradient is seeded N(0, 1) bf16, h the prefill's input."""
    import torch
    import nvfp4_weight_only_amd as qn
    import synth
    m, n, k = 8192, shape.inter, shape.hidden
    s = lambda t: synth.seed_for(5, 1, t)
    g = bf16_dev(synth.normal_bf16(s("eps_norm1"), (m, n)), dev)
    h = bf16_dev(synth.normal_bf16(s("x"), (m, k)), dev)
    A, B = base.lora["gate"]
    w = base.w["gate"]
    stream = torch.cuda.current_stream()
    out = {}

    def run(want):
        out["r"] = qn.lora_linear_backward(g, h, w, A, B, 2.0, torch.float32, want)

    nsteps = max(5, steps // 2)
    t_all = time_steps(lambda i: run(("dh", "dA", "dB")), nsteps, max(1, warmup // 2))
    t_dh = time_steps(lambda i: run(("dh",)), nsteps, 1)
    fl_dh = 2 * m * n * k + 2 * m * shape.rank * (n + k)  # W^T g, and u = B^T g with A^T u
    fl_all = 2 * m * n * k + 2 * m * shape.rank * (2 * n + 2 * k)  # + t = A h, dA, dB
    return {"us_per_step": t_all * 1e6, "flops_per_step": fl_all, "step_TFLOPs": fl_all / t_all / 1e12,
            "dh_us": t_dh * 1e6, "dh_TFLOPs": fl_dh / t_dh / 1e12,
            "dh_frac_of_mfma_peak": fl_dh / t_dh / 1e12 / MFMA_PEAK_TFLOPS,
            "kernels": "k_bt + k_skinny (u) + k_dh (dh, bf16 MFMA, weight dequantized to LDS transposed); "
                       "k_skinny (t) + k_outer/k_outer_sum (dA, dB)"}


# ---- the oracle on the host ----------------------------------------------------------------------------------------
def cpu_threads():
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cap = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(avail, cap, 16))


def cpu_baseline(shape, m, sigma, row_stride=4, threads=1):
    """The oracle (fp64 C++) on a row-sampled layer step: both norms in full, every `row_stride`-th output row of each
    of the seven projections, split over `threads` host threads by output rows; time x row_stride to the full layer."""
    import numpy as np

    import oracle
    import synth

    s = lambda t: synth.seed_for(2, 0, t)
    x = synth.normal_bf16(s("x"), (m, shape.hidden))
    g = synth.bf16_const(1.0, (shape.hidden,))
    e1 = synth.normal_f32(s("eps_norm1"), (shape.hidden,))
    e2 = synth.normal_f32(s("eps_norm2"), (shape.hidden,))
    proj = {}
    for nm, (n, k) in shape.projections().items():
        w = synth.normal_bf16(s("w_" + nm), (n, k), std=0.02)[::row_stride]
        c, sb, sg, _ = oracle.nvfp4_quantize(w)
        A = synth.normal_bf16(s("a_" + nm), (shape.rank, k), std=0.02)
        B = np.ascontiguousarray(synth.normal_bf16(s("b_" + nm), (n, shape.rank), std=0.02)[::row_stride])
        proj[nm] = (c, sb, sg, A, B)
    act = {k: synth.normal_bf16(99, (m, k)) for k in {shape.hidden, shape.q_dim, shape.inter}}
    pool = ThreadPoolExecutor(threads) if threads > 1 else None

    def lin(h, nm):
        c, sb, sg, A, B = proj[nm]
        if pool is None:
            return oracle.lora_linear(h, c, sb, sg, A, B, 2.0)
        cuts = np.linspace(0, c.shape[0], threads + 1).astype(int)
        parts = pool.map(lambda ab: oracle.lora_linear(h, c[ab[0]:ab[1]], sb[ab[0]:ab[1]], sg, A, B[ab[0]:ab[1]], 2.0),
                         [(cuts[i], cuts[i + 1]) for i in range(threads)])
        return np.concatenate(list(parts), axis=1)

    best = float("inf")
    for _ in range(2):
        t0 = time.perf_counter()
        _, h1 = oracle.aqn_rmsnorm(x, g, e1, sigma)
        for nm in ("q", "k", "v"):
            lin(h1, nm)
        lin(act[shape.q_dim], "o")
        _, h2 = oracle.aqn_rmsnorm(x, g, e2, sigma)
        oracle.silu_mul(lin(h2, "gate"), lin(h2, "up"))
        lin(act[shape.inter], "down")
        best = min(best, time.perf_counter() - t0)
    if pool:
        pool.shutdown()
    t_layer = best * row_stride
    return {"value": m / (28 * t_layer), "unit": "tokens/s (28-layer equivalent)", "cores": threads, "kind": "oracle",
            "sample": f"one 7B layer step at M={m}: both norms in full, every {row_stride}th output row of all seven "
                      f"projections (fp64), output rows split over {threads} thread(s), best of 2; time x{row_stride} "
                      f"to the full layer",
            "layer_step_s": t_layer}


def prefill_cpu_baseline(shape, rows=2048, tokens=64):
    """The oracle (single-threaded fp64 C++) on a sample of the prefill GEMM, scaled to TFLOP/s."""
    import numpy as np

    import oracle
    import synth

    s = lambda t: synth.seed_for(5, 0, t)
    n, k, r = shape.inter, shape.hidden, shape.rank
    x = synth.normal_bf16(s("x"), (tokens, k))
    ws = {nm: synth.normal_bf16(s("w_" + nm), (n, k), std=0.02)[:rows] for nm in ("gate", "up")}
    lo = {nm: (synth.normal_bf16(s("a_" + nm), (r, k), std=0.02),
               np.ascontiguousarray(synth.normal_bf16(s("b_" + nm), (n, r), std=0.02)[:rows])) for nm in ("gate", "up")}
    q = {nm: oracle.nvfp4_quantize(w) for nm, w in ws.items()}
    t0 = time.perf_counter()
    yg = oracle.lora_linear(x, *q["gate"][:3], lo["gate"][0], lo["gate"][1], 2.0)
    yu = oracle.lora_linear(x, *q["up"][:3], lo["up"][0], lo["up"][1], 2.0)
    oracle.silu_mul(yg, yu)
    dt = time.perf_counter() - t0
    flop = 2 * (2 * tokens * rows * k + 2 * tokens * r * (rows + k))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{tokens} tokens x {rows} rows of gate and of up (fp64, single thread), SiLU*up"}


# ---- main ----------------------------------------------------------------------------------------------------------
def base_result(args, metric, value, unit, ms, config, dtype):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded SplitMix64/Box-Muller; W ~ N(0,0.02) quantized on device, x ~ N(0,1))",
            "config": config}


DTYPE = "nvfp4 weights x bf16 activations (f16 MFMA operands), f32 accumulate"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=["decode", "prefill"], default="decode",
                    help="decode: the 7B layer at M tokens (the headline) plus every other configuration; prefill: "
                         "the 8192-token gate|up GEMM alone")
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=16, help="decode tokens per step (M) of the headline")
    ap.add_argument("--copies", type=int, default=5, help="layer weight copies rotated for cold-HBM timing")
    ap.add_argument("--event-every", type=int, default=4,
                    help="headline: the gate|up main kernel records its own launch events on every n-th timed step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="headline only (no other configurations)")
    ap.add_argument("--only", default="", help="comma-separated subset of the extra configurations to run")
    ap.add_argument("--noise", choices=["input", "device"], default="input",
                    help="headline: the norms read a fixed noise vector (input) or draw one row per response inside "
                         "the norm prologues (device)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported (the decode path needs "
              f"no exchange between GPUs: each GPU decodes its own prompts)", file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_weight_only_amd as qn
    from nvfp4_weight_only_amd import NoiseDraw
    from nvfp4_weight_only_amd.layer import QWEN25_7B, QWEN25_32B
    import synth

    dev = torch.device("cuda:0")
    shape = QWEN25_7B
    sigma = float(qn.aqn_sigma(1))
    if args.workload == "prefill":
        log("building the 7B gate|up weights for 8192-token prefill")
        base = build_layer(shape, 2, dev, sigma)
        r = run_c5(base, shape, dev, args.steps, args.warmup)
        res = base_result(args, "prefill TFLOP/s (% of dense MFMA peak), 7B gate|up NVFP4+LoRA, 8192 tokens",
                          r["step_TFLOPs"], "TFLOP/s", r["us_per_step"] / 1e3,
                          {"workload": "prefill / log-prob forward GEMM: 8192 tokens through the 7B gate|up NVFP4 "
                                       "weights (18944 x 3584 each) + rank-32 bf16 LoRA, SiLU(gate)*up, then group "
                                       "advantages (8 groups of 8)", "global_batch": 8192}, DTYPE)
        res["roofline"] = {"kernel": r["kernel"], "bound": "mfma", "achieved": r["kernel_TFLOPs_events"],
                           "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": r["frac_of_mfma_peak_events"],
                           "traffic": profile_value(PREFILL_PROFILE, "traffic_bytes_per_launch", "k_gemm gate|up"),
                           "frac_profile": r.get("frac_of_mfma_peak_profile")}
        res["prefill"] = r
        if not args.no_cpu:
            res["cpu_baseline"] = prefill_cpu_baseline(shape)
        print(json.dumps(res), flush=True)
        return

    # ---- headline: the 7B layer at M tokens, weights rotated over copies
    m = args.batch
    log(f"building the 7B layer ({args.copies} copies), M={m}")
    base = build_layer(shape, 2, dev, sigma)
    if args.noise == "device":
        base.draws = (NoiseDraw(synth.seed_for(2, 0, "eps_norm1"), 0, 0, 1), NoiseDraw(synth.seed_for(2, 0, "eps_norm2"), 0, 0, 1))
    layers = copies_of(base, args.copies)
    ws = qn.Workspace(dev)
    x = bf16_dev(synth.normal_bf16(synth.seed_for(2, 0, "x"), (m, shape.hidden)), dev)
    bound = [L.bind(x, ws) for L in layers]
    stream = torch.cuda.current_stream()
    # every n-th timed step, the first n - 1 skipped (step 0 follows the synchronisation that opens the timed region)
    sampled = [i for i in range(args.steps) if i % args.event_every == args.event_every - 1]
    ev = launch_event_pairs(sampled, stream)
    timed = {"on": False}

    def step(i):
        c = bound[i % len(bound)].calls
        c[0]()
        c[1]()
        # sampled timed steps: the gate|up kernel records its own begin and end in the step's event pair
        c[2](main_events=ev[i] if timed["on"] and i in ev else None)
        c[3]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    timed["on"] = True
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {elapsed:.4f} s")
    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
    ms_step = elapsed * 1e3 / args.steps
    main_s = sum(a.elapsed_time(b) for a, b in ev.values()) / len(ev) * 1e-3
    step_bytes = layer_bytes(shape, m)
    gu_bytes = gateup_main_bytes(shape, m)
    achieved = gu_bytes / main_s / 1e9
    prof_us = profile_value(PROFILE, "avg_duration_us", "k_gemv gate|up")
    res = base_result(args, "decode tokens/s & achieved HBM GB/s (% of peak), Qwen2.5-7B-shaped NVFP4+LoRA",
                      m / (28 * ms_step * 1e-3), "tokens/s", ms_step,
                      {"workload": "Qwen2.5-7B-shaped decoder layer at decode, NVFP4 + rank-32 bf16 LoRA on every "
                                   "projection, two AQN-RMSNorms (sigma 1e-2), attention scores excluded",
                       "global_batch": m, "hidden": shape.hidden, "intermediate": shape.inter, "lora_rank": shape.rank,
                       "layer_copies_rotated": args.copies, "tokens_per_s_basis": "M / (28 x layer step time)",
                       "noise": "read: one seeded N(0,1) vector per norm, shared by the batch" if args.noise == "input"
                       else "drawn in the norm prologues: Philox4x64-10 + Box-Muller, one row per response"}, DTYPE)
    res.update({"layer_step_us": ms_step * 1e3, "step_algorithmic_bytes": step_bytes,
                "step_achieved_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
                "step_frac_of_hbm_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "step_tflops": layer_flops(shape, m) / (ms_step * 1e-3) / 1e12})
    res["roofline"] = {"kernel": "k_gemv gate|up (SiLU epilogue)", "bound": "hbm", "achieved": achieved,
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                       "traffic": profile_value(PROFILE, "traffic_bytes_per_launch", "k_gemv gate|up"),
                       "bytes_per_launch": gu_bytes, "launch_us_events": main_s * 1e6, "event_samples": len(ev),
                       "launch_us_profile": prof_us,
                       "frac_profile": (gu_bytes / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS) if prof_us else None}
    del bound

    if not args.no_extras:
        only = set(filter(None, args.only.split(",")))
        want = lambda name: not only or name in only
        cfg = {}
        stream_gbs = None
        if want("hbm_stream_read"):
            log("streaming-read ceiling")
            res["hbm_stream_read"] = run_stream_read(dev, args.steps)
            stream_gbs = res["hbm_stream_read"]["GBps"]
            res["roofline"]["frac_of_stream_read"] = achieved / stream_gbs
        if want("c1"):
            log("config 1: 4096 x 4096 projection, M=1")
            cfg["c1_proj4096_m1"] = run_c1(dev, sigma, args.steps, args.warmup, stream_gbs)
        for mm in (1, 8):
            if want(f"c2_m{mm}"):
                log(f"config 2: 7B layer, M={mm}")
                cfg[f"c2_layer7b_m{mm}"] = run_layer(layers, shape, mm, dev, args.steps, args.warmup, stream_gbs, 28,
                                                     synth.seed_for(2, 0, "x") + mm)
        if want("c3"):
            log("config 3: 28 chained 7B layers, M=64")
            cfg["c3_stack28_7b_m64"] = run_c3(base, shape, dev, args.steps, args.warmup, stream_gbs)
        if want("f3"):
            log("MXFP4 weights: 7B layer, M=16")
            cfg["f3_mxfp4_layer7b_m16"] = run_f3(base, shape, dev, args.steps, args.warmup, stream_gbs)
        if want("f3p"):
            log("MXFP4 weights: prefill 8192 tokens on the scaled-MFMA kernel")
            cfg["f3_mxfp4_prefill_m8192"] = run_f3_prefill(base, shape, dev, args.steps, args.warmup)
        if want("c5"):
            log("config 5: prefill 8192 tokens")
            cfg["c5_prefill_m8192"] = run_c5(base, shape, dev, args.steps, args.warmup)
        if want("f2"):
            log("backward through the 7B gate weight, 8192 tokens")
            cfg["f2_backward_gate_m8192"] = run_f2(base, shape, dev, args.steps, args.warmup)
        if want("f4"):
            log("GRPO ratio and clipped surrogate, 8192 tokens")
            cfg["f4_grpo_surrogate_8192"] = run_f4(dev, args.steps, args.warmup)
        del layers
        torch.cuda.empty_cache()
        if want("c4"):
            log("config 4: 32B layer, heavy-tailed weights (building)")
            base32 = build_layer(QWEN25_32B, 4, dev, sigma, wdist="t4")
            l32 = copies_of(base32, 3)
            for mm in (32, 128):
                log(f"config 4: 32B layer, M={mm}")
                cfg[f"c4_layer32b_m{mm}"] = run_layer(l32, QWEN25_32B, mm, dev, args.steps, args.warmup, stream_gbs,
                                                      64, synth.seed_for(4, 0, "x") + mm)
            del l32, base32
        res["configs"] = cfg
    if not args.no_cpu:
        nthreads = cpu_threads()
        log(f"oracle baseline on the host: {nthreads} threads, then 1")
        cb = cpu_baseline(shape, m, sigma, threads=nthreads)
        cb["nproc"] = os.cpu_count()
        one = cpu_baseline(shape, m, sigma, threads=1)
        cb["single_thread"] = {"value": one["value"], "cores": 1, "layer_step_s": one["layer_step_s"]}
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
