#!/usr/bin/env python3
"""Decode benchmark: one Qwen2.5-7B-shaped decoder layer on NVFP4 weights with rank-32 bf16 LoRA on every
projection and two AQN-RMSNorms (hidden 3584; q/o 3584x3584; k/v 512x3584; gate/up 18944x3584; down 3584x18944).

A step is one decode pass of the whole layer over a batch of M tokens: AQN-RMSNorm -> q|k|v (v broadcast to its
query heads; attention scores excluded) -> o + residual -> AQN-RMSNorm -> gate|up + SiLU*up -> down + residual.
Steps rotate over several copies of the layer's weights so the working set is well beyond the 256 MB Infinity Cache
(cold HBM). All inputs are seeded synthetic tensors (synth/), W ~ N(0, 0.02) quantized on the GPU, x ~ N(0, 1),
sigma = 1e-2.

Prints one JSON line. `value` is 28-layer-equivalent decode tokens/s: M / (28 * layer step time), i.e. the rate of
a 28-layer linear stack of this layer with attention scores excluded.

`--workload prefill` instead times the prefill / log-prob forward GEMM: 8192 tokens (8 prompts x 8 responses x 128
tokens, x ~ N(0,1) bf16) through the 7B gate|up NVFP4 weights (18944 x 3584 each) with rank-32 LoRA and the
SiLU(gate) * up epilogue on the MFMA path, followed by the group advantages of 8 groups of 8 Bernoulli(0.3) rewards;
`value` is TFLOP/s of the whole step and the roofline is the MFMA kernel's against the 2.5 PFLOP/s dense f16/bf16 peak.
"""
from __future__ import annotations

import argparse
import functools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16 / bf16 matrix peak, published
PROFILE = os.path.join(ROOT, "profiles", "decode_layer_7b_m16.md")
PREFILL_PROFILE = os.path.join(ROOT, "profiles", "prefill_gateup_7b_m8192.md")
KERNEL_SOURCE = os.path.join(ROOT, "nvfp4_weight_only_amd", "csrc", "linear.hip")


def measured_traffic(profile=PROFILE, tag="k_gemv gate|up"):
    """HBM bytes per launch of the tagged kernel from a committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's readings), or None when the kernel source has changed since it was taken."""
    import hashlib
    import re
    try:
        text = open(profile).read()
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    mt = re.search(r"traffic_bytes_per_launch\[" + re.escape(tag) + r"\] = (\d+) \(linear\.hip sha256 ([0-9a-f]{64})\)",
                   text)
    if not mt or mt.group(2) != sha:
        return None
    return int(mt.group(1))


def algorithmic_bytes(shape, m):
    """NVFP4 9NK/16 + 4, LoRA 2r(N+K), activations in/out 2M(N+K) per projection; gamma + noise 6d per norm."""
    total = 0
    for n, k in shape.projections().values():
        total += 9 * n * k // 16 + 4 + 2 * shape.rank * (n + k) + 2 * m * (n + k)
    return total + 2 * 6 * shape.hidden


def gateup_main_bytes(shape, m):
    """Algorithmic bytes of the gate|up main kernel: both NVFP4 weights, both LoRA-B, the activation in, a out."""
    n, k = shape.inter, shape.hidden
    return 2 * (9 * n * k // 16 + 4) + 2 * 2 * shape.rank * n + 2 * m * k + 2 * m * n


def flops(shape, m):
    return sum(2 * m * n * k + 2 * m * shape.rank * (n + k) for n, k in shape.projections().values())


def build_layers(shape, m, copies, sigma, dev, noise="input"):
    """noise: "input" (each norm reads a seeded noise vector shared by the batch) or "device" (each norm draws one
    noise row per response on the device: Philox4x64-10 + Box-Muller, a key per layer copy and norm)."""
    import numpy as np
    import torch

    import synth
    from nvfp4_weight_only_amd.layer import DecoderLayer

    def bf16_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    s = lambda t: synth.seed_for(2, 0, t)
    w = {nm: bf16_dev(synth.normal_bf16(s("w_" + nm), nk, std=0.02)) for nm, nk in shape.projections().items()}
    lora = {nm: (bf16_dev(synth.normal_bf16(s("a_" + nm), (shape.rank, nk[1]), std=0.02)),
                 bf16_dev(synth.normal_bf16(s("b_" + nm), (nk[0], shape.rank), std=0.02)))
            for nm, nk in shape.projections().items()}
    g1 = bf16_dev(synth.bf16_const(1.0, (shape.hidden,)))
    g2 = bf16_dev(synth.bf16_const(1.0, (shape.hidden,)))
    e1 = torch.from_numpy(synth.normal_f32(s("eps_norm1"), (shape.hidden,))).to(dev)
    e2 = torch.from_numpy(synth.normal_f32(s("eps_norm2"), (shape.hidden,))).to(dev)
    x = bf16_dev(synth.normal_bf16(s("x"), (m, shape.hidden)))
    from nvfp4_weight_only_amd import NoiseDraw

    def draws(i):
        if noise != "device":
            return None
        return (NoiseDraw(s("eps_norm1"), i, 0, 1), NoiseDraw(s("eps_norm2"), i, 0, 1))

    base = DecoderLayer.from_bf16(shape, w, lora, g1, g2, e1, e2, sigma, 2.0)
    base.draws = draws(0)
    del w
    layers = [base]
    for i in range(1, copies):  # distinct copies of the packed weights and adapters (same values, new addresses)
        wq = {nm: type(q)(q.codes.clone(), q.scales.clone(), q.tensor_scale.clone(), q.n, q.k, q.layout)
              for nm, q in base.w.items()}
        lo = {nm: (a.clone(), b.clone()) for nm, (a, b) in lora.items()}
        layers.append(DecoderLayer(shape, wq, lo, g1, g2, e1, e2, sigma, 2.0, draws=draws(i)))
    torch.cuda.synchronize()
    return layers, x


def cpu_baseline(shape, m, sigma, row_stride=4, repeats=2):
    """The oracle (single-threaded fp64 C++) timed on a row-sampled layer step: both norms in full, every
    `row_stride`-th output row of each of the seven projections; time scaled by row_stride to the full layer."""
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
        B = synth.normal_bf16(s("b_" + nm), (n, shape.rank), std=0.02)[::row_stride]
        proj[nm] = (c, sb, sg, A, np.ascontiguousarray(B))
    act = {k: synth.normal_bf16(99, (m, k)) for k in {shape.hidden, shape.q_dim, shape.inter}}
    best = float("inf")
    for _ in range(repeats):
        t0 = time.perf_counter()
        _, h1 = oracle.aqn_rmsnorm(x, g, e1, sigma)
        for nm in ("q", "k", "v"):
            oracle.lora_linear(h1, *proj[nm][:3], proj[nm][3], proj[nm][4], 2.0)
        oracle.lora_linear(act[shape.q_dim], *proj["o"][:3], proj["o"][3], proj["o"][4], 2.0)
        _, h2 = oracle.aqn_rmsnorm(x, g, e2, sigma)
        yg = oracle.lora_linear(h2, *proj["gate"][:3], proj["gate"][3], proj["gate"][4], 2.0)
        yu = oracle.lora_linear(h2, *proj["up"][:3], proj["up"][3], proj["up"][4], 2.0)
        oracle.silu_mul(yg, yu)
        oracle.lora_linear(act[shape.inter], *proj["down"][:3], proj["down"][3], proj["down"][4], 2.0)
        best = min(best, time.perf_counter() - t0)
    t_layer = best * row_stride
    return {"value": m / (28 * t_layer), "unit": "tokens/s (28-layer equivalent)", "cores": 1, "kind": "oracle",
            "sample": f"one layer step at M={m}: both norms in full, every {row_stride}th output row of all seven "
                      f"projections (fp64, single thread), best of {repeats}; time x{row_stride} to the full layer",
            "layer_step_s": t_layer}


def prefill_flops(shape, m):
    """gate and up: 2 M N K each, plus the rank-r LoRA of each (down 2 M r K, up 2 M r N)."""
    n, k, r = shape.inter, shape.hidden, shape.rank
    return 2 * (2 * m * n * k + 2 * m * r * (n + k))


def prefill_cpu_baseline(shape, rows=2048, tokens=64):
    """The oracle (single-threaded fp64 C++) on a sample of the prefill GEMM: `tokens` tokens through `rows` output rows
    of gate and of up (quantization of those rows included, as the GPU step excludes it: reported separately),
    scaled to FLOP/s and so to the full step's time."""
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
            "sample": f"{tokens} tokens x {rows} rows of gate and of up (fp64, single thread), SiLU*up; TFLOP/s of "
                      f"that sample, i.e. the full step would take {prefill_flops(shape, 8192) / (flop / dt):.0f} s"}


def run_prefill(args):
    import numpy as np
    import torch

    import nvfp4_weight_only_amd as qn
    import synth
    from nvfp4_weight_only_amd.layer import QWEN25_7B

    shape = QWEN25_7B
    m, n, k, r = 8192, shape.inter, shape.hidden, shape.rank
    dev = torch.device("cuda:0")

    def bf16_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    s = lambda t: synth.seed_for(5, 0, t)
    print("[bench] building the prefill gate|up weights, M=8192", file=sys.stderr, flush=True)
    wq = {nm: qn.quantize(bf16_dev(synth.normal_bf16(s("w_" + nm), (n, k), std=0.02)), qn.LAYOUT_TILED)
          for nm in ("gate", "up")}
    lora = {nm: (bf16_dev(synth.normal_bf16(s("a_" + nm), (r, k), std=0.02)),
                 bf16_dev(synth.normal_bf16(s("b_" + nm), (n, r), std=0.02))) for nm in ("gate", "up")}
    x = bf16_dev(synth.normal_bf16(s("x"), (m, k)))
    y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    rewards = torch.from_numpy(synth.bernoulli_f32(s("rewards"), (8, 8), 0.3)).to(dev)
    call = qn.LinearCall(x, [qn.Projection(wq["gate"], y, *lora["gate"], 2.0),
                             qn.Projection(wq["up"], None, *lora["up"], 2.0)], None, qn.EPI_SILU_MUL)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i, timed):
        call(phases=qn.RUN_PROLOGUE_ONLY)
        if timed:
            ev[i][0].record(stream)
        call(phases=qn.RUN_MAIN_ONLY)
        if timed:
            ev[i][1].record(stream)
        qn.group_advantage(rewards)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
    ms_step = elapsed * 1e3 / args.steps
    main_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / args.steps
    fl = prefill_flops(shape, m)
    achieved = fl / (main_ms * 1e-3) / 1e12
    result = {
        "metric": "prefill TFLOP/s (% of dense MFMA peak), 7B gate|up NVFP4+LoRA, 8192 tokens",
        "value": fl / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 weights x bf16 activations (f16 MFMA operands), f32 accumulate",
        "data": "synthetic (seeded; W ~ N(0,0.02) quantized on device, x ~ N(0,1), R ~ Bernoulli(0.3))",
        "config": {"workload": "prefill / log-prob forward GEMM: 8192 tokens through the 7B gate|up NVFP4 weights "
                               "(18944 x 3584 each) + rank-32 bf16 LoRA, SiLU(gate)*up, then group advantages "
                               "(8 groups of 8)", "global_batch": m, "hidden": k, "intermediate": n, "lora_rank": r},
        "prefill_tokens_per_s": m / (ms_step * 1e-3),
        "roofline": {"kernel": "k_gemm (prefill MFMA GEMM, SiLU epilogue)", "bound": "mfma", "achieved": achieved,
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFLOPS,
                     "traffic": measured_traffic(PREFILL_PROFILE, "k_gemm gate|up"), "launch_us": main_ms * 1e3,
                     "flops_per_launch": fl},
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = prefill_cpu_baseline(shape)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=["decode", "prefill"], default="decode",
                    help="decode: one 7B layer at M tokens (the headline); prefill: the 8192-token gate|up GEMM")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=16, help="decode tokens per step (M)")
    ap.add_argument("--copies", type=int, default=5, help="layer weight copies rotated for cold-HBM timing")
    ap.add_argument("--event-every", type=int, default=8,
                    help="decode: put HIP events around the gate|up kernel on every n-th timed step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--noise", choices=["input", "device", "standalone"], default="input",
                    help="decode: the norms read a fixed noise vector (input), draw one row per response inside the "
                         "norm prologues (device), or read rows written by the standalone generator before each "
                         "norm (standalone: the same draws, one more launch per norm)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.workload == "prefill":
        if args.steps == ap.get_default("steps"):
            args.steps, args.warmup = 20, 3
        return run_prefill(args)

    import torch

    import nvfp4_weight_only_amd as qn
    from nvfp4_weight_only_amd.layer import QWEN25_7B

    shape = QWEN25_7B
    m = args.batch
    sigma = float(qn.aqn_sigma(1))
    dev = torch.device("cuda:0")
    print(f"[bench] building {args.copies} layer copies, M={m}", file=sys.stderr, flush=True)
    layers, x = build_layers(shape, m, args.copies, sigma, dev, "device" if args.noise == "device" else "input")
    if args.noise == "standalone":
        # per-response rows written by aqn_noise before each norm, read by the norm (noise_per_row)
        for i, L in enumerate(layers):
            L.noise1 = torch.empty(m, shape.hidden, dtype=torch.float32, device=dev)
            L.noise2 = torch.empty(m, shape.hidden, dtype=torch.float32, device=dev)
            L.noise_rows = True
            # the generator calls with their arguments bound once (a step's host work stays below its GPU time)
            sh = qn._stream(torch.cuda.current_stream())
            L.fresh = tuple(functools.partial(qn.lib.aqn_noise, j + 1, i, 0, 1, m, shape.hidden, qn._ptr(buf),
                                              shape.hidden, sh) for j, buf in enumerate((L.noise1, L.noise2)))
    ws = qn.Workspace(dev)
    bound = [L.bind(x, ws) for L in layers]
    stream = torch.cuda.current_stream()

    # On every event_every-th timed step the gate|up call is split into its prologue and main kernel, with events
    # around the main kernel (an event pair costs a few microseconds of GPU time, so not every step carries one).
    sampled = [i for i in range(args.steps) if i % args.event_every == 0]
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in sampled}

    def step(i, timed):
        b = bound[i % len(bound)]
        c = b.calls
        if args.noise == "standalone":
            L = layers[i % len(layers)]
            L.fresh[0]()
        c[0]()
        c[1]()
        if args.noise == "standalone":
            L.fresh[1]()
        if timed and i in ev:
            c[2](phases=qn.RUN_PROLOGUE_ONLY)
            ev[i][0].record(stream)
            c[2](phases=qn.RUN_MAIN_ONLY)
            ev[i][1].record(stream)
        else:
            c[2]()
        c[3]()

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    ms_step = elapsed * 1e3 / args.steps
    main_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev.values()) / len(ev)
    step_bytes = algorithmic_bytes(shape, m)
    gu_bytes = gateup_main_bytes(shape, m)
    achieved = gu_bytes / (main_ms * 1e-3) / 1e9
    result = {
        "metric": "decode tokens/s & achieved HBM GB/s (% of peak), Qwen2.5-7B-shaped NVFP4+LoRA",
        "value": m / (28 * ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 weights x bf16 activations (f16 MFMA operands), f32 accumulate",
        "data": "synthetic (seeded SplitMix64/Box-Muller; W ~ N(0,0.02) quantized on device, x ~ N(0,1))",
        "config": {"workload": "Qwen2.5-7B-shaped decoder layer at decode, NVFP4 + rank-32 bf16 LoRA on every "
                               "projection, two AQN-RMSNorms (sigma 1e-2), attention scores excluded",
                   "global_batch": m, "hidden": shape.hidden, "intermediate": shape.inter, "lora_rank": shape.rank,
                   "layer_copies_rotated": args.copies, "tokens_per_s_basis": "M / (28 x layer step time)",
                   "noise": {"input": "read: one seeded N(0,1) vector per norm, shared by the batch",
                             "device": "drawn in the norm prologues: Philox4x64-10 + Box-Muller, one row per response",
                             "standalone": "one row per response, written by aqn_noise before each norm and read"
                             }[args.noise]},
        "layer_step_us": ms_step * 1e3,
        "step_algorithmic_bytes": step_bytes,
        "step_achieved_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_tflops": flops(shape, m) / (ms_step * 1e-3) / 1e12,
        "roofline": {"kernel": "k_gemv gate|up (SiLU epilogue)", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(), "launch_us": main_ms * 1e3, "bytes_per_launch": gu_bytes,
                     "event_samples": len(ev)},
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(shape, m, sigma)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
