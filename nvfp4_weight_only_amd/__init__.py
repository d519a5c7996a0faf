"""Python binding of libqerl_nvfp4.so (include/qerl_nvfp4.h): argument marshalling only.

Every computation runs in the HIP library. PyTorch provides device memory and the current stream. Importing this
package without the built library raises, and calls never fall back to anything else.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QERL_NVFP4_LIB: another build of this library to load instead (the sanitizer test's host-only build)
LIB_PATH = os.environ.get("QERL_NVFP4_LIB") or os.path.join(_HERE, "libqerl_nvfp4.so")

QN_OK, QN_ERR_NULL, QN_ERR_SHAPE, QN_ERR_ALIGN, QN_ERR_VALUE, QN_ERR_WORKSPACE, QN_ERR_UNSUPPORTED, QN_ERR_HIP = range(8)
LAYOUT_ROWMAJOR, LAYOUT_TILED = 0, 1
BF16, F32 = 0, 1
EPI_NONE, EPI_SILU_MUL = 0, 1
RUN_PROLOGUE_ONLY, RUN_MAIN_ONLY = 0x100, 0x200

KERNEL_AUTO, KERNEL_GENERAL, KERNEL_DECODE, KERNEL_MANY, KERNEL_FUSED, KERNEL_WIDE = range(6)

EXPORTS = ["nvfp4_quantize", "nvfp4_tiled_codes_bytes", "nvfp4_tiled_scales_bytes", "nvfp4_dequantize", "aqn_rmsnorm",
           "aqn_noise",
           "nvfp4_lora_linear_workspace", "nvfp4_lora_linear", "nvfp4_lora_linear_workspace_opts",
           "nvfp4_lora_linear_opts", "nvfp4_lora_linear_noalloc", "nvfp4_lora_linear_noalloc_max_bytes",
           "aqn_sigma", "grpo_group_advantage", "grpo_clipped_surrogate", "qn_stream_read", "qn_status_string",
           "nvfp4_lora_linear_backward", "nvfp4_lora_linear_backward_workspace", "mxfp4_quantize",
           "mxfp4_dequantize", "mxfp4_scales_bytes", "mxfp4_lora_linear", "mxfp4_lora_linear_workspace"]


class QnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class QnAqn(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("noise", ctypes.c_void_p), ("noise_ld", ctypes.c_int64),
                ("sigma", ctypes.c_float), ("eps", ctypes.c_float), ("draw", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("subseed", ctypes.c_uint64), ("row_offset", ctypes.c_uint64),
                ("draw_rows", ctypes.c_int64)]


class QnProj(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("block_scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("lora_a", ctypes.c_void_p), ("lora_b", ctypes.c_void_p), ("r", ctypes.c_int32),
                ("lambda_", ctypes.c_float), ("y", ctypes.c_void_p), ("y_dtype", ctypes.c_int32),
                ("ldy", ctypes.c_int64), ("residual", ctypes.c_void_p), ("ld_res", ctypes.c_int64),
                ("y_repeat", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class QnLinearOpts(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("decode_kchunks", ctypes.c_int32), ("decode_depth", ctypes.c_int32),
                ("general_rows", ctypes.c_int32), ("general_waves", ctypes.c_int32), ("elem_store", ctypes.c_int32),
                ("main_begin", ctypes.c_void_p), ("main_end", ctypes.c_void_p)]


@dataclass
class LinearOpts:
    """Explicit kernel choice of one linear call (qn_linear_opts); the defaults are the library's own choice."""
    kernel: int = KERNEL_AUTO
    decode_kchunks: int = 0
    decode_depth: int = 0
    general_rows: int = 0
    general_waves: int = 0
    elem_store: int = 0
    main_events: tuple = None  # (begin, end): timing events as objects with a `cuda_event` handle, each recorded once

    def to_c(self) -> QnLinearOpts:
        ev = (None, None) if self.main_events is None else tuple(e.cuda_event for e in self.main_events)
        return QnLinearOpts(self.kernel, self.decode_kchunks, self.decode_depth, self.general_rows,
                            self.general_waves, self.elem_store, ev[0], ev[1])


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc for gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double,
                                 ctypes.c_size_t)
    sig = {
        "nvfp4_quantize": ([P, i64, i64, i64, i32, i32, P, P, P, P, P], i32),
        "nvfp4_tiled_codes_bytes": ([i64, i64], sz),
        "nvfp4_tiled_scales_bytes": ([i64, i64], sz),
        "nvfp4_dequantize": ([P, P, P, i64, i64, i32, P, i64, P], i32),
        "mxfp4_quantize": ([P, i64, i64, i64, i32, P, P, P, P, P], i32),
        "mxfp4_dequantize": ([P, P, i64, i64, P, i64, P], i32),
        "mxfp4_scales_bytes": ([i64, i64], sz),
        "aqn_rmsnorm": ([P, i64, i64, i64, ctypes.POINTER(QnAqn), P, i64, P], i32),
        "aqn_noise": ([ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, i64, i64, i64, P, i64, P], i32),
        "nvfp4_lora_linear_workspace": ([i64, i64, ctypes.POINTER(QnProj), i32], sz),
        "mxfp4_lora_linear_workspace": ([i64, i64, ctypes.POINTER(QnProj), i32], sz),
        "mxfp4_lora_linear": ([P, i64, i64, i64, ctypes.POINTER(QnAqn), ctypes.POINTER(QnProj), i32, i32, P, sz, P],
                              i32),
        "nvfp4_lora_linear": ([P, i64, i64, i64, ctypes.POINTER(QnAqn), ctypes.POINTER(QnProj), i32, i32, P, sz, P],
                              i32),
        "nvfp4_lora_linear_workspace_opts": ([i64, i64, ctypes.POINTER(QnProj), i32, ctypes.POINTER(QnLinearOpts)],
                                             sz),
        "nvfp4_lora_linear_opts": ([P, i64, i64, i64, ctypes.POINTER(QnAqn), ctypes.POINTER(QnProj), i32, i32,
                                    ctypes.POINTER(QnLinearOpts), P, sz, P], i32),
        "nvfp4_lora_linear_noalloc": ([P, i64, i64, i64, ctypes.POINTER(QnAqn), ctypes.POINTER(QnProj), i32, i32, P],
                                      i32),
        "nvfp4_lora_linear_noalloc_max_bytes": ([], sz),
        "aqn_sigma": ([i32, f64, f64], f64),
        "qn_stream_read": ([P, sz, P, P], i32),
        "nvfp4_lora_linear_backward": ([P, i64, i64, i64, P, i64, i64, P, P, P, P, P, i32, f32, P, i32, i64, P, P, P, sz,
                                        P], i32),
        "nvfp4_lora_linear_backward_workspace": ([i64, i64, i64, i32], sz),
        "grpo_clipped_surrogate": ([P, P, i64, P, P, i32, i32, f32, f32, i32, P, P, P, P], i32),
        "grpo_group_advantage": ([P, i32, i32, f32, P, P], i32),
        "qn_status_string": ([i32], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = _load()


def status_string(s: int) -> str:
    return lib.qn_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != QN_OK:
        raise QnError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocations the binding makes for a call on `stream` come from that stream's pool of the caching allocator, so
    they never alias memory another stream still has work pending on."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


# ---- NVFP4 weights ------------------------------------------------------------------------------------------------
@dataclass
class NVFP4Weight:
    """A packed NVFP4 weight [n x k]: codes + E4M3 block scales (in `layout`) + one f32 tensor scale (device)."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    n: int
    k: int
    layout: int

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel() + 4


def tiled_bytes(n: int, k: int):
    return int(lib.nvfp4_tiled_codes_bytes(n, k)), int(lib.nvfp4_tiled_scales_bytes(n, k))


def alloc_weight(n: int, k: int, layout: int = LAYOUT_TILED, device="cuda") -> NVFP4Weight:
    if layout == LAYOUT_TILED:
        cb, sb = tiled_bytes(n, k)
    else:
        cb, sb = n * k // 2, n * k // 16
    return NVFP4Weight(torch.zeros(max(cb, 16), dtype=torch.uint8, device=device),
                       torch.zeros(max(sb, 4), dtype=torch.uint8, device=device),
                       torch.zeros(1, dtype=torch.float32, device=device), n, k, layout)


def quantize(w: torch.Tensor, layout: int = LAYOUT_TILED, scale_mode: int = 0, out: Optional[NVFP4Weight] = None,
             flags: Optional[torch.Tensor] = None, stream=None) -> NVFP4Weight:
    """bf16 W [n, k] (device) -> NVFP4Weight. scale_mode 1 reads the scales already in `out`."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2
    n, k = w.shape
    if out is None:
        with _on(stream):
            out = alloc_weight(n, k, layout, w.device)
    _check(lib.nvfp4_quantize(_ptr(w), n, k, w.stride(0), scale_mode, out.layout, _ptr(out.codes), _ptr(out.scales),
                              _ptr(out.tensor_scale), _ptr(flags), _stream(stream)), "nvfp4_quantize")
    for t in (out.codes, out.scales, out.tensor_scale):
        _keep_for(t, stream)
    return out


def dequantize(wq: NVFP4Weight, stream=None) -> torch.Tensor:
    with _on(stream):
        out = torch.empty(wq.n, wq.k, dtype=torch.float32, device=wq.codes.device)
    _check(lib.nvfp4_dequantize(_ptr(wq.codes), _ptr(wq.scales), _ptr(wq.tensor_scale), wq.n, wq.k, wq.layout,
                                _ptr(out), wq.k, _stream(stream)), "nvfp4_dequantize")
    _keep_for(out, stream)
    return out


# ---- MXFP4 weights ------------------------------------------------------------------------------------------------
@dataclass
class MXFP4Weight:
    """A packed MXFP4 weight [n x k] in the canonical MX layout: codes [n][k/2] and E8M0 scales [n][k/32] (device)."""
    codes: torch.Tensor
    scales: torch.Tensor
    n: int
    k: int


def mxfp4_quantize(w: torch.Tensor, layout: int = LAYOUT_TILED, flags: Optional[torch.Tensor] = None, stream=None):
    """bf16 W [n, k] (device, k % 32 == 0) -> MXFP4 (OCP MX: E8M0 scale per 32 weights). LAYOUT_ROWMAJOR gives the
    canonical MXFP4Weight; LAYOUT_TILED gives the same weight re-expressed exactly as an NVFP4Weight (power-of-two
    block scales and tensor scale) for nvfp4_lora_linear and the other kernels; bit 1 of `flags` reports a block too
    far below the tensor's largest for that form."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2
    n, k = w.shape
    with _on(stream):
        if layout == LAYOUT_TILED:
            out = alloc_weight(n, k, LAYOUT_TILED, w.device)
            codes, scales, ts = out.codes, out.scales, out.tensor_scale
        else:
            codes = torch.zeros(max(n * k // 2, 16), dtype=torch.uint8, device=w.device)
            scales = torch.zeros(max(int(lib.mxfp4_scales_bytes(n, k)), 4), dtype=torch.uint8, device=w.device)
            ts = None
            out = MXFP4Weight(codes, scales, n, k)
    _check(lib.mxfp4_quantize(_ptr(w), n, k, w.stride(0), layout, _ptr(codes), _ptr(scales), _ptr(ts), _ptr(flags),
                              _stream(stream)), "mxfp4_quantize")
    for t in (codes, scales, ts):
        _keep_for(t, stream)
    return out


def mxfp4_dequantize(wq: MXFP4Weight, stream=None) -> torch.Tensor:
    with _on(stream):
        out = torch.empty(wq.n, wq.k, dtype=torch.float32, device=wq.codes.device)
    _check(lib.mxfp4_dequantize(_ptr(wq.codes), _ptr(wq.scales), wq.n, wq.k, _ptr(out), wq.k, _stream(stream)),
           "mxfp4_dequantize")
    _keep_for(out, stream)
    return out


# ---- AQN ----------------------------------------------------------------------------------------------------------
def aqn_sigma(stage: int, start: float = 1e-2, end: float = 5e-4) -> float:
    return float(lib.aqn_sigma(stage, start, end))


@dataclass
class NoiseDraw:
    """Noise drawn on the device (see aqn_noise): key (seed, subseed); row i takes draw row_offset + i // draw_rows
    (draw_rows > 0) or row_offset (draw_rows == 0)."""
    seed: int
    subseed: int = 0
    row_offset: int = 0
    draw_rows: int = 1


class AqnParams:
    """AQN-RMSNorm parameters: keeps the device tensors alive for as long as the C struct that points at them."""

    def __init__(self, gamma: torch.Tensor, noise: Optional[torch.Tensor], sigma: float, eps: float = 1e-6,
                 noise_per_row: bool = False, draw: Optional[NoiseDraw] = None):
        if draw is not None and noise is not None:
            raise ValueError("AQN noise is either read (noise) or drawn on the device (draw), not both")
        self.gamma, self.noise = gamma, noise
        self.c = QnAqn()
        self.c.gamma = gamma.data_ptr()
        self.c.noise = None if noise is None else noise.data_ptr()
        self.c.noise_ld = noise.shape[-1] if (noise is not None and noise_per_row) else 0
        self.c.sigma = sigma
        self.c.eps = eps
        if draw is not None:
            self.c.draw = 1
            self.c.seed, self.c.subseed = draw.seed, draw.subseed
            self.c.row_offset, self.c.draw_rows = draw.row_offset, draw.draw_rows


def make_aqn(gamma: torch.Tensor, noise: Optional[torch.Tensor], sigma: float, eps: float = 1e-6,
             noise_per_row: bool = False, draw: Optional[NoiseDraw] = None) -> AqnParams:
    return AqnParams(gamma, noise, sigma, eps, noise_per_row, draw)


def aqn_noise(draw: NoiseDraw, m: int, d: int, device, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Seeded standard-normal noise [m, d] f32 on the device (Philox4x64-10 + Box-Muller)."""
    with _on(stream):
        eps = out if out is not None else torch.empty(m, d, dtype=torch.float32, device=device)
    _check(lib.aqn_noise(draw.seed, draw.subseed, draw.row_offset, draw.draw_rows, m, d, _ptr(eps), eps.stride(0),
                         _stream(stream)), "aqn_noise")
    _keep_for(eps, stream)
    return eps


def aqn_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, noise: Optional[torch.Tensor], sigma: float, eps: float = 1e-6,
                noise_per_row: bool = False, out: Optional[torch.Tensor] = None, stream=None,
                draw: Optional[NoiseDraw] = None) -> torch.Tensor:
    m, d = x.shape
    with _on(stream):
        h = out if out is not None else torch.empty(m, d, dtype=torch.bfloat16, device=x.device)
    a = make_aqn(gamma, noise, sigma, eps, noise_per_row, draw)
    _check(lib.aqn_rmsnorm(_ptr(x), m, d, x.stride(0), ctypes.byref(a.c), _ptr(h), h.stride(0), _stream(stream)),
           "aqn_rmsnorm")
    _keep_for(h, stream)
    return h


# ---- linear -------------------------------------------------------------------------------------------------------
@dataclass
class Projection:
    weight: NVFP4Weight
    y: Optional[torch.Tensor]
    lora_a: Optional[torch.Tensor] = None
    lora_b: Optional[torch.Tensor] = None
    lam: float = 1.0
    residual: Optional[torch.Tensor] = None
    y_repeat: int = 0
    head_dim: int = 0

    def to_c(self) -> QnProj:
        p = QnProj()
        w = self.weight
        ts = getattr(w, "tensor_scale", None)  # (an MXFP4Weight in the canonical layout has none)
        p.codes, p.block_scales = w.codes.data_ptr(), w.scales.data_ptr()
        p.tensor_scale = ts.data_ptr() if ts is not None else None
        p.n = w.n
        if self.lora_a is not None:
            p.lora_a, p.lora_b, p.r = self.lora_a.data_ptr(), self.lora_b.data_ptr(), self.lora_a.shape[0]
        p.lambda_ = self.lam
        if self.y is not None:
            p.y = self.y.data_ptr()
            p.y_dtype = F32 if self.y.dtype == torch.float32 else BF16
            p.ldy = self.y.stride(0)
        if self.residual is not None:
            p.residual, p.ld_res = self.residual.data_ptr(), self.residual.stride(0)
        p.y_repeat, p.head_dim = self.y_repeat, self.head_dim
        return p


def _keep_for(t: Optional[torch.Tensor], stream) -> None:
    """A tensor that kernels on `stream` use while the caller's current stream runs ahead: the caching allocator must
    not hand its memory out again before that stream is done with it."""
    if t is not None and stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


class Workspace:
    """Grow-only device workspace for nvfp4_lora_linear (allocated zero-filled by torch, outside the timed calls; the
    library leaves its control words zero after every call)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = torch.empty(0, dtype=torch.uint8, device=device)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            # the old buffer's memory is recycled only after every stream it was used on reaches this point
            # (LinearCall records those streams on it)
            self.buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=self.device)
        return self.buf


def linear_workspace_bytes(m: int, k: int, projs: Sequence[Projection], opts: Optional[LinearOpts] = None) -> int:
    arr = (QnProj * len(projs))(*[p.to_c() for p in projs])
    oc = opts.to_c() if opts is not None else None
    return int(lib.nvfp4_lora_linear_workspace_opts(m, k, arr, len(projs), ctypes.byref(oc) if oc else None))


class LinearCall:
    """A prepared nvfp4_lora_linear call: the C structs are built once, so repeated launches only cross ctypes.
    opts: an explicit kernel choice (LinearOpts), None for the library's own. The workspace belongs to the stream
    current when it was allocated; a call on another stream is recorded on it, so its memory is not recycled while
    that stream may still use it."""

    def __init__(self, x: torch.Tensor, projs: Sequence[Projection], aqn: Optional[AqnParams] = None,
                 epilogue: int = EPI_NONE, workspace: Optional[Workspace] = None, opts: Optional[LinearOpts] = None):
        self.x = x
        self.m, self.k = x.shape
        self.projs = list(projs)
        self.arr = (QnProj * len(projs))(*[p.to_c() for p in projs])
        self.aqn = aqn
        self.epilogue = epilogue
        self.opts = opts.to_c() if opts is not None else None
        self.opts_ref = ctypes.byref(self.opts) if self.opts is not None else None
        need = int(lib.nvfp4_lora_linear_workspace_opts(self.m, self.k, self.arr, len(projs), self.opts_ref))
        self.ws = (workspace or Workspace(x.device)).get(need)
        self.ws_bytes = self.ws.numel()

    def __call__(self, stream=None, phases: int = 0, main_events=None):
        """main_events: a (begin, end) pair of timing events (objects with a `cuda_event` handle, such as
        torch.cuda.Event), each recorded once before so it exists, that this launch's main kernel records at its own
        begin and end (qn_linear_opts main_begin / main_end)."""
        ref = self.opts_ref
        if main_events is not None:
            oc = QnLinearOpts.from_buffer_copy(self.opts) if self.opts is not None else QnLinearOpts()
            oc.main_begin, oc.main_end = main_events[0].cuda_event, main_events[1].cuda_event
            ref = ctypes.byref(oc)
        _check(lib.nvfp4_lora_linear_opts(_ptr(self.x), self.m, self.k, self.x.stride(0),
                                          ctypes.byref(self.aqn.c) if self.aqn is not None else None, self.arr,
                                          len(self.projs), self.epilogue | phases, ref, _ptr(self.ws),
                                          self.ws_bytes, _stream(stream)),
               "nvfp4_lora_linear")
        _keep_for(self.ws, stream)


def lora_linear(x: torch.Tensor, projs: Sequence[Projection], aqn: Optional[AqnParams] = None, epilogue: int = EPI_NONE,
                workspace: Optional[Workspace] = None, stream=None, opts: Optional[LinearOpts] = None):
    """One call. Without a workspace, the call's own comes from `stream`'s allocator pool and is released on return
    (its memory is reused only by later work on that stream). The caller orders `stream` after any work on its tensors
    (torch's usual rule for tensors shared between streams)."""
    with _on(stream):
        LinearCall(x, projs, aqn, epilogue, workspace, opts)(stream)


def mxfp4_lora_linear(x: torch.Tensor, projs: Sequence[Projection], aqn: Optional[AqnParams] = None,
                      epilogue: int = EPI_NONE, workspace: Optional[Workspace] = None, stream=None):
    """mxfp4_lora_linear: the call on MXFP4 weights in the canonical MX layout (MXFP4Weight from mxfp4_quantize with
    LAYOUT_ROWMAJOR), on the scaled FP4 x FP8 MFMA kernel. Same arguments and workspace rules as lora_linear."""
    m, k = x.shape
    arr = (QnProj * len(projs))(*[p.to_c() for p in projs])
    with _on(stream):
        need = int(lib.mxfp4_lora_linear_workspace(m, k, arr, len(projs)))
        ws = (workspace or Workspace(x.device)).get(need)
    _check(lib.mxfp4_lora_linear(_ptr(x), m, k, x.stride(0), ctypes.byref(aqn.c) if aqn is not None else None, arr,
                                 len(projs), epilogue, _ptr(ws), ws.numel(), _stream(stream)), "mxfp4_lora_linear")
    _keep_for(ws, stream)


def lora_linear_noalloc(x: torch.Tensor, projs: Sequence[Projection], aqn: Optional[AqnParams] = None,
                        epilogue: int = EPI_NONE, stream=None):
    """nvfp4_lora_linear_noalloc: the same call with the library's own scratch array (no workspace, no allocation).
    Calls that overlap on one GPU share that array and must not run concurrently."""
    arr = (QnProj * len(projs))(*[p.to_c() for p in projs])
    m, k = x.shape
    _check(lib.nvfp4_lora_linear_noalloc(_ptr(x), m, k, x.stride(0), ctypes.byref(aqn.c) if aqn is not None else None,
                                         arr, len(projs), epilogue, _stream(stream)), "nvfp4_lora_linear_noalloc")


GRPO_STATS_DTYPE = [("loss", "f8"), ("ratio_mean", "f8"), ("ratio_min", "f4"), ("ratio_max", "f4"),
                    ("tokens", "i8"), ("clipped", "i8")]
GRPO_STATS_BYTES = 40


def grpo_surrogate(logp: torch.Tensor, logp_old: torch.Tensor, lengths: torch.Tensor, adv: torch.Tensor,
                   clip_low: float = 0.2, clip_high: float = 0.2, agg: int = 0, stream=None):
    """grpo_clipped_surrogate: logp, logp_old [n_seq, t_max] f32; lengths int32 [n_seq]; adv f32 [n_seq] (device) ->
    (surrogate [n_seq, t_max] f32, grad [n_seq, t_max] f32, stats: a 40-byte device buffer, see grpo_stats)."""
    n_seq, t_max = logp.shape
    with _on(stream):
        sur = torch.empty(n_seq, t_max, dtype=torch.float32, device=logp.device)
        grad = torch.empty_like(sur)
        stats = torch.zeros(GRPO_STATS_BYTES, dtype=torch.uint8, device=logp.device)
    _check(lib.grpo_clipped_surrogate(_ptr(logp), _ptr(logp_old), logp.stride(0), _ptr(lengths), _ptr(adv), n_seq,
                                      t_max, clip_low, clip_high, agg, _ptr(sur), _ptr(grad), _ptr(stats),
                                      _stream(stream)), "grpo_clipped_surrogate")
    return sur, grad, stats


def grpo_stats(stats: torch.Tensor) -> dict:
    """The device statistics buffer of grpo_surrogate as a dict (copies to the host)."""
    import numpy as np
    rec = np.frombuffer(stats.cpu().numpy().tobytes(), dtype=np.dtype(GRPO_STATS_DTYPE))[0]
    return {k: rec[k].item() for k, _ in GRPO_STATS_DTYPE}


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """qn_stream_read over the whole of `buf` (a measurement helper: plain streaming reads)."""
    _check(lib.qn_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "qn_stream_read")


def lora_linear_backward(g: torch.Tensor, h: Optional[torch.Tensor], weight: NVFP4Weight,
                         lora_a: Optional[torch.Tensor], lora_b: Optional[torch.Tensor], lam: float = 1.0,
                         dh_dtype=torch.float32, want=("dh", "dA", "dB"), stream=None):
    """Backward of one projection through the frozen tiled NVFP4 weight: g = dL/dy bf16 [m, n], h = the forward's
    input bf16 [m, k] -> dict with dh [m, k] (dh_dtype), dA f32 [r, k], dB f32 [n, r] (those in `want`)."""
    m, n = g.shape
    k = weight.k
    r = 0 if lora_a is None else lora_a.shape[0]
    need = int(lib.nvfp4_lora_linear_backward_workspace(m, n, k, r))
    with _on(stream):
        out = {"dh": torch.empty(m, k, dtype=dh_dtype, device=g.device) if "dh" in want else None,
               "dA": torch.empty(r, k, dtype=torch.float32, device=g.device) if ("dA" in want and r) else None,
               "dB": torch.empty(n, r, dtype=torch.float32, device=g.device) if ("dB" in want and r) else None}
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=g.device)
    dh = out["dh"]
    _check(lib.nvfp4_lora_linear_backward(_ptr(g), m, n, g.stride(0), _ptr(h), k, h.stride(0) if h is not None else k,
                                          _ptr(weight.codes), _ptr(weight.scales), _ptr(weight.tensor_scale),
                                          _ptr(lora_a), _ptr(lora_b), r, lam, _ptr(dh),
                                          F32 if dh_dtype == torch.float32 else BF16, dh.stride(0) if dh is not None else k,
                                          _ptr(out["dA"]), _ptr(out["dB"]), _ptr(ws), ws.numel(), _stream(stream)),
           "nvfp4_lora_linear_backward")
    _keep_for(ws, stream)
    return {key: v for key, v in out.items() if v is not None}


def group_advantage(rewards: torch.Tensor, eps: float = 1e-6, stream=None) -> torch.Tensor:
    groups, g = rewards.shape
    with _on(stream):
        adv = torch.empty_like(rewards)
    _check(lib.grpo_group_advantage(_ptr(rewards), groups, g, eps, _ptr(adv), _stream(stream)),
           "grpo_group_advantage")
    _keep_for(adv, stream)
    return adv
