"""One Qwen2.5-shaped decoder layer at decode time, on NVFP4 weights with rank-r bf16 LoRA on every projection.

The layer is four nvfp4_lora_linear calls (the library does all arithmetic):
  1. AQN-RMSNorm(x) feeding q | k | v   (one shared noise vector, [review §5.1]); v's output is broadcast to its query
     heads, which stands in for attention with the score computation excluded (attention over one key position)
  2. o_proj(attn) + x                   (residual in the epilogue)
  3. AQN-RMSNorm(x2) feeding gate | up, epilogue SiLU(gate) * up   (Gate/Up share the feed-forward norm)
  4. down(a) + x2
[review] = "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import (BF16, EPI_NONE, EPI_SILU_MUL, LAYOUT_TILED, LinearCall, NVFP4Weight, Projection, Workspace,
               make_aqn, quantize)


@dataclass
class LayerShape:
    hidden: int
    q_dim: int
    kv_dim: int
    inter: int
    head_dim: int = 128
    rank: int = 32

    @property
    def group(self) -> int:
        return self.q_dim // self.kv_dim

    def projections(self):
        h, q, kv, i = self.hidden, self.q_dim, self.kv_dim, self.inter
        return {"q": (q, h), "k": (kv, h), "v": (kv, h), "o": (h, q), "gate": (i, h), "up": (i, h), "down": (h, i)}

    def nvfp4_bytes(self) -> int:
        return sum(9 * n * k // 16 + 4 for n, k in self.projections().values())

    def lora_bytes(self) -> int:
        return sum(2 * self.rank * (n + k) for n, k in self.projections().values())


QWEN25_7B = LayerShape(hidden=3584, q_dim=3584, kv_dim=512, inter=18944)
QWEN25_32B = LayerShape(hidden=5120, q_dim=5120, kv_dim=1024, inter=27648)


class DecoderLayer:
    """Device state of one layer: packed weights, adapters, norm scales and noise, plus prepared calls per batch."""

    def __init__(self, shape: LayerShape, weights: Dict[str, NVFP4Weight], lora: Dict[str, tuple],
                 gamma1: torch.Tensor, gamma2: torch.Tensor, noise1: Optional[torch.Tensor],
                 noise2: Optional[torch.Tensor], sigma: float, lam: float = 2.0, eps: float = 1e-6,
                 draws: Optional[tuple] = None, noise_rows: bool = False):
        """draws: None (the norms read noise1, noise2: one vector for every row, or with noise_rows one row per token),
        or a pair of NoiseDraw: the two norms draw their noise on the device instead (noise1, noise2 not read)."""
        self.shape, self.w, self.lora = shape, weights, lora
        self.gamma1, self.gamma2, self.noise1, self.noise2 = gamma1, gamma2, noise1, noise2
        self.sigma, self.lam, self.eps = sigma, lam, eps
        self.draws = draws
        self.noise_rows = noise_rows

    @staticmethod
    def from_bf16(shape: LayerShape, w_bf16: Dict[str, torch.Tensor], lora: Dict[str, tuple], gamma1, gamma2,
                  noise1, noise2, sigma, lam=2.0, eps=1e-6) -> "DecoderLayer":
        weights = {name: quantize(w, LAYOUT_TILED) for name, w in w_bf16.items()}
        return DecoderLayer(shape, weights, lora, gamma1, gamma2, noise1, noise2, sigma, lam, eps)

    def bind(self, x: torch.Tensor, ws: Optional[Workspace] = None) -> "BoundLayer":
        return BoundLayer(self, x, ws or Workspace(x.device))


class BoundLayer:
    """A layer bound to an input buffer x [m, hidden] (bf16): owns the intermediate buffers and prepared calls."""

    def __init__(self, layer: DecoderLayer, x: torch.Tensor, ws: Workspace):
        L, S = layer, layer.shape
        m = x.shape[0]
        dev = x.device
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.x = x
        self.q = torch.empty(m, S.q_dim, **bf)
        self.k = torch.empty(m, S.kv_dim, **bf)
        self.attn = torch.empty(m, S.q_dim, **bf)   # v broadcast to the query heads
        self.x2 = torch.empty(m, S.hidden, **bf)
        self.a = torch.empty(m, S.inter, **bf)
        self.out = torch.empty(m, S.hidden, **bf)

        def proj(name, y, **kw):
            A, B = L.lora.get(name, (None, None))
            return Projection(L.w[name], y, A, B, L.lam, **kw)

        if L.draws is None:
            aqn1 = make_aqn(L.gamma1, L.noise1, L.sigma, L.eps, noise_per_row=L.noise_rows)
            aqn2 = make_aqn(L.gamma2, L.noise2, L.sigma, L.eps, noise_per_row=L.noise_rows)
        else:
            aqn1 = make_aqn(L.gamma1, None, L.sigma, L.eps, draw=L.draws[0])
            aqn2 = make_aqn(L.gamma2, None, L.sigma, L.eps, draw=L.draws[1])
        self.calls = [
            LinearCall(x, [proj("q", self.q), proj("k", self.k),
                           proj("v", self.attn, y_repeat=S.group, head_dim=S.head_dim)], aqn1, EPI_NONE, ws),
            LinearCall(self.attn, [proj("o", self.x2, residual=x)], None, EPI_NONE, ws),
            LinearCall(self.x2, [proj("gate", self.a), proj("up", None)], aqn2, EPI_SILU_MUL, ws),
            LinearCall(self.a, [proj("down", self.out, residual=self.x2)], None, EPI_NONE, ws),
        ]

    def __call__(self, stream=None) -> torch.Tensor:
        for c in self.calls:
            c(stream)
        return self.out
