"""Helpers shared by the GPU parity tests: numpy <-> device tensors and the error measure."""
import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

# max |y - r| / max |r| on the f32 output, compared with the fp64 oracle (the bar fixed for this path)
LINEAR_TOL = 2e-3


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def rel_err(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(y - ref).max() / np.abs(ref).max())


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
